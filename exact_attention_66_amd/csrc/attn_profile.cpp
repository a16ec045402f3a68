// Opt-in kernel timing: while a profiling window is open, every kernel the
// library launches is bracketed by a HIP event pair taken by the launch
// itself (hipExtLaunchKernel), so the durations are those of the kernels on
// the stream they run on.  Closed by default; the launch path then calls
// hipLaunchKernel directly and keeps no state.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace attn {

namespace {

struct Rec {
  int kind;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
// Events created when the window opens, so that timed launches do not pay
// for hipEventCreate (about 10 us per short launch).  All are destroyed when
// the window closes.
std::vector<hipEvent_t> g_pool;
constexpr int kPoolEvents = 1024;

void destroy_all_locked() {
  for (auto& r : g_recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_recs.clear();
  for (hipEvent_t ev : g_pool) (void)hipEventDestroy(ev);
  g_pool.clear();
}

// An event from the pool, or a new one when the pool is empty.
hipError_t take_event(hipEvent_t* ev) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_pool.empty()) {
      *ev = g_pool.back();
      g_pool.pop_back();
      return hipSuccess;
    }
  }
  return hipEventCreate(ev);
}

void give_back(hipEvent_t ev) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_pool.push_back(ev);
}

}  // namespace

hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream, int kind) {
  if (!g_on.load(std::memory_order_acquire)) return hipLaunchKernel(fn, grid, block, args, 0, stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = take_event(&e0);
  if (e == hipSuccess) e = take_event(&e1);
  if (e != hipSuccess) {
    if (e0) give_back(e0);
    return e;
  }
  e = hipExtLaunchKernel(fn, grid, block, args, 0, stream, e0, e1, 0);
  if (e != hipSuccess) {
    give_back(e0);
    give_back(e1);
    return e;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back({kind, e0, e1});
  return hipSuccess;
}

int persistent_grid(const void* fn, int block, int units) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  int n = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDev) n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev >= 0 && dev < kMaxDev) cus[dev].store(n, std::memory_order_relaxed);
  }
  // resident workgroups per CU of this kernel: asked once per (device, kernel, block size)
  struct Occ {
    int dev;
    const void* fn;
    int block;
    int per_cu;
  };
  static std::mutex occ_mu;
  static std::vector<Occ> occ;
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> lk(occ_mu);
    for (const Occ& o : occ)
      if (o.dev == dev && o.fn == fn && o.block == block) per_cu = o.per_cu;
  }
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    std::lock_guard<std::mutex> lk(occ_mu);
    occ.push_back({dev, fn, block, per_cu});
  }
  const int per_xcd = (n * per_cu + 7) / 8;
  const int need = (units + 7) / 8;
  return 8 * (need < per_xcd ? need : per_xcd);
}

}  // namespace attn

extern "C" {

int attn_profile_start(void) {
  std::lock_guard<std::mutex> lk(attn::g_mu);
  attn::destroy_all_locked();
  attn::g_pool.reserve(attn::kPoolEvents);
  for (int i = 0; i < attn::kPoolEvents; ++i) {
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess) break;   // launches create what the pool lacks
    attn::g_pool.push_back(ev);
  }
  attn::g_on.store(true, std::memory_order_release);
  return ATTN_OK;
}

int attn_profile_stop(int64_t counts[ATTN_KERNEL_KINDS], double total_ms[ATTN_KERNEL_KINDS]) {
  attn::g_on.store(false, std::memory_order_release);
  std::lock_guard<std::mutex> lk(attn::g_mu);
  int status = ATTN_OK;
  for (int i = 0; i < ATTN_KERNEL_KINDS; ++i) {
    if (counts) counts[i] = 0;
    if (total_ms) total_ms[i] = 0.0;
  }
  for (auto& r : attn::g_recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) {
      status = ATTN_ERR_HIP;
    } else if (r.kind >= 0 && r.kind < ATTN_KERNEL_KINDS) {
      if (counts) counts[r.kind] += 1;
      if (total_ms) total_ms[r.kind] += ms;
    }
  }
  attn::destroy_all_locked();
  return status;
}

}  // extern "C"
