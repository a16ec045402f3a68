// Internal launch interface between the C ABI (attn_api.cpp) and the kernel
// translation units.  Arguments are already validated when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Element strides of one [B, H, N, d] tensor of 16-bit values whose last
// dimension is contiguous: element (b, h, n, c) sits at b*sb + h*sh + n*sn + c.
struct Lay {
  int64_t sb, sh;
  int32_t sn;
  int32_t unused;
};

inline Lay contiguous_lay(int64_t H, int64_t N, int64_t d) { return Lay{H * N * d, N * d, (int32_t)d, 0}; }

// One dropout draw on P, passed to kernels by value (t == 0: no dropout).
struct DropCfg {
  uint32_t t;              // drop threshold in 1/256 steps: bytes below t are dropped
  uint32_t key0;           // seed, low word
  uint32_t key1;           // seed, high word
  uint32_t offset;         // fourth counter word
  float keep_scale;        // 256 / (256 - t)
  float log2_keep_scale;   // log2 of keep_scale
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t B, H, N, d;
  float scale;
  bool causal;
  int dtype;  // 0 bf16, 1 fp16
  hipStream_t stream;
  Lay lq, lk, lv, lo;
  const float* alibi_slopes;   // [H] fp32 device array, or NULL: no position bias
  DropCfg drop;                // dropout on P (drop.t == 0: none)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t B, H, N, d;
  float scale;
  bool causal;
  int dtype;
  // workspace parts; Np = N rounded up to a multiple of 64, entries for
  // tokens N .. Np-1 are padding
  float* delta;   // [B,H,Np] fp32: -D_i = -dO_i . O_i (0 for padding)
  float* nlse;    // [B,H,Np] fp32: -lse_i / scale (-inf for padding)
  void* qt;       // [B,H,d,Np] 16-bit: Q transposed (tokens in slot order per 16, padding 0)
  void* kt;       // [B,H,d,Np] 16-bit: K transposed
  void* dot;      // [B,H,d,Np] 16-bit: dO transposed
  // [B,H,64,d] 16-bit: the last 64-token tile of Q, dO, K, V, zero past N;
  // only when N is not a multiple of 64 (else NULL and never read)
  void* qtail;
  void* dotail;
  void* ktail;
  void* vtail;
  hipStream_t stream;
  // Layouts of the eight 16-bit tensors.  When `strided`, the preprocess
  // reads q, k, v, o, dO in their layouts and writes contiguous [B,H,N,d]
  // copies of q, k, v, dO to qc, kc, vc, doc (workspace), and dq, dk, dv are
  // stored in their layouts; otherwise every tensor is contiguous and the
  // copies are NULL.
  bool strided;
  Lay lq, lk, lv, lo, ldo, ldq, ldk, ldv;
  void* qc;
  void* kc;
  void* vc;
  void* doc;
  const float* alibi_slopes;   // [H] fp32 device array, or NULL (contiguous calls only)
  DropCfg drop;                // dropout on P (drop.t == 0: none)
};

// Forward for KV-cache shapes: Nq queries against Nk keys, the key axis cut
// into `splits` ranges of `chunk` keys (a multiple of 32), each computed by
// its own wave, then merged.
struct KvArgs {
  const void* q;   // [B,H,Nq,d]
  const void* k;   // [B,H,Nk,d]
  const void* v;   // [B,H,Nk,d]
  void* o;         // [B,H,Nq,d]
  float* lse;      // [B,H,Nq]
  int64_t B, H, Nq, Nk, d;
  float scale;
  bool causal;     // query i sees keys j <= i + Nk - Nq
  int dtype;
  int splits;
  int chunk;
  float* part_acc;   // workspace [B,H,Nq,splits,d] fp32: unnormalised O of each split
  float* part_stat;  // workspace [B,H,Nq,splits,4] fp32: m (log2 units), l, rounded l, unused
  hipStream_t stream;
  Lay lq, lk, lv, lo;  // q, o: [B,H,Nq,d]; k, v: [B,Hkv,Nk,d]
  const float* alibi_slopes;   // [H] fp32 device array, or NULL
  int64_t Hkv;         // KV heads; query head h uses KV head h / (H / Hkv)
};

// Split plan: `requested` splits (0: about 1024 waves in all, i.e. one per
// SIMD of the chip, and at least 128 keys per split), then the keys per split rounded up to a multiple of 32
// and the split count recomputed from it, so that no split is empty unless
// the causal mask empties it.  A pure function of the sizes: the workspace
// size and the launch agree on it.
// For grouped heads (H query heads on Hkv KV heads) the plan is made for
// BH = B * Hkv units of G * Nq query rows, G = H / Hkv.
inline void kv_split_plan(int64_t BH, int64_t Nq, int64_t Nk, int requested, int* splits, int* chunk) {
  const int64_t units = BH * ((Nq + 31) / 32);
  int64_t P = requested;
  if (P <= 0) {
    P = (1024 + units - 1) / units;
    const int64_t cap = (Nk + 127) / 128;
    if (P > cap) P = cap;
  }
  if (P < 1) P = 1;
  if (P > 4096) P = 4096;
  int64_t c = (Nk + P - 1) / P;
  c = (c + 31) / 32 * 32;
  *chunk = (int)c;
  *splits = (int)((Nk + c - 1) / c);
}

// hipLaunchKernel, or an event-timed launch while a profiling window is open;
// kind is an attn_kernel_kind value.
hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream, int kind);

// Grid of a persistent kernel: as many workgroups of `block` threads as fit
// on the device at once, rounded to a multiple of 8 (one share per XCD), and
// no more than `units` work units need.
int persistent_grid(const void* fn, int block, int units);

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_kvcache(const KvArgs& a);
// Device address, on the current device, of the library's static scratch
// buffer (ATTN_KV_SCRATCH_BYTES bytes, 256-byte aligned) for the
// no-allocation KV-cache entry point; looked up once per device.
hipError_t kv_scratch_address(void** ptr);
hipError_t launch_dropout_draws(uint8_t* out, int64_t BH, int64_t Nq, int64_t Nk, const DropCfg& drop,
                                hipStream_t stream);

// Workspace split used by attn_bwd: delta, nlse, then Q^T, K^T, dO^T, then
// (N not a multiple of 64) the tail tiles of Q, dO, K, V, each part starting
// on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t bwd_padded_n(int64_t N) { return (N + 63) / 64 * 64; }
inline size_t bwd_delta_bytes(int64_t B, int64_t H, int64_t N) {
  return align256((size_t)(B * H * bwd_padded_n(N)) * 4);
}
inline size_t bwd_tcopy_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return align256((size_t)(B * H * bwd_padded_n(N) * d) * 2);
}
inline size_t kv_acc_bytes(int64_t BH, int64_t Nq, int splits, int64_t d) {
  return align256((size_t)(BH * Nq * splits * d) * 4);
}
inline size_t kv_stat_bytes(int64_t BH, int64_t Nq, int splits) {
  return align256((size_t)(BH * Nq * splits) * 16);
}
inline size_t bwd_tail_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return N % 64 ? align256((size_t)(B * H * 64 * d) * 2) : 0;
}

}  // namespace attn
