// C ABI of the exact-attention library: argument validation (pure host code,
// no HIP call before every check has passed), then dispatch to the kernels.
#include "../../include/attn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>

#include "attn_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [p, p+n) overlap?
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na != 0 && nb != 0 && x < y + nb && y < x + na;
}

// Element count B*H*N*d, or -1 when any size is < 1 or the byte size of an
// fp32 [B,H,N,d] array would overflow int64.
int64_t checked_elems(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return -1;
  const int64_t lim = std::numeric_limits<int64_t>::max() / 8;
  int64_t x = B;
  for (int64_t f : {H, N, d}) {
    if (x > lim / f) return -1;
    x *= f;
  }
  return x;
}

int check_common(int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype) {
  const int64_t elems = checked_elems(B, H, N, d);
  if (elems < 0) return ATTN_ERR_BAD_SHAPE;
  // grid sizes: B*H*ceil(N/64) work units must fit the launch limits
  if (B * H > (int64_t)1 << 24 || N > (int64_t)1 << 24 || B * H * ((N + 63) / 64) > (int64_t)INT32_MAX)
    return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP16) return ATTN_ERR_BAD_DTYPE;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_ERR_BAD_SCALE;
  return ATTN_OK;
}

// A caller-supplied [B, H, N, d] layout (element strides, d contiguous):
// strides non-negative and multiples of 8 (every row 16-byte aligned when the
// base is), token stride below 2^24 (copy offsets of a 128-row tile stay
// within 32 bits), batch and head strides below 2^40.
bool lay_ok(const attn::Lay& l) {
  const int64_t big = (int64_t)1 << 40;
  return l.sb >= 0 && l.sh >= 0 && l.sn >= 0 && l.sb < big && l.sh < big && l.sn < (1 << 24) && l.sb % 8 == 0 &&
         l.sh % 8 == 0 && l.sn % 8 == 0;
}

// Bytes from the base to the end of the last element of a layout.
size_t lay_extent(const attn::Lay& l, int64_t B, int64_t H, int64_t N, int64_t d) {
  return (size_t)((B - 1) * l.sb + (H - 1) * l.sh + (N - 1) * l.sn + d) * 2;
}

// No two elements of an output layout share an address: with the
// dimensions of size > 1 sorted by stride, each stride must reach past
// everything the smaller ones span (the d elements of a row included).
// An optional fourth dimension (count n4, stride s4) stands for a second
// tensor of the same layout s4 elements further on.
bool lay_injective(const attn::Lay& l, int64_t B, int64_t H, int64_t N, int64_t d, int64_t n4 = 1, int64_t s4 = 0) {
  struct Dm { int64_t n, s; } dims[4] = {{B, l.sb}, {H, l.sh}, {N, l.sn}, {n4, s4}};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (dims[j].s < dims[i].s) std::swap(dims[i], dims[j]);
  int64_t span = d;
  for (const Dm& x : dims) {
    if (x.n <= 1) continue;
    if (x.s < span) return false;
    span = x.s * (x.n - 1) + span;
  }
  return true;
}

// Two output tensors share no element: their address ranges are apart, or
// they have one layout and sit a whole number of elements apart such that
// the pair is itself an injective layout (e.g. dQ, dK, dV interleaved in one
// packed [B, N, 3, H, d] gradient buffer).
bool outputs_disjoint(const void* a, const attn::Lay& la, const void* b, const attn::Lay& lb, int64_t B, int64_t H,
                      int64_t N, int64_t d) {
  if (!overlaps(a, lay_extent(la, B, H, N, d), b, lay_extent(lb, B, H, N, d))) return true;
  if (la.sb != lb.sb || la.sh != lb.sh || la.sn != lb.sn) return false;
  const intptr_t delta = reinterpret_cast<intptr_t>(b) - reinterpret_cast<intptr_t>(a);
  if (delta % 2 != 0) return false;
  const int64_t de = (int64_t)(delta < 0 ? -delta : delta) / 2;
  return lay_injective(la, B, H, N, d, 2, de);
}

int launch_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip_error = (int)e;
  return ATTN_ERR_HIP;
}

// Forward with per-tensor layouts (lays: q, k, v, o); lse is contiguous.
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
             int64_t d, const attn::Lay* lays, float scale, int causal, int dtype, void* stream,
             const float* slopes = nullptr, const attn::DropCfg* drop = nullptr) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_PTR;
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != ATTN_OK) return st;
  for (int i = 0; i < 4; ++i)
    if (!lay_ok(lays[i])) return ATTN_ERR_BAD_LAYOUT;
  if (!lay_injective(lays[3], B, H, N, d)) return ATTN_ERR_BAD_LAYOUT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_MISALIGNED;
  const size_t lb = (size_t)(B * H * N) * 4, ob = lay_extent(lays[3], B, H, N, d);
  const void* ins[] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    const size_t ib = lay_extent(lays[i], B, H, N, d);
    if (overlaps(o, ob, ins[i], ib) || overlaps(lse, lb, ins[i], ib)) return ATTN_ERR_ALIASING;
  }
  if (overlaps(o, ob, lse, lb)) return ATTN_ERR_ALIASING;
  if (slopes && (overlaps(o, ob, slopes, (size_t)H * 4) || overlaps(lse, lb, slopes, (size_t)H * 4)))
    return ATTN_ERR_ALIASING;

  attn::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal != 0, dtype, (hipStream_t)stream,
                  lays[0], lays[1], lays[2], lays[3], slopes};
  if (drop) a.drop = *drop;
  return launch_status(attn::launch_fwd(a));
}

// Sizes of a KV-cache call: both lengths as in check_common (B*H*ceil(len/64)
// units fit a launch), plus the split grid and the merge rows.  Hkv KV heads
// serve H query heads (H a multiple of Hkv; Hkv = H without grouping).
int check_kvcache(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                  int num_splits, int64_t Hkv = -1) {
  if (Hkv == -1) Hkv = H;   // no grouping
  if (Hkv < 1 || H < 1 || H % Hkv != 0) return ATTN_ERR_BAD_SHAPE;
  int st = check_common(B, H, Nq, d, scale, dtype);
  if (st != ATTN_OK) return st;
  st = check_common(B, Hkv, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (causal && Nk < Nq) return ATTN_ERR_BAD_SHAPE;   // rows with no visible key
  if (num_splits < 0 || num_splits > 4096) return ATTN_ERR_BAD_SHAPE;
  const int64_t rows = (H / Hkv) * Nq;                // query rows per KV head
  int P = 1, chunk = 32;
  attn::kv_split_plan(B * Hkv, rows, Nk, num_splits, &P, &chunk);
  if (B * Hkv * ((rows + 31) / 32) * P > (int64_t)INT32_MAX || B * H * Nq > (int64_t)INT32_MAX - 3)
    return ATTN_ERR_BAD_SHAPE;
  if (checked_elems(B * Hkv, rows, P, d) < 0) return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}

// KV-cache forward with per-tensor layouts (lays: q, k, v, o); lse contiguous.
int kv_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t Nq,
            int64_t Nk, int64_t d, const attn::Lay* lays, float scale, int causal, int dtype, int num_splits,
            void* workspace, size_t workspace_bytes, void* stream, const float* slopes = nullptr,
            int64_t Hkv = -1, bool noalloc = false) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_PTR;
  if (Hkv == -1) Hkv = H;   // no grouping
  int st = check_kvcache(B, H, Nq, Nk, d, scale, causal, dtype, num_splits, Hkv);
  if (st != ATTN_OK) return st;
  for (int i = 0; i < 4; ++i)
    if (!lay_ok(lays[i])) return ATTN_ERR_BAD_LAYOUT;
  if (!lay_injective(lays[3], B, H, Nq, d)) return ATTN_ERR_BAD_LAYOUT;
  int P = 1, chunk = 32;
  attn::kv_split_plan(B * Hkv, (H / Hkv) * Nq, Nk, num_splits, &P, &chunk);
  const size_t need = attn::kv_acc_bytes(B * H, Nq, P, d) + attn::kv_stat_bytes(B * H, Nq, P);
  if (noalloc) {
    // the library's static buffer stands in for the workspace (no caller
    // memory to check it against)
    if (need > ATTN_KV_SCRATCH_BYTES) return ATTN_ERR_SCRATCH_TOO_SMALL;
  } else if (!workspace || workspace_bytes < need) {
    return ATTN_ERR_WORKSPACE_TOO_SMALL;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (!noalloc && (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return ATTN_ERR_MISALIGNED;
  const size_t lb = (size_t)(B * H * Nq) * 4;
  struct R { const void* p; size_t n; };
  const R ins[] = {{q, lay_extent(lays[0], B, H, Nq, d)}, {k, lay_extent(lays[1], B, Hkv, Nk, d)},
                   {v, lay_extent(lays[2], B, Hkv, Nk, d)}, {slopes, slopes ? (size_t)H * 4 : 0}};
  const R outs[] = {{o, lay_extent(lays[3], B, H, Nq, d)}, {lse, lb}, {noalloc ? nullptr : workspace, noalloc ? 0 : need}};
  for (const R& x : outs) {
    for (const R& y : ins)
      if (overlaps(x.p, x.n, y.p, y.n)) return ATTN_ERR_ALIASING;
    for (const R& y : outs)
      if (&x != &y && overlaps(x.p, x.n, y.p, y.n)) return ATTN_ERR_ALIASING;
  }
  if (noalloc) {   // every check has passed: now the first HIP call
    const hipError_t e = attn::kv_scratch_address(&workspace);
    if (e != hipSuccess) return launch_status(e);
  }
  char* ws = (char*)workspace;
  attn::KvArgs a{q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal != 0, dtype, P, chunk,
                 (float*)ws, (float*)(ws + attn::kv_acc_bytes(B * H, Nq, P, d)), (hipStream_t)stream,
                 lays[0], lays[1], lays[2], lays[3], slopes, Hkv};
  return launch_status(attn::launch_kvcache(a));
}

size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  // the padded length (N rounded up to 64) must not overflow either
  if (checked_elems(B, H, N, d) < 0 || checked_elems(B, H, attn::bwd_padded_n(N), d) < 0 || (d != 64 && d != 128))
    return 0;
  return 2 * attn::bwd_delta_bytes(B, H, N) + 3 * attn::bwd_tcopy_bytes(B, H, N, d) +
         4 * attn::bwd_tail_bytes(B, H, N, d);
}

// Backward with per-tensor layouts (lays: q, k, v, o, dO, dq, dk, dv); lse
// contiguous.  strided: the workspace also holds contiguous copies of q, k,
// v and dO, written by the preprocess.
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, const attn::Lay* lays,
             bool strided, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
             void* stream, const float* slopes = nullptr, const attn::DropCfg* drop = nullptr) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL_PTR;
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != ATTN_OK) return st;
  for (int i = 0; i < 8; ++i)
    if (!lay_ok(lays[i])) return ATTN_ERR_BAD_LAYOUT;
  for (int i = 5; i < 8; ++i)
    if (!lay_injective(lays[i], B, H, N, d)) return ATTN_ERR_BAD_LAYOUT;
  const size_t base_need = bwd_workspace_bytes(B, H, N, d);
  if (base_need == 0) return ATTN_ERR_BAD_SHAPE;
  const size_t cb = attn::align256((size_t)(B * H * N * d) * 2);   // one contiguous copy
  const size_t need = base_need + (strided ? 4 * cb : 0);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(lse) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return ATTN_ERR_MISALIGNED;
  const size_t lb = (size_t)(B * H * N) * 4;
  struct R { const void* p; size_t n; };
  const R ins[] = {{q, lay_extent(lays[0], B, H, N, d)},  {k, lay_extent(lays[1], B, H, N, d)},
                   {v, lay_extent(lays[2], B, H, N, d)},  {o, lay_extent(lays[3], B, H, N, d)},
                   {dO, lay_extent(lays[4], B, H, N, d)}, {lse, lb}, {slopes, slopes ? (size_t)H * 4 : 0}};
  const R outs[] = {{dq, lay_extent(lays[5], B, H, N, d)}, {dk, lay_extent(lays[6], B, H, N, d)},
                    {dv, lay_extent(lays[7], B, H, N, d)}, {workspace, need}};
  for (int i = 0; i < 4; ++i) {
    for (const R& y : ins)
      if (overlaps(outs[i].p, outs[i].n, y.p, y.n)) return ATTN_ERR_ALIASING;
    if (i < 3 && overlaps(outs[i].p, outs[i].n, workspace, need)) return ATTN_ERR_ALIASING;
  }
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (!outputs_disjoint(outs[i].p, lays[5 + i], outs[j].p, lays[5 + j], B, H, N, d)) return ATTN_ERR_ALIASING;

  char* ws = (char*)workspace;
  const size_t sb = attn::bwd_delta_bytes(B, H, N), t0 = 2 * sb, tcb = attn::bwd_tcopy_bytes(B, H, N, d);
  const size_t tl0 = t0 + 3 * tcb, tlb = attn::bwd_tail_bytes(B, H, N, d);
  char* tail = tlb ? ws + tl0 : nullptr;
  attn::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal != 0, dtype,
                  (float*)ws, (float*)(ws + sb), ws + t0, ws + t0 + tcb, ws + t0 + 2 * tcb,
                  tail, tail ? tail + tlb : nullptr, tail ? tail + 2 * tlb : nullptr, tail ? tail + 3 * tlb : nullptr,
                  (hipStream_t)stream, strided, lays[0], lays[1], lays[2], lays[3], lays[4], lays[5], lays[6],
                  lays[7], nullptr, nullptr, nullptr, nullptr, slopes};
  if (drop) a.drop = *drop;
  if (strided) {
    char* cp = ws + base_need;
    a.qc = cp;
    a.kc = cp + cb;
    a.vc = cp + 2 * cb;
    a.doc = cp + 3 * cb;
  }
  return launch_status(attn::launch_bwd(a));
}

// ALiBi slopes: a device array of H fp32, 4-byte aligned.
int check_slopes(const float* slopes) {
  if (!slopes) return ATTN_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(slopes) & 3u) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

// Dropout threshold t = floor(256 p + 1/2), or -1 when p is not one of the
// probabilities the 8-bit draws can realise to within half a step: NaN,
// p < 0, p > 0 that rounds to t = 0 (p < 1/512), and p that rounds to
// t = 256 (p >= 511/512).
int drop_threshold(float p) {
  if (!(p >= 0.f && p < 1.f)) return -1;
  const int t = (int)std::floor(256.0 * (double)p + 0.5);
  if (t > 255 || (t == 0 && p > 0.f)) return -1;
  return t;
}

int make_drop(float p, uint64_t seed, uint32_t offset, attn::DropCfg* c) {
  const int t = drop_threshold(p);
  if (t < 0) return ATTN_ERR_BAD_DROPOUT;
  c->t = (uint32_t)t;
  c->key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  c->key1 = (uint32_t)(seed >> 32);
  c->offset = offset;
  c->keep_scale = (float)(256.0 / (256 - t));
  c->log2_keep_scale = (float)std::log2(256.0 / (256 - t));
  return ATTN_OK;
}

attn::Lay lay_from(const int64_t* s) { return attn::Lay{s[0], s[1], (int32_t)std::min<int64_t>(s[2], INT32_MAX), 0}; }

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
             int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  if (checked_elems(B, H, N, d) < 0) return ATTN_ERR_BAD_SHAPE;
  const attn::Lay c = attn::contiguous_lay(H, N, d);
  const attn::Lay lays[4] = {c, c, c, c};
  return fwd_impl(q, k, v, o, lse, B, H, N, d, lays, scale, causal, dtype, stream);
}

int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t N, int64_t d, const int64_t* strides, float scale, int causal, int dtype, void* stream) {
  if (!strides) return ATTN_ERR_NULL_PTR;
  for (int i = 0; i < 12; ++i)
    if (strides[i] < 0 || strides[i] > ((int64_t)1 << 40)) return ATTN_ERR_BAD_LAYOUT;
  const attn::Lay lays[4] = {lay_from(strides), lay_from(strides + 3), lay_from(strides + 6), lay_from(strides + 9)};
  return fwd_impl(q, k, v, o, lse, B, H, N, d, lays, scale, causal, dtype, stream);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return bwd_workspace_bytes(B, H, N, d);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
             int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (checked_elems(B, H, N, d) < 0) return ATTN_ERR_BAD_SHAPE;
  const attn::Lay c = attn::contiguous_lay(H, N, d);
  const attn::Lay lays[8] = {c, c, c, c, c, c, c, c};
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, lays, false, scale, causal, dtype, workspace,
                  workspace_bytes, stream);
}

size_t attn_bwd_strided_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  const size_t base = attn_bwd_workspace_bytes(B, H, N, d);
  return base ? base + 4 * attn::align256((size_t)(B * H * N * d) * 2) : 0;
}

int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                     void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* strides,
                     float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!strides) return ATTN_ERR_NULL_PTR;
  for (int i = 0; i < 24; ++i)
    if (strides[i] < 0 || strides[i] > ((int64_t)1 << 40)) return ATTN_ERR_BAD_LAYOUT;
  attn::Lay lays[8];
  for (int i = 0; i < 8; ++i) lays[i] = lay_from(strides + 3 * i);
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, lays, true, scale, causal, dtype, workspace,
                  workspace_bytes, stream);
}

int attn_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t N, int64_t d, const float* alibi_slopes, float scale, int causal, int dtype, void* stream) {
  if (checked_elems(B, H, N, d) < 0) return ATTN_ERR_BAD_SHAPE;
  const int st = check_slopes(alibi_slopes);
  if (st != ATTN_OK) return st;
  const attn::Lay c = attn::contiguous_lay(H, N, d);
  const attn::Lay lays[4] = {c, c, c, c};
  return fwd_impl(q, k, v, o, lse, B, H, N, d, lays, scale, causal, dtype, stream, alibi_slopes);
}

int attn_bwd_alibi(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, const float* alibi_slopes,
                   float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (checked_elems(B, H, N, d) < 0) return ATTN_ERR_BAD_SHAPE;
  const int st = check_slopes(alibi_slopes);
  if (st != ATTN_OK) return st;
  const attn::Lay c = attn::contiguous_lay(H, N, d);
  const attn::Lay lays[8] = {c, c, c, c, c, c, c, c};
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, lays, false, scale, causal, dtype, workspace,
                  workspace_bytes, stream, alibi_slopes);
}

int attn_fwd_kvcache_alibi(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                           int64_t Nq, int64_t Nk, int64_t d, const float* alibi_slopes, float scale, int causal,
                           int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (checked_elems(B, H, Nq, d) < 0 || checked_elems(B, H, Nk, d) < 0) return ATTN_ERR_BAD_SHAPE;
  const int st = check_slopes(alibi_slopes);
  if (st != ATTN_OK) return st;
  const attn::Lay cq = attn::contiguous_lay(H, Nq, d), ck = attn::contiguous_lay(H, Nk, d);
  const attn::Lay lays[4] = {cq, ck, ck, cq};
  return kv_impl(q, k, v, o, lse, B, H, Nq, Nk, d, lays, scale, causal, dtype, num_splits, workspace,
                 workspace_bytes, stream, alibi_slopes);
}

size_t attn_fwd_kvcache_gqa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                                            int num_splits) {
  if (Hkv < 1) return 0;
  if (check_kvcache(B, Hq, Nq, Nk, d, 1.0f, 0, ATTN_DTYPE_BF16, num_splits, Hkv) != ATTN_OK) return 0;
  int P = 1, chunk = 32;
  attn::kv_split_plan(B * Hkv, (Hq / Hkv) * Nq, Nk, num_splits, &P, &chunk);
  return attn::kv_acc_bytes(B * Hq, Nq, P, d) + attn::kv_stat_bytes(B * Hq, Nq, P);
}

int attn_fwd_kvcache_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, const float* alibi_slopes, float scale,
                         int causal, int dtype, int num_splits, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (Hkv < 1 || checked_elems(B, Hq, Nq, d) < 0 || checked_elems(B, Hkv, Nk, d) < 0) return ATTN_ERR_BAD_SHAPE;
  if (alibi_slopes && (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u)) return ATTN_ERR_MISALIGNED;
  const attn::Lay cq = attn::contiguous_lay(Hq, Nq, d), ck = attn::contiguous_lay(Hkv, Nk, d);
  const attn::Lay lays[4] = {cq, ck, ck, cq};
  return kv_impl(q, k, v, o, lse, B, Hq, Nq, Nk, d, lays, scale, causal, dtype, num_splits, workspace,
                 workspace_bytes, stream, alibi_slopes, Hkv);
}

size_t attn_fwd_kvcache_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int num_splits) {
  if (check_kvcache(B, H, Nq, Nk, d, 1.0f, 0, ATTN_DTYPE_BF16, num_splits) != ATTN_OK) return 0;
  int P = 1, chunk = 32;
  attn::kv_split_plan(B * H, Nq, Nk, num_splits, &P, &chunk);
  return attn::kv_acc_bytes(B * H, Nq, P, d) + attn::kv_stat_bytes(B * H, Nq, P);
}

int attn_fwd_kvcache_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int num_splits) {
  if (check_kvcache(B, H, Nq, Nk, d, 1.0f, 0, ATTN_DTYPE_BF16, num_splits) != ATTN_OK) return 0;
  int P = 1, chunk = 32;
  attn::kv_split_plan(B * H, Nq, Nk, num_splits, &P, &chunk);
  return P;
}

int attn_fwd_kvcache(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype, int num_splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (checked_elems(B, H, Nq, d) < 0 || checked_elems(B, H, Nk, d) < 0) return ATTN_ERR_BAD_SHAPE;
  const attn::Lay cq = attn::contiguous_lay(H, Nq, d), ck = attn::contiguous_lay(H, Nk, d);
  const attn::Lay lays[4] = {cq, ck, ck, cq};
  return kv_impl(q, k, v, o, lse, B, H, Nq, Nk, d, lays, scale, causal, dtype, num_splits, workspace,
                 workspace_bytes, stream);
}

int attn_fwd_kvcache_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                             int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                             int num_splits, void* stream) {
  if (checked_elems(B, H, Nq, d) < 0 || checked_elems(B, H, Nk, d) < 0) return ATTN_ERR_BAD_SHAPE;
  const attn::Lay cq = attn::contiguous_lay(H, Nq, d), ck = attn::contiguous_lay(H, Nk, d);
  const attn::Lay lays[4] = {cq, ck, ck, cq};
  return kv_impl(q, k, v, o, lse, B, H, Nq, Nk, d, lays, scale, causal, dtype, num_splits, nullptr, 0, stream,
                 nullptr, -1, true);
}

int attn_fwd_kvcache_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                             int64_t Nq, int64_t Nk, int64_t d, const int64_t* strides, float scale, int causal,
                             int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!strides) return ATTN_ERR_NULL_PTR;
  for (int i = 0; i < 12; ++i)
    if (strides[i] < 0 || strides[i] > ((int64_t)1 << 40)) return ATTN_ERR_BAD_LAYOUT;
  const attn::Lay lays[4] = {lay_from(strides), lay_from(strides + 3), lay_from(strides + 6), lay_from(strides + 9)};
  return kv_impl(q, k, v, o, lse, B, H, Nq, Nk, d, lays, scale, causal, dtype, num_splits, workspace,
                 workspace_bytes, stream);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE: return "B, H and N must be >= 1 and the sizes must not overflow";
    case ATTN_ERR_UNSUPPORTED_HEAD_DIM: return "head dimension d must be 64 or 128";
    case ATTN_ERR_BAD_DTYPE: return "dtype must be ATTN_DTYPE_BF16 (0) or ATTN_DTYPE_FP16 (1)";
    case ATTN_ERR_MISALIGNED: return "pointers must be 16-byte aligned (workspace 256-byte aligned)";
    case ATTN_ERR_UNSUPPORTED_SEQLEN: return "unsupported sequence length (reserved; not returned)";
    case ATTN_ERR_BAD_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace is NULL or smaller than attn_bwd_workspace_bytes()";
    case ATTN_ERR_ALIASING: return "an output overlaps an input or another output";
    case ATTN_ERR_HIP: return "a HIP kernel launch failed (see attn_last_hip_error())";
    case ATTN_ERR_BAD_LAYOUT:
      return "strides must be >= 0 and multiples of 8 elements (token stride < 2^24), and an output's elements "
             "must not overlap";
    case ATTN_ERR_BAD_DROPOUT: return "dropout_p must be 0 or lie in [1/512, 511/512)";
    case ATTN_ERR_SCRATCH_TOO_SMALL: return "the call needs more split partials than ATTN_KV_SCRATCH_BYTES holds";
    default: return "unknown status";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

int attn_dropout_threshold(float dropout_p) { return drop_threshold(dropout_p); }

int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t N, int64_t d, float scale, int causal, int dtype, float dropout_p, uint64_t seed,
                     uint32_t offset, void* stream) {
  if (checked_elems(B, H, N, d) < 0) return ATTN_ERR_BAD_SHAPE;
  attn::DropCfg c{};
  const int st = make_drop(dropout_p, seed, offset, &c);
  if (st != ATTN_OK) return st;
  const attn::Lay cl = attn::contiguous_lay(H, N, d);
  const attn::Lay lays[4] = {cl, cl, cl, cl};
  return fwd_impl(q, k, v, o, lse, B, H, N, d, lays, scale, causal, dtype, stream, nullptr, &c);
}

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                     void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     int causal, int dtype, float dropout_p, uint64_t seed, uint32_t offset, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (checked_elems(B, H, N, d) < 0) return ATTN_ERR_BAD_SHAPE;
  attn::DropCfg c{};
  const int st = make_drop(dropout_p, seed, offset, &c);
  if (st != ATTN_OK) return st;
  const attn::Lay cl = attn::contiguous_lay(H, N, d);
  const attn::Lay lays[8] = {cl, cl, cl, cl, cl, cl, cl, cl};
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, lays, false, scale, causal, dtype, workspace,
                  workspace_bytes, stream, nullptr, &c);
}

int attn_fwd_dropout_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                             int64_t H, int64_t N, int64_t d, const int64_t* strides, float scale, int causal,
                             int dtype, float dropout_p, uint64_t seed, uint32_t offset, void* stream) {
  if (!strides) return ATTN_ERR_NULL_PTR;
  for (int i = 0; i < 12; ++i)
    if (strides[i] < 0 || strides[i] > ((int64_t)1 << 40)) return ATTN_ERR_BAD_LAYOUT;
  attn::DropCfg c{};
  const int st = make_drop(dropout_p, seed, offset, &c);
  if (st != ATTN_OK) return st;
  const attn::Lay lays[4] = {lay_from(strides), lay_from(strides + 3), lay_from(strides + 6), lay_from(strides + 9)};
  return fwd_impl(q, k, v, o, lse, B, H, N, d, lays, scale, causal, dtype, stream, nullptr, &c);
}

int attn_bwd_dropout_strided(const void* q, const void* k, const void* v, const void* o, const void* dO,
                             const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                             int64_t d, const int64_t* strides, float scale, int causal, int dtype, float dropout_p,
                             uint64_t seed, uint32_t offset, void* workspace, size_t workspace_bytes, void* stream) {
  if (!strides) return ATTN_ERR_NULL_PTR;
  for (int i = 0; i < 24; ++i)
    if (strides[i] < 0 || strides[i] > ((int64_t)1 << 40)) return ATTN_ERR_BAD_LAYOUT;
  attn::DropCfg c{};
  const int st = make_drop(dropout_p, seed, offset, &c);
  if (st != ATTN_OK) return st;
  attn::Lay lays[8];
  for (int i = 0; i < 8; ++i) lays[i] = lay_from(strides + 3 * i);
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, lays, true, scale, causal, dtype, workspace,
                  workspace_bytes, stream, nullptr, &c);
}

int attn_dropout_draws(uint8_t* draws, int64_t BH, int64_t Nq, int64_t Nk, uint64_t seed, uint32_t offset,
                       void* stream) {
  if (!draws) return ATTN_ERR_NULL_PTR;
  if (BH < 1 || Nq < 1 || Nk < 1 || BH > INT32_MAX || Nq > INT32_MAX - 31 || Nk > INT32_MAX - 31 ||
      checked_elems(BH, Nq, Nk, 1) < 0)
    return ATTN_ERR_BAD_SHAPE;
  attn::DropCfg c{};
  make_drop(0.f, seed, offset, &c);
  return launch_status(attn::launch_dropout_draws(draws, BH, Nq, Nk, c, (hipStream_t)stream));
}

}  // extern "C"
