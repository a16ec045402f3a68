// Forward pass for KV-cache shapes on gfx950: Nq new queries (decoding, a
// few speculative tokens) against Nk cached keys and values, Nq << Nk.
//
// Method: the same exact attention as the square forward (blockwise softmax
// with a running max and denominator, page "突破单卡显存极限：FlashAttention-2
// 技术解析与实战指南" §2.1), with the keys and values of earlier positions
// reused from the cache (page "FlashAttention技术解析 如何让GPT训练速度提升5-9倍"
// §4.1).  With only a handful of queries per head the work is one pass over
// K and V, so it is bound by HBM bandwidth, and a grid over (batch, head,
// query block) alone would leave most compute units idle.  The key axis is
// therefore split as well: the online-softmax state (running max m, the sum
// of the weights l, the weighted sum of V rows) of disjoint key ranges
// merges exactly, by rescaling each part with exp(m_part - m_max).
//
//  * kv_split_kernel: one wave per (batch*head, 32-query block, key split).
//    The wave streams its key range in 32-key blocks through its own two LDS
//    buffers (direct global->LDS copies, next block in flight while the
//    current one is used; no barriers, since no other wave reads them) and
//    runs the square forward's per-block step: S^T = K Q^T and O^T += V^T P^T
//    on v_mfma_f32_32x32x16, softmax in registers.  It writes its unnormalised
//    O^T rows and (m, l, l_rounded) per query to a workspace.
//  * kv_merge_kernel: one workgroup per query row combines the splits and
//    writes O (normalised by the merged sum of the rounded weights, as in the
//    square forward) and the natural-log lse.
//
// Causal alignment for Nq != Nk: query i is position Nk - Nq + i of the
// sequence, so it sees keys j <= i + Nk - Nq.  The ALIBI instantiation adds
// the linear position bias -m_h |position - j| to the scores before the row
// max (the ALiBi entry point of the C ABI).
#include <mutex>

#include "../../include/attn.h"
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// How far the running max may trail the row max (log2 units) before O, l
// and lse are rescaled.  A weight taken against a stale max is not exactly 1
// at the row's largest score, and rounding it to 16 bits for the P V product
// then puts up to half an ulp of the dominant weight into O; bf16 weights
// keep the max exact, fp16 weights (three more bits) take a slack of 2^8.
template <typename E>
constexpr float rescale_slack() {
  return std::is_same<E, f16_t>::value ? 8.0f : 0.0f;
}

template <int D>
struct KvTile {
  static constexpr int LK = D + 8;              // K row (elements): 16-byte reads, rows 4 banks apart
  static constexpr int LV = D + 32;             // V row: transpose reads, rows 16 banks apart
  static constexpr int KSL = LK / 8, VSL = LV / 8;   // 16-byte slots per row
  static constexpr int KI = (32 * KSL + 63) / 64;     // 64-slot copy blocks per K block
  static constexpr int VI = (32 * VSL + 63) / 64;
  static constexpr int KSZ = KI * 512, VSZ = VI * 512;  // elements per buffer
};

// Wait until at most N of this wave's vector-memory loads are in flight.  As
// inline asm with a memory clobber, so that the compiler moves no LDS read of
// the block being waited for above it (copies are invisible to it).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename E, int D, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(64) void kv_split_kernel(const typename E::T* __restrict__ Q,
                                                      const typename E::T* __restrict__ K,
                                                      const typename E::T* __restrict__ V,
                                                      float* __restrict__ part_acc, float* __restrict__ part_stat,
                                                      Lay lq, Lay lk, Lay lv, int Hkv, int G, int Nq, int Nk, int nqb,
                                                      int P, int chunk, float scale_log2,
                                                      const float* __restrict__ slopes) {
  using T = typename E::T;
  using v8 = typename E::v8;
  using Tl = KvTile<D>;
  constexpr int KS = D / 16;   // reduction steps over d for S
  constexpr int DB = D / 32;   // 32-wide d blocks of O^T
  constexpr int LK = Tl::LK, LV = Tl::LV, KSL = Tl::KSL, VSL = Tl::VSL, KI = Tl::KI, VI = Tl::VI;

  __shared__ __attribute__((aligned(16))) T lds_k[2][Tl::KSZ];
  __shared__ __attribute__((aligned(16))) T lds_v[2][Tl::VSZ];

  const int lane = threadIdx.x;
  const int h = lane >> 5;
  const int r = lane & 31;
  const int p = (int)(blockIdx.x % (unsigned)P);
  const int rest = (int)(blockIdx.x / (unsigned)P);
  const int qb = rest % nqb;
  const int bhk = rest / nqb;  // batch * Hkv + KV head
  const int shift = Nk - Nq;   // causal: query q sees keys <= q + shift
  // Rows of the 32-row query tile are (query head in the group, query)
  // pairs t = g * Nq + q, so the G query heads that share this K and V are
  // computed from one pass over them; with G = 1 a row is just a query.
  const int npair = G * Nq;
  const int t0 = qb * 32, t1 = min(npair, t0 + 32) - 1;
  const bool wraps = t1 - t0 + 1 >= Nq || t0 % Nq > t1 % Nq;
  const int qmin = wraps ? 0 : t0 % Nq, qmax = wraps ? Nq - 1 : t1 % Nq;
  const int trow = t0 + r;                    // this lane's pair
  const bool row_valid = trow < npair;
  const int qg = row_valid ? trow / Nq : 0, qq = row_valid ? trow % Nq : 0;

  // keys this query block may see, and this split's share of them
  const int kvis = CAUSAL ? min(Nk, qmax + shift + 1) : Nk;
  const int k_beg = p * chunk;
  const int k_end = min(kvis, k_beg + chunk);
  const int nblk = k_end > k_beg ? (k_end - k_beg + 31) / 32 : 0;

  const int bi = bhk / Hkv, hk = bhk - bi * Hkv;   // batch and KV head of this unit
  const int hq = hk * G + qg;                        // this lane's query head
  const T* Kh = K + (bi * lk.sb + hk * lk.sh);
  const T* Vh = V + (bi * lv.sb + hk * lv.sh);
  // ALiBi: score bias -slope * |query position - key position|, in log2 units
  // (the slope of this lane's query head)
  const float nslope2 = ALIBI ? -slopes[hq] * kLog2e : 0.f;
  float alibi_k[16];   // causal ALiBi: the per-slot part of the bias, -nslope2 * (4h + c_j)
#pragma unroll
  for (int j = 0; j < 16; ++j) alibi_k[j] = ALIBI && CAUSAL ? -nslope2 * (float)(4 * h + 8 * (j / 4) + j % 4) : 0.f;

  // per-lane copy offsets (bytes) inside a 32-row block; padding slots at a
  // row's end duplicate its last chunk, slots past row 31 duplicate row 31
  unsigned koff[KI], voff[VI];
  int krow[KI], vrow[VI];
#pragma unroll
  for (int c = 0; c < KI; ++c) {
    const int sl = 64 * c + lane;
    const int row = min(sl / KSL, 31), col = min(sl % KSL, D / 8 - 1);
    koff[c] = (unsigned)(row * lk.sn + col * 8) * 2u;
    krow[c] = row;
  }
#pragma unroll
  for (int c = 0; c < VI; ++c) {
    const int sl = 64 * c + lane;
    const int row = min(sl / VSL, 31), col = min(sl % VSL, D / 8 - 1);
    voff[c] = (unsigned)(row * lv.sn + col * 8) * 2u;
    vrow[c] = row;
  }
  // Copy key block i of this split into buffer b.  In the split's last
  // block, rows past its end are clamped to its last key (finite duplicates,
  // masked below: the clamp takes (row - lim) row strides off the offset),
  // so no copy reads past the end of K or V.
  auto copy_block = [&](const int i, const int b) {
    const int k0 = k_beg + 32 * i;
    const char* gk = (const char*)(Kh + (size_t)k0 * lk.sn);
    const char* gv = (const char*)(Vh + (size_t)k0 * lv.sn);
    if (k0 + 32 <= k_end) {
#pragma unroll
      for (int c = 0; c < KI; ++c) lds_copy16(gk, koff[c], &lds_k[b][c * 512]);
#pragma unroll
      for (int c = 0; c < VI; ++c) lds_copy16(gv, voff[c], &lds_v[b][c * 512]);
    } else {
      const int lim = k_end - 1 - k0;
#pragma unroll
      for (int c = 0; c < KI; ++c)
        lds_copy16(gk, koff[c] - (unsigned)(max(krow[c] - lim, 0) * lk.sn) * 2u, &lds_k[b][c * 512]);
#pragma unroll
      for (int c = 0; c < VI; ++c)
        lds_copy16(gv, voff[c] - (unsigned)(max(vrow[c] - lim, 0) * lv.sn) * 2u, &lds_v[b][c * 512]);
    }
  };

  if (nblk > 0) copy_block(0, 0);

  // Q fragments (B operand of S^T = K Q^T): lane holds row (head hq, query
  // qq), d = 16 ks + 8 h .. +7; zero for rows past the last pair (their
  // results are never stored)
  v8 qf[KS];
  {
    const T* qrow = Q + (bi * lq.sb + hq * lq.sh) + (size_t)qq * lq.sn;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      v8 x = *(const v8*)(qrow + ks * 16 + 8 * h);
      qf[ks] = row_valid ? x : v8{};
    }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) materialize(qf[ks]);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  // m_run: running max (log2 units, may trail the true max by < rescale_slack<E>(),
  // -inf while the row has seen no key); l_run: sum of the fp32 weights;
  // lr_run: sum of the same weights rounded to 16 bits (those the P V product used)
  float m_run = -__builtin_inff(), l_run = 0.f, lr_run = 0.f;

  const int offK = r * LK + 8 * h;
  const int offV = (4 * h + ((lane & 15) >> 2)) * LV + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int qrow_lim = qq + shift;   // causal: last key this lane's query sees

  for (int i = 0; i < nblk; ++i) {
    const int b = i & 1;
    // block i + 1 goes to the other buffer, whose reads (block i - 1) this
    // wave has already consumed; then wait for block i's copies only
    if (i + 1 < nblk) {
      copy_block(i + 1, b ^ 1);
      wait_vmcnt<KI + VI>();
    } else {
      wait_vmcnt<0>();
    }
    const T* kl = lds_k[b] + offK;
    const T* vl = lds_v[b] + offV;
    v8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const v8*)(kl + ks * 16);
    v8 vf[2][DB];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vf[kk][db] = concat44<E>(E::tr_read(vl + kk * 16 * LV + db * 32), E::tr_read(vl + (kk * 16 + 8) * LV + db * 32));
    // ---- S^T = K Q^T
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = E::mfma32(kf[ks], qf[ks], s);
    // ---- mask: keys past the split's end; causal keys after the query's position
    const int k0 = k_beg + 32 * i;
    const bool tail = k0 + 32 > k_end;
    const bool diag = CAUSAL && k0 + 31 > qmin + shift;
    if (tail || diag) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + acc_row(j, h);
        if (key >= k_end || (CAUSAL && key > qrow_lim)) s[j] = -__builtin_inff();
      }
    }
    // ---- online softmax in the log2 domain (with ALiBi the scores first get
    // their bias: key k0 + 4h + c, c = 8(j/4) + j%4, at distance dq - c)
    // (causal: every visible key is at distance >= 0, so the bias splits into
    // the per-lane constants alibi_k and a block part bshift that enters only
    // the row max and the exponent offset)
    float bshift = 0.f;
    if constexpr (ALIBI && CAUSAL) {
      bshift = nslope2 * (float)(qq + shift - k0);
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = fmaf(s[j], scale_log2, alibi_k[j]);
    } else if constexpr (ALIBI) {
      const float dq = (float)(qq + shift - k0 - 4 * h);
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = fmaf(s[j], scale_log2, nslope2 * fabsf(dq - (float)(8 * (j / 4) + j % 4)));
    }
    float mx = fmax3(fmax3(fmax3(s[0], s[1], s[2]), fmax3(s[3], s[4], s[5]), fmax3(s[6], s[7], s[8])),
                     fmax3(fmax3(s[9], s[10], s[11]), fmax3(s[12], s[13], s[14]), s[15]), -__builtin_inff());
    mx = xhalf_max(mx);
    const float mt = ALIBI ? mx + bshift : mx * scale_log2;   // -inf when every key of the block is masked for this row
    if (__builtin_amdgcn_ballot_w64(mt > m_run + rescale_slack<E>()) != 0) {
      const float mn = fmaxf(m_run, mt);
      // equal maxima (also both -inf: a row that has seen no key yet) need no rescale
      const float alpha = mn == m_run ? 1.0f : fast_exp2(m_run - mn);
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = mn;
    }
    // a row with no visible key so far has only -inf scores: weight exp2(-inf) = 0
    float neg_m = m_run == -__builtin_inff() ? 0.0f : -m_run;
    if constexpr (ALIBI) neg_m += bshift;
    float pw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) pw[j] = fast_exp2(ALIBI ? s[j] + neg_m : fmaf(s[j], scale_log2, neg_m));
    float q4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) q4[g] = (pw[4 * g] + pw[4 * g + 1]) + (pw[4 * g + 2] + pw[4 * g + 3]);
    l_run += (q4[0] + q4[1]) + (q4[2] + q4[3]);
    v8 pf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      pf[kk] = pack8<E>(pw[8 * kk + 0], pw[8 * kk + 1], pw[8 * kk + 2], pw[8 * kk + 3], pw[8 * kk + 4],
                        pw[8 * kk + 5], pw[8 * kk + 6], pw[8 * kk + 7]);
    lr_run += sum8<E>(pf[0], 0.f) + sum8<E>(pf[1], 0.f);
    // ---- O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = E::mfma32(vf[kk][db], pf[kk], oacc[db]);
  }

  // ---- this split's partial state of each valid query row
  const float l = xhalf_sum(l_run);
  const float lr = xhalf_sum(lr_run);
  if (!row_valid) return;
  const size_t row = (((size_t)bi * Hkv * G + hq) * Nq + qq) * P + p;
  float* acc_row_ptr = part_acc + row * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      f32x4 x;
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = oacc[db][4 * jg + u];
      *(f32x4*)(acc_row_ptr + db * 32 + 8 * jg + 4 * h) = x;
    }
  if (h == 0) *(f32x4*)(part_stat + row * 4) = f32x4{m_run, l, lr, 0.f};
}

// One workgroup (four waves) per query row merges the P partial states of
// that row: the row max M over the splits first (each thread a strided share
// of the splits, then a tree over the workgroup), then wave w sums splits
// w, w + 4, ... with weights 2^(m_p - M), every lane over its own elements of
// the row, eight splits' loads in flight at a time; the four waves' sums are
// added through LDS.
template <typename E, int D>
__global__ __launch_bounds__(256) void kv_merge_kernel(const float* __restrict__ part_acc,
                                                       const float* __restrict__ part_stat,
                                                       typename E::T* __restrict__ O, float* __restrict__ LSE,
                                                       Lay lo, int H, int Nq, int P) {
  using T = typename E::T;
  constexpr int EL = D / 64;   // elements of the row per lane
  constexpr int U = 8;         // splits per batch of loads
  __shared__ float red_m[4];
  __shared__ float red_acc[4][D];
  __shared__ float red_s[4][2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t row = blockIdx.x;
  const float* st = part_stat + row * P * 4;
  const float* acc = part_acc + row * P * D + lane * EL;

  float M = -__builtin_inff();
  for (int p = tid; p < P; p += 256) M = fmaxf(M, st[4 * p]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red_m[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float num[EL], den = 0.f, lsum = 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e) num[e] = 0.f;
  for (int p0 = w; p0 < P; p0 += 4 * U) {
    float m[U], l[U], lr[U], x[U][EL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + 4 * u;
      const bool ok = p < P;
      m[u] = ok ? st[4 * p] : -__builtin_inff();
      l[u] = ok ? st[4 * p + 1] : 0.f;
      lr[u] = ok ? st[4 * p + 2] : 0.f;
#pragma unroll
      for (int e = 0; e < EL; ++e) x[u][e] = ok ? acc[(size_t)p * D + e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a split in which this row saw no key holds m = -inf and zero sums
      const float a = m[u] == -__builtin_inff() ? 0.0f : fast_exp2(m[u] - M);
      lsum = fmaf(a, l[u], lsum);
      den = fmaf(a, lr[u], den);
#pragma unroll
      for (int e = 0; e < EL; ++e) num[e] = fmaf(a, x[u][e], num[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EL; ++e) red_acc[w][lane * EL + e] = num[e];
  if (lane == 0) {
    red_s[w][0] = den;
    red_s[w][1] = lsum;
  }
  __syncthreads();
  if (w != 0) return;
  den = (red_s[0][0] + red_s[1][0]) + (red_s[2][0] + red_s[3][0]);
  lsum = (red_s[0][1] + red_s[1][1]) + (red_s[2][1] + red_s[3][1]);
  const float inv = 1.0f / den;
  const int qi = (int)(row % (unsigned)Nq), bh = (int)(row / (unsigned)Nq);
  const int bi = bh / H, hi = bh - bi * H;
  T* orow = O + (bi * lo.sb + hi * lo.sh) + (size_t)qi * lo.sn + lane * EL;
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    const int d = lane * EL + e;
    orow[e] = (T)(((red_acc[0][d] + red_acc[1][d]) + (red_acc[2][d] + red_acc[3][d])) * inv);
  }
  if (lane == 0) LSE[row] = (M + __builtin_amdgcn_logf(lsum)) * kLn2;
}

template <typename E, int D, bool CAUSAL, bool ALIBI>
hipError_t launch_kv_cfg(const KvArgs& a) {
  const int Hkv = (int)a.Hkv, G = (int)(a.H / a.Hkv);
  const int BHk = (int)(a.B * a.Hkv);
  const int Nq = (int)a.Nq, Nk = (int)a.Nk, P = a.splits, chunk = a.chunk;
  const int nqb = (G * Nq + 31) / 32;   // 32-row tiles of (query head in group, query) pairs
  const float scale_log2 = a.scale * kLog2e;
  const typename E::T* q = (const typename E::T*)a.q;
  const typename E::T* k = (const typename E::T*)a.k;
  const typename E::T* v = (const typename E::T*)a.v;
  float* pacc = a.part_acc;
  float* pst = a.part_stat;
  Lay lq = a.lq, lk = a.lk, lv = a.lv, lo = a.lo;
  const int H = (int)a.H;
  const float* slopes = a.alibi_slopes;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&pacc, (void*)&pst, (void*)&lq, (void*)&lk, (void*)&lv,
                  (void*)&Hkv, (void*)&G, (void*)&Nq, (void*)&Nk, (void*)&nqb, (void*)&P, (void*)&chunk,
                  (void*)&scale_log2, (void*)&slopes};
  hipError_t e = launch_kernel((const void*)kv_split_kernel<E, D, CAUSAL, ALIBI>, dim3((unsigned)(BHk * nqb * P)),
                               dim3(64), args, a.stream, 4);
  if (e != hipSuccess) return e;
  const int rows = (int)(a.B * a.H) * Nq;
  typename E::T* o = (typename E::T*)a.o;
  float* lse = a.lse;
  const float* cacc = pacc;
  const float* cst = pst;
  void* margs[] = {(void*)&cacc, (void*)&cst, (void*)&o, (void*)&lse, (void*)&lo, (void*)&H, (void*)&Nq, (void*)&P};
  return launch_kernel((const void*)kv_merge_kernel<E, D>, dim3((unsigned)rows), dim3(256), margs, a.stream, 5);
}

template <typename E, int D>
hipError_t launch_kv_d(const KvArgs& a) {
  if (a.alibi_slopes) return a.causal ? launch_kv_cfg<E, D, true, true>(a) : launch_kv_cfg<E, D, false, true>(a);
  return a.causal ? launch_kv_cfg<E, D, true, false>(a) : launch_kv_cfg<E, D, false, false>(a);
}

}  // namespace

hipError_t launch_kvcache(const KvArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? launch_kv_d<bf16_t, 64>(a) : launch_kv_d<bf16_t, 128>(a);
  return a.d == 64 ? launch_kv_d<f16_t, 64>(a) : launch_kv_d<f16_t, 128>(a);
}

// Split partials of attn_fwd_kvcache_noalloc.  Each device that runs the
// library holds its own copy of this array for the life of the process.  In
// host code the name stands for a host-side shadow, not a device address:
// kernels receive the address hipGetSymbolAddress returns for the current
// device, cached per device below.
static __device__ __align__(256) unsigned char scratch[ATTN_KV_SCRATCH_BYTES];

hipError_t kv_scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidValue;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace attn
