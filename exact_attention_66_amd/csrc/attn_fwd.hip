// Forward pass of exact attention on gfx950: one workgroup per
// (batch*head, block of BM queries), K/V tiles staged through LDS,
// scores and P V on MFMA, online softmax in registers.
//
// Method: page "突破单卡显存极限：FlashAttention-2技术解析与实战指南" §2.1
// (blockwise softmax with a running row max m and denominator l, rescaled by
// exp(m_old - m_new)); page "FlashAttention-2：GPU利用率从50%干到90%"
// improvements 1-3 (grid over batch x head x query block, most work kept on
// the matrix units with the normalisation deferred to the end, each
// wavefront owning its own query rows so waves never exchange softmax state).
//
// gfx950 mapping (not the pages' A100 tiling):
//  * each wave owns 32*QB queries and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16, so a lane holds one query's scores for 16 keys per
//    32-key block: the row max is in-lane plus one permlane32 swap, and the
//    row sum needs no exchange until the epilogue;
//  * the S^T accumulator, converted to 16-bit, is directly the B operand of
//    O^T += V^T P^T (keys relabelled per slot_key), and V^T comes from LDS
//    with ds_read_b64_tr_b16, so P never leaves registers;
//  * K/V tiles reach LDS by direct global->LDS copies (no staging registers,
//    no LDS write instructions);
//  * two launch shapes, chosen per call from the work per head (see
//    launch_fwd_a): 8 waves (256 queries) per workgroup with 128-key tiles in
//    two buffers at d = 128 (64-key tiles in three at d = 64), or 4 waves
//    (128 queries) with 64-key tiles in two buffers, two workgroups per CU;
//    both walk each query row's keys in the same 32-key blocks in the same
//    order, so they give bitwise-identical results;
//  * within a tile each wave pipelines its 32-key blocks: a block's V^T
//    fragments are read before its S^T product and the next block's K
//    fragments before its P V product, so the LDS latency hides under MFMAs;
//  * exponentials use exp2 with scale*log2(e) folded into one FMA, and the
//    O rescale is skipped while the running max grows by less than 2^8
//    (exact: the same stale max is used for O, l and lse) unless, with bf16
//    weights, the new largest weight would carry a large share of the row
//    (kDominantFraction); row max and sums are trees rather than dependent
//    chains;
//  * causal launches order work units heaviest query block first;
//  * any N: rows past the end are neither read nor stored, and the last
//    tile's keys past the end are masked (the TAIL instantiation, chosen
//    when N is not a multiple of 64, so that other launches pay nothing);
//  * every tensor is addressed through its own (batch, head, token) strides
//    with a contiguous head dimension, so any such layout is read in place;
//  * the ALIBI instantiation adds the linear position bias
//    -m_h |i - j| (page "FlashAttention技术解析 如何让GPT训练速度提升5-9倍"
//    §4.1 names ALiBi) to the scores before the row max;
//  * the DROP instantiation zeroes the dropped 16-bit weights of P after
//    the row sums are taken (the softmax and lse are those of all keys) and
//    scales O by 256 / (256 - t) in the epilogue; each lane draws one
//    generator call per 32-key block (attn_dropout.h).
#include <cstdlib>

#include "attn_device.h"
#include "attn_dropout.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// Lazy rescale.  The running max m may trail the true row max by up to
// kRescaleSlack (log2 units) before O, l and lse are rescaled: the same
// stale max serves all three, so the result is exact up to rounding.  But a
// weight exp2(s - m) taken against a stale max is no longer exactly 1 at
// the row's largest score, and rounding it to 16 bits for the P V product
// costs up to half an ulp of that weight; where one key carries most of a
// row's weight this shows up in O (at bf16, on top of the output's own
// rounding, enough to exceed 1e-2 at |O| in [2, 4)).  So with bf16 weights
// (8 significant bits) the max is also made exact whenever the block's
// largest weight against the stale max would exceed kDominantFraction (1/8) of
// the row's sum so far: every key that is not rounded as exactly 1 then
// ends up with less than that fraction of the row's weight, and its
// rounding error in O stays below 2^-9 kDominantFraction |V - O|.  The
// test compares the growth of the max, log2 of that weight, with a lower
// bound of log2(kDominantFraction l) taken from the exponent bits of l (full-
// rate instructions; the bound only makes the rescale more frequent).  fp16
// weights (11 bits) make the effect 8x smaller and skip the check.
#ifndef ATTN_FWD_SLACK
#define ATTN_FWD_SLACK 8.0f
#endif
#ifndef ATTN_FWD_DOMINANT_LOG2
#define ATTN_FWD_DOMINANT_LOG2 (-3.0f)   // kDominantFraction = 1/8
#endif
constexpr float kRescaleSlack = ATTN_FWD_SLACK;
constexpr float kLog2DominantFraction = ATTN_FWD_DOMINANT_LOG2;
template <typename E>
constexpr bool exact_dominant_weight() {
  return !std::is_same<E, f16_t>::value && kLog2DominantFraction < 0.0f;
}

#ifndef ATTN_FWD_COPY_AT
#define ATTN_FWD_COPY_AT (-1)  // key block after which the next tile's copy goes out; -1: 1 if causal, else 0
#endif
#ifndef ATTN_FWD_QB
#define ATTN_FWD_QB 1    // 32-query blocks per wave
#endif
#ifndef ATTN_FWD_NW
#define ATTN_FWD_NW 0    // waves per workgroup: 0 chooses 4 or 8 per call (launch_fwd_a)
#endif
#ifndef ATTN_FWD_BN
#define ATTN_FWD_BN 0    // keys per LDS tile of the 8-wave shape; 0: 128 for d = 128, 64 for d = 64
#endif
#ifndef ATTN_FWD_NBUF
#define ATTN_FWD_NBUF 0  // LDS tile buffers; 0: three for 64-key tiles at 8 waves, else two
#endif
#ifndef ATTN_FWD_MINW
#define ATTN_FWD_MINW 2  // waves per SIMD the register budget is sized for
#endif
#ifndef ATTN_FWD_GRID_XCD
#define ATTN_FWD_GRID_XCD 0  // workgroup order: xcd_head_major (1) or heavy-first over all heads (0)
#endif

// LDS tiles: K [BN][D + 8] is read with ds_read_b128 by 16 lanes of 16
// consecutive rows (rows 4 banks apart: conflict free); V [BN][D + 32] is read
// with ds_read_b64_tr_b16 by 32 lanes covering 4 rows x 64 bytes (rows 16
// banks apart: the 4 rows land on 4 disjoint 16-bank groups).  Both are
// affine, so every read is one per-lane base plus an immediate offset.
template <typename E, int D, bool CAUSAL, int QB, int NW, int BN, bool TAIL, bool ALIBI, bool DROP>
__global__ __launch_bounds__(NW * 64, ATTN_FWD_MINW) void fwd_kernel(const typename E::T* __restrict__ Q,
                                                                     const typename E::T* __restrict__ K,
                                                                     const typename E::T* __restrict__ V,
                                                                     typename E::T* __restrict__ O,
                                                                     float* __restrict__ LSE, Lay lq, Lay lk,
                                                                     Lay lv, Lay lo, int H, int BH, int N,
                                                                     int nqb, float scale_log2,
                                                                     const float* __restrict__ slopes,
                                                                     DropCfg drop) {
  using T = typename E::T;
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  constexpr int BM = NW * 32 * QB;   // queries per workgroup
  constexpr int KS = D / 16;         // reduction steps over d for S
  constexpr int DB = D / 32;         // 32-wide d blocks of O^T
  constexpr int KB = BN / 32;        // 32-key blocks per tile
  constexpr int LK = D + 8;          // K tile row (elements)
  constexpr int LV = D + 32;         // V tile row (elements)
  constexpr int KSL = LK / 8;        // 16-byte slots per K row (D/8 data + padding)
  constexpr int VSL = LV / 8;        // 16-byte slots per V row
  constexpr int KI = (BN * KSL + 63) / 64;   // 64-slot copy blocks per K tile
  constexpr int VI = (BN * VSL + 63) / 64;   // 64-slot copy blocks per V tile
  constexpr int KC = (KI + NW - 1) / NW;     // blocks per wave (upper bound)
  constexpr int VC = (VI + NW - 1) / NW;
  constexpr int KSZ = KI * 64 * 8;           // elements per K tile buffer
  constexpr int VSZ = VI * 64 * 8;
  // tile t in buffer t % NBUF: with 8 waves, 64-key tiles in three buffers,
  // copied two tiles ahead, and 128-key tiles in two, copied one tile ahead;
  // with 4 waves, 64-key tiles in two
  constexpr int NBUF = ATTN_FWD_NBUF ? ATTN_FWD_NBUF : (BN == 64 && NW == 8 ? 3 : 2);

  __shared__ __attribute__((aligned(16))) T lds_k[NBUF][KSZ];
  __shared__ __attribute__((aligned(16))) T lds_v[NBUF][VSZ];

  const int tid = threadIdx.x;
  (void)tid;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int r = lane & 31;

  int qblk, bh;
#if ATTN_FWD_GRID_XCD
  xcd_head_major((int)blockIdx.x, (int)gridDim.x, nqb, bh, qblk);
  if (CAUSAL) qblk = nqb - 1 - qblk;  // heaviest query blocks of a head first
#else
  if (CAUSAL) {  // heaviest query blocks first, across all heads
    qblk = nqb - 1 - (int)(blockIdx.x / BH);
    bh = (int)(blockIdx.x % BH);
  } else {
    bh = (int)(blockIdx.x / nqb);
    qblk = (int)(blockIdx.x % nqb);
  }
#endif
  const int q0 = qblk * BM;
  const int qw0 = q0 + w * 32 * QB;
  const bool wave_valid = qw0 < N;
  const int bi = bh / H, hi = bh - bi * H;   // batch and head of this unit
  const T* Qh = Q + (bi * lq.sb + hi * lq.sh);
  const T* Kh = K + (bi * lk.sb + hi * lk.sh);
  const T* Vh = V + (bi * lv.sb + hi * lv.sh);
  // ALiBi: score bias -slope * |query position - key position|, in log2 units
  const float nslope2 = ALIBI ? -slopes[hi] * kLog2e : 0.f;
  // causal ALiBi: the per-slot part of the bias, -nslope2 * (4h + c_j)
  float alibi_k[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) alibi_k[j] = ALIBI && CAUSAL ? -nslope2 * (float)(4 * h + 8 * (j / 4) + j % 4) : 0.f;

  // Q fragments, B operand of S^T = K Q^T: lane holds Q[q = qw0+32qb+r][16ks + 8h .. +7]
  // (loaded below, while the first tile copies are in flight)
  v8 qf[QB][KS];

  f32x16 oacc[QB][DB];
  // m_run: running max (log2 units, may trail the true max by < kRescaleSlack);
  // l_run: sum of the fp32 exponentials (gives lse); lr_run: sum of the same
  // exponentials after rounding to 16 bits, i.e. of the weights the P V
  // product really used, so that O is normalised by exactly its own weights.
  float m_run[QB], l_run[QB], lr_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.f;
    lr_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  }

  // per-lane parts of the LDS read addresses (elements)
  const int offK = opaque(r * LK + 8 * h);
  const int offV = opaque((4 * h + ((lane & 15) >> 2)) * LV + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int q_last = qw0 + 32 * QB - 1;

  // Tiles reach LDS by direct global->LDS copies: a copy instruction fills
  // 64 consecutive 16-byte slots, so the padding slots at the end of each
  // row get duplicates of the row's last chunk and a tile is a whole number
  // of 64-slot blocks.  Per-lane byte offsets are the same for every tile.
  const int wu = wave_id() & (NW - 1);
  unsigned koff[KC], voff[VC];
  int krow[TAIL ? KC : 1], vrow[TAIL ? VC : 1];   // rows of the copies, for the tail clamp
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int sl = 64 * (wu + NW * c) + lane;
    const int row = min(sl / KSL, BN - 1);
    const int col = min(sl % KSL, D / 8 - 1);
    koff[c] = (unsigned)(row * lk.sn + col * 8) * 2u;
    if constexpr (TAIL) krow[c] = row;
  }
#pragma unroll
  for (int c = 0; c < VC; ++c) {
    const int sl = 64 * (wu + NW * c) + lane;
    const int row = min(sl / VSL, BN - 1);
    const int col = min(sl % VSL, D / 8 - 1);
    voff[c] = (unsigned)(row * lv.sn + col * 8) * 2u;
    if constexpr (TAIL) vrow[c] = row;
  }
  // Without TAIL (N a multiple of 64) only a 128-key tile can run past the
  // end of the sequence, by exactly 64 keys: it is copied as its first half,
  // since 64 rows of either layout fill whole 64-slot blocks, and its second
  // half is never read.  With TAIL (any other N) the last tile's copies clamp
  // every row to the last key, N - 1, so the rows past the end hold finite
  // duplicates that are read only under the key mask, and no copy reads
  // beyond the input.  The clamp takes (row - lim) row strides off a copy's
  // offset when its row lies past the last key.
  static_assert((64 * KSL) % 64 == 0 && (64 * VSL) % 64 == 0, "half tiles are whole blocks");
  auto clamp_row = [](unsigned off, int row, int lim, int sn) {
    return off - (unsigned)(max(row - lim, 0) * sn) * 2u;
  };
  auto copy_tile = [&](const int t, const int b) {
    const char* gk = (const char*)(Kh + (size_t)t * BN * lk.sn);
    const char* gv = (const char*)(Vh + (size_t)t * BN * lv.sn);
    if constexpr (!TAIL) {
      const bool half = t * BN + BN > N;
      const int ki = half ? 64 * KSL / 64 : KI;
      const int vi = half ? 64 * VSL / 64 : VI;
#pragma unroll
      for (int c = 0; c < KC; ++c)
        if (wu + NW * c < ki) lds_copy16(gk, koff[c], &lds_k[b][(wu + NW * c) * 512]);
#pragma unroll
      for (int c = 0; c < VC; ++c)
        if (wu + NW * c < vi) lds_copy16(gv, voff[c], &lds_v[b][(wu + NW * c) * 512]);
    } else {
      const int lim = min(N - 1 - t * BN, BN - 1);   // last row of tile t inside the sequence
#pragma unroll
      for (int c = 0; c < KC; ++c)
        if (wu + NW * c < KI) lds_copy16(gk, clamp_row(koff[c], krow[c], lim, lk.sn), &lds_k[b][(wu + NW * c) * 512]);
#pragma unroll
      for (int c = 0; c < VC; ++c)
        if (wu + NW * c < VI) lds_copy16(gv, clamp_row(voff[c], vrow[c], lim, lv.sn), &lds_v[b][(wu + NW * c) * 512]);
    }
  };
  // Wait until at most one tile's copies (the most recent) are outstanding:
  // vmcnt counts this wave's copies in issue order.
  auto wait_copies_but_last = [&]() {
    constexpr auto cnt = [](int w) {
      int n = 0;
      for (int c = 0; c < KC; ++c) n += (w + NW * c < KI);
      for (int c = 0; c < VC; ++c) n += (w + NW * c < VI);
      return n;
    };
    static_assert(NBUF == 2 || KC + VC < 16, "vmcnt immediate");
    static_assert(NW == 8 || NW == 4, "one case per wave");
    switch (wu) {
      case 0: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(1)); break;
      case 2: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(2)); break;
      case 3: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(3)); break;
      case 4: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(4)); break;
      case 5: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(5)); break;
      case 6: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(6)); break;
      default: __builtin_amdgcn_s_waitcnt(0x0F70 | cnt(7)); break;
    }
  };

  // one 32-key block: S^T, mask, online softmax, O^T += V^T P^T
  // K fragments of a 32-key block, A operand of S^T = K Q^T
  auto read_k = [&](const int buf, const int kb, v8 (&kf)[KS]) {
    const T* kl = lds_k[buf] + offK + kb * 32 * LK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const v8*)(kl + ks * 16);
  };
  // one 32-key block: S^T, mask, online softmax, O^T += V^T P^T.  The block's
  // K fragments are already in kf (read during the previous block's P V);
  // its V^T fragments are read first, to arrive during S^T; the next block's
  // K fragments are read before the P V product.
  auto key_block = [&](const int buf, const int kb, const int kbk0, v8 (&kf)[KS]) {
    const T* vl = lds_v[buf] + offV + kb * 32 * LV;
    v8 vf[2][DB];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vf[kk][db] = concat44<E>(E::tr_read(vl + kk * 16 * LV + db * 32), E::tr_read(vl + (kk * 16 + 8) * LV + db * 32));
    // DROP: this lane's generator call, issued before the MFMAs so that it
    // can overlap them, is block u = lane % 4 of the quad's four 4 x 4
    // (query, key) blocks (keys kbk0 + 8u + 4h ..); the quad transpose gives
    // each lane its own query's word of every block
    u32x4 dtw[QB];
    if constexpr (DROP) {
      const int u = lane & 3;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        dtw[qb] = quad_transpose(philox4x32_10((uint32_t)(qw0 + qb * 32 + r) >> 2,
                                               (uint32_t)((kbk0 >> 2) + 2 * u + h), (uint32_t)bh, drop.offset,
                                               drop.key0, drop.key1),
                                 u);
    }
    // ---- S^T = K Q^T
    f32x16 s[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = E::mfma32(kf[ks], qf[qb][ks], s[qb]);
    sched_fence();
    // ---- causal mask (key > query -> -inf) on blocks that cross the
    // diagonal; without it, keys past the end of the sequence are masked
    // (with it they lie above the diagonal of every stored row)
    if (TAIL && !CAUSAL && kbk0 + 32 > N) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (kbk0 + acc_row(j, h) >= N) s[qb][j] = -__builtin_inff();
    }
    if (CAUSAL && kbk0 + 31 > qw0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (kbk0 + acc_row(j, h) > qw0 + qb * 32 + r) s[qb][j] = -__builtin_inff();
    }
    // ---- online softmax (log2 domain); P is rounded to 16 bits and kept
    // packed as the B operand of the P V product.  Max and sums are trees,
    // not chains, so that the dependent latency stays short.
    v8 pf[2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // With ALiBi the scores are first taken to the log2 domain with their
      // bias (key kbk0 + 4h + c, c = 8(j/4) + j%4, at distance dq - c from
      // the query), so that the row max is over biased scores.  Causal: every
      // visible key is at distance >= 0, so the bias is nslope2 * (dq0 - 4h - c)
      // with dq0 = query - kbk0 the same in both halves of the wave; the
      // per-slot part is a per-lane constant (alibi_k) and the block part
      // bshift enters only the row max and the exponent offset.
      f32x16 x = s[qb];
      float bshift = 0.f;
      if constexpr (ALIBI && CAUSAL) {
        bshift = nslope2 * (float)(qw0 + qb * 32 + r - kbk0);
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = fmaf(x[j], scale_log2, alibi_k[j]);
      } else if constexpr (ALIBI) {
        const float dq = (float)(qw0 + qb * 32 + r - kbk0 - 4 * h);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          x[j] = fmaf(x[j], scale_log2, nslope2 * fabsf(dq - (float)(8 * (j / 4) + j % 4)));
      }
      const float m0 = fmax3(x[0], x[1], x[2]), m1 = fmax3(x[3], x[4], x[5]);
      const float m2 = fmax3(x[6], x[7], x[8]), m3 = fmax3(x[9], x[10], x[11]);
      const float m4 = fmax3(x[12], x[13], x[14]);
      float mx = fmax3(fmax3(m0, m1, m2), fmax3(m3, m4, x[15]), -__builtin_inff());
      mx = xhalf_max(mx);
      const float mt = ALIBI ? mx + bshift : mx * scale_log2;
      const float grow = mt - m_run[qb];
      bool need;
      if constexpr (exact_dominant_weight<E>()) {
        // l = f 2^e with f in [0.5, 1), so log2 l >= e - 1.  Both tests as one
        // threshold: grow > slack, or grow > 0 and grow > log2(theta) + e - 1
        const int e = __builtin_amdgcn_frexp_expf(l_run[qb]);
        need = grow > __builtin_amdgcn_fmed3f((kLog2DominantFraction - 1.0f) + (float)e, 0.0f, kRescaleSlack);
      } else {
        need = grow > kRescaleSlack;
      }
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float mn = fmaxf(m_run[qb], mt);
        const float alpha = fast_exp2(m_run[qb] - mn);
        l_run[qb] *= alpha;
        lr_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
        m_run[qb] = mn;
      }
      const float neg_m = ALIBI ? bshift - m_run[qb] : -m_run[qb];
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = fast_exp2(ALIBI ? x[j] + neg_m : fmaf(x[j], scale_log2, neg_m));
      float q4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) q4[g] = (p[4 * g] + p[4 * g + 1]) + (p[4 * g + 2] + p[4 * g + 3]);
      l_run[qb] += (q4[0] + q4[1]) + (q4[2] + q4[3]);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        pf[kk][qb] = pack8<E>(p[8 * kk + 0], p[8 * kk + 1], p[8 * kk + 2], p[8 * kk + 3], p[8 * kk + 4],
                              p[8 * kk + 5], p[8 * kk + 6], p[8 * kk + 7]);
      // one chain of dot products straight into the running sum (no zeroed partials)
      lr_run[qb] = sum8<E>(pf[1][qb], sum8<E>(pf[0][qb], lr_run[qb]));
      if constexpr (DROP) {
        const u32x4 tw = dtw[qb];
        const uint32_t add = (256u - drop.t) * 0x00010001u;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 pw = __builtin_bit_cast(u32x4, pf[kk][qb]);
          uint32_t lo, hi;
          keep_halves(tw[2 * kk], add, lo, hi);
          pw[0] &= half_masks(lo);
          pw[1] &= half_masks(hi);
          keep_halves(tw[2 * kk + 1], add, lo, hi);
          pw[2] &= half_masks(lo);
          pw[3] &= half_masks(hi);
          pf[kk][qb] = __builtin_bit_cast(v8, pw);
        }
      }
    }
    if (kb + 1 < KB) read_k(buf, kb + 1, kf);
    sched_fence();
    // ---- O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma32(vf[kk][db], pf[kk][qb], oacc[qb][db]);
  };

  copy_tile(0, 0);
  if (NBUF == 3 && ntiles > 1) copy_tile(1, 1);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = min(qw0 + qb * 32 + r, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = *(const v8*)(Qh + (size_t)q * lq.sn + ks * 16 + 8 * h);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) materialize(qf[qb][ks]);
  wait_all_vmem_loads();
  __syncthreads();

  constexpr int AHEAD = NBUF - 1;   // tiles between a copy and its use
  auto k_tile = [&](const int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    // buffer (t + AHEAD) % NBUF held tile t - 1, which every wave has finished
    // The next tile's copy goes out before the tile's first key block, or
    // (causal, and every 4-wave launch) before its second: right after the
    // barrier every wave starts the tile at once, and a copy burst there
    // stalls all of them together; one block later the waves are out of step.
    constexpr int copy_at = ATTN_FWD_COPY_AT >= 0 ? ATTN_FWD_COPY_AT : (CAUSAL || NW == 4 ? 1 : 0);
    if (copy_at == 0 && t + AHEAD < ntiles) copy_tile(t + AHEAD, (buf + AHEAD) % NBUF);
    const int k0 = t * BN;
    const bool run = wave_valid && (!CAUSAL || k0 <= q_last);
    v8 kf[KS];
    if (run) read_k(buf, 0, kf);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (copy_at > 0 && kb == copy_at && t + AHEAD < ntiles) copy_tile(t + AHEAD, (buf + AHEAD) % NBUF);
      const int kbk0 = k0 + kb * 32;
      if (run && (!CAUSAL || kbk0 <= q_last) && kbk0 < N) key_block(buf, kb, kbk0, kf);
    }
    mfma_drain();
    // tile t + 1 must be in LDS: with three buffers its copies are the ones
    // before the most recent, with two they are the most recent
    if (NBUF == 3 && t + 2 < ntiles) wait_copies_but_last();
    else wait_all_vmem_loads();
    __syncthreads();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, NBUF == 3 ? 2 : 0>;
  int t = 0;
  if constexpr (NBUF == 3) {
    for (; t + 2 < ntiles; t += 3) {
      k_tile(t, B0{});
      k_tile(t + 1, B1{});
      k_tile(t + 2, B2{});
    }
  } else {
    for (; t + 1 < ntiles; t += 2) {
      k_tile(t, B0{});
      k_tile(t + 1, B1{});
    }
  }
  if (t < ntiles) k_tile(t, B0{});
  if (NBUF == 3 && t + 1 < ntiles) k_tile(t + 1, B1{});

  if (!wave_valid) return;
  // ---- epilogue: O = acc / l, lse = (m + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = xhalf_sum(l_run[qb]);
    const float inv = (DROP ? drop.keep_scale : 1.0f) / xhalf_sum(lr_run[qb]);
    const int q = qw0 + qb * 32 + r;
    if (TAIL && q >= N) continue;   // rows past the end of the sequence
    T* orow = O + (bi * lo.sb + hi * lo.sh) + (size_t)q * lo.sn;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        v4 ov;
        ov[0] = (T)(oacc[qb][db][4 * jg + 0] * inv);
        ov[1] = (T)(oacc[qb][db][4 * jg + 1] * inv);
        ov[2] = (T)(oacc[qb][db][4 * jg + 2] * inv);
        ov[3] = (T)(oacc[qb][db][4 * jg + 3] * inv);
        *(v4*)(orow + db * 32 + 8 * jg + 4 * h) = ov;
      }
    if (h == 0) LSE[(size_t)bh * N + q] = (m_run[qb] + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

template <typename E, int D, bool CAUSAL, int QB, int NW, int BN, bool TAIL, bool ALIBI, bool DROP>
hipError_t launch_fwd_cfg(const FwdArgs& a) {
  constexpr int BM = NW * 32 * QB;
  const int BH = (int)(a.B * a.H);
  const int N = (int)a.N;
  const int nqb = (N + BM - 1) / BM;
  dim3 grid((unsigned)(nqb * BH)), block(NW * 64);
  const float scale_log2 = a.scale * kLog2e;
  const typename E::T* q = (const typename E::T*)a.q;
  const typename E::T* k = (const typename E::T*)a.k;
  const typename E::T* v = (const typename E::T*)a.v;
  typename E::T* o = (typename E::T*)a.o;
  float* lse = a.lse;
  Lay lq = a.lq, lk = a.lk, lv = a.lv, lo = a.lo;
  const int H = (int)a.H;
  const float* slopes = a.alibi_slopes;
  DropCfg drop = a.drop;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&lq, (void*)&lk, (void*)&lv,
                  (void*)&lo, (void*)&H, (void*)&BH, (void*)&N, (void*)&nqb, (void*)&scale_log2,
                  (void*)&slopes, (void*)&drop};
  return launch_kernel((const void*)fwd_kernel<E, D, CAUSAL, QB, NW, BN, TAIL, ALIBI, DROP>, grid, block, args,
                       a.stream, 0);
}

template <typename E, int D, int QB, int NW, int BN, bool ALIBI, bool DROP>
hipError_t launch_fwd_shape(const FwdArgs& a) {
  if (a.N % 64 == 0) {
    if (a.causal) return launch_fwd_cfg<E, D, true, QB, NW, BN, false, ALIBI, DROP>(a);
    return launch_fwd_cfg<E, D, false, QB, NW, BN, false, ALIBI, DROP>(a);
  }
  if (a.causal) return launch_fwd_cfg<E, D, true, QB, NW, BN, true, ALIBI, DROP>(a);
  return launch_fwd_cfg<E, D, false, QB, NW, BN, true, ALIBI, DROP>(a);
}

// Launch shape.  The 4-wave shape (128 queries, 64-key tiles in two buffers,
// 76 KB of LDS at d = 128) puts two workgroups on a CU: the two waves that
// share a SIMD then belong to different workgroups and never meet at the same
// tile barrier, and one workgroup's start and end overlap the other's work.
// It reads each K/V tile for twice as many query blocks, which costs more than
// it saves once a head's rows are long.  Measured on MI355X (forward alone,
// same box): at d = 128 the 4-wave shape is 5-10 % faster for causal
// N <= 4096, 2 % at N = 8192, about even at 16384 and 3 % slower at 32768;
// non-causal, 4-7 % faster for N <= 2048 and 2-5 % slower from 4096 on; at
// d = 64 it is ahead for causal N <= 4096 and non-causal N <= 2048.
// ATTN_FWD_WAVES=4 or 8 in the environment (read on every call) forces one
// shape, so that tests can run each case in both.
inline int forced_fwd_waves() {
  const char* e = std::getenv("ATTN_FWD_WAVES");
  return e ? std::atoi(e) : 0;
}

template <typename E, int D, bool ALIBI, bool DROP>
hipError_t launch_fwd_a(const FwdArgs& a) {
  constexpr int BN = ATTN_FWD_BN ? ATTN_FWD_BN : (D == 128 ? 128 : 64);
  const int64_t small_n = a.causal ? (D == 128 ? 8192 : 4096) : 2048;
  const int forced = forced_fwd_waves();
  const bool four = ATTN_FWD_NW ? ATTN_FWD_NW == 4 : (forced == 4 || (forced != 8 && a.N <= small_n));
  if (four) return launch_fwd_shape<E, D, 1, 4, 64, ALIBI, DROP>(a);
  return launch_fwd_shape<E, D, ATTN_FWD_QB, 8, BN, ALIBI, DROP>(a);
}

// Dropout and ALiBi are not combined (no entry point takes both).
template <typename E, int D>
hipError_t launch_fwd_d(const FwdArgs& a) {
  if (a.drop.t) return launch_fwd_a<E, D, false, true>(a);
  return a.alibi_slopes ? launch_fwd_a<E, D, true, false>(a) : launch_fwd_a<E, D, false, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? launch_fwd_d<bf16_t, 64>(a) : launch_fwd_d<bf16_t, 128>(a);
  return a.d == 64 ? launch_fwd_d<f16_t, 64>(a) : launch_fwd_d<f16_t, 128>(a);
}

}  // namespace attn
