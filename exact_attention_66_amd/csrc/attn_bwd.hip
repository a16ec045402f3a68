// Backward pass of exact attention on gfx950.
//
// Method: page "Flash Attention V2 大模型时代的算力救星" §3.2 and page
// "突破单卡显存极限：FlashAttention-2技术解析与实战指南" §2.2: the forward keeps
// only the per-row softmax statistic (lse), and the backward recomputes the
// scores from Q and K.  The gradients are the exact chain rule of
// O = softmax(scale Q K^T) V:
//   P = exp(scale S - lse),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_j P_ij dP_ij = dO_i . O_i,  dS = P o (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels on the caller's stream, no atomics anywhere (every output
// element is written by exactly one lane, so all of dQ, dK, dV are bitwise
// reproducible):
//  1. bwd_prep: -D_i = -dO_i . O_i and -lse_i / scale (fp32), and transposed
//     copies Q^T, dO^T, K^T ([B*H][d][Np]) in the workspace.  Inside every group of 16 tokens
//     the copies store tokens in MFMA reduction-slot order (slot_key), so
//     each operand fragment the main kernels need is one contiguous 16-byte
//     LDS read; the LDS transpose reads happen once here instead of once per
//     wave per tile.
//  2. bwd_dkdv: a persistent grid; each workgroup runs a list of units
//     (batch*head, block of 32*NW keys).  Each wave keeps its 32 keys' K and
//     V as MFMA operands and their dK, dV fp32 accumulators for the whole
//     sweep over query tiles.  S = Q K^T and dP = dO V^T put one key per
//     lane, so P and dS are directly the A operands of dV += P^T dO and
//     dK += dS^T Q (B operands from the transposed tiles).
//  3. bwd_dq: a persistent grid walking units (batch*head, block of 32*NW
//     queries), shaped like the forward: each wave keeps Q and dO rows as
//     operands and dQ^T in accumulators, computes S^T = K Q^T and
//     dP^T = V dO^T (one query per lane: lse and D are per-lane scalars),
//     and adds dQ^T += K^T dS^T.
// The price of (3) is recomputing S and dP once more (7 matrix products in
// total instead of 5); in exchange there is no cross-workgroup reduction.
// Any N is accepted: the workspace is padded to Np = 64 ceil(N / 64) tokens
// and (TAIL instantiations, N not a multiple of 64) the last partial tiles of
// Q, dO, K, V come from zero-padded copies made by (1).
//
// Softmax arithmetic folded into the products: (2) and (3) start the S and
// dP accumulators at -lse / scale and -D instead of zero, so the MFMAs
// deliver S - lse / scale and dP - D directly: per score only
// P = exp2(scale log2(e) acc) and dS = P acc remain.  The 16-bit Q and K
// operands stay exactly as given (scaling one of them by scale log2(e) in
// 16 bits would save the multiply but round the operand, an error of up to
// 2^-9 |S| log2(e) in the exponent, large for rows of large scores); the
// fp32 start value carries lse / scale with a relative error of 2^-24.
// This file is compiled with MFMA results in VGPRs (the softmax reads them
// without copies out of AGPRs); the operands read from LDS are steered into
// AGPRs instead (in_agpr).
// Three more instantiation flags: STRIDED (the inputs in callers' layouts:
// (1) reads them through their strides and writes contiguous copies of Q, K,
// V, dO that (2) and (3) read, whose epilogues store dQ, dK, dV through
// their strides), ALIBI (the linear position bias -m_h |i - j| added to
// the exponent of P in (2) and (3)) and DROP (dropout on P, regenerated in
// (2) and (3) from the generator of attn_dropout.h: with the keep factor k,
// P is computed as k P and dP starts at -D / k, so a kept score's dS is
// P (k dP - D) and a dropped one's -P D, and dV's operand has the dropped
// weights cleared).  Without them the code is unchanged.
#include "attn_device.h"
#include "attn_dropout.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

#ifndef ATTN_DQ_NW
#define ATTN_DQ_NW 8      // waves per workgroup (32 queries each)
#endif
#ifndef ATTN_DQ_BN
#define ATTN_DQ_BN 64     // keys per LDS tile
#endif
#ifndef ATTN_DQ_MINW
#define ATTN_DQ_MINW 2
#endif
#ifndef ATTN_DQ_KTSTAGE
#define ATTN_DQ_KTSTAGE 0  // read all K^T fragments before the softmax
#endif
#ifndef ATTN_DQ_KSTAGE
#define ATTN_DQ_KSTAGE 2  // K and V operand fragments read ahead per batch
#endif

// ---------------------------------------------------------------- prep
// One workgroup per (batch*head, 64-token block) of the padded length
// Np = 64 ceil(N / 64).  Q, K, dO tiles go through swizzled LDS; the
// transposed copies are read back with ds_read_b64_tr_b16 (lane gets 4
// tokens of one d column, twice = 8 tokens in slot order) and written as
// 16-byte rows of [d][token] with row stride Np.  Tokens past N are padding:
// zero in the transposed copies, -D = 0 and -lse / scale = -inf, so a padded
// query gets P = 0 and dS = 0 in the kernels that follow and adds nothing to
// dK, dV.  When N is not a multiple of 64 the block holding the last tokens
// also writes them, zero-padded to 64 rows, as row-major tail tiles of Q,
// dO, K and V ([B*H][64][d]): the main kernels take their last partial tile
// from there and never read past the end of an input.  TAIL (N not a
// multiple of 64) is a template flag, so that the checks cost nothing when
// there is no padding.
template <typename E, int D, bool TAIL, bool STRIDED>
__global__ __launch_bounds__(256) void bwd_prep(const typename E::T* __restrict__ Q,
                                                const typename E::T* __restrict__ K,
                                                const typename E::T* __restrict__ V,
                                                const typename E::T* __restrict__ O,
                                                const typename E::T* __restrict__ dO,
                                                const float* __restrict__ LSE, float* __restrict__ Dvec,
                                                float* __restrict__ NLSE, typename E::T* __restrict__ QT,
                                                typename E::T* __restrict__ KT, typename E::T* __restrict__ dOT,
                                                typename E::T* __restrict__ QTail, typename E::T* __restrict__ dOTail,
                                                typename E::T* __restrict__ KTail, typename E::T* __restrict__ VTail,
                                                int N, int Np, float inv_scale, Lay lq, Lay lk, Lay lv, Lay lo,
                                                Lay ldo, int H, typename E::T* __restrict__ Qc,
                                                typename E::T* __restrict__ Kc, typename E::T* __restrict__ Vc,
                                                typename E::T* __restrict__ dOc) {
  using T = typename E::T;
  using v8 = typename E::v8;
  constexpr int R = 64;                // tokens per workgroup
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int CPT = R * CPR / 256;   // chunks per thread per tensor
  __shared__ __attribute__((aligned(16))) T tile[3][R * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int r = lane & 31;
  const int nrb = Np / R;
  const int bh = (int)(blockIdx.x / nrb);
  const int rb = (int)(blockIdx.x % nrb);
  const size_t head = (size_t)bh * N * D;     // inputs [B*H][N][d] (contiguous copies when STRIDED)
  const size_t headp = (size_t)bh * Np * D;   // transposed copies [B*H][d][Np]
  const int bi = bh / H, hi = bh - bi * H;    // batch and head (STRIDED: the inputs' own layouts)
  const int row0 = rb * R;
  const bool tail = TAIL && row0 + R > N;     // the block holding the last tokens of a ragged N

#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = tid + c * 256;
    const int row = idx / CPR;
    const int col = (idx % CPR) * 8;
    const int tok = row0 + row;
    const bool in = !TAIL || tok < N;
    const size_t g = head + (size_t)tok * D + col;
    v8 qv = {}, kv = {}, dov = {}, ov = {}, vv = {};
    if constexpr (STRIDED) {
      // read each input in its own layout and keep contiguous copies of Q,
      // K, V and dO for the dK/dV and dQ kernels
      if (in) {
        auto at = [&](const Lay& l) { return bi * l.sb + hi * l.sh + (int64_t)tok * l.sn + col; };
        qv = *(const v8*)(Q + at(lq));
        kv = *(const v8*)(K + at(lk));
        dov = *(const v8*)(dO + at(ldo));
        ov = *(const v8*)(O + at(lo));
        vv = *(const v8*)(V + at(lv));
        *(v8*)(Qc + g) = qv;
        *(v8*)(Kc + g) = kv;
        *(v8*)(Vc + g) = vv;
        *(v8*)(dOc + g) = dov;
      }
    } else if (in) {
      qv = *(const v8*)(Q + g);
      kv = *(const v8*)(K + g);
      dov = *(const v8*)(dO + g);
      ov = *(const v8*)(O + g);
    }
    *(v8*)(&tile[0][swz<D>(row, col)]) = qv;
    *(v8*)(&tile[1][swz<D>(row, col)]) = kv;
    *(v8*)(&tile[2][swz<D>(row, col)]) = dov;
    // D_i: the CPR chunks of a row are held by CPR consecutive lanes
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)ov[i], (float)dov[i], acc);
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CPR);
    if ((idx % CPR) == 0) {
      const size_t i = (size_t)bh * Np + tok;
      Dvec[i] = -acc;
      NLSE[i] = in ? -LSE[(size_t)bh * N + tok] * inv_scale : -__builtin_inff();
    }
    if (tail) {
      const size_t gt = (size_t)bh * R * D + (size_t)row * D + col;
      if (!STRIDED && in) vv = *(const v8*)(V + g);
      *(v8*)(QTail + gt) = qv;
      *(v8*)(dOTail + gt) = dov;
      *(v8*)(KTail + gt) = kv;
      *(v8*)(VTail + gt) = vv;
    }
  }
  __syncthreads();

  // transposed copies: step = (16-token group pg, 32-wide d block db)
  T* const outs[3] = {QT, KT, dOT};
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  constexpr int STEPS = (R / 16) * (D / 32);
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    for (int st = w; st < STEPS; st += 4) {
      const int pg = st / (D / 32);
      const int db = st % (D / 32);
      const int rr = pg * 16 + tr_row;
      const v8 val = concat44<E>(E::tr_read(&tile[t][swz<D>(rr, db * 32 + tr_col)]),
                                 E::tr_read(&tile[t][swz<D>(rr + 8, db * 32 + tr_col)]));
      *(v8*)(outs[t] + headp + (size_t)(db * 32 + r) * Np + row0 + pg * 16 + 8 * h) = val;
    }
  }
}

// ---------------------------------------------------------------- dK, dV
// A persistent grid of NW-wave workgroups, as many as fit on the device; each
// runs its share of the units (batch*head, block of 32*NW keys) one after
// another (xcd_snake_unit), which saves the launch gap between workgroups
// and lets the next unit's first loads overlap this unit's stores.  A wave
// keeps its 32 keys' K and V as MFMA operands and their dK, dV fp32
// accumulators for the whole sweep over 64-query tiles.
//
// Tiles reach LDS by direct global->LDS copies (no staging registers, no LDS
// write instructions), double-buffered; a tile's copies go out in four
// parts spread over four MFMA groups (a wave that issues a whole tile's
// copies at once stalls on its full memory queue).  LDS rows are padded so
// that the 16-lane groups of every ds_read_b128 hit distinct banks and every
// read address is one per-lane base plus an immediate: row-major Q and dO tiles
// use rows of D + 8 elements, the transposed Q^T and dO^T tiles rows of
// 64 + 8.  A copy instruction fills 64 consecutive 16-byte slots, so the
// padding slot at the end of each row is filled with a duplicate of the
// row's last chunk, and a tile is a whole number of 64-slot blocks.
//
// Each 32-query sub-tile runs as four groups of MFMAs, and every group has
// the LDS reads or the softmax work of a later group interleaved with it,
// so that each read has a whole group of MFMAs to arrive in:
//   X  S' = -lse / scale + Q K^T   | dO^T fragments (B operands of Z)
//   Y  dP' = -D + dO V^T  | P = exp2(scale log2e S'); Q^T fragments (W)
//   Z  dV += P^T dO       | dS = P dP'; next sub-tile's Q fragments (X)
//   W  dK += dS^T Q       | next sub-tile's dO fragments (Y) and lse, D (X, Y)
// (S, dP with one key per lane: P and dS are directly the A operands of the
// dV and dK products.)  The barrier between tiles sits after Y of the second
// sub-tile: every read of the tile has then been issued, so the next tile's
// first reads (Z, W) can already use the other buffer, and the copy of the
// tile after it starts into the buffer just released.  Tiles that reach the
// causal diagonal come first and run the same pipeline with the mask applied
// (sub-tiles entirely above the diagonal come out as P = 0).
template <typename E, int D, bool CAUSAL, int NW, int BMQ, bool TAIL, bool STRIDED, bool ALIBI, bool DROP>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const typename E::T* __restrict__ QT, const typename E::T* __restrict__ dOT,
    const typename E::T* __restrict__ QTail, const typename E::T* __restrict__ dOTail,
    const float* __restrict__ NLSE, const float* __restrict__ Dvec, typename E::T* __restrict__ dK,
    typename E::T* __restrict__ dV, int BH, int N, int Np_arg, int nkb, float scale, float scale_log2, Lay ldk,
    Lay ldv, int H, const float* __restrict__ slopes, DropCfg drop) {
  using T = typename E::T;
  using v8 = typename E::v8;
  const int Np = TAIL ? Np_arg : N;     // padded length: N itself unless TAIL
  static_assert(BMQ == 64, "the pipeline handles two 32-query sub-tiles per tile");
  static_assert(!CAUSAL || NW * 32 == 2 * BMQ, "causal: exactly two diagonal tiles per workgroup");
  static_assert((NW & (NW - 1)) == 0, "power-of-two wave count");
  constexpr int BN = NW * 32;          // keys per workgroup
  constexpr int KS = D / 16;           // reduction steps over d
  constexpr int DB = D / 32;           // 32-wide d blocks
  constexpr int LR = D + 8;            // padded row-major row (elements)
  constexpr int LT = BMQ + 8;          // padded transposed row (elements)
  constexpr int RSL = LR / 8;          // 16-byte slots per row-major row
  constexpr int TSL = LT / 8;          // 16-byte slots per transposed row
  constexpr int RI = (BMQ * RSL + 63) / 64;  // 64-slot copy blocks per row-major tile
  constexpr int TI = (D * TSL + 63) / 64;    // 64-slot copy blocks per transposed tile
  constexpr int RC = (RI + NW - 1) / NW;     // blocks per wave
  constexpr int TC = (TI + NW - 1) / NW;
  constexpr int RSZ = RI * 64 * 8;     // elements per row-major tile buffer
  constexpr int TSZ = TI * 64 * 8;

  // separate objects per buffer; buffer indices are compile-time constants
  __shared__ __attribute__((aligned(16))) T lq0[RSZ], lq1[RSZ], ldo0[RSZ], ldo1[RSZ];
  __shared__ __attribute__((aligned(16))) T lqt0[TSZ], lqt1[TSZ], ldot0[TSZ], ldot1[TSZ];
  __shared__ __attribute__((aligned(16))) float ll0[64], ll1[64], ld0[64], ld1[64];

  const int lane = threadIdx.x & 63;
  const int wu = wave_id() & (NW - 1);
  const int h = lane >> 5;
  const int r = lane & 31;

  // Persistent grid: the workgroup runs its units (batch*head, block of BN
  // keys; xcd_snake_unit) one after another.  The next unit's first tile
  // copy and K, V loads are issued before this unit's dK, dV stores, so the
  // stores and both load latencies overlap.
  int round = 0;
  int unit = xcd_snake_unit((int)blockIdx.x, (int)gridDim.x, BH * nkb, 0);
  if (unit < 0) return;
  const int nqt = Np / BMQ;             // query tiles (the last may be padded)
  const int nfull = N / BMQ;            // tiles wholly inside the sequence
  int kb0, kw0, it0, ntile, nmask;
  size_t head;
  int64_t out_k = 0, out_v = 0;         // STRIDED: dK, dV offsets of (batch, head, key kw0)
  float nslope2 = 0.f;                  // ALIBI: -slope * log2(e) of this unit's head
  const T *Qh, *dOh, *QTh, *dOTh, *Qtl, *dOtl;
  const float *lse_h, *dd_h;
  int unit_bh = 0;                      // DROP: batch*head of this unit (generator counter)
  auto set_unit = [&](const int u) {
    const int bh = u / nkb;
    unit_bh = bh;
    kb0 = (u % nkb) * BN;
    kw0 = kb0 + wu * 32;                 // first key of this wave
    head = (size_t)bh * (size_t)N * D;
    if constexpr (ALIBI) nslope2 = -slopes[bh % H] * kLog2e;
    if constexpr (STRIDED) {
      const int bi = bh / H, hi = bh - bi * H;
      out_k = bi * ldk.sb + hi * ldk.sh + (int64_t)kw0 * ldk.sn;
      out_v = bi * ldv.sb + hi * ldv.sh + (int64_t)kw0 * ldv.sn;
    }
    const size_t headp = (size_t)bh * (size_t)Np * D;
    Qh = Q + head;
    dOh = dO + head;
    QTh = QT + headp;
    dOTh = dOT + headp;
    Qtl = QTail + (size_t)bh * BMQ * D;
    dOtl = dOTail + (size_t)bh * BMQ * D;
    lse_h = NLSE + (size_t)bh * Np;
    dd_h = Dvec + (size_t)bh * Np;
    it0 = CAUSAL ? kb0 / BMQ : 0;        // earlier tiles lie entirely above the diagonal
    ntile = nqt - it0;                   // visited in order it0, it0 + 1, ...; the first two are on the diagonal
    nmask = CAUSAL ? min(2, ntile) : 0;
  };
  set_unit(unit);

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  // per-lane byte offsets of the tile copies, the same for every tile
  unsigned roff[RC], toff[TC];
#pragma unroll
  for (int c = 0; c < RC; ++c) {
    const int s = 64 * (wu + NW * c) + lane;
    const int row = min(s / RSL, BMQ - 1);
    const int col = min(s % RSL, RSL - 2);
    roff[c] = (unsigned)(row * D + col * 8) * 2u;
  }
#pragma unroll
  for (int c = 0; c < TC; ++c) {
    const int s = 64 * (wu + NW * c) + lane;
    const int row = min(s / TSL, D - 1);
    const int col = min(s % TSL, TSL - 2);
    toff[c] = ((unsigned)row * (unsigned)Np + (unsigned)(col * 8)) * 2u;
  }
  // A tile's copies in four parts (Q, dO, Q^T, dO^T with the statistics),
  // so that they can be spread over the MFMA groups instead of filling the
  // wave's memory queue at once.  A padded last tile takes its Q and dO rows
  // from the zero-padded tail tiles (a scalar choice of base address).
  auto copy_part = [&](const int it, auto bufc, auto partc) {
    constexpr int b = decltype(bufc)::value;
    constexpr int part = decltype(partc)::value;
    if constexpr (part < 2) {
      T* const dst = part == 0 ? (b ? lq1 : lq0) : (b ? ldo1 : ldo0);
      const T* const src =
          !TAIL || it < nfull ? (part == 0 ? Qh : dOh) + (size_t)it * BMQ * D : (part == 0 ? Qtl : dOtl);
      const char* g = (const char*)src;
#pragma unroll
      for (int c = 0; c < RC; ++c)
        if (wu + NW * c < RI) lds_copy16(g, roff[c], dst + (wu + NW * c) * 512);
    } else {
      T* const dst = part == 2 ? (b ? lqt1 : lqt0) : (b ? ldot1 : ldot0);
      const char* g = (const char*)((part == 2 ? QTh : dOTh) + (size_t)it * BMQ);
#pragma unroll
      for (int c = 0; c < TC; ++c)
        if (wu + NW * c < TI) lds_copy16(g, toff[c], dst + (wu + NW * c) * 512);
      if constexpr (part == 3) {
        if (wu == 0) lds_copy4(lse_h + (size_t)it * BMQ, 4u * lane, b ? ll1 : ll0);
        if (wu == NW - 1) lds_copy4(dd_h + (size_t)it * BMQ, 4u * lane, b ? ld1 : ld0);
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  auto copy_tile = [&](const int it, auto bufc) {
    copy_part(it, bufc, P0{});
    copy_part(it, bufc, P1{});
    copy_part(it, bufc, P2{});
    copy_part(it, bufc, P3{});
  };

  // per-lane parts of the LDS read addresses (elements); everything else in
  // an address is a compile-time immediate
  const int offA = opaque(r * LR + 8 * h);      // row-major tiles: row r, column 8h
  const int offB = opaque(r * LT + 8 * h);      // transposed tiles: row r (d), column 8h
  const int offL = opaque(h);                   // lse / D: 4 consecutive queries (16-byte units)

  auto read_q = [&](auto bufc, const int qs, v8 (&qa)[KS]) {
    const T* ql = (decltype(bufc)::value ? lq1 : lq0) + offA + qs * 32 * LR;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = *(const v8*)(ql + ks * 16);
  };
  auto read_do = [&](auto bufc, const int qs, v8 (&da)[KS]) {
    const T* dol = (decltype(bufc)::value ? ldo1 : ldo0) + offA + qs * 32 * LR;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) da[ks] = *(const v8*)(dol + ks * 16);
  };
  auto read_stats = [&](auto bufc, const int qs, f32x4 (&l4)[4], f32x4 (&d4)[4]) {
    constexpr int b = decltype(bufc)::value;
    const f32x4* lp = (const f32x4*)(b ? ll1 : ll0) + offL;
    const f32x4* dp = (const f32x4*)(b ? ld1 : ld0) + offL;
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      l4[jg] = lp[qs * 8 + 2 * jg];
      d4[jg] = dp[qs * 8 + 2 * jg];
    }
  };
  // B operands of dV (dO^T) or dK (Q^T): row 32db + r of the transposed tile, 8 queries in slot order
  auto read_t = [&](const T* tl, const int qs, v8 (&x)[2][DB]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) x[kk][db] = *(const v8*)(tl + offB + qs * 32 + db * 32 * LT + 16 * kk);
  };

  // operands of the sub-tile about to start, read one group ahead
  v8 qa[KS], da[KS];
  f32x4 l4[4], d4[4];

  // this wave's K and V as B operands: lane holds row kw0 + r, d = 16ks + 8h .. +7
  v8 kB[KS], vB[KS];
  auto load_kv = [&]() {
    const int key = min(kw0 + r, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kB[ks] = *(const v8*)(K + head + (size_t)key * D + ks * 16 + 8 * h);
      vB[ks] = *(const v8*)(V + head + (size_t)key * D + ks * 16 + 8 * h);
    }
  };

  auto sub_tile = [&](const int it, auto maskc, auto bufc, auto qsc) {
    constexpr int b = decltype(bufc)::value;
    constexpr int qs = decltype(qsc)::value;
    // where the next sub-tile's operands live
    using NB = std::integral_constant<int, qs == 0 ? b : (b ^ 1)>;
    constexpr int nqs = qs ^ 1;
    const int qs0 = it * BMQ + qs * 32;

    // Tile it + 2 is copied into this tile's buffer in four parts: Q and dO
    // in Z and W of the second sub-tile (after the barrier has released the
    // buffer), Q^T and dO^T in X and Y of the next tile's first sub-tile.
    // The first two tiles of a unit are copied whole before the loop.
    using OB = std::integral_constant<int, b ^ 1>;
    const bool spread = qs == 0 && it >= it0 + 1 && it + 1 < nqt;
    if (spread) copy_part(it + 1, OB{}, P2{});

    // X: S = Q K^T | dO^T fragments
    v8 dob[2][DB];
    read_t(b ? ldot1 : ldot0, qs, dob);
    f32x16 sacc = join16(l4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      in_agpr(qa[ks]);
      sacc = E::mfma32(qa[ks], kB[ks], sacc);
    }
    sched_interleave<KS, kSchedMfma, 1, kSchedDsRead, 2 * DB / KS>();
    // (no fence: X and Y form one scheduling region, so the group patterns
    // place the whole S chain first and the exponentials between dP MFMAs)

    // Y: dP = dO V^T | P, Q^T fragments
    if (spread) copy_part(it + 1, OB{}, P3{});
    v8 qbv[2][DB];
    read_t(b ? lqt1 : lqt0, qs, qbv);
    // DROP: dP' starts at -D / k (k = 256 / (256 - t)) and P is computed as
    // k P, so that a kept element's dS = k P dP' = P (k dP - D) and a
    // dropped one's is k P (-D / k) = -P D
    const f32x16 dinit = DROP ? join16(d4) * (1.0f / drop.keep_scale) : join16(d4);
    f32x16 dpacc = dinit;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      in_agpr(da[ks]);
      dpacc = E::mfma32(da[ks], vB[ks], dpacc);
    }
    float p[16];
    // DROP: the draws of this lane's key against the sub-tile's 16 queries.
    // Lane u of the quad makes the call for block u (queries qs0 + 8u + 4h ..,
    // the quad's 4 keys); the bytes of its 4 words are regrouped by key
    // (word c = byte c of words 0..3) and the quad transpose hands every lane
    // its own key's word of each block: byte w of tw[m] is query
    // qs0 + 8m + 4h + w.
    u32x4 tw;
    if constexpr (DROP) {
      const int qu = lane & 3;
      const u32x4 wv = philox4x32_10((uint32_t)((qs0 >> 2) + 2 * qu + h), (uint32_t)(kw0 + r) >> 2,
                                     (uint32_t)unit_bh, drop.offset, drop.key0, drop.key1);
      u32x4 xv;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        xv[c] = ((wv[0] >> (8 * c)) & 0xFFu) | (((wv[1] >> (8 * c)) & 0xFFu) << 8) |
                (((wv[2] >> (8 * c)) & 0xFFu) << 16) | (((wv[3] >> (8 * c)) & 0xFFu) << 24);
      tw = quad_transpose(xv, qu);
    }
    if constexpr (ALIBI) {   // query qs0 + 4h + c (c = 8(j/4) + j%4) at distance dqk + c from key kw0 + r
      const float dqk = (float)(qs0 + 4 * h - kw0 - r);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        p[j] = fast_exp2(fmaf(sacc[j], scale_log2, nslope2 * fabsf(dqk + (float)(8 * (j / 4) + j % 4))));
    } else if constexpr (DROP) {
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = fast_exp2(fmaf(sacc[j], scale_log2, drop.log2_keep_scale));
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = fast_exp2(sacc[j] * scale_log2);
    }
    if constexpr (decltype(maskc)::value) {  // key > query -> P = 0
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kw0 + r > qs0 + acc_row(j, h)) p[j] = 0.f;
    }
    v8 pa[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      pa[kk] = pack8<E>(p[8 * kk + 0], p[8 * kk + 1], p[8 * kk + 2], p[8 * kk + 3], p[8 * kk + 4], p[8 * kk + 5],
                        p[8 * kk + 6], p[8 * kk + 7]);
    uint32_t km[16];   // DROP: all-ones for kept elements
    if constexpr (DROP) {
      const uint32_t add = (256u - drop.t) * 0x00010001u;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pw = __builtin_bit_cast(u32x4, pa[kk]);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          uint32_t lo, hi;
          keep_halves(tw[2 * kk + g], add, lo, hi);
          pw[2 * g] &= half_masks(lo);
          pw[2 * g + 1] &= half_masks(hi);
          km[8 * kk + 4 * g + 0] = full_mask(lo, 0);
          km[8 * kk + 4 * g + 1] = full_mask(lo, 1);
          km[8 * kk + 4 * g + 2] = full_mask(hi, 0);
          km[8 * kk + 4 * g + 3] = full_mask(hi, 1);
        }
        pa[kk] = __builtin_bit_cast(v8, pw);
      }
    }
    sched_interleave<KS, kSchedMfma, 1, kSchedDsRead, 2 * DB / KS, kSchedValu, 3>();
    sched_fence();

    if constexpr (qs == 1) {
      // every read of this tile is issued: wait for the next tile's copy,
      // meet the other waves, then refill this buffer
      mfma_drain();
      wait_all_vmem_loads();
      __syncthreads();
      sched_fence();
    }

    // Z: dV += P^T dO | dS, next Q fragments (stale but harmless after the last tile)
    if (qs == 1 && it + 2 < nqt) copy_part(it + 2, bufc, P0{});
    read_q(NB{}, nqs, qa);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        in_agpr(dob[kk][db]);
        dv_acc[db] = E::mfma32(pa[kk], dob[kk][db], dv_acc[db]);
      }
    float ds[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) ds[j] = p[j] * (DROP ? bit_select(km[j], dpacc[j], dinit[j]) : dpacc[j]);
    v8 sa[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      sa[kk] = pack8<E>(ds[8 * kk + 0], ds[8 * kk + 1], ds[8 * kk + 2], ds[8 * kk + 3], ds[8 * kk + 4],
                        ds[8 * kk + 5], ds[8 * kk + 6], ds[8 * kk + 7]);
    sched_interleave<2 * DB, kSchedMfma, 1, kSchedDsRead, KS / (2 * DB), kSchedValu, 3>();
    sched_fence();

    // W: dK += dS^T Q | next dO fragments and statistics
    if (qs == 1 && it + 2 < nqt) copy_part(it + 2, bufc, P1{});
    read_do(NB{}, nqs, da);
    read_stats(NB{}, nqs, l4, d4);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        in_agpr(qbv[kk][db]);
        dk_acc[db] = E::mfma32(sa[kk], qbv[kk][db], dk_acc[db]);
      }
    sched_interleave<2 * DB, kSchedMfma, 1, kSchedDsRead, (KS + 8) / (2 * DB)>();
    sched_fence();
  };
  auto tile = [&](const int it, auto maskc, auto bufc) {
    sub_tile(it, maskc, bufc, std::integral_constant<int, 0>{});
    sub_tile(it, maskc, bufc, std::integral_constant<int, 1>{});
  };

  // tiles it0 .. nqt-1 on buffers 0, 1, 0, ...; the diagonal ones first
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using MaskOn = std::integral_constant<bool, true>;
  using MaskOff = std::integral_constant<bool, false>;

  copy_tile(it0, B0{});
  load_kv();
  for (;;) {
    wait_all_vmem_loads();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {  // MFMA operands only: keep them in AGPRs
      asm volatile("" : "+a"(kB[ks]));
      asm volatile("" : "+a"(vB[ks]));
    }
    read_q(B0{}, 0, qa);
    read_do(B0{}, 0, da);
    read_stats(B0{}, 0, l4, d4);
    if (ntile > 1) copy_tile(it0 + 1, B1{});

    int it = it0;
    if (nmask > 0) tile(it++, MaskOn{}, B0{});
    if (nmask > 1) tile(it++, MaskOn{}, B1{});
    // nmask is 0 or 2 unless a single tile remains, so the unmasked tiles start on buffer 0
    for (; it + 1 < nqt; it += 2) {
      tile(it, MaskOff{}, B0{});
      tile(it + 1, MaskOff{}, B1{});
    }
    if (it < nqt) tile(it, MaskOff{}, B0{});
    mfma_drain();

    // start the next unit, then store this one's dK = scale * acc, dV = acc
    // (lane holds key kw0 + acc_row(j, h), d = 32db + r)
    const size_t out = head + (size_t)kw0 * D;
    const int64_t ok0 = out_k, ov0 = out_v;
    const int nvalid = N - kw0;          // keys of this wave inside the sequence
    unit = xcd_snake_unit((int)blockIdx.x, (int)gridDim.x, BH * nkb, ++round);
    __syncthreads();  // every wave is done with this unit's tiles
    if (unit >= 0) {
      set_unit(unit);
      copy_tile(it0, B0{});
      load_kv();
    }
    // (a unit holds 4 * 32 keys and N is only a multiple of 64 without TAIL,
    // so whole waves can lie past the end: nvalid <= 0)
    if (nvalid >= 32) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if constexpr (STRIDED) {
            dK[ok0 + (int64_t)acc_row(j, h) * ldk.sn + db * 32 + r] = (T)(dk_acc[db][j] * scale);
            dV[ov0 + (int64_t)acc_row(j, h) * ldv.sn + db * 32 + r] = (T)dv_acc[db][j];
          } else {
            const size_t off = out + (size_t)acc_row(j, h) * D + db * 32 + r;
            dK[off] = (T)(dk_acc[db][j] * scale);
            dV[off] = (T)dv_acc[db][j];
          }
        }
    } else if (TAIL && nvalid > 0) {  // the sequence ends inside this wave's keys
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (acc_row(j, h) < nvalid) {
            if constexpr (STRIDED) {
              dK[ok0 + (int64_t)acc_row(j, h) * ldk.sn + db * 32 + r] = (T)(dk_acc[db][j] * scale);
              dV[ov0 + (int64_t)acc_row(j, h) * ldv.sn + db * 32 + r] = (T)dv_acc[db][j];
            } else {
              const size_t off = out + (size_t)acc_row(j, h) * D + db * 32 + r;
              dK[off] = (T)(dk_acc[db][j] * scale);
              dV[off] = (T)dv_acc[db][j];
            }
          }
    }
    if (unit < 0) break;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dk_acc[db] = f32x16{};
      dv_acc[db] = f32x16{};
    }
  }
}

// ---------------------------------------------------------------- dQ
// Shaped like the forward: each wave keeps 32 queries' Q and dO rows as B
// operands and dQ^T in accumulators, computes
// S^T = K Q^T and dP^T = V dO^T (one query per lane: lse and D are per-lane
// scalars), and adds dQ^T += K^T dS^T (A operands from the K^T tile).  A
// persistent grid, like the dK/dV kernel's: workgroups walk their units
// (xcd_snake_unit) and start the next unit's loads before the dQ stores;
// keeping a head's units on one XCD, and sweeping the key tiles in
// alternate directions on alternate rounds, lets them share its K, V, K^T
// tiles in that XCD's L2.  K, V [BN][D + 8] and
// K^T [D][BN + 8] tiles (padded rows: conflict-free ds_read_b128, affine
// addresses) reach LDS by direct global->LDS copies into three rotating
// buffers, two tiles ahead of their use; a copy instruction fills 64
// consecutive 16-byte slots, so the padding slot of each row gets a
// duplicate of the row's last chunk and a tile is a whole number of blocks.
template <typename E, int D, bool CAUSAL, int NW, int BN, bool TAIL, bool STRIDED, bool ALIBI, bool DROP>
__global__ __launch_bounds__(NW * 64, ATTN_DQ_MINW) void bwd_dq(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const typename E::T* __restrict__ KT, const typename E::T* __restrict__ KTail,
    const typename E::T* __restrict__ VTail, const float* __restrict__ NLSE, const float* __restrict__ ND,
    typename E::T* __restrict__ dQ, int BH, int N, int Np_arg, int nqb, float scale, float scale_log2, Lay ldq,
    int H, const float* __restrict__ slopes, DropCfg drop) {
  using T = typename E::T;
  const int Np = TAIL ? Np_arg : N;     // padded length: N itself unless TAIL
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  constexpr int BM = NW * 32;        // queries per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KB = BN / 32;        // 32-key blocks per tile
  constexpr int LR = D + 8;          // padded K / V row (elements)
  constexpr int LT = BN + 8;         // padded K^T row (elements)
  constexpr int RSL = LR / 8;        // 16-byte slots per K / V row
  constexpr int TSL = LT / 8;        // 16-byte slots per K^T row
  constexpr int RI = (BN * RSL + 63) / 64;   // 64-slot copy blocks per K or V tile
  constexpr int TI = (D * TSL + 63) / 64;    // per K^T tile
  constexpr int RC = (RI + NW - 1) / NW;
  constexpr int TC = (TI + NW - 1) / NW;
  constexpr int RSZ = RI * 64 * 8;   // elements per K or V tile buffer
  constexpr int TSZ = TI * 64 * 8;
  constexpr int NBUF = 3;            // tile t in buffer t % 3, copied two tiles ahead
  static_assert(BN == 64, "K^T rows of 64 keys");

  __shared__ __attribute__((aligned(16))) T lds_k[NBUF][RSZ];
  __shared__ __attribute__((aligned(16))) T lds_v[NBUF][RSZ];
  __shared__ __attribute__((aligned(16))) T lds_kt[NBUF][TSZ];

  const int lane = threadIdx.x & 63;
  const int wu = wave_id() & (NW - 1);
  const int h = lane >> 5;
  const int r = lane & 31;

  // Persistent grid: the workgroup runs its units (batch*head, block of BM
  // queries) one after another (xcd_snake_unit: the units of a head stay on
  // one XCD, so its K, V, K^T tiles are shared in that XCD's L2; within a
  // head the heaviest query blocks come first).  The next unit's first tile
  // copies and Q, dO loads are issued before this unit's dQ stores.
  int round = 0;
  int unit = xcd_snake_unit((int)blockIdx.x, (int)gridDim.x, BH * nqb, 0);
  if (unit < 0) return;
  const int nfull = N / BN;   // key tiles wholly inside the sequence
  int bh, q0, qw0, kv_end, ntiles, q_last;
  bool desc = false;    // this unit walks its key tiles last to first
  float nslope2 = 0.f;   // ALIBI: -slope * log2(e) of this unit's head
  bool wave_valid;
  size_t head;
  const T *Kh, *Vh, *KTh, *Ktl, *Vtl;
  auto set_unit = [&](const int u) {
    bh = u / nqb;
    const int qblk = CAUSAL ? nqb - 1 - u % nqb : u % nqb;
    q0 = qblk * BM;
    qw0 = q0 + wu * 32;
    wave_valid = qw0 < N;
    if constexpr (ALIBI) nslope2 = -slopes[bh % H] * kLog2e;
    head = (size_t)bh * (size_t)N * D;
    Kh = K + head;
    Vh = V + head;
    KTh = KT + (size_t)bh * (size_t)Np * D;
    Ktl = KTail + (size_t)bh * BN * D;
    Vtl = VTail + (size_t)bh * BN * D;
    kv_end = CAUSAL ? min(N, q0 + BM) : N;
    ntiles = (kv_end + BN - 1) / BN;
    // Units of odd rounds walk their key tiles last to first.  With the
    // heaviest-first snake order, the workgroups of an XCD start the units
    // of an even round together and end those of an odd round together, so
    // in either direction they sweep the same key tile at about the same
    // time and its K, V, K^T come from HBM about once per round instead of
    // once per unit.
    desc = (round & 1) != 0;
    q_last = qw0 + 31;
  };
  set_unit(unit);

  // this wave's Q and dO rows and the accumulator starting values; filled
  // in once the first tile copies are issued
  v8 qf[KS], dof[KS];
  f32x16 s_init, dp_init;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  const int offA = opaque(r * LR + 8 * h);
  const int offB = opaque(r * LT + 8 * h);

  // ---- tile copies: per-lane byte offsets, the same for every tile
  unsigned roff[RC], toff[TC];
#pragma unroll
  for (int c = 0; c < RC; ++c) {
    const int sl = 64 * (wu + NW * c) + lane;
    const int row = min(sl / RSL, BN - 1);
    const int col = min(sl % RSL, D / 8 - 1);
    roff[c] = (unsigned)(row * D + col * 8) * 2u;
  }
#pragma unroll
  for (int c = 0; c < TC; ++c) {
    const int sl = 64 * (wu + NW * c) + lane;
    const int row = min(sl / TSL, D - 1);
    const int col = min(sl % TSL, BN / 8 - 1);
    toff[c] = ((unsigned)row * (unsigned)Np + (unsigned)(col * 8)) * 2u;
  }
  // a tile's copies in three parts (K, V, K^T), so that they can be spread
  // over the tile instead of filling the wave's memory queue at once; a
  // padded last tile takes its K and V rows from the zero-padded tail tiles
  auto copy_part = [&](const int t, const int b, const int part) {
    if (part < 2) {
      const T* const src = !TAIL || t < nfull ? (part == 0 ? Kh : Vh) + (size_t)t * BN * D : (part == 0 ? Ktl : Vtl);
      const char* g = (const char*)src;
      T* const dst = part == 0 ? lds_k[b] : lds_v[b];
#pragma unroll
      for (int c = 0; c < RC; ++c)
        if (wu + NW * c < RI) lds_copy16(g, roff[c], dst + (wu + NW * c) * 512);
    } else {
      const char* g = (const char*)(KTh + (size_t)t * BN);
#pragma unroll
      for (int c = 0; c < TC; ++c)
        if (wu + NW * c < TI) lds_copy16(g, toff[c], &lds_kt[b][(wu + NW * c) * 512]);
    }
  };
  auto copy_tile = [&](const int t, const int b) {
    copy_part(t, b, 0);
    copy_part(t, b, 1);
    copy_part(t, b, 2);
  };
  // Wait until at most one tile's copies (the most recent) are outstanding:
  // vmcnt counts this wave's copies in issue order.
  auto wait_copies_but_last = [&]() {
    constexpr auto cnt = [](int w) {
      int n = 0;
      for (int c = 0; c < RC; ++c) n += 2 * (w + NW * c < RI);
      for (int c = 0; c < TC; ++c) n += (w + NW * c < TI);
      return n;
    };
    static_assert(2 * RC + TC < 16, "vmcnt immediate");
    static_assert(NW == 8, "one case per wave");
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

  auto key_block = [&](const int buf, const int kb, const int kbk0) {
    const T* kl = lds_k[buf] + offA + kb * 32 * LR;
    const T* vl = lds_v[buf] + offA + kb * 32 * LR;
    const T* ktl = lds_kt[buf] + offB + kb * 32;
    // S^T = K Q^T, dP^T = V dO^T: lane holds query qw0 + r, keys acc_row(j, h).
    // Operand reads go in batches of KSTAGE per operand, each batch issued
    // ahead of its MFMAs.
    f32x16 sacc = s_init, dpacc = dp_init;
    constexpr int KH = ATTN_DQ_KSTAGE < KS ? ATTN_DQ_KSTAGE : KS;
#pragma unroll
    for (int part = 0; part < KS / KH; ++part) {
      v8 ka[KH], va[KH];
#pragma unroll
      for (int u = 0; u < KH; ++u) {
        ka[u] = *(const v8*)(kl + (part * KH + u) * 16);
        va[u] = *(const v8*)(vl + (part * KH + u) * 16);
      }
      sched_fence();
#pragma unroll
      for (int u = 0; u < KH; ++u) {
        sacc = E::mfma32(ka[u], qf[part * KH + u], sacc);
        dpacc = E::mfma32(va[u], dof[part * KH + u], dpacc);
      }
      sched_fence();
    }
#if ATTN_DQ_KTSTAGE
    v8 kta[2][DB];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) kta[kk][db] = *(const v8*)(ktl + db * 32 * LT + 16 * kk);
#endif
    float ds[16];
    // DROP: the draws of this lane's query against the block's 16 keys (as in
    // the forward: lane u of the quad calls for keys kbk0 + 8u + 4h ..)
    uint32_t km[16];
    if constexpr (DROP) {
      const int qu = lane & 3;
      const u32x4 tw = quad_transpose(philox4x32_10((uint32_t)(qw0 + r) >> 2, (uint32_t)((kbk0 >> 2) + 2 * qu + h),
                                                    (uint32_t)bh, drop.offset, drop.key0, drop.key1),
                                      qu);
      const uint32_t add = (256u - drop.t) * 0x00010001u;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t lo, hi;
        keep_halves(tw[m], add, lo, hi);
        km[4 * m + 0] = full_mask(lo, 0);
        km[4 * m + 1] = full_mask(lo, 1);
        km[4 * m + 2] = full_mask(hi, 0);
        km[4 * m + 3] = full_mask(hi, 1);
      }
    }
    if constexpr (ALIBI) {   // key kbk0 + 4h + c (c = 8(j/4) + j%4) at distance dq - c from query qw0 + r
      const float dq = (float)(qw0 + r - kbk0 - 4 * h);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        ds[j] = fast_exp2(fmaf(sacc[j], scale_log2, nslope2 * fabsf(dq - (float)(8 * (j / 4) + j % 4))));
    } else if constexpr (DROP) {   // k P with k = 256 / (256 - t); dP' started at -D / k
#pragma unroll
      for (int j = 0; j < 16; ++j) ds[j] = fast_exp2(fmaf(sacc[j], scale_log2, drop.log2_keep_scale));
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) ds[j] = fast_exp2(sacc[j] * scale_log2);
    }
    if (TAIL && !CAUSAL && kbk0 + 32 > N) {   // keys past the end of the sequence -> P = 0
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kbk0 + acc_row(j, h) >= N) ds[j] = 0.f;
    }
    if (CAUSAL && kbk0 + 31 > qw0) {   // block crosses the diagonal: key > query -> P = 0
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kbk0 + acc_row(j, h) > qw0 + r) ds[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) ds[j] = ds[j] * (DROP ? bit_select(km[j], dpacc[j], dp_init[j]) : dpacc[j]);
    // dQ^T += K^T dS^T: A from the K^T tile (row d, 8 keys in slot order)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const v8 sb = pack8<E>(ds[8 * kk + 0], ds[8 * kk + 1], ds[8 * kk + 2], ds[8 * kk + 3], ds[8 * kk + 4],
                             ds[8 * kk + 5], ds[8 * kk + 6], ds[8 * kk + 7]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#if ATTN_DQ_KTSTAGE
        const v8 a = kta[kk][db];
#else
        const v8 a = *(const v8*)(ktl + db * 32 * LT + 16 * kk);
#endif
        acc[db] = E::mfma32(a, sb, acc[db]);
      }
    }
  };

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T, and the
  // statistics (spread over the accumulator starting values once they have arrived)
  float nlse, ndd;
  auto load_q = [&]() {
    const int qrow = min(qw0 + r, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const v8*)(Q + head + (size_t)qrow * D + ks * 16 + 8 * h);
      dof[ks] = *(const v8*)(dO + head + (size_t)qrow * D + ks * 16 + 8 * h);
    }
    nlse = NLSE[(size_t)bh * Np + qrow];
    ndd = ND[(size_t)bh * Np + qrow];
  };

  // key tile of the unit's sq-th step
  auto tile_of = [&](const int sq) { return desc ? ntiles - 1 - sq : sq; };
  auto k_tile = [&](const int sq, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int t = tile_of(sq);
    // buffer (sq + 2) % 3 held the tile of step sq - 1, which every wave has
    // finished; the copy of step sq + 2's tile into it goes out in three
    // parts: K before the first key block, V before the second, K^T after
    // the last
    constexpr int NB = (buf + 2) % NBUF;
    const bool more = sq + 2 < ntiles;
    if (more) copy_part(tile_of(sq + 2), NB, 0);
    const int k0 = t * BN;
    const bool run = wave_valid && (!CAUSAL || k0 <= q_last);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb == KB / 2 && more) copy_part(tile_of(sq + 2), NB, 1);
      const int kbk0 = k0 + kb * 32;
      if (run && (!CAUSAL || kbk0 <= q_last) && (!TAIL || kbk0 < N)) key_block(buf, kb, kbk0);
    }
    if (more) copy_part(tile_of(sq + 2), NB, 2);
    mfma_drain();
    // step sq + 1's tile must be in LDS: its copies are the ones before the most recent
    if (more) wait_copies_but_last();
    else wait_all_vmem_loads();
    __syncthreads();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  copy_tile(tile_of(0), 0);
  if (ntiles > 1) copy_tile(tile_of(1), 1);
  load_q();
  for (;;) {
    wait_all_vmem_loads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      materialize(qf[ks]);
      materialize(dof[ks]);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s_init[j] = nlse;
      dp_init[j] = DROP ? ndd * (1.0f / drop.keep_scale) : ndd;
    }
    __syncthreads();

    int sq = 0;
    for (; sq + 2 < ntiles; sq += 3) {
      k_tile(sq, B0{});
      k_tile(sq + 1, B1{});
      k_tile(sq + 2, B2{});
    }
    if (sq < ntiles) k_tile(sq, B0{});
    if (sq + 1 < ntiles) k_tile(sq + 1, B1{});

    // every wave has passed the last tile's barrier: start the next unit,
    // then store this one's dQ = scale * dQ^T (lane holds query qw0 + r,
    // d = 32db + acc_row(j, h))
    const bool valid = wave_valid && (!TAIL || qw0 + r < N);   // rows past the end are not stored
    T* const qrow_out = STRIDED ? dQ + ((bh / H) * ldq.sb + (bh % H) * ldq.sh + (int64_t)(qw0 + r) * ldq.sn)
                                : dQ + head + (size_t)(qw0 + r) * D;
    unit = xcd_snake_unit((int)blockIdx.x, (int)gridDim.x, BH * nqb, ++round);
    if (unit >= 0) {
      set_unit(unit);
      copy_tile(tile_of(0), 0);
      if (ntiles > 1) copy_tile(tile_of(1), 1);
      load_q();
    }
    if (valid) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          v4 ov;
          ov[0] = (T)(acc[db][4 * jg + 0] * scale);
          ov[1] = (T)(acc[db][4 * jg + 1] * scale);
          ov[2] = (T)(acc[db][4 * jg + 2] * scale);
          ov[3] = (T)(acc[db][4 * jg + 3] * scale);
          *(v4*)(qrow_out + db * 32 + 8 * jg + 4 * h) = ov;
        }
    }
    if (unit < 0) break;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  }
}

template <typename E, int D, bool CAUSAL, bool TAIL, bool STRIDED, bool ALIBI, bool DROP>
hipError_t launch_bwd_cfg(const BwdArgs& a) {
  constexpr int NWK = 4;            // dK/dV: waves per workgroup (32 keys each)
  constexpr int NWQ = ATTN_DQ_NW;
  constexpr int BNQ = ATTN_DQ_BN;
  const int BH = (int)(a.B * a.H);
  const int N = (int)a.N;
  const int Np = (int)bwd_padded_n(a.N);
  using T = typename E::T;
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* o = (const T*)a.o;
  const T* dO = (const T*)a.dO;
  // STRIDED: the preprocess reads the inputs in their layouts and writes
  // contiguous copies of Q, K, V, dO, which the dK/dV and dQ kernels read
  T* qc = (T*)a.qc;
  T* kc = (T*)a.kc;
  T* vc = (T*)a.vc;
  T* doc = (T*)a.doc;
  const T* q2 = STRIDED ? qc : q;
  const T* k2 = STRIDED ? kc : k;
  const T* v2 = STRIDED ? vc : v;
  const T* dO2 = STRIDED ? doc : dO;
  Lay lq = a.lq, lk = a.lk, lv = a.lv, lo = a.lo, ldo = a.ldo, ldq = a.ldq, ldk = a.ldk, ldv = a.ldv;
  int H = (int)a.H;
  const float* slopes = a.alibi_slopes;
  DropCfg drop = a.drop;
  const float* lse = a.lse;
  T* dq = (T*)a.dq;
  T* dk = (T*)a.dk;
  T* dv = (T*)a.dv;
  float* delta = a.delta;
  float* nlse = a.nlse;
  T* qt = (T*)a.qt;
  T* kt = (T*)a.kt;
  T* dot = (T*)a.dot;
  T* qtail = (T*)a.qtail;
  T* dotail = (T*)a.dotail;
  T* ktail = (T*)a.ktail;
  T* vtail = (T*)a.vtail;
  float scale = a.scale;
  float scale_log2 = a.scale * kLog2e;
  float inv_scale = (float)(1.0 / (double)a.scale);

  {
    void* args[] = {(void*)&q,   (void*)&k,     (void*)&v,    (void*)&o,     (void*)&dO,    (void*)&lse,
                    (void*)&delta, (void*)&nlse, (void*)&qt, (void*)&kt, (void*)&dot, (void*)&qtail,
                    (void*)&dotail, (void*)&ktail, (void*)&vtail, (void*)&N, (void*)&Np, (void*)&inv_scale,
                    (void*)&lq, (void*)&lk, (void*)&lv, (void*)&lo, (void*)&ldo, (void*)&H, (void*)&qc, (void*)&kc,
                    (void*)&vc, (void*)&doc};
    hipError_t e = launch_kernel((const void*)bwd_prep<E, D, TAIL, STRIDED>, dim3((unsigned)(BH * (Np / 64))), dim3(256), args,
                                 a.stream, 1);
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (N + NWK * 32 - 1) / (NWK * 32);
    void* args[] = {(void*)&q2,    (void*)&k2, (void*)&v2, (void*)&dO2, (void*)&qt,  (void*)&dot,
                    (void*)&qtail, (void*)&dotail, (void*)&nlse, (void*)&delta, (void*)&dk, (void*)&dv,
                    (void*)&BH, (void*)&N, (void*)&Np, (void*)&nkb, (void*)&scale, (void*)&scale_log2,
                    (void*)&ldk, (void*)&ldv, (void*)&H, (void*)&slopes, (void*)&drop};
    const void* fn = (const void*)bwd_dkdv<E, D, CAUSAL, NWK, 64, TAIL, STRIDED, ALIBI, DROP>;
    hipError_t e = launch_kernel(fn, dim3((unsigned)persistent_grid(fn, NWK * 64, nkb * BH)), dim3(NWK * 64), args,
                                 a.stream, 2);
    if (e != hipSuccess) return e;
  }
  {
    const int nqb = (N + NWQ * 32 - 1) / (NWQ * 32);
    void* args[] = {(void*)&q2,   (void*)&k2, (void*)&v2, (void*)&dO2, (void*)&kt, (void*)&ktail, (void*)&vtail,
                    (void*)&nlse, (void*)&delta, (void*)&dq, (void*)&BH, (void*)&N, (void*)&Np, (void*)&nqb,
                    (void*)&scale, (void*)&scale_log2, (void*)&ldq, (void*)&H, (void*)&slopes, (void*)&drop};
    const void* fn = (const void*)bwd_dq<E, D, CAUSAL, NWQ, BNQ, TAIL, STRIDED, ALIBI, DROP>;
    return launch_kernel(fn, dim3((unsigned)persistent_grid(fn, NWQ * 64, nqb * BH)), dim3(NWQ * 64), args,
                         a.stream, 3);
  }
}

template <typename E, int D, bool STRIDED, bool ALIBI, bool DROP = false>
hipError_t launch_bwd_s(const BwdArgs& a) {
  if (a.N % 64 == 0) {
    if (a.causal) return launch_bwd_cfg<E, D, true, false, STRIDED, ALIBI, DROP>(a);
    return launch_bwd_cfg<E, D, false, false, STRIDED, ALIBI, DROP>(a);
  }
  if (a.causal) return launch_bwd_cfg<E, D, true, true, STRIDED, ALIBI, DROP>(a);
  return launch_bwd_cfg<E, D, false, true, STRIDED, ALIBI, DROP>(a);
}

// ALiBi calls are contiguous, and ALiBi and dropout are never combined (no
// entry point of the C ABI takes both)
template <typename E, int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  if (a.drop.t) return a.strided ? launch_bwd_s<E, D, true, false, true>(a) : launch_bwd_s<E, D, false, false, true>(a);
  if (a.alibi_slopes) return launch_bwd_s<E, D, false, true>(a);
  return a.strided ? launch_bwd_s<E, D, true, false>(a) : launch_bwd_s<E, D, false, false>(a);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? launch_bwd_d<bf16_t, 64>(a) : launch_bwd_d<bf16_t, 128>(a);
  return a.d == 64 ? launch_bwd_d<f16_t, 64>(a) : launch_bwd_d<f16_t, 128>(a);
}

}  // namespace attn
