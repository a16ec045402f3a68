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
//  1. bwd_prep: D_i = dO_i . O_i (fp32), and transposed copies Q^T, dO^T,
//     K^T ([B*H][d][N]) in the workspace.  Inside every group of 16 tokens
//     the copies store tokens in MFMA reduction-slot order (slot_key), so
//     each operand fragment the main kernels need is one contiguous 16-byte
//     LDS read; the LDS transpose reads happen once here instead of once per
//     wave per tile.
//  2. bwd_dkdv: one workgroup per (batch*head, block of 32*NW keys).  Each
//     wave keeps its 32 keys' K and V as MFMA operands and their dK, dV fp32
//     accumulators for the whole sweep over query tiles.  S = Q K^T and
//     dP = dO V^T put one key per lane, so P and dS are directly the A
//     operands of dV += P^T dO and dK += dS^T Q (B operands from the
//     transposed tiles).
//  3. bwd_dq: one workgroup per (batch*head, block of 32*NW queries), shaped
//     like the forward: each wave keeps Q and dO rows as operands and dQ^T
//     in accumulators, computes S^T = K Q^T and dP^T = V dO^T (one query per
//     lane: lse and D are per-lane scalars), and adds dQ^T += K^T dS^T.
// The price of (3) is recomputing S and dP once more (7 matrix products in
// total instead of 5); in exchange there is no cross-workgroup reduction.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

#ifndef ATTN_DKDV_NW
#define ATTN_DKDV_NW 4   // waves per workgroup (32 keys each)
#endif
#ifndef ATTN_DKDV_BMQ
#define ATTN_DKDV_BMQ 64  // queries per LDS tile
#endif
#ifndef ATTN_DKDV_MINW
#define ATTN_DKDV_MINW 1  // waves per SIMD the register budget is sized for
#endif
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
// One workgroup per (batch*head, 64-token block).  Q, K, dO tiles go through
// swizzled LDS; the transposed copies are read back with ds_read_b64_tr_b16
// (lane gets 4 tokens of one d column, twice = 8 tokens in slot order) and
// written as 16-byte rows of [d][token].
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_prep(const typename E::T* __restrict__ Q,
                                                const typename E::T* __restrict__ K,
                                                const typename E::T* __restrict__ O,
                                                const typename E::T* __restrict__ dO,
                                                float* __restrict__ Dvec, typename E::T* __restrict__ QT,
                                                typename E::T* __restrict__ KT, typename E::T* __restrict__ dOT,
                                                int N) {
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
  const int nrb = N / R;
  const int bh = (int)(blockIdx.x / nrb);
  const int rb = (int)(blockIdx.x % nrb);
  const size_t head = (size_t)bh * N * D;
  const size_t row0 = (size_t)rb * R;

#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = tid + c * 256;
    const int row = idx / CPR;
    const int col = (idx % CPR) * 8;
    const size_t g = head + (row0 + row) * D + col;
    const v8 qv = *(const v8*)(Q + g);
    const v8 kv = *(const v8*)(K + g);
    const v8 dov = *(const v8*)(dO + g);
    const v8 ov = *(const v8*)(O + g);
    *(v8*)(&tile[0][swz<D>(row, col)]) = qv;
    *(v8*)(&tile[1][swz<D>(row, col)]) = kv;
    *(v8*)(&tile[2][swz<D>(row, col)]) = dov;
    // D_i: the CPR chunks of a row are held by CPR consecutive lanes
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)ov[i], (float)dov[i], acc);
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CPR);
    if ((idx % CPR) == 0) Dvec[(size_t)bh * N + row0 + row] = acc;
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
      *(v8*)(outs[t] + head + (size_t)(db * 32 + r) * N + row0 + pg * 16 + 8 * h) = val;
    }
  }
}

// ---------------------------------------------------------------- dK, dV
// LDS tiles here are read only with ds_read_b128 by 16 lanes of 16
// consecutive rows at the same column, so plain row padding keeps them free
// of bank conflicts and their addresses affine (one per-lane base plus
// immediate offsets): rows of D + 8 elements (D*2 + 16 bytes, 4 banks of
// shift per row) and, for the transposed tiles, rows of BMQ + 8 elements
// (BMQ = 64: 144 bytes, 36 banks of shift: 16 distinct 4-bank groups).
template <typename E, int D, bool CAUSAL, int NW, int BMQ>
__global__ __launch_bounds__(NW * 64, ATTN_DKDV_MINW) void bwd_dkdv(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const typename E::T* __restrict__ QT, const typename E::T* __restrict__ dOT,
    const float* __restrict__ LSE, const float* __restrict__ Dvec, typename E::T* __restrict__ dK,
    typename E::T* __restrict__ dV, int BH, int N, int nkb, float scale, float scale_log2) {
  using T = typename E::T;
  using v8 = typename E::v8;
  constexpr int BN = NW * 32;     // keys per workgroup
  constexpr int KS = D / 16;      // reduction steps over d
  constexpr int DB = D / 32;      // 32-wide d blocks
  constexpr int QSB = BMQ / 32;   // 32-query sub-blocks per tile
  constexpr int NT = NW * 64;
  constexpr int CHUNKS = BMQ * D / 8;       // 16-byte chunks per tile
  constexpr int CPT = (CHUNKS + NT - 1) / NT;  // chunks per thread per tile
  constexpr int LR = D + 8;       // row-major tile row (elements)
  constexpr int LT = BMQ + 8;     // transposed tile row (elements)
  static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "query tile must split evenly over threads");
  static_assert(BMQ <= NT, "lse/D staging uses one thread per query");

  __shared__ __attribute__((aligned(16))) T lds_q[2][BMQ * LR];
  __shared__ __attribute__((aligned(16))) T lds_do[2][BMQ * LR];
  __shared__ __attribute__((aligned(16))) T lds_qt[2][D * LT];
  __shared__ __attribute__((aligned(16))) T lds_dot[2][D * LT];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][BMQ];
  __shared__ __attribute__((aligned(16))) float lds_dd[2][BMQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int r = lane & 31;

  int kblk, bh;
  if (CAUSAL) {  // key blocks near the start see the most queries: run them first
    kblk = (int)(blockIdx.x / BH);
    bh = (int)(blockIdx.x % BH);
  } else {
    bh = (int)(blockIdx.x / nkb);
    kblk = (int)(blockIdx.x % nkb);
  }
  const int kb0 = kblk * BN;
  const int kw0 = kb0 + w * 32;            // first key of this wave
  const bool wave_valid = kw0 < N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const T* Qh = Q + head;
  const T* dOh = dO + head;
  const T* QTh = QT + head;
  const T* dOTh = dOT + head;
  const float* lse_h = LSE + (size_t)bh * N;
  const float* dd_h = Dvec + (size_t)bh * N;

  // this wave's K and V as B operands: lane holds row kw0 + r, d = 16ks + 8h .. +7
  v8 kB[KS], vB[KS];
  {
    const int key = min(kw0 + r, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kB[ks] = *(const v8*)(K + head + (size_t)key * D + ks * 16 + 8 * h);
      vB[ks] = *(const v8*)(V + head + (size_t)key * D + ks * 16 + 8 * h);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      materialize(kB[ks]);
      materialize(vB[ks]);
    }
  }
  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  // per-lane parts of the LDS read addresses (element offsets); everything
  // else in an address is a compile-time immediate
  const int offA = opaque(r * LR + 8 * h);      // row-major tiles: row r, column 8h
  const int offB = opaque(r * LT + 8 * h);      // transposed tiles: row r (d), column 8h
  const int offL = opaque(4 * h);               // lse / D: 4 consecutive queries

  const int nqt = N / BMQ;
  const int it0 = CAUSAL ? kb0 / BMQ : 0;

  v8 qreg[CPT], doreg[CPT], qtreg[CPT], dotreg[CPT];
  float lse_reg = 0.f, d_reg = 0.f;
  auto gload = [&](int it) {
    const int qt0 = it * BMQ;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      if (idx >= CHUNKS) break;
      const int row = idx / (D / 8);           // row-major tile: query, d chunk
      const int col = (idx % (D / 8)) * 8;
      qreg[c] = *(const v8*)(Qh + (size_t)(qt0 + row) * D + col);
      doreg[c] = *(const v8*)(dOh + (size_t)(qt0 + row) * D + col);
      const int trow = idx / (BMQ / 8);        // transposed tile: d, token chunk
      const int tcol = (idx % (BMQ / 8)) * 8;
      qtreg[c] = *(const v8*)(QTh + (size_t)trow * N + qt0 + tcol);
      dotreg[c] = *(const v8*)(dOTh + (size_t)trow * N + qt0 + tcol);
    }
    if (tid < BMQ) {
      lse_reg = lse_h[qt0 + tid];
      d_reg = dd_h[qt0 + tid];
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      if (idx >= CHUNKS) break;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      *(v8*)(&lds_q[buf][row * LR + col]) = qreg[c];
      *(v8*)(&lds_do[buf][row * LR + col]) = doreg[c];
      const int trow = idx / (BMQ / 8);
      const int tcol = (idx % (BMQ / 8)) * 8;
      *(v8*)(&lds_qt[buf][trow * LT + tcol]) = qtreg[c];
      *(v8*)(&lds_dot[buf][trow * LT + tcol]) = dotreg[c];
    }
    if (tid < BMQ) {
      lds_lse[buf][tid] = lse_reg * kLog2e;
      lds_dd[buf][tid] = d_reg;
    }
  };

  // one 32-query sub-block: S, dP, softmax, dV, dK
  auto sub_tile = [&](const int buf, const int qs, const int qs0) {
    const T* ql = lds_q[buf] + offA + qs * 32 * LR;
    const T* dol = lds_do[buf] + offA + qs * 32 * LR;
    const T* qtl = lds_qt[buf] + offB + qs * 32;
    const T* dotl = lds_dot[buf] + offB + qs * 32;
    // every LDS read of the S/dP operands is issued before their MFMAs
    v8 qa[KS], da[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = *(const v8*)(ql + ks * 16);
      da[ks] = *(const v8*)(dol + ks * 16);
    }
    sched_fence();
    // S = Q K^T and dP = dO V^T: lane holds key kw0 + r, queries acc_row(j, h)
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sacc = E::mfma32(qa[ks], kB[ks], sacc);
      dpacc = E::mfma32(da[ks], vB[ks], dpacc);
    }
    sched_fence();
    // operands of the dV / dK products and the row statistics: their reads
    // do not depend on the softmax, so their latency hides behind it
    v8 dob[2][DB], qbv[2][DB];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dob[kk][db] = *(const v8*)(dotl + db * 32 * LT + 16 * kk);
        qbv[kk][db] = *(const v8*)(qtl + db * 32 * LT + 16 * kk);
      }
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      l4[jg] = *(const f32x4*)(&lds_lse[buf][offL + qs * 32 + 8 * jg]);
      d4[jg] = *(const f32x4*)(&lds_dd[buf][offL + qs * 32 + 8 * jg]);
    }
    sched_fence();
    float p[16], ds[16];
#pragma unroll
    for (int jg = 0; jg < 4; ++jg)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = 4 * jg + u;
        p[j] = fast_exp2(fmaf(sacc[j], scale_log2, -l4[jg][u]));
      }
    if (CAUSAL && qs0 < kw0 + 31) {   // sub-block crosses the diagonal: key > query -> P = 0
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kw0 + r > qs0 + acc_row(j, h)) p[j] = 0.f;
    }
#pragma unroll
    for (int jg = 0; jg < 4; ++jg)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = 4 * jg + u;
        ds[j] = p[j] * (dpacc[j] - d4[jg][u]);
      }
    // dV += P^T dO and dK += dS^T Q (scale applied at the end)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const v8 pa = pack8<E>(p[8 * kk + 0], p[8 * kk + 1], p[8 * kk + 2], p[8 * kk + 3], p[8 * kk + 4],
                             p[8 * kk + 5], p[8 * kk + 6], p[8 * kk + 7]);
      const v8 sa = pack8<E>(ds[8 * kk + 0], ds[8 * kk + 1], ds[8 * kk + 2], ds[8 * kk + 3], ds[8 * kk + 4],
                             ds[8 * kk + 5], ds[8 * kk + 6], ds[8 * kk + 7]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dv_acc[db] = E::mfma32(pa, dob[kk][db], dv_acc[db]);
        dk_acc[db] = E::mfma32(sa, qbv[kk][db], dk_acc[db]);
      }
    }
  };

  if (it0 < nqt) {
    gload(it0);
    lstore(it0 & 1);
  }
  wait_all_vmem_loads();
  __syncthreads();

  auto q_tile = [&](const int it, const int buf) {
    const int qt0 = it * BMQ;
    if (it + 1 < nqt) gload(it + 1);
#pragma unroll
    for (int qs = 0; qs < QSB; ++qs) {
      const int qs0 = qt0 + qs * 32;
      if (wave_valid && (!CAUSAL || qs0 + 31 >= kw0)) sub_tile(buf, qs, qs0);
    }
    if (it + 1 < nqt) lstore(buf ^ 1);
    mfma_drain();
    __syncthreads();
  };
  // unrolled by two so that the LDS buffer index is a compile-time constant
  int it = it0;
  if (it < nqt && (it & 1)) {
    q_tile(it, 1);
    ++it;
  }
  for (; it + 1 < nqt; it += 2) {
    q_tile(it, 0);
    q_tile(it + 1, 1);
  }
  if (it < nqt) q_tile(it, 0);

  if (!wave_valid) return;
  // epilogue: dK = scale * acc, dV = acc; lane holds key kw0 + acc_row(j, h), d = 32db + r
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const size_t off = head + (size_t)(kw0 + acc_row(j, h)) * D + db * 32 + r;
      dK[off] = (T)(dk_acc[db][j] * scale);
      dV[off] = (T)dv_acc[db][j];
    }
}

// ---------------------------------------------------------------- dQ
// Same padding rule as above: K and V tiles [BN][D + 8], K^T tile [D][BN + 8].
template <typename E, int D, bool CAUSAL, int NW, int BN>
__global__ __launch_bounds__(NW * 64, ATTN_DQ_MINW) void bwd_dq(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const typename E::T* __restrict__ KT, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    typename E::T* __restrict__ dQ, int BH, int N, int nqb, float scale, float scale_log2) {
  using T = typename E::T;
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  constexpr int BM = NW * 32;        // queries per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KB = BN / 32;        // 32-key blocks per tile
  constexpr int NT = NW * 64;
  constexpr int CHUNKS = BN * D / 8;
  constexpr int CPT = (CHUNKS + NT - 1) / NT;
  constexpr int LR = D + 8;
  constexpr int LT = BN + 8;
  static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "key tile must split evenly over threads");

  __shared__ __attribute__((aligned(16))) T lds_k[2][BN * LR];
  __shared__ __attribute__((aligned(16))) T lds_v[2][BN * LR];
  __shared__ __attribute__((aligned(16))) T lds_kt[2][D * LT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int r = lane & 31;

  int qblk, bh;
  if (CAUSAL) {  // heaviest query blocks first
    qblk = nqb - 1 - (int)(blockIdx.x / BH);
    bh = (int)(blockIdx.x % BH);
  } else {
    bh = (int)(blockIdx.x / nqb);
    qblk = (int)(blockIdx.x % nqb);
  }
  const int q0 = qblk * BM;
  const int qw0 = q0 + w * 32;
  const bool wave_valid = qw0 < N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const T* Kh = K + head;
  const T* Vh = V + head;
  const T* KTh = KT + head;

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T
  const int qrow = min(qw0 + r, N - 1);
  v8 qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = *(const v8*)(Q + head + (size_t)qrow * D + ks * 16 + 8 * h);
    dof[ks] = *(const v8*)(dO + head + (size_t)qrow * D + ks * 16 + 8 * h);
  }
  const float lse2 = LSE[(size_t)bh * N + qrow] * kLog2e;
  const float dd = Dvec[(size_t)bh * N + qrow];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    materialize(qf[ks]);
    materialize(dof[ks]);
  }
  materialize(lse2);
  materialize(dd);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  const int offA = opaque(r * LR + 8 * h);
  const int offB = opaque(r * LT + 8 * h);

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int q_last = qw0 + 31;

  v8 kreg[CPT], vreg[CPT], ktreg[CPT];
  auto gload = [&](int t) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      if (idx >= CHUNKS) break;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      const int key = min(t * BN + row, N - 1);
      kreg[c] = *(const v8*)(Kh + (size_t)key * D + col);
      vreg[c] = *(const v8*)(Vh + (size_t)key * D + col);
      const int trow = idx / (BN / 8);
      const int tcol = (idx % (BN / 8)) * 8;
      ktreg[c] = *(const v8*)(KTh + (size_t)trow * N + min(t * BN + tcol, N - 8));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      if (idx >= CHUNKS) break;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      *(v8*)(&lds_k[buf][row * LR + col]) = kreg[c];
      *(v8*)(&lds_v[buf][row * LR + col]) = vreg[c];
      const int trow = idx / (BN / 8);
      const int tcol = (idx % (BN / 8)) * 8;
      *(v8*)(&lds_kt[buf][trow * LT + tcol]) = ktreg[c];
    }
  };

  auto key_block = [&](const int buf, const int kb, const int kbk0) {
    const T* kl = lds_k[buf] + offA + kb * 32 * LR;
    const T* vl = lds_v[buf] + offA + kb * 32 * LR;
    const T* ktl = lds_kt[buf] + offB + kb * 32;
    // S^T = K Q^T, dP^T = V dO^T: lane holds query qw0 + r, keys acc_row(j, h).
    // Operand reads go in batches of KSTAGE per operand, each batch issued
    // ahead of its MFMAs.
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
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
#pragma unroll
    for (int j = 0; j < 16; ++j) ds[j] = fast_exp2(fmaf(sacc[j], scale_log2, -lse2));
    if (CAUSAL && kbk0 + 31 > qw0) {   // block crosses the diagonal: key > query -> P = 0
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kbk0 + acc_row(j, h) > qw0 + r) ds[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) ds[j] = ds[j] * (dpacc[j] - dd);
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

  gload(0);
  lstore(0);
  wait_all_vmem_loads();
  __syncthreads();

  auto k_tile = [&](const int t, const int buf) {
    if (t + 1 < ntiles) gload(t + 1);
    const int k0 = t * BN;
    if (wave_valid && (!CAUSAL || k0 <= q_last)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int kbk0 = k0 + kb * 32;
        if (!CAUSAL || kbk0 <= q_last) key_block(buf, kb, kbk0);
      }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    mfma_drain();
    __syncthreads();
  };
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    k_tile(t, 0);
    k_tile(t + 1, 1);
  }
  if (t < ntiles) k_tile(t, 0);

  if (!wave_valid) return;
  // epilogue: dQ = scale * dQ^T; lane holds query qw0 + r, d = 32db + acc_row(j, h)
  T* qrow_out = dQ + head + (size_t)(qw0 + r) * D;
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

template <typename E, int D, bool CAUSAL>
hipError_t launch_bwd_cfg(const BwdArgs& a) {
  constexpr int NWK = ATTN_DKDV_NW;
  constexpr int BMQ = ATTN_DKDV_BMQ;
  constexpr int NWQ = ATTN_DQ_NW;
  constexpr int BNQ = ATTN_DQ_BN;
  const int BH = (int)(a.B * a.H);
  const int N = (int)a.N;
  using T = typename E::T;
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* o = (const T*)a.o;
  const T* dO = (const T*)a.dO;
  const float* lse = a.lse;
  T* dq = (T*)a.dq;
  T* dk = (T*)a.dk;
  T* dv = (T*)a.dv;
  float* delta = a.delta;
  T* qt = (T*)a.qt;
  T* kt = (T*)a.kt;
  T* dot = (T*)a.dot;
  float scale = a.scale;
  float scale_log2 = a.scale * kLog2e;

  {
    void* args[] = {(void*)&q, (void*)&k, (void*)&o, (void*)&dO, (void*)&delta, (void*)&qt, (void*)&kt,
                    (void*)&dot, (void*)&N};
    hipError_t e = launch_kernel((const void*)bwd_prep<E, D>, dim3((unsigned)(BH * (N / 64))), dim3(256), args,
                                 a.stream, 1);
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (N + NWK * 32 - 1) / (NWK * 32);
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dO, (void*)&qt, (void*)&dot, (void*)&lse,
                    (void*)&delta, (void*)&dk, (void*)&dv, (void*)&BH, (void*)&N, (void*)&nkb,
                    (void*)&scale, (void*)&scale_log2};
    hipError_t e = launch_kernel((const void*)bwd_dkdv<E, D, CAUSAL, NWK, BMQ>, dim3((unsigned)(nkb * BH)),
                                 dim3(NWK * 64), args, a.stream, 2);
    if (e != hipSuccess) return e;
  }
  {
    const int nqb = (N + NWQ * 32 - 1) / (NWQ * 32);
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dO, (void*)&kt, (void*)&lse, (void*)&delta,
                    (void*)&dq, (void*)&BH, (void*)&N, (void*)&nqb, (void*)&scale, (void*)&scale_log2};
    return launch_kernel((const void*)bwd_dq<E, D, CAUSAL, NWQ, BNQ>, dim3((unsigned)(nqb * BH)), dim3(NWQ * 64),
                         args, a.stream, 3);
  }
}

template <typename E, int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  if (a.causal) return launch_bwd_cfg<E, D, true>(a);
  return launch_bwd_cfg<E, D, false>(a);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? launch_bwd_d<bf16_t, 64>(a) : launch_bwd_d<bf16_t, 128>(a);
  return a.d == 64 ? launch_bwd_d<f16_t, 64>(a) : launch_bwd_d<f16_t, 128>(a);
}

}  // namespace attn
