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
// Three kernels on the caller's stream:
//  1. bwd_pre:  D_i = dO_i . O_i (fp32) and zeroing of the fp32 dQ accumulator;
//  2. bwd_main: one workgroup per (batch*head, block of 32*NW keys); each
//     wave keeps its 32 keys' K and V as MFMA operands and their dK, dV in
//     fp32 accumulators for the whole sweep over query tiles (no atomics for
//     dK/dV); query tiles of Q, dO, lse, D are double-buffered in LDS;
//     S = Q K^T and dP = dO V^T put one key per lane, so P and dS feed the
//     dV and dK products directly; dS^T goes through LDS once so that
//     dQ += dS K can be split over waves by (query block, d block) and added
//     to the fp32 accumulator with atomics;
//  3. bwd_dq_cast: dQ = scale * accumulator, rounded to the I/O type.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------- preprocess
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_pre(const typename E::T* __restrict__ O,
                                               const typename E::T* __restrict__ dO,
                                               float* __restrict__ Dvec, float* __restrict__ dq_acc,
                                               int64_t rows) {
  using v8 = typename E::v8;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPB = 256 / CPR;        // rows per workgroup
  const int t = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + t / CPR;
  const int c = t % CPR;
  float acc = 0.f;
  if (row < rows) {
    const v8 a = *(const v8*)(O + row * D + c * 8);
    const v8 b = *(const v8*)(dO + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)a[i], (float)b[i], acc);
    f32x4* z = (f32x4*)(dq_acc + row * D + c * 8);
    z[0] = f32x4{};
    z[1] = f32x4{};
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CPR);
  if (row < rows && c == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------- dQ cast
template <typename E>
__global__ __launch_bounds__(256) void bwd_dq_cast(const float* __restrict__ acc, typename E::T* __restrict__ dq,
                                                   int64_t n8, float scale) {
  using v8 = typename E::v8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(acc + i * 8);
  const f32x4 b = *(const f32x4*)(acc + i * 8 + 4);
  *(v8*)(dq + i * 8) = pack8<E>(a[0] * scale, a[1] * scale, a[2] * scale, a[3] * scale, b[0] * scale,
                                b[1] * scale, b[2] * scale, b[3] * scale);
}

// ---------------------------------------------------------------- main kernel
template <typename E, int D, bool CAUSAL, int NW, int BMQ>
__global__ __launch_bounds__(NW * 64) void bwd_main(const typename E::T* __restrict__ Q,
                                                    const typename E::T* __restrict__ K,
                                                    const typename E::T* __restrict__ V,
                                                    const typename E::T* __restrict__ dO,
                                                    const float* __restrict__ LSE, const float* __restrict__ Dvec,
                                                    typename E::T* __restrict__ dK, typename E::T* __restrict__ dV,
                                                    float* __restrict__ dq_acc, int BH, int N, int nkb, float scale,
                                                    float scale_log2) {
  using T = typename E::T;
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  constexpr int BN = NW * 32;     // keys per workgroup
  constexpr int KS = D / 16;      // reduction steps over d
  constexpr int DB = D / 32;      // 32-wide d blocks
  constexpr int QSB = BMQ / 32;   // 32-query sub-blocks per query tile
  constexpr int LD = D + 8;       // padded row of the Q, dO, K tiles (elements)
  constexpr int LS = BMQ + 8;     // padded row of the dS^T tile (elements)
  constexpr int NT = NW * 64;
  constexpr int CPT = BMQ * D / 8 / NT;   // 16-byte chunks per thread per tile
  constexpr int KCPT = BN * D / 8 / NT;
  static_assert(CPT >= 1 && (BMQ * D / 8) % NT == 0, "query tile must split evenly over threads");
  static_assert(BMQ <= NT, "lse/D staging uses one thread per query");

  __shared__ __attribute__((aligned(16))) T lds_q[2][BMQ * LD];
  __shared__ __attribute__((aligned(16))) T lds_do[2][BMQ * LD];
  __shared__ __attribute__((aligned(16))) T lds_k[BN * LD];
  __shared__ __attribute__((aligned(16))) T lds_ds[BN * LS];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][BMQ];
  __shared__ __attribute__((aligned(16))) float lds_dv[2][BMQ];

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
  const T* Kh = K + head;
  const T* Vh = V + head;
  const T* dOh = dO + head;
  const float* lse_h = LSE + (size_t)bh * N;
  const float* dv_h = Dvec + (size_t)bh * N;
  float* dqa_h = dq_acc + head;

  // ---- K tile of the workgroup into LDS (B operand of dQ += dS K)
#pragma unroll
  for (int c = 0; c < KCPT; ++c) {
    const int idx = tid + c * NT;
    const int row = idx / (D / 8);
    const int col = (idx % (D / 8)) * 8;
    const int key = min(kb0 + row, N - 1);
    *(v8*)(&lds_k[row * LD + col]) = *(const v8*)(Kh + (size_t)key * D + col);
  }
  // ---- this wave's K and V as B operands: lane holds row kw0 + r, d = 16ks + 8h .. +7
  v8 kB[KS], vB[KS];
  {
    const int key = min(kw0 + r, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kB[ks] = *(const v8*)(Kh + (size_t)key * D + ks * 16 + 8 * h);
      vB[ks] = *(const v8*)(Vh + (size_t)key * D + ks * 16 + 8 * h);
    }
  }
  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  const int nqt = N / BMQ;
  const int it0 = CAUSAL ? kb0 / BMQ : 0;

  v8 qreg[CPT], doreg[CPT];
  float lse_reg = 0.f, d_reg = 0.f;
  auto gload = [&](int it) {
    const int qt0 = it * BMQ;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      qreg[c] = *(const v8*)(Qh + (size_t)(qt0 + row) * D + col);
      doreg[c] = *(const v8*)(dOh + (size_t)(qt0 + row) * D + col);
    }
    if (tid < BMQ) {
      lse_reg = lse_h[qt0 + tid] * kLog2e;
      d_reg = dv_h[qt0 + tid];
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      *(v8*)(&lds_q[buf][row * LD + col]) = qreg[c];
      *(v8*)(&lds_do[buf][row * LD + col]) = doreg[c];
    }
    if (tid < BMQ) {
      lds_lse[buf][tid] = lse_reg;
      lds_dv[buf][tid] = d_reg;
    }
  };

  if (it0 < nqt) {
    gload(it0);
    lstore(it0 & 1);
  }
  __syncthreads();

  // tr-read coordinates inside a 16-row reduction step
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int it = it0; it < nqt; ++it) {
    const int buf = it & 1;
    const int qt0 = it * BMQ;
    if (it + 1 < nqt) gload(it + 1);
    const T* ql = lds_q[buf];
    const T* dol = lds_do[buf];

#pragma unroll
    for (int qs = 0; qs < QSB; ++qs) {
      const int qs0 = qt0 + qs * 32;
      const bool any = wave_valid && (!CAUSAL || qs0 + 31 >= kw0);
      T* dsrow = lds_ds + (w * 32 + r) * LS + qs * 32 + 4 * h;
      if (any) {
        // S = Q K^T and dP = dO V^T: lane holds key kw0 + r, queries acc_row(j, h)
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const v8 qa = *(const v8*)(ql + (qs * 32 + r) * LD + ks * 16 + 8 * h);
          const v8 da = *(const v8*)(dol + (qs * 32 + r) * LD + ks * 16 + 8 * h);
          sacc = E::mfma32(qa, kB[ks], sacc);
          dpacc = E::mfma32(da, vB[ks], dpacc);
        }
        float p[16], ds[16];
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const f32x4 l4 = *(const f32x4*)(&lds_lse[buf][qs * 32 + 8 * jg + 4 * h]);
          const f32x4 d4 = *(const f32x4*)(&lds_dv[buf][qs * 32 + 8 * jg + 4 * h]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = 4 * jg + u;
            float pj = fast_exp2(fmaf(sacc[j], scale_log2, -l4[u]));
            if (CAUSAL && kw0 + r > qs0 + acc_row(j, h)) pj = 0.f;
            p[j] = pj;
            ds[j] = pj * (dpacc[j] - d4[u]);
          }
        }
        // dV += P^T dO and dK += dS^T Q (scale applied at the end)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const v8 pa = pack8<E>(p[8 * kk + 0], p[8 * kk + 1], p[8 * kk + 2], p[8 * kk + 3], p[8 * kk + 4],
                                 p[8 * kk + 5], p[8 * kk + 6], p[8 * kk + 7]);
          const v8 sa = pack8<E>(ds[8 * kk + 0], ds[8 * kk + 1], ds[8 * kk + 2], ds[8 * kk + 3], ds[8 * kk + 4],
                                 ds[8 * kk + 5], ds[8 * kk + 6], ds[8 * kk + 7]);
          const int row = qs * 32 + kk * 16 + tr_row;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const v8 dob = concat44<E>(E::tr_read(dol + row * LD + db * 32 + tr_col),
                                       E::tr_read(dol + (row + 8) * LD + db * 32 + tr_col));
            dv_acc[db] = E::mfma32(pa, dob, dv_acc[db]);
            const v8 qbv = concat44<E>(E::tr_read(ql + row * LD + db * 32 + tr_col),
                                       E::tr_read(ql + (row + 8) * LD + db * 32 + tr_col));
            dk_acc[db] = E::mfma32(sa, qbv, dk_acc[db]);
          }
          // dS^T tile for the dQ product: row = key, 4 consecutive queries per store
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            v4 o4;
            o4[0] = sa[4 * g + 0]; o4[1] = sa[4 * g + 1]; o4[2] = sa[4 * g + 2]; o4[3] = sa[4 * g + 3];
            *(v4*)(dsrow + 16 * kk + 8 * g) = o4;
          }
        }
      } else {
        const v4 z = {};
#pragma unroll
        for (int g = 0; g < 4; ++g) *(v4*)(dsrow + 8 * g) = z;
      }
    }
    __syncthreads();

    // ---- dQ(tile) += dS K over the workgroup's BN keys, split by (query block, d block)
    for (int b = w; b < QSB * DB; b += NW) {
      const int qb = b / DB;
      const int db = b % DB;
      if (CAUSAL && qt0 + qb * 32 + 31 < kb0) continue;  // every key of the block is masked
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kstep = 0; kstep < BN / 16; ++kstep) {
        const int row = kstep * 16 + tr_row;
        const v8 a = concat44<E>(E::tr_read(lds_ds + row * LS + qb * 32 + tr_col),
                                 E::tr_read(lds_ds + (row + 8) * LS + qb * 32 + tr_col));
        const v8 bk = concat44<E>(E::tr_read(lds_k + row * LD + db * 32 + tr_col),
                                  E::tr_read(lds_k + (row + 8) * LD + db * 32 + tr_col));
        acc = E::mfma32(a, bk, acc);
      }
      float* dst = dqa_h + (size_t)(qt0 + qb * 32) * D + db * 32 + r;
#pragma unroll
      for (int j = 0; j < 16; ++j) atomicAdd(dst + (size_t)acc_row(j, h) * D, acc[j]);
    }

    if (it + 1 < nqt) lstore(buf ^ 1);
    __syncthreads();
  }

  if (!wave_valid) return;
  // ---- epilogue: dK = scale * acc, dV = acc; lane holds key kw0 + acc_row(j, h), d = 32db + r
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const size_t off = (size_t)(kw0 + acc_row(j, h)) * D + db * 32 + r;
      dK[head + off] = (T)(dk_acc[db][j] * scale);
      dV[head + off] = (T)dv_acc[db][j];
    }
}

template <typename E, int D, bool CAUSAL, int NW, int BMQ>
hipError_t launch_bwd_cfg(const BwdArgs& a) {
  constexpr int BN = NW * 32;
  const int BH = (int)(a.B * a.H);
  const int N = (int)a.N;
  const int64_t rows = (int64_t)BH * N;
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
  float* dqa = a.dq_acc;
  float scale = a.scale;
  float scale_log2 = a.scale * kLog2e;

  {
    constexpr int RPB = 256 / (D / 8);
    void* args[] = {(void*)&o, (void*)&dO, (void*)&delta, (void*)&dqa, (void*)&rows};
    hipError_t e = launch_kernel((const void*)bwd_pre<E, D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                                 args, a.stream, 1);
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (N + BN - 1) / BN;
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dO, (void*)&lse, (void*)&delta, (void*)&dk,
                    (void*)&dv, (void*)&dqa, (void*)&BH, (void*)&N, (void*)&nkb, (void*)&scale,
                    (void*)&scale_log2};
    hipError_t e = launch_kernel((const void*)bwd_main<E, D, CAUSAL, NW, BMQ>, dim3((unsigned)(nkb * BH)),
                                 dim3(NW * 64), args, a.stream, 2);
    if (e != hipSuccess) return e;
  }
  {
    int64_t n8 = rows * D / 8;
    void* args[] = {(void*)&dqa, (void*)&dq, (void*)&n8, (void*)&scale};
    return launch_kernel((const void*)bwd_dq_cast<E>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), args,
                         a.stream, 3);
  }
}

template <typename E, int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  if (a.causal) return launch_bwd_cfg<E, D, true, 4, 64>(a);
  return launch_bwd_cfg<E, D, false, 4, 64>(a);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? launch_bwd_d<bf16_t, 64>(a) : launch_bwd_d<bf16_t, 128>(a);
  return a.d == 64 ? launch_bwd_d<f16_t, 64>(a) : launch_bwd_d<f16_t, 128>(a);
}

}  // namespace attn
