// The dropout draws themselves: writes the 8-bit generator output that the
// attention kernels compare with the drop threshold, for every (query, key)
// of the requested heads, so that a caller can see or reuse the mask.
//
// Method: dropout on the attention probabilities (page "FlashAttention技术解析
// 如何让GPT训练速度提升5-9倍" §2.2); generator and mask layout as in
// attn_dropout.h.  The kernel walks the same lane layout as the forward
// kernel (one query per lane, keys kbk0 + 8m + 4h + c of a 32-key block) and
// the same per-quad generator calls and transpose, so its output is exactly
// what the forward and backward kernels draw.
#include "attn_device.h"
#include "attn_dropout.h"
#include "attn_launch.h"

namespace attn {

namespace {

// One wave per (head, 32-query block, 32-key block); the unit index is the
// same for the whole wave, so every lane of a quad takes part in the
// transpose.
__global__ __launch_bounds__(256) void dropout_draws_kernel(uint8_t* __restrict__ out, int BH, int Nq, int Nk,
                                                            int nqb, int nkb, DropCfg drop) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31, u = lane & 3;
  const int64_t units = (int64_t)BH * nqb * nkb;
  for (int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); unit < units; unit += (int64_t)gridDim.x * 4) {
    const int kb = (int)(unit % nkb);
    const int64_t rest = unit / nkb;
    const int qb = (int)(rest % nqb);
    const int bh = (int)(rest / nqb);
    const int q = qb * 32 + r;
    const int kbk0 = kb * 32;
    const u32x4 tw = quad_transpose(philox4x32_10((uint32_t)q >> 2, (uint32_t)((kbk0 >> 2) + 2 * u + h),
                                                  (uint32_t)bh, drop.offset, drop.key0, drop.key1),
                                    u);
    if (q < Nq) {
      uint8_t* row = out + ((size_t)bh * Nq + q) * Nk;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int key = kbk0 + 8 * m + 4 * h + c;
          if (key < Nk) row[key] = (uint8_t)((tw[m] >> (8 * c)) & 0xFFu);
        }
    }
  }
}

}  // namespace

hipError_t launch_dropout_draws(uint8_t* out, int64_t BH, int64_t Nq, int64_t Nk, const DropCfg& drop,
                                hipStream_t stream) {
  int bh = (int)BH, nq = (int)Nq, nk = (int)Nk;
  int nqb = (nq + 31) / 32, nkb = (nk + 31) / 32;
  const int64_t units = BH * nqb * nkb;
  const int64_t want = (units + 3) / 4;
  dim3 grid((unsigned)(want < 4096 ? want : 4096)), block(256);
  DropCfg d = drop;
  void* args[] = {(void*)&out, (void*)&bh, (void*)&nq, (void*)&nk, (void*)&nqb, (void*)&nkb, (void*)&d};
  return hipLaunchKernel((const void*)dropout_draws_kernel, grid, block, args, 0, stream);
}

}  // namespace attn
