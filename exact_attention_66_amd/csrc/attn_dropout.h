// Dropout on the attention probabilities, generated inside the kernels.
//
// Method: dropout is one of the elementwise steps fused into the attention
// kernel (page "FlashAttention技术解析 如何让GPT训练速度提升5-9倍" §2.2; the
// dropout_p argument of page "Flash Attention V2 大模型时代的算力救星" §4.2).
// The pages name no generator; this library draws with Philox4x32-10
// (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
// 3", SC 2011), a counter-based generator, so that the forward and both
// backward kernels regenerate the same mask from (position, seed) without
// storing it.
//
// Mask: the 4 x 4 block of (query, key) rows (4a .. 4a+3, 4b .. 4b+3) of head
// bh = b * H + h is one generator call with counter (a, b, bh, offset) and key
// (seed low word, seed high word); query 4a + u takes output word u, key
// 4b + c byte c of it (least significant first).  An element is dropped when
// its byte is below t = floor(256 p + 1/2) and kept ones are scaled by
// 256 / (256 - t).
//
// In every kernel the four lanes of a quad (lanes 4a' .. 4a'+3) hold the
// same four runs of 4 consecutive keys (or queries) for four consecutive
// queries (or keys), i.e. four 4 x 4 blocks: each lane makes one generator
// call, for block u = lane % 4, and a two-step butterfly over the quad
// (quad_transpose) hands every lane the word of each block that belongs to
// its own row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return u32x4{c0, c1, c2, c3};
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_quad(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}

// Transpose of the 4 x 4 word matrix held by a quad: lane u holds w = M[u][.]
// and receives M[.][u].  Step one exchanges 2 x 2 blocks between lanes u and
// u ^ 2, step two the off-diagonal words of each block between u and u ^ 1.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 w, int u) {
  constexpr int kXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);   // quad_perm [2, 3, 0, 1]
  constexpr int kXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);   // quad_perm [1, 0, 3, 2]
  const bool b1 = (u & 2) != 0, b0 = (u & 1) != 0;
  {
    const uint32_t r0 = dpp_quad<kXor2>(b1 ? w[0] : w[2]);
    const uint32_t r1 = dpp_quad<kXor2>(b1 ? w[1] : w[3]);
    w = b1 ? u32x4{r0, r1, w[2], w[3]} : u32x4{w[0], w[1], r0, r1};
  }
  {
    const uint32_t r0 = dpp_quad<kXor1>(b0 ? w[0] : w[1]);
    const uint32_t r1 = dpp_quad<kXor1>(b0 ? w[2] : w[3]);
    w = b0 ? u32x4{r0, w[1], r1, w[3]} : u32x4{w[0], r0, w[2], r1};
  }
  return w;
}

// The four bytes of a word spread to the 16-bit halves of two words (bytes
// 0, 1 -> lo; 2, 3 -> hi), each plus 256 - t: bit 8 of a half is then set
// exactly when its byte is >= t, i.e. when the element is kept.
__device__ __forceinline__ void keep_halves(uint32_t x, uint32_t add, uint32_t& lo, uint32_t& hi) {
  lo = ((x & 0xFFu) | ((x & 0xFF00u) << 8)) + add;
  hi = (((x >> 16) & 0xFFu) | ((x >> 8) & 0xFF0000u)) + add;
}

// 16-bit element masks (0xFFFF kept, 0 dropped) of the two halves.
__device__ __forceinline__ uint32_t half_masks(uint32_t y) { return ((y >> 8) & 0x00010001u) * 0xFFFFu; }

// 32-bit mask (all ones kept, 0 dropped) of half c (0, 1) of y.
__device__ __forceinline__ uint32_t full_mask(uint32_t y, int c) {
  return 0u - ((y >> (8 + 16 * c)) & 1u);
}

// a where the mask is all ones, b where it is 0 (one v_bfi_b32)
__device__ __forceinline__ float bit_select(uint32_t m, float a, float b) {
  return __builtin_bit_cast(float, (m & __builtin_bit_cast(uint32_t, a)) | (~m & __builtin_bit_cast(uint32_t, b)));
}

}  // namespace attn
