/*
 * attn.h - C ABI of the exact-attention library for AMD MI355X (gfx950).
 *
 * Exact scaled-dot-product attention, forward and backward, computed in
 * tiles with an online softmax so that the N x N score matrix never reaches
 * device memory.
 *
 *   Forward  O = softmax(scale * Q K^T  [causal mask]) V,  lse = per-row log-sum-exp.
 *   Backward dQ, dK, dV from Q, K, V, O, dO and lse, recomputing the scores.
 *
 * The operation is the attention of page "FlashAttention技术解析 如何让GPT训练
 * 速度提升5-9倍" §2.1 (plain softmax(QK^T / sqrt(d_k)) V, and the tiled form
 * that never stores the score matrix), with the softmax_scale and causal
 * arguments of page "Flash Attention V2 大模型时代的算力救星" §4.2; the
 * blockwise softmax follows page "突破单卡显存极限：FlashAttention-2技术解析与
 * 实战指南" §2.1, and the backward pass keeps only the softmax normalisation
 * statistic and recomputes the scores (page "Flash Attention V2 …" §3.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout:    Q, K, V, O, dO, dQ, dK, dV are contiguous [B, H, N, d] arrays of
 *            16-bit floats (dtype ATTN_DTYPE_BF16 or ATTN_DTYPE_FP16);
 *            lse is a contiguous [B, H, N] array of fp32 holding natural-log
 *            m + ln(sum exp(s - m)) per query row.
 * Causal:    nonzero = query i sees keys j <= i (top-left, diagonal kept).
 * Scale:     fp32 multiplier of Q K^T; must be finite and > 0
 *            (1/sqrt(d) is the usual value).
 * Pointers:  device pointers (hipMalloc / torch CUDA tensors) on the current
 *            device, each 16-byte aligned.  The caller owns all memory; the
 *            library allocates no device memory and keeps no state between
 *            calls (apart from the opt-in profiling window below and a
 *            per-device cache of the compute-unit count, read once and used
 *            to size the persistent backward grids).
 * Sizes:     B, H, N >= 1 (any N: a last tile that runs past the end of the
 *            sequence is masked, never read past the inputs' end and never
 *            stored past row N - 1); d in {64, 128}; N <= 2^24.
 * Streams:   work is enqueued on `stream` (a hipStream_t; NULL = the null
 *            stream) and the call returns without synchronising.
 * Errors:    every argument check runs before any HIP call: an argument
 *            error writes nothing and enqueues nothing.  ATTN_ERR_HIP means a
 *            launch was refused (kernels of the same call launched before it
 *            stay enqueued).  Faults inside a kernel surface at the caller's
 *            next synchronisation.
 * Threads:   calls are re-entrant; calls on different streams may overlap.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_dtype {
  ATTN_DTYPE_BF16 = 0,
  ATTN_DTYPE_FP16 = 1,
};

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = 1,              /* a required pointer is NULL */
  ATTN_ERR_BAD_SHAPE = 2,             /* B, H or N < 1, or the sizes overflow int64 */
  ATTN_ERR_UNSUPPORTED_HEAD_DIM = 3,  /* d not in {64, 128} */
  ATTN_ERR_BAD_DTYPE = 4,             /* dtype not an attn_dtype value */
  ATTN_ERR_MISALIGNED = 5,            /* a pointer is not 16-byte aligned */
  ATTN_ERR_UNSUPPORTED_SEQLEN = 6,    /* reserved; no longer returned (any N >= 1 is accepted) */
  ATTN_ERR_BAD_SCALE = 7,             /* scale NaN, infinite or <= 0 */
  ATTN_ERR_WORKSPACE_TOO_SMALL = 8,   /* workspace NULL or below attn_bwd_workspace_bytes() */
  ATTN_ERR_ALIASING = 9,              /* an output overlaps an input or another output */
  ATTN_ERR_HIP = 10,                  /* a kernel launch failed; see attn_last_hip_error() */
  ATTN_ERR_BAD_LAYOUT = 11,           /* strides negative, not multiples of 8 elements, token stride
                                         >= 2^24, or an output layout whose elements overlap */
  ATTN_ERR_BAD_DROPOUT = 12,          /* dropout probability NaN, < 0, in (0, 1/512) or >= 511/512 */
  ATTN_ERR_SCRATCH_TOO_SMALL = 13,    /* attn_fwd_kvcache_noalloc: the call needs more than
                                         ATTN_KV_SCRATCH_BYTES of split partials */
};

/*
 * attn_fwd - forward pass.
 *   q, k, v  [B,H,N,d] inputs (read only).
 *   o        [B,H,N,d] output, same dtype: softmax(scale Q K^T) V, rounded to
 *            nearest-even from fp32.
 *   lse      [B,H,N] fp32 output: natural-log log-sum-exp of each row of the
 *            (masked, scaled) scores; the only statistic the backward needs.
 * o and lse must not overlap q, k, v or each other.
 * The launch shape (8 waves and 256 queries, or 4 waves and 128 queries, per
 * workgroup) is chosen on every call from N, d and causal; both give the same
 * results bit for bit.  The environment variable ATTN_FWD_WAVES=4 or 8, read
 * on every call, forces one (also for the strided, ALiBi and dropout forms).
 * Returns ATTN_OK or an attn_status error code.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
             int dtype, void* stream);

/*
 * attn_fwd_strided - attn_fwd for tensors in any [B, H, N, d] layout whose
 * last dimension is contiguous, e.g. [B, N, H, d] (token-major, "NHD"), a
 * packed [B, N, 3, H, d] QKV buffer, or a head stride of 0 to share one K
 * and V over all heads.  Page "Flash Attention V2 大模型时代的算力救星" §4.2
 * names the layout and 128-bit alignment demands of attention kernels as an
 * integration cost; here the kernels address the caller's layout directly.
 *   strides  12 int64 element strides, (batch, head, token) for q, k, v, o in
 *            that order; element (b, h, n, c) of a tensor is at
 *            base + b*s_batch + h*s_head + n*s_token + c.
 * Every stride must be >= 0 and a multiple of 8 (so every row is 16-byte
 * aligned), token strides < 2^24, batch and head strides <= 2^40; o's
 * layout must not map two elements to one address (ATTN_ERR_BAD_LAYOUT
 * otherwise).  lse stays a contiguous [B,H,N] fp32 array.  Aliasing is
 * checked on each tensor's address range [base, last element].
 * attn_fwd(...) is attn_fwd_strided with the contiguous strides
 * (H*N*d, N*d, d) for all four tensors.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* strides,
                     float scale, int causal, int dtype, void* stream);

/*
 * attn_bwd_workspace_bytes - size of the scratch buffer attn_bwd needs.  With
 * Np = N rounded up to a multiple of 64: two fp32 per padded query row
 * (-D_i = -dO_i . O_i and -lse_i / scale) plus three 16-bit [B,H,d,Np]
 * transposed copies of Q, K and dO; when N is not a multiple of 64, also four
 * 16-bit [B,H,64,d] copies of the last, zero-padded 64-token tile of Q, dO,
 * K and V.  Each part is rounded up to 256 bytes: about 8*B*H*Np +
 * 6*B*H*Np*d (+ 512*B*H*d) bytes.  It grows as O(B*H*N*d), never with N^2
 * (the memory bound of page "突破单卡显存极限…" §2.2).  Returns 0 when the
 * sizes are invalid (B, H, N < 1, d not in {64,128}, or overflow).
 */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * attn_bwd - backward pass for the loss gradient dO = dL/dO.
 *   q, k, v, o, lse  exactly the inputs and outputs of the matching attn_fwd
 *                    call (same scale, causal and dtype).
 *   dO       [B,H,N,d] upstream gradient.
 *   dq, dk, dv [B,H,N,d] outputs (dtype), rounded to nearest-even.
 *   workspace  device buffer of at least attn_bwd_workspace_bytes(B,H,N,d)
 *              bytes, 256-byte aligned; overwritten, contents undefined
 *              afterwards.  Concurrent calls need distinct workspaces.
 * dq, dk, dv and workspace must not overlap any input or each other.
 * No atomics are used: every output element is accumulated by one lane, so
 * dQ, dK and dV are bitwise reproducible from run to run.
 * Returns ATTN_OK or an attn_status error code.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dO, const float* lse, void* dq, void* dk, void* dv,
             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
             int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * KV-cache forward: Nq new queries against Nk cached keys and values
 * (decoding one or a few tokens), the reuse of earlier positions' keys and
 * values described on page "FlashAttention技术解析 如何让GPT训练速度提升5-9倍"
 * §4.1, computed exactly as attn_fwd computes the square case.
 *
 * attn_fwd_kvcache - forward pass with Q shorter than K.
 *   q        [B,H,Nq,d] queries.
 *   k, v     [B,H,Nk,d] cached keys and values (read only).
 *   o        [B,H,Nq,d] output, same dtype; lse [B,H,Nq] fp32 (natural log).
 *   causal   nonzero = the queries are the last Nq positions of the
 *            sequence: query i sees keys j <= i + Nk - Nq (bottom-right;
 *            for Nq == Nk the same mask as attn_fwd).  Requires Nk >= Nq.
 *   num_splits  key splits: the key axis is cut into about this many ranges,
 *            each computed by its own wave and merged afterwards (the merge
 *            by per-range maxima and sums is exact).  0 = chosen by the
 *            library from the sizes; at most 4096; ranges are whole 32-key
 *            blocks, so fewer are used when Nk is short.
 *   workspace  device buffer of at least attn_fwd_kvcache_workspace_bytes()
 *            bytes for the same sizes and num_splits, 256-byte aligned;
 *            overwritten.  Concurrent calls need distinct workspaces.
 * Other conventions as above (16-byte aligned pointers, no overlap between
 * outputs, workspace and inputs, checks before any HIP call, asynchronous).
 * Any Nq, Nk >= 1; the kernels are built for Nq much smaller than Nk
 * (their cost is one pass over K and V per 32 queries).
 * Returns ATTN_OK or an attn_status error code (ATTN_ERR_BAD_SHAPE also for
 * causal with Nk < Nq and for num_splits outside 0..4096).
 */
int attn_fwd_kvcache(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                     int causal, int dtype, int num_splits, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * attn_fwd_kvcache_noalloc - attn_fwd_kvcache for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace.  The split partials go to a static buffer of the library
 * (ATTN_KV_SCRATCH_BYTES per device, held until the process ends); the
 * call allocates nothing.
 *   Limit: attn_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d, num_splits)
 *   must not exceed ATTN_KV_SCRATCH_BYTES, else ATTN_ERR_SCRATCH_TOO_SMALL
 *   (checked, like every argument, before any HIP call).  At the default
 *   split plan this admits up to about 60,000 (query row, key range) pairs at
 *   d = 128, e.g. B * H * Nq = 7,500 query rows at 8 ranges.
 *   Sharing: every call on one device uses that device's one buffer, and the
 *   merge of a call reads what its own split pass wrote there.  Calls that
 *   overlap on one GPU (different streams with no ordering between them, or
 *   different threads) race on the buffer and give wrong results; calls on
 *   one stream are ordered and safe.  No part of the buffer needs clearing:
 *   each call writes every partial it later reads.
 *   Returns ATTN_ERR_HIP (attn_last_hip_error) if the buffer's device address
 *   cannot be obtained on the current device.
 */
#define ATTN_KV_SCRATCH_BYTES ((size_t)32 << 20)
int attn_fwd_kvcache_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                             int causal, int dtype, int num_splits, void* stream);

/*
 * attn_fwd_kvcache_strided - attn_fwd_kvcache for tensors in any layout with
 * a contiguous last dimension, strides as for attn_fwd_strided (q and o
 * [B,H,Nq,d], k and v [B,H,Nk,d]).  A token-major cache [B, Nmax, H, d]
 * allocated for Nmax >= Nk positions is passed as it is: batch stride
 * Nmax*H*d, head stride d, token stride H*d.
 */
int attn_fwd_kvcache_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                             const int64_t* strides, float scale, int causal, int dtype,
                             int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_kvcache_gqa - attn_fwd_kvcache with grouped heads: Hq query heads
 * share Hkv KV heads (Hq a multiple of Hkv; query head h attends with KV
 * head h / (Hq / Hkv)), as caches of grouped-query models are stored.  The
 * result is the attention of each query head against its group's K and V
 * (the same as attn_fwd_kvcache with K and V repeated per query head); the
 * query heads of a group are packed into the rows of one query tile, so
 * each cached byte is read once per call, not once per query head.
 *   q, o     [B,Hq,Nq,d];  k, v [B,Hkv,Nk,d];  lse [B,Hq,Nq] (contiguous).
 *   alibi_slopes  NULL, or Hq fp32 slopes (device array) for the ALiBi bias.
 *   workspace  at least attn_fwd_kvcache_gqa_workspace_bytes() bytes; the
 *            split count is attn_fwd_kvcache_splits(B, Hkv, (Hq/Hkv)*Nq, Nk,
 *            d, num_splits).
 * Other arguments and errors as for attn_fwd_kvcache (ATTN_ERR_BAD_SHAPE
 * also when Hq is not a multiple of Hkv).
 */
int attn_fwd_kvcache_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                         const float* alibi_slopes, float scale, int causal, int dtype,
                         int num_splits, void* workspace, size_t workspace_bytes, void* stream);
size_t attn_fwd_kvcache_gqa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                                            int64_t Nk, int64_t d, int num_splits);

/*
 * attn_fwd_kvcache_workspace_bytes - workspace of attn_fwd_kvcache: per
 * query row and split, d fp32 partial sums plus 4 fp32 statistics, each part
 * rounded up to 256 bytes (about 4*B*H*Nq*P*(d+4) bytes for P splits).
 * Returns 0 for invalid sizes.
 */
size_t attn_fwd_kvcache_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                        int num_splits);

/* attn_fwd_kvcache_splits - the number of key splits a call with these sizes
 * uses (0 for invalid sizes). */
int attn_fwd_kvcache_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int num_splits);

/*
 * attn_bwd_strided - attn_bwd for tensors in any [B, H, N, d] layout with a
 * contiguous last dimension (see attn_fwd_strided).
 *   strides  24 int64 element strides, (batch, head, token) for q, k, v, o,
 *            dO, dq, dk, dv in that order.
 *   workspace  at least attn_bwd_strided_workspace_bytes(B,H,N,d) bytes: the
 *            preprocess reads q, k, v, o, dO in their layouts and also writes
 *            contiguous copies of q, k, v and dO there, which the dK/dV and
 *            dQ kernels read; dq, dk, dv are stored in their own layouts.
 * dq, dk and dv may interleave in one buffer when they share a layout and
 * no element is shared (a packed [B, N, 3, H, d] gradient); otherwise outputs
 * must not overlap inputs, each other or the workspace by address range.
 * Layout rules and errors as for attn_fwd_strided.
 */
int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                     const void* dO, const float* lse, void* dq, void* dk, void* dv,
                     int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* strides,
                     float scale, int causal, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* attn_bwd_strided_workspace_bytes - attn_bwd_workspace_bytes plus four
 * contiguous 16-bit [B,H,N,d] copies (each rounded up to 256 bytes). */
size_t attn_bwd_strided_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * ALiBi: attn_fwd, attn_bwd and attn_fwd_kvcache with a linear position bias
 * added to the scaled scores before the softmax (page "FlashAttention技术
 * 解析 如何让GPT训练速度提升5-9倍" §4.1 names ALiBi for long contexts):
 *   S_ij = scale * q_i . k_j - m_h * |p_i - j|,  p_i = i + Nk - Nq
 * (the query's position; Nk = Nq = N outside the KV-cache call), with m_h
 * the slope of head h.  Causal rows see j <= p_i only, so the bias is
 * -m_h (p_i - j) there; non-causal rows take the distance both ways.  The
 * bias enters lse, and the backward recomputes it; no gradient flows to the
 * slopes.
 *   alibi_slopes  device array of H fp32 slopes (4-byte aligned; read only;
 *                 any finite values), the same array for the forward and
 *                 backward of one computation.
 * Tensors are contiguous as for attn_fwd / attn_bwd / attn_fwd_kvcache;
 * every other argument, the workspace sizes and the errors are theirs.
 */
int attn_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d, const float* alibi_slopes,
                   float scale, int causal, int dtype, void* stream);
int attn_bwd_alibi(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv,
                   int64_t B, int64_t H, int64_t N, int64_t d, const float* alibi_slopes,
                   float scale, int causal, int dtype, void* workspace,
                   size_t workspace_bytes, void* stream);
int attn_fwd_kvcache_alibi(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                           const float* alibi_slopes, float scale, int causal, int dtype,
                           int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dropout on the attention probabilities, fused into the kernels.
 *
 * Source: dropout is one of the elementwise steps the method fuses into the
 * attention kernel (page "FlashAttention技术解析 如何让GPT训练速度提升5-9倍"
 * §2.2); the op of page "Flash Attention V2 大模型时代的算力救星" §4.2 takes
 * a dropout probability.  The pages name no generator; the mask here is
 * drawn with Philox4x32-10 (Salmon et al., SC 2011) and regenerated, never
 * stored, by the forward and both backward kernels:
 *   - the 4 x 4 block of (query row, key row) (4a .. 4a+3, 4b .. 4b+3) of head
 *     bh = b * H + h is one call with counter (a, b, bh, offset) and key
 *     (seed & 0xFFFFFFFF, seed >> 32); query 4a + u takes output word u and
 *     key 4b + c its byte c (least significant byte first);
 *   - t = attn_dropout_threshold(dropout_p) = floor(256 dropout_p + 1/2):
 *     an element whose byte is below t is dropped (its weight in P V is 0),
 *     the others are multiplied by 256 / (256 - t).  The effective
 *     probability is t / 256, within 1/512 of dropout_p; a dropout_p that
 *     would round to t = 0 while positive (below 1/512) or to t = 256
 *     (511/512 and above) is rejected rather than run at another
 *     probability.
 *   O = (P o M) V with M the scaled keep mask; lse is that of the softmax
 *   over all visible keys (dropout does not change it).  The backward with
 *   the same (dropout_p, seed, offset) differentiates that O.
 *
 * attn_dropout_threshold: t for dropout_p, or -1 if dropout_p is NaN, < 0,
 * in (0, 1/512) or >= 511/512.
 * attn_fwd_dropout / attn_bwd_dropout: as attn_fwd / attn_bwd (contiguous
 * tensors, same workspace, same errors) plus the dropout arguments; the
 * mask depends on (batch, head, query row, key row), not on the layout;
 * ATTN_ERR_BAD_DROPOUT for a dropout_p that attn_dropout_threshold rejects.
 * dropout_p = 0 runs the kernels without dropout.
 * attn_dropout_draws: writes the 8-bit draws of heads 0 .. BH-1 for query
 * rows 0 .. Nq-1 and key rows 0 .. Nk-1 to draws (device, uint8,
 * [BH, Nq, Nk] contiguous, caller-owned); an element is dropped exactly when
 * its draw is below t.  ATTN_ERR_NULL_PTR, ATTN_ERR_BAD_SHAPE (any size < 1
 * or too large), ATTN_ERR_HIP.
 */
int attn_dropout_threshold(float dropout_p);
int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                     int dtype, float dropout_p, uint64_t seed, uint32_t offset, void* stream);
int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                     const void* dO, const float* lse, void* dq, void* dk, void* dv,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                     int dtype, float dropout_p, uint64_t seed, uint32_t offset,
                     void* workspace, size_t workspace_bytes, void* stream);
int attn_dropout_draws(uint8_t* draws, int64_t BH, int64_t Nq, int64_t Nk, uint64_t seed,
                       uint32_t offset, void* stream);
/* attn_fwd_dropout_strided / attn_bwd_dropout_strided: the same on tensors in
 * any [B, H, N, d] layout with a contiguous head dimension, strides and
 * layout rules as for attn_fwd_strided / attn_bwd_strided (12 and 24
 * strides; the backward's workspace is attn_bwd_strided_workspace_bytes). */
int attn_fwd_dropout_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* strides,
                             float scale, int causal, int dtype, float dropout_p, uint64_t seed,
                             uint32_t offset, void* stream);
int attn_bwd_dropout_strided(const void* q, const void* k, const void* v, const void* o,
                             const void* dO, const float* lse, void* dq, void* dk, void* dv,
                             int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* strides,
                             float scale, int causal, int dtype, float dropout_p, uint64_t seed,
                             uint32_t offset, void* workspace, size_t workspace_bytes, void* stream);

/* Kernels the library launches, as counted by the profiling window below. */
enum attn_kernel_kind {
  ATTN_KERNEL_FWD = 0,         /* forward: O and lse */
  ATTN_KERNEL_BWD_PREP = 1,    /* backward: D = rowsum(dO * O), transposed Q, K, dO */
  ATTN_KERNEL_BWD_DKDV = 2,    /* backward: recompute per key block, dK and dV */
  ATTN_KERNEL_BWD_DQ = 3,      /* backward: recompute per query block, dQ */
  ATTN_KERNEL_KV_SPLIT = 4,    /* KV-cache forward: one key range per wave */
  ATTN_KERNEL_KV_MERGE = 5,    /* KV-cache forward: merge of the ranges, O and lse */
  ATTN_KERNEL_KINDS = 6,
};

/*
 * attn_profile_start / attn_profile_stop - kernel timing for measurement.
 * Between the two calls (process-wide, all threads and streams) every kernel
 * launch is bracketed by a HIP event pair recorded by the launch itself on
 * the kernel's own stream; the events are created by the library and are the
 * only resource it holds, until attn_profile_stop.  attn_profile_start
 * discards earlier records, creates a pool of 1024 events (so that launches
 * inside the window do not pay for creating them; more are created if the
 * pool runs out) and returns ATTN_OK.  attn_profile_stop closes the
 * window, waits for the recorded events, and writes, per attn_kernel_kind,
 * the number of launches (counts) and their summed duration in milliseconds
 * (total_ms); either array may be NULL.  Returns ATTN_OK, or ATTN_ERR_HIP if
 * an event could not be read (those launches are left out of the sums).
 * Launches that fail to create their events return ATTN_ERR_HIP.  The
 * timing is not part of the attention computation (not described on the
 * pages); it exists to measure the kernels against their roofline.
 */
int attn_profile_start(void);
int attn_profile_stop(int64_t counts[ATTN_KERNEL_KINDS], double total_ms[ATTN_KERNEL_KINDS]);

/* attn_status_string - static, NUL-terminated description of a status code. */
const char* attn_status_string(int status);

/*
 * attn_last_hip_error - the hipError_t value of the most recent failed launch
 * on the calling thread (0 if none), valid after ATTN_ERR_HIP.
 */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
