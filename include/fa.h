/*
 * fa.h -- C ABI of libfa.so: exact attention for AMD Instinct MI355X (gfx950).
 *
 * Two operations, both exact (no approximation of softmax):
 *
 *  1. fa_fwd: the FlashAttention forward pass, O = softmax(scale * Q K^T
 *     [+ causal mask]) V for every (batch, head), computed tile by tile with
 *     the online-softmax running max m and running sum l so that the N x N
 *     score matrix never reaches HBM.  Defined by "FlashAttention: GPU 메모리
 *     계층을 활용한 어텐션 최적화 분석" (youngju.dev), sections 2.1 (standard
 *     attention), 5.1-5.2 (tiling), 6.2 (online softmax) and 8.1-8.3
 *     (FlashAttention-2 order); "Flash Attention" (suniverse77.github.io),
 *     Eq. (1)-(4).
 *
 *  2. fa_bwd: the backward pass of fa_fwd / fa_fwd_gqa, dQ, dK, dV for an
 *     upstream gradient dO, with the blocks of P recomputed on chip from Q,
 *     K and the saved lse instead of being stored (youngju.dev section 7.2).
 *
 *  3. fa_quant_fp8 / fa_fwd_fp8: the forward pass in FP8 (E4M3) with one
 *     scale factor per block of the inputs (block quantisation, youngju.dev
 *     section 9.2 item 3).
 *
 *  4. fa_paged_decode: single-query attention of one new token per sequence
 *     against its context stored in a paged (block-table) KV cache, split
 *     into context partitions whose partial results (m, l, O) are merged with
 *     Eq. (4) of "Flash Attention" generalised to P parts.  The cache layout
 *     and the decode structure are those of "PagedAttention"
 *     (data-sketchers.com wiki), sections "Inputs", "Concepts", "Key",
 *     "Softmax", "Value", "Output".
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE memory owned by the caller; the library
 *    allocates nothing and keeps no pointer after the call returns.
 *  - Calls enqueue work on `stream` (a hipStream_t passed as void*, NULL for
 *    the default stream) and return at once; results are ready after the
 *    caller synchronises that stream.
 *  - Arguments are validated on the host before anything is launched.  On a
 *    non-zero status nothing was launched and nothing was written.  A launch
 *    failure reported by the HIP runtime returns FA_ERR_HIP.  Device faults
 *    surface at the caller's next synchronisation.  (The debug build of the
 *    library, compiled with FA_DEBUG_SYNC, waits for `stream` before every
 *    call returns and reports a fault of the call's own kernels as
 *    FA_ERR_HIP; it cannot be used under stream capture.)
 *  - Thread-safe.  Deterministic: identical inputs give bitwise identical
 *    outputs (fixed reduction order, no atomics).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of q, k, v (fa_fwd, fa_bwd) and of q, caches, out (fa_paged_decode) */
typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_F16 = 2 } fa_dtype_t;

/* status codes */
enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad scale ...   */
    FA_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head dim 96)     */
    FA_ERR_ALIGNMENT = -3,   /* a pointer is not aligned as documented           */
    FA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required       */
    FA_ERR_HIP = -5,         /* the HIP runtime refused a launch                 */
    FA_ERR_SCRATCH = -6      /* fa_paged_decode_noalloc: the sizes need more     */
                             /* than FA_DECODE_NOALLOC_SCRATCH_BYTES of scratch  */
};

/*
 * fa_fwd -- exact attention forward.
 *
 *   q, k, v : [B, H, N, d] contiguous (d fastest), element type `dtype`,
 *             16-byte aligned.  Read only.
 *   o       : [B, H, N, d] contiguous fp32, 16-byte aligned.  Written:
 *             o[b,h,i,:] = sum_j P_ij v[b,h,j,:] with
 *             P_ij = exp(s_ij - m_i) / l_i,  s_ij = scale * q_i . k_j,
 *             m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i), over the keys j
 *             that row i may see.
 *   lse     : [B, H, N] fp32, 4-byte aligned.  Written: lse_i = m_i + ln l_i
 *             (natural log of sum_j exp(s_ij)), the per-row statistic kept
 *             for a recomputing backward pass (youngju.dev section 7.2).
 *   B, H, N : batch, heads, sequence length, each >= 1; one head of K or V
 *             must stay below 2 GiB (N * d * sizeof(element) < 2^31) and
 *             B * H * ceil(N / 128) below 2^31, else FA_ERR_UNSUPPORTED.
 *   d       : head dimension, 64 or 128 (else FA_ERR_UNSUPPORTED).
 *   scale   : finite and >= 0 (usually 1/sqrt(d)); else FA_ERR_INVALID_ARG.
 *   causal  : non-zero: row i sees keys j <= i only (top-left aligned square
 *             mask, youngju.dev section 11.3); zero: all N keys.
 *   dtype   : FA_F32, FA_BF16 or FA_F16.  For FA_BF16 and FA_F16 the
 *             elementwise products are exact in fp32 and accumulate in fp32;
 *             for FA_F32 each product is rounded to fp32 (the matrix cores'
 *             fp32 instruction) before it accumulates in fp32.  The softmax
 *             probabilities are rounded (round to nearest even) to `dtype`
 *             before the P.V product on the matrix cores (kept in fp32 for
 *             FA_F32).
 *   stream  : hipStream_t or NULL.
 * q/k/v may alias each other; o and lse must not overlap any input.
 */
int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H, int N,
           int d, float scale, int causal, int dtype, void *stream);

/*
 * fa_fwd_gqa -- fa_fwd with grouped-query heads: k and v have Hkv heads
 * that H / Hkv consecutive query heads share (the num_kv_heads of the paged
 * cache in the PagedAttention walkthrough, data-sketchers.com wiki, section
 * "Concepts", applied to the forward pass).
 *
 *   q       : [B, H, N, d];  k, v : [B, Hkv, N, d];  o : [B, H, N, d] fp32;
 *             lse : [B, H, N] fp32.  Layout, alignment and dtype as fa_fwd.
 *   Hkv     : >= 1 and divides H (else FA_ERR_INVALID_ARG).  Query head h
 *             reads kv head h / (H / Hkv).  Hkv = H is fa_fwd; Hkv = 1 is
 *             multi-query attention.
 * Every other argument, the result for each query head and the error
 * behaviour are those of fa_fwd.
 */
int fa_fwd_gqa(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H,
               int Hkv, int N, int d, float scale, int causal, int dtype, void *stream);

/*
 * fa_fwd_ext -- fa_fwd_gqa with general masks: a different number of keys
 * than queries, a causal mask aligned to the bottom-right corner, a sliding
 * window and a boolean mask (youngju.dev section 11.3: is_causal or an
 * explicit boolean attn_mask in which True marks a pair that takes part;
 * section 11.6 names sliding-window attention).
 *
 *   q         : [B, H, Nq, d];  k, v : [B, Hkv, Nk, d];  o : [B, H, Nq, d]
 *               fp32;  lse : [B, H, Nq] fp32.  Types and alignment as fa_fwd.
 *   Query row i sees key j < Nk iff
 *       (causal == 0 or j <= i + off)
 *       and (window_left < 0 or j >= i + off - window_left)
 *       and (window_right < 0 or j <= i + off + window_right)
 *       and (mask == NULL or mask[b * mask_stride_b + h * mask_stride_h
 *                                 + i * mask_ld + j] != 0),
 *   with off = Nk - Nq: the last query row is aligned with the last key (new
 *   tokens appended to a context).  Nq = Nk, causal, no window and no mask
 *   is fa_fwd's causal mask.
 *   mask      : uint8 (0 = masked), or NULL: the (b, h) slice starts at byte
 *               b * mask_stride_b + h * mask_stride_h (0 broadcasts over that
 *               dimension) and holds Nq rows mask_ld bytes apart, of which
 *               the first Nk are used.  mask, mask_ld and both strides must
 *               be multiples of 16 (else FA_ERR_ALIGNMENT; pad the rows),
 *               mask_ld >= Nk, and Nq * mask_ld below 2^31.
 *   mask_blocks : NULL, or the block map of this mask that fa_mask_blocks
 *               wrote for the same B, H, Nq, Nk and strides (4-byte aligned;
 *               requires a mask, else FA_ERR_INVALID_ARG).  With it, key
 *               tiles the map marks empty are skipped without being read and
 *               tiles it marks full skip the mask bytes; the result is the
 *               same as without it.  A map that does not describe the mask
 *               (stale, or another mask's) gives wrong results but never
 *               reads outside q, k, v, the mask or the map.
 *   A row that sees no key gets o = 0 and lse = -inf.
 * Every other argument and the error behaviour are those of fa_fwd_gqa; o
 * and lse must not overlap q, k, v, the mask or its map.
 */
int fa_fwd_ext(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H,
               int Hkv, int Nq, int Nk, int d, float scale, int causal, int window_left,
               int window_right, const uint8_t *mask, int64_t mask_stride_b, int64_t mask_stride_h,
               int64_t mask_ld, const uint32_t *mask_blocks, int dtype, void *stream);

/*
 * fa_fwd_paged -- chunked prefill over the paged KV cache: Nq new query
 * tokens per sequence attend to the sequence's context, read in place from
 * the cache of fa_paged_decode (the layouts of the PagedAttention
 * walkthrough, data-sketchers.com wiki, sections "Inputs" and "Concepts").
 * The queries are the context's last Nq tokens, so the causal mask is
 * aligned to the bottom-right corner (youngju.dev section 11.3, is_causal):
 * query row i of sequence s sees the context tokens
 *     t < ctx_s   and   (causal == 0 or t <= i + ctx_s - Nq),
 * with ctx_s = context_lens[s]; a row that sees no token gets o = 0 and
 * lse = -inf.
 *
 *   q            : [num_seqs, num_heads, Nq, head_size], 16-byte aligned.
 *   k_cache      : [num_blocks, num_kv_heads, head_size/8, block_size, 8].
 *   v_cache      : [num_blocks, num_kv_heads, head_size, block_size].
 *                  Both 16-byte aligned; one cache must stay below 4 GiB.
 *   block_tables : [num_seqs, max_blocks_per_seq] int32; token t of sequence
 *                  s is in block block_tables[s][t / block_size], slot
 *                  t % block_size.
 *   context_lens : [num_seqs] int32, device.  Not validated on the device:
 *                  each must lie in [0, block_size * max_blocks_per_seq] and
 *                  every table entry below ceil(ctx_s / block_size) in
 *                  [0, num_blocks).  A length or entry outside that gives
 *                  wrong results but reads nothing outside the caches,
 *                  tables and lengths.
 *   o            : [num_seqs, num_heads, Nq, head_size] fp32;  lse :
 *                  [num_seqs, num_heads, Nq] fp32 (natural log), as fa_fwd.
 *   head_size 128, block_size 16, dtype FA_BF16 or FA_F16 (q and both
 *   caches), num_kv_heads dividing num_heads (query head h reads kv head
 *   h / (num_heads / num_kv_heads)); else FA_ERR_UNSUPPORTED /
 *   FA_ERR_INVALID_ARG.  Products and accumulation as fa_fwd.
 *   FA_ERR_UNSUPPORTED also when Nq + 16 * max_blocks_per_seq >= 2^29.
 * o and lse must not overlap any input or each other; stream as fa_fwd.
 */
int fa_fwd_paged(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
                 const int32_t *context_lens, float *o, float *lse, int num_seqs, int num_heads,
                 int num_kv_heads, int Nq, int head_size, int block_size, int num_blocks,
                 int max_blocks_per_seq, float scale, int causal, int dtype, void *stream);

/*
 * Block map of a boolean mask, for fa_fwd_ext: which blocks of
 * FA_MASK_BLOCK_ROWS query rows x FA_MASK_BLOCK_COLS keys hold a visible
 * pair, and which hold no masked one.  The map is this library's own
 * acceleration structure for the boolean attn_mask of youngju.dev section
 * 11.3 (the pages define the mask, not the map): a mask that is reused
 * (across heads, layers or steps) is summarised once.
 *
 * Layout: uint32 words [Bs][Hs][ceil(Nq / 128)][2][nkw], with Bs = B if
 * mask_stride_b != 0 else 1, Hs likewise from H and mask_stride_h, and
 * nkw = ceil(ceil(Nk / 64) / 32).  For slice (b, h) and query block qb,
 * bit i of word w of the first half is set iff key block kb = 32 w + i
 * holds a nonzero mask byte (rows qb*128 .. +127 below Nq, keys kb*64 ..
 * +63 below Nk); of the second half, iff it holds no zero byte there (and
 * lies inside the key range).  Bits of blocks past Nk are 0.
 */
#define FA_MASK_BLOCK_ROWS 128
#define FA_MASK_BLOCK_COLS 64

/* Words of the block map for these sizes and strides (0 for invalid sizes). */
size_t fa_mask_blocks_words(int B, int H, int Nq, int Nk, int64_t mask_stride_b,
                            int64_t mask_stride_h);

/*
 * fa_mask_blocks -- write the block map of a mask (layout above).
 *   mask, B, H, Nq, Nk, mask_stride_b, mask_stride_h, mask_ld : as in
 *               fa_fwd_ext (mask not NULL), with its checks and error codes.
 *   blocks    : device, 4-byte aligned, blocks_words >= fa_mask_blocks_words
 *               (else FA_ERR_INVALID_ARG); must not overlap the mask.
 *   stream    : hipStream_t or NULL; the map is ready in stream order.
 * Returns FA_ERR_UNSUPPORTED when Bs * Hs * ceil(Nq/128) * nkw >= 2^31.
 */
int fa_mask_blocks(const uint8_t *mask, int B, int H, int Nq, int Nk, int64_t mask_stride_b,
                   int64_t mask_stride_h, int64_t mask_ld, uint32_t *blocks, size_t blocks_words,
                   void *stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace that fa_bwd needs: two
 * fp32 values per query row (D_i = dO_i . O_i and lse_i * log2 e),
 * 2 * B * H * N * 4 bytes rounded up to 256.  Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N);

/*
 * fa_bwd -- gradients of the attention forward pass (youngju.dev sections
 * 7.1-7.3: S and P are not stored; each block of P is recomputed from Q, K
 * and lse).  With s_ij = scale q_i . k_j and P_ij = exp(s_ij - lse_i) over
 * the keys row i may see:
 *     dV_j = sum_i P_ij dO_i,  dP_ij = dO_i . v_j,  D_i = dO_i . O_i,
 *     dS_ij = P_ij (dP_ij - D_i),
 *     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 * the chain rule of the forward definition (dK, dV of a kv head sum over the
 * query heads that read it).
 *
 *   q, dout : [B, H, N, d], element type `dtype`, 16-byte aligned.
 *   k, v    : [B, Hkv, N, d], element type `dtype`, 16-byte aligned.
 *   o, lse  : the forward pass's outputs for these q, k, v, scale and mask:
 *             o [B, H, N, d] fp32 (16-byte aligned), lse [B, H, N] fp32
 *             (4-byte aligned).  Read only.
 *   dq      : [B, H, N, d] fp32, 16-byte aligned.  Written.
 *   dk, dv  : [B, Hkv, N, d] fp32, 16-byte aligned.  Written.
 *   Hkv     : >= 1 and divides H; query head h reads kv head h / (H / Hkv).
 *   B, H, N, d, scale, causal : as fa_fwd (d 64 or 128).
 *   dtype   : FA_BF16 or FA_F16 (FA_F32: FA_ERR_UNSUPPORTED).  Products are
 *             exact and accumulate in fp32; P and dS are rounded to `dtype`
 *             (round to nearest even) before the products dV = P^T dO,
 *             dK = dS^T Q and dQ = dS K on the matrix cores.
 *   workspace : device buffer of at least fa_bwd_workspace_size(B, H, N)
 *             bytes, 256-byte aligned, overwritten by the call.  Concurrent
 *             calls need separate workspaces.
 *   stream  : hipStream_t or NULL.
 * Inputs may alias each other; dq, dk, dv and workspace must not overlap
 * one another or any input.
 */
int fa_bwd(const void *q, const void *k, const void *v, const float *o, const float *lse,
           const void *dout, float *dq, float *dk, float *dv, int B, int H, int Hkv, int N, int d,
           float scale, int causal, int dtype, void *workspace, size_t workspace_bytes,
           void *stream);

/*
 * Block-scaled FP8 (youngju.dev section 9.2, item 3: FP8 with a separate
 * scale factor per block).  Format: OCP E4M3 ("E4M3FN": 1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals, largest finite 448).  A
 * block is FA_FP8_BLOCK_ROWS consecutive rows of one (b, h) with all d
 * columns; its scale is 2^e with e = floor(log2 amax) - 7 (amax = largest
 * magnitude in the block; e = 0 for an all-zero block), and element x is
 * stored as the E4M3 rounding (nearest, ties to even) of x * 2^-e, its value
 * being value(code) * 2^e.
 *
 * Code layouts:
 *   layout 0 (q, k): [B, H, N, d] bytes, like the input;
 *   layout 1 (v):    [B, H, ceil(N/64), d, 64] bytes: each tile of 64 keys is
 *                    stored d-major (element (key, c) of tile t at
 *                    [t][c][key - 64 t]); keys >= N hold code 0.
 * Exponents: [B, H, ceil(N / FA_FP8_BLOCK_ROWS)] int32.
 */
#define FA_FP8_BLOCK_ROWS 128

/* fa_fp8_codes_bytes -- bytes of the code tensor of a [B, H, N, d] input in
 * `layout` (0 or 1); 0 for invalid sizes. */
size_t fa_fp8_codes_bytes(int B, int H, int N, int d, int layout);

/*
 * fa_quant_fp8 -- block-scaled E4M3 quantisation of x.
 *
 *   x       : [B, H, N, d] contiguous, element type `dtype` (FA_F32, FA_BF16
 *             or FA_F16), finite, 16-byte aligned.  Read only.
 *   layout  : 0 or 1 (see above); d: 64 or 128 (else FA_ERR_UNSUPPORTED).
 *   codes   : fa_fp8_codes_bytes(B, H, N, d, layout) bytes, 16-byte aligned.
 *             Written.
 *   exps    : [B, H, ceil(N / FA_FP8_BLOCK_ROWS)] int32, 4-byte aligned.
 *             Written.
 * codes and exps must not overlap x or each other.
 */
int fa_quant_fp8(const void *x, int dtype, int B, int H, int N, int d, int layout, void *codes,
                 int32_t *exps, void *stream);

/*
 * fa_fwd_fp8 -- the attention forward on block-scaled E4M3 inputs.
 *
 *   q8, q_exp : q codes in layout 0 ([B, H, N, d]) and exponents [B, H, nblk].
 *   k8, k_exp : k codes in layout 0 ([B, Hkv, N, d]) and exponents [B, Hkv, nblk].
 *   v8, v_exp : v codes in layout 1 ([B, Hkv, ceil(N/64), d, 64]) and
 *               exponents [B, Hkv, nblk].
 *   o, lse    : as fa_fwd: o [B, H, N, d] fp32 and lse [B, H, N] fp32 of
 *               attention on the dequantised values (value(code) * 2^e).
 *   Hkv, B, H, N, scale, causal : as fa_fwd_gqa.  d: 128 (else
 *               FA_ERR_UNSUPPORTED).
 * Products of codes are exact and accumulate in fp32; the probabilities
 * are rounded to E4M3 for the P.V product and normalised by the sum of the
 * unrounded probabilities.  Code pointers and o 16-byte aligned, exponents
 * and lse 4-byte aligned; o and lse must not overlap any input.
 */
int fa_fwd_fp8(const void *q8, const void *k8, const void *v8, const int32_t *q_exp,
               const int32_t *k_exp, const int32_t *v_exp, float *o, float *lse, int B, int H,
               int Hkv, int N, int d, float scale, int causal, void *stream);

/*
 * fa_paged_decode_workspace_size -- bytes of device workspace that
 * fa_paged_decode needs for these sizes: the per-partition partial results
 * O_p [S, H, P, head_size] fp32 plus m_p and l_p [S, H, P] fp32, where
 * P = ceil(max_context_len / FA_DECODE_PARTITION_TOKENS).  Returns 0 for
 * invalid sizes.
 */
#define FA_DECODE_PARTITION_TOKENS 256
size_t fa_paged_decode_workspace_size(int num_seqs, int num_heads, int head_size,
                                      int max_context_len);

/*
 * fa_paged_decode -- single-query attention over a paged KV cache.
 *
 *   q            : [num_seqs, num_heads, head_size], element type `dtype`.
 *   k_cache      : [num_blocks, num_kv_heads, head_size / x, block_size, x]
 *                  with x = 16 / sizeof(element) (8 for fp16/bf16): every
 *                  16-byte vector holds x consecutive head elements of one
 *                  token ("PagedAttention", sections "Concepts" and "Key").
 *   v_cache      : [num_blocks, num_kv_heads, head_size, block_size]
 *                  ("PagedAttention", section "Value").
 *   block_tables : [num_seqs, max_blocks_per_seq] int32: context token t of
 *                  sequence s lives in physical block block_tables[s][t /
 *                  block_size], slot t % block_size.
 *   context_lens : [num_seqs] int32, each in [0, max_context_len].  Not
 *                  checked on the device: the grid covers
 *                  ceil(max_context_len / FA_DECODE_PARTITION_TOKENS)
 *                  partitions, so tokens of a larger value past that range
 *                  are left out of its softmax.
 *   out          : [num_seqs, num_heads, head_size], element type `dtype`.
 *                  out[s,h,:] = sum_t p_t V_t with p = softmax_t(scale * q[s,h]
 *                  . K_t) over t < context_lens[s], rounded to nearest even.
 *                  A context of length 0 gives out = 0.
 *   num_kv_heads : divides num_heads; query head h reads kv head
 *                  h / (num_heads / num_kv_heads).
 *   head_size    : 128.  block_size: 16.  dtype: FA_F16 or FA_BF16.
 *   max_blocks_per_seq * block_size >= max_context_len >= 0.
 *   scale        : finite and >= 0.
 *   workspace    : device buffer of at least
 *                  fa_paged_decode_workspace_size(...) bytes, 256-byte
 *                  aligned, that the call may overwrite; not read before it
 *                  is written.  Concurrent calls need separate workspaces.
 * The first ceil(context_lens[s] / block_size) entries of each table row must
 * be valid block ids; they are not checked on the device.
 * out and workspace must not overlap q, block_tables, context_lens or each
 * other (FA_ERR_INVALID_ARG); the caches' extent is not passed, so overlap
 * with them is the caller's to avoid.
 */
int fa_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, void *out,
                    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
                    int max_blocks_per_seq, int max_context_len, float scale, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_paged_decode_noalloc -- fa_paged_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and validation
 * as fa_paged_decode, without the workspace: the per-partition partials go
 * to a scratch array of FA_DECODE_NOALLOC_SCRATCH_BYTES that the library
 * holds in each GPU's memory from its first use on that GPU until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine).
 *   - Sizes whose workspace (fa_paged_decode_workspace_size) exceeds
 *     FA_DECODE_NOALLOC_SCRATCH_BYTES return FA_ERR_SCRATCH and launch
 *     nothing; 32 MiB holds num_seqs * num_heads *
 *     ceil(max_context_len / 256) <= 64,000 partitions (e.g. 64 sequences x
 *     32 heads at contexts up to 8,000 tokens).
 *   - The scratch belongs to the device that is current when the call is
 *     made; `stream` must belong to that device (else FA_ERR_INVALID_ARG).
 *     Its address is looked up once per device (hipGetSymbolAddress), so the
 *     first call on a device makes that HIP query before launching.
 *   - Every call on one GPU shares that GPU's scratch, and a call leaves its
 *     partials there: calls that overlap in time on one GPU (different
 *     streams, or different threads, without ordering between them) race
 *     and may return wrong results.  Calls ordered on one stream are safe.
 *     Nothing in the scratch needs clearing between calls: a call reads
 *     only partials it wrote itself.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int fa_paged_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens, void *out,
                            int num_seqs, int num_heads, int num_kv_heads, int head_size,
                            int block_size, int max_blocks_per_seq, int max_context_len,
                            float scale, int dtype, void *stream);

/* fa_strerror -- a static, human-readable string for a status code. */
const char *fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
