// fa_capi.cpp -- the C ABI of libfa.so (declared in include/fa.h): host-side
// validation of every argument, then dispatch to the gfx950 kernels.
// Validation runs before any HIP call, so an invalid call launches nothing
// and writes nothing.
#include "fa.h"
#include "fa_sizes.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

namespace fa {
hipError_t fwd_dispatch(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                        int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                        hipStream_t stream);
hipError_t decode_dispatch(const void *q, const void *kc, const void *vc, const int32_t *bt,
                           const int32_t *cl, void *out, int S, int H, int Hkv, int MB,
                           int max_ctx, float scale, int dtype, void *workspace,
                           hipStream_t stream);
hipError_t decode_noalloc_dispatch(const void *q, const void *kc, const void *vc, const int32_t *bt,
                                   const int32_t *cl, void *out, int S, int H, int Hkv, int MB,
                                   int max_ctx, float scale, int dtype, hipStream_t stream);
hipError_t bwd_dispatch(const void *q, const void *k, const void *v, const float *o,
                        const float *lse, const void *dout, float *dq, float *dk, float *dv, int B,
                        int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                        void *workspace, hipStream_t stream);
hipError_t fwd_ext_dispatch(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                            int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int wl,
                            int wr, const uint8_t *mask, int64_t msb, int64_t msh, int ldm,
                            const uint32_t *blocks, int dtype, hipStream_t stream);
hipError_t fwd_paged_dispatch(const void *q, const void *kc, const void *vc, const int32_t *tables,
                              const int32_t *ctx_lens, float *o, float *lse, int S, int H, int Hkv,
                              int Nq, int mbps, uint64_t cache_bytes, float scale, int causal,
                              int dtype, hipStream_t stream);
hipError_t mask_blocks_dispatch(const uint8_t *mask, int B, int H, int Nq, int Nk, int64_t msb,
                                int64_t msh, int ldm, uint32_t *blocks, hipStream_t stream);
hipError_t quant_fp8_dispatch(const void *x, int dtype, int B, int H, int N, int d, int layout,
                              void *codes, int32_t *exps, hipStream_t stream);
hipError_t fwd_fp8_dispatch(const void *q8, const void *k8, const void *v8, const int32_t *qe,
                            const int32_t *ke, const int32_t *ve, float *o, float *lse, int B, int H,
                            int Hkv, int N, float scale, int causal, hipStream_t stream);
}  // namespace fa

namespace {

constexpr int kFwdRowsPerWorkgroup = 128;
constexpr int kMaxGridYZ = 65535;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int elem_bytes(int dtype)
{
    switch (dtype) {
    case FA_F32: return 4;
    case FA_BF16:
    case FA_F16: return 2;
    default: return 0;
    }
}

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool valid_scale(float s) { return std::isfinite(s) && s >= 0.f; }

// Status of a call whose work was enqueued with result e.  A library built
// with FA_DEBUG_SYNC (the debug build) also waits for the stream, so that a
// fault of the launched kernels is reported, as FA_ERR_HIP, by the call that
// launched them instead of by a later call; such a build cannot be used
// under stream capture.
int launched(hipError_t e, void *stream)
{
#ifdef FA_DEBUG_SYNC
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipGetLastError();
#else
    (void)stream;
#endif
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

namespace {

// Validation shared by fa_fwd (Hkv = H) and fa_fwd_gqa, then the launch.
int fwd_checked(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H,
                int Hkv, int N, int d, float scale, int causal, int dtype, void *stream)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
    const int es = elem_bytes(dtype);
    if (es == 0) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const int64_t qtiles = ((int64_t)N + kFwdRowsPerWorkgroup - 1) / kFwdRowsPerWorkgroup;
    if ((int64_t)B * H * qtiles > INT_MAX) return FA_ERR_UNSUPPORTED;
    // one head of K or V is addressed with 32-bit byte offsets
    if ((int64_t)N * d * es > INT_MAX) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return FA_ERR_ALIGNMENT;
    const uint64_t rows = (uint64_t)B * H * N, kv_rows = (uint64_t)B * Hkv * N;
    const uint64_t q_bytes = rows * d * es, kv_bytes = kv_rows * d * es;
    const uint64_t o_bytes = rows * d * 4, l_bytes = rows * 4;
    if (overlap(o, o_bytes, lse, l_bytes)) return FA_ERR_INVALID_ARG;
    const void *ins[3] = {q, k, v};
    const uint64_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
    for (int i = 0; i < 3; ++i)
        if (overlap(o, o_bytes, ins[i], in_bytes[i]) || overlap(lse, l_bytes, ins[i], in_bytes[i]))
            return FA_ERR_INVALID_ARG;
    const hipError_t e = fa::fwd_dispatch(q, k, v, o, lse, B, H, Hkv, N, d, scale,
                                          causal ? 1 : 0, dtype, (hipStream_t)stream);
    return launched(e, stream);
}

}  // namespace

extern "C" int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                      int H, int N, int d, float scale, int causal, int dtype, void *stream)
{
    return fwd_checked(q, k, v, o, lse, B, H, H, N, d, scale, causal, dtype, stream);
}

extern "C" int fa_fwd_gqa(const void *q, const void *k, const void *v, float *o, float *lse,
                          int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                          void *stream)
{
    return fwd_checked(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, dtype, stream);
}

// The mask arguments shared by fa_fwd_ext and fa_mask_blocks (mask not null).
static int check_mask(const uint8_t *mask, int Nq, int Nk, int64_t msb, int64_t msh, int64_t ldm)
{
    if (msb < 0 || msh < 0 || ldm < Nk) return FA_ERR_INVALID_ARG;
    if ((int64_t)Nq * ldm > INT_MAX) return FA_ERR_UNSUPPORTED;  // one mask slice < 2 GiB
    if (!aligned(mask, 16) || ldm % 16 || msb % 16 || msh % 16) return FA_ERR_ALIGNMENT;
    return FA_OK;
}

// bytes from the mask's first slice to the end of its last
static uint64_t mask_extent(int B, int H, int Nq, int64_t msb, int64_t msh, int64_t ldm)
{
    return (uint64_t)(B - 1) * msb + (uint64_t)(H - 1) * msh + (uint64_t)Nq * ldm;
}

extern "C" size_t fa_mask_blocks_words(int B, int H, int Nq, int Nk, int64_t mask_stride_b,
                                       int64_t mask_stride_h)
{
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || mask_stride_b < 0 || mask_stride_h < 0) return 0;
    return fa::mask_blocks_words(B, H, Nq, Nk, mask_stride_b, mask_stride_h);
}

extern "C" int fa_mask_blocks(const uint8_t *mask, int B, int H, int Nq, int Nk, int64_t mask_stride_b,
                              int64_t mask_stride_h, int64_t mask_ld, uint32_t *blocks,
                              size_t blocks_words, void *stream)
{
    if (!mask || !blocks) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID_ARG;
    const int mc = check_mask(mask, Nq, Nk, mask_stride_b, mask_stride_h, mask_ld);
    if (mc != FA_OK) return mc;
    if (!aligned(blocks, 4)) return FA_ERR_ALIGNMENT;
    const size_t words = fa::mask_blocks_words(B, H, Nq, Nk, mask_stride_b, mask_stride_h);
    if (blocks_words < words) return FA_ERR_INVALID_ARG;
    // one workgroup per (slice, 128-row block, 2048 keys)
    if (words / 2 > (size_t)INT_MAX) return FA_ERR_UNSUPPORTED;
    if (overlap(blocks, (uint64_t)words * 4, mask,
                mask_extent(B, H, Nq, mask_stride_b, mask_stride_h, mask_ld)))
        return FA_ERR_INVALID_ARG;
    const hipError_t e = fa::mask_blocks_dispatch(mask, B, H, Nq, Nk, mask_stride_b, mask_stride_h,
                                                  (int)mask_ld, blocks, (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" int fa_fwd_ext(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                          int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                          int window_left, int window_right, const uint8_t *mask,
                          int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_ld,
                          const uint32_t *mask_blocks, int dtype, void *stream)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
    if (mask && (mask_stride_b < 0 || mask_stride_h < 0 || mask_ld < Nk)) return FA_ERR_INVALID_ARG;
    if (mask_blocks && !mask) return FA_ERR_INVALID_ARG;
    const int es = elem_bytes(dtype);
    if (es == 0) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const int64_t qtiles = ((int64_t)Nq + kFwdRowsPerWorkgroup - 1) / kFwdRowsPerWorkgroup;
    if ((int64_t)B * H * qtiles > INT_MAX) return FA_ERR_UNSUPPORTED;
    if ((int64_t)Nk * d * es > INT_MAX || (int64_t)Nq + Nk > INT_MAX / 4) return FA_ERR_UNSUPPORTED;
    if (mask && (int64_t)Nq * mask_ld > INT_MAX) return FA_ERR_UNSUPPORTED;  // one mask slice < 2 GiB
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return FA_ERR_ALIGNMENT;
    if (mask && (!aligned(mask, 16) || mask_ld % 16 || mask_stride_b % 16 || mask_stride_h % 16))
        return FA_ERR_ALIGNMENT;
    if (mask_blocks && !aligned(mask_blocks, 4)) return FA_ERR_ALIGNMENT;
    const uint64_t rows = (uint64_t)B * H * Nq, kv_rows = (uint64_t)B * Hkv * Nk;
    const uint64_t o_bytes = rows * d * 4, l_bytes = rows * 4;
    const uint64_t m_bytes = mask ? mask_extent(B, H, Nq, mask_stride_b, mask_stride_h, mask_ld) : 0;
    const uint64_t mb_bytes =
        mask_blocks ? (uint64_t)fa::mask_blocks_words(B, H, Nq, Nk, mask_stride_b, mask_stride_h) * 4 : 0;
    if (overlap(o, o_bytes, lse, l_bytes)) return FA_ERR_INVALID_ARG;
    const void *ins[5] = {q, k, v, mask, mask_blocks};
    const uint64_t in_bytes[5] = {rows * d * es, kv_rows * d * es, kv_rows * d * es, m_bytes, mb_bytes};
    for (int i = 0; i < 5; ++i)
        if (ins[i] && (overlap(o, o_bytes, ins[i], in_bytes[i]) || overlap(lse, l_bytes, ins[i], in_bytes[i])))
            return FA_ERR_INVALID_ARG;
    const hipError_t e =
        fa::fwd_ext_dispatch(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal ? 1 : 0, window_left,
                             window_right, mask, mask_stride_b, mask_stride_h, (int)mask_ld,
                             mask_blocks, dtype, (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" int fa_fwd_paged(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens, float *o,
                            float *lse, int num_seqs, int num_heads, int num_kv_heads, int Nq,
                            int head_size, int block_size, int num_blocks, int max_blocks_per_seq,
                            float scale, int causal, int dtype, void *stream)
{
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (num_seqs < 1 || num_heads < 1 || num_kv_heads < 1 || Nq < 1 || head_size < 1 ||
        block_size < 1 || num_blocks < 1 || max_blocks_per_seq < 1)
        return FA_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return FA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
    const int es = elem_bytes(dtype);
    if (es == 0) return FA_ERR_INVALID_ARG;
    if (dtype == FA_F32 || head_size != 128 || block_size != 16) return FA_ERR_UNSUPPORTED;
    const uint64_t cache_bytes = (uint64_t)num_blocks * num_kv_heads * head_size * block_size * es;
    if (cache_bytes >= (1ull << 32)) return FA_ERR_UNSUPPORTED;  // 32-bit buffer offsets
    if ((int64_t)Nq + 16 * (int64_t)max_blocks_per_seq >= (1 << 29)) return FA_ERR_UNSUPPORTED;
    const int64_t qtiles = ((int64_t)Nq + kFwdRowsPerWorkgroup - 1) / kFwdRowsPerWorkgroup;
    if ((int64_t)num_seqs * num_heads * qtiles > INT_MAX) return FA_ERR_UNSUPPORTED;
    if ((int64_t)num_seqs * max_blocks_per_seq > INT_MAX) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
        !aligned(lse, 4) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return FA_ERR_ALIGNMENT;
    const uint64_t rows = (uint64_t)num_seqs * num_heads * Nq;
    const uint64_t o_bytes = rows * head_size * 4, l_bytes = rows * 4;
    if (overlap(o, o_bytes, lse, l_bytes)) return FA_ERR_INVALID_ARG;
    const void *ins[5] = {q, k_cache, v_cache, block_tables, context_lens};
    const uint64_t in_bytes[5] = {rows * head_size * es, cache_bytes, cache_bytes,
                                  (uint64_t)num_seqs * max_blocks_per_seq * 4, (uint64_t)num_seqs * 4};
    for (int i = 0; i < 5; ++i)
        if (overlap(o, o_bytes, ins[i], in_bytes[i]) || overlap(lse, l_bytes, ins[i], in_bytes[i]))
            return FA_ERR_INVALID_ARG;
    const hipError_t e = fa::fwd_paged_dispatch(q, k_cache, v_cache, block_tables, context_lens, o, lse,
                                                num_seqs, num_heads, num_kv_heads, Nq, max_blocks_per_seq,
                                                cache_bytes, scale, causal ? 1 : 0, dtype,
                                                (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" size_t fa_bwd_workspace_size(int B, int H, int N)
{
    if (B < 1 || H < 1 || N < 1) return 0;
    return fa::bwd_workspace_bytes(B, H, N);
}

extern "C" int fa_bwd(const void *q, const void *k, const void *v, const float *o,
                      const float *lse, const void *dout, float *dq, float *dk, float *dv, int B,
                      int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
    const int es = elem_bytes(dtype);
    if (es == 0) return FA_ERR_INVALID_ARG;
    if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const int64_t blocks = ((int64_t)N + kFwdRowsPerWorkgroup - 1) / kFwdRowsPerWorkgroup;
    if ((int64_t)B * H * blocks > INT_MAX) return FA_ERR_UNSUPPORTED;
    if ((int64_t)N * d * es > INT_MAX) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(lse, 4))
        return FA_ERR_ALIGNMENT;
    const size_t need = fa::bwd_workspace_bytes(B, H, N);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGNMENT;
    const uint64_t rows = (uint64_t)B * H * N, kv_rows = (uint64_t)B * Hkv * N;
    const void *ins[6] = {q, k, v, o, lse, dout};
    const uint64_t in_bytes[6] = {rows * d * es, kv_rows * d * es, kv_rows * d * es,
                                  rows * d * 4,  rows * 4,         rows * d * es};
    void *outs[4] = {dq, dk, dv, workspace};
    const uint64_t out_bytes[4] = {rows * d * 4, kv_rows * d * 4, kv_rows * d * 4, need};
    for (int a = 0; a < 4; ++a) {
        for (int i = 0; i < 6; ++i)
            if (overlap(outs[a], out_bytes[a], ins[i], in_bytes[i])) return FA_ERR_INVALID_ARG;
        for (int c = a + 1; c < 4; ++c)
            if (overlap(outs[a], out_bytes[a], outs[c], out_bytes[c])) return FA_ERR_INVALID_ARG;
    }
    const hipError_t e = fa::bwd_dispatch(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, scale,
                                          causal ? 1 : 0, dtype, workspace, (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" size_t fa_fp8_codes_bytes(int B, int H, int N, int d, int layout)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || (layout != 0 && layout != 1)) return 0;
    const size_t rows = layout == 0 ? (size_t)N : (size_t)(N + 63) / 64 * 64;
    return (size_t)B * H * rows * d;
}

extern "C" int fa_quant_fp8(const void *x, int dtype, int B, int H, int N, int d, int layout,
                            void *codes, int32_t *exps, void *stream)
{
    if (!x || !codes || !exps) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || d < 1 || (layout != 0 && layout != 1)) return FA_ERR_INVALID_ARG;
    const int es = elem_bytes(dtype);
    if (es == 0) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const int64_t nblk = ((int64_t)N + FA_FP8_BLOCK_ROWS - 1) / FA_FP8_BLOCK_ROWS;
    if ((int64_t)B * H * nblk > INT_MAX) return FA_ERR_UNSUPPORTED;
    if ((int64_t)N * d * es > INT_MAX) return FA_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(exps, 4)) return FA_ERR_ALIGNMENT;
    const uint64_t x_bytes = (uint64_t)B * H * N * d * es;
    const uint64_t c_bytes = fa_fp8_codes_bytes(B, H, N, d, layout);
    const uint64_t e_bytes = (uint64_t)B * H * nblk * 4;
    if (overlap(codes, c_bytes, x, x_bytes) || overlap(exps, e_bytes, x, x_bytes) ||
        overlap(codes, c_bytes, exps, e_bytes))
        return FA_ERR_INVALID_ARG;
    const hipError_t e = fa::quant_fp8_dispatch(x, dtype, B, H, N, d, layout, codes, exps,
                                                (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" int fa_fwd_fp8(const void *q8, const void *k8, const void *v8, const int32_t *q_exp,
                          const int32_t *k_exp, const int32_t *v_exp, float *o, float *lse, int B,
                          int H, int Hkv, int N, int d, float scale, int causal, void *stream)
{
    if (!q8 || !k8 || !v8 || !q_exp || !k_exp || !v_exp || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    const int64_t qtiles = ((int64_t)N + kFwdRowsPerWorkgroup - 1) / kFwdRowsPerWorkgroup;
    if ((int64_t)B * H * qtiles > INT_MAX) return FA_ERR_UNSUPPORTED;
    if ((int64_t)((N + 63) / 64) * 64 * d > INT_MAX) return FA_ERR_UNSUPPORTED;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) ||
        !aligned(q_exp, 4) || !aligned(k_exp, 4) || !aligned(v_exp, 4) || !aligned(lse, 4))
        return FA_ERR_ALIGNMENT;
    const int64_t nblk = ((int64_t)N + FA_FP8_BLOCK_ROWS - 1) / FA_FP8_BLOCK_ROWS;
    const uint64_t rows = (uint64_t)B * H * N;
    const uint64_t o_bytes = rows * d * 4, l_bytes = rows * 4;
    const void *ins[6] = {q8, k8, v8, q_exp, k_exp, v_exp};
    const uint64_t in_bytes[6] = {fa_fp8_codes_bytes(B, H, N, d, 0), fa_fp8_codes_bytes(B, Hkv, N, d, 0),
                                  fa_fp8_codes_bytes(B, Hkv, N, d, 1), (uint64_t)B * H * nblk * 4,
                                  (uint64_t)B * Hkv * nblk * 4, (uint64_t)B * Hkv * nblk * 4};
    if (overlap(o, o_bytes, lse, l_bytes)) return FA_ERR_INVALID_ARG;
    for (int i = 0; i < 6; ++i)
        if (overlap(o, o_bytes, ins[i], in_bytes[i]) || overlap(lse, l_bytes, ins[i], in_bytes[i]))
            return FA_ERR_INVALID_ARG;
    const hipError_t e = fa::fwd_fp8_dispatch(q8, k8, v8, q_exp, k_exp, v_exp, o, lse, B, H, Hkv, N,
                                              scale, causal ? 1 : 0, (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" size_t fa_paged_decode_workspace_size(int num_seqs, int num_heads, int head_size,
                                                 int max_context_len)
{
    if (num_seqs < 1 || num_heads < 1 || head_size != 128 || max_context_len < 0) return 0;
    return fa::decode_workspace_bytes(num_seqs, num_heads, max_context_len);
}

namespace {

// Validation of fa_paged_decode's arguments other than the workspace; on
// success *need is the workspace the sizes call for.
int decode_args(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *block_tables, const int32_t *context_lens, const void *out,
                int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
                int max_blocks_per_seq, int max_context_len, float scale, int dtype, size_t *need)
{
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
        return FA_ERR_INVALID_ARG;
    if (num_seqs < 1 || num_heads < 1 || num_kv_heads < 1 || head_size < 1 || block_size < 1 ||
        max_blocks_per_seq < 1 || max_context_len < 0)
        return FA_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return FA_ERR_INVALID_ARG;
    if ((int64_t)max_blocks_per_seq * block_size < max_context_len) return FA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
    const int es = elem_bytes(dtype);
    if (es == 0) return FA_ERR_INVALID_ARG;
    if (dtype == FA_F32 || head_size != 128 || block_size != 16) return FA_ERR_UNSUPPORTED;
    const int64_t nparts =
        ((int64_t)max_context_len + FA_DECODE_PARTITION_TOKENS - 1) / FA_DECODE_PARTITION_TOKENS;
    if (num_seqs > kMaxGridYZ || nparts > kMaxGridYZ) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return FA_ERR_ALIGNMENT;
    // out must not overlap what the call reads (the caches' extent is not
    // passed, so they cannot be checked here)
    const uint64_t qo_bytes = (uint64_t)num_seqs * num_heads * head_size * es;
    const uint64_t bt_bytes = (uint64_t)num_seqs * max_blocks_per_seq * 4;
    const uint64_t cl_bytes = (uint64_t)num_seqs * 4;
    if (overlap(out, qo_bytes, q, qo_bytes) || overlap(out, qo_bytes, block_tables, bt_bytes) ||
        overlap(out, qo_bytes, context_lens, cl_bytes))
        return FA_ERR_INVALID_ARG;
    *need = fa::decode_workspace_bytes(num_seqs, num_heads, max_context_len);
    return FA_OK;
}

}  // namespace

extern "C" int fa_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, const int32_t *context_lens,
                               void *out, int num_seqs, int num_heads, int num_kv_heads,
                               int head_size, int block_size, int max_blocks_per_seq,
                               int max_context_len, float scale, int dtype, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    size_t need = 0;
    const int st = decode_args(q, k_cache, v_cache, block_tables, context_lens, out, num_seqs,
                               num_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                               max_context_len, scale, dtype, &need);
    if (st != FA_OK) return st;
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGNMENT;
    // the workspace is written: it must not overlap q, the tables, the
    // context lengths or out
    const uint64_t qo_bytes = (uint64_t)num_seqs * num_heads * head_size * elem_bytes(dtype);
    if (overlap(workspace, need, q, qo_bytes) || overlap(workspace, need, out, qo_bytes) ||
        overlap(workspace, need, block_tables, (uint64_t)num_seqs * max_blocks_per_seq * 4) ||
        overlap(workspace, need, context_lens, (uint64_t)num_seqs * 4))
        return FA_ERR_INVALID_ARG;
    const hipError_t e = fa::decode_dispatch(q, k_cache, v_cache, block_tables, context_lens, out,
                                             num_seqs, num_heads, num_kv_heads, max_blocks_per_seq,
                                             max_context_len, scale, dtype, workspace,
                                             (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" int fa_paged_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, const int32_t *context_lens,
                                       void *out, int num_seqs, int num_heads, int num_kv_heads,
                                       int head_size, int block_size, int max_blocks_per_seq,
                                       int max_context_len, float scale, int dtype, void *stream)
{
    size_t need = 0;
    const int st = decode_args(q, k_cache, v_cache, block_tables, context_lens, out, num_seqs,
                               num_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                               max_context_len, scale, dtype, &need);
    if (st != FA_OK) return st;
    if (need > FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    // the scratch is the current device's: the stream must belong to it
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return FA_ERR_HIP;
        if (sdev != dev) return FA_ERR_INVALID_ARG;
    }
    const hipError_t e = fa::decode_noalloc_dispatch(q, k_cache, v_cache, block_tables, context_lens,
                                                     out, num_seqs, num_heads, num_kv_heads,
                                                     max_blocks_per_seq, max_context_len, scale,
                                                     dtype, (hipStream_t)stream);
    return launched(e, stream);
}

extern "C" const char *fa_strerror(int status)
{
    switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_ALIGNMENT: return "misaligned pointer";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    case FA_ERR_SCRATCH: return "sizes need more than the no-allocation decode's scratch holds";
    default: return "unknown status";
    }
}
