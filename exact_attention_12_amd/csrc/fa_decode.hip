// fa_decode.hip -- single-query attention over a paged KV cache, gfx950.
//
// Structure follows "PagedAttention" (data-sketchers.com wiki): one
// workgroup per (head, sequence, context partition); the query is held by
// every lane; each wave walks a share of the partition's cache blocks, forms
// q.k for the 16 tokens of a block with 16-byte vector loads and a cross-lane
// reduction (section "QK"); the logits go to LDS; a workgroup-wide max and
// exp-sum follow (sections "qk_max and logits", "exp_sum"); the values are
// accumulated per head element (sections "Value", "LV") and the partition's
// normalised partial result is written out (section "Output").  A second
// kernel merges the partitions with Eq. (4) of "Flash Attention"
// (suniverse77.github.io), generalised to P parts:
//     m = max_p m_p,  w_p = l_p e^(m_p - m),  out = sum_p w_p O_p / sum_p w_p.
//
// The lane map is this library's own, for 64-wide waves:
//  K block (16 tokens, [head/8][16][8] elements, 4 KiB contiguous): lane l
//    loads the 16-byte vectors l, l+64, l+128, l+192, i.e. token l % 16 and
//    head groups l/16 + 4c (c = 0..3); the 4 lanes of a token combine their
//    partial dots with two cross-lane exchanges.
//  V block ([head][16] elements, 4 KiB contiguous): lane l loads vectors
//    l + 64c, i.e. head element l/2 + 32c and tokens 8*(l%2) .. +7; partial
//    sums combine across the lane pair and then across waves through LDS.
#include "fa.h"
#include "fa_device.h"
#include "fa_sizes.h"
#include "fa_tile.h"

#include <atomic>

namespace fa {

constexpr int kDecD = 128;        // head size
constexpr int kDecBS = 16;        // tokens per cache block
constexpr int kDecPart = FA_DECODE_PARTITION_TOKENS;  // context tokens per partition
constexpr int kDecBlk = kDecPart / kDecBS;  // cache blocks per partition (16)
constexpr int kDecThreads = 256;  // 4 waves
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecBPW = kDecBlk / kDecWaves;  // blocks per wave (4)
static_assert(kDecThreads == kDecPart, "the softmax takes one token per thread");
// Dynamic LDS the partition launch reserves (unused) so that at most two
// workgroups share a compute unit's 160 KiB: a third one, which the register
// count would allow, adds concurrent streams of scattered 4 KiB blocks and
// measured about 3 % slower on the 64 x 32-head workload.
constexpr int kDecLdsReserve = 56 * 1024;

template <typename T> __device__ __forceinline__ float elem_to_f32(uint32_t bits16);
template <> __device__ __forceinline__ float elem_to_f32<_Float16>(uint32_t b)
{
    _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)b);
    return (float)x;
}
template <> __device__ __forceinline__ float elem_to_f32<__bf16>(uint32_t b)
{
    return __builtin_bit_cast(float, b << 16);
}

// element e (0..7) of a 16-byte vector of 16-bit values, widened exactly
template <typename T> __device__ __forceinline__ float vec_elem(const u32x4 &v, int e)
{
    return elem_to_f32<T>((v[e / 2] >> (16 * (e % 2))) & 0xffffu);
}

// c + a.lo * b.lo + a.hi * b.hi for two packed 16-bit pairs, accumulated in
// fp32 by the hardware's two-element dot instruction (the products of two
// 16-bit values are exact in fp32).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <> __device__ __forceinline__ float dot2<_Float16>(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}
template <> __device__ __forceinline__ float dot2<__bf16>(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// q . k over the 8 head elements of one 16-byte vector pair
template <typename T> __device__ __forceinline__ float dot8(const u32x4 &a, const u32x4 &b, float c)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) c = dot2<T>(a[e], b[e], c);
    return c;
}

// Cache block ids of the blocks a wave handles (b = wave + kDecWaves * i of
// the partition), read together with the context length rather than after
// it: the index is clamped to the sequence's table row (which holds at
// least one entry whenever a partition kernel runs), and entries past the
// context are never used.
template <int NB>
__device__ __forceinline__ void load_block_ids(int (&blk)[NB], const int32_t *__restrict__ row, int first,
                                               int stride, int max_blocks_per_seq)
{
#pragma unroll
    for (int i = 0; i < NB; ++i) blk[i] = row[min(first + stride * i, max_blocks_per_seq - 1)];
    // empty uses keep the loads above the caller's early exit
#pragma unroll
    for (int i = 0; i < NB; ++i) asm volatile("" : "+s"(blk[i]));
}

// Blocks i0 .. i0 + NP - 1 of a wave's share (block b = wave + kDecWaves * i
// of the partition) of one cache, K or V, 16 bytes per lane per load, as
// buffer loads that every path issues: a block past the partition's end
// gets a resource with an empty range (its loads return zeros and touch no
// memory).  With a fixed count of loads in flight the compiler's waits are
// exact.  The loads are non-temporal: each cache block is read once per
// call.  (The single-head kernel keeps its own loads.)
template <typename T, int NP>
__device__ __forceinline__ void load_blocks(u32x4 (&r)[NP][4], const T *cache, const int (&blk)[kDecBPW], int i0,
                                            int wave, int nblk, int num_kv_heads, int kvh, int lane)
{
    constexpr int kBlockBytes = kDecD * kDecBS * (int)sizeof(T);
    constexpr int kNonTemporal = 2;  // cache policy bit of the load
#pragma unroll
    for (int ii = 0; ii < NP; ++ii) {
        const int i = i0 + ii;
        const bool valid = wave + kDecWaves * i < nblk;
        const int64_t off = valid ? ((int64_t)blk[i] * num_kv_heads + kvh) * (kDecD * kDecBS) : 0;
        const __amdgpu_buffer_rsrc_t res =
            __builtin_amdgcn_make_buffer_rsrc((void *)(cache + off), 0, valid ? kBlockBytes : 0, kBufferFlags);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            r[ii][c] = __builtin_amdgcn_raw_buffer_load_b128(res, (lane + 64 * c) * 16, 0, kNonTemporal);
    }
}

struct DecWs {
    float *o;  // [S, H, P, D]
    float *m;  // [S, H, P]
    float *l;  // [S, H, P]
};

template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_decode_partition_kernel(const T *__restrict__ q, const T *__restrict__ kc,
                                const T *__restrict__ vc, const int32_t *__restrict__ block_tables,
                                const int32_t *__restrict__ context_lens, int num_heads,
                                int num_kv_heads, int max_blocks_per_seq, int nparts,
                                float scale, DecWs ws)
{
    const int h = blockIdx.x, s = blockIdx.y, p = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int t0 = p * kDecPart;
    const int ctx = context_lens[s];
    int blk[kDecBPW];
    load_block_ids(blk, block_tables + (int64_t)s * max_blocks_per_seq, t0 / kDecBS + wave, kDecWaves,
                   max_blocks_per_seq);
    const int64_t pidx = ((int64_t)s * num_heads + h) * nparts + p;
    if (t0 >= ctx) return;  // empty partition: the merge reads only partitions below ctx
    const int ntok = min(kDecPart, ctx - t0);
    const int nblk = (ntok + kDecBS - 1) / kDecBS;
    const int kvh = h / (num_heads / num_kv_heads);

    __shared__ __attribute__((aligned(16))) float logits[kDecPart];
    __shared__ float red[2][kDecWaves];
    __shared__ float part[kDecWaves][kDecD];
    poison_lds(logits, sizeof(logits));
    poison_lds(red, sizeof(red));
    poison_lds(part, sizeof(part));

    // q elements this lane dots with, packed: head groups g = lane/16 + 4c.
    u32x4 qv[4];
    {
        const T *qp = q + ((int64_t)s * num_heads + h) * kDecD;
#pragma unroll
        for (int c = 0; c < 4; ++c) qv[c] = *(const u32x4 *)(qp + (lane / 16 + 4 * c) * 8);
    }

    // Issue every K and V load of this wave's blocks up front.  Each cache
    // block is read once per call: the loads are non-temporal (streamed past
    // the caches), which measured 8 % faster than cached loads.
    u32x4 kr[kDecBPW][4], vr[kDecBPW][4];
#pragma unroll
    for (int i = 0; i < kDecBPW; ++i) {
        const int b = wave + kDecWaves * i;
        if (b < nblk) {
            const int64_t base = ((int64_t)blk[i] * num_kv_heads + kvh) * (kDecD * kDecBS);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                kr[i][c] = __builtin_nontemporal_load((const u32x4 *)(kc + base + (lane + 64 * c) * 8));
                vr[i][c] = __builtin_nontemporal_load((const u32x4 *)(vc + base + (lane + 64 * c) * 8));
            }
        }
    }

    // logits = scale * q . k for the tokens of each block
    float wmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < kDecBPW; ++i) {
        const int b = wave + kDecWaves * i;
        if (b < nblk) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) dot = dot8<T>(qv[c], kr[i][c], dot);
            dot += __shfl_xor(dot, 16, kWave);
            dot += __shfl_xor(dot, 32, kWave);
            const int tok = t0 + b * kDecBS + lane % 16;
            const float lg = (tok < ctx) ? scale * dot : -INFINITY;
            if (lane < 16) logits[b * kDecBS + lane] = lg;
            wmax = fmaxf(wmax, lg);
        }
    }
#pragma unroll
    for (int off = 8; off >= 1; off /= 2) wmax = fmaxf(wmax, __shfl_xor(wmax, off, kWave));
    if (lane == 0) red[0][wave] = wmax;
    __syncthreads();
    float m_p = red[0][0];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) m_p = fmaxf(m_p, red[0][w]);

    // p_t = exp(logit_t - m_p); l_p = sum_t p_t  (one token per thread)
    float pt = 0.f;
    if (tid < nblk * kDecBS) {
        pt = exp2_hw((logits[tid] - m_p) * kLog2e);  // masked: exp2(-inf) = 0
        logits[tid] = pt;
    }
    float ps = pt;
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) ps += __shfl_xor(ps, off, kWave);
    if (lane == 0) red[1][wave] = ps;
    __syncthreads();
    float l_p = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) l_p += red[1][w];

    // acc[c] = sum_t p_t V_t[e] for e = lane/2 + 32c over this lane's tokens
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kDecBPW; ++i) {
        const int b = wave + kDecWaves * i;
        if (b < nblk) {
            const int tb = b * kDecBS + 8 * (lane % 2);  // partition-relative first token
            const f32x4 pa = *(const f32x4 *)(logits + tb);
            const f32x4 pb = *(const f32x4 *)(logits + tb + 4);
            const float pw[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
            const int nvalid = ntok - tb;  // tokens >= ntok are outside the context
            if (nvalid >= 8) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[c] = __builtin_fmaf(pw[e], vec_elem<T>(vr[i][c], e), acc[c]);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (e < nvalid) acc[c] = __builtin_fmaf(pw[e], vec_elem<T>(vr[i][c], e), acc[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        acc[c] += __shfl_xor(acc[c], 1, kWave);
        if (lane % 2 == 0) part[wave][lane / 2 + 32 * c] = acc[c];
    }
    __syncthreads();
    if (tid < kDecD) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) o += part[w][tid];
        ws.o[pidx * kDecD + tid] = o / l_p;  // normalised partial ("exp_sum": logits * inv_sum)
    }
    if (tid == 0) {
        ws.m[pidx] = m_p;
        ws.l[pidx] = l_p;
    }
}

// Grouped-query variant (num_heads / num_kv_heads = G > 1): one workgroup per
// (kv head, sequence, partition) serves up to GM query heads of the group,
// so each K/V block is read from HBM once per kv head instead of once per
// query head.  The lane maps and the per-head softmax are those of the
// kernel above; the queries sit in LDS (16-bit) instead of registers, and every
// head has its own logits row, reductions and partial.
template <typename T, int GM>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_decode_gqa_partition_kernel(const T *__restrict__ q, const T *__restrict__ kc,
                                    const T *__restrict__ vc, const int32_t *__restrict__ block_tables,
                                    const int32_t *__restrict__ context_lens, int num_heads,
                                    int num_kv_heads, int max_blocks_per_seq, int nparts,
                                    float scale, DecWs ws)
{
    const int G = num_heads / num_kv_heads;
    const int ngroups = (G + GM - 1) / GM;
    const int kvh = blockIdx.x / ngroups, g0 = (blockIdx.x % ngroups) * GM;
    const int ng = min(GM, G - g0);  // query heads of this workgroup: kvh*G + g0 + g, g < ng
    const int s = blockIdx.y, p = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int t0 = p * kDecPart;
    const int ctx = context_lens[s];
    int blk[kDecBPW];
    load_block_ids(blk, block_tables + (int64_t)s * max_blocks_per_seq, t0 / kDecBS + wave, kDecWaves,
                   max_blocks_per_seq);
    if (t0 >= ctx) return;  // empty partition: the merge reads only partitions below ctx
    const int ntok = min(kDecPart, ctx - t0);
    const int nblk = (ntok + kDecBS - 1) / kDecBS;
    const int h0 = kvh * G + g0;

    // the group's queries, kept in their 16-bit type (64 words per head)
    __shared__ __attribute__((aligned(16))) uint32_t qs[GM][kDecD / 2];
    __shared__ __attribute__((aligned(16))) float logits[GM][kDecPart];
    __shared__ float red[2][GM][kDecWaves];
    __shared__ float part[kDecWaves][GM][kDecD];
    poison_lds(qs, sizeof(qs));
    poison_lds(logits, sizeof(logits));
    poison_lds(red, sizeof(red));
    poison_lds(part, sizeof(part));

    // Load order: the queries, then the K blocks; the V blocks only after the
    // logits, into registers that K leaves free, and in two halves, the
    // second after the first half's P.V products.  Holding all of K and V
    // took 156 registers (three workgroups per compute unit); this takes 96
    // (five), and the softmax's reductions still overlap V's arrival.
    constexpr int QW = (GM * (kDecD / 2) + kDecThreads - 1) / kDecThreads;  // query words per thread
    uint32_t qw[QW];
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        // (clamped rather than skipped: a load under a branch is waited for
        // at the branch's end)
        const int i = min(tid + j * kDecThreads, ng * (kDecD / 2) - 1);
        qw[j] = ((const uint32_t *)(q + ((int64_t)s * num_heads + h0) * kDecD))[i];
    }
    u32x4 kr[kDecBPW][4], vr[2][4];
    load_blocks<T, kDecBPW>(kr, kc, blk, 0, wave, nblk, num_kv_heads, kvh, lane);
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        const int i = tid + j * kDecThreads;
        if (i < ng * (kDecD / 2)) qs[i / (kDecD / 2)][i % (kDecD / 2)] = qw[j];
    }
    __syncthreads();

    // logits per head: lane l dots token l % 16 with head groups l/16 + 4c
    float wmax[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) wmax[g] = -INFINITY;
#pragma unroll
    for (int i = 0; i < kDecBPW; ++i) {
        const int b = wave + kDecWaves * i;
        if (b < nblk) {
            const int tok = t0 + b * kDecBS + lane % 16;
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                if (g < ng) {
                    float dot = 0.f;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        dot = dot8<T>(*(const u32x4 *)(&qs[g][(lane / 16 + 4 * c) * 4]), kr[i][c], dot);
                    dot += __shfl_xor(dot, 16, kWave);
                    dot += __shfl_xor(dot, 32, kWave);
                    const float lg = (tok < ctx) ? scale * dot : -INFINITY;
                    if (lane < 16) logits[g][b * kDecBS + lane] = lg;
                    wmax[g] = fmaxf(wmax[g], lg);
                }
            }
        }
    }
    load_blocks<T, 2>(vr, vc, blk, 0, wave, nblk, num_kv_heads, kvh, lane);  // V blocks 0, 1
#pragma unroll
    for (int g = 0; g < GM; ++g) {
#pragma unroll
        for (int off = 8; off >= 1; off /= 2) wmax[g] = fmaxf(wmax[g], __shfl_xor(wmax[g], off, kWave));
        if (lane == 0) red[0][g][wave] = wmax[g];
    }
    __syncthreads();

    // p_t = exp(logit_t - m_g), l_g = sum_t p_t, one token per thread, per head
    float l_p[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        float m_g = red[0][g][0];
#pragma unroll
        for (int w = 1; w < kDecWaves; ++w) m_g = fmaxf(m_g, red[0][g][w]);
        float pt = 0.f;
        if (g < ng && tid < nblk * kDecBS) {
            pt = exp2_hw((logits[g][tid] - m_g) * kLog2e);
            logits[g][tid] = pt;
        }
#pragma unroll
        for (int off = 32; off >= 1; off /= 2) pt += __shfl_xor(pt, off, kWave);
        if (lane == 0) red[1][g][wave] = pt;
        wmax[g] = m_g;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        l_p[g] = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) l_p[g] += red[1][g][w];
    }

    // acc[g][c] = sum_t p_t V_t[e], e = lane/2 + 32c, tokens 8*(lane%2) .. +7 of each block
    float acc[GM][4];
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[g][c] = 0.f;
    static_assert(kDecBPW == 4, "V in two halves of two blocks");
#pragma unroll
    for (int i = 0; i < kDecBPW; ++i) {
        if (i == 2) load_blocks<T, 2>(vr, vc, blk, 2, wave, nblk, num_kv_heads, kvh, lane);  // V blocks 2, 3
        const int b = wave + kDecWaves * i;
        if (b < nblk) {
            const int tb = b * kDecBS + 8 * (lane % 2);
            const int nvalid = ntok - tb;
            // tokens >= ntok are outside the context (their cache slots may
            // hold anything): their value halves are cleared, and p_t = 0
            u32x4 vv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) vv[c] = vr[i % 2][c];
            if (nvalid < 8) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        vv[c][e] &= (2 * e < nvalid ? 0xffffu : 0u) | (2 * e + 1 < nvalid ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                if (g < ng) {
                    // p rounded to the cache type, as the PagedAttention kernel
                    // does before its value dot ("LV"), then two tokens per
                    // dot instruction with fp32 accumulation
                    const f32x4 pa = *(const f32x4 *)(&logits[g][tb]);
                    const f32x4 pb = *(const f32x4 *)(&logits[g][tb + 4]);
                    const u32x4 pp = {Mma<T>::pack2(pa[0], pa[1]), Mma<T>::pack2(pa[2], pa[3]),
                                      Mma<T>::pack2(pb[0], pb[1]), Mma<T>::pack2(pb[2], pb[3])};
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[g][c] = dot8<T>(pp, vv[c], acc[g][c]);
                }
            }
        }
    }
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc[g][c] += __shfl_xor(acc[g][c], 1, kWave);
            if (lane % 2 == 0) part[wave][g][lane / 2 + 32 * c] = acc[g][c];
        }
    __syncthreads();
    if (tid < kDecD) {
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < ng) {
                float o = 0.f;
#pragma unroll
                for (int w = 0; w < kDecWaves; ++w) o += part[w][g][tid];
                const int64_t pidx = ((int64_t)s * num_heads + h0 + g) * nparts + p;
                ws.o[pidx * kDecD + tid] = o / l_p[g];
                if (tid == 0) {
                    ws.m[pidx] = wmax[g];
                    ws.l[pidx] = l_p[g];
                }
            }
        }
    }
}

template <typename T> __device__ __forceinline__ T f32_to_elem(float x) { return (T)x; }

// Merge of the partitions of one (sequence, head) row per wave, four rows
// per workgroup, in chunks of kMergeChunk partitions: every load of a chunk
// (maxima and sums on lanes 0..15, two head elements of each partial on
// every lane) is issued at once, and the chunks combine with Eq. (4) of
// "Flash Attention", the running result rescaled by e^(M_old - M_new).
constexpr int kMergeRows = 4;
constexpr int kMergeChunk = 16;
template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_decode_merge_kernel(const int32_t *__restrict__ context_lens, T *__restrict__ out,
                            int rows, int num_heads, int nparts, DecWs ws)
{
    const int r = blockIdx.x * kMergeRows + threadIdx.x / kWave;
    if (r >= rows) return;
    const int lane = threadIdx.x % kWave;
    const int ctx = context_lens[r / num_heads];
    const int np = min(nparts, (ctx + kDecPart - 1) / kDecPart);
    const int64_t base = (int64_t)r * nparts;
    float M = -INFINITY, wsum = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p0 = 0; p0 < np; p0 += kMergeChunk) {
        const int n = min(kMergeChunk, np - p0);
        float mj = -INFINITY, lj = 0.f;
        if (lane < n) {
            mj = ws.m[base + p0 + lane];
            lj = ws.l[base + p0 + lane];
        }
        f32x2 ov[kMergeChunk];
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k)
            ov[k] = k < n ? *(const f32x2 *)(ws.o + (base + p0 + k) * kDecD + 2 * lane) : f32x2{0.f, 0.f};
        // every partition below np holds at least one token, so mc is finite
        float mc = mj;
#pragma unroll
        for (int off = kMergeChunk / 2; off >= 1; off /= 2) mc = fmaxf(mc, __shfl_xor(mc, off, kWave));
        const float Mn = fmaxf(M, __shfl(mc, 0, kWave));
        const float a = exp2_hw((M - Mn) * kLog2e);  // 0 for the first chunk
        const float w = lane < n ? lj * exp2_hw((mj - Mn) * kLog2e) : 0.f;
        wsum = wsum * a + w;
        o0 *= a;
        o1 *= a;
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
            const float wk = __shfl(w, k, kWave);
            o0 = __builtin_fmaf(wk, ov[k][0], o0);
            o1 = __builtin_fmaf(wk, ov[k][1], o1);
        }
        M = Mn;
    }
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) wsum += __shfl_xor(wsum, off, kWave);
    const float inv = np > 0 ? 1.f / wsum : 0.f;
    T *orow = out + (int64_t)r * kDecD + 2 * lane;
    orow[0] = f32_to_elem<T>(o0 * inv);
    orow[1] = f32_to_elem<T>(o1 * inv);
}

template <typename T>
static hipError_t launch_decode(const void *q, const void *kc, const void *vc, const int32_t *bt,
                                const int32_t *cl, void *out, int S, int H, int Hkv, int MB,
                                int max_ctx, float scale, void *workspace, hipStream_t stream)
{
    const int np = (max_ctx + kDecPart - 1) / kDecPart;
    if (np == 0) {
        // every context is empty: the merge writes zeros
        DecWs ws{(float *)workspace, (float *)workspace, (float *)workspace};
        hipLaunchKernelGGL(fa_decode_merge_kernel<T>, dim3((S * H + kMergeRows - 1) / kMergeRows),
                           dim3(kMergeRows * kWave), 0, stream, cl, (T *)out, S * H, H, 0, ws);
        return hipGetLastError();
    }
    const int64_t parts = (int64_t)S * H * np;
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    char *w = (char *)workspace;
    DecWs ws{(float *)w, (float *)(w + up(parts * kDecD * 4)),
             (float *)(w + up(parts * kDecD * 4) + up(parts * 4))};
    const int G = H / Hkv;
    if (G == 1) {
        hipLaunchKernelGGL(fa_decode_partition_kernel<T>, dim3(H, S, np), dim3(kDecThreads), kDecLdsReserve,
                           stream, (const T *)q, (const T *)kc, (const T *)vc, bt, cl, H, Hkv, MB,
                           np, scale, ws);
    } else {
        // one workgroup per (kv head, group of up to GM query heads)
        auto gqa = [&](auto kern, int gm) {
            const int ngroups = (G + gm - 1) / gm;
            hipLaunchKernelGGL(kern, dim3(Hkv * ngroups, S, np), dim3(kDecThreads), 0, stream,
                               (const T *)q, (const T *)kc, (const T *)vc, bt, cl, H, Hkv, MB, np,
                               scale, ws);
        };
        if (G <= 2)
            gqa(fa_decode_gqa_partition_kernel<T, 2>, 2);
        else if (G <= 4)
            gqa(fa_decode_gqa_partition_kernel<T, 4>, 4);
        else
            gqa(fa_decode_gqa_partition_kernel<T, 8>, 8);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fa_decode_merge_kernel<T>, dim3((S * H + kMergeRows - 1) / kMergeRows),
                       dim3(kMergeRows * kWave), 0, stream, cl, (T *)out, S * H, H, np, ws);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of fa_paged_decode_noalloc: the per-partition partials go to this
// file-scope device array instead of a caller's workspace.  Every GPU the
// library runs on holds its own copy (loaded with the code object, kept until
// the process ends).  In host code the name `scratch` is only a host-side
// stand-in: the device address comes from hipGetSymbolAddress, taken once
// per device with that device current and kept in scratch_ptr[].
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
static std::atomic<void *> scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`.
static hipError_t scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // two threads may both look it up the first time: same address
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t decode_dispatch(const void *q, const void *kc, const void *vc, const int32_t *bt,
                           const int32_t *cl, void *out, int S, int H, int Hkv, int MB,
                           int max_ctx, float scale, int dtype, void *workspace,
                           hipStream_t stream)
{
    if (dtype == 2)
        return launch_decode<_Float16>(q, kc, vc, bt, cl, out, S, H, Hkv, MB, max_ctx, scale,
                                       workspace, stream);
    return launch_decode<__bf16>(q, kc, vc, bt, cl, out, S, H, Hkv, MB, max_ctx, scale, workspace,
                                 stream);
}

// The paged decode with its partials in `scratch`.  Arguments validated by
// the caller, including decode_workspace_bytes(S, H, max_ctx) <=
// FA_DECODE_NOALLOC_SCRATCH_BYTES; `stream` belongs to the current device.
// Nothing in the scratch needs clearing: the merge reads only partitions
// below each context's end, which this call's partition kernel writes.
hipError_t decode_noalloc_dispatch(const void *q, const void *kc, const void *vc, const int32_t *bt,
                                   const int32_t *cl, void *out, int S, int H, int Hkv, int MB,
                                   int max_ctx, float scale, int dtype, hipStream_t stream)
{
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return decode_dispatch(q, kc, vc, bt, cl, out, S, H, Hkv, MB, max_ctx, scale, dtype, ws, stream);
}

}  // namespace fa
