// fa_fp8.hip -- block-scaled FP8 (E4M3) attention forward for gfx950.
//
// FlashAttention-3 runs attention in FP8 and keeps a separate scale factor per
// block of the inputs so that each block uses the FP8 range ("FlashAttention:
// GPU 메모리 계층을 활용한 어텐션 최적화 분석", youngju.dev, section 9.2,
// item 3).  Here:
//  - E4M3 is the OCP format (bias 7, largest finite 448), which gfx950's
//    matrix cores and conversion instructions use;
//  - a block is 128 consecutive rows of one (b, h) with all d columns; its
//    scale is the power of two 2^e, e = floor(log2 amax) - 7, so that every
//    scaled value is below 256 and the scaling itself is exact;
//  - code = E4M3 rounding (nearest, ties to even) of x * 2^-e.
//
// fa_quant_fp8_kernel quantises one block per workgroup.  Q and K codes keep
// the [B, H, N, d] layout; V codes are stored as 64-key tiles, each d-major
// ([B, H, ceil(N/64), d, 64]), so that the P.V product reads its operand
// straight from rows of the tile.
//
// fa_fwd_fp8_kernel is the FA2-order forward of fa_fwd.hip on the FP8 matrix
// instruction v_mfma_f32_32x32x64_f8f6f4 (64-deep contraction, 32 bytes per
// lane):
//  - S^T = K Q^T with Q rows in registers and K tiles (64 keys) in LDS;
//    the raw dot products of the codes are scaled by scale * 2^(e_q + e_k)
//    per tile.  The matrix instruction sums its products in groups of 8 along
//    the contraction, and inside a group drops the bits of a product below
//    about 2^-13 of the group's largest one (measured: 256 + 7 x 2^-6 gives
//    256); across groups it accumulates in fp32.  Scores are therefore exact
//    only when the products of a group are within ~2^13 of each other, as
//    they are for data without a dominant head dimension;
//  - the rows of each K tile are permuted as they land in LDS, so that the
//    accumulator register r of block kb in lane half h holds key
//    32 h + 16 kb + r of the tile.  The 32 probabilities a lane packs (one
//    byte each) then belong to keys 32 h .. 32 h + 31, which is exactly the
//    run of bytes the lane reads from a row of the d-major V tile: the P.V
//    operands need no transpose and no shuffle;
//  - P~ = 2^(s c - m_ref) is rounded to E4M3 for the P.V product.  The V
//    block scale enters that product through the instruction's E8M0 scale
//    operand as 2^(e_v - e_vmax) (exact, and P~ keeps its own precision
//    whatever the V block's magnitude); the output is multiplied by 2^e_vmax
//    at the end;
//  - the lazy reference max of the bf16 forward, with the bound on P~ at 2^8
//    so that every probability is a finite E4M3 value; O = acc / l with l
//    the fp32 sum of the unrounded probabilities; lse = m + ln l.
#include "fa_tile.h"

#include <climits>
#include <type_traits>

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace f8 {

constexpr int D = 128;            // head dimension
constexpr int NT = 256;           // threads per workgroup (4 waves)
constexpr int BR = 128;           // query rows per workgroup
constexpr int BC = 64;            // keys per K/V tile
constexpr int KROWB = D;          // bytes per K row
constexpr int KTILEB = BC * KROWB;  // 8 KiB
constexpr int VROWB = BC;         // bytes per d-row of a V tile
constexpr int VTILEB = D * VROWB; // 8 KiB
constexpr int STAGEB = KTILEB + VTILEB;
constexpr int QSTEPS = D / 64;    // matrix steps over d
constexpr int DB = D / 32;        // 32-row blocks of O^T
constexpr int QBLK = 128;         // rows per quantisation block
constexpr float kPMax = 256.0f;   // bound on P~: every value is a finite E4M3 number
// the forward takes one Q block exponent per workgroup: its query tile must be
// exactly one quantisation block
static_assert(BR == QBLK, "a query tile is one block of Q's scales");

// 16-byte chunk swizzles (position = chunk ^ swz(row)); both keep a 16-lane
// pass of row-fragment reads (16 consecutive rows, one chunk) on 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 7; }  // 8 chunks per K row
__device__ __forceinline__ int vswz(int row) { return (row >> 2) & 3; }  // 4 chunks per V row

// Tile key held by LDS row R of a K tile: block kb = R / 32, accumulator row
// i = R % 32 = 8 (r / 4) + 4 h + r % 4 holds key 32 h + 16 kb + r.
__device__ __forceinline__ int krow_key(int R)
{
    const int kb = R / 32, i = R % 32;
    const int h = (i / 4) % 2, r = (i / 8) * 4 + i % 4;
    return 32 * h + 16 * kb + r;
}

}  // namespace f8

// ---------------------------------------------------------------------------
// Quantisation: one workgroup per (b*h, 128-row block)
// ---------------------------------------------------------------------------
template <typename T, int DD, int LAYOUT>
__global__ __launch_bounds__(256) void fa_quant_fp8_kernel(const T *__restrict__ X,
                                                           uint8_t *__restrict__ codes,
                                                           int32_t *__restrict__ exps, int N)
{
    constexpr int ES = (int)sizeof(T);
    constexpr int VEC = 16 / ES;                  // elements per 16-byte load
    constexpr int PER = f8::QBLK * DD / 256;      // elements per thread
    constexpr int NV = PER / VEC;                 // 16-byte loads per thread
    constexpr int CPR = DD / VEC;                 // loads per row
    __shared__ float red[4];
    __shared__ __attribute__((aligned(16))) uint8_t tile[f8::QBLK * DD];
    poison_lds(red, sizeof(red));
    poison_lds(tile, sizeof(tile));

    const int nblk = (N + f8::QBLK - 1) / f8::QBLK;
    const int64_t bh = blockIdx.x / nblk;
    const int blk = blockIdx.x % nblk;
    const int r0 = blk * f8::QBLK;
    const int rows = min(f8::QBLK, N - r0);
    const T *src = X + (bh * N + r0) * DD;
    const int tid = threadIdx.x;

    float v[PER];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = i * 256 + tid;  // 16-byte chunk index within the block
        const int row = c / CPR;
        if (row < rows) {
            typedef T tvec __attribute__((ext_vector_type(VEC)));
            // read once: streamed past the caches (measured 9 % faster)
            const tvec x = __builtin_nontemporal_load((const tvec *)(src + (int64_t)c * VEC));
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                v[i * VEC + e] = (float)x[e];
                amax = fmaxf(amax, fabsf(v[i * VEC + e]));
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[i * VEC + e] = 0.f;
        }
    }
    // workgroup max (exact: max of exact values)
#pragma unroll
    for (int m = 32; m >= 1; m /= 2) amax = fmaxf(amax, __shfl_xor(amax, m));
    if (tid % kWave == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (amax > 0.f) {
        int ex;
        frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1)
        e = (ex - 1) - 7;
    }
    if (tid == 0) exps[bh * nblk + blk] = e;

    // codes: x * 2^-e is exact (a power-of-two scaling of a value below 2^8);
    // the conversion rounds to nearest even
    uint32_t w[PER / 4];
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * j], -e), ldexpf(v[4 * j + 1], -e), 0, false);
        w[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * j + 2], -e), ldexpf(v[4 * j + 3], -e), lo, true);
    }
    if constexpr (LAYOUT == 0) {
        uint8_t *dst = codes + (bh * N + r0) * DD;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = i * 256 + tid;
            if (c / CPR < rows) {
                if constexpr (VEC == 8)
                    *(u32x2 *)(dst + (int64_t)c * VEC) = u32x2{w[2 * i], w[2 * i + 1]};
                else
                    *(uint32_t *)(dst + (int64_t)c * VEC) = w[i];
            }
        }
    } else {
        // stage the block's codes row-major in LDS, then write each 64-key
        // tile d-major: output byte (t, col, key) = code (64 t + key, col)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = i * 256 + tid;
            if constexpr (VEC == 8)
                *(u32x2 *)(tile + c * VEC) = u32x2{w[2 * i], w[2 * i + 1]};
            else
                *(uint32_t *)(tile + c * VEC) = w[i];
        }
        __syncthreads();
        const int ntile = (N + 63) / 64;
        const int t0 = blk * 2;  // first 64-key tile of this block
        // 2 tiles x DD rows x 4 chunks of 16 keys
        for (int q = tid; q < 2 * DD * 4; q += 256) {
            const int t = q / (DD * 4), col = (q / 4) % DD, kc = q % 4;
            if (t0 + t >= ntile) continue;
            uint8_t b[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int row = t * 64 + kc * 16 + k;  // row within the block
                b[k] = row < rows ? tile[row * DD + col] : (uint8_t)0;
            }
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = (uint32_t)b[4 * k] | ((uint32_t)b[4 * k + 1] << 8) | ((uint32_t)b[4 * k + 2] << 16) |
                       ((uint32_t)b[4 * k + 3] << 24);
            *(u32x4 *)(codes + ((bh * ntile + t0 + t) * DD + col) * 64 + kc * 16) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 forward
// Quantisation to the d-major V layout without an LDS pass: thread (g, j)
// of a workgroup takes rows RT g .. RT g + RT-1 and columns 8 j .. 8 j + 7 of
// the 128-row block (RT = 8 for d = 128, 4 for d = 64), computes their codes
// as above, transposes its RT x 8 bytes in registers, and writes for each of
// its 8 columns the RT consecutive keys that the output holds contiguously:
// byte (t, col, key) = code (64 t + key, col).  Rows past N are written as
// code 0 up to the end of their 64-key tile.
template <typename T, int DD>
__global__ __launch_bounds__(256) void fa_quant_fp8_vt_kernel(const T *__restrict__ X,
                                                              uint8_t *__restrict__ codes,
                                                              int32_t *__restrict__ exps, int N)
{
    constexpr int RT = f8::QBLK * DD / 256 / 8;  // rows per thread (8 columns each)
    constexpr int NGR = f8::QBLK / RT;           // row groups
    static_assert(NGR * (DD / 8) == 256, "one 8-column x RT-row piece per thread");
    constexpr int ES = (int)sizeof(T);
    constexpr int LPR = 8 * ES / 16;             // 16-byte loads per 8 columns of a row
    constexpr int VEC = 16 / ES;
    __shared__ float red[4];
    poison_lds(red, sizeof(red));

    const int nblk = (N + f8::QBLK - 1) / f8::QBLK;
    const int64_t bh = blockIdx.x / nblk;
    const int blk = blockIdx.x % nblk;
    const int r0 = blk * f8::QBLK;
    const int rows = min(f8::QBLK, N - r0);
    const int tid = threadIdx.x;
    const int g = tid % NGR, j = tid / NGR;
    const T *src = X + (bh * N + r0) * DD + 8 * j;

    typedef T tvec __attribute__((ext_vector_type(VEC)));
    float v[RT][8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int row = RT * g + i;
#pragma unroll
        for (int l = 0; l < LPR; ++l) {
            if (row < rows) {
                const tvec x = __builtin_nontemporal_load((const tvec *)(src + (int64_t)row * DD + l * VEC));
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    v[i][l * VEC + e] = (float)x[e];
                    amax = fmaxf(amax, fabsf(v[i][l * VEC + e]));
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) v[i][l * VEC + e] = 0.f;
            }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m /= 2) amax = fmaxf(amax, __shfl_xor(amax, m));
    if (tid % kWave == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (amax > 0.f) {
        int ex;
        frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1)
        e = (ex - 1) - 7;
    }
    if (tid == 0) exps[bh * nblk + blk] = e;

    // codes of row i: w[i][0] = columns 0..3, w[i][1] = columns 4..7 (byte c % 4)
    uint32_t w[RT][2];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const float *x = &v[i][4 * hlf];
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[0], -e), ldexpf(x[1], -e), 0, false);
            w[i][hlf] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[2], -e), ldexpf(x[3], -e), lo, true);
        }
    const int ntile = (N + 63) / 64;
    const int t = 2 * blk + (RT * g) / 64, key0 = (RT * g) % 64;
    if (t >= ntile) return;
    uint8_t *dst = codes + ((bh * ntile + t) * DD + 8 * j) * 64 + key0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        // keys key0 .. key0 + RT-1 of column 8 j + c, 4 per word
        uint32_t o[RT / 4];
#pragma unroll
        for (int q = 0; q < RT / 4; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) word |= ((w[4 * q + b][c / 4] >> (8 * (c % 4))) & 0xffu) << (8 * b);
            o[q] = word;
        }
        if constexpr (RT == 8)
            *(u32x2 *)(dst + c * 64) = u32x2{o[0], o[1]};
        else
            *(uint32_t *)(dst + c * 64) = o[0];
    }
}

// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K,
                       const uint8_t *__restrict__ V, const int32_t *__restrict__ QE,
                       const int32_t *__restrict__ KE, const int32_t *__restrict__ VE,
                       float *__restrict__ O, float *__restrict__ LSE, int N, int num_qtiles,
                       float scale, int H, int group)
{
    using namespace f8;
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGEB];
    poison_lds(smem, sizeof(smem));

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col = lane % 32;
    const int h = lane / 32;

    int wid = blockIdx.x;
    const int G = gridDim.x;
    if (G % 8 == 0) wid = (wid % 8) * (G / 8) + wid / 8;
    const int wg_per_head = CAUSAL ? (num_qtiles + 1) / 2 : num_qtiles;
    const int bh = wid / wg_per_head;
    const int pi = wid % wg_per_head;
    const int kvh = (bh / H) * (H / group) + (bh % H) / group;
    const int nblk = (N + QBLK - 1) / QBLK;
    const int NTk = (N + BC - 1) / BC;  // 64-key tiles of V
    const uint8_t *Qh = Q + (int64_t)bh * N * D;
    const uint8_t *Kh = K + (int64_t)kvh * N * D;
    const uint8_t *Vh = V + (int64_t)kvh * NTk * VTILEB;
    const int32_t *QEh = QE + (int64_t)bh * nblk;
    const int32_t *KEh = KE + (int64_t)kvh * nblk;
    const int32_t *VEh = VE + (int64_t)kvh * nblk;

    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)Kh, 0, N * KROWB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)Vh, 0, NTk * VTILEB, kBufferFlags);

    // Direct-to-LDS loads: 8 of 1 KiB per tile for K and for V, 2 each per
    // wave.  Lane l of load I writes LDS chunk position p = I*64 + l.
    // K: LDS row R = p / 8 holds tile key krow_key(R); V: LDS row p / 4 is
    // d-row p / 4 of the tile.
    int k_row[2], k_off[2], v_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = (wave * 2 + i) * kWave + lane;
        const int R = p / 8;
        k_row[i] = krow_key(R);
        k_off[i] = k_row[i] * KROWB + ((p % 8) ^ kswz(R)) * 16;
        const int vr = p / 4;
        v_off[i] = vr * VROWB + ((p % 4) ^ vswz(vr)) * 16;
    }
    auto load_tile = [&](int j, int buf) __attribute__((always_inline)) {
        const int k0 = j * BC;
        char *kd = smem + buf * STAGEB;
        char *vd = kd + KTILEB;
        if (k0 + BC <= N) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int I = wave * 2 + i;
                buffer_load_lds16(krs, kd + I * 1024, k_off[i], k0 * KROWB);
                buffer_load_lds16(vrs, vd + I * 1024, v_off[i], j * VTILEB);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int I = wave * 2 + i;
                // keys past the end re-read key N-1 (finite; masked below)
                const int over = k0 + k_row[i] - (N - 1);
                buffer_load_lds16(krs, kd + I * 1024, over > 0 ? k_off[i] - over * KROWB : k_off[i], k0 * KROWB);
                buffer_load_lds16(vrs, vd + I * 1024, v_off[i], j * VTILEB);
            }
        }
    };
    // per-lane LDS read offsets: K row fragment (row col of block kb, bytes
    // st*64 + 32h .. +31 = chunks 4st + 2h, +1); V row (d-row db*32 + col,
    // bytes 32h .. +31 = chunks 2h, 2h + 1)
    int k_rd[QSTEPS][2], v_rd[DB][2];
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) k_rd[st][c2] = col * KROWB + (((4 * st + 2 * h + c2) ^ kswz(col)) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            const int vr = db * 32 + col;
            v_rd[db][c2] = vr * VROWB + (((2 * h + c2) ^ vswz(vr)) * 16);
        }

    int evmax = INT_MIN;
    for (int b = 0; b < nblk; ++b) evmax = max(evmax, VEh[b]);
    const float c0 = fmaxf(scale * kLog2e, 1e-30f);

    for (int item = 0; item < (CAUSAL ? 2 : 1); ++item) {
        const int qt = CAUSAL ? (item == 0 ? num_qtiles - 1 - pi : pi) : pi;
        if (CAUSAL && item == 1 && qt == num_qtiles - 1 - pi) break;
        const int q0 = qt * BR;
        const int qrow = q0 + wave * 32 + col;
        const int wq_lo = q0 + wave * 32, wq_hi = wq_lo + 31;
        i32x8 qf[QSTEPS];
#pragma unroll
        for (int st = 0; st < QSTEPS; ++st)
            qf[st] = qrow < N ? *(const i32x8 *)(Qh + (int64_t)qrow * D + st * 64 + h * 32) : i32x8{};
        // c for this query block: scale * log2(e) * 2^e_q (times 2^e_k per tile)
        const float cq = ldexpf(c0, QEh[q0 / QBLK]);
        const int kend = CAUSAL ? min(N, q0 + BR) : N;
        const int ntiles = (kend + BC - 1) / BC;
        const int nt_w = CAUSAL ? min(ntiles, wq_hi / BC + 1) : ntiles;

        f32x16 acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
        float mref = -INFINITY;  // reference max of s*c (log2 units)
        float l_run = 0.f;       // sum of the unrounded P~ (unshifted)

        load_tile(0, 0);
        // block scale exponents of the tile being processed; those of the
        // next tile are read one tile ahead so that the scalar load latency
        // hides behind the tile's work
        int ke_next = KEh[0], ve_next = VEh[0];
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        auto tile = [&](int j, auto stage_c) __attribute__((always_inline)) {
            constexpr int STAGE = decltype(stage_c)::value;
            if (j + 1 < ntiles) load_tile(j + 1, STAGE ^ 1);
            const int k0 = j * BC;
            const char *Ks = smem + STAGE * STAGEB;
            const char *Vs = Ks + KTILEB;
            const float c = ldexpf(cq, ke_next);
            // V block scale relative to the largest, <= 0; applied to the V
            // operand of the P.V product through the instruction's E8M0
            // scale (2^(x - 127)).  A block more than 2^127 below the largest
            // contributes nothing (no E8M0 value represents its scale).
            const int vsh = ve_next - evmax;

            // S^T = K Q^T: lane (col = query, h), register r of block kb holds
            // tile key 32h + 16kb + r
            f32x16 s[2];
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int st = 0; st < QSTEPS; ++st) {
                    const char *kr = Ks + kb * 32 * KROWB;
                    const u32x4 a0 = *(const u32x4 *)(kr + k_rd[st][0]);
                    const u32x4 a1 = *(const u32x4 *)(kr + k_rd[st][1]);
                    const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                    s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[st], st == 0 ? f32x16{} : s[kb],
                                                                            0, 0, 0, 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            {
                const int nb = min((k0 + BC) / QBLK, nblk - 1);
                ke_next = KEh[nb];
                ve_next = VEh[nb];
            }

            // masks: key k0 + 32h + 16kb + r is visible iff 16kb + r <= lim
            const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > wq_lo);
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - k0 - 32 * h;
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (16 * kb + r > lim) s[kb][r] = -INFINITY;
            }
            // lazy reference max (see fa_fwd.hip): set on the first tile,
            // moved only when some P~ would exceed kPMax
            auto rebase = [&]() __attribute__((always_inline)) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
                mx = halves_max(mx) * c;
                const float mnew = fmaxf(mref, mx);
                const float msafe = mnew == -INFINITY ? 0.f : mnew;
                const float alpha = exp2_hw(mref - msafe);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
                mref = msafe;
            };
            // P~ = 2^(s c - mref); returns this lane's sum
            auto exponentiate = [&](f32x16 (&p)[2]) __attribute__((always_inline)) {
                const float sub = mref;
                float part[4];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        p[kb][r] = exp2_hw(__builtin_fmaf(s[kb][r], c, -sub));
                        part[r % 4] = (kb == 0 && r < 4) ? p[kb][r] : part[r % 4] + p[kb][r];
                    }
                return (part[0] + part[1]) + (part[2] + part[3]);
            };
            f32x16 p[2];
            if (j == 0) rebase();
            float rs = exponentiate(p);
            if (j != 0 && __builtin_amdgcn_ballot_w64(!(rs <= kPMax)) != 0) {
                rebase();
                rs = exponentiate(p);
            }
            l_run += rs;

            // P~ as E4M3: byte 16kb + r of the lane's 32 is register r of block kb
            // (the first conversion of a word writes its low half and the
            // second its high half, so the word's prior contents never show)
            i32x8 pb;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    int undef_word;
                    asm volatile("" : "=v"(undef_word));
                    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][4 * w], p[kb][4 * w + 1], undef_word, false);
                    pb[4 * kb + w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][4 * w + 2], p[kb][4 * w + 3], lo, true);
                }
            // O^T += 2^vsh V^T P~^T: lane (col = d row of the block, h) reads
            // bytes 32h .. 32h+31 of its V tile row: keys 32h .. 32h+31
            if (vsh >= -127) {
                const int vscale = 127 + vsh;  // E8M0 code of 2^vsh
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x4 a0 = *(const u32x4 *)(Vs + v_rd[db][0]);
                    const u32x4 a1 = *(const u32x4 *)(Vs + v_rd[db][1]);
                    const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                    acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, acc[db], 0, 0, 0, vscale, 0, 127);
                }
                __builtin_amdgcn_s_setprio(0);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };

        int j = 0;
        for (; j + 1 < nt_w; j += 2) {
            tile(j, std::integral_constant<int, 0>{});
            tile(j + 1, std::integral_constant<int, 1>{});
        }
        if (j < nt_w) {
            tile(j, std::integral_constant<int, 0>{});
            ++j;
        }
        for (; j < ntiles; ++j) {
            if (j + 1 < ntiles) load_tile(j + 1, (j + 1) & 1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // O = acc 2^evmax / l, lse = (mref + log2 l) ln 2
        const float l_tot = halves_sum(l_run);
        const float inv = ldexpf(1.f / l_tot, evmax);
        if (qrow < N) {
            float *orow = O + (int64_t)bh * N * D + (int64_t)qrow * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = db * 32 + 8 * r4 + 4 * h;
                    *(f32x4 *)(orow + d) = f32x4{acc[db][4 * r4 + 0] * inv, acc[db][4 * r4 + 1] * inv,
                                                acc[db][4 * r4 + 2] * inv, acc[db][4 * r4 + 3] * inv};
                }
            if (h == 0) LSE[(int64_t)bh * N + qrow] = (mref + log2_hw(l_tot)) * kLn2;
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <typename T, int DD>
static hipError_t launch_quant(const void *x, int B, int H, int N, int layout, void *codes, int32_t *exps,
                               hipStream_t stream)
{
    const int nblk = (N + f8::QBLK - 1) / f8::QBLK;
    const dim3 grid((unsigned)((int64_t)B * H * nblk));
    if (layout == 0)
        hipLaunchKernelGGL((fa_quant_fp8_kernel<T, DD, 0>), grid, dim3(256), 0, stream, (const T *)x,
                           (uint8_t *)codes, exps, N);
    else
        hipLaunchKernelGGL((fa_quant_fp8_vt_kernel<T, DD>), grid, dim3(256), 0, stream, (const T *)x,
                           (uint8_t *)codes, exps, N);
    return hipGetLastError();
}

// Arguments validated by the caller: dtype 0/1/2 = fp32/bf16/fp16, d in
// {64, 128}, layout 0 or 1.
hipError_t quant_fp8_dispatch(const void *x, int dtype, int B, int H, int N, int d, int layout,
                              void *codes, int32_t *exps, hipStream_t stream)
{
    switch (dtype) {
    case 0:
        return d == 64 ? launch_quant<float, 64>(x, B, H, N, layout, codes, exps, stream)
                       : launch_quant<float, 128>(x, B, H, N, layout, codes, exps, stream);
    case 1:
        return d == 64 ? launch_quant<__bf16, 64>(x, B, H, N, layout, codes, exps, stream)
                       : launch_quant<__bf16, 128>(x, B, H, N, layout, codes, exps, stream);
    default:
        return d == 64 ? launch_quant<_Float16, 64>(x, B, H, N, layout, codes, exps, stream)
                       : launch_quant<_Float16, 128>(x, B, H, N, layout, codes, exps, stream);
    }
}

// Arguments validated by the caller: d = 128, Hkv divides H.
hipError_t fwd_fp8_dispatch(const void *q8, const void *k8, const void *v8, const int32_t *qe,
                            const int32_t *ke, const int32_t *ve, float *o, float *lse, int B, int H,
                            int Hkv, int N, float scale, int causal, hipStream_t stream)
{
    const int nqt = (N + f8::BR - 1) / f8::BR;
    const int64_t grid = (int64_t)B * H * (causal ? (nqt + 1) / 2 : nqt);
    if (causal)
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<true>), dim3((unsigned)grid), dim3(f8::NT), 0, stream,
                           (const uint8_t *)q8, (const uint8_t *)k8, (const uint8_t *)v8, qe, ke, ve, o,
                           lse, N, nqt, scale, H, H / Hkv);
    else
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<false>), dim3((unsigned)grid), dim3(f8::NT), 0, stream,
                           (const uint8_t *)q8, (const uint8_t *)k8, (const uint8_t *)v8, qe, ke, ve, o,
                           lse, N, nqt, scale, H, H / Hkv);
    return hipGetLastError();
}

}  // namespace fa
