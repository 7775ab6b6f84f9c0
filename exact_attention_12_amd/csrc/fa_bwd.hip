// fa_bwd.hip -- FlashAttention backward pass for gfx950.
//
// Gradients dQ, dK, dV of O = softmax(scale * Q K^T [+ causal mask]) V for an
// upstream gradient dO.  As the pages describe ("FlashAttention: GPU 메모리
// 계층을 활용한 어텐션 최적화 분석", youngju.dev, sections 7.1-7.3), neither S
// nor P is stored by the forward pass: the blocks of P are recomputed on chip
// from Q, K and the per-row log-sum-exp lse that the forward pass saved,
//     P_ij = exp(scale q_i.k_j - lse_i),
// and the gradients follow from the chain rule:
//     dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   D_i = dO_i . O_i,
//     dS_ij = P_ij (dP_ij - D_i),
//     dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i.
// (D_i = sum_j P_ij dP_ij equals dO_i . O_i, which costs one pass over the
// rows instead of a pass over all key blocks.)
//
// Three kernels, no atomics, so the result is deterministic:
//  1. prep: D_i = dO_i . O_i and lse_i * log2(e) per query row;
//  2. dK/dV: one workgroup of 4 waves per (b, kv head, 128-key block), 32
//     keys per wave.  Each wave keeps its K and V rows in registers as
//     matrix-core operands and its dK^T, dV^T accumulators in registers
//     (one wave per SIMD: that state alone takes 192 of its 512 registers);
//     the Q and dO tiles (128 rows) of every query head that reads this kv
//     head stream through LDS, double buffered.  Per 32-query block:
//       S = Q K^T, dP = dO V^T        (lane = key, registers = queries)
//       P, dS elementwise
//       dV^T += dO^T P,  dK^T += Q^T dS   (P and dS feed the matrix core
//                                          straight from the registers; the
//                                          Q^T, dO^T operands come from the
//                                          LDS transpose read)
//     The four blocks of a tile run as a three-stage software pipeline:
//     the products of S, dP for block n and of dV, dK for block n-2 are
//     issued together, with the elementwise work of block n-1 spread over
//     them, and every LDS operand is read two products ahead.  With a single
//     wave per SIMD nothing else hides the vector work or the LDS latency;
//  3. dQ: one workgroup of 4 waves per (b, h, 128-query tile), 32 queries per
//     wave, the forward pass's layout: Q and dO rows in registers, K and V
//     tiles (64 keys) streamed through LDS, two waves per SIMD;
//       S^T = K Q^T, dP^T = V dO^T    (lane = query, registers = keys)
//       dQ^T += K^T dS^T.
// Splitting dQ from dK/dV recomputes S and dP once more (7 matrix products
// per block instead of 5) in exchange for no cross-workgroup reduction.
// Causal: workgroups take a heavy and a light block of the same head, blocks
// entirely on the masked side of the diagonal are skipped, and only blocks
// that straddle it (or the ragged tail) pay for element masks.
#include "fa_sizes.h"
#include "fa_tile.h"

#include <climits>
#include <type_traits>
#include <utility>

namespace fa {

template <typename T, int D> struct BwdCfg {
    static constexpr int KW = Mma<T>::KW;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int VEC = 16 / ES;           // elements per 16-byte chunk
    static constexpr int NT = 256;                 // threads per workgroup (4 waves)
    static constexpr int BW = 128;                 // rows a workgroup owns (keys, or queries for dQ)
    static constexpr int BT = 64;                  // rows per streamed LDS tile
    static constexpr int NB = BT / 32;             // 32-row blocks per tile
    static constexpr int CPR = D / VEC;            // 16-byte chunks per row
    static constexpr int ROWB = D * ES;            // bytes per row in LDS
    static constexpr int TILEB = BT * ROWB;        // bytes per tile
    static constexpr int NLD = BT * CPR / kWave;   // direct-to-LDS loads per tile
    static constexpr int NLD_W = NLD / 4;          // ... per wave
    static constexpr int QK_STEPS = D / (2 * KW);  // matrix steps over d
    static constexpr int PV_STEPS = 32 / (2 * KW); // matrix steps per 32-row block
    static constexpr int DB = D / 32;              // 32-row blocks of a d-by-32 accumulator
    static_assert(ES == 2, "16-bit element types only");
    static_assert(NLD % 4 == 0 && D % 32 == 0, "tile shapes");
};

// Per-lane byte offsets of the direct-to-LDS loads that fill one BT-row tile
// (the same for every tile).  Load I of the tile fills LDS bytes
// [I*1024, I*1024 + 1024); lane l writes chunk position p = I*64 + l, i.e.
// LDS row p / CPR, position p % CPR, which holds global chunk
// (p % CPR) ^ swz(row).  Rows at or past the end of the sequence re-read row
// N-1, so every LDS row holds finite values.
template <class C, int ROWS> struct TileLoader {
    static constexpr int NLD_W = ROWS * C::CPR / kWave / 4;  // 1 KiB loads per wave
    static_assert(ROWS * C::CPR % (4 * kWave) == 0, "tile loads must split evenly over the waves");
    int row[NLD_W], off[NLD_W];
    __device__ __forceinline__ void init(int wave, int lane)
    {
#pragma unroll
        for (int i = 0; i < NLD_W; ++i) {
            const int p = (wave * NLD_W + i) * kWave + lane;
            row[i] = p / C::CPR;
            off[i] = (row[i] * (C::ROWB / C::ES) + ((p % C::CPR) ^ swz<C::CPR, C::ES>(row[i])) * C::VEC) * C::ES;
        }
    }
    // tile of rows [r0, r0 + ROWS) of the buffer r into LDS at dst
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, char *dst, int wave, int r0, int N) const
    {
        const int soff = r0 * C::ROWB;
        if (r0 + ROWS <= N) {
#pragma unroll
            for (int i = 0; i < NLD_W; ++i)
                buffer_load_lds16(r, dst + (wave * NLD_W + i) * 1024, off[i], soff);
        } else {
#pragma unroll
            for (int i = 0; i < NLD_W; ++i) {
                const int over = r0 + row[i] - (N - 1);
                buffer_load_lds16(r, dst + (wave * NLD_W + i) * 1024,
                                  over > 0 ? off[i] - over * C::ROWB : off[i], soff);
            }
        }
    }
};

template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F &&f)
{
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order
template <int N, class F> __device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// byte offset of element e of row r in a swizzled tile
template <class C> __device__ __forceinline__ int tile_off(int r, int e)
{
    const int cc = (e * C::ES) / 16, o = (e * C::ES) % 16;
    return r * C::ROWB + ((cc ^ swz<C::CPR, C::ES>(r)) * 16) + o;
}

// Transpose-read sources: lane (g = lane / 16, r16 = lane % 16) points at row
// 8*hi + 4*(g/2) + r16/4 of a 16-row block, elements db*32 + 16*(g%2) +
// 4*(r16%4) .. +3.  The two reads (hi = 0, 1) give lane (col, half) the 8
// values of column db*32 + col at rows 4*half + 0..3 and 8 + 4*half + 0..3 of
// the block -- the row order of the accumulator registers.
template <class C> __device__ __forceinline__ void tr_offsets(int lane, int (&tr)[2][C::DB])
{
    const int g = lane / 16, r16 = lane % 16;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
            tr[hi][db] = tile_off<C>(8 * hi + 4 * (g / 2) + r16 / 4, db * 32 + 16 * (g % 2) + 4 * (r16 % 4));
}

template <typename frag> __device__ __forceinline__ frag tr_read(const char *blk, int o0, int o1)
{
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(blk + o0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(blk + o1));
    return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// the 8 (or KW) registers [st*KW, st*KW + KW) of x, rounded into one operand
template <typename T> __device__ __forceinline__ typename Mma<T>::frag pack_regs(const f32x16 &x, int st)
{
    constexpr int KW = Mma<T>::KW;
    float t[KW];
#pragma unroll
    for (int e = 0; e < KW; ++e) t[e] = x[st * KW + e];
    return Mma<T>::pack(t);
}

// Workgroup id with the XCD remap: consecutive ids are dispatched
// round-robin over the 8 XCDs; remap so that the workgroups resident on one
// XCD (sharing its L2) work on the same head.
__device__ __forceinline__ int xcd_remapped_id()
{
    int wid = blockIdx.x;
    const int G = gridDim.x;
    if (G % 8 == 0) wid = (wid % 8) * (G / 8) + wid / 8;
    return wid;
}

// ---------------------------------------------------------------------------
// 1. prep: D_i = dO_i . O_i (fp32) and lse_i * log2(e), one row per D/8 lanes
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(const float *__restrict__ O,
                                                          const T *__restrict__ dO,
                                                          const float *__restrict__ LSE,
                                                          float *__restrict__ L2,
                                                          float *__restrict__ Dl, int64_t rows)
{
    constexpr int LPR = D / 8;   // lanes per row
    constexpr int RPB = 256 / LPR;
    typedef typename Mma<T>::frag frag;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const f32x4 a = *(const f32x4 *)(O + row * D + part * 8);
        const f32x4 b = *(const f32x4 *)(O + row * D + part * 8 + 4);
        const frag x = *(const frag *)(dO + row * D + part * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_fmaf((float)x[e], a[e], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_fmaf((float)x[4 + e], b[e], acc);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m);
    if (row < rows && part == 0) {
        Dl[row] = acc;
        L2[row] = LSE[row] * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// 2. dK, dV
// ---------------------------------------------------------------------------
// Schedule of one full tile of the dK/dV kernel: NB 32-query blocks and NP
// matrix pairs per block for S/dP and again for dV/dK.  Step s issues the
// S/dP pairs of block s (s < NB) and the dV/dK pairs of block s-2 (s >= 2),
// alternating when both are present; the elementwise work of block s-1
// (1 <= s <= NB) is spread over the pairs of step s, so that every matrix
// instruction has a share of it to hide.
template <int NB, int NP> struct DkdvSched {
    static constexpr int NSTEP = NB + 2;
    static constexpr int NOPS = 2 * NB * NP;
    static constexpr int nsdp(int s) { return s < NB ? NP : 0; }
    static constexpr int ndvdk(int s) { return s >= 2 && s < NB + 2 ? NP : 0; }
    static constexpr int nops(int s) { return nsdp(s) + ndvdk(s); }
    static constexpr int first(int s)
    {
        int g = 0;
        for (int i = 0; i < s; ++i) g += nops(i);
        return g;
    }
    static constexpr int step_of(int g)
    {
        int s = 0;
        while (g >= nops(s)) {
            g -= nops(s);
            ++s;
        }
        return s;
    }
    static constexpr bool both(int s) { return nsdp(s) > 0 && ndvdk(s) > 0; }
    // 0: S/dP pair, 1: dV/dK pair
    static constexpr int kind(int g)
    {
        const int s = step_of(g), k = g - first(s);
        return both(s) ? (k & 1) : (nsdp(s) ? 0 : 1);
    }
    static constexpr int block(int g) { return kind(g) == 0 ? step_of(g) : step_of(g) - 2; }
    static constexpr int pair(int g)
    {
        const int s = step_of(g), k = g - first(s);
        return both(s) ? k / 2 : k;
    }
    // element e (0..15) of block b: with the pair at this index (step b+1,
    // starting one pair in, so that the scores of block b have landed)
    static constexpr int elem_op(int b, int e) { return first(b + 1) + 1 + e * (nops(b + 1) - 1) / 16; }
    // statistics of 4-row group r of block b are read two pairs ahead
    static constexpr int stats_op(int b, int r)
    {
        const int g = elem_op(b, 4 * r) - 2;
        return g < 0 ? 0 : g;
    }
};

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkdv_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                        const T *__restrict__ dO, const float *__restrict__ L2,
                        const float *__restrict__ Dl, float *__restrict__ dK,
                        float *__restrict__ dV, int N, int num_ktiles, float scale, int H, int group)
{
    using C = BwdCfg<T, D>;
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int KW = C::KW;
    constexpr int BQ = 128;                      // query rows per streamed tile
    constexpr int NBQ = BQ / 32;                 // 32-query blocks per tile
    constexpr int QTB = BQ * C::ROWB;            // bytes of a Q or dO tile
    constexpr int STATB = BQ * 4;                // lse2 or D of one tile
    constexpr int NP = C::QK_STEPS;              // matrix pairs per block, S/dP and dV/dK alike
    static_assert(C::PV_STEPS * C::DB == NP, "S/dP and dV/dK take the same number of pairs");
    using S = DkdvSched<NBQ, NP>;
    // LDS, two stages: the Q tiles of both in [0, 2 QTB), the dO tiles in
    // [OBASE, OBASE + 2 QTB), then lse2 and D of stage s at SBASE + 2 STATB s.
    // A ds_read reaches 64 KiB past its address register with the offset
    // field; regions beyond that (the dO tiles at d = 128 in 16-bit types, the
    // statistics) are read from copies of the per-lane offsets that carry the
    // region's base (OREG, SREG) from setup, kept opaque to the compiler, which
    // would otherwise fold the base back into each read and add it there.
    constexpr int OBASE = 2 * QTB, SBASE = 4 * QTB;
    constexpr int OREG = OBASE + 2 * QTB > 65536 ? OBASE : 0;
    constexpr int SREG = SBASE;
    static_assert(2 * QTB <= 65536 && 2 * QTB - OREG <= 65536 && 4 * STATB <= 65536, "regions within reach");
    __shared__ __attribute__((aligned(1024))) char smem[SBASE + 4 * STATB];
    poison_lds(smem, sizeof(smem));

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col = lane % 32;  // key of this lane within the wave's 32
    const int h = lane / 32;    // lane half

    // Causal: workgroup p takes the key blocks p (heavy: every query from p
    // on sees it) and nkt-1-p (light).
    const int wid = xcd_remapped_id();
    const int wg_per_head = CAUSAL ? (num_ktiles + 1) / 2 : num_ktiles;
    const int bkv = wid / wg_per_head;  // b * Hkv + kv head
    const int pi = wid % wg_per_head;
    const int Hkv = H / group;
    const int b = bkv / Hkv, g = bkv % Hkv;
    const int64_t kv_head = (int64_t)bkv * N * D;
    const int head_bytes = N * C::ROWB;

    TileLoader<C, BQ> ld;
    ld.init(wave, lane);
    int q_rd[C::QK_STEPS];  // row-fragment read: row col, elements st*2KW + h*KW
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) q_rd[st] = tile_off<C>(col, st * 2 * KW + h * KW);
    int tr[2][C::DB];
    tr_offsets<C>(lane, tr);
    // the same offsets for the dO tiles (+ OREG), and the statistics' (+ SREG)
    int o_rd[C::QK_STEPS], tro[2][C::DB];
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) o_rd[st] = q_rd[st] + OREG;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) tro[hi][db] = tr[hi][db] + OREG;
    if constexpr (OREG != 0) {
#pragma unroll
        for (int st = 0; st < C::QK_STEPS; ++st) asm volatile("" : "+v"(o_rd[st]));
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) asm volatile("" : "+v"(tro[hi][db]));
    }
    int s_rd = 16 * h + SREG;  // lse2 / D: rows 8i + 4h .. +3 of a 32-row block
    asm volatile("" : "+v"(s_rd));

    const float c = fmaxf(scale * kLog2e, 1e-30f);
    const int nqt = (N + BQ - 1) / BQ;

    for (int item = 0; item < (CAUSAL ? 2 : 1); ++item) {
        const int kt = CAUSAL ? (item == 0 ? pi : num_ktiles - 1 - pi) : pi;
        if (CAUSAL && item == 1 && kt == pi) break;  // odd count: middle block alone
        const int kw0 = kt * C::BW + wave * 32;      // first key of this wave
        const int key = kw0 + col;

        // K and V rows of this lane's key as B operands: d = st*2KW + h*KW ..
        frag kf[C::QK_STEPS], vf[C::QK_STEPS];
#pragma unroll
        for (int st = 0; st < C::QK_STEPS; ++st) {
            if (key < N) {
                kf[st] = *(const frag *)(K + kv_head + (int64_t)key * D + st * 2 * KW + h * KW);
                vf[st] = *(const frag *)(V + kv_head + (int64_t)key * D + st * 2 * KW + h * KW);
            } else {
                kf[st] = frag{};
                vf[st] = frag{};
            }
        }
        f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            dk[db] = f32x16{};
            dv[db] = f32x16{};
        }
        // query tiles that can see a key of this block
        const int qt0 = CAUSAL ? (kt * C::BW) / BQ : 0;

        for (int t = 0; t < group; ++t) {
            const int64_t bh = (int64_t)b * H + (int64_t)g * group + t;
            const __amdgpu_buffer_rsrc_t qrs =
                __builtin_amdgcn_make_buffer_rsrc((void *)(Q + bh * N * D), 0, head_bytes, kBufferFlags);
            const __amdgpu_buffer_rsrc_t ors =
                __builtin_amdgcn_make_buffer_rsrc((void *)(dO + bh * N * D), 0, head_bytes, kBufferFlags);
            const __amdgpu_buffer_rsrc_t lrs =
                __builtin_amdgcn_make_buffer_rsrc((void *)(L2 + bh * N), 0, N * 4, kBufferFlags);
            const __amdgpu_buffer_rsrc_t drs =
                __builtin_amdgcn_make_buffer_rsrc((void *)(Dl + bh * N), 0, N * 4, kBufferFlags);

            auto load_tile = [&](int j, int buf) __attribute__((always_inline)) {
                ld.load(qrs, smem + buf * QTB, wave, j * BQ, N);
                ld.load(ors, smem + OBASE + buf * QTB, wave, j * BQ, N);
                // lse2 (waves 0, 1) and D (waves 2, 3) of rows j*BQ + 64*(wave%2) + lane;
                // rows past the end re-read N-1
                const int r = 64 * (wave % 2) + lane;
                buffer_load_lds4(wave < 2 ? lrs : drs,
                                 smem + SBASE + buf * 2 * STATB + (wave / 2) * STATB + 64 * 4 * (wave % 2),
                                 min(j * BQ + r, N - 1) * 4, 0);
            };

            // One 32-query block with masks or a causal skip (diagonal and
            // ragged tiles): S/dP, then P/dS, then dV/dK, in sequence.
            // Qb: the block's Q rows; Ob, Lb, Db: its dO rows, lse2 and D less
            // OREG, SREG, SREG (carried by o_rd / tro and s_rd).
            auto masked_block = [&](const char *Qb, const char *Ob, const char *Lb, const char *Db,
                                    int qf0) __attribute__((always_inline)) {
                if (CAUSAL && qf0 + 31 < kw0) return;  // every query before every key
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int st = 0; st < C::QK_STEPS; ++st) {
                    s = M::mma(*(const frag *)(Qb + q_rd[st]), kf[st], s);
                    dp = M::mma(*(const frag *)(Ob + o_rd[st]), vf[st], dp);
                }
                f32x4 l4[4], d4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    l4[i] = *(const f32x4 *)(Lb + 32 * i + s_rd);
                    d4[i] = *(const f32x4 *)(Db + 32 * i + s_rd);
                }
                const int lo = CAUSAL ? key - qf0 - 4 * h : INT_MIN;  // visible iff acc_row(r,0) >= lo
                const int hi = N - qf0 - 4 * h;                       // ... and acc_row(r,0) < hi
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2_hw(__builtin_fmaf(s[r], c, -l4[r / 4][r % 4]));
                    const int ar = acc_row(r, 0);
                    if (ar < lo || ar >= hi) p = 0.f;
                    s[r] = p;
                    dp[r] = p * (dp[r] - d4[r / 4][r % 4]);
                }
#pragma unroll
                for (int st = 0; st < C::PV_STEPS; ++st) {
                    float pv[KW], sv[KW];
#pragma unroll
                    for (int e = 0; e < KW; ++e) {
                        pv[e] = s[st * KW + e];
                        sv[e] = dp[st * KW + e];
                    }
                    const frag pb = M::pack(pv);
                    const frag sb = M::pack(sv);
                    const char *oblk = Ob + 16 * st * C::ROWB;
                    const char *qblk = Qb + 16 * st * C::ROWB;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        dv[db] = M::mma(tr_read<frag>(oblk, tro[0][db], tro[1][db]), pb, dv[db]);
                        dk[db] = M::mma(tr_read<frag>(qblk, tr[0][db], tr[1][db]), sb, dk[db]);
                    }
                }
            };

            // A tile every query of which sees every key of this wave: the
            // schedule above, every LDS operand read two pairs ahead of its
            // use (a ring of three register slots), fenced so that the
            // compiler keeps the order.
            auto full_tile = [&](const char *Qs, const char *Os, const char *Ls, const char *Ds)
                __attribute__((always_inline)) {
                f32x16 sa[NBQ], da[NBQ];                        // S then P; dP then dS
                frag pp[NBQ][C::PV_STEPS], sp[NBQ][C::PV_STEPS];  // P, dS packed for the matrix core
                frag opr[3][2];
                f32x4 sl[4], sd[4];                             // lse2, D of 4-row groups
                auto rd_op = [&](auto gc) __attribute__((always_inline)) {
                    constexpr int G = decltype(gc)::value;
                    if constexpr (G < S::NOPS) {
                        constexpr int kd = S::kind(G), blk = S::block(G), pr = S::pair(G), slot = G % 3;
                        const char *Qb = Qs + blk * 32 * C::ROWB, *Ob = Os + blk * 32 * C::ROWB;
                        if constexpr (kd == 0) {
                            opr[slot][0] = *(const frag *)(Qb + q_rd[pr]);
                            opr[slot][1] = *(const frag *)(Ob + o_rd[pr]);
                        } else {
                            constexpr int st = pr / C::DB, db = pr % C::DB;
                            opr[slot][0] = tr_read<frag>(Ob + 16 * st * C::ROWB, tro[0][db], tro[1][db]);
                            opr[slot][1] = tr_read<frag>(Qb + 16 * st * C::ROWB, tr[0][db], tr[1][db]);
                        }
                    }
                };
                auto mma_op = [&](auto gc) __attribute__((always_inline)) {
                    constexpr int G = decltype(gc)::value;
                    constexpr int kd = S::kind(G), blk = S::block(G), pr = S::pair(G), slot = G % 3;
                    if constexpr (kd == 0) {
                        sa[blk] = M::mma(opr[slot][0], kf[pr], pr == 0 ? f32x16{} : sa[blk]);
                        da[blk] = M::mma(opr[slot][1], vf[pr], pr == 0 ? f32x16{} : da[blk]);
                    } else {
                        constexpr int st = pr / C::DB, db = pr % C::DB;
                        dv[db] = M::mma(opr[slot][0], pp[blk][st], dv[db]);
                        dk[db] = M::mma(opr[slot][1], sp[blk][st], dk[db]);
                    }
                };
                auto extras = [&](auto gc) __attribute__((always_inline)) {
                    constexpr int G = decltype(gc)::value;
                    static_for<NBQ>([&](auto bc) __attribute__((always_inline)) {
                        constexpr int B_ = decltype(bc)::value;
                        static_for<4>([&](auto rc) __attribute__((always_inline)) {
                            constexpr int R = decltype(rc)::value;
                            if constexpr (S::stats_op(B_, R) == G) {
                                sl[R] = *(const f32x4 *)(Ls + (B_ * 32 + 8 * R) * 4 + s_rd);
                                sd[R] = *(const f32x4 *)(Ds + (B_ * 32 + 8 * R) * 4 + s_rd);
                            }
                        });
                    });
                };
                auto elems = [&](auto gc) __attribute__((always_inline)) {
                    constexpr int G = decltype(gc)::value;
                    static_for<NBQ>([&](auto bc) __attribute__((always_inline)) {
                        constexpr int B_ = decltype(bc)::value;
                        static_for<16>([&](auto ec) __attribute__((always_inline)) {
                            constexpr int E = decltype(ec)::value;
                            if constexpr (S::elem_op(B_, E) == G) {
                                const float p = exp2_hw(__builtin_fmaf(sa[B_][E], c, -sl[E / 4][E % 4]));
                                sa[B_][E] = p;
                                da[B_][E] = p * (da[B_][E] - sd[E / 4][E % 4]);
                                if constexpr (E % KW == KW - 1) {
                                    pp[B_][E / KW] = pack_regs<T>(sa[B_], E / KW);
                                    sp[B_][E / KW] = pack_regs<T>(da[B_], E / KW);
                                }
                            }
                        });
                    });
                };
                rd_op(std::integral_constant<int, 0>{});
                rd_op(std::integral_constant<int, 1>{});
                static_for<S::NOPS>([&](auto gc) __attribute__((always_inline)) {
                    constexpr int G = decltype(gc)::value;
                    rd_op(std::integral_constant<int, G + 2>{});
                    extras(gc);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_op(gc);
                    elems(gc);
                    __builtin_amdgcn_sched_barrier(0);
                });
            };

            // The tiles that need masks are uniform over the workgroup: the
            // causal diagonal tile first (queries [128 kt, 128 kt + 128) against
            // keys [128 kt, 128 kt + 128)) and the ragged last tile.  They run
            // outside the loop of full tiles.
            auto tile_full = [&](int j, auto stage_c) __attribute__((always_inline)) {
                constexpr int STAGE = decltype(stage_c)::value;
                if (j + 1 < nqt) load_tile(j + 1, STAGE ^ 1);
                const char *Qs = smem + STAGE * QTB;
                const char *Os = smem + OBASE - OREG + STAGE * QTB;
                const char *Ls = smem + SBASE - SREG + STAGE * 2 * STATB;
                full_tile(Qs, Os, Ls, Ls + STATB);
                // this wave's loads of the next tile have landed, and after the
                // barrier every wave's have, and nobody reads the current buffer
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            };
            auto tile_masked = [&](int j, int stage) __attribute__((always_inline)) {
                if (j + 1 < nqt) load_tile(j + 1, stage ^ 1);
                const char *Qs = smem + stage * QTB;
                const char *Os = smem + OBASE - OREG + stage * QTB;
                const char *Ls = smem + SBASE - SREG + stage * 2 * STATB;
                const char *Ds = Ls + STATB;
                for (int qb = 0; qb < NBQ; ++qb)
                    masked_block(Qs + qb * 32 * C::ROWB, Os + qb * 32 * C::ROWB, Ls + qb * 32 * 4,
                                 Ds + qb * 32 * 4, j * BQ + qb * 32);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            };

            load_tile(qt0, 0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            int j = qt0, stage = 0;
            if (CAUSAL) {
                tile_masked(j, 0);
                ++j;
                stage = 1;
            }
            const int jfull = (N % BQ) ? nqt - 1 : nqt;  // tiles [j, jfull) are full
            if (stage == 1 && j < jfull) {
                tile_full(j, std::integral_constant<int, 1>{});
                ++j;
                stage = 0;
            }
            for (; j + 1 < jfull; j += 2) {
                tile_full(j, std::integral_constant<int, 0>{});
                tile_full(j + 1, std::integral_constant<int, 1>{});
            }
            if (j < jfull) {
                tile_full(j, std::integral_constant<int, 0>{});
                ++j;
                stage = 1;
            }
            if (j < nqt) tile_masked(j, stage);
        }

        // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane (col, h) holds key
        // kw0 + col, elements db*32 + 8*(r/4) + 4*h + r%4.
        if (key < N) {
            float *dkr = dK + kv_head + (int64_t)key * D;
            float *dvr = dV + kv_head + (int64_t)key * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int e = db * 32 + 8 * r4 + 4 * h;
                    *(f32x4 *)(dkr + e) = f32x4{dk[db][4 * r4 + 0] * scale, dk[db][4 * r4 + 1] * scale,
                                                dk[db][4 * r4 + 2] * scale, dk[db][4 * r4 + 3] * scale};
                    *(f32x4 *)(dvr + e) = f32x4{dv[db][4 * r4 + 0], dv[db][4 * r4 + 1],
                                                dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
                }
        }
    }
}

// ---------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                      const T *__restrict__ dO, const float *__restrict__ L2,
                      const float *__restrict__ Dl, float *__restrict__ dQ, int N, int num_qtiles,
                      float scale, int H, int group)
{
    using C = BwdCfg<T, D>;
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int KW = C::KW;
    constexpr int NKB = C::NB;                 // 32-key blocks per K/V tile
    constexpr int STAGEB = 2 * C::TILEB;       // K + V
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGEB];
    poison_lds(smem, sizeof(smem));

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col = lane % 32;  // query row of this lane within the wave's 32
    const int h = lane / 32;

    const int wid = xcd_remapped_id();
    const int wg_per_head = CAUSAL ? (num_qtiles + 1) / 2 : num_qtiles;
    const int bh = wid / wg_per_head;
    const int pi = wid % wg_per_head;
    const int64_t head = (int64_t)bh * N * D;
    const int64_t kv_head = ((int64_t)(bh / H) * (H / group) + (bh % H) / group) * N * D;
    const int head_bytes = N * C::ROWB;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)(K + kv_head), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(V + kv_head), 0, head_bytes, kBufferFlags);

    TileLoader<C, C::BT> ld;
    ld.init(wave, lane);
    int k_rd[C::QK_STEPS];
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) k_rd[st] = tile_off<C>(col, st * 2 * KW + h * KW);
    int tr[2][C::DB];
    tr_offsets<C>(lane, tr);
    const float c = fmaxf(scale * kLog2e, 1e-30f);

    auto load_tile = [&](int j, int buf) __attribute__((always_inline)) {
        char *kd = smem + buf * STAGEB;
        ld.load(krs, kd, wave, j * C::BT, N);
        ld.load(vrs, kd + C::TILEB, wave, j * C::BT, N);
    };

    for (int item = 0; item < (CAUSAL ? 2 : 1); ++item) {
        const int qt = CAUSAL ? (item == 0 ? num_qtiles - 1 - pi : pi) : pi;
        if (CAUSAL && item == 1 && qt == num_qtiles - 1 - pi) break;
        const int q0 = qt * C::BW;
        const int wq_lo = q0 + wave * 32, wq_hi = wq_lo + 31;
        const int qrow = wq_lo + col;

        frag qf[C::QK_STEPS], of[C::QK_STEPS];
#pragma unroll
        for (int st = 0; st < C::QK_STEPS; ++st) {
            if (qrow < N) {
                qf[st] = *(const frag *)(Q + head + (int64_t)qrow * D + st * 2 * KW + h * KW);
                of[st] = *(const frag *)(dO + head + (int64_t)qrow * D + st * 2 * KW + h * KW);
            } else {
                qf[st] = frag{};
                of[st] = frag{};
            }
        }
        const float l2 = qrow < N ? L2[(int64_t)bh * N + qrow] : 0.f;
        const float dd = qrow < N ? Dl[(int64_t)bh * N + qrow] : 0.f;
        f32x16 acc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

        const int kend = CAUSAL ? min(N, q0 + C::BW) : N;
        const int ntiles = (kend + C::BT - 1) / C::BT;
        const int nt_w = CAUSAL ? min(ntiles, wq_hi / C::BT + 1) : ntiles;

        // X^T = Y B^T for the BT rows of the tile at Ys: lane = query,
        // registers = rows acc_row(r, h) of each 32-row block
        auto rows_dot = [&](const char *Ys, const frag (&bf)[C::QK_STEPS], f32x16 (&x)[NKB])
            __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) x[kb] = f32x16{};
#pragma unroll
            for (int st = 0; st < C::QK_STEPS; ++st)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    x[kb] = M::mma(*(const frag *)(Ys + kb * 32 * C::ROWB + k_rd[st]), bf[st], x[kb]);
        };

        auto tile = [&](int j, auto stage_c) __attribute__((always_inline)) {
            constexpr int STAGE = decltype(stage_c)::value;
            if (j + 1 < ntiles) load_tile(j + 1, STAGE ^ 1);
            const int k0 = j * C::BT;
            const char *Ks = smem + STAGE * STAGEB;
            const char *Vs = Ks + C::TILEB;
            f32x16 s[NKB], dp[NKB];
            __builtin_amdgcn_s_setprio(1);
            rows_dot(Ks, qf, s);
            rows_dot(Vs, of, dp);
            __builtin_amdgcn_s_setprio(0);
            const bool need_mask = (k0 + C::BT > N) || (CAUSAL && k0 + C::BT - 1 > wq_lo);
            // key k0 + kb*32 + acc_row(r, h) is visible iff acc_row(r, 0) <= lim
            const int last = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int lim = last - k0 - kb * 32 - 4 * h;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2_hw(__builtin_fmaf(s[kb][r], c, -l2));
                    if (need_mask && acc_row(r, 0) > lim) p = 0.f;
                    dp[kb][r] = p * (dp[kb][r] - dd);
                }
            }
            // dQ^T += K^T dS^T, keys in the accumulator's register order
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int st = 0; st < C::PV_STEPS; ++st) {
                    float sv[KW];
#pragma unroll
                    for (int e = 0; e < KW; ++e) sv[e] = dp[kb][st * KW + e];
                    const frag sb = M::pack(sv);
                    const char *kblk = Ks + (kb * 32 + 16 * st) * C::ROWB;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
                        acc[db] = M::mma(tr_read<frag>(kblk, tr[0][db], tr[1][db]), sb, acc[db]);
                }
            __builtin_amdgcn_s_setprio(0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };

        load_tile(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int j = 0;
        for (; j + 1 < nt_w; j += 2) {
            tile(j, std::integral_constant<int, 0>{});
            tile(j + 1, std::integral_constant<int, 1>{});
        }
        if (j < nt_w) {
            tile(j, std::integral_constant<int, 0>{});
            ++j;
        }
        // tiles this wave's rows cannot see are still loaded for the others
        for (; j < ntiles; ++j) {
            if (j + 1 < ntiles) load_tile(j + 1, (j + 1) & 1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        if (qrow < N) {
            float *row = dQ + head + (int64_t)qrow * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int e = db * 32 + 8 * r4 + 4 * h;
                    *(f32x4 *)(row + e) = f32x4{acc[db][4 * r4 + 0] * scale, acc[db][4 * r4 + 1] * scale,
                                                acc[db][4 * r4 + 2] * scale, acc[db][4 * r4 + 3] * scale};
                }
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// (bwd_workspace_bytes, the workspace size, is in fa_sizes.h)

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd(const void *q, const void *k, const void *v, const float *o,
                             const float *lse, const void *dout, float *dq, float *dk, float *dv,
                             int B, int H, int Hkv, int N, float scale, void *workspace,
                             hipStream_t stream)
{
    using C = BwdCfg<T, D>;
    const int64_t rows = (int64_t)B * H * N;
    float *L2 = (float *)workspace;
    float *Dl = L2 + rows;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((fa_bwd_prep_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       stream, o, (const T *)dout, lse, L2, Dl, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nt = (N + C::BW - 1) / C::BW;
    const int per_head = CAUSAL ? (nt + 1) / 2 : nt;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, D, CAUSAL>), dim3((unsigned)((int64_t)B * Hkv * per_head)),
                       dim3(C::NT), 0, stream, (const T *)q, (const T *)k, (const T *)v,
                       (const T *)dout, L2, Dl, dk, dv, N, nt, scale, H, H / Hkv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, CAUSAL>), dim3((unsigned)((int64_t)B * H * per_head)),
                       dim3(C::NT), 0, stream, (const T *)q, (const T *)k, (const T *)v,
                       (const T *)dout, L2, Dl, dq, N, nt, scale, H, H / Hkv);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_bwd_c(const void *q, const void *k, const void *v, const float *o,
                               const float *lse, const void *dout, float *dq, float *dk, float *dv,
                               int B, int H, int Hkv, int N, float scale, int causal, void *ws,
                               hipStream_t stream)
{
    return causal ? launch_bwd<T, D, true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, scale, ws, stream)
                  : launch_bwd<T, D, false>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, scale, ws, stream);
}

// Dispatch to the instantiation for (dtype, d, causal).  Arguments were
// validated by the caller: dtype 1/2 = bf16/fp16, d in {64, 128}, Hkv
// divides H, workspace holds bwd_workspace_bytes(B, H, N).
hipError_t bwd_dispatch(const void *q, const void *k, const void *v, const float *o,
                        const float *lse, const void *dout, float *dq, float *dk, float *dv, int B,
                        int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                        void *workspace, hipStream_t stream)
{
    if (dtype == 1)
        return d == 64 ? launch_bwd_c<__bf16, 64>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, scale, causal, workspace, stream)
                       : launch_bwd_c<__bf16, 128>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, scale, causal, workspace, stream);
    return d == 64 ? launch_bwd_c<_Float16, 64>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, scale, causal, workspace, stream)
                   : launch_bwd_c<_Float16, 128>(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, scale, causal, workspace, stream);
}

}  // namespace fa
