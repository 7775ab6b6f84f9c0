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
//     matrix-core operands and its dK^T, dV^T accumulators in registers; the
//     Q and dO tiles (64 rows) of every query head that reads this kv head
//     stream through LDS, double buffered.  Per 32-query block:
//       S = Q K^T, dP = dO V^T        (lane = key, registers = queries)
//       P, dS elementwise
//       dV^T += dO^T P,  dK^T += Q^T dS   (P and dS feed the matrix core
//                                          straight from the registers; the
//                                          Q^T, dO^T operands come from the
//                                          LDS transpose read)
//  3. dQ: one workgroup of 4 waves per (b, h, 128-query tile), 32 queries per
//     wave, the forward pass's layout: Q and dO rows in registers, K and V
//     tiles (64 keys) streamed through LDS;
//       S^T = K Q^T, dP^T = V dO^T    (lane = query, registers = keys)
//       dQ^T += K^T dS^T.
// Splitting dQ from dK/dV recomputes S and dP once more (7 matrix products
// per block instead of 5) in exchange for no cross-workgroup reduction.
// Causal: workgroups take a heavy and a light block of the same head, blocks
// entirely on the masked side of the diagonal are skipped, and only blocks
// that straddle it (or the ragged tail) pay for element masks.
#include "fa_tile.h"

#include <climits>
#include <type_traits>

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
template <class C> struct TileLoader {
    int row[C::NLD_W], off[C::NLD_W];
    __device__ __forceinline__ void init(int wave, int lane)
    {
#pragma unroll
        for (int i = 0; i < C::NLD_W; ++i) {
            const int p = (wave * C::NLD_W + i) * kWave + lane;
            row[i] = p / C::CPR;
            off[i] = (row[i] * (C::ROWB / C::ES) + ((p % C::CPR) ^ swz<C::CPR, C::ES>(row[i])) * C::VEC) * C::ES;
        }
    }
    // tile of rows [r0, r0 + BT) of the buffer r into LDS at dst
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, char *dst, int wave, int r0, int N) const
    {
        const int soff = r0 * C::ROWB;
        if (r0 + C::BT <= N) {
#pragma unroll
            for (int i = 0; i < C::NLD_W; ++i)
                buffer_load_lds16(r, dst + (wave * C::NLD_W + i) * 1024, off[i], soff);
        } else {
#pragma unroll
            for (int i = 0; i < C::NLD_W; ++i) {
                const int over = r0 + row[i] - (N - 1);
                buffer_load_lds16(r, dst + (wave * C::NLD_W + i) * 1024,
                                  over > 0 ? off[i] - over * C::ROWB : off[i], soff);
            }
        }
    }
};

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
    constexpr int STATB = C::BT * 4;                  // lse2 or D of one tile
    constexpr int STAGEB = 2 * C::TILEB + 2 * STATB;  // Q, dO, lse2, D
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGEB];

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

    TileLoader<C> ld;
    ld.init(wave, lane);
    int q_rd[C::QK_STEPS];  // row-fragment read: row col, elements st*2KW + h*KW
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) q_rd[st] = tile_off<C>(col, st * 2 * KW + h * KW);
    int tr[2][C::DB];
    tr_offsets<C>(lane, tr);

    const float c = fmaxf(scale * kLog2e, 1e-30f);
    const int nqt = (N + C::BT - 1) / C::BT;

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
        const int qt0 = CAUSAL ? (kt * C::BW) / C::BT : 0;

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
                char *qd = smem + buf * STAGEB;
                ld.load(qrs, qd, wave, j * C::BT, N);
                ld.load(ors, qd + C::TILEB, wave, j * C::BT, N);
                // lse2 and D of rows j*BT + lane (rows past the end re-read N-1)
                if (wave < 2) {
                    const int voff = min(j * C::BT + lane, N - 1) * 4;
                    buffer_load_lds4(wave == 0 ? lrs : drs, qd + 2 * C::TILEB + wave * STATB, voff, 0);
                }
            };

            auto tile = [&](int j, auto stage_c) __attribute__((always_inline)) {
                constexpr int STAGE = decltype(stage_c)::value;
                if (j + 1 < nqt) load_tile(j + 1, STAGE ^ 1);
                const char *Qs = smem + STAGE * STAGEB;
                const char *Os = Qs + C::TILEB;
                const float *Ls = (const float *)(Qs + 2 * C::TILEB);
                const float *Ds = Ls + C::BT;
#pragma unroll
                for (int qb = 0; qb < C::NB; ++qb) {
                    const int qf0 = j * C::BT + qb * 32;  // first query of the block
                    if (CAUSAL && qf0 + 31 < kw0) continue;  // every query before every key
                    const bool need_mask = (CAUSAL && qf0 < kw0 + 31) || (qf0 + 32 > N);
                    const char *Qb = Qs + qb * 32 * C::ROWB;
                    const char *Ob = Os + qb * 32 * C::ROWB;

                    // S = Q K^T and dP = dO V^T: lane (col, h), register r
                    // holds query qf0 + acc_row(r, h), key kw0 + col.
                    f32x16 s = f32x16{}, dp = f32x16{};
                    __builtin_amdgcn_s_setprio(1);
#pragma unroll
                    for (int st = 0; st < C::QK_STEPS; ++st) {
                        s = M::mma(*(const frag *)(Qb + q_rd[st]), kf[st], s);
                        dp = M::mma(*(const frag *)(Ob + q_rd[st]), vf[st], dp);
                    }
                    __builtin_amdgcn_s_setprio(0);

                    // P = 2^(s*c - lse2), dS = P (dP - D); masked pairs (a key
                    // after the query, or a query row past the end) get 0.
                    f32x4 l4[4], d4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        l4[i] = *(const f32x4 *)(Ls + qb * 32 + 8 * i + 4 * h);
                        d4[i] = *(const f32x4 *)(Ds + qb * 32 + 8 * i + 4 * h);
                    }
                    const int lo = CAUSAL ? key - qf0 - 4 * h : INT_MIN;  // visible iff acc_row(r,0) >= lo
                    const int hi = N - qf0 - 4 * h;                       // ... and acc_row(r,0) < hi
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float p = exp2_hw(__builtin_fmaf(s[r], c, -l4[r / 4][r % 4]));
                        if (need_mask) {
                            const int ar = acc_row(r, 0);
                            if (ar < lo || ar >= hi) p = 0.f;
                        }
                        s[r] = p;
                        dp[r] = p * (dp[r] - d4[r / 4][r % 4]);
                    }

                    // dV^T += dO^T P and dK^T += Q^T dS.  Step st contracts
                    // registers [st*KW, st*KW + KW) of both lane halves: slot
                    // h*KW + e is query qf0 + acc_row(st*KW + e, h), the order
                    // the transpose read delivers.
                    __builtin_amdgcn_s_setprio(1);
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
                            dv[db] = M::mma(tr_read<frag>(oblk, tr[0][db], tr[1][db]), pb, dv[db]);
                            dk[db] = M::mma(tr_read<frag>(qblk, tr[0][db], tr[1][db]), sb, dk[db]);
                        }
                    }
                    __builtin_amdgcn_s_setprio(0);
                }
                // this wave's loads of the next tile have landed, and after the
                // barrier every wave's have, and nobody reads the current buffer
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            };

            load_tile(qt0, 0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            int j = qt0;
            for (; j + 1 < nqt; j += 2) {
                tile(j, std::integral_constant<int, 0>{});
                tile(j + 1, std::integral_constant<int, 1>{});
            }
            if (j < nqt) tile(j, std::integral_constant<int, 0>{});
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
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
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

    TileLoader<C> ld;
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
size_t bwd_workspace_bytes(int B, int H, int N)
{
    const size_t rows = (size_t)B * H * N;
    return ((2 * rows * sizeof(float)) + 255) / 256 * 256;
}

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
