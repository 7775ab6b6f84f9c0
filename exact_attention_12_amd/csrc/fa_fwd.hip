// fa_fwd.hip -- FlashAttention forward pass for gfx950.
//
// Computes O = softmax(scale * Q K^T [+ causal mask]) V for every (b, h) of
// [B, H, N, d] tensors, tile by tile with the online softmax, so the N x N
// score matrix never leaves the chip ("FlashAttention: GPU 메모리 계층을
// 활용한 어텐션 최적화 분석", youngju.dev, sections 5 and 6; "Flash
// Attention", suniverse77.github.io, Eq. (1)-(4)).
//
// Work decomposition (FlashAttention-2 order, youngju.dev sections 8.2-8.3):
//  - one workgroup of 4 waves per (b, h, 128-row query tile); the query tile
//    is split across the waves, 32 rows each, with no communication between
//    waves (split-Q);
//  - every wave keeps its Q rows in registers as matrix-core operands and
//    streams the K/V tiles (BC keys each) that all four waves share through
//    LDS, double buffered, with 16-byte global loads;
//  - S^T = K Q^T is formed on the matrix cores, so each lane owns one query
//    row and 16 keys of each 32-key block: the row max and the row sum are
//    in-lane except for one exchange between the two lane halves;
//  - the probabilities P~ = exp(S - m_new) stay in the accumulator registers
//    and feed O^T += V^T P~^T directly (the key order inside a tile is
//    permuted to match the operand layout, which a sum over keys does not
//    see); V is transposed once while it is staged into LDS;
//  - the accumulator stays unnormalised and is divided by l once at the end
//    (FlashAttention-2, youngju.dev section 8.1);
//  - causal: tiles entirely above the diagonal are never loaded; a wave skips
//    the arithmetic of tiles that are fully masked for its 32 rows; only
//    diagonal and ragged-tail tiles pay for element masks.
#include "fa_device.h"

namespace fa {

template <typename T, int D> struct FwdCfg {
    static constexpr int KW = Mma<T>::KW;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int VEC = 16 / ES;                 // elements per 16-byte vector
    static constexpr int NT = 256;                       // threads per workgroup
    static constexpr int BR = 128;                       // query rows per workgroup
    static constexpr int BC = (ES == 4) ? 32 : 64;       // keys per K/V tile
    static constexpr int NKB = BC / 32;                  // 32-key blocks per tile
    static constexpr int KLD = D + VEC;                  // K row stride in LDS (16 B pad)
    static constexpr int VLD = BC + VEC;                 // V^T row stride in LDS (16 B pad)
    static constexpr int K_ELEMS = BC * KLD;
    static constexpr int V_ELEMS = D * VLD;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;      // one LDS buffer (elements)
    static constexpr int QK_STEPS = D / (2 * KW);        // MFMA steps over d for S
    static constexpr int PV_STEPS = 32 / (2 * KW);       // MFMA steps per 32-key block for PV
    static constexpr int DB = D / 32;                    // 32-row blocks of O^T
    static constexpr int K_CHUNKS = BC * D / VEC;        // 16-byte chunks per K tile
    static constexpr int K_PER_T = K_CHUNKS / NT;
    static constexpr int V_BLOCKS = (BC / 4) * (D / VEC);  // 4-key x VEC-d blocks per V tile
    static constexpr int V_PER_T = (V_BLOCKS + NT - 1) / NT;
    static_assert(K_CHUNKS % NT == 0, "K tile must split evenly over the workgroup");
    static_assert(D % 32 == 0 && BC % 32 == 0, "tile shapes");
};

// Position of tile-relative key k inside a V^T row in LDS.  Key k of 32-key
// block kb sits in accumulator register r = 4*(kk/8) + kk%4 of lane-half
// h = (kk/4)%2 (kk = k % 32); the PV step st = r / KW consumes registers
// [st*KW, st*KW + KW) of both halves as contraction slots h*KW + r%KW.
template <int KW> __device__ __forceinline__ int vt_pos(int k)
{
    const int kb = k / 32, kk = k % 32;
    const int r = 4 * (kk / 8) + kk % 4;
    const int h = (kk / 4) % 2;
    return kb * 32 + (r / KW) * (2 * KW) + h * KW + r % KW;
}

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                   float *__restrict__ O, float *__restrict__ LSE, int N, int num_qtiles,
                   float scale)
{
    using C = FwdCfg<T, D>;
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int KW = C::KW;
    __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int col = lane % 32;  // query row of this lane within the wave's 32
    const int h = lane / 32;    // lane half

    // Workgroup -> (b*H + h, query tile).  Consecutive workgroup ids are
    // dispatched round-robin over the 8 XCDs; remap so that the workgroups
    // resident on one XCD (sharing its L2) work on the same head, and visit
    // causal tiles heaviest first.
    int wid = blockIdx.x;
    const int G = gridDim.x;
    if (G % 8 == 0) wid = (wid % 8) * (G / 8) + wid / 8;
    const int bh = wid / num_qtiles;
    const int ti = wid % num_qtiles;
    const int qt = CAUSAL ? (num_qtiles - 1 - ti) : ti;
    const int q0 = qt * C::BR;

    const int64_t head = (int64_t)bh * N * D;
    const T *Qh = Q + head;
    const T *Kh = K + head;
    const T *Vh = V + head;

    const int qrow = q0 + wave * 32 + col;
    const int wq_lo = q0 + wave * 32;  // first query row of this wave
    const int wq_hi = wq_lo + 31;      // last query row of this wave

    // Q rows of this lane as B operands: d = st*2KW + h*KW .. +KW.
    frag qf[C::QK_STEPS];
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) {
        if (qrow < N)
            qf[st] = *(const frag *)(Qh + (int64_t)qrow * D + st * 2 * KW + h * KW);
        else
            qf[st] = frag{};
    }

    const int kend = CAUSAL ? min(N, q0 + C::BR) : N;  // keys [0, kend) can be seen
    const int ntiles = (kend + C::BC - 1) / C::BC;

    // ---- staging of one K/V tile: global -> registers -> LDS -------------
    u32x4 kr[C::K_PER_T];
    u32x4 vr[C::V_PER_T][4];

    auto load_tile = [&](int j) {
        const int k0 = j * C::BC;
#pragma unroll
        for (int i = 0; i < C::K_PER_T; ++i) {
            const int ci = tid + C::NT * i;
            const int row = ci / (D / C::VEC);
            const int cc = (ci % (D / C::VEC)) * C::VEC;
            kr[i] = (k0 + row < N) ? *(const u32x4 *)(Kh + (int64_t)(k0 + row) * D + cc)
                                   : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < C::V_PER_T; ++i) {
            const int bi = tid + C::NT * i;
            const int quad = bi / (D / C::VEC);
            const int cc = (bi % (D / C::VEC)) * C::VEC;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + 4 * quad + r;
                vr[i][r] = (bi < C::V_BLOCKS && key < N)
                               ? *(const u32x4 *)(Vh + (int64_t)key * D + cc)
                               : u32x4{0, 0, 0, 0};
            }
        }
    };

    auto store_tile = [&](int buf) {
        T *Ks = smem + buf * C::STAGE;
        T *Vs = Ks + C::K_ELEMS;
#pragma unroll
        for (int i = 0; i < C::K_PER_T; ++i) {
            const int ci = tid + C::NT * i;
            const int row = ci / (D / C::VEC);
            const int cc = (ci % (D / C::VEC)) * C::VEC;
            *(u32x4 *)(Ks + row * C::KLD + cc) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < C::V_PER_T; ++i) {
            const int bi = tid + C::NT * i;
            if (bi < C::V_BLOCKS) {
                const int quad = bi / (D / C::VEC);
                const int d0 = (bi % (D / C::VEC)) * C::VEC;
                if constexpr (C::ES == 2) {
                    // 4 keys x 8 d -> 8 d-rows of 4 keys; the 4 keys stay
                    // contiguous under vt_pos<8> (it permutes whole quads).
                    const int p0 = vt_pos<KW>(4 * quad);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int sh = 16 * (e % 2);
                        const uint32_t a = (vr[i][0][e / 2] >> sh) & 0xffffu;
                        const uint32_t b = (vr[i][1][e / 2] >> sh) & 0xffffu;
                        const uint32_t c = (vr[i][2][e / 2] >> sh) & 0xffffu;
                        const uint32_t d = (vr[i][3][e / 2] >> sh) & 0xffffu;
                        *(u32x2 *)(Vs + (d0 + e) * C::VLD + p0) = u32x2{a | (b << 16), c | (d << 16)};
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int p = vt_pos<KW>(4 * quad + r);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            *(uint32_t *)(Vs + (d0 + e) * C::VLD + p) = vr[i][r][e];
                    }
                }
            }
        }
    };

    // ---- running state (per lane: one query row, partial over its keys) --
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY;   // running max of raw scores q.k
    float mc_run = -INFINITY;  // m_run * c
    float l_run = 0.f;         // partial row sum over this lane's keys
    const float c = scale * kLog2e;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        if (j + 1 < ntiles) load_tile(j + 1);

        const int k0 = j * C::BC;
        const bool active = !CAUSAL || k0 <= wq_hi;
        if (active) {
            const T *Ks = smem + (j & 1) * C::STAGE;
            const T *Vs = Ks + C::K_ELEMS;

            // S^T = K Q^T for the BC keys of the tile (raw dot products).
            f32x16 s[C::NKB];
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
            for (int st = 0; st < C::QK_STEPS; ++st) {
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb) {
                    const frag a = *(const frag *)(Ks + (kb * 32 + col) * C::KLD + st * 2 * KW + h * KW);
                    s[kb] = M::mma(a, qf[st], s[kb]);
                }
            }

            // Masks: keys >= N (ragged tail) and, causal, keys > query row.
            const bool need_mask = (k0 + C::BC > N) || (CAUSAL && k0 + C::BC - 1 > wq_lo);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + kb * 32 + acc_row(r, h);
                        if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
                    }
            }

            // Row max over the tile: in-lane, then across the two halves.
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, swap_halves(mx));

            const float m_new = fmaxf(m_run, mx);
            const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
            const float mc_new = m_safe * c;
            const float alpha = exp2_hw(mc_run - mc_new);  // e^(scale*(m_old - m_new))

            // P~ = exp(scale*(s - m_new)) = 2^(s*c - m_new*c)
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2_hw(__builtin_fmaf(s[kb][r], c, -mc_new));
                    if (need_mask && s[kb][r] == -INFINITY) p = 0.f;
                    s[kb][r] = p;
                    rs += p;
                }
            l_run = alpha * l_run + rs;
            m_run = m_new;
            mc_run = mc_new;

#pragma unroll
            for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;

            // O^T += V^T P~^T
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                for (int st = 0; st < C::PV_STEPS; ++st) {
                    float pv[KW];
#pragma unroll
                    for (int e = 0; e < KW; ++e) pv[e] = s[kb][st * KW + e];
                    const frag b = M::pack(pv);
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const frag a = *(const frag *)(Vs + (db * 32 + col) * C::VLD + kb * 32 +
                                                       st * 2 * KW + h * KW);
                        acc[db] = M::mma(a, b, acc[db]);
                    }
                }
            }
        }

        if (j + 1 < ntiles) store_tile((j + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, lse = scale*m + ln l ----------------------
    const float l_tot = l_run + swap_halves(l_run);
    const float inv = 1.f / l_tot;
    if (qrow < N) {
        float *orow = O + head + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * h;
                *(f32x4 *)(orow + d) = f32x4{acc[db][4 * r4 + 0] * inv, acc[db][4 * r4 + 1] * inv,
                                            acc[db][4 * r4 + 2] * inv, acc[db][4 * r4 + 3] * inv};
            }
        if (h == 0) LSE[(int64_t)bh * N + qrow] = scale * m_run + log2_hw(l_tot) * kLn2;
    }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd(const void *q, const void *k, const void *v, float *o, float *lse,
                             int B, int H, int N, float scale, hipStream_t stream)
{
    using C = FwdCfg<T, D>;
    const int nqt = (N + C::BR - 1) / C::BR;
    const int64_t grid = (int64_t)B * H * nqt;
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, o, lse, N, nqt, scale);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_c(const void *q, const void *k, const void *v, float *o, float *lse,
                               int B, int H, int N, float scale, int causal, hipStream_t stream)
{
    return causal ? launch_fwd<T, D, true>(q, k, v, o, lse, B, H, N, scale, stream)
                  : launch_fwd<T, D, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

// Dispatch to the instantiation for (dtype, d, causal).  Arguments were
// validated by the caller; dtype 0/1/2 = fp32/bf16/fp16, d in {64, 128}.
hipError_t fwd_dispatch(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                        int H, int N, int d, float scale, int causal, int dtype,
                        hipStream_t stream)
{
    switch (dtype) {
    case 0:
        return d == 64 ? launch_fwd_c<float, 64>(q, k, v, o, lse, B, H, N, scale, causal, stream)
                       : launch_fwd_c<float, 128>(q, k, v, o, lse, B, H, N, scale, causal, stream);
    case 1:
        return d == 64 ? launch_fwd_c<__bf16, 64>(q, k, v, o, lse, B, H, N, scale, causal, stream)
                       : launch_fwd_c<__bf16, 128>(q, k, v, o, lse, B, H, N, scale, causal, stream);
    default:
        return d == 64
                   ? launch_fwd_c<_Float16, 64>(q, k, v, o, lse, B, H, N, scale, causal, stream)
                   : launch_fwd_c<_Float16, 128>(q, k, v, o, lse, B, H, N, scale, causal, stream);
    }
}

}  // namespace fa
