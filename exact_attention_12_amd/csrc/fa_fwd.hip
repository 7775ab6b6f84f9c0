// fa_fwd.hip -- FlashAttention forward pass for gfx950.
//
// Computes O = softmax(scale * Q K^T [+ causal mask]) V for every (b, h) of
// [B, H, N, d] tensors, tile by tile with the online softmax, so the N x N
// score matrix never leaves the chip ("FlashAttention: GPU 메모리 계층을
// 활용한 어텐션 최적화 분석", youngju.dev, sections 5 and 6; "Flash
// Attention", suniverse77.github.io, Eq. (1)-(4)).
//
// Work decomposition (FlashAttention-2 order, youngju.dev sections 8.2-8.3):
//  - one workgroup of NW waves per (b, h, 32 NW-row query tile): 8 waves
//    (256 rows) for the plain forward on 16-bit inputs at d = 128, 4 waves
//    (128 rows) otherwise; the query tile is split across the waves, 32 rows each,
//    with no communication between waves (split-Q).  Causal: a workgroup
//    takes a heavy and a light query tile of the same head one after the
//    other, so all workgroups carry about the same work;
//  - every wave keeps its Q rows in registers as matrix-core operands; the
//    K/V tiles (BC keys each) that all the waves share stream from HBM
//    straight into LDS (16-byte direct-to-LDS loads, no register staging),
//    row-major with an XOR swizzle of the 16-byte chunks that keeps both
//    read patterns below free of bank conflicts.  Double buffered with one
//    barrier per tile, or, for the 8-wave form, a 4-slot ring whose tiles
//    go in pairs: a pair loads the next two tiles, computes its two, and
//    takes one barrier (the ring keeps the K tiles of all slots below
//    64 KiB and the V tiles above, within the LDS reads' offset reach);
//  - S^T = K Q^T is formed on the matrix cores, so each lane owns one query
//    row and 16 keys of each 32-key block: the row max and the row sum are
//    in-lane except for one exchange between the two lane halves;
//  - the probabilities P~ stay in the accumulator registers and feed
//    O^T += V^T P~^T directly.  The key order inside a tile is permuted to
//    match the operand layout (a sum over keys does not see the order), and
//    the V^T operand is read from the row-major V tile with the LDS
//    transpose read (4-byte reads for fp32);
//  - the accumulator stays unnormalised and is divided by l once at the end
//    (FlashAttention-2, youngju.dev section 8.1);
//  - the exponentials are taken against a reference max that is set on the
//    first tile and moved only when a tile's probabilities would exceed
//    2^14; the row max is not computed on the other tiles at all;
//  - waves raise their issue priority over the matrix sections, so that the
//    other wave on the SIMD fills the matrix pipe's shadow with its vector
//    work rather than the reverse;
//  - causal: tiles entirely above the diagonal are never loaded; a wave skips
//    the arithmetic of tiles that are fully masked for its 32 rows; only
//    diagonal and ragged-tail tiles pay for element masks.
#include "fa_sizes.h"
#include "fa_tile.h"

#include <type_traits>

namespace fa {

template <typename T, int D, int NWV = 4> struct FwdCfg {
    static constexpr int NW = NWV;                    // waves per workgroup
    static constexpr int KW = Mma<T>::KW;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int VEC = 16 / ES;              // elements per 16-byte chunk
    static constexpr int NT = NW * kWave;             // threads per workgroup (NW waves)
    static constexpr int BR = NW * 32;                // query rows per workgroup
    static constexpr int BC = (ES == 4) ? 32 : 64;    // keys per K/V tile
    static constexpr int NKB = BC / 32;               // 32-key blocks per tile
    static constexpr int CPR = D / VEC;               // 16-byte chunks per row
    static constexpr int ROWB = D * ES;               // bytes per K/V row in LDS
    static constexpr int TILEB = BC * ROWB;           // bytes per K or V tile
    static constexpr int STAGEB = 2 * TILEB;          // K + V
    static constexpr int NLD = BC * CPR / kWave;      // direct-to-LDS loads per tile
    static constexpr int NLD_W = NLD / NW;            // ... per wave
    static constexpr int QK_STEPS = D / (2 * KW);     // MFMA steps over d for S
    static constexpr int PV_STEPS = 32 / (2 * KW);    // MFMA steps per 32-key block for PV
    static constexpr int DB = D / 32;                 // 32-row blocks of O^T
    // waves per SIMD: two when the registers allow
    static constexpr int WPE = (ES == 4 && D == 128) ? 1 : 2;
    static_assert(NLD % NW == 0, "tile loads must split evenly over the waves");
    static_assert(NW == 4 || NW == 8, "workgroups of 4 or 8 waves");
    static_assert(D % 32 == 0 && BC % 32 == 0, "tile shapes");
};

// Bound on the probabilities taken against a stale reference max (see the
// softmax step in the kernel): 2^14, representable in every input type.
constexpr float kPMax = 16384.0f;

// General masks (rectangular, windowed, boolean; the EXT kernels).  Query row
// i of Nq rows sees key j < Nk iff  i + off - wl <= j <= i + off + wr  and, with
// a mask, mask[i][j] != 0; off = Nk - Nq aligns the diagonal to the
// bottom-right corner.  Unbounded sides come in as bounds beyond the key range.
struct FwdExt {
    int Nk;               // keys (the kernel's N counts query rows)
    int off, wl, wr;      // diagonal offset and window, all pre-clamped by the host
    const uint8_t *mask;  // uint8 [.., Nq, ldm] or null
    int64_t msb, msh;     // byte strides of the mask between batches and heads
    int ldm;              // byte stride between mask rows (a multiple of 16, >= Nk)
    // Block map of the mask (fa_mask_blocks) or null.  Per (slice, 128-row
    // query block): nkw words with bit k set if 64-key block k holds a
    // visible pair, then nkw words with bit k set if it holds no masked one.
    const uint32_t *blocks;
    int nkw;              // words per half of a query block's entry
    int64_t bmb, bmh;     // word strides of the map between batches and heads
    // Paged K/V (EXT 4): K and V are the caches [blocks, Hkv, D/8, 16, 8] and
    // [blocks, Hkv, D, 16]; sequence b's keys are its context_lens[b] context
    // tokens, token t in block tables[b * mbps + t / 16] at slot t % 16.
    const int32_t *tables, *ctx_lens;
    int mbps;               // block-table entries per sequence
    uint32_t cache_bytes;   // bytes of one cache (< 4 GiB)
};

// EXT: 0 = square path (N queries and keys, optional top-left causal mask),
// 1 = general ranges (rectangular / windowed / bottom-right causal), 2 = 1
// plus a boolean mask, 3 = 2 with the mask's block map, 4 = 1 with K/V read
// from the paged cache (the number of keys and the diagonal's offset come
// from each sequence's context length).
// Transpose read (ds_read_b64_tr_b16) through a restrict parameter: once
// inlined, the read carries alias-scope information, and the compiler's
// wait-count insertion then does not wait for direct-to-LDS loads still in
// flight before it (without it, every pair of tiles of the 4-slot ring waits
// for both next tiles' loads in the middle of its first tile).  Valid where
// the loads in flight never target the slot being read: in the 4-slot ring
// a pair reads slots whose loads were waited for (vmcnt(0), then a barrier)
// at the end of the previous pair, while it loads the other two.
__device__ __forceinline__ s16x4 lds_read_tr16_scoped(const lds_s16x4 *__restrict__ p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
}

// Waves per workgroup.  The plain forward on 16-bit inputs at d = 128 takes
// 8: 256 query rows share each K/V tile, so every tile is loaded into LDS
// once per 256 rows instead of per 128, with one workgroup (two waves per
// SIMD) per CU; measured 1.4-4 % faster than two 4-wave workgroups per CU.
// At d = 64 (155 registers) three 4-wave workgroups fit a CU, and 8 waves
// measured ~10 % slower.  fp32 (one wave per SIMD at d = 128) and the
// general-mask and paged forms, whose block maps and cache walks are laid
// out for 128-row workgroups, take 4.
template <typename T, int D, int EXT> constexpr int fwd_waves()
{
    return (EXT == 0 && sizeof(T) == 2 && D == 128) ? 8 : 4;
}

template <typename T, int D, bool CAUSAL, int EXT>
__global__ __attribute__((amdgpu_flat_work_group_size(FwdCfg<T, D, fwd_waves<T, D, EXT>()>::NT,
                                                      FwdCfg<T, D, fwd_waves<T, D, EXT>()>::NT),
                          amdgpu_waves_per_eu(FwdCfg<T, D>::WPE, FwdCfg<T, D>::WPE)))
void fa_fwd_kernel(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                   float *__restrict__ O, float *__restrict__ LSE, int N, int num_qtiles,
                   float scale, int H, int group, FwdExt ext)
{
    static_assert(EXT == 0 || !CAUSAL, "general masks fold causality into the window");
    using C = FwdCfg<T, D, fwd_waves<T, D, EXT>()>;
    constexpr bool HAS_MASK = EXT == 2 || EXT == 3;  // a boolean mask rides along
    static_assert(EXT != 4 || (C::ES == 2 && D == 128 && C::BC == 64 && C::NLD_W == 4),
                  "paged K/V: each wave loads one 16-token cache block of K and of V per tile");
    static_assert(EXT != 3 || (C::BR == 128 && 64 % C::BC == 0),
                  "a block of the mask's map (128 x 64) is whole tiles");
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int KW = C::KW;
    // boolean mask: a (BR x BC)-byte tile of it rides along with each K/V tile,
    // rows of BC bytes with the 16-byte chunks swizzled by swzm()
    constexpr int MCPR = C::BC / 16;                            // 16-byte chunks per mask row
    constexpr int MASKB = HAS_MASK ? C::BR * C::BC : 0;         // mask tile bytes
    constexpr int NLDM_W = HAS_MASK ? C::BR * MCPR / kWave / 4 : 0;  // its 1 KiB loads per wave
    constexpr int SB = C::STAGEB + MASKB;                        // bytes per stage
    auto swzm = [](int row) { return MCPR == 4 ? (row >> 2) & 3 : (row >> 3) & 1; };
    // LDS ring of K/V tiles: 2 slots (one barrier per tile), or 4 for the
    // 8-wave plain forward, whose tiles go in pairs (one barrier per two tiles)
    constexpr int RING = (EXT == 0 && C::NW == 8) ? 4 : 2;
    __shared__ __attribute__((aligned(1024))) char smem[RING * SB];
    poison_lds(smem, sizeof(smem));
    // Slot placement.  Two slots: K, V (and the mask) of a slot side by side.
    // Four: the K tiles of all slots first, then the V tiles, so that every
    // K operand read reaches its slot with the instruction's 16-bit offset
    // field from one per-lane address, and every V read from another (the
    // ring spans 128 KiB; a slot-major layout would need an address add per
    // read of the upper half).
    static_assert(RING == 2 || (MASKB == 0 && C::ES == 2 && RING * C::TILEB <= 65536), "K slots within 64 KiB");
    constexpr int KSLOT = RING == 4 ? C::TILEB : SB;  // K tile of slot b at b * KSLOT
    constexpr int VBASE = RING == 4 ? RING * C::TILEB : C::TILEB;  // V tile of slot b at VBASE + b * KSLOT

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    // wave index in a scalar register: every branch on it is uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col = lane % 32;  // query row of this lane within the wave's 32
    const int h = lane / 32;    // lane half

    // Workgroup -> (b*H + h, query tile).  Consecutive workgroup ids are
    // dispatched round-robin over the 8 XCDs; remap so that the workgroups
    // resident on one XCD (sharing its L2) work on the same head.
    int wid = blockIdx.x;
    const int G = gridDim.x;
    // Causal: workgroup p of a head takes the query tiles nqt-1-p (heavy)
    // and p (light) one after the other, so that every workgroup has about
    // the same work and the grid drains evenly.
    const int wg_per_head = CAUSAL ? (num_qtiles + 1) / 2 : num_qtiles;
    int bh, pi;
    if constexpr (EXT == 4) {
        // Sequences differ in length, so a contiguous share of the grid per
        // XCD would leave the XCDs unevenly loaded.  Instead the units
        // (sequence, kv head) are dealt round-robin over the XCDs: with 8 | S*Hkv
        // XCD x takes units x, x+8, ..., each unit's group * nqt workgroups in
        // a row (they read the same K/V through that XCD's L2).  Sequences go
        // longest first (ranked from the context lengths, up to 64
        // sequences), so that the short ones fill the grid's tail.
        const int W = group * wg_per_head;
        const int units = G / W;
        const int hkv = H / group;
        int u = wid, r = 0;
        if (units % 8 == 0) {
            const int t = wid / 8;
            u = (t / W) * 8 + wid % 8;
            r = t % W;
        } else {
            u = wid / W;
            r = wid % W;
        }
        int seq = u / hkv;
        const int S = units / hkv;
        if (S <= kWave) {
            const int mine = lane < S ? ext.ctx_lens[lane] : INT_MIN;
            int rank = 0;
            for (int j = 0; j < S; ++j) {
                const int cj = __builtin_amdgcn_readlane(mine, j);
                rank += (cj > mine || (cj == mine && j < lane)) ? 1 : 0;
            }
            const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < S && rank == seq);
            seq = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
        }
        bh = seq * H + (u % hkv) * group + r / wg_per_head;
        pi = r % wg_per_head;
    } else {
        if (G % 8 == 0) wid = (wid % 8) * (G / 8) + wid / 8;
        bh = wid / wg_per_head;
        pi = wid % wg_per_head;
    }

    // keys of this head and the diagonal's offset (paged: per sequence)
    int NK = EXT ? ext.Nk : N;
    int OFF = ext.off;
    if constexpr (EXT == 4) {
        NK = ext.ctx_lens[bh / H];
        OFF = NK - N;
    }

    // Q, O, lse: head bh = b*H + h.  K, V: kv head b*(H/group) + h/group
    // (group query heads share one kv head; group = 1 is multi-head attention).
    const int64_t head = (int64_t)bh * N * D;
    const int kvh = (bh % H) / group;  // paged: the kv head inside a cache block
    const int64_t kv_head = EXT == 4 ? 0 : ((int64_t)(bh / H) * (H / group) + kvh) * NK * D;
    const T *Qh = Q + head;
    const T *Kh = K + kv_head;
    const T *Vh = V + kv_head;

    // state of the current query tile (set per tile below)
    int q0 = 0, qrow = 0, wq_lo = 0, wq_hi = 0, ntiles = 0;
    frag qf[C::QK_STEPS];

    // With a boolean mask at d = 128 in 16-bit types, a wave's live values
    // exceed the 256 registers it has at two waves per SIMD.  There, values
    // that are cheap to derive from the lane id are derived again where they
    // are used (from a copy of the lane id that the compiler cannot hoist)
    // instead of being held across the key loop, where the register
    // allocator would spill them: a reload from scratch waits for every load
    // issued before it, the next tile's prefetch included.
    constexpr bool TIGHT = HAS_MASK && D == 128 && C::ES == 2;
    auto lane_id = [&]() __attribute__((always_inline)) {
        int l = lane;
        if constexpr (TIGHT) asm volatile("" : "+v"(l));
        return l;
    };

    // ---- K/V tile j -> LDS buffer buf, straight from global memory --------
    // Load instruction I of a tile fills LDS bytes [I*1024, I*1024 + 1024):
    // lane l writes chunk position q = I*64 + l, i.e. row q / CPR, position
    // q % CPR, which holds global chunk (q % CPR) ^ swz(row).  The element
    // offset of that chunk relative to the tile's first row is the same for
    // every tile.  Rows past the end of the sequence re-read row N-1: their
    // scores are masked, and the values stay finite so that 0 * V is 0.
    // Loads go through buffer resources (base = this head's K or V, scalar
    // registers); the per-lane byte offset within a tile is fixed, the tile's
    // offset is a scalar.
    int ld_row[C::NLD_W], ld_off[C::NLD_W];
#pragma unroll
    for (int i = 0; i < C::NLD_W; ++i) {
        const int q = (wave * C::NLD_W + i) * kWave + lane;
        ld_row[i] = q / C::CPR;
        ld_off[i] = (ld_row[i] * D + ((q % C::CPR) ^ swz<C::CPR, C::ES>(ld_row[i])) * C::VEC) * C::ES;
    }
    const int head_bytes = EXT == 4 ? (int)ext.cache_bytes : NK * C::ROWB;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)Kh, 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)Vh, 0, head_bytes, kBufferFlags);
    const uint8_t *mbase = nullptr;
    if constexpr (HAS_MASK) mbase = ext.mask + (int64_t)(bh / H) * ext.msb + (int64_t)(bh % H) * ext.msh;
    const __amdgpu_buffer_rsrc_t mrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)mbase, 0, HAS_MASK ? N * ext.ldm : 0, kBufferFlags);
    // per-lane mask-tile load offsets (set per query tile): load I, lane l
    // fills chunk position p = I*64 + l = row p / MCPR, position p % MCPR
    // holding chunk (p % MCPR) ^ swzm(row) of mask row q0 + row
    int m_off[NLDM_W > 0 ? NLDM_W : 1];
    auto set_mask_offsets = [&](int q0_) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NLDM_W; ++i) {
            const int p = (wave * NLDM_W + i) * kWave + lane;
            const int row = p / MCPR;
            m_off[i] = (q0_ + row) * ext.ldm + ((p % MCPR) ^ swzm(row)) * 16;
        }
    };
    // Paged K/V: wave w loads cache block 4j + w of tile j (its 16 keys).
    // K keeps the layout above: LDS chunk position q of the wave's loads
    // holds chunk (q % CPR) ^ swz(row) of token row % 16, which the cache
    // block holds at byte ((chunk * 16) + row % 16) * 16.  V is copied block
    // by block as the cache holds it, [d][16 tokens] (4 KiB per block), with
    // the two 16-byte halves of a d-row swapped for d & 8 (bank spread for
    // the operand reads below).  The block id, a scalar load from the table
    // row (which stays in the scalar cache across consecutive tiles), is the
    // load's scalar offset.  Blocks past the context re-read its last block:
    // their keys are masked and their values are zeroed before use.
    int kp_off[EXT == 4 ? C::NLD_W : 1], vp_off[EXT == 4 ? C::NLD_W : 1];
    const int32_t *trow = nullptr;  // this sequence's block-table row
    int last_blk = 0;
    if constexpr (EXT == 4) {
#pragma unroll
        for (int i = 0; i < C::NLD_W; ++i) {
            const int q = (wave * C::NLD_W + i) * kWave + lane;
            const int row = q / C::CPR;
            kp_off[i] = (((q % C::CPR) ^ swz<C::CPR, C::ES>(row)) * 16 + row % 16) * 16;
            const int p = i * kWave + lane, d = p / 2;
            vp_off[i] = (d * 2 + ((p % 2) ^ ((d >> 3) & 1))) * 16;
        }
        trow = ext.tables + (int64_t)(bh / H) * ext.mbps;
        last_blk = min(max(NK - 1, 0) / 16, ext.mbps - 1);
    }
    auto load_tile = [&](int j, int buf, bool with_mask) {
        const int k0 = j * C::BC;
        char *kd = smem + buf * KSLOT;
        char *vd = smem + VBASE + buf * KSLOT;
        if constexpr (EXT == 4) {
            const uint32_t blk = (uint32_t)trow[min(j * 4 + wave, last_blk)];
            // (block, kv head) slab of 4 KiB; below 4 GiB (checked by the host)
            const int boff = (int)((blk * (uint32_t)(H / group) + (uint32_t)kvh) * (uint32_t)(D * 16 * C::ES));
#pragma unroll
            for (int i = 0; i < C::NLD_W; ++i) {
                const int I = wave * C::NLD_W + i;
                buffer_load_lds16(krs, kd + I * 1024, kp_off[i], boff);
                buffer_load_lds16(vrs, vd + I * 1024, vp_off[i], boff);
            }
            return;
        }
        const int soff = k0 * C::ROWB;
        if (k0 + C::BC <= NK) {
#pragma unroll
            for (int i = 0; i < C::NLD_W; ++i) {
                const int I = wave * C::NLD_W + i;
                buffer_load_lds16(krs, kd + I * 1024, ld_off[i], soff);
                buffer_load_lds16(vrs, vd + I * 1024, ld_off[i], soff);
            }
        } else {
            // ragged last tile: rows >= N re-read row N-1
#pragma unroll
            for (int i = 0; i < C::NLD_W; ++i) {
                const int I = wave * C::NLD_W + i;
                int row = ld_row[i];
                if constexpr (TIGHT) row = (I * kWave + lane_id()) / C::CPR;
                const int over = k0 + row - (NK - 1);
                const int off = over > 0 ? ld_off[i] - over * C::ROWB : ld_off[i];
                buffer_load_lds16(krs, kd + I * 1024, off, soff);
                buffer_load_lds16(vrs, vd + I * 1024, off, soff);
            }
        }
        if constexpr (HAS_MASK) {
            // rows past the end of the mask read as 0 (buffer bounds)
            if (with_mask) {
#pragma unroll
                for (int i = 0; i < NLDM_W; ++i)
                    buffer_load_lds16(mrs, kd + C::STAGEB + (wave * NLDM_W + i) * 1024, m_off[i], k0);
            }
        }
    };
    // byte offset of element e of row r in a swizzled tile
    auto lds_off = [](int r, int e) {
        const int cc = (e * C::ES) / 16, o = (e * C::ES) % 16;
        return r * C::ROWB + ((cc ^ swz<C::CPR, C::ES>(r)) * 16) + o;
    };
    // Per-lane LDS read offsets that are the same for every tile.  The
    // swizzle depends on the row only through row % 16, and the key-block and
    // step offsets below are multiples of 16 rows.
    int k_rd[C::QK_STEPS];  // K operand of step st: row col, elements st*2KW + h*KW
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) k_rd[st] = lds_off(col, st * 2 * KW + h * KW);
    int v_rd[2][C::DB];  // 16-bit V^T transpose-read sources of block db (rows +0 / +8)
    {
        const int g = lane / 16, r16 = lane % 16;
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
                v_rd[hi][db] = lds_off(8 * hi + 4 * (g / 2) + r16 / 4,
                                       db * 32 + 16 * (g % 2) + 4 * (r16 % 4));
    }
    // Four slots: the V reads add VBASE here, once, in a register the
    // compiler cannot see through (so it does not fold VBASE back into each
    // read's offset, past the field's range); Vs below then leaves it out.
    constexpr int VREG = RING == 4 ? VBASE : 0;
    if constexpr (RING == 4) {
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                v_rd[hi][db] += VREG;
                asm volatile("" : "+v"(v_rd[hi][db]));
            }
    }

    // ---- running state (per lane: one query row, partial over its keys) --
    f32x16 acc[C::DB];
    float m_ref, mc_ref;  // reference max of the raw scores q.k (see below), and m_ref * c
    float l_run, l_hat;   // partial row sum of P~ (fp32), and of P~ as rounded for the matrix core
    // c > 0 even for scale 0 (or a scale so small that c would be a
    // denormal): -inf * c must stay -inf for masked keys.  In that range
    // s * c rounds every probability to exactly 1 either way.
    const float c = fmaxf(scale * kLog2e, 1e-30f);

    // S^T = K Q^T for the BC keys of the tile at Ks (raw dot products).  The
    // K operands are read from LDS in groups of two steps, one group
    // ahead of the matrix products that use them.
    auto qk = [&](const char *Ks, f32x16 (&s)[C::NKB]) {
        constexpr int G = HAS_MASK ? 1 : 2;  // registers for the boolean mask
        constexpr int NG = C::QK_STEPS / G;
        frag kf[2][G][C::NKB];
        auto rd = [&](int g, int b) {
#pragma unroll
            for (int i = 0; i < G; ++i)
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
                    kf[b][i][kb] = *(const frag *)(Ks + kb * 32 * C::ROWB + k_rd[g * G + i]);
        };
        rd(0, 0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) rd(g + 1, (g + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < G; ++i)
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
                    s[kb] = M::mma(kf[g & 1][i][kb], qf[g * G + i], (g == 0 && i == 0) ? f32x16{} : s[kb]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // Masks: keys >= N (ragged tail) and, causal, keys > query row.  Key
    // k0 + kb*32 + acc_row(r, h) is visible iff acc_row(r, 0) <= lim[kb].
    // General masks add a lower bound lo[kb] (visible iff acc_row(r, 0) >=
    // lo[kb]) and the mask bytes of the lane's 16 keys per block.
    auto limits = [&](int k0, int (&lim)[C::NKB], int (&lo)[C::NKB]) {
        int last = CAUSAL ? min(qrow, N - 1) : N - 1;
        int first = 0;
        if constexpr (EXT != 0) {
            int qr = qrow;
            if constexpr (TIGHT) qr = q0 + wave * 32 + lane_id() % 32;
            qr = min(qr, N - 1);  // rows past the end behave like row N-1
            last = min(qr + OFF + ext.wr, NK - 1);
            first = qr + OFF - ext.wl;
        }
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            lim[kb] = last - k0 - kb * 32 - 4 * h;
            lo[kb] = first - k0 - kb * 32 - 4 * h;
        }
    };
    // mask bytes of keys k0 + kb*32 + 8g + 4h + 0..3 of this lane's row, one
    // dword per (kb, g), from the tile's mask in LDS
    auto read_mask = [&](const char *Ms, uint32_t (&mw)[C::NKB][4]) __attribute__((always_inline)) {
        const int l = lane_id(), row = wave * 32 + l % 32, hh = l / 32;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int chunk = 2 * kb + g / 2;
                mw[kb][g] = *(const uint32_t *)(Ms + row * C::BC + ((chunk ^ swzm(row)) * 16) + 8 * (g % 2) + 4 * hh);
            }
    };
    // returns the visible scores as bits kb*16 + r (used by the boolean mask)
    auto apply_mask = [&](f32x16 (&s)[C::NKB], const int (&lim)[C::NKB], const int (&lo)[C::NKB],
                          const uint32_t (&mw)[C::NKB][4]) {
        uint32_t bits = 0;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                bool off_ = acc_row(r, 0) > lim[kb];
                if constexpr (EXT != 0) off_ = off_ || acc_row(r, 0) < lo[kb];
                if constexpr (HAS_MASK) off_ = off_ || ((mw[kb][r / 4] >> (8 * (r % 4))) & 0xffu) == 0;
                if (off_) s[kb][r] = -INFINITY;
                else bits |= 1u << (kb * 16 + r);
            }
        return bits;
    };
    auto apply_bits = [&](f32x16 (&s)[C::NKB], uint32_t bits) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (!((bits >> (kb * 16 + r)) & 1u)) s[kb][r] = -INFINITY;
    };
    // first and last key tiles of this wave's rows (general masks)
    int jw_beg = 0, jw_end = 0;

    // Move the reference to the row max of this tile where that is larger,
    // rescaling what was accumulated against the old reference.
    auto rebase = [&](const f32x16 (&s)[C::NKB]) {
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = halves_max(mx);
        const float m_new = fmaxf(m_ref, mx);
        const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
        const float mc_new = m_safe * c;
        // a row that saw no key yet (m_ref = -inf) has nothing to rescale
        const float alpha = (EXT != 0 && m_ref == -INFINITY) ? 0.f : exp2_hw(mc_ref - mc_new);  // e^(scale*(m_old - m_new)); 0 at start
        l_run *= alpha;
        l_hat *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
        m_ref = m_new;
        mc_ref = mc_new;
    };
    // P~ = exp(scale*(s - m_ref)) = 2^(s*c - m_ref*c) in place; returns this
    // lane's sum.  Masked keys (s = -inf) give 0 since c > 0.
    auto exponentiate = [&](f32x16 (&s)[C::NKB]) {
        float part[4];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = exp2_hw(__builtin_fmaf(s[kb][r], c, -mc_ref));
                part[r % 4] = (kb == 0 && r < 4) ? s[kb][r] : part[r % 4] + s[kb][r];
            }
        return (part[0] + part[1]) + (part[2] + part[3]);
    };

    // One K/V tile: j is the tile, STAGE its LDS slot; jn is the tile to
    // load next (ntiles: none).  Boolean mask: part (part_n) tells whether
    // tile j (jn) needs its mask bytes; without them it is fully visible.
    // SYNC: the tile issues the load of jn into the other of two slots and
    // ends with the barrier; otherwise it only computes (the 4-slot ring's
    // pairs load and synchronise around two tiles).
    auto tile = [&](int j, int jn, bool part, bool part_n, auto stage_c, auto sync_c) {
        constexpr int STAGE = decltype(stage_c)::value;
        constexpr bool SYNC = decltype(sync_c)::value;
        const int k0 = j * C::BC;
        if (SYNC && jn < ntiles) load_tile(jn, STAGE ^ 1, part_n);
        uint32_t mcur[C::NKB][4];
        if constexpr (HAS_MASK) {
            if (part) {
                read_mask(smem + STAGE * SB + C::STAGEB, mcur);
            } else {
                // every pair of the block takes part; rows past the end stay
                // masked, as the mask bytes read for them are 0
                const uint32_t all = qrow < N ? 0xffffffffu : 0u;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) mcur[kb][g] = all;
            }
        }
        const char *Ks = smem + STAGE * KSLOT;
        const char *Vs = smem + VBASE - VREG + STAGE * KSLOT;  // VREG: in v_rd

        bool skip = EXT != 0 && (j < jw_beg || j >= jw_end);  // no row of the wave sees a key here
        if constexpr (HAS_MASK) {
            // ... or the mask hides every key of the tile from every row of the wave
            if (part) {
                uint32_t any = 0;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) any |= mcur[kb][g];
                skip = skip || __builtin_amdgcn_ballot_w64(any != 0) == 0;
            }
        }
        if (skip) {
            if constexpr (SYNC) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            }
            return;
        }
        f32x16 s[C::NKB];
        qk(Ks, s);
        bool need_mask = (k0 + C::BC > NK) || (CAUSAL && k0 + C::BC - 1 > wq_lo);
        if constexpr (EXT != 0)
            need_mask = k0 < min(wq_hi, N - 1) + OFF - ext.wl ||
                        k0 + C::BC - 1 > min(wq_lo + OFF + ext.wr, NK - 1);
        if constexpr (HAS_MASK) need_mask = need_mask || part || wq_hi >= N;
        int lim[C::NKB], lo[C::NKB];
        limits(k0, lim, lo);
        uint32_t vis = 0;
        if (need_mask) vis = apply_mask(s, lim, lo, mcur);

        // Lazy reference max.  The probabilities are taken relative to a
        // reference m_ref instead of the running max: exp(s - m) =
        // exp(s - m') exp(m' - m) for any m, m', so the result does not
        // depend on it as long as nothing overflows.  The first tile sets
        // m_ref to its row max (every row sees key 0, so it is finite);
        // later tiles exponentiate against the stale reference first and
        // only if some lane's sum exceeds kPMax = 2^14 (which bounds every
        // probability, keeping it representable even in fp16) recompute the
        // tile's scores and move the reference.
        // General masks: a row may see no key of its first tiles, so the
        // reference is (re)set while any row of the wave has none yet.  With
        // a boolean mask, rows past the end see no key at all and take no
        // part in that decision (their mc_ref starts at 0, so that their
        // probabilities come out as exp2(-inf) = 0 without a reference).
        if (EXT == 0 ? j == 0
                     : __builtin_amdgcn_ballot_w64(m_ref == -INFINITY && (!HAS_MASK || qrow < N)) != 0)
            rebase(s);
        float rs = exponentiate(s);
        if ((EXT != 0 || j != 0) && __builtin_amdgcn_ballot_w64(!(rs <= kPMax)) != 0) {
            qk(Ks, s);
            if (need_mask) {
                if constexpr (HAS_MASK) apply_bits(s, vis);
                else apply_mask(s, lim, lo, mcur);
            }
            rebase(s);
            rs = exponentiate(s);
        }
        l_run += rs;

        __builtin_amdgcn_s_setprio(1);
        // O^T += V^T P~^T.  PV step st of key block kb contracts the
        // registers [st*KW, st*KW + KW) of both lane halves; slot h*KW + e
        // holds key kb*32 + acc_row(st*KW + e, h).
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int st = 0; st < C::PV_STEPS; ++st) {
                float pv[KW];
#pragma unroll
                for (int e = 0; e < KW; ++e) pv[e] = s[kb][st * KW + e];
                const frag b = M::pack(pv);
                l_hat = M::sum(b, l_hat);
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    frag a;
                    if constexpr (EXT == 4) {
                        // Paged V, [d][16 tokens] per 4 KiB block: block 2kb+st of
                        // the tile holds keys kb*32 + 16*st + 0..15; this lane takes
                        // tokens 4h..4h+3 and 8+4h..8+4h+3 of head element d.
                        const int dd = db * 32 + col, sw = (dd >> 3) & 1;
                        const char *vb = Vs + (2 * kb + st) * 4096 + dd * 32 + 8 * h;
                        s16x4 lo = *(const s16x4 *)(vb + 16 * sw);
                        s16x4 hi = *(const s16x4 *)(vb + 16 * (sw ^ 1));
                        if (k0 + C::BC > NK) {
                            // slots past the context may hold anything: 0 * V must be 0
                            const int t0 = k0 + (2 * kb + st) * 16 + 4 * h;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if (t0 + e >= NK) lo[e] = 0;
                                if (t0 + 8 + e >= NK) hi[e] = 0;
                            }
                        }
                        a = __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    } else if constexpr (C::ES == 2) {
                        // Two transpose reads, each giving this lane 4
                        // consecutive keys of head element db*32 + col: keys
                        // kb*32 + 16*st + 4*h (+8) + 0..3.  Source lane r of
                        // each 16-lane group g points at row kb*32 + 16*st +
                        // 4*(g/2) + r/4 (+8), elements db*32 + 16*(g%2) +
                        // 4*(r%4) .. +3.
                        const char *vblk = Vs + (kb * 32 + 16 * st) * C::ROWB;
                        s16x4 lo, hi;
                        if constexpr (RING == 4) {
                            lo = lds_read_tr16_scoped((const lds_s16x4 *)(vblk + v_rd[0][db]));
                            hi = lds_read_tr16_scoped((const lds_s16x4 *)(vblk + v_rd[1][db]));
                        } else {
                            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vblk + v_rd[0][db]));
                            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vblk + v_rd[1][db]));
                        }
                        a = __builtin_bit_cast(frag,
                                               __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    } else {
                        a = *(const frag *)(Vs + lds_off(kb * 32 + acc_row(st, h), db * 32 + col));
                    }
                    acc[db] = M::mma(a, b, acc[db]);
                }
            }
        }

        __builtin_amdgcn_s_setprio(0);
        if constexpr (SYNC) {
            // this wave's loads of the next tile have landed, and after the
            // barrier every wave's have, and nobody reads the current buffer
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    };

  for (int item = 0; item < (CAUSAL ? 2 : 1); ++item) {
    // General masks: the last query tiles see the most keys when the diagonal
    // is aligned bottom-right; dispatch them first so the grid drains evenly.
    const int qt = CAUSAL ? (item == 0 ? num_qtiles - 1 - pi : pi) : (EXT != 0 ? num_qtiles - 1 - pi : pi);
    if (CAUSAL && item == 1 && qt == num_qtiles - 1 - pi) break;  // odd count: middle tile alone
    q0 = qt * C::BR;
    qrow = q0 + wave * 32 + col;
    wq_lo = q0 + wave * 32;  // first query row of this wave
    wq_hi = wq_lo + 31;      // last query row of this wave
    // Q rows of this lane as B operands: d = st*2KW + h*KW .. +KW.
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) {
        if (qrow < N)
            qf[st] = *(const frag *)(Qh + (int64_t)qrow * D + st * 2 * KW + h * KW);
        else
            qf[st] = frag{};
    }
    int kend = CAUSAL ? min(N, q0 + C::BR) : N;  // keys [0, kend) can be seen
    int jbeg = 0;
    if constexpr (EXT != 0) {
        // keys [kbeg, kend) can be seen by the workgroup's rows, and
        // [kw_beg, kw_end) by this wave's
        const int q_last = min(q0 + C::BR, N) - 1;
        const int kbeg = max(0, q0 + OFF - ext.wl);
        kend = min(NK, q_last + OFF + ext.wr + 1);
        jbeg = kbeg / C::BC;
        const int w_last = min(wq_hi, N - 1);
        const int kw_beg = max(0, wq_lo + OFF - ext.wl);
        const int kw_end = min(NK, w_last + OFF + ext.wr + 1);
        jw_beg = kw_beg / C::BC;
        jw_end = (wq_lo < N && kw_end > kw_beg) ? (kw_end + C::BC - 1) / C::BC : 0;
        if constexpr (HAS_MASK) set_mask_offsets(q0);
    }
    ntiles = kend > jbeg * C::BC ? (kend + C::BC - 1) / C::BC : jbeg;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
    m_ref = -INFINITY;
    mc_ref = HAS_MASK ? 0.f : -INFINITY;
    l_run = 0.f;
    l_hat = 0.f;

    if constexpr (EXT == 3) {
        // Boolean mask with its block map: tiles whose 64-key block holds no
        // visible pair for this query block are never loaded, and tiles whose
        // block holds no masked pair skip the mask bytes; the tiles left run
        // in key order, alternating LDS buffers.  The map's words are read
        // with scalar loads, one word (32 blocks) at a time.
        const uint32_t *mrow = ext.blocks + (int64_t)(bh / H) * ext.bmb + (int64_t)(bh % H) * ext.bmh +
                               (int64_t)qt * 2 * ext.nkw;
        int wi = -1;
        uint32_t w_any = 0, w_full = 0;
        auto word = [&](int w) {
            if (w != wi) {
                wi = w;
                w_any = mrow[w];
                w_full = mrow[ext.nkw + w];
            }
        };
        // first tile after jj that the map does not rule out (ntiles: none)
        auto next = [&](int jj) {
            int jn = jj + 1;
            while (jn < ntiles) {
                const int bl = jn * C::BC / 64;
                word(bl / 32);
                const uint32_t rest = w_any >> (bl % 32);
                if (rest & 1u) return jn;
                jn = (rest ? bl + (int)__builtin_ctz(rest) : (bl / 32 + 1) * 32) * 64 / C::BC;
            }
            return ntiles;
        };
        auto partial = [&](int jj) {
            if (jj >= ntiles) return true;
            const int bl = jj * C::BC / 64;
            word(bl / 32);
            return ((w_full >> (bl % 32)) & 1u) == 0;
        };
        int j = next(jbeg - 1);
        bool part = partial(j);
        if (j < ntiles) {
            load_tile(j, 0, part);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        while (j < ntiles) {
            int jn = next(j);
            bool pn = partial(jn);
            tile(j, jn, part, pn, std::integral_constant<int, 0>{}, std::integral_constant<bool, true>{});
            j = jn;
            part = pn;
            if (j >= ntiles) break;
            jn = next(j);
            pn = partial(jn);
            tile(j, jn, part, pn, std::integral_constant<int, 1>{}, std::integral_constant<bool, true>{});
            j = jn;
            part = pn;
        }
    } else if constexpr (RING == 4) {
        // Tiles in pairs over a 4-slot ring: tile t sits in slot
        // (t - jbeg) % 4.  A pair (a, a+1) first issues the loads of a+2 and
        // a+3 into the slots that a-2 and a-1 left before the last barrier,
        // computes a and a+1 (the wave's visible ones), and ends with one
        // barrier.  The pair loop runs over the workgroup's tiles, so every
        // wave meets the same barriers.
        const int nt_w = CAUSAL ? min(ntiles, wq_hi / C::BC + 1) : ntiles;
        if (jbeg < ntiles) load_tile(jbeg, 0, false);
        if (jbeg + 1 < ntiles) load_tile(jbeg + 1, 1, false);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        auto pair = [&](int a, auto s0_c) __attribute__((always_inline)) {
            constexpr int S0 = decltype(s0_c)::value;  // slot of tile a: 0 or 2
            if (a + 2 < ntiles) load_tile(a + 2, (S0 + 2) % 4, false);
            if (a + 3 < ntiles) load_tile(a + 3, (S0 + 3) % 4, false);
            if (a < nt_w)
                tile(a, ntiles, true, true, std::integral_constant<int, S0>{}, std::integral_constant<bool, false>{});
            if (a + 1 < nt_w)
                tile(a + 1, ntiles, true, true, std::integral_constant<int, S0 + 1>{},
                     std::integral_constant<bool, false>{});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };
        for (int a = jbeg; a < ntiles; a += 4) {
            pair(a, std::integral_constant<int, 0>{});
            if (a + 2 < ntiles) pair(a + 2, std::integral_constant<int, 2>{});
        }
    } else {
        if (jbeg < ntiles) {
            load_tile(jbeg, 0, EXT == 2);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // Causal: this wave's rows see no key of tiles j >= nt_w; those tiles
        // are still loaded for the other waves (same barrier count for every
        // wave).  General masks: every tile of the workgroup's range runs
        // through tile(), which skips the arithmetic for the wave's tiles
        // outside [jw_beg, jw_end).
        const int nt_w = CAUSAL ? min(ntiles, wq_hi / C::BC + 1) : ntiles;
        int j = jbeg;
        for (; j + 1 < nt_w; j += 2) {
            tile(j, j + 1, true, true, std::integral_constant<int, 0>{}, std::integral_constant<bool, true>{});
            tile(j + 1, j + 2, true, true, std::integral_constant<int, 1>{}, std::integral_constant<bool, true>{});
        }
        if (j < nt_w) {
            tile(j, j + 1, true, true, std::integral_constant<int, 0>{}, std::integral_constant<bool, true>{});
            ++j;
        }
        for (; j < ntiles; ++j) {
            if (j + 1 < ntiles) load_tile(j + 1, (j + 1 - jbeg) & 1, EXT == 2);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }

    // ---- epilogue: O = acc / l, lse = scale*m + ln l ----------------------
    // O is normalised by the sum of the probabilities exactly as the matrix
    // core saw them (rounded to the input type), so the output is a convex
    // combination of the value rows with consistently rounded weights; lse
    // uses the unrounded fp32 sum.
    const float l_tot = halves_sum(l_run);
    float inv = 1.f / halves_sum(l_hat);
    if (EXT != 0 && !(l_tot > 0.f)) inv = 0.f;  // no visible key: O = 0, lse = -inf
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
        // a row with no visible key has m_ref = -inf: its lse is -inf, also at
        // scale 0 (where scale * m_ref alone would give NaN)
        if (h == 0)
            LSE[(int64_t)bh * N + qrow] = (EXT != 0 && !(l_tot > 0.f)) ? -INFINITY
                                                                       : scale * m_ref + log2_hw(l_tot) * kLn2;
    }
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd(const void *q, const void *k, const void *v, float *o, float *lse,
                             int B, int H, int Hkv, int N, float scale, hipStream_t stream)
{
    using C = FwdCfg<T, D, fwd_waves<T, D, 0>()>;
    const int nqt = (N + C::BR - 1) / C::BR;
    const int64_t grid = (int64_t)B * H * (CAUSAL ? (nqt + 1) / 2 : nqt);
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, 0>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, o, lse, N, nqt, scale, H, H / Hkv,
                       FwdExt{N, 0, 0, 0, nullptr, 0, 0, 0, nullptr, 0, 0, 0});
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_ext(const void *q, const void *k, const void *v, float *o, float *lse,
                                 int B, int H, int Hkv, int Nq, float scale, const FwdExt &ext,
                                 hipStream_t stream)
{
    using C = FwdCfg<T, D, 4>;  // EXT 1..3: fwd_waves() is 4
    const int nqt = (Nq + C::BR - 1) / C::BR;
    const int64_t grid = (int64_t)B * H * nqt;
    if (ext.mask && ext.blocks)
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, false, 3>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                           (const T *)q, (const T *)k, (const T *)v, o, lse, Nq, nqt, scale, H, H / Hkv, ext);
    else if (ext.mask)
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, false, 2>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                           (const T *)q, (const T *)k, (const T *)v, o, lse, Nq, nqt, scale, H, H / Hkv, ext);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, false, 1>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                           (const T *)q, (const T *)k, (const T *)v, o, lse, Nq, nqt, scale, H, H / Hkv, ext);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_c(const void *q, const void *k, const void *v, float *o, float *lse,
                               int B, int H, int Hkv, int N, float scale, int causal,
                               hipStream_t stream)
{
    return causal ? launch_fwd<T, D, true>(q, k, v, o, lse, B, H, Hkv, N, scale, stream)
                  : launch_fwd<T, D, false>(q, k, v, o, lse, B, H, Hkv, N, scale, stream);
}

// Dispatch to the instantiation for (dtype, d, causal).  Arguments were
// validated by the caller; dtype 0/1/2 = fp32/bf16/fp16, d in {64, 128},
// Hkv divides H.
hipError_t fwd_dispatch(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                        int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                        hipStream_t stream)
{
    switch (dtype) {
    case 0:
        return d == 64 ? launch_fwd_c<float, 64>(q, k, v, o, lse, B, H, Hkv, N, scale, causal, stream)
                       : launch_fwd_c<float, 128>(q, k, v, o, lse, B, H, Hkv, N, scale, causal, stream);
    case 1:
        return d == 64 ? launch_fwd_c<__bf16, 64>(q, k, v, o, lse, B, H, Hkv, N, scale, causal, stream)
                       : launch_fwd_c<__bf16, 128>(q, k, v, o, lse, B, H, Hkv, N, scale, causal, stream);
    default:
        return d == 64
                   ? launch_fwd_c<_Float16, 64>(q, k, v, o, lse, B, H, Hkv, N, scale, causal, stream)
                   : launch_fwd_c<_Float16, 128>(q, k, v, o, lse, B, H, Hkv, N, scale, causal, stream);
    }
}

// (map_shape, the block map's shape, is in fa_sizes.h)

// x has a zero byte
__device__ __forceinline__ bool zero_byte(uint32_t x) { return ((x - 0x01010101u) & ~x & 0x80808080u) != 0; }

// Block map of a boolean mask: one workgroup of 16 waves per (slice, query
// block qb, word w of 32 key blocks = 2048 keys).  Thread t reads the
// 16-byte chunk (t % 128) of the word's keys in the 16 rows qb*128 +
// 16*(t / 128) + .., all 16 loads at once: the mask is streamed once, and a
// compute unit needs many loads in flight (four waves of 8-row batches ran
// at half the speed).  Bytes past Nk and rows past Nq do not count.  Bit i
// of the "any" word: key block 32w + i holds a nonzero byte; of the "full"
// word: it holds no zero byte (and at least one byte, so full implies any).
constexpr int kMapThreads = 1024, kMapRowsPerWave = kMapRows / (kMapThreads / kWave / 2);
__global__ __attribute__((amdgpu_flat_work_group_size(kMapThreads, kMapThreads)))
void fa_mask_blocks_kernel(const uint8_t *__restrict__ mask, int Hs, int Nq, int Nk, int64_t msb,
                           int64_t msh, int ldm, int nqb, int nkw, uint32_t *__restrict__ blocks)
{
    const int wid = blockIdx.x;
    const int w = wid % nkw, qb = (wid / nkw) % nqb, slice = wid / (nkw * nqb);
    const uint8_t *base = mask + (int64_t)(slice / Hs) * msb + (int64_t)(slice % Hs) * msh;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = (wave % 2) * kWave + lane;
    const int r0 = qb * kMapRows + (wave / 2) * kMapRowsPerWave;
    const int key0 = w * 32 * kMapCols + c * 16;
    const int nvalid = min(max(Nk - key0, 0), 16);  // bytes of the chunk inside the key range
    const int nrows = min(kMapRowsPerWave, Nq - r0);
    uint32_t keep[4];  // 0xff on the bytes inside the key range
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int nb = min(max(nvalid - 4 * i, 0), 4);
        keep[i] = nb == 4 ? 0xffffffffu : (1u << (8 * nb)) - 1u;
    }
    bool any = false, all = true;
    if (nvalid > 0 && nrows > 0) {
        const uint8_t *p = base + (int64_t)r0 * ldm + key0;
        for (int r = 0; r < nrows; r += 16) {
            u32x4 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (r + k < nrows) v[k] = *(const u32x4 *)(p + (int64_t)(r + k) * ldm);
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (r + k < nrows) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        any = any || (v[k][i] & keep[i]) != 0;
                        all = all && !zero_byte(v[k][i] | ~keep[i]);
                    }
                }
        }
    }
    // key block i of the wave's 64 chunks: lanes 4i .. 4i+3
    const uint64_t A = __builtin_amdgcn_ballot_w64(any), L = __builtin_amdgcn_ballot_w64(all);
    uint32_t ba = 0, bl = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if ((A >> (4 * i)) & 0xfu) ba |= 1u << i;
        if (((L >> (4 * i)) & 0xfu) == 0xfu) bl |= 1u << i;
    }
    __shared__ uint32_t sa[kMapThreads / kWave], sl[kMapThreads / kWave];
    poison_lds(sa, sizeof(sa));
    poison_lds(sl, sizeof(sl));
    if (lane == 0) {
        sa[wave] = ba;
        sl[wave] = bl;
    }
    __syncthreads();
    if (tid == 0) {
        // even waves hold key blocks 0..15 of the word, odd waves 16..31
        uint32_t a0 = 0, a1 = 0, f0 = ~0u, f1 = ~0u;
#pragma unroll
        for (int rg = 0; rg < kMapThreads / kWave / 2; ++rg) {
            a0 |= sa[2 * rg];
            a1 |= sa[2 * rg + 1];
            f0 &= sl[2 * rg];
            f1 &= sl[2 * rg + 1];
        }
        const uint32_t a = a0 | (a1 << 16);
        const uint32_t f = (f0 & 0xffffu) | (f1 << 16);
        uint32_t *out = blocks + ((int64_t)slice * nqb + qb) * 2 * nkw;
        out[w] = a;
        out[nkw + w] = f & a;
    }
}

// Arguments validated by the caller (the mask as for fwd_ext_dispatch; the
// grid below fits an int).
hipError_t mask_blocks_dispatch(const uint8_t *mask, int B, int H, int Nq, int Nk, int64_t msb,
                                int64_t msh, int ldm, uint32_t *blocks, hipStream_t stream)
{
    const MapShape m = map_shape(B, H, Nq, Nk, msb, msh);
    const int64_t grid = (int64_t)m.Bs * m.Hs * m.nqb * m.nkw;
    hipLaunchKernelGGL(fa_mask_blocks_kernel, dim3((unsigned)grid), dim3(kMapThreads), 0, stream, mask, m.Hs, Nq,
                       Nk, msb, msh, ldm, m.nqb, m.nkw, blocks);
    return hipGetLastError();
}

// General masks.  Arguments validated by the caller: Nq, Nk >= 1; wl, wr are
// the window bounds (< 0 = unbounded); causal limits the right bound to 0;
// blocks, if not null, is the mask's block map (mask_blocks_dispatch).
hipError_t fwd_ext_dispatch(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                            int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int wl,
                            int wr, const uint8_t *mask, int64_t msb, int64_t msh, int ldm,
                            const uint32_t *blocks, int dtype, hipStream_t stream)
{
    // bounds beyond Nq + Nk are unbounded; keep every sum inside int
    const int big = Nq + Nk;
    int r = wr < 0 ? big : min(wr, big);
    if (causal) r = min(r, 0);
    const int l = wl < 0 ? big : min(wl, big);
    const MapShape m = map_shape(B, H, Nq, Nk, msb, msh);
    const FwdExt ext{Nk, Nk - Nq, l, r, mask, msb, msh, ldm, mask ? blocks : nullptr, m.nkw, m.bmb, m.bmh};
    switch (dtype) {
    case 0:
        return d == 64 ? launch_fwd_ext<float, 64>(q, k, v, o, lse, B, H, Hkv, Nq, scale, ext, stream)
                       : launch_fwd_ext<float, 128>(q, k, v, o, lse, B, H, Hkv, Nq, scale, ext, stream);
    case 1:
        return d == 64 ? launch_fwd_ext<__bf16, 64>(q, k, v, o, lse, B, H, Hkv, Nq, scale, ext, stream)
                       : launch_fwd_ext<__bf16, 128>(q, k, v, o, lse, B, H, Hkv, Nq, scale, ext, stream);
    default:
        return d == 64 ? launch_fwd_ext<_Float16, 64>(q, k, v, o, lse, B, H, Hkv, Nq, scale, ext, stream)
                       : launch_fwd_ext<_Float16, 128>(q, k, v, o, lse, B, H, Hkv, Nq, scale, ext, stream);
    }
}

// Chunked prefill over the paged cache (EXT 4).  Arguments validated by the
// caller: dtype 1/2, head size 128, block size 16, one cache below 4 GiB,
// Nq + 16 * mbps < 2^29.
hipError_t fwd_paged_dispatch(const void *q, const void *kc, const void *vc, const int32_t *tables,
                              const int32_t *ctx_lens, float *o, float *lse, int S, int H, int Hkv,
                              int Nq, int mbps, uint64_t cache_bytes, float scale, int causal,
                              int dtype, hipStream_t stream)
{
    const int big = Nq + 16 * mbps;  // beyond every row's reach: unbounded
    const FwdExt ext{0, 0, big, causal ? 0 : big, nullptr, 0, 0, 0, nullptr, 0, 0, 0,
                     tables, ctx_lens, mbps, (uint32_t)cache_bytes};
    const int nqt = (Nq + 127) / 128;
    const dim3 grid((unsigned)((int64_t)S * H * nqt));
    if (dtype == 2)
        hipLaunchKernelGGL((fa_fwd_kernel<_Float16, 128, false, 4>), grid, dim3(256), 0, stream,
                           (const _Float16 *)q, (const _Float16 *)kc, (const _Float16 *)vc, o, lse, Nq, nqt,
                           scale, H, H / Hkv, ext);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<__bf16, 128, false, 4>), grid, dim3(256), 0, stream,
                           (const __bf16 *)q, (const __bf16 *)kc, (const __bf16 *)vc, o, lse, Nq, nqt, scale,
                           H, H / Hkv, ext);
    return hipGetLastError();
}

}  // namespace fa
