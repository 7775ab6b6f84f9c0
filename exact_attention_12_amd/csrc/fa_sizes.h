// fa_sizes.h -- host-side sizes shared by the kernels' dispatch code and the
// C ABI's validation: workspace bytes of the paged decode and the backward
// pass, and the shape of a boolean mask's block map.  Plain C++ (no device
// code), so the argument checks can also be built on their own.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

// Paged decode: per-partition partials O_p [S, H, P, 128] fp32, then m_p and
// l_p [S, H, P] fp32, each section rounded up to 256 bytes;
// P = ceil(max_context_len / FA_DECODE_PARTITION_TOKENS), at least 1.
inline size_t decode_workspace_bytes(int num_seqs, int num_heads, int max_context_len)
{
    const int64_t np = (max_context_len + FA_DECODE_PARTITION_TOKENS - 1) / FA_DECODE_PARTITION_TOKENS;
    const int64_t parts = (int64_t)num_seqs * num_heads * (np > 0 ? np : 1);
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    return (size_t)(up(parts * 128 * 4) + 2 * up(parts * 4));
}

// Backward: lse * log2(e) and D = dO . O, one fp32 each per query row.
inline size_t bwd_workspace_bytes(int B, int H, int N)
{
    const size_t rows = (size_t)B * H * N;
    return ((2 * rows * sizeof(float)) + 255) / 256 * 256;
}

// Block map of a mask: query blocks of kMapRows rows, key blocks of kMapCols
// keys, 32 key blocks per word; the map of slice (b, h) is shared along a
// dimension the mask broadcasts over.
constexpr int kMapRows = FA_MASK_BLOCK_ROWS, kMapCols = FA_MASK_BLOCK_COLS;
struct MapShape {
    int nqb, nkw, Bs, Hs;
    int64_t bmb, bmh;  // word strides between batches and heads (0: broadcast)
};
inline MapShape map_shape(int B, int H, int Nq, int Nk, int64_t msb, int64_t msh)
{
    MapShape m;
    m.nqb = (Nq + kMapRows - 1) / kMapRows;
    m.nkw = ((Nk + kMapCols - 1) / kMapCols + 31) / 32;
    m.Bs = msb ? B : 1;
    m.Hs = msh ? H : 1;
    m.bmh = msh ? (int64_t)m.nqb * 2 * m.nkw : 0;
    m.bmb = msb ? (int64_t)m.Hs * m.nqb * 2 * m.nkw : 0;
    return m;
}
inline size_t mask_blocks_words(int B, int H, int Nq, int Nk, int64_t msb, int64_t msh)
{
    const MapShape m = map_shape(B, H, Nq, Nk, msb, msh);
    return (size_t)m.Bs * m.Hs * m.nqb * 2 * m.nkw;
}

}  // namespace fa
