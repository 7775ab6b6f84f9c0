// fa_tile.h -- LDS tile format shared by the forward and backward kernels:
// row-major tiles of [rows][d] 16-bit (or fp32) elements, filled straight
// from global memory by 16-byte direct-to-LDS buffer loads, with an XOR
// swizzle of the 16-byte chunks of each row.  Two read patterns are served
// without bank conflicts: the row-fragment read (lane r % 32 reads 16 bytes
// of row r) and the 8-byte transpose read (ds_read_b64_tr_b16) that turns
// row-major data into a column operand.
#pragma once

#include "fa_device.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle: the 16-byte chunk c of LDS row r is stored at position
// c ^ swz(r).  LDS serves a 16-byte read 16 lanes per pass and an 8-byte read
// 32 lanes per pass, 64 banks of 4 bytes each.  The form below (found by
// exhaustive search over XOR-of-shifted-row-bit forms under that model)
// gives both read patterns the minimum number of passes: the row-fragment
// read (16 consecutive rows, one chunk) and the transpose read (4 rows x 4
// chunks per 32 lanes).  It depends on the row only through row % 16.
template <int CPR, int ES> __device__ __forceinline__ int swz(int row)
{
    if constexpr (ES == 2)
        return CPR >= 16 ? (((row & 3) << 2) ^ ((row >> 2) & 3)) : (((row & 3) << 1) ^ ((row >> 2) & 3));
    else
        return row & 15;
}

// Buffer resource word 3 for raw (unformatted, unswizzled) byte addressing.
constexpr int kBufferFlags = 0x00020000;

// 16 bytes per lane from buffer r at byte offset voff + soff into LDS at
// lds + 16 * lane (the LDS base must be the same for the whole wave).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, char *lds, int voff,
                                                  int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}

// 4 bytes per lane from buffer r at byte offset voff + soff into LDS at
// lds + 4 * lane.
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, char *lds, int voff,
                                                 int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 4, voff, soff, 0, 0);
}

}  // namespace fa
