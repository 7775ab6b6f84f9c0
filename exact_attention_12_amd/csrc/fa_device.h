// fa_device.h -- device-side building blocks for gfx950 (CDNA4): vector
// types, the matrix-core (MFMA) operand traits per element type, and small
// wave-level helpers.  Included only by the .hip sources of libfa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// log2(e): exp(x) = 2^(x * log2 e); the hardware exponential is base 2.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware transcendental unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// Matrix-core traits.  One 32x32 output tile per instruction; the contraction
// depth per instruction is 2*KW, and every lane supplies KW consecutive
// k-elements of one A row / one B column:
//   A (32 x 2KW): lane l holds A[l % 32][KW*(l/32) .. KW*(l/32)+KW-1]
//   B (2KW x 32): lane l holds B[KW*(l/32) .. +KW-1][l % 32]
//   C (32 x 32) : lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
// 16-bit types use v_mfma_f32_32x32x16_{bf16,f16} (KW = 8, one 16-byte
// fragment per lane); fp32 uses v_mfma_f32_32x32x2_f32 (KW = 1).
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
    static constexpr int KW = 8;
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // 8 fp32 -> 8 bf16, round to nearest even (v_cvt_pk_bf16_f32)
    static __device__ __forceinline__ frag pack(const float *x)
    {
        frag r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
        return r;
    }
    // two fp32 -> two bf16 in one 32-bit word (round to nearest even)
    static __device__ __forceinline__ uint32_t pack2(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
    }
    // acc + the two values of a packed word
    static __device__ __forceinline__ float sum2(uint32_t w, float acc)
    {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
    }
    // acc + (sum of the 8 rounded values), two at a time (v_dot2 with 1, 1)
    static __device__ __forceinline__ float sum(frag x, float acc)
    {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[2 * i], x[2 * i + 1]}, one, acc, false);
        return acc;
    }
};

template <> struct Mma<_Float16> {
    static constexpr int KW = 8;
    typedef f16x8 frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag pack(const float *x)
    {
        frag r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (_Float16)x[i];
        return r;
    }
    static __device__ __forceinline__ uint32_t pack2(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
    }
    static __device__ __forceinline__ float sum2(uint32_t w, float acc)
    {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
    }
    static __device__ __forceinline__ float sum(frag x, float acc)
    {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(f16x2{x[2 * i], x[2 * i + 1]}, one, acc, false);
        return acc;
    }
};

template <> struct Mma<float> {
    static constexpr int KW = 1;
    typedef float frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag pack(const float *x) { return x[0]; }
    static __device__ __forceinline__ float sum(frag x, float acc) { return acc + x; }
};

// Row (within a 32-row tile) held by lane-half h in accumulator register r.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r / 4) + 4 * h + r % 4; }

// The two lane halves exchange a value: both halves get op(x[l % 32],
// x[l % 32 + 32]) with the operands in the same order, so the result is
// bitwise the same in both.
__device__ __forceinline__ void lane_halves(float x, float &lo, float &hi)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float halves_max(float x)
{
    float lo, hi;
    lane_halves(x, lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float halves_sum(float x)
{
    float lo, hi;
    lane_halves(x, lo, hi);
    return lo + hi;
}

// Debug builds (compiled with FA_DEBUG_POISON): fill an LDS array with 0xff
// bytes -- NaN as fp32, bf16 and fp16 -- and wait for the whole workgroup,
// before the kernel's first LDS write.  A later read of a slot that this
// launch never wrote then yields NaN instead of whatever an earlier
// workgroup left there.  Every thread of the workgroup must call it (no
// thread may have returned).  A no-op in the product build.
__device__ __forceinline__ void poison_lds(void *p, int bytes)
{
#ifdef FA_DEBUG_POISON
    const int nthreads = (int)(blockDim.x * blockDim.y * blockDim.z);
    for (int i = (int)threadIdx.x; i < bytes / 4; i += nthreads) ((uint32_t *)p)[i] = 0xffffffffu;
    __syncthreads();
#else
    (void)p;
    (void)bytes;
#endif
}

}  // namespace fa
