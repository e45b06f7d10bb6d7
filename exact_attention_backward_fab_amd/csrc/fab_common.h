// fab_common.h -- device-side building blocks shared by the libfab kernels
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fab {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Block-map classes of a 32x32 (query x key) block of the additive mask.
enum : uint8_t { kBlockSkip = 0, kBlockFree = 1, kBlockMixed = 2 };
constexpr int kMapTile = 32;

// ---------------------------------------------------------------- MFMA
// 32x32 output tile C[i][j] (i = row, j = column) as held by a wave64:
//   lane l holds column j = l & 31 and, in accumulator slot r = 0..15,
//   row i = 8*(r>>2) + 4*(l>>5) + (r&3).
// The A operand (32 x K) gives each lane one row (l & 31), the B operand
// (K x 32) one column (l & 31); both spread K over the lane half (l >> 5) and
// the lane's slots.  Which k a (half, slot) pair denotes is the same for A and
// B, so any fixed k-permutation used consistently on both sides is correct.
__device__ __forceinline__ int crow(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16()
{
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Round-to-nearest-even f32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 to_bf16x8(const float *x)
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
    return r;
}

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4 &x)
{
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (__bf16)x[i];
    return r;
}

// ---------------------------------------------------------------- loads
// Four consecutive floats row[c..c+3] of a row of length D; entries at or past
// D read as 0.  vec: D % 4 == 0 and the row start is 16-byte aligned.
__device__ __forceinline__ f32x4 load_row4(const float *row, int c, int D, bool vec)
{
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    if (c >= D) return r;
    if (vec) return *reinterpret_cast<const f32x4 *>(row + c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (c + i < D) r[i] = row[c + i];
    return r;
}

// Additive f16 mask value (as f32) from its bit pattern.
__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- reductions
// Butterfly sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float x, int width)
{
    for (int off = width >> 1; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ float swap_halves_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float swap_halves_sum(float x) { return x + __shfl_xor(x, 32, 64); }

}  // namespace fab
