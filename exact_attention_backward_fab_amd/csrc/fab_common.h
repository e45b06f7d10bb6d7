// fab_common.h -- device-side building blocks shared by the libfab kernels
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fab_launch.h"

namespace fab {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Block map of the additive mask, one byte per 32x32 (query x key) block:
// bits 0-1 the block class, bit 2 set when every entry of the block equals the
// causal rule (0 where key <= query, -inf elsewhere).
enum : uint8_t { kBlockSkip = 0, kBlockFree = 1, kBlockMixed = 2, kBlockCausalBit = 4 };
// Classes of a kernel tile (a rectangle of map blocks).
enum : int { kTileSkip = 0, kTileFree = 1, kTileMixed = 2, kTileCausal = 3 };
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

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j addresses 4 consecutive 16-bit elements; lane i then receives, in
// slot k, element (i & 3) of the 4 read by lane 4k + (i >> 2).  When lane j of
// the group points at row r0 + (j >> 2), column c0 + 4 (j & 3) of a row-major
// matrix X, lane i receives X[r0 + k][c0 + i] for k = 0..3: four consecutive
// rows of one column, the operand shape of a matrix-core B (or A) fragment.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16 *p)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Matrix-core operand of 8 bf16 for the lane's column c0 + (l & 31) of a
// row-major LDS matrix X (leading dimension ld): rows r0..r0+3 in slots 0-3 and
// r0+dr..r0+dr+3 in slots 4-7.
__device__ __forceinline__ bf16x8 lds_col8(const __bf16 *X, int ld, int r0, int dr, int c0, int lane)
{
    const int j = lane & 15, grp = (lane >> 4) & 1;
    const __bf16 *p = X + (r0 + (j >> 2)) * ld + c0 + 16 * grp + 4 * (j & 3);
    const bf16x4 lo = lds_read_tr16(p);
    const bf16x4 hi = lds_read_tr16(p + dr * ld);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- buffer access
// Raw buffer resources: accesses past num_bytes read as zero and writes or
// atomics past it are dropped by the hardware, so tiles that run over the end
// of a (batch, head) slice need no bounds checks.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw 32-bit buffer, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t num_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, num_bytes, kRsrcFlags);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u16(rsrc_t r, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ void buf_atomic_add_f32(rsrc_t r, uint32_t byte_off, float v)
{
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, byte_off, 0, 0);
}
// A 16-byte store either through the caches (cached) or streamed past the L2
// (the nontemporal cache policy, immediate 2).  The two are separate intrinsic calls
// with different immediates, so the compiler cannot merge them into one store with
// the policy dropped (as it does with a nontemporal and a plain store of one value).
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t byte_off, const bf16x8 &v, bool cached)
{
    const u32x4 x = __builtin_bit_cast(u32x4, v);
    if (cached) __builtin_amdgcn_raw_buffer_store_b128(x, r, byte_off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b128(x, r, byte_off, 0, 2);
}

// ---------------------------------------------------------------- LDS tile layouts
// Row-major bf16 tiles of D columns, stored without padding; the 16-byte chunks
// of each row are permuted by an XOR with a function of (row mod 16), chosen so
// that the two access patterns on these tiles hit distinct LDS banks: 16
// consecutive rows reading the same chunk (one row per lane, 16-byte reads) and
// 4 consecutive rows x 4 consecutive chunks (transposing reads).  The same
// permutation is applied by the bf16 pack kernels to rows in global memory, so
// a tile can be copied linearly from global memory into LDS.
//   D = 128 (16 chunks):      chunk ^ (4 (row & 3) + ((row >> 2) & 3))
//   D = 64, 192 (8k chunks):  within each group of 8: chunk ^ f((row >> 1) & 7),
//                             f(x) = 4 (x & 1) + (x >> 1)
//   D = 32 (4 chunks):        chunk ^ ((row >> 2) & 3)
__host__ __device__ __forceinline__ int swz_chunk(int row, int chunk, int nchunks)
{
    if (nchunks == 16) return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
    if (nchunks == 4) return chunk ^ ((row >> 2) & 3);
    const int x = (row >> 1) & 7;
    return (chunk & ~7) | ((chunk & 7) ^ (((x & 1) << 2) | (x >> 1)));
}

template <int D>
struct RowTile {
    static constexpr int kLd = D;   // elements per row
    // element offset of (row, col); col is a multiple of 4
    __device__ static __forceinline__ int off(int row, int col)
    {
        return row * kLd + (swz_chunk(row, col >> 3, D / 8) << 3) + (col & 7);
    }
};

// Matrix-core operand of 8 bf16 for the lane's column c0 + (lane & 31) of a
// row-major LDS tile: rows r0..r0+3 in slots 0-3, rows r0+dr..r0+dr+3 in slots 4-7.
template <typename Layout>
__device__ __forceinline__ bf16x8 tile_col8(const __bf16 *X, int r0, int dr, int c0, int lane)
{
    const int j = lane & 15, grp = (lane >> 4) & 1;
    const int col = c0 + 16 * grp + 4 * (j & 3);
    const bf16x4 lo = lds_read_tr16(X + Layout::off(r0 + (j >> 2), col));
    const bf16x4 hi = lds_read_tr16(X + Layout::off(r0 + dr + (j >> 2), col));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// dS^T tile [key][query] with BR = 32 queries per row (64 bytes): chunk' = chunk ^ ((row >> 2) & 3).
struct StTile {
    static constexpr int kLd = 32;
    __device__ static __forceinline__ int off(int row, int col)
    {
        return row * kLd + ((((col >> 3) ^ ((row >> 2) & 3))) << 3) + (col & 7);
    }
};

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

// The same from a row of bf16 values (widened to f32, exactly); vec: D % 4 == 0
// (8-byte loads).
__device__ __forceinline__ f32x4 load_row4(const __bf16 *row, int c, int D, bool vec)
{
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    if (c >= D) return r;
    if (vec) {
        const bf16x4 x = *reinterpret_cast<const bf16x4 *>(row + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (float)x[i];
        return r;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (c + i < D) r[i] = (float)row[c + i];
    return r;
}

// The same from a row of IEEE binary16 values (widened to f32, exactly).
__device__ __forceinline__ f32x4 load_row4(const _Float16 *row, int c, int D, bool vec)
{
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    if (c >= D) return r;
    if (vec) {
        const f16x4 x = *reinterpret_cast<const f16x4 *>(row + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (float)x[i];
        return r;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (c + i < D) r[i] = (float)row[c + i];
    return r;
}

// Row m of a tensor of f32, bf16 or f16 elements (fmt), elem_off elements past base:
// four entries from column c, as f32 (the 16-bit forms widened exactly).
__device__ __forceinline__ f32x4 load_row4_any(const void *base, int64_t elem_off, int c, int D, bool vec, int fmt)
{
    if (fmt == kBF16) return load_row4(static_cast<const __bf16 *>(base) + elem_off, c, D, vec);
    if (fmt == kF16) return load_row4(static_cast<const _Float16 *>(base) + elem_off, c, D, vec);
    return load_row4(static_cast<const float *>(base) + elem_off, c, D, vec);
}

// Additive f16 mask value (as f32) from its bit pattern.
__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// The mask [N][M] (f16 bits) as a buffer resource: it holds below 2^31 entries, so its
// byte offsets fit 32 bits.
__device__ __forceinline__ rsrc_t mask_rsrc(const uint16_t *mask, int N, int M)
{
    return make_rsrc(mask, mask ? (uint32_t)((size_t)N * M * 2u) : 0u);
}

// Key-outer kernels (C layout of S with one key per lane): adds, in log2 units, the
// mask entries of the lane's key and the 16 queries q0 + crow(r, half) to s[r].
// All 16 loads are issued before the first is used, so one latency is paid, not 16;
// indices are clamped to the mask (entries past N or M carry no weight anyway).
__device__ __forceinline__ void add_mask_column(f32x16 &s, rsrc_t rmask, int key, int q0, int half, int N, int M)
{
    const uint32_t kofs = 2u * (uint32_t)min(key, M - 1);
    uint32_t mk[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        mk[r] = buf_load_u16(rmask, 2u * (uint32_t)M * (uint32_t)min(q0 + crow(r, half), N - 1) + kofs);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += half_bits_to_float((uint16_t)mk[r]) * kLog2e;
}

// Work-groups that meet on a shared result exchange partial results through
// global memory with device-coherent accesses (agent-scope atomic stores and
// loads, which bypass the non-coherent caches).  Every wave waits for its own
// stores (s_waitcnt vmcnt(0)) before the work-group barrier; one lane then takes
// the result's ticket with an agent-scope acquire-release add, which orders the
// work-group's partial stores (made visible to it by the barrier) before the
// ticket, and the ticket before the loads of the other work-group's partial that
// follow the next barrier.
__device__ __forceinline__ void coherent_store(float *p, float x)
{
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ticket_take(int *t)
{
    return __hip_atomic_fetch_add(t, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- work order
// Work-group -> (query block, head) of the query-block-outer kernels.  Heads are
// dealt to the XCDs in contiguous ranges (a work-group's XCD is its index mod 8),
// so the heads of a key/value group share that XCD's L2.  Query blocks go latest
// first: under a causal mask those see the most keys, so on a grid of several
// rounds the longest blocks start first.  When the whole grid is resident at once
// (fold), the dispatcher gives every CU its first work-group before any its
// second, so the second half of the order shares CUs with the first; running
// that half from the earliest block up puts long and short blocks together on a
// CU.
__device__ __forceinline__ void query_block_work(int bid, int nqt, int HB, int fold, int *qt, int *hb)
{
    int sl;
    if (HB % 8 == 0) {
        const int xcd = bid % 8, j = bid / 8, per = HB / 8;
        sl = j / per;
        *hb = xcd * per + j % per;
    } else {
        sl = bid / HB;
        *hb = bid % HB;
    }
    const int hn = (nqt + 1) / 2;
    *qt = (!fold || sl < hn) ? nqt - 1 - sl : sl - hn;
}

// ---------------------------------------------------------------- result stores
// A result slice holds f32 elements, or 16-bit ones (kBF16 / kF16) rounded to
// nearest even from the f32 value.  The 16-bit bits of x in format fmt:
__device__ __forceinline__ uint16_t result_bits16(float x, int fmt)
{
    // x as an f32 value in a register: without this the compiler may fuse the
    // product or sum that made x into one mixed-precision operation that rounds
    // the exact result to 16 bits once (no longer the f32 value rounded)
    asm("" : "+v"(x));
    const __bf16 b = (__bf16)x;
    const _Float16 h = (_Float16)x;
    return fmt == kF16 ? __builtin_bit_cast(uint16_t, h) : __builtin_bit_cast(uint16_t, b);
}
// Element i of a result slice at base.  W16 (compile time): 16-bit elements of
// format fmt (the choice between the two is a select, not a branch); else f32.
template <bool W16>
__device__ __forceinline__ void store_as(float *base, size_t i, float x, int fmt)
{
    if constexpr (W16)
        reinterpret_cast<uint16_t *>(base)[i] = result_bits16(x, fmt);
    else
        base[i] = x;
}
// fn(std::bool_constant<W16>) with W16 = (fmt is a 16-bit format): a store loop
// inside fn is compiled once per element width and carries no per-element branch.
template <class Fn>
__device__ __forceinline__ void with_result_width(int fmt, Fn &&fn)
{
    if (fmt == kF32)
        fn(std::bool_constant<false>{});
    else
        fn(std::bool_constant<true>{});
}
// The same with the width chosen at run time (single stores off the hot loops).
__device__ __forceinline__ void store_result(float *base, size_t i, float x, int fmt)
{
    if (fmt == kF32)
        base[i] = x;
    else
        reinterpret_cast<uint16_t *>(base)[i] = result_bits16(x, fmt);
}
// Elements 4 q .. 4 q + 3 (16-byte aligned for f32, 8-byte for 16-bit elements).
__device__ __forceinline__ void store_result4(float *base, size_t q, f32x4 x, int fmt)
{
    if (fmt == kF32) {
        reinterpret_cast<f32x4 *>(base)[q] = x;
        return;
    }
    asm("" : "+v"(x));   // the f32 sums themselves are rounded (see result_bits16)
    if (fmt == kBF16) {
        reinterpret_cast<bf16x4 *>(base)[q] = to_bf16x4(x);
    } else {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        reinterpret_cast<f16x4 *>(base)[q] = f16x4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    }
}

// ---------------------------------------------------------------- grouped-query reduction
// Item i of a ReduceJob (fab_launch.h): the sum of the rk2 partials of a group
// (one per head unit) of one float4 (or float) of a key/value head's dK or dV
// slice, in head order.
__device__ __forceinline__ void reduce_item(const ReduceJob &r, int rk2, int64_t i)
{
    if (r.vec) {
        const int64_t c4 = r.chunk / 4, gb = i / c4, off = i - gb * c4;
        const f32x4 *src = reinterpret_cast<const f32x4 *>(r.part) + gb * rk2 * c4 + off;
        f32x4 s = src[0];
        for (int k = 1; k < rk2; ++k) s += src[k * c4];
        store_result4(r.dst, (size_t)i, s, r.out_fmt);
    } else {
        const int64_t gb = i / r.chunk, off = i - gb * r.chunk;
        const float *src = r.part + gb * rk2 * r.chunk + off;
        float s = src[0];
        for (int k = 1; k < rk2; ++k) s += src[k * r.chunk];
        store_result(r.dst, (size_t)i, s, r.out_fmt);
    }
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

// Class of a kernel tile made of NQ x NK map blocks starting at (qb0, kb0):
// SKIP if every block is all -inf, FREE if every block is all zero, CAUSAL if
// every block follows the causal rule exactly, MIXED otherwise; blocks past the
// map's extent do not count.  Without a map: FREE, or with the causal flag (the
// pages' boolean mask: key m is seen by query n iff m <= n) the same classes from
// the tile's extent alone, counted over the queries < N and keys < M as the map
// counts them.  The map bytes of a tile are loaded together (one latency).
template <int NQ, int NK>
__device__ __forceinline__ int tile_class(const uint8_t *map, int causal, int N, int M, int nqb, int nkb, int qb0,
                                          int kb0)
{
    if (!map) {
        if (!causal) return kTileFree;
        const int qlo = kMapTile * qb0, qhi = min(kMapTile * (qb0 + NQ), N) - 1;
        const int klo = kMapTile * kb0, khi = min(kMapTile * (kb0 + NK), M) - 1;
        if (qlo > qhi || klo > khi || klo > qhi) return kTileSkip;   // no pair, or every key after every query
        if (khi <= qlo) return kTileFree;
        return kTileCausal;
    }
    uint8_t c[NQ][NK];
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const bool in = qb0 + i < nqb && kb0 + j < nkb;
            // a block outside the map counts as SKIP, FREE and causal at once
            c[i][j] = in ? map[(qb0 + i) * nkb + kb0 + j] : (uint8_t)0xFF;
        }
    bool all_skip = true, all_free = true, all_causal = true;
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const uint8_t x = c[i][j];
            const bool out = x == 0xFF;
            all_skip = all_skip && (out || (x & 3) == kBlockSkip);
            all_free = all_free && (out || (x & 3) == kBlockFree);
            all_causal = all_causal && (out || (x & kBlockCausalBit) != 0);
        }
    if (all_skip) return kTileSkip;
    if (all_free) return kTileFree;
    return all_causal ? kTileCausal : kTileMixed;
}

// Ordered list of the live (not SKIP) tiles lo..hi-1 of a work-group of W waves:
// sList[i] = 4 * tile + class for the i-th live tile; returns their number.
// class_of(tile) gives a tile's class.  sCount holds W + 1 ints.  Every thread
// of the work-group must call it; it synchronises the work-group on entry, so
// a previous list may be read up to the call.
template <int W, typename ClassOf>
__device__ __forceinline__ int build_live_list(int *sList, int *sCount, int lo, int hi, int tid, int lane, int w,
                                               ClassOf class_of)
{
    constexpr int NT = 64 * W;
    __syncthreads();
    if (tid == 0) sCount[W] = 0;
    __syncthreads();
    for (int c0 = lo; c0 < hi; c0 += NT) {
        const int it = c0 + tid;
        const int cls = it < hi ? class_of(it) : (int)kTileSkip;
        const bool live = cls != kTileSkip;
        const uint64_t ball = __ballot(live);
        const int before = __popcll(ball & ((1ull << lane) - 1ull));
        if (lane == 0) sCount[w] = __popcll(ball);
        __syncthreads();
        int base = sCount[W];
        for (int v = 0; v < w; ++v) base += sCount[v];
        if (live) sList[base + before] = 4 * it + cls;
        __syncthreads();
        if (tid == 0) {
            int t = sCount[W];
            for (int v = 0; v < W; ++v) t += sCount[v];
            sCount[W] = t;
        }
        __syncthreads();
    }
    return sCount[W];
}

}  // namespace fab
