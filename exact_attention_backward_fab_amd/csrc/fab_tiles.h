// fab_tiles.h -- bf16 tiles in the layout shared by the packing kernels and the
// matrix-core kernels of libfab (gfx950), and the LDS access helpers for them.
#pragma once

#include "fab_common.h"

namespace fab {

// The bf16 copies of K, V, Q and dO are stored as tiles of 64 rows, each tile as its
// 16-byte chunk columns one after the other: chunk c (head-dim columns 8c..8c+7)
// of row r of a tile lies at byte c * 1024 + r * 16 of the tile.  One chunk column
// is thus 1 KiB of contiguous memory, the unit the global -> LDS copies move.  In
// LDS each chunk column gets 128 bytes of padding (stride kChunkL), so that
//   * 16-byte row reads (matrix-core operands with one row per lane) are a
//     contiguous 512-byte run per lane half, and
//   * transposing 8-byte reads (ds_read_b64_tr_b16) of 4 rows x 4 chunk columns
//     hit every LDS bank exactly twice,
// and every address in a step is a per-lane base plus a compile-time offset.
constexpr int kTR = 64;              // rows per tile
constexpr int kChunkG = 1024;        // bytes per chunk column of a tile, global memory
constexpr int kChunkL = 1152;        // ... in LDS

// Element offset of (row, column c) in one head of tiles with DP columns.
__host__ __device__ __forceinline__ size_t tile_elem(int row, int c, int DP)
{
    return (size_t)(row >> 6) * 64 * DP + (size_t)(c >> 3) * 512 + (size_t)(row & 63) * 8 + (c & 7);
}

// Per-query statistics of the backward, one block of 128 floats per 64-query tile:
// [0, 64) the row LSE in log2 units (+inf where the row has no weight: all-masked
// or past N), [64, 128) D = rowsum(dO o O).
constexpr int kStatsTile = 128;

// dS^T tiles (written by the dK/dV kernel, read by the dQ product): 64 key rows
// per tile and the 64 queries of a step as 8 chunk columns.  Chunk c = 4 qq +
// 2 u + half holds, at position e, the dS value of query 32 qq + 16 u + 8 (e >> 2)
// + 4 half + (e & 3) -- the matrix-core k order in which the dK product consumes
// it.  Column p = 8 c + e is thus query p with bits 2 and 3 swapped.
__host__ __device__ __forceinline__ int ds_query(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// Per-lane byte offsets inside an LDS tile (see the tile layout above):
//   row operand   16 bytes of row l32 (+32 kk), chunk column 2t + half:
//                 row_off + 512 kk + 2304 t
//   transposed    rows 16u + 4 half + (j >> 2) (+32 kk, +8 for the upper 4 slots),
//                 columns 32 dt + 16 grp + 4 (j & 3), j = lane & 15, grp = bit 4 of
//                 the lane: tr_off + 4608 dt + 512 kk + 256 u (+128)
__device__ __forceinline__ int tile_row_off(int lane) { return (lane >> 5) * kChunkL + (lane & 31) * 16; }
__device__ __forceinline__ int tile_tr_off(int lane)
{
    const int j = lane & 15, grp = (lane >> 4) & 1, half = lane >> 5;
    return (2 * grp + ((j & 3) >> 1)) * kChunkL + ((j >> 2) + 4 * half) * 16 + (j & 1) * 8;
}
__device__ __forceinline__ bf16x8 lds_row8(const char *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x8 lds_tr8(const char *p)
{
    const bf16x4 lo = lds_read_tr16(reinterpret_cast<const __bf16 *>(p));
    const bf16x4 hi = lds_read_tr16(reinterpret_cast<const __bf16 *>(p + 128));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One 16-byte global -> LDS copy per lane (buffer_load_dwordx4 ... lds): lane i
// writes LDS bytes [la + 16 i, la + 16 i + 16); la must be wave-uniform.  Issued
// as inline assembly so that the compiler does not make every later LDS read wait
// for it; the caller orders it with explicit vmcnt waits and barriers.  The copy
// takes its LDS address from m0: the asm saves m0, sets it (the copy reads it one
// wait state later, at issue) and restores it, so whatever the compiler keeps in
// m0 is unchanged across the statement and m0 is not a clobber.  The asm writes no
// VGPR (the data goes to LDS), so no register is left pending on the load.
// NT: the non-temporal policy, for data read once (it streams past the L2 instead
// of displacing lines that other reads reuse).
template <bool NT = false>
__device__ __forceinline__ void lds_copy16(rsrc_t r, uint32_t la, uint32_t voff)
{
    uint32_t saved;
    if constexpr (NT)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "s"(la), "v"(voff), "s"(r) : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "s"(la), "v"(voff), "s"(r) : "memory");
}

// Waits until at most k * PER of this wave's vector-memory operations are in flight.
template <int PER>
__device__ __forceinline__ void wait_vm_steps(int k)
{
    static_assert(3 * PER <= 63, "vmcnt range");
    if (k <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (k == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PER) : "memory");
    else if (k == 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * PER) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(3 * PER) : "memory");
}

}  // namespace fab
