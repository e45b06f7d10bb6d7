// fab_launch.h -- host-side launch interface between the C ABI (fab_api.cpp)
// and the kernels (fab_aux.hip, fab_fwd.hip, fab_bwd.hip, fab_qouter.hip).
// Internal to libfab.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fab {

// Storage formats of an input tensor.
constexpr int kF32 = 0, kBF16 = 1, kF16 = 2;

struct Dims {
    int B, H, Hkv, N, M, DK, DV;
    int causal = 0;   // the mask is the causal rule (key m seen by query n iff m <= n), given as a flag
    int in_fmt = 0;   // storage of q, k, v and d: kF32, kBF16 or kF16 (the 16-bit forms in bf16 mode only)
    int o_bf16 = 0;   // O is bf16 (bf16 mode only): written so by the forward, read so by the prep
    int out_fmt = 0;  // element type of the result blob: kF32, or kBF16 / kF16 (bf16 mode only)
    const float *alibi = nullptr;   // per-query-head ALiBi slopes [H] (device) or NULL: score += slope_h (m - n)
};

// Padded head dimensions (DKP, DVP) the kernels are instantiated for; a shape
// uses the first pair that covers both of its head dims.
struct HeadDims {
    int dk, dv;
};
constexpr HeadDims kHeadDims[] = {{32, 32}, {64, 64}, {128, 128}, {192, 128}, {192, 192}, {256, 256}};

// Work-groups of one kernel (no dynamic LDS, `threads` per group) that the
// current device holds resident at once: occupancy per CU times the CU count,
// asked of the runtime once per device and kept; 0 if the runtime cannot say.
struct ResidentCache {
    static constexpr int kDevices = 16;
    std::atomic<int> n[kDevices] = {};
    int get(const void *kernel, int threads)
    {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
        if (dev < kDevices) {
            const int c = n[dev].load(std::memory_order_relaxed);
            if (c > 0) return c;
        }
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        const int c = per_cu * cus;
        if (dev < kDevices && c > 0) n[dev].store(c, std::memory_order_relaxed);
        return c;
    }
};

inline bool pick_head_dims(int DK, int DV, HeadDims *out)
{
    for (const HeadDims &h : kHeadDims)
        if (DK <= h.dk && DV <= h.dv) {
            *out = h;
            return true;
        }
    return false;
}

// Calls FN<DKP, DVP, BF16>(ARGS, STREAM) for the instantiated pair HD and
// returns its result.
#define FAB_DISPATCH_HEAD_DIMS(FN, ARGS, STREAM, HD, BF)                                           \
    do {                                                                                          \
        if ((HD).dk == 32 && (HD).dv == 32)                                                       \
            return (BF) ? FN<32, 32, true>(ARGS, STREAM) : FN<32, 32, false>(ARGS, STREAM);       \
        if ((HD).dk == 64 && (HD).dv == 64)                                                       \
            return (BF) ? FN<64, 64, true>(ARGS, STREAM) : FN<64, 64, false>(ARGS, STREAM);       \
        if ((HD).dk == 128 && (HD).dv == 128)                                                     \
            return (BF) ? FN<128, 128, true>(ARGS, STREAM) : FN<128, 128, false>(ARGS, STREAM);   \
        if ((HD).dk == 192 && (HD).dv == 128)                                                     \
            return (BF) ? FN<192, 128, true>(ARGS, STREAM) : FN<192, 128, false>(ARGS, STREAM);   \
        if ((HD).dk == 192 && (HD).dv == 192)                                                     \
            return (BF) ? FN<192, 192, true>(ARGS, STREAM) : FN<192, 192, false>(ARGS, STREAM);   \
        if ((HD).dk == 256 && (HD).dv == 256)                                                     \
            return (BF) ? FN<256, 256, true>(ARGS, STREAM) : FN<256, 256, false>(ARGS, STREAM);   \
        return hipErrorInvalidValue;                                                              \
    } while (0)

// Block map of the additive mask: u8 [ceil(N/32)][ceil(M/32)].
hipError_t launch_block_map(const uint16_t *mask, uint8_t *map, const Dims &d, hipStream_t s);

// Forward with row log-sum-exp (natural log, -inf for all-masked rows): f32
// operands, or bf16 operands read from the packed K / V (launch_pack_qkv, Mp rows
// per head).
hipError_t launch_forward_f32(const float *q, const float *k, const float *v, const uint16_t *mask,
                              const uint8_t *map, float scale, float *O, float *lse, const Dims &d,
                              hipStream_t s);
hipError_t launch_forward_bf16(const void *q, const __bf16 *k16, const __bf16 *v16, const uint16_t *mask,
                               const uint8_t *map, float scale, void *O, float *lse, int Mp, const Dims &d,
                               hipStream_t s);
// The backward's own forward in bf16 mode: instead of O and the LSE it writes
// what the backward kernels read, as launch_pack_prep_bf16 does
// from a stored O and LSE: the bf16 tiles of Q and dO, the LSE/D blocks, the blob
// pads (nq, off_k, nk, off_v, nv, total as there) and nzero zeroed ints.
hipError_t launch_forward_prep_bf16(const void *q, const __bf16 *k16, const __bf16 *v16, const uint16_t *mask,
                                    const uint8_t *map, float scale, const void *dO, __bf16 *q16, __bf16 *o16,
                                    float *stats, float *blob, int64_t nq, int64_t off_k, int64_t nk, int64_t off_v,
                                    int64_t nv, int64_t total, int *zero, int nzero, int Np, int Mp, const Dims &d,
                                    hipStream_t s);

// f32 mode prep: Delta = rowsum(d o O) [N,H,B]; zero the dQ slice [0, off_k)
// (the atomics target) and the other blob pads.
hipError_t launch_prep(const float *dO, const float *O, float *delta, float *blob, int64_t off_k, int64_t nk,
                       int64_t off_v, int64_t nv, int64_t total, const Dims &d, hipStream_t s);

// bf16 mode with O and LSE supplied: launch_pack_qkv's work and the prep, in one
// launch: D and the LSE/D blocks (stats, [B][H][Np/64][128]) from d, O and lse,
// d as bf16 tiles [B][H][Np][DVP] (fab_tiles.h, zero-padded), the pads of the
// result blob zeroed ([nq, off_k), [off_k + nk, off_v), [off_v + nv, total)) and
// nzero ints of zero written.
hipError_t launch_pack_prep_bf16(const void *q, const void *k, const void *v, __bf16 *q16, __bf16 *k16,
                                 __bf16 *v16, const uint16_t *mask, uint8_t *map, const void *dO, const void *O,
                                 const float *lse, __bf16 *dO16, float *stats, float *blob, int64_t nq, int64_t off_k,
                                 int64_t nk, int64_t off_v, int64_t nv, int64_t total, int *zero, int nzero, int Np,
                                 int Mp, const Dims &d, hipStream_t s);

// Rows of the bf16 tiles are padded per head to a multiple of this.
constexpr int kPackRows = 64;

// f32 rows -> bf16 tiles (fab_tiles.h), one launch: q [DK,N,H,B] -> q16 [B,H,Np,DKP]
// (skipped when q is NULL), k / v -> k16 / v16 [B,Hkv,Mp,DKP / DVP]; rows past the
// data and columns past DK / DV zero.  With map, the same launch also builds the
// mask's block map (as launch_block_map).
hipError_t launch_pack_qkv(const void *q, const void *k, const void *v, __bf16 *q16, __bf16 *k16, __bf16 *v16,
                           const uint16_t *mask, uint8_t *map, int Np, int Mp, const Dims &d, hipStream_t s);

// f32-mode dK/dV kernel: keys per work-group (32 per key sub-block of waves: 4
// sub-blocks for head-dim pairs up to 64 + 64, 2 up to 192 + 192, else 1).
constexpr int f32_keys_per_wg(int dkp, int dvp) { return 32 * (dkp + dvp <= 128 ? 4 : dkp + dvp <= 384 ? 2 : 1); }

// Query splits of the f32 dK/dV kernel: below two work-groups per CU (256 CUs: two
// rounds, in which the heaviest-first order balances the causal key blocks), each
// (key block, query head) is run by 2 or 4 work-groups that take interleaved live
// query steps, each with its own dK/dV partial.
inline int f32_query_splits(const Dims &d, int dkp, int dvp)
{
    const int64_t wgs = (int64_t)((d.M + f32_keys_per_wg(dkp, dvp) - 1) / f32_keys_per_wg(dkp, dvp)) * d.H * d.B;
    int qs = 1;
    while (qs < 4 && wgs * qs < 512) qs *= 2;
    return qs;
}

// dK/dV partials per key/value head of the f32 dK/dV kernel: query heads of the
// group times query splits; 1 = no partials (the kernel writes the result).
inline int f32_units_per_group(const Dims &d, int dkp, int dvp) { return d.H / d.Hkv * f32_query_splits(d, dkp, dvp); }

// Key-block-outer backward, f32 mode: dV, dK per key tile and dQ by f32 atomics into
// dq (zeroed beforehand).  With part_heads (f32_units_per_group > 1), one partial per
// unit (query head x query split) into dk/dv [D,M,Hkv*upg,B]; else into dk/dv
// [D,M,Hkv,B].
hipError_t launch_backward_f32(const float *q, const float *k, const float *v, const float *dO,
                               const uint16_t *mask, const uint8_t *map, const float *lse, const float *delta,
                               float scale, float *dq, float *dk, float *dv, int part_heads, const Dims &d,
                               hipStream_t s);

// dQ in bf16 mode comes either from the dS^T tiles the dK/dV kernel stores
// (launch_dq_from_ds: a plain product, no recompute) or, for shapes whose tiles
// would pass kDsMaxBytes, from the query-block-outer kernel that recomputes S and
// dP (launch_dq).  The tiles are bf16, 128 keys x
// 128 queries per (batch, head, query-step pair, key block), dense over all pairs.
constexpr int64_t kDsMaxBytes = int64_t(4) << 30;
inline int64_t ds_bytes(const Dims &d, int Np)
{
    return (int64_t)d.B * d.H * ((Np / 64 + 1) / 2) * ((d.M + 127) / 128) * 32768;
}
// (strictly below 4 GiB: one head's query-step-pair row of tiles, nkb128 * 32 KiB,
// is then below 2^32 bytes too, the range of a buffer resource)
inline bool dq_from_ds(const Dims &d, int Np, int dkp, int dvp)
{
    (void)dkp;
    (void)dvp;   // every head-dim pair: both dK/dV kernels store the tiles
    return ds_bytes(d, Np) < kDsMaxBytes;
}

// Query heads per work-group of the bf16 dK/dV kernel (1 or 2): two heads of one
// group share a work-group, their dK/dV summed in registers, when the one-head grid
// has at least four rounds of work-groups on the 256 CUs (the grouped-query
// partials and the per-work-group set-up then halve at no cost in balance).
inline int bwd_heads_per_wg(const Dims &d, int dkp, int dvp)
{
    const int rk2 = d.H / d.Hkv;
    return (dkp + dvp <= 256 && rk2 % 2 == 0 && (int64_t)((d.M + 127) / 128) * d.H * d.B >= 1024) ? 2 : 1;
}

// Query splits of the 8-wave dK/dV kernel (bf16 mode): on a grid smaller than one
// work-group per CU, each (key block, head unit) is run by qs work-groups that take
// interleaved live query steps, each writing its own dK/dV partial (summed with the
// grouped-query reduction).  The 4-wave kernel of the 192- and 256-wide heads does not split.
inline int bwd_query_splits(const Dims &d, int dkp, int dvp)
{
    if (dkp + dvp > 256) return 1;
    const int64_t wgs = (int64_t)((d.M + 127) / 128) * (d.H / bwd_heads_per_wg(d, dkp, dvp)) * d.B;
    int qs = 1;
    while (qs < 4 && wgs * qs < 256) qs *= 2;
    return qs;
}

// dK/dV partials per key/value head of the bf16 dK/dV kernels: head units (of
// bwd_heads_per_wg query heads) times query splits; 1 = no partials (the kernel
// writes the result).
inline int bwd_units_per_group(const Dims &d, int dkp, int dvp)
{
    return d.H / d.Hkv / bwd_heads_per_wg(d, dkp, dvp) * bwd_query_splits(d, dkp, dvp);
}

// Key-block-outer backward, bf16 mode: dV, dK from the bf16 tiles of Q, dO
// (launch_pack_prep_bf16 or the forward of launch_forward_prep_bf16, Np rows per head), K, V (Mp rows per head)
// and the LSE/D blocks.  With part_heads (bwd_units_per_group > 1), one partial per
// unit into dk/dv [D,M,Hkv*upg,B] (unit = head unit of bwd_heads_per_wg query heads
// times query split); else (a unit covers its group) into dk/dv [D,M,Hkv,B].  With ds (dq_from_ds shapes only) it also stores the
// dS^T tiles of every pair it visits.
hipError_t launch_backward_bf16(const __bf16 *q16, const __bf16 *o16, const float *stats, const __bf16 *k16,
                                const __bf16 *v16, const uint16_t *mask, const uint8_t *map, float scale, float *dk,
                                float *dv, __bf16 *ds, int part_heads, int Np, int Mp, const Dims &d, hipStream_t s);

// dq [DK,N,H,B] = scale dS K from the dS^T tiles of launch_backward_bf16 and the
// bf16 K tiles; every element written once.  With pk (H > Hkv) the same launch
// also runs the grouped-query reduction of launch_gqa_reduce (extra work-groups
// that take the CU slots the short query blocks free).
hipError_t launch_dq_from_ds(const __bf16 *ds, const __bf16 *k16, const uint8_t *map, float scale, float *dq, int Np,
                             int Mp, const float *pk, float *dk, const float *pv, float *dv, int upg, const Dims &d,
                             hipStream_t s);

// dQ work split.  Query blocks have kDqBlock rows.  A grid of at most
// kDqSplitBlocks blocks fills one round of two work-groups per CU on the 256 CUs
// of an MI355X, so the latest (heaviest, when causal) blocks would bound the
// kernel; there each block is run by two work-groups that take alternate live
// key steps and merge their partial sums (dq_part_floats floats of scratch and
// dq_split_blocks zeroed counters).
constexpr int kDqBlock = 128, kDqSplitBlocks = 512;
inline int64_t dq_blocks(const Dims &d) { return (int64_t)((d.N + kDqBlock - 1) / kDqBlock) * d.H * d.B; }
inline int dq_split(const Dims &d) { return dq_blocks(d) <= kDqSplitBlocks ? 2 : 1; }
inline int64_t dq_split_blocks(const Dims &d) { return dq_split(d) == 2 ? dq_blocks(d) : 0; }
inline int64_t dq_part_floats(const Dims &d, int dkp) { return dq_split_blocks(d) * 2 * kDqBlock * dkp; }

// Query-block-outer dQ (bf16 mode): dq [DK,N,H,B] = scale dS K, every element
// written once; inputs as for launch_backward_bf16.  part and ticket as sized
// above (ticket zeroed by the launch that writes the tiles), used when dq_split(d) == 2.
hipError_t launch_dq(const __bf16 *q16, const __bf16 *o16, const float *stats, const __bf16 *k16, const __bf16 *v16,
                     const uint16_t *mask, const uint8_t *map, float scale, float *dq, float *part, int *ticket,
                     int Np, int Mp, const Dims &d, hipStream_t s);

// Grouped-query reduction: dst[c, m, g, b] = sum_{r < rk2} part[c, m, g*rk2 + r, b]
// (r in order) for dK (pk -> dk) and dV (pv -> dv).  One job per tensor: items
// are float4 (chunk % 4 == 0) or single floats, numbered over all groups.
struct ReduceJob {
    const float *part;
    float *dst;      // elements of out_fmt (the result blob) or f32
    int out_fmt;
    int64_t chunk;   // floats of one head's slice (D * M)
    int vec;         // chunk % 4 == 0: float4 items
    int64_t items;   // work items (float4 or float) over all groups
};
// Fills the two jobs for upg partials per group; returns upg.
inline int gqa_reduce_jobs(const float *pk, float *dk, const float *pv, float *dv, const Dims &d, int upg,
                           ReduceJob j[2])
{
    const int64_t groups = (int64_t)d.Hkv * d.B;
    const float *part[2] = {pk, pv};
    float *dst[2] = {dk, dv};
    const int D[2] = {d.DK, d.DV};
    for (int t = 0; t < 2; ++t) {
        j[t].part = part[t];
        j[t].dst = dst[t];
        j[t].out_fmt = d.out_fmt;
        j[t].chunk = (int64_t)D[t] * d.M;
        j[t].vec = (j[t].chunk % 4 == 0);
        j[t].items = (j[t].vec ? j[t].chunk / 4 : j[t].chunk) * groups;
    }
    return upg;
}

// The reduction above, one launch.
hipError_t launch_gqa_reduce(const float *pk, float *dk, const float *pv, float *dv, const Dims &d, int upg,
                             hipStream_t s);

// Records the detail of an error for fab_last_error (thread-local) and returns code.
int set_error(int code, const char *fmt, ...);

// Fill n floats with zero.
hipError_t launch_zero(float *p, int64_t n, hipStream_t s);

}  // namespace fab
