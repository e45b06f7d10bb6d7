// fab_aux.hip -- the memory-bound kernels of libfab (gfx950):
//   block_map_kernel   one byte per 32x32 (query x key) block of the additive
//                      f16 mask: SKIP (all -inf), FREE (all zero) or MIXED, plus
//                      a bit telling whether the block follows the causal rule
//                      (f32 mode; in bf16 mode the pack launches build the map)
//   prep_kernel        f32 mode: D = rowsum(dO o O) (labml "Flash Attention",
//                      "Backward pass"); zeroes the dQ slice (atomics target) and
//                      the pads of the result blob
//   pack_qkv_kernel    f32 (or bf16) rows of Q, K, V -> bf16 64-row tiles
//                      (fab_tiles.h), one tile per work-group through LDS so that
//                      the row reads and the tile writes are both contiguous,
//                      and the block map of the mask in the same launch
//   pack_prep_kernel   the same with O and the LSE supplied, plus the bf16-mode
//                      prep: the dO tiles, D = rowsum(dO o O) and the per-query
//                      LSE/D blocks
//   gqa_reduce_kernel  sums per-query-head dK/dV partials over each group of
//                      H/Hkv heads (grouped-query attention, head map h/(H/Hkv))
//   zero_kernel        zero fill
#include <algorithm>

#include "fab_common.h"
#include "fab_launch.h"
#include "fab_tiles.h"

namespace fab {

// ============================================================== block map
// A work-group classifies one 32-row strip of 8 blocks (32 x 256 mask entries):
// thread t reads row t / 8, the 64 bytes of block t % 8 in that row, so each wave
// reads 8 rows of 512 contiguous bytes.  A block's flags are and-ed over its 32
// rows in LDS.  Entries past N or M do not count.
constexpr int kMapStrip = 8;   // blocks per work-group
__device__ __forceinline__ void block_map_strip(const uint16_t *__restrict__ mask, uint8_t *__restrict__ map, int N,
                                                int M, int nqb, int nkb, int group)
{
    __shared__ int sFlag[kMapStrip][3];   // all -inf, all zero, follows the causal rule
    const int strips = (nkb + kMapStrip - 1) / kMapStrip;
    const int qb = group / strips, kb0 = (group - qb * strips) * kMapStrip;
    const int tid = threadIdx.x, j = tid & (kMapStrip - 1), kb = kb0 + j;
    if (tid < kMapStrip * 3) sFlag[tid / 3][tid % 3] = 1;
    __syncthreads();
    const int n = qb * kMapTile + (tid >> 3);
    const int m0 = kb * kMapTile;
    bool all_inf = true, all_zero = true, causal = true;
    if (n < N && kb < nkb) {
        const uint16_t *row = mask + (size_t)n * M;
        uint16_t x[kMapTile];
        if ((M & 7) == 0 && m0 + kMapTile <= M) {
#pragma unroll
            for (int c = 0; c < kMapTile / 8; ++c) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(row + m0 + 8 * c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[8 * c + 2 * i] = (uint16_t)(a[i] & 0xFFFFu);
                    x[8 * c + 2 * i + 1] = (uint16_t)(a[i] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kMapTile; ++i) x[i] = m0 + i < M ? row[m0 + i] : (uint16_t)0xFC00u;
        }
#pragma unroll
        for (int i = 0; i < kMapTile; ++i) {
            const int m = m0 + i;
            if (m < M) {
                const bool is_inf = x[i] == 0xFC00u, is_zero = (x[i] & 0x7FFFu) == 0;
                all_inf = all_inf && is_inf;
                all_zero = all_zero && is_zero;
                causal = causal && (m <= n ? is_zero : is_inf);
            }
        }
    }
    if (!all_inf) atomicAnd(&sFlag[j][0], 0);
    if (!all_zero) atomicAnd(&sFlag[j][1], 0);
    if (!causal) atomicAnd(&sFlag[j][2], 0);
    __syncthreads();
    if (tid < kMapStrip && kb0 + tid < nkb) {
        const uint8_t cls = sFlag[tid][0] ? kBlockSkip : (sFlag[tid][1] ? kBlockFree : kBlockMixed);
        map[qb * nkb + kb0 + tid] = cls | (sFlag[tid][2] ? kBlockCausalBit : 0);
    }
}

__global__ __launch_bounds__(256) void block_map_kernel(const uint16_t *__restrict__ mask,
                                                        uint8_t *__restrict__ map, int N, int M,
                                                        int nqb, int nkb)
{
    block_map_strip(mask, map, N, M, nqb, nkb, blockIdx.x);
}

inline int64_t map_groups(int N, int M)
{
    const int nqb = (N + kMapTile - 1) / kMapTile, nkb = (M + kMapTile - 1) / kMapTile;
    return (int64_t)nqb * ((nkb + kMapStrip - 1) / kMapStrip);
}

// ============================================================== zero fill
__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n4 = n / 4;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j = i; j < n4; j += stride) reinterpret_cast<f32x4 *>(p)[j] = z;
    for (int64_t j = n4 * 4 + i; j < n; j += stride) p[j] = 0.f;
}

// ============================================================== prep (f32 mode)
struct PrepArgs {
    const float *dO, *O;
    float *delta, *blob;
    int64_t zero_lo, zero_hi;         // zero blob[zero_lo, zero_hi): the dQ slice and its pad
    int64_t pad1_lo, pad1_hi, pad2_lo, pad2_hi;
    int rows, DV, N, H, lpr_log2, vec;
};

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a)
{
    const int lpr = 1 << a.lpr_log2;
    const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
    const int nthr = gridDim.x * blockDim.x;
    const int sub = threadIdx.x & (lpr - 1);
    // rows r = h + H*(n + N*b): the row order of d and O
    const int groups = nthr >> a.lpr_log2;
    for (int r = gtid >> a.lpr_log2; r < a.rows; r += groups) {
        const float *x = a.dO + (size_t)r * a.DV;
        const float *y = a.O + (size_t)r * a.DV;
        const int h = r % a.H, n = (r / a.H) % a.N, b = r / (a.H * a.N);
        float acc = 0.f;
        for (int c = sub * 4; c < a.DV; c += lpr * 4) {
            const f32x4 u = load_row4(x, c, a.DV, a.vec);
            const f32x4 v = load_row4(y, c, a.DV, a.vec);
            acc += u[0] * v[0] + u[1] * v[1] + u[2] * v[2] + u[3] * v[3];
        }
        acc = group_sum(acc, lpr);
        if (sub == 0) a.delta[n + a.N * (h + a.H * b)] = acc;
    }
    // zero the dQ slice for the atomics, and the two other pads
    const int64_t z4 = (a.zero_lo + 3) / 4, n4 = a.zero_hi / 4;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j = z4 + gtid; j < n4; j += nthr) reinterpret_cast<f32x4 *>(a.blob)[j] = z;
    if (gtid < 4 && a.zero_lo + gtid < 4 * z4 && a.zero_lo + gtid < a.zero_hi) a.blob[a.zero_lo + gtid] = 0.f;
    if (gtid < 4) {
        if (a.pad1_lo + gtid < a.pad1_hi) a.blob[a.pad1_lo + gtid] = 0.f;
        if (a.pad2_lo + gtid < a.pad2_hi) a.blob[a.pad2_lo + gtid] = 0.f;
    }
}

// ============================================================== bf16 tiles
// One packing job: heads of M rows of D floats -> bf16 tiles [heads][Mp][DP].  Row
// m of head hd = hh + H*bb starts at src + hh*sh + bb*sb + m*rs floats.
struct PackJob {
    const void *src;                  // rows of f32, bf16 or f16 elements (src_fmt: kF32, kBF16, kF16)
    int src_fmt;
    __bf16 *dst;
    int64_t sh, sb, rs;
    int H, M, Mp, D, vec;
    int tiles;                        // heads * Mp / 64: work-groups of this job
};

// Extra outputs of the bf16-mode prep (second input O, LSE/D blocks, blob pads).
struct PrepExtra {
    const void *O;                    // rows like the job's src; f32, or bf16 when O_bf16
    int O_bf16;
    const float *lse;                 // row LSE [N,H,B] (natural log)
    float *stats;                     // LSE/D blocks [heads][Mp/64][128]
    float *blob;                      // result blob whose pads are zeroed (work-group 0)
    int64_t pad_lo[3], pad_hi[3];     // the pads, in 16-bit units (zero in every element type)
    int *zero;                        // nzero ints set to 0 (the dQ split counters)
    int nzero;
};

// One 64-row tile of job j (tile index bt within the job), through LDS so that the
// row reads and the tile writes are both contiguous.  With x (prep), also the
// row dot products with O and the tile's LSE/D block.
template <int DP>
__device__ __forceinline__ void pack_tile(const PackJob &j, int bt, const PrepExtra *x)
{
    constexpr int C4 = DP / 4;                        // 4-column groups per row
    constexpr int IT = (64 * C4 + 255) / 256;         // per thread
    __shared__ __attribute__((aligned(16))) __bf16 tile[64 * DP];
    __shared__ float part[64][C4 + 1];
    const int tid = threadIdx.x;
    const int ntile = j.Mp / 64;
    const int hd = bt / ntile, t = bt - hd * ntile;
    const int hh = hd % j.H, bb = hd / j.H;
    const int64_t head_off = hh * j.sh + bb * j.sb;
    const void *obase = x ? x->O : nullptr;   // with the head's offset head_off (elements)
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    // all loads of the tile first (independent, so they are in flight together)
    f32x4 xv[IT], yv[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int idx = tid + 256 * i;
        const int r = idx / C4, col = 4 * (idx - r * C4);
        const int m = t * 64 + r;
        const bool ok = idx < 64 * C4 && m < j.M;
        xv[i] = ok ? load_row4_any(j.src, head_off + m * j.rs, col, j.D, j.vec, j.src_fmt) : z;
        yv[i] = (ok && obase) ? load_row4_any(obase, head_off + m * j.rs, col, j.D, j.vec, x->O_bf16 ? kBF16 : kF32) : z;
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int idx = tid + 256 * i;
        if (idx >= 64 * C4) break;
        const int r = idx / C4, col = 4 * (idx - r * C4);
        *reinterpret_cast<bf16x4 *>(&tile[((col >> 3) * 64 + r) * 8 + (col & 7)]) = to_bf16x4(xv[i]);
        if (obase) part[r][col >> 2] = xv[i][0] * yv[i][0] + xv[i][1] * yv[i][1] + xv[i][2] * yv[i][2] + xv[i][3] * yv[i][3];
    }
    __syncthreads();
    bf16x8 *out = reinterpret_cast<bf16x8 *>(j.dst + ((size_t)hd * j.Mp + t * 64) * DP);
    for (int i = tid; i < 8 * DP; i += 256) out[i] = reinterpret_cast<const bf16x8 *>(tile)[i];
    if (x && tid < 64) {
        const int m = t * 64 + tid;
        float dsum = 0.f;
        for (int c = 0; c < C4; ++c) dsum += part[tid][c];
        float *st = x->stats + ((size_t)hd * ntile + t) * kStatsTile + tid;
        float lse2 = INFINITY;   // rows past M (padding) and all-masked rows: no weight
        if (m < j.M) {
            const float L = x->lse[(size_t)j.M * hd + m];
            if (L != -INFINITY) lse2 = L * kLog2e;
        }
        st[0] = lse2;
        st[64] = m < j.M ? dsum : 0.f;
    }
}

// Up to three packing jobs in one launch (Q and K with DKP columns, V with DVP):
// work-groups [0, t0) job 0, [t0, t0 + t1) job 1, the rest job 2.
struct PackJobs {
    PackJob j[3];
    // the mask's block map in the same launch (work-groups [0, map_groups))
    const uint16_t *mask;
    uint8_t *map;
    int N, M, nqb, nkb, map_groups;
};

template <int DKP, int DVP>
__global__ __launch_bounds__(256) void pack_qkv_kernel(PackJobs a)
{
    int bt = blockIdx.x;
    if (bt < a.map_groups) {
        block_map_strip(a.mask, a.map, a.N, a.M, a.nqb, a.nkb, bt);
        return;
    }
    bt -= a.map_groups;
    if (bt < a.j[0].tiles) {
        pack_tile<DKP>(a.j[0], bt, nullptr);
        return;
    }
    bt -= a.j[0].tiles;
    if (bt < a.j[1].tiles) {
        pack_tile<DKP>(a.j[1], bt, nullptr);
        return;
    }
    bt -= a.j[1].tiles;
    pack_tile<DVP>(a.j[2], bt, nullptr);
}

// The pack (Q, K, V, block map) and the prep of a supplied O and LSE (dO tiles,
// LSE/D blocks, blob pads, counters) in one launch: the prep tiles (two input rows
// each, the heavier work-groups) first, then the pack.
template <int DKP, int DVP>
__global__ __launch_bounds__(256) void pack_prep_kernel(PackJobs a, PackJob j, PrepExtra x)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < x.nzero; i += gridDim.x * 256) x.zero[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x < 8)   // pads below 16 bytes: at most 7 16-bit units
        for (int k = 0; k < 3; ++k)
            if (x.pad_lo[k] + threadIdx.x < x.pad_hi[k]) reinterpret_cast<uint16_t *>(x.blob)[x.pad_lo[k] + threadIdx.x] = 0;
    int bt = blockIdx.x;
    if (bt < j.tiles) {
        pack_tile<DVP>(j, bt, &x);
        return;
    }
    bt -= j.tiles;
    if (bt < a.map_groups) {
        block_map_strip(a.mask, a.map, a.N, a.M, a.nqb, a.nkb, bt);
        return;
    }
    bt -= a.map_groups;
    if (bt < a.j[0].tiles) {
        pack_tile<DKP>(a.j[0], bt, nullptr);
        return;
    }
    bt -= a.j[0].tiles;
    if (bt < a.j[1].tiles) {
        pack_tile<DKP>(a.j[1], bt, nullptr);
        return;
    }
    bt -= a.j[1].tiles;
    pack_tile<DVP>(a.j[2], bt, nullptr);
}

namespace {
PackJob rows_job(const void *src, int src_fmt, __bf16 *dst, int64_t heads, int M, int Mp, int D)
{
    PackJob j = {};
    j.src = src; j.src_fmt = src_fmt; j.dst = dst;
    j.H = 1; j.sh = 0; j.sb = (int64_t)M * D; j.rs = D;   // heads are consecutive blocks of M rows
    j.M = M; j.Mp = Mp; j.D = D; j.vec = (D % 4 == 0);
    j.tiles = (int)(heads * (Mp / 64));
    return j;
}

template <int DKP, int DVP, bool BF16>
hipError_t run_pack(const PackJobs &a, hipStream_t s)
{
    const int64_t grid = (int64_t)a.map_groups + a.j[0].tiles + a.j[1].tiles + a.j[2].tiles;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((pack_qkv_kernel<DKP, DVP>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}
}  // namespace

namespace {
PackJobs pack_jobs(const void *q, const void *k, const void *v, __bf16 *q16, __bf16 *k16, __bf16 *v16,
                   const uint16_t *mask, uint8_t *map, int Np, int Mp, const Dims &d)
{
    PackJobs a = {};
    const int64_t qh = q ? (int64_t)d.H * d.B : 0, kh = (int64_t)d.Hkv * d.B;
    a.j[0] = rows_job(q, d.in_fmt, q16, qh, d.N, Np, d.DK);
    a.j[1] = rows_job(k, d.in_fmt, k16, kh, d.M, Mp, d.DK);
    a.j[2] = rows_job(v, d.in_fmt, v16, kh, d.M, Mp, d.DV);
    if (map) {
        a.mask = mask; a.map = map; a.N = d.N; a.M = d.M;
        a.nqb = (d.N + kMapTile - 1) / kMapTile; a.nkb = (d.M + kMapTile - 1) / kMapTile;
        a.map_groups = (int)map_groups(d.N, d.M);
    }
    return a;
}

void prep_job(const void *dO, const void *O, const float *lse, __bf16 *dO16, float *stats, float *blob, int Np,
              int64_t nq, int64_t off_k, int64_t nk, int64_t off_v, int64_t nv, int64_t total, int *zero, int nzero,
              const Dims &d, PackJob *pj, PrepExtra *px)
{
    PackJob j = {};
    j.src = dO; j.src_fmt = d.in_fmt; j.dst = dO16;
    // d, O [DV,H,N,B]: row n of head (h, b) at DV*(h + H*(n + N*b))
    j.H = d.H; j.sh = d.DV; j.sb = (int64_t)d.DV * d.H * d.N; j.rs = (int64_t)d.DV * d.H;
    j.M = d.N; j.Mp = Np; j.D = d.DV; j.vec = (d.DV % 4 == 0);
    j.tiles = d.H * d.B * (Np / 64);
    PrepExtra x = {};
    x.O = O; x.O_bf16 = d.o_bf16; x.lse = lse; x.stats = stats; x.blob = blob;
    const int u = d.out_fmt == kF32 ? 2 : 1;   // 16-bit units per blob element
    x.pad_lo[0] = u * nq; x.pad_hi[0] = u * off_k;
    x.pad_lo[1] = u * (off_k + nk); x.pad_hi[1] = u * off_v;
    x.pad_lo[2] = u * (off_v + nv); x.pad_hi[2] = u * total;
    x.zero = zero; x.nzero = nzero;
    *pj = j;
    *px = x;
}

struct PackPrep {
    PackJobs a;
    int npack;
    PackJob j;
    PrepExtra x;
};

template <int DKP, int DVP, bool BF16>
hipError_t run_pack_prep(const PackPrep &p, hipStream_t s)
{
    const int64_t grid = (int64_t)p.npack + p.j.tiles;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((pack_prep_kernel<DKP, DVP>), dim3((unsigned)grid), dim3(256), 0, s, p.a, p.j, p.x);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_pack_qkv(const void *q, const void *k, const void *v, __bf16 *q16, __bf16 *k16, __bf16 *v16,
                           const uint16_t *mask, uint8_t *map, int Np, int Mp, const Dims &d, hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    const PackJobs a = pack_jobs(q, k, v, q16, k16, v16, mask, map, Np, Mp, d);
    FAB_DISPATCH_HEAD_DIMS(run_pack, a, s, hd, true);
}

hipError_t launch_pack_prep_bf16(const void *q, const void *k, const void *v, __bf16 *q16, __bf16 *k16,
                                 __bf16 *v16, const uint16_t *mask, uint8_t *map, const void *dO, const void *O,
                                 const float *lse, __bf16 *dO16, float *stats, float *blob, int64_t nq, int64_t off_k,
                                 int64_t nk, int64_t off_v, int64_t nv, int64_t total, int *zero, int nzero, int Np,
                                 int Mp, const Dims &d, hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    PackPrep p;
    p.a = pack_jobs(q, k, v, q16, k16, v16, mask, map, Np, Mp, d);
    p.npack = p.a.map_groups + p.a.j[0].tiles + p.a.j[1].tiles + p.a.j[2].tiles;
    prep_job(dO, O, lse, dO16, stats, blob, Np, nq, off_k, nk, off_v, nv, total, zero, nzero, d, &p.j, &p.x);
    FAB_DISPATCH_HEAD_DIMS(run_pack_prep, p, s, hd, true);
}

// ============================================================== GQA reduce
// dK and dV in one launch: work items [0, n0) reduce job 0, the rest job 1; each
// sums the rk2 partials of a group in unit order.
__global__ __launch_bounds__(256) void gqa_reduce_kernel(ReduceJob j0, ReduceJob j1, int rk2)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t total = j0.items + j1.items;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        if (i < j0.items)
            reduce_item(j0, rk2, i);
        else
            reduce_item(j1, rk2, i - j0.items);
    }
}

// ============================================================== launchers
hipError_t launch_block_map(const uint16_t *mask, uint8_t *map, const Dims &d, hipStream_t s)
{
    const int nqb = (d.N + kMapTile - 1) / kMapTile, nkb = (d.M + kMapTile - 1) / kMapTile;
    if (nqb == 0 || nkb == 0) return hipSuccess;
    hipLaunchKernelGGL(block_map_kernel, dim3((unsigned)map_groups(d.N, d.M)), dim3(256), 0, s, mask, map, d.N, d.M,
                       nqb, nkb);
    return hipGetLastError();
}

hipError_t launch_prep(const float *dO, const float *O, float *delta, float *blob, int64_t off_k, int64_t nk,
                       int64_t off_v, int64_t nv, int64_t total, const Dims &d, hipStream_t s)
{
    PrepArgs a;
    a.dO = dO; a.O = O; a.delta = delta; a.blob = blob;
    a.zero_lo = 0;
    a.zero_hi = off_k;  // off_k = pad4(nq), a multiple of 4
    a.pad1_lo = off_k + nk; a.pad1_hi = off_v;
    a.pad2_lo = off_v + nv; a.pad2_hi = total;
    a.rows = d.B * d.N * d.H;
    a.DV = d.DV; a.N = d.N; a.H = d.H;
    a.vec = (d.DV % 4 == 0);
    int lpr = 1, lg = 0;
    while (lpr * 4 < a.DV && lpr < 64) { lpr *= 2; ++lg; }
    a.lpr_log2 = lg;
    const int64_t work = std::max<int64_t>((int64_t)a.rows * lpr, off_k / 4);
    int grid = (int)std::min<int64_t>((work + 255) / 256, 4096);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gqa_reduce(const float *pk, float *dk, const float *pv, float *dv, const Dims &d, int upg,
                             hipStream_t s)
{
    ReduceJob j[2];
    const int rk2 = gqa_reduce_jobs(pk, dk, pv, dv, d, upg, j);
    const int64_t work = j[0].items + j[1].items;
    if (work == 0) return hipSuccess;
    const int grid = (int)std::min<int64_t>((work + 255) / 256, 8192);
    hipLaunchKernelGGL(gqa_reduce_kernel, dim3(grid), dim3(256), 0, s, j[0], j[1], rk2);
    return hipGetLastError();
}

hipError_t launch_zero(float *p, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int grid = (int)std::min<int64_t>((n / 4 + 255) / 256 + 1, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace fab
