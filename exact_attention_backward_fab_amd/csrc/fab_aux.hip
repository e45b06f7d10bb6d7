// fab_aux.hip -- the memory-bound kernels of libfab (gfx950):
//   block_map_kernel   one byte per 32x32 (query x key) block of the additive
//                      f16 mask: SKIP (all -inf), FREE (all zero) or MIXED, plus
//                      a bit telling whether the block follows the causal rule
//   prep_kernel        f32 mode: D = rowsum(dO o O) (labml "Flash Attention",
//                      "Backward pass"); zeroes the dQ slice (atomics target) and
//                      the pads of the result blob
//   pack_tiles_kernel  f32 rows -> bf16 64-row tiles (fab_tiles.h), one tile per
//                      work-group through LDS, so that the row reads and the tile
//                      writes are both contiguous; with a second input it also
//                      forms D = rowsum(dO o O) and the per-query LSE/D blocks
//                      (the bf16-mode prep)
//   gqa_reduce_kernel  sums per-query-head dK/dV partials over each group of
//                      H/Hkv heads (grouped-query attention, head map h/(H/Hkv))
//   zero_kernel        zero fill
#include <algorithm>

#include "fab_common.h"
#include "fab_launch.h"
#include "fab_tiles.h"

namespace fab {

// ============================================================== block map
__global__ __launch_bounds__(64) void block_map_kernel(const uint16_t *__restrict__ mask,
                                                       uint8_t *__restrict__ map, int N, int M,
                                                       int nkb)
{
    const int kb = blockIdx.x, qb = blockIdx.y;
    const int lane = threadIdx.x;
    const int n = qb * kMapTile + (lane >> 1);
    const int m0 = kb * kMapTile + (lane & 1) * 16;
    bool all_inf = true, all_zero = true, causal = true;
    if (n < N) {
        const uint16_t *row = mask + (size_t)n * M;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + i;
            if (m < M) {
                const uint16_t x = row[m];
                const bool is_inf = x == 0xFC00u, is_zero = (x & 0x7FFFu) == 0;
                all_inf = all_inf && is_inf;
                all_zero = all_zero && is_zero;
                causal = causal && (m <= n ? is_zero : is_inf);
            }
        }
    }
    all_inf = __all(all_inf);
    all_zero = __all(all_zero);
    causal = __all(causal);
    if (lane == 0) {
        const uint8_t cls = all_inf ? kBlockSkip : (all_zero ? kBlockFree : kBlockMixed);
        map[qb * nkb + kb] = cls | (causal ? kBlockCausalBit : 0);
    }
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
// Row m of head hd = hh + H*bb of src starts at src + hh*sh + bb*sb + m*rs floats.
struct PackArgs {
    const float *src, *O;             // O: second input of the prep (rows like src), or NULL
    const float *lse;                 // prep: row LSE [N,H,B] (natural log)
    __bf16 *dst;                      // tiles [heads][Mp][DP]
    float *stats;                     // prep: LSE/D blocks [heads][Mp/64][128]
    float *blob;                      // prep: result blob whose pads are zeroed (work-group 0)
    int64_t sh, sb, rs;
    int H, M, Mp, D, DP, vec;
    int64_t pad_lo[3], pad_hi[3];
};

template <int DP>
__global__ __launch_bounds__(256) void pack_tiles_kernel(PackArgs a)
{
    constexpr int C4 = DP / 4;                        // 4-column groups per row
    __shared__ __attribute__((aligned(16))) __bf16 tile[64 * DP];
    __shared__ float part[64][C4 + 1];
    const int tid = threadIdx.x;
    const int ntile = a.Mp / 64;
    const int hd = blockIdx.x / ntile, t = blockIdx.x - hd * ntile;
    const int hh = hd % a.H, bb = hd / a.H;
    const float *base = a.src + hh * a.sh + bb * a.sb;
    const float *obase = a.O ? a.O + hh * a.sh + bb * a.sb : nullptr;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    constexpr int IT = (64 * C4 + 255) / 256;         // 4-column groups per thread
    // all loads of the tile first (independent, so they are in flight together)
    f32x4 x[IT], y[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int idx = tid + 256 * i;
        const int r = idx / C4, col = 4 * (idx - r * C4);
        const int m = t * 64 + r;
        const bool ok = idx < 64 * C4 && m < a.M;
        x[i] = ok ? load_row4(base + m * a.rs, col, a.D, a.vec) : z;
        y[i] = (ok && obase) ? load_row4(obase + m * a.rs, col, a.D, a.vec) : z;
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int idx = tid + 256 * i;
        if (idx >= 64 * C4) break;
        const int r = idx / C4, col = 4 * (idx - r * C4);
        *reinterpret_cast<bf16x4 *>(&tile[((col >> 3) * 64 + r) * 8 + (col & 7)]) = to_bf16x4(x[i]);
        if (obase) part[r][col >> 2] = x[i][0] * y[i][0] + x[i][1] * y[i][1] + x[i][2] * y[i][2] + x[i][3] * y[i][3];
    }
    __syncthreads();
    bf16x8 *out = reinterpret_cast<bf16x8 *>(a.dst + ((size_t)hd * a.Mp + t * 64) * DP);
    for (int i = tid; i < 8 * DP; i += 256) out[i] = reinterpret_cast<const bf16x8 *>(tile)[i];
    if (obase && tid < 64) {
        const int m = t * 64 + tid;
        float dsum = 0.f;
        for (int c = 0; c < C4; ++c) dsum += part[tid][c];
        float *st = a.stats + ((size_t)hd * ntile + t) * kStatsTile + tid;
        float lse2 = INFINITY;   // rows past M (padding) and all-masked rows: no weight
        if (m < a.M) {
            const float L = a.lse[(size_t)a.M * hd + m];
            if (L != -INFINITY) lse2 = L * kLog2e;
        }
        st[0] = lse2;
        st[64] = m < a.M ? dsum : 0.f;
    }
    if (a.blob && blockIdx.x == 0 && tid < 4)
        for (int k = 0; k < 3; ++k)
            if (a.pad_lo[k] + tid < a.pad_hi[k]) a.blob[a.pad_lo[k] + tid] = 0.f;
}

namespace {
template <int DP>
hipError_t run_pack(const PackArgs &a, int64_t heads, hipStream_t s)
{
    const int64_t grid = heads * (a.Mp / 64);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_tiles_kernel<DP>, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t dispatch_pack(const PackArgs &a, int64_t heads, hipStream_t s)
{
    switch (a.DP) {
    case 32: return run_pack<32>(a, heads, s);
    case 64: return run_pack<64>(a, heads, s);
    case 128: return run_pack<128>(a, heads, s);
    case 192: return run_pack<192>(a, heads, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_pack_rows_bf16(const float *src, __bf16 *dst, int64_t heads, int M, int Mp, int D, int DP,
                                 hipStream_t s)
{
    PackArgs a = {};
    a.src = src; a.dst = dst;
    a.sh = (int64_t)M * D; a.sb = 0; a.rs = D;   // heads are consecutive blocks of M rows
    a.H = 1; a.M = M; a.Mp = Mp; a.D = D; a.DP = DP; a.vec = (D % 4 == 0);
    // with H = 1 every head index hd maps to hh = 0, bb = hd: make sb the head stride
    a.sb = a.sh; a.sh = 0;
    return dispatch_pack(a, heads, s);
}

hipError_t launch_prep_bf16(const float *dO, const float *O, const float *lse, __bf16 *dO16, float *stats, float *blob,
                            int dvp, int Np, int64_t nq, int64_t off_k, int64_t nk, int64_t off_v, int64_t nv,
                            int64_t total, const Dims &d, hipStream_t s)
{
    PackArgs a = {};
    a.src = dO; a.O = O; a.lse = lse; a.dst = dO16; a.stats = stats; a.blob = blob;
    // d, O [DV,H,N,B]: row n of head (h, b) at DV*(h + H*(n + N*b))
    a.sh = d.DV; a.sb = (int64_t)d.DV * d.H * d.N; a.rs = (int64_t)d.DV * d.H;
    a.H = d.H; a.M = d.N; a.Mp = Np; a.D = d.DV; a.DP = dvp; a.vec = (d.DV % 4 == 0);
    a.pad_lo[0] = nq; a.pad_hi[0] = off_k;
    a.pad_lo[1] = off_k + nk; a.pad_hi[1] = off_v;
    a.pad_lo[2] = off_v + nv; a.pad_hi[2] = total;
    return dispatch_pack(a, (int64_t)d.H * d.B, s);
}

// ============================================================== GQA reduce
__global__ __launch_bounds__(256) void gqa_reduce_kernel(const float *__restrict__ part,
                                                         float *__restrict__ dst, int64_t chunk,
                                                         int rk2, int64_t groups, int vec)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (vec) {
        const int64_t c4 = chunk / 4, total4 = c4 * groups;
        for (int64_t i = i0; i < total4; i += stride) {
            const int64_t gb = i / c4, off = i - gb * c4;
            const f32x4 *src = reinterpret_cast<const f32x4 *>(part) + gb * rk2 * c4 + off;
            f32x4 s = src[0];
            for (int r = 1; r < rk2; ++r) s += src[r * c4];
            reinterpret_cast<f32x4 *>(dst)[i] = s;
        }
    } else {
        const int64_t total = chunk * groups;
        for (int64_t i = i0; i < total; i += stride) {
            const int64_t gb = i / chunk, off = i - gb * chunk;
            const float *src = part + gb * rk2 * chunk + off;
            float s = src[0];
            for (int r = 1; r < rk2; ++r) s += src[r * chunk];
            dst[i] = s;
        }
    }
}

// ============================================================== launchers
hipError_t launch_block_map(const uint16_t *mask, uint8_t *map, const Dims &d, hipStream_t s)
{
    const int nqb = (d.N + kMapTile - 1) / kMapTile, nkb = (d.M + kMapTile - 1) / kMapTile;
    if (nqb == 0 || nkb == 0) return hipSuccess;
    hipLaunchKernelGGL(block_map_kernel, dim3(nkb, nqb), dim3(64), 0, s, mask, map, d.N, d.M, nkb);
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

hipError_t launch_gqa_reduce(const float *part, float *dst, int D, const Dims &d, hipStream_t s)
{
    const int rk2 = d.H / d.Hkv;
    const int64_t chunk = (int64_t)D * d.M, groups = (int64_t)d.Hkv * d.B;
    const int vec = (chunk % 4 == 0);
    const int64_t work = vec ? chunk / 4 * groups : chunk * groups;
    if (work == 0) return hipSuccess;
    const int grid = (int)std::min<int64_t>((work + 255) / 256, 8192);
    hipLaunchKernelGGL(gqa_reduce_kernel, dim3(grid), dim3(256), 0, s, part, dst, chunk, rk2,
                       groups, vec);
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
