// fab_aux.hip -- the memory-bound kernels of libfab (gfx950):
//   block_map_kernel   one byte per 32x32 (query x key) block of the additive
//                      f16 mask: SKIP (all -inf), FREE (all zero) or MIXED, plus
//                      a bit telling whether the block follows the causal rule
//   prep_kernel        D = rowsum(dO o O) (labml "Flash Attention", "Backward
//                      pass"); zeroes the dQ slice and the pads of the result
//                      blob; in bf16 mode also writes dO as bf16, one contiguous
//                      [N][DVP] matrix per (batch, head), zero-padded columns
//   gqa_reduce_kernel  sums per-query-head dK/dV partials over each group of
//                      H/Hkv heads (grouped-query attention, head map h/(H/Hkv))
//   zero_kernel        zero fill
#include <algorithm>

#include "fab_common.h"
#include "fab_launch.h"

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

// ============================================================== prep
struct PrepArgs {
    const float *dO, *O;
    float *delta, *blob;
    __bf16 *dO16;                     // bf16 copy [B][H][N][DVP], or NULL
    int64_t zero_lo, zero_hi;         // zero blob[zero_lo, zero_hi): the dQ slice (or its pad)
    int64_t pad1_lo, pad1_hi, pad2_lo, pad2_hi;
    int rows, DV, DVP, N, H, lpr_log2, vec;
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
        __bf16 *o16 = a.dO16 ? a.dO16 + ((size_t)(b * a.H + h) * a.N + n) * a.DVP : nullptr;
        float acc = 0.f;
        for (int c = sub * 4; c < a.DVP; c += lpr * 4) {
            const f32x4 u = load_row4(x, c, a.DV, a.vec);
            if (c < a.DV) {
                const f32x4 v = load_row4(y, c, a.DV, a.vec);
                acc += u[0] * v[0] + u[1] * v[1] + u[2] * v[2] + u[3] * v[3];
            }
            if (o16) *reinterpret_cast<bf16x4 *>(o16 + c) = to_bf16x4(u);
        }
        acc = group_sum(acc, lpr);
        if (sub == 0) a.delta[n + a.N * (h + a.H * b)] = acc;
    }
    // zero the dQ slice for the atomics (or only its pad), and the two other pads
    const int64_t z4 = (a.zero_lo + 3) / 4, n4 = a.zero_hi / 4;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j = z4 + gtid; j < n4; j += nthr) reinterpret_cast<f32x4 *>(a.blob)[j] = z;
    if (gtid < 4 && a.zero_lo + gtid < 4 * z4 && a.zero_lo + gtid < a.zero_hi) a.blob[a.zero_lo + gtid] = 0.f;
    if (gtid < 4) {
        if (a.pad1_lo + gtid < a.pad1_hi) a.blob[a.pad1_lo + gtid] = 0.f;
        if (a.pad2_lo + gtid < a.pad2_hi) a.blob[a.pad2_lo + gtid] = 0.f;
    }
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

hipError_t launch_prep(const float *dO, const float *O, float *delta, float *blob, __bf16 *dO16,
                       int dvp, int64_t zero_lo, int64_t off_k, int64_t nk, int64_t off_v, int64_t nv,
                       int64_t total, const Dims &d, hipStream_t s)
{
    PrepArgs a;
    a.dO = dO; a.O = O; a.delta = delta; a.blob = blob; a.dO16 = dO16;
    a.zero_lo = zero_lo;
    a.zero_hi = off_k;  // off_k = pad4(nq), a multiple of 4
    a.pad1_lo = off_k + nk; a.pad1_hi = off_v;
    a.pad2_lo = off_v + nv; a.pad2_hi = total;
    a.rows = d.B * d.N * d.H;
    a.DV = d.DV; a.DVP = dO16 ? dvp : d.DV; a.N = d.N; a.H = d.H;
    a.vec = (d.DV % 4 == 0);
    int lpr = 1, lg = 0;
    while (lpr * 4 < a.DVP && lpr < 64) { lpr *= 2; ++lg; }
    a.lpr_log2 = lg;
    const int64_t work = std::max<int64_t>((int64_t)a.rows * lpr, (off_k - zero_lo) / 4);
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
