// fab_kernels.hip -- HIP kernels of libfab for gfx950 (CDNA4).
//
// Kernels (one launch each, all on the caller's stream):
//   block_map_kernel  classify every 32x32 (query x key) block of the additive
//                     f16 mask as SKIP (all -inf), FREE (all zero) or MIXED
//   fwd_kernel        query-block-outer forward with the running max / running
//                     sum of the labml "Flash Attention" page ("Flash Attention
//                     Optimization"); writes O and the row log-sum-exp
//   prep_kernel       D = rowsum(dO o O) (labml page, "Backward pass"), zeroes
//                     the dQ slice and the pads of the result blob
//   bwd_kernel        key-block-outer backward: recomputes S and P from the row
//                     LSE, forms dV += P^T dO, dP = dO V^T, dS = P o (dP - D),
//                     dK += scale dS^T Q and dQ += scale dS K on the matrix cores;
//                     dK/dV stay in registers for the whole key block, dQ goes to
//                     the blob through f32 atomics
//   gqa_reduce_kernel sums per-query-head dK/dV partials over each group of
//                     H/Hkv heads (grouped-query attention)
//
// Layouts are ggml ne order (see include/fab.h).  Every kernel keeps its
// accesses inside the tensors' extents by explicit bounds checks, so any
// N, M, DK <= 192, DV <= 192 runs through the same code.
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
    bool all_inf = true, all_zero = true;
    if (n < N) {
        const uint16_t *row = mask + (size_t)n * M;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + i;
            if (m < M) {
                const uint16_t x = row[m];
                all_inf = all_inf && (x == 0xFC00u);
                all_zero = all_zero && ((x & 0x7FFFu) == 0);
            }
        }
    }
    all_inf = __all(all_inf);
    all_zero = __all(all_zero);
    if (lane == 0)
        map[qb * nkb + kb] = all_inf ? kBlockSkip : (all_zero ? kBlockFree : kBlockMixed);
}

// Class of a tile made of nq x nk map blocks starting at (qb0, kb0).
__device__ __forceinline__ int tile_class(const uint8_t *map, int nqb, int nkb, int qb0, int nq,
                                          int kb0, int nk)
{
    if (!map) return kBlockFree;
    bool all_skip = true, all_free = true;
    const int qe = min(qb0 + nq, nqb), ke = min(kb0 + nk, nkb);
    for (int i = qb0; i < qe; ++i)
        for (int j = kb0; j < ke; ++j) {
            const uint8_t c = map[i * nkb + j];
            all_skip = all_skip && (c == kBlockSkip);
            all_free = all_free && (c == kBlockFree);
        }
    return all_skip ? kBlockSkip : (all_free ? kBlockFree : kBlockMixed);
}

// ============================================================== zero fill
__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n4 = n / 4;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j = i; j < n4; j += stride) reinterpret_cast<f32x4 *>(p)[j] = z;
    for (int64_t j = n4 * 4 + i; j < n; j += stride) p[j] = 0.f;
}

// ============================================================== prep: D, zero dQ, pads
struct PrepArgs {
    const float *dO, *O;
    float *delta, *blob;
    int64_t zero_end;                 // zero blob[0, zero_end): dQ slice and its pad
    int64_t pad1_lo, pad1_hi, pad2_lo, pad2_hi;
    int rows, DV, N, H, lpr_log2, vec;
};

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a)
{
    const int lpr = 1 << a.lpr_log2;
    const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
    const int nthr = gridDim.x * blockDim.x;
    const int sub = threadIdx.x & (lpr - 1);
    // D rows: r = h + H*(n + N*b) over rows of DV floats (the layout of d and O)
    const int groups = nthr >> a.lpr_log2;
    for (int r = gtid >> a.lpr_log2; r < a.rows; r += groups) {
        const float *x = a.dO + (size_t)r * a.DV;
        const float *y = a.O + (size_t)r * a.DV;
        float acc = 0.f;
        for (int c = sub * 4; c < a.DV; c += lpr * 4) {
            const f32x4 u = load_row4(x, c, a.DV, a.vec);
            const f32x4 v = load_row4(y, c, a.DV, a.vec);
            acc += u[0] * v[0] + u[1] * v[1] + u[2] * v[2] + u[3] * v[3];
        }
        acc = group_sum(acc, lpr);
        if (sub == 0) {
            const int h = r % a.H, n = (r / a.H) % a.N, b = r / (a.H * a.N);
            a.delta[n + a.N * (h + a.H * b)] = acc;
        }
    }
    // zero the dQ slice (+ its pad) for the atomics, and the two other pads
    const int64_t n4 = a.zero_end / 4;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j = gtid; j < n4; j += nthr) reinterpret_cast<f32x4 *>(a.blob)[j] = z;
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

// ============================================================== forward
struct FwdArgs {
    const float *q, *k, *v;
    const uint16_t *mask;
    const uint8_t *map;
    float *O, *lse;
    int B, H, Hkv, N, M, DK, DV;
    int nqb, nkb, vecK, vecV;
    float scale;
};

template <int DKP, int DVP, bool BF16>
struct FwdCfg {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;
    static constexpr int BR = 32 * WAVES;  // queries per work-group (32 per wave)
    static constexpr int BC = 64;          // keys per step
    static constexpr int PADE = BF16 ? 8 : 4;
    static constexpr int LK = DKP + PADE;                        // sK row stride
    static constexpr int LV = BF16 ? (BC + PADE) : (DVP + PADE);  // sVt (bf16) / sV (f32)
    static constexpr int SV = BF16 ? DVP * LV : BC * LV;
    using T = typename std::conditional<BF16, __bf16, float>::type;
};

template <int DKP, int DVP, bool BF16>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdArgs p)
{
    using C = FwdCfg<DKP, DVP, BF16>;
    using T = typename C::T;
    constexpr int BC = C::BC, BR = C::BR, NT = C::NT, LK = C::LK, LV = C::LV;
    constexpr int NKT = BC / 32;
    __shared__ __attribute__((aligned(16))) T sK[BC * LK];
    __shared__ __attribute__((aligned(16))) T sV[C::SV];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int nqt = (p.N + BR - 1) / BR;
    const int qt = blockIdx.x % nqt, hb = blockIdx.x / nqt;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int n = qt * BR + w * 32 + l32;  // this lane's query (C-layout column)
    const bool nok = n < p.N;
    const float *kbase = p.k + (size_t)p.DK * p.M * (g + p.Hkv * b);
    const float *vbase = p.v + (size_t)p.DV * p.M * (g + p.Hkv * b);
    const float *qrow = p.q + (size_t)p.DK * (nok ? (n + p.N * (h + p.H * b)) : 0);

    // Q fragments: B operand of S^T = K Q^T (column = query, k = head dim)
    constexpr int NQF = BF16 ? DKP / 16 : DKP / 2;
    typename std::conditional<BF16, bf16x8, float>::type qf[NQF];
    if constexpr (BF16) {
#pragma unroll
        for (int t = 0; t < DKP / 16; ++t) {
            float x[8];
            const f32x4 lo = nok ? load_row4(qrow, 16 * t + 8 * half, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
            const f32x4 hi = nok ? load_row4(qrow, 16 * t + 8 * half + 4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[i] = lo[i]; x[4 + i] = hi[i]; }
            qf[t] = to_bf16x8(x);
        }
    } else {
#pragma unroll
        for (int t = 0; t < DKP / 2; t += 4) {
            const f32x4 x = nok ? load_row4(qrow, half * (DKP / 2) + t, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) qf[t + i] = x[i];
        }
    }

    f32x16 oacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) oacc[i] = zero16();
    float m_run = -INFINITY, l_half = 0.f;
    const float sl2 = p.scale * kLog2e;
    const int nkt_total = (p.M + BC - 1) / BC;

    for (int kt = 0; kt < nkt_total; ++kt) {
        const int key0 = kt * BC;
        const int cls = tile_class(p.map, p.nqb, p.nkb, qt * (BR / kMapTile), BR / kMapTile,
                                   key0 / kMapTile, BC / kMapTile);
        if (cls == kBlockSkip) continue;
        __syncthreads();
        // ---- stage K (row-major) and V (bf16: transposed, keys in MFMA order)
        if constexpr (BF16) {
            for (int c = tid; c < BC * (DKP / 4); c += NT) {
                const int r = c / (DKP / 4), c4 = c % (DKP / 4);
                const int key = key0 + r;
                const f32x4 x = key < p.M ? load_row4(kbase + (size_t)p.DK * key, 4 * c4, p.DK, p.vecK)
                                          : f32x4{0, 0, 0, 0};
                *reinterpret_cast<bf16x4 *>(&sK[r * LK + 4 * c4]) = to_bf16x4(x);
            }
            for (int c = tid; c < (BC / 8) * (DVP / 4); c += NT) {
                const int kg = c / (DVP / 4), c4 = c % (DVP / 4);
                f32x4 x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int key = key0 + 8 * kg + i;
                    x[i] = key < p.M ? load_row4(vbase + (size_t)p.DV * key, 4 * c4, p.DV, p.vecV)
                                     : f32x4{0, 0, 0, 0};
                }
                // key index bits 2 and 3 swapped within each 16 (MFMA operand order)
                const int base = 16 * (kg >> 1) + 4 * (kg & 1);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 lo, hi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) { lo[i] = (__bf16)x[i][jj]; hi[i] = (__bf16)x[4 + i][jj]; }
                    *reinterpret_cast<bf16x4 *>(&sV[(4 * c4 + jj) * LV + base]) = lo;
                    *reinterpret_cast<bf16x4 *>(&sV[(4 * c4 + jj) * LV + base + 8]) = hi;
                }
            }
        } else {
            for (int c = tid; c < BC * (DKP / 4); c += NT) {
                const int r = c / (DKP / 4), c4 = c % (DKP / 4);
                const int key = key0 + r;
                *reinterpret_cast<f32x4 *>(&sK[r * LK + 4 * c4]) =
                    key < p.M ? load_row4(kbase + (size_t)p.DK * key, 4 * c4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
            }
            for (int c = tid; c < BC * (DVP / 4); c += NT) {
                const int r = c / (DVP / 4), c4 = c % (DVP / 4);
                const int key = key0 + r;
                *reinterpret_cast<f32x4 *>(&sV[r * LV + 4 * c4]) =
                    key < p.M ? load_row4(vbase + (size_t)p.DV * key, 4 * c4, p.DV, p.vecV) : f32x4{0, 0, 0, 0};
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T for NKT 32-key sub-tiles (lane = query, rows = keys)
        f32x16 s[NKT];
#pragma unroll
        for (int kk = 0; kk < NKT; ++kk) {
            s[kk] = zero16();
            if constexpr (BF16) {
#pragma unroll
                for (int t = 0; t < DKP / 16; ++t) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sK[(kk * 32 + l32) * LK + 16 * t + 8 * half]);
                    s[kk] = mfma_bf16(a, qf[t], s[kk]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < DKP / 2; t += 4) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(&sK[(kk * 32 + l32) * LK + half * (DKP / 2) + t]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[kk] = mfma_f32(a[i], qf[t + i], s[kk]);
                }
            }
        }
        // ---- scale, mask, running max (log2 units)
        float mloc = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < NKT; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + kk * 32 + crow(r, half);
                float x = s[kk][r] * sl2;
                if (cls == kBlockMixed && nok && key < p.M)
                    x += half_bits_to_float(p.mask[key + (size_t)p.M * n]) * kLog2e;
                if (key >= p.M || !nok) x = -INFINITY;
                s[kk][r] = x;
                mloc = fmaxf(mloc, x);
            }
        mloc = swap_halves_max(mloc);
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKT; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = exp2f(s[kk][r] - m_use);
                s[kk][r] = e;
                lsum += e;
            }
        l_half = l_half * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < DVP / 32; ++i) oacc[i] *= alpha;

        // ---- O^T += V^T P^T (lane = query, rows = head dim)
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt) {
#pragma unroll
            for (int kk = 0; kk < NKT; ++kk) {
                if constexpr (BF16) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float pv[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) pv[i] = s[kk][8 * u + i];
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                            &sV[(dt * 32 + l32) * LV + kk * 32 + 16 * u + 8 * half]);
                        oacc[dt] = mfma_bf16(a, to_bf16x8(pv), oacc[dt]);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        const float a = sV[(kk * 32 + crow(u, half)) * LV + dt * 32 + l32];
                        oacc[dt] = mfma_f32(a, s[kk][u], oacc[dt]);
                    }
                }
            }
        }
    }

    // ---- normalise and store O [DV,H,N,B] and the natural-log LSE [N,H,B]
    const float l = swap_halves_sum(l_half);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (nok) {
        float *orow = p.O + (size_t)p.DV * (h + p.H * (n + p.N * b));
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c0 = dt * 32 + 8 * r4 + 4 * half;
                if (c0 >= p.DV) continue;
                f32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = oacc[dt][4 * r4 + i] * inv;
                if (p.vecV) {
                    *reinterpret_cast<f32x4 *>(orow + c0) = o;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c0 + i < p.DV) orow[c0 + i] = o[i];
                }
            }
        if (half == 0)
            p.lse[n + p.N * (h + p.H * b)] = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    }
}

// ============================================================== backward
struct BwdArgs {
    const float *q, *k, *v, *dO;
    const uint16_t *mask;
    const uint8_t *map;
    const float *lse, *delta;
    float *dq, *dk, *dv;
    int B, H, Hkv, N, M, DK, DV;
    int part_heads, nqb, nkb, vecK, vecV;
    float scale;
};

template <int DKP, int DVP, bool BF16>
struct BwdCfg {
    static constexpr int WAVES = BF16 ? 4 : ((DKP + DVP <= 128) ? 4 : 2);
    static constexpr int NT = 64 * WAVES;
    static constexpr int BC = 32 * WAVES;                  // keys per work-group (32 per wave)
    static constexpr int BR = BF16 ? (DKP <= 128 ? 64 : 32) : 32;  // queries per step
    static constexpr int PADE = BF16 ? 8 : 4;              // 16-byte row padding
    static constexpr int LQ = DKP + PADE, LDO = DVP + PADE;   // sQ, sdO row strides
    static constexpr int LQT = BR + PADE, LDOT = BR + PADE;   // sQt, sdOt (bf16)
    static constexpr int LKT = BC + PADE;                      // sKt (bf16)
    static constexpr int LK = DKP + PADE, LV = DVP + PADE;     // sK, sV (f32)
    static constexpr int LS = BC + PADE;                       // sdS
    // LDS element counts
    static constexpr int N_KT = BF16 ? DKP * LKT : 1;
    static constexpr int N_K = BF16 ? 1 : BC * LK;
    static constexpr int N_V = BF16 ? 1 : BC * LV;
    static constexpr int N_QT = BF16 ? DKP * LQT : 1;
    static constexpr int N_DOT = BF16 ? DVP * LDOT : 1;
    using T = typename std::conditional<BF16, __bf16, float>::type;
};

template <int DKP, int DVP, bool BF16>
__global__ __launch_bounds__((BwdCfg<DKP, DVP, BF16>::NT), 1) void bwd_kernel(BwdArgs p)
{
    using C = BwdCfg<DKP, DVP, BF16>;
    using T = typename C::T;
    constexpr int BC = C::BC, BR = C::BR, W = C::WAVES, NT = C::NT;
    constexpr int LQ = C::LQ, LDO = C::LDO, LQT = C::LQT, LDOT = C::LDOT, LKT = C::LKT;
    constexpr int LK = C::LK, LV = C::LV, LS = C::LS;
    constexpr int NQT = BR / 32;
    __shared__ __attribute__((aligned(16))) T sKt[C::N_KT];
    __shared__ __attribute__((aligned(16))) T sK[C::N_K];
    __shared__ __attribute__((aligned(16))) T sV[C::N_V];
    __shared__ __attribute__((aligned(16))) T sQ[BR * LQ];
    __shared__ __attribute__((aligned(16))) T sQt[C::N_QT];
    __shared__ __attribute__((aligned(16))) T sdO[BR * LDO];
    __shared__ __attribute__((aligned(16))) T sdOt[C::N_DOT];
    __shared__ __attribute__((aligned(16))) T sdS[BR * LS];
    __shared__ __attribute__((aligned(16))) float sLSE[BR];
    __shared__ __attribute__((aligned(16))) float sDel[BR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int HB = p.H * p.B;
    const int j = blockIdx.x / HB, hb = blockIdx.x % HB;  // key tile slowest: heaviest first under a causal mask
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int key0 = j * BC;
    const int mykey = key0 + 32 * w + l32;  // C-layout column of this lane in S, dP
    const bool keyok = mykey < p.M;
    const float *kbase = p.k + (size_t)p.DK * p.M * (g + p.Hkv * b);
    const float *vbase = p.v + (size_t)p.DV * p.M * (g + p.Hkv * b);
    const float *qbase = p.q + (size_t)p.DK * p.N * (h + p.H * b);
    const size_t dstride = (size_t)p.DV * p.H;                       // d / O row stride
    const float *dbase = p.dO + (size_t)p.DV * h + dstride * p.N * b;  // row n at + n*dstride

    // ---- stage K and V for this key block
    constexpr int NKF = BF16 ? DKP / 16 : 1, NVF = BF16 ? DVP / 16 : 1;
    bf16x8 kf[NKF], vf[NVF];  // bf16: B operands of S = Q K^T and dP = dO V^T
    if constexpr (BF16) {
        const float *kr = kbase + (size_t)p.DK * (keyok ? mykey : 0);
        const float *vr = vbase + (size_t)p.DV * (keyok ? mykey : 0);
#pragma unroll
        for (int t = 0; t < DKP / 16; ++t) {
            float x[8];
            const f32x4 lo = keyok ? load_row4(kr, 16 * t + 8 * half, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
            const f32x4 hi = keyok ? load_row4(kr, 16 * t + 8 * half + 4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[i] = lo[i]; x[4 + i] = hi[i]; }
            kf[t] = to_bf16x8(x);
        }
#pragma unroll
        for (int t = 0; t < DVP / 16; ++t) {
            float x[8];
            const f32x4 lo = keyok ? load_row4(vr, 16 * t + 8 * half, p.DV, p.vecV) : f32x4{0, 0, 0, 0};
            const f32x4 hi = keyok ? load_row4(vr, 16 * t + 8 * half + 4, p.DV, p.vecV) : f32x4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[i] = lo[i]; x[4 + i] = hi[i]; }
            vf[t] = to_bf16x8(x);
        }
        // K^T in LDS (head dim major, keys in natural order): B operand of dQ = dS K
        for (int c = tid; c < (BC / 8) * (DKP / 4); c += NT) {
            const int kg = c / (DKP / 4), c4 = c % (DKP / 4);
            f32x4 x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int key = key0 + 8 * kg + i;
                x[i] = key < p.M ? load_row4(kbase + (size_t)p.DK * key, 4 * c4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x8 col;
#pragma unroll
                for (int i = 0; i < 8; ++i) col[i] = (__bf16)x[i][jj];
                *reinterpret_cast<bf16x8 *>(&sKt[(4 * c4 + jj) * LKT + 8 * kg]) = col;
            }
        }
    } else {
        for (int c = tid; c < BC * (DKP / 4); c += NT) {
            const int r = c / (DKP / 4), c4 = c % (DKP / 4);
            const int key = key0 + r;
            *reinterpret_cast<f32x4 *>(&sK[r * LK + 4 * c4]) =
                key < p.M ? load_row4(kbase + (size_t)p.DK * key, 4 * c4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
        }
        for (int c = tid; c < BC * (DVP / 4); c += NT) {
            const int r = c / (DVP / 4), c4 = c % (DVP / 4);
            const int key = key0 + r;
            *reinterpret_cast<f32x4 *>(&sV[r * LV + 4 * c4]) =
                key < p.M ? load_row4(vbase + (size_t)p.DV * key, 4 * c4, p.DV, p.vecV) : f32x4{0, 0, 0, 0};
        }
    }

    f32x16 dkacc[DKP / 32], dvacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DKP / 32; ++i) dkacc[i] = zero16();
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) dvacc[i] = zero16();
    const float sl2 = p.scale * kLog2e;
    const int nqtiles = (p.N + BR - 1) / BR;

    for (int it = 0; it < nqtiles; ++it) {
        const int cls = tile_class(p.map, p.nqb, p.nkb, it * (BR / kMapTile), BR / kMapTile,
                                   key0 / kMapTile, BC / kMapTile);
        if (cls == kBlockSkip) continue;
        const int q0 = it * BR;
        __syncthreads();  // the previous step is done with sQ, sdO, sdS
        // ---- stage Q_i and dO_i (bf16: also transposed, queries in MFMA operand order)
        if constexpr (BF16) {
            for (int c = tid; c < (BR / 8) * (DKP / 4); c += NT) {
                const int rg = c / (DKP / 4), c4 = c % (DKP / 4);
                f32x4 x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int n = q0 + 8 * rg + i;
                    x[i] = n < p.N ? load_row4(qbase + (size_t)p.DK * n, 4 * c4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
                    *reinterpret_cast<bf16x4 *>(&sQ[(8 * rg + i) * LQ + 4 * c4]) = to_bf16x4(x[i]);
                }
                const int base = 16 * (rg >> 1) + 4 * (rg & 1);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 lo, hi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) { lo[i] = (__bf16)x[i][jj]; hi[i] = (__bf16)x[4 + i][jj]; }
                    *reinterpret_cast<bf16x4 *>(&sQt[(4 * c4 + jj) * LQT + base]) = lo;
                    *reinterpret_cast<bf16x4 *>(&sQt[(4 * c4 + jj) * LQT + base + 8]) = hi;
                }
            }
            for (int c = tid; c < (BR / 8) * (DVP / 4); c += NT) {
                const int rg = c / (DVP / 4), c4 = c % (DVP / 4);
                f32x4 x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int n = q0 + 8 * rg + i;
                    x[i] = n < p.N ? load_row4(dbase + dstride * n, 4 * c4, p.DV, p.vecV) : f32x4{0, 0, 0, 0};
                    *reinterpret_cast<bf16x4 *>(&sdO[(8 * rg + i) * LDO + 4 * c4]) = to_bf16x4(x[i]);
                }
                const int base = 16 * (rg >> 1) + 4 * (rg & 1);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 lo, hi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) { lo[i] = (__bf16)x[i][jj]; hi[i] = (__bf16)x[4 + i][jj]; }
                    *reinterpret_cast<bf16x4 *>(&sdOt[(4 * c4 + jj) * LDOT + base]) = lo;
                    *reinterpret_cast<bf16x4 *>(&sdOt[(4 * c4 + jj) * LDOT + base + 8]) = hi;
                }
            }
        } else {
            for (int c = tid; c < BR * (DKP / 4); c += NT) {
                const int r = c / (DKP / 4), c4 = c % (DKP / 4);
                const int n = q0 + r;
                *reinterpret_cast<f32x4 *>(&sQ[r * LQ + 4 * c4]) =
                    n < p.N ? load_row4(qbase + (size_t)p.DK * n, 4 * c4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
            }
            for (int c = tid; c < BR * (DVP / 4); c += NT) {
                const int r = c / (DVP / 4), c4 = c % (DVP / 4);
                const int n = q0 + r;
                *reinterpret_cast<f32x4 *>(&sdO[r * LDO + 4 * c4]) =
                    n < p.N ? load_row4(dbase + dstride * n, 4 * c4, p.DV, p.vecV) : f32x4{0, 0, 0, 0};
            }
        }
        if (tid < BR) {
            const int n = q0 + tid;
            float L = -INFINITY, Dl = 0.f;
            if (n < p.N) {
                L = p.lse[n + p.N * (h + p.H * b)];
                Dl = p.delta[n + p.N * (h + p.H * b)];
            }
            // an all-masked row (LSE = -inf) gets P = exp2(s - inf) = 0
            sLSE[tid] = (L == -INFINITY) ? INFINITY : L * kLog2e;
            sDel[tid] = Dl;
        }
        __syncthreads();

        // ---- S = Q K^T and dP = dO V^T for this wave's 32 keys (lane = key, rows = queries)
        f32x16 sacc[NQT], pacc[NQT];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) { sacc[qt] = zero16(); pacc[qt] = zero16(); }
        if constexpr (BF16) {
#pragma unroll
            for (int t = 0; t < DKP / 16; ++t)
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sQ[(qt * 32 + l32) * LQ + 16 * t + 8 * half]);
                    sacc[qt] = mfma_bf16(a, kf[t], sacc[qt]);
                }
#pragma unroll
            for (int t = 0; t < DVP / 16; ++t)
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sdO[(qt * 32 + l32) * LDO + 16 * t + 8 * half]);
                    pacc[qt] = mfma_bf16(a, vf[t], pacc[qt]);
                }
        } else {
            const T *kr = &sK[(32 * w + l32) * LK + half * (DKP / 2)];
            const T *vr = &sV[(32 * w + l32) * LV + half * (DVP / 2)];
#pragma unroll
            for (int t = 0; t < DKP / 2; t += 4) {
                const f32x4 bk = *reinterpret_cast<const f32x4 *>(kr + t);
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(&sQ[(qt * 32 + l32) * LQ + half * (DKP / 2) + t]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) sacc[qt] = mfma_f32(a[i], bk[i], sacc[qt]);
                }
            }
#pragma unroll
            for (int t = 0; t < DVP / 2; t += 4) {
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(vr + t);
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(&sdO[(qt * 32 + l32) * LDO + half * (DVP / 2) + t]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) pacc[qt] = mfma_f32(a[i], bv[i], pacc[qt]);
                }
            }
        }

        // ---- P = exp(scale*S + mask - LSE), dS = P o (dP - D)
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int qr = qt * 32 + 8 * r4 + 4 * half;
                const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(&sLSE[qr]);
                const f32x4 del4 = *reinterpret_cast<const f32x4 *>(&sDel[qr]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * r4 + c;
                    float x = sacc[qt][r] * sl2;
                    if (cls == kBlockMixed) {
                        const int n = q0 + qr + c;
                        if (n < p.N && keyok) x += half_bits_to_float(p.mask[mykey + (size_t)p.M * n]) * kLog2e;
                    }
                    const float P = keyok ? exp2f(x - lse4[c]) : 0.f;
                    sacc[qt][r] = P;
                    pacc[qt][r] = P * (pacc[qt][r] - del4[c]);
                }
            }

        // ---- dV += P^T dO and dK += dS^T Q (lane = head-dim column, rows = keys)
        if constexpr (BF16) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float pv[8], dv8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) { pv[i] = sacc[qt][8 * u + i]; dv8[i] = pacc[qt][8 * u + i]; }
                    const bf16x8 pa = to_bf16x8(pv), da = to_bf16x8(dv8);
#pragma unroll
                    for (int dt = 0; dt < DVP / 32; ++dt) {
                        const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(
                            &sdOt[(dt * 32 + l32) * LDOT + qt * 32 + 16 * u + 8 * half]);
                        dvacc[dt] = mfma_bf16(pa, bb, dvacc[dt]);
                    }
#pragma unroll
                    for (int dt = 0; dt < DKP / 32; ++dt) {
                        const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(
                            &sQt[(dt * 32 + l32) * LQT + qt * 32 + 16 * u + 8 * half]);
                        dkacc[dt] = mfma_bf16(da, bb, dkacc[dt]);
                    }
                }
        } else {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int qr = qt * 32 + crow(u, half);
#pragma unroll
                    for (int dt = 0; dt < DVP / 32; ++dt)
                        dvacc[dt] = mfma_f32(sacc[qt][u], sdO[qr * LDO + dt * 32 + l32], dvacc[dt]);
#pragma unroll
                    for (int dt = 0; dt < DKP / 32; ++dt)
                        dkacc[dt] = mfma_f32(pacc[qt][u], sQ[qr * LQ + dt * 32 + l32], dkacc[dt]);
                }
        }

        // ---- dS to LDS as [query][key] for dQ = dS K
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sdS[(qt * 32 + crow(r, half)) * LS + 32 * w + l32] = (T)pacc[qt][r];
        __syncthreads();

        // ---- dQ tiles (32 queries x 32 head dims), round-robin over the waves
        constexpr int NDT = DKP / 32;
        for (int ti = w; ti < NQT * NDT; ti += W) {
            const int qt = ti / NDT, dt = ti % NDT;
            f32x16 acc = zero16();
            if constexpr (BF16) {
#pragma unroll
                for (int t = 0; t < BC / 16; ++t) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sdS[(qt * 32 + l32) * LS + 16 * t + 8 * half]);
                    const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(&sKt[(dt * 32 + l32) * LKT + 16 * t + 8 * half]);
                    acc = mfma_bf16(a, bb, acc);
                }
            } else {
#pragma unroll
                for (int t = 0; t < BC / 2; t += 4) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(&sdS[(qt * 32 + l32) * LS + half * (BC / 2) + t]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = mfma_f32(a[i], sK[(half * (BC / 2) + t + i) * LK + dt * 32 + l32], acc);
                }
            }
            const int col = dt * 32 + l32;
            if (col < p.DK) {
                float *dqcol = p.dq + col + (size_t)p.DK * p.N * (h + p.H * b);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = q0 + qt * 32 + crow(r, half);
                    if (n < p.N) unsafeAtomicAdd(dqcol + (size_t)p.DK * n, acc[r] * p.scale);
                }
            }
        }
    }

    // ---- store dK (scaled) and dV for this key block
    const int hd = p.part_heads ? h : g, Hd = p.part_heads ? p.H : p.Hkv;
    float *dkb = p.dk + (size_t)p.DK * p.M * (hd + Hd * b);
    float *dvb = p.dv + (size_t)p.DV * p.M * (hd + Hd * b);
#pragma unroll
    for (int dt = 0; dt < DKP / 32; ++dt) {
        const int col = dt * 32 + l32;
        if (col < p.DK)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * w + crow(r, half);
                if (key < p.M) dkb[col + (size_t)p.DK * key] = dkacc[dt][r] * p.scale;
            }
    }
#pragma unroll
    for (int dt = 0; dt < DVP / 32; ++dt) {
        const int col = dt * 32 + l32;
        if (col < p.DV)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * w + crow(r, half);
                if (key < p.M) dvb[col + (size_t)p.DV * key] = dvacc[dt][r];
            }
    }
}

// ============================================================== launchers
int padded_dim(int d)
{
    if (d <= 0) return 0;
    if (d <= 32) return 32;
    if (d <= 64) return 64;
    if (d <= 128) return 128;
    if (d <= 192) return 192;
    return 0;
}

namespace {
// Instantiated (DKP, DVP) pairs; a shape uses the first pair covering both dims.
struct Pair { int dk, dv; };
constexpr Pair kPairs[] = {{32, 32}, {64, 64}, {128, 128}, {192, 128}, {192, 192}};

bool pick_pair(int DK, int DV, Pair *out)
{
    for (const Pair &pr : kPairs)
        if (DK <= pr.dk && DV <= pr.dv) { *out = pr; return true; }
    return false;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int DKP, int DVP, bool BF16>
hipError_t run_fwd(const FwdArgs &a, hipStream_t s)
{
    using C = FwdCfg<DKP, DVP, BF16>;
    const int grid = ceil_div(a.N, C::BR) * a.H * a.B;
    hipLaunchKernelGGL((fwd_kernel<DKP, DVP, BF16>), dim3(grid), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

template <int DKP, int DVP, bool BF16>
hipError_t run_bwd(const BwdArgs &a, hipStream_t s)
{
    using C = BwdCfg<DKP, DVP, BF16>;
    const int grid = ceil_div(a.M, C::BC) * a.H * a.B;
    hipLaunchKernelGGL((bwd_kernel<DKP, DVP, BF16>), dim3(grid), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

#define FAB_DISPATCH(FN, ARGS, STREAM, PR, BF)                                   \
    do {                                                                         \
        if ((PR).dk == 32 && (PR).dv == 32) return BF ? FN<32, 32, true>(ARGS, STREAM) : FN<32, 32, false>(ARGS, STREAM);          \
        if ((PR).dk == 64 && (PR).dv == 64) return BF ? FN<64, 64, true>(ARGS, STREAM) : FN<64, 64, false>(ARGS, STREAM);          \
        if ((PR).dk == 128 && (PR).dv == 128) return BF ? FN<128, 128, true>(ARGS, STREAM) : FN<128, 128, false>(ARGS, STREAM);    \
        if ((PR).dk == 192 && (PR).dv == 128) return BF ? FN<192, 128, true>(ARGS, STREAM) : FN<192, 128, false>(ARGS, STREAM);    \
        if ((PR).dk == 192 && (PR).dv == 192) return BF ? FN<192, 192, true>(ARGS, STREAM) : FN<192, 192, false>(ARGS, STREAM);    \
        return hipErrorInvalidValue;                                             \
    } while (0)
}  // namespace

bool bwd_supported(int dk, int dv, int)
{
    Pair pr;
    return pick_pair(dk, dv, &pr);
}

hipError_t launch_block_map(const uint16_t *mask, uint8_t *map, const Dims &d, hipStream_t s)
{
    const int nqb = ceil_div(d.N, kMapTile), nkb = ceil_div(d.M, kMapTile);
    if (nqb == 0 || nkb == 0) return hipSuccess;
    hipLaunchKernelGGL(block_map_kernel, dim3(nkb, nqb), dim3(64), 0, s, mask, map, d.N, d.M, nkb);
    return hipGetLastError();
}

hipError_t launch_forward(const float *q, const float *k, const float *v, const uint16_t *mask,
                          const uint8_t *map, float scale, int bf16, float *O, float *lse,
                          const Dims &d, hipStream_t s)
{
    Pair pr;
    if (!pick_pair(d.DK, d.DV, &pr)) return hipErrorInvalidValue;
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.mask = mask; a.map = map; a.O = O; a.lse = lse;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.DK = d.DK; a.DV = d.DV;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile);
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0);
    a.scale = scale;
    FAB_DISPATCH(run_fwd, a, s, pr, bf16);
}

hipError_t launch_prep(const float *dO, const float *O, float *delta, float *blob, int64_t nq,
                       int64_t off_k, int64_t nk, int64_t off_v, int64_t nv, int64_t total,
                       const Dims &d, hipStream_t s)
{
    PrepArgs a;
    a.dO = dO; a.O = O; a.delta = delta; a.blob = blob;
    a.zero_end = off_k;  // off_k = pad4(nq): a multiple of 4
    (void)nq;
    a.pad1_lo = off_k + nk; a.pad1_hi = off_v;
    a.pad2_lo = off_v + nv; a.pad2_hi = total;
    a.rows = d.B * d.N * d.H;
    a.DV = d.DV; a.N = d.N; a.H = d.H;
    a.vec = (d.DV % 4 == 0);
    int lpr = 1, lg = 0;
    while (lpr * 4 < d.DV && lpr < 64) { lpr *= 2; ++lg; }
    a.lpr_log2 = lg;
    const int64_t work = std::max<int64_t>((int64_t)a.rows * lpr, off_k / 4);
    int grid = (int)std::min<int64_t>((work + 255) / 256, 4096);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_backward(const float *q, const float *k, const float *v, const float *dO,
                           const uint16_t *mask, const uint8_t *map, const float *lse,
                           const float *delta, float scale, int bf16, float *dq, float *dk,
                           float *dv, int part_heads, const Dims &d, hipStream_t s)
{
    Pair pr;
    if (!pick_pair(d.DK, d.DV, &pr)) return hipErrorInvalidValue;
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dO = dO; a.mask = mask; a.map = map; a.lse = lse; a.delta = delta;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.DK = d.DK; a.DV = d.DV;
    a.part_heads = part_heads;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile);
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0);
    a.scale = scale;
    FAB_DISPATCH(run_bwd, a, s, pr, bf16);
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
