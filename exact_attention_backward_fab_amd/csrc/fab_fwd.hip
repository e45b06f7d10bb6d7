// fab_fwd.hip -- f32-mode forward with row log-sum-exp (gfx950): O =
// softmax(scale*q.k + mask) v and LSE = log sum exp, by query blocks with the
// running max and running sum of the labml "Flash Attention" page ("Flash
// Attention Optimization"); the dense products run on the f32 matrix cores
// (v_mfma_f32_32x32x2_f32).  The bf16 forward is fwd_bf16_kernel in
// fab_qouter.hip.
#include <algorithm>

#include "fab_common.h"
#include "fab_launch.h"

namespace fab {

// ============================================================== forward
struct FwdArgs {
    const float *q, *k, *v;
    const uint16_t *mask;
    const uint8_t *map;
    float *O, *lse;
    int B, H, Hkv, N, M, DK, DV;
    int nqb, nkb, vecK, vecV;
    int causal;                     // causal rule as a flag (no mask, no map)
    int fold;                       // the whole grid is resident at once (query_block_work)
    float scale;
    const float *alibi;             // per-head ALiBi slopes [H] or NULL
};

// KS = 2 (grids with fewer work-groups than one resident round can hold): each
// 32-query tile is shared by two waves that take the two 32-key halves of every
// step, each with its own running max, sum and O, merged once at the end.  KS = 4
// (smaller grids, head dims up to 64): one 32-query tile per work-group, 128-key
// steps whose four 32-key parts go to the four waves.
template <int DKP, int DVP, int KS = 1>
struct FwdCfg {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;
    static constexpr int BR = 32 * WAVES / KS;  // queries per work-group (32 per query tile)
    static constexpr int BC = KS == 4 ? 128 : 64;   // keys per step
    static constexpr int LK = DKP + 4;     // sK row stride (floats)
    static constexpr int LV = DVP + 4;     // sV row stride
};

// Two waves per SIMD where the operands fit 256 registers per wave (the head
// dims up to 128), else one.
template <int DKP, int DVP>
struct FwdF32Occ {
    static constexpr int v = DKP + DVP <= 256 ? 2 : 1;
};

template <int DKP, int DVP, bool AB, int KS = 1>
__global__ __launch_bounds__(256, (FwdF32Occ<DKP, DVP>::v))
__attribute__((amdgpu_waves_per_eu(FwdF32Occ<DKP, DVP>::v, FwdF32Occ<DKP, DVP>::v))) void fwd_f32_kernel(FwdArgs p)
{
    using C = FwdCfg<DKP, DVP, KS>;
    constexpr int BC = C::BC, BR = C::BR, NT = C::NT, LK = C::LK, LV = C::LV;
    constexpr int NKT = BC / 32, NKW = NKT / KS;   // 32-key sub-tiles of a step, of a wave
    constexpr int QW = C::WAVES / KS;              // 32-query tiles of the work-group
    __shared__ __attribute__((aligned(16))) float sK[BC * LK];
    __shared__ __attribute__((aligned(16))) float sV[BC * LV];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int qw = KS == 1 ? w : w % QW, kh = KS == 1 ? 0 : w / QW;   // query tile, key half of this wave
    const int kk0 = KS == 1 ? 0 : kh * NKW;  // first sub-tile of each step this wave takes
    const int nqt = (p.N + BR - 1) / BR;
    int qt, hb;
    query_block_work(blockIdx.x, nqt, p.H * p.B, p.fold, &qt, &hb);
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int n = qt * BR + qw * 32 + l32;  // this lane's query (C-layout column)
    const bool nok = n < p.N;
    const float *kbase = p.k + (size_t)p.DK * p.M * (g + p.Hkv * b);
    const float *vbase = p.v + (size_t)p.DV * p.M * (g + p.Hkv * b);
    const float *qrow = p.q + (size_t)p.DK * (nok ? (n + p.N * (h + p.H * b)) : 0);

    // Q fragments: B operand of S^T = K Q^T (column = query, k = head dim)
    float qf[DKP / 2];
#pragma unroll
    for (int t = 0; t < DKP / 2; t += 4) {
        const f32x4 x = nok ? load_row4(qrow, half * (DKP / 2) + t, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) qf[t + i] = x[i];
    }

    f32x16 oacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) oacc[i] = zero16();
    float m_run = -INFINITY, l_half = 0.f;
    const float sl2 = p.scale * kLog2e;
    const float slope2 = AB ? p.alibi[h] * kLog2e : 0.f;   // ALiBi, log2 units
    const int nkt_total = (p.M + BC - 1) / BC;

    // Live key steps only.  Where one work-group fills the CU (the wide heads), no
    // other work-group covers the latency of a step's K and V loads: where the
    // registers also allow it (the 192/128 pair; wider pairs would spill), the rows of
    // the next live step are loaded into registers while the current step computes
    // and written to LDS at the top of the next one.
    auto next_live = [&](int from, int *c) {
        for (int kt = from; kt < nkt_total; ++kt) {
            // (a 32-query block takes the class of the 64-row map tile around it)
            *c = tile_class<(BR >= kMapTile ? BR / kMapTile : 1), BC / kMapTile>(p.map, p.causal, p.N, p.M, p.nqb,
                                                                             p.nkb, qt * BR / kMapTile, kt * (BC / kMapTile));
            if (*c != kTileSkip) return kt;
        }
        return nkt_total;
    };
    constexpr bool PF = FwdF32Occ<DKP, DVP>::v == 1 && DKP + DVP <= 320;
    constexpr int PK = BC * (DKP / 4) / NT, PV = BC * (DVP / 4) / NT;   // float4 per thread and step
    static_assert(!PF || (PK * NT == BC * (DKP / 4) && PV * NT == BC * (DVP / 4)), "prefetch split");
    f32x4 pk[PF ? PK : 1], pv[PF ? PV : 1];
    auto fetch = [&](int kt) {
        const int k0 = kt * BC;
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int c = tid + i * NT, r = c / (DKP / 4), c4 = c % (DKP / 4), key = k0 + r;
            pk[i] = key < p.M ? load_row4(kbase + (size_t)p.DK * key, 4 * c4, p.DK, p.vecK) : f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int c = tid + i * NT, r = c / (DVP / 4), c4 = c % (DVP / 4), key = k0 + r;
            pv[i] = key < p.M ? load_row4(vbase + (size_t)p.DV * key, 4 * c4, p.DV, p.vecV) : f32x4{0, 0, 0, 0};
        }
    };
    int cls = kTileSkip;
    int kt = next_live(0, &cls);
    if constexpr (PF)
        if (kt < nkt_total) fetch(kt);
    while (kt < nkt_total) {
        const int key0 = kt * BC;
        int ncls = kTileSkip;
        const int nx = next_live(kt + 1, &ncls);
        __syncthreads();   // the previous step is done with sK, sV
        // ---- stage K and V rows
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < PK; ++i) {
                const int c = tid + i * NT, r = c / (DKP / 4), c4 = c % (DKP / 4);
                *reinterpret_cast<f32x4 *>(&sK[r * LK + 4 * c4]) = pk[i];
            }
#pragma unroll
            for (int i = 0; i < PV; ++i) {
                const int c = tid + i * NT, r = c / (DVP / 4), c4 = c % (DVP / 4);
                *reinterpret_cast<f32x4 *>(&sV[r * LV + 4 * c4]) = pv[i];
            }
            if (nx < nkt_total) fetch(nx);
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

        // ---- S^T = K Q^T for this wave's 32-key sub-tiles (lane = query, rows = keys)
        f32x16 s[NKW];
#pragma unroll
        for (int j = 0; j < NKW; ++j) {
            const int kk = kk0 + j;
            s[j] = zero16();
#pragma unroll
            for (int t = 0; t < DKP / 2; t += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sK[(kk * 32 + l32) * LK + half * (DKP / 2) + t]);
#pragma unroll
                for (int i = 0; i < 4; ++i) s[j] = mfma_f32(a[i], qf[t + i], s[j]);
            }
        }
        // ---- scale, mask, running max (log2 units)
        float mloc = -INFINITY;
#pragma unroll
        for (int j = 0; j < NKW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + (kk0 + j) * 32 + crow(r, half);
                float x = s[j][r] * sl2;
                if (AB && slope2 != 0.f) x += slope2 * (float)(key - n);
                if (cls == kTileMixed && nok && key < p.M)
                    x += half_bits_to_float(p.mask[key + (size_t)p.M * n]) * kLog2e;
                if (key >= p.M || !nok || (cls == kTileCausal && key > n)) x = -INFINITY;
                s[j][r] = x;
                mloc = fmaxf(mloc, x);
            }
        mloc = swap_halves_max(mloc);
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < NKW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(s[j][r] - m_use);
                s[j][r] = e;
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
            for (int j = 0; j < NKW; ++j) {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const float a = sV[((kk0 + j) * 32 + crow(u, half)) * LV + dt * 32 + l32];
                    oacc[dt] = mfma_f32(a, s[j][u], oacc[dt]);
                }
            }
        }
        kt = nx;
        cls = ncls;
    }

    // ---- KS = 2: the second key half hands its running max, sum and O to the first
    // through the K rows (no longer read); the first rescales both to the larger max
    if constexpr (KS >= 2) {
        constexpr int XO = DVP / 32 * 16;   // O values per lane
        static_assert(QW * (KS - 1) * (XO + 2) * 64 <= BC * LK, "key-part exchange area");
        auto xch = [&](int part) { return sK + ((part - 1) * QW + qw) * (XO + 2) * 64; };
        __syncthreads();   // every wave is done with sK
        if (kh >= 1) {
            float *x = xch(kh);
#pragma unroll
            for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) x[(dt * 16 + r) * 64 + lane] = oacc[dt][r];
            x[XO * 64 + lane] = m_run;
            x[(XO + 1) * 64 + lane] = l_half;
        }
        __syncthreads();
        if (kh >= 1) return;
        float m = m_run;
#pragma unroll
        for (int k = 1; k < KS; ++k) m = fmaxf(m, xch(k)[XO * 64 + lane]);
        // a part that saw no weight has max -inf and zero sum and O: its factor is 0
        const float a0 = m == -INFINITY ? 0.f : fast_exp2(m_run - m);
        l_half *= a0;
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt) oacc[dt] *= a0;
#pragma unroll
        for (int k = 1; k < KS; ++k) {
            const float *x = xch(k);
            const float ak = m == -INFINITY ? 0.f : fast_exp2(x[XO * 64 + lane] - m);
            l_half = l_half + x[(XO + 1) * 64 + lane] * ak;
#pragma unroll
            for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] = oacc[dt][r] + x[(dt * 16 + r) * 64 + lane] * ak;
        }
        m_run = m;
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

// ============================================================== launcher
namespace {
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int DKP, int DVP, bool BF16>
hipError_t run_fwd(const FwdArgs &a, hipStream_t s)
{
    if constexpr (BF16) {
        return hipErrorInvalidValue;
    } else {
        using C = FwdCfg<DKP, DVP>;
        const int grid = ceil_div(a.N, C::BR) * a.H * a.B;
        static ResidentCache slots;
        FwdArgs b = a;
        // (the instantiations have the same LDS and occupancy: one occupancy query)
        const int res = slots.get(reinterpret_cast<const void *>(&fwd_f32_kernel<DKP, DVP, false>), C::NT);
        if constexpr (DKP + DVP <= 256) {
            // each query tile's keys split over two waves (twice the work-groups of half
            // the queries, each wave holding half the scores): where the plain grid
            // leaves CUs without a work-group, where a mask or the causal rule makes the
            // query blocks' work unequal (smaller blocks balance better), and for the
            // 32-wide heads (twice the waves per SIMD); measured slower only on unmasked
            // 128-wide heads with a full grid
            const int grid2 = ceil_div(a.N, FwdCfg<DKP, DVP, 2>::BR) * a.H * a.B;
            const bool idle = grid < res / FwdF32Occ<DKP, DVP>::v;
            if constexpr (DKP + DVP <= 128) {
                // four key parts of 32 (128-key steps, 32-query work-groups) where the
                // two-part grid fills at most half of the resident slots and the four-part
                // one still fits them: causal MHA N=1024, 64-wide heads 92 -> 69 us
                const int grid4 = ceil_div(a.N, FwdCfg<DKP, DVP, 4>::BR) * a.H * a.B;
                if (grid4 <= res) {
                    b.fold = grid4 <= res;
                    if (a.alibi)
                        hipLaunchKernelGGL((fwd_f32_kernel<DKP, DVP, true, 4>), dim3(grid4), dim3(C::NT), 0, s, b);
                    else
                        hipLaunchKernelGGL((fwd_f32_kernel<DKP, DVP, false, 4>), dim3(grid4), dim3(C::NT), 0, s, b);
                    return hipGetLastError();
                }
            }
            if (DKP + DVP <= 64 || idle || a.causal || a.map) {
                b.fold = grid2 <= res;
                if (a.alibi)
                    hipLaunchKernelGGL((fwd_f32_kernel<DKP, DVP, true, 2>), dim3(grid2), dim3(C::NT), 0, s, b);
                else
                    hipLaunchKernelGGL((fwd_f32_kernel<DKP, DVP, false, 2>), dim3(grid2), dim3(C::NT), 0, s, b);
                return hipGetLastError();
            }
        }
        b.fold = grid <= res;
        if (a.alibi)
            hipLaunchKernelGGL((fwd_f32_kernel<DKP, DVP, true>), dim3(grid), dim3(C::NT), 0, s, b);
        else
            hipLaunchKernelGGL((fwd_f32_kernel<DKP, DVP, false>), dim3(grid), dim3(C::NT), 0, s, b);
        return hipGetLastError();
    }
}
}  // namespace

hipError_t launch_forward_f32(const float *q, const float *k, const float *v, const uint16_t *mask,
                              const uint8_t *map, float scale, float *O, float *lse, const Dims &d,
                              hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.mask = mask; a.map = map; a.O = O; a.lse = lse;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.DK = d.DK; a.DV = d.DV;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile); a.causal = d.causal; a.alibi = d.alibi;
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0);
    a.fold = 0;
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_fwd, a, s, hd, false);
}

}  // namespace fab
