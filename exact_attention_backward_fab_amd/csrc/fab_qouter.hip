// fab_qouter.hip -- bf16 row packing and the query-block-outer dQ kernel (gfx950).
//
//   pack_rows_bf16_kernel  f32 rows [rows][D] -> bf16 rows [rows][DP] (zero-padded
//                          columns), 16-byte chunks permuted by swz_chunk so that
//                          a tile can be copied linearly into LDS
//   dq_bf16_kernel         dQ = scale dS K by query blocks: a work-group owns 128
//                          queries of one (batch, head) and streams the key
//                          blocks that see them (block map), recomputing
//                          S^T = K Q^T and dP^T = V dO^T on the matrix cores,
//                          P = exp(scale S + mask - LSE), dS = P o (dP - D)
//                          (labml "Flash Attention", "Backward pass"), and
//                          accumulating dQ in registers.  Every dQ element is
//                          written once; no atomics.
#include <algorithm>
#include <climits>

#include "fab_common.h"
#include "fab_launch.h"

namespace fab {

// ============================================================== bf16 pack
// src: heads of M rows of D floats; dst: heads of Mp >= M rows of DP bf16, rows
// M..Mp-1 and columns D..DP-1 zero.
__global__ __launch_bounds__(256) void pack_rows_bf16_kernel(const float *__restrict__ src, __bf16 *__restrict__ dst,
                                                             int64_t heads, int M, int Mp, int D, int DP, int vec)
{
    const int nch = DP / 8;
    const int64_t total = heads * Mp * nch;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t row = i / nch;                 // row of dst
        const int ch = (int)(i - row * nch);
        const int64_t hd = row / Mp;
        const int m = (int)(row - hd * Mp);
        f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
        if (m < M) {
            const float *sr = src + (hd * M + m) * D;
            lo = load_row4(sr, 8 * ch, D, vec);
            hi = load_row4(sr, 8 * ch + 4, D, vec);
        }
        __bf16 *dr = dst + row * DP + 8 * swz_chunk(m, ch, nch);
        *reinterpret_cast<bf16x8 *>(dr) = __builtin_shufflevector(to_bf16x4(lo), to_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

hipError_t launch_pack_rows_bf16(const float *src, __bf16 *dst, int64_t heads, int M, int Mp, int D, int DP,
                                 hipStream_t s)
{
    const int64_t work = heads * Mp * (DP / 8);
    if (work == 0) return hipSuccess;
    const int grid = (int)std::min<int64_t>((work + 255) / 256, 16384);
    hipLaunchKernelGGL(pack_rows_bf16_kernel, dim3(grid), dim3(256), 0, s, src, dst, heads, M, Mp, D, DP,
                       (int)(D % 4 == 0));
    return hipGetLastError();
}

// ============================================================== dQ by query blocks
struct DqArgs {
    const float *q;                 // f32 [B,H,N,DK]
    const __bf16 *k16, *v16;        // bf16 swizzled [B,Hkv,Mp,DKP] / [B,Hkv,Mp,DVP], rows >= M zero
    const __bf16 *dO16;             // bf16 [B,H,N,DVP]
    const uint16_t *mask;
    const uint8_t *map;
    const float *lse, *delta;       // [N,H,B]
    float *dq;                      // [DK,N,H,B] slice of the result blob
    int B, H, Hkv, N, M, Mp, DK, DV, nqb, nkb, vecK;
    float scale;
};

template <int DKP, int DVP>
struct DqCfg {
    static constexpr int W = 4, NT = 64 * W;
    static constexpr int BQ = 32 * W;   // queries per work-group (32 per wave)
    static constexpr int BK = 64;       // keys per step
    static constexpr int KCH = BK * DKP / (8 * NT), VCH = BK * DVP / (8 * NT);  // 16-byte copies per thread
    static constexpr int LIST = 2048;
    static_assert(KCH * 8 * NT == BK * DKP && VCH * 8 * NT == BK * DVP, "tile copy split");
};

template <int DKP, int DVP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void dq_bf16_kernel(DqArgs p)
{
    using C = DqCfg<DKP, DVP>;
    using KL = RowTile<DKP>;
    using VL = RowTile<DVP>;
    constexpr int BQ = C::BQ, BK = C::BK, W = C::W, NT = C::NT;
    __shared__ __attribute__((aligned(16))) __bf16 sK[2][BK * DKP];
    __shared__ __attribute__((aligned(16))) __bf16 sV[2][BK * DVP];
    __shared__ int sList[C::LIST];
    __shared__ int sCount[W + 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int HB = p.H * p.B;
    const int nqt = (p.N + BQ - 1) / BQ;
    const int qt = nqt - 1 - (int)(blockIdx.x / HB);  // latest queries first: most keys under a causal mask
    const int hb = blockIdx.x % HB;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int q0 = qt * BQ;
    const int myq = q0 + 32 * w + l32;  // this lane's query (C-layout column of S^T and dP^T)
    const bool qok = myq < p.N;
    const size_t hrow = (size_t)p.N * (h + p.H * b);
    const size_t kvrow = (size_t)p.Mp * (g + p.Hkv * b);
    const rsrc_t rk = make_rsrc(p.k16 + kvrow * DKP, (uint32_t)(p.Mp * DKP) * 2u);
    const rsrc_t rv = make_rsrc(p.v16 + kvrow * DVP, (uint32_t)(p.Mp * DVP) * 2u);

    // ---- this lane's query: LSE (log2 units, +inf when all-masked or past N), D,
    // and the B operands Q^T and dO^T of S^T = K Q^T and dP^T = V dO^T
    float lse2 = INFINITY, dl = 0.f;
    if (qok) {
        const float L = p.lse[hrow + myq];
        lse2 = (L == -INFINITY) ? INFINITY : L * kLog2e;
        dl = p.delta[hrow + myq];
    }
    bf16x8 qf[DKP / 16], of[DVP / 16];
    {
        const float *qr = p.q + (hrow + (qok ? myq : 0)) * p.DK;
        const __bf16 *orow = p.dO16 + (hrow + (qok ? myq : 0)) * DVP;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DKP / 16; ++t) {
            const f32x4 lo = qok ? load_row4(qr, 16 * t + 8 * half, p.DK, p.vecK) : z;
            const f32x4 hi = qok ? load_row4(qr, 16 * t + 8 * half + 4, p.DK, p.vecK) : z;
            qf[t] = __builtin_shufflevector(to_bf16x4(lo), to_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int t = 0; t < DVP / 16; ++t) {
            const u32x4 x = qok ? *reinterpret_cast<const u32x4 *>(orow + 16 * t + 8 * half) : u32x4{0u, 0u, 0u, 0u};
            of[t] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 dqacc[DKP / 32];
#pragma unroll
    for (int i = 0; i < DKP / 32; ++i) dqacc[i] = zero16();
    const float sl2 = p.scale * kLog2e;
    const int nks = (p.M + BK - 1) / BK;

    // copies key step s into buffer bf, straight from global memory into LDS
    auto issue = [&](int s, int bf) {
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
            const int blk = i * W + w;   // 1 KiB block of the tile
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void *)&sK[bf][blk * 512], 16,
                                                     (uint32_t)(s * BK * DKP) * 2u + (uint32_t)(blk * 64 + lane) * 16u,
                                                     0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::VCH; ++i) {
            const int blk = i * W + w;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void *)&sV[bf][blk * 512], 16,
                                                     (uint32_t)(s * BK * DVP) * 2u + (uint32_t)(blk * 64 + lane) * 16u,
                                                     0, 0, 0);
        }
    };

    for (int seg = 0; seg < nks; seg += C::LIST) {
        const int count = build_live_list<W>(
            sList, sCount, seg, min(seg + C::LIST, nks), tid, lane, w,
            [&](int s) { return tile_class(p.map, p.nqb, p.nkb, q0 / kMapTile, BQ / kMapTile, s * (BK / kMapTile),
                                           BK / kMapTile); });
        if (count == 0) continue;
        issue(sList[0] >> 2, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        int buf = 0;
        for (int li = 0; li < count; ++li) {
            const int e = sList[li];
            const int s = e >> 2, cls = e & 3;
            const int key0 = s * BK;
            if (li + 1 < count) issue(sList[li + 1] >> 2, buf ^ 1);
            const __bf16 *Kb = sK[buf];
            const __bf16 *Vb = sV[buf];

            // ---- S^T = K Q^T and dP^T = V dO^T for two 32-key sub-tiles (lane = query)
            f32x16 st[2], pt[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                st[kk] = zero16();
                pt[kk] = zero16();
                bf16x8 a[DKP / 16];
#pragma unroll
                for (int t = 0; t < DKP / 16; ++t)
                    a[t] = *reinterpret_cast<const bf16x8 *>(&Kb[KL::off(kk * 32 + l32, 16 * t + 8 * half)]);
#pragma unroll
                for (int t = 0; t < DKP / 16; ++t) st[kk] = mfma_bf16(a[t], qf[t], st[kk]);
                bf16x8 av[DVP / 16];
#pragma unroll
                for (int t = 0; t < DVP / 16; ++t)
                    av[t] = *reinterpret_cast<const bf16x8 *>(&Vb[VL::off(kk * 32 + l32, 16 * t + 8 * half)]);
#pragma unroll
                for (int t = 0; t < DVP / 16; ++t) pt[kk] = mfma_bf16(av[t], of[t], pt[kk]);
            }

            // ---- P and dS; keys past M and (causal tiles) keys after the query get -inf
            const int lim = min(cls == kTileCausal ? myq : INT_MAX, p.M - 1);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = st[kk][r] * sl2;
                    st[kk][r] = (key0 + kk * 32 + crow(r, half) <= lim) ? x : -INFINITY;
                }
            if (cls == kTileMixed) {
                const uint16_t *mrow = p.mask + (size_t)p.M * min(myq, p.N - 1);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        st[kk][r] += half_bits_to_float(mrow[min(key0 + kk * 32 + crow(r, half), p.M - 1)]) * kLog2e;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float P = fast_exp2(st[kk][r] - lse2);
                    pt[kk][r] = P * (pt[kk][r] - dl);
                }

            // ---- dQ += dS K: A = dS (lane = query, keys in operand order), B = K via
            // transposing reads (key rows 16u + 4*half (+8) of the sub-tile)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float d8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) d8[i] = pt[kk][8 * u + i];
                    const bf16x8 da = to_bf16x8(d8);
                    bf16x8 bk[DKP / 32];
#pragma unroll
                    for (int dt = 0; dt < DKP / 32; ++dt)
                        bk[dt] = tile_col8<KL>(Kb, kk * 32 + 16 * u + 4 * half, 8, dt * 32, lane);
#pragma unroll
                    for (int dt = 0; dt < DKP / 32; ++dt) dqacc[dt] = mfma_bf16(da, bk[dt], dqacc[dt]);
                }

            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of the next step landed
            __syncthreads();                                   // every wave is done with this buffer
            buf ^= 1;
        }
    }

    // ---- store dQ (scaled): lane = head-dim column, rows = this wave's queries
    float *dqh = p.dq + hrow * p.DK;
#pragma unroll
    for (int dt = 0; dt < DKP / 32; ++dt) {
        const int col = dt * 32 + l32;
        if (col < p.DK)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = q0 + 32 * w + crow(r, half);
                if (n < p.N) dqh[(size_t)n * p.DK + col] = dqacc[dt][r] * p.scale;
            }
    }
}

namespace {
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int DKP, int DVP, bool BF16>
hipError_t run_dq(const DqArgs &a, hipStream_t s)
{
    if constexpr (!BF16) {
        return hipErrorInvalidValue;
    } else {
        using C = DqCfg<DKP, DVP>;
        hipLaunchKernelGGL((dq_bf16_kernel<DKP, DVP>), dim3(ceil_div(a.N, C::BQ) * a.H * a.B), dim3(C::NT), 0, s, a);
        return hipGetLastError();
    }
}
}  // namespace

hipError_t launch_dq(const float *q, const __bf16 *k16, const __bf16 *v16, const __bf16 *dO16, const uint16_t *mask,
                     const uint8_t *map, const float *lse, const float *delta, float scale, float *dq, int Mp,
                     const Dims &d, hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    DqArgs a;
    a.q = q; a.k16 = k16; a.v16 = v16; a.dO16 = dO16; a.mask = mask; a.map = map;
    a.lse = lse; a.delta = delta; a.dq = dq;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.Mp = Mp; a.DK = d.DK; a.DV = d.DV;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile);
    a.vecK = (d.DK % 4 == 0);
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_dq, a, s, hd, true);
}

}  // namespace fab
