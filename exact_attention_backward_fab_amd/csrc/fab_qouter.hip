// fab_qouter.hip -- bf16 row packing and the query-block-outer kernels (gfx950).
//
//   pack_rows_bf16_kernel  f32 rows [rows][D] -> bf16 rows [rows][DP] (zero-padded
//                          columns), 16-byte chunks permuted by swz_chunk so that
//                          a tile can be copied linearly into LDS
//   fwd_bf16_kernel        O = softmax(scale S + mask) V and the row LSE by query
//                          blocks, with the running max and running sum of the
//                          labml "Flash Attention" page ("Flash Attention
//                          Optimization")
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

// Work-group shape of the query-block-outer kernels: 4 waves, 32 queries each;
// keys stream through LDS 64 at a time.
constexpr int kQW = 4, kQNT = 64 * kQW, kQBQ = 32 * kQW, kQBK = 64;
constexpr int kQList = 1024;   // live key steps listed at a time

// Streams the live key steps (block map) of one query block through two LDS
// buffers: the bf16 K and V rows of step s+1 are copied from global memory
// straight into LDS (buffer_load ... lds, 16 bytes per lane, consecutive lanes
// to consecutive LDS addresses) while body(step, class, K tile, V tile) works on
// step s.  Copies are issued per wave in 1 KiB blocks; a wave waits for its own
// copies and the barrier publishes them to the work-group.
template <int DKP, int DVP, typename ClassOf, typename Body>
__device__ __forceinline__ void stream_key_steps(rsrc_t rk, rsrc_t rv, __bf16 *sK, __bf16 *sV, int *sList,
                                                 int *sCount, int nks, int tid, int lane, int w, ClassOf class_of,
                                                 Body body)
{
    constexpr int KCH = kQBK * DKP / (8 * kQNT), VCH = kQBK * DVP / (8 * kQNT);   // copies per lane
    static_assert(KCH * 8 * kQNT == kQBK * DKP && VCH * 8 * kQNT == kQBK * DVP, "tile copy split");
    typedef __attribute__((address_space(3))) void lds_void;
    auto issue = [&](int s, int bf) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int blk = i * kQW + w;   // 1 KiB block of the tile
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)&sK[bf * kQBK * DKP + blk * 512], 16,
                                                     (uint32_t)(s * kQBK * DKP) * 2u + (uint32_t)(blk * 64 + lane) * 16u,
                                                     0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int blk = i * kQW + w;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)&sV[bf * kQBK * DVP + blk * 512], 16,
                                                     (uint32_t)(s * kQBK * DVP) * 2u + (uint32_t)(blk * 64 + lane) * 16u,
                                                     0, 0, 0);
        }
    };
    for (int seg = 0; seg < nks; seg += kQList) {
        const int count = build_live_list<kQW>(sList, sCount, seg, min(seg + kQList, nks), tid, lane, w, class_of);
        if (count == 0) continue;
        issue(sList[0] >> 2, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int buf = 0;
        for (int li = 0; li < count; ++li) {
            const int e = sList[li];
            if (li + 1 < count) issue(sList[li + 1] >> 2, buf ^ 1);
            body(e >> 2, e & 3, (const __bf16 *)&sK[buf * kQBK * DKP], (const __bf16 *)&sV[buf * kQBK * DVP]);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of the next step landed
            __syncthreads();                                   // every wave is done with this buffer
            buf ^= 1;
        }
    }
}

// Per-lane query operands: B operands of S^T = K Q^T (Q rows, f32 -> bf16) for
// query row `row` (all zero when !ok).
template <int DKP>
__device__ __forceinline__ void load_q_operand(bf16x8 *qf, const float *qr, bool ok, int DK, int vecK, int half)
{
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DKP / 16; ++t) {
        const f32x4 lo = ok ? load_row4(qr, 16 * t + 8 * half, DK, vecK) : z;
        const f32x4 hi = ok ? load_row4(qr, 16 * t + 8 * half + 4, DK, vecK) : z;
        qf[t] = __builtin_shufflevector(to_bf16x4(lo), to_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// S^T for one 32-key sub-tile (rows kk*32.. of the K tile): lane = query.
template <int DKP>
__device__ __forceinline__ f32x16 st_tile(const __bf16 *Kb, const bf16x8 *qf, int kk, int l32, int half)
{
    using KL = RowTile<DKP>;
    f32x16 acc = zero16();
    bf16x8 a[DKP / 16];
#pragma unroll
    for (int t = 0; t < DKP / 16; ++t)
        a[t] = *reinterpret_cast<const bf16x8 *>(&Kb[KL::off(kk * 32 + l32, 16 * t + 8 * half)]);
#pragma unroll
    for (int t = 0; t < DKP / 16; ++t) acc = mfma_bf16(a[t], qf[t], acc);
    return acc;
}

// Scaled scores (log2 units) of a 64-key step for the lane's query: keys past
// lim get -inf; MIXED steps add the mask row of the query.
__device__ __forceinline__ void scale_and_mask(f32x16 *st, int key0, int lim, bool mixed, const uint16_t *mrow, int M,
                                               float sl2, int half)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = st[kk][r] * sl2;
            st[kk][r] = (key0 + kk * 32 + crow(r, half) <= lim) ? x : -INFINITY;
        }
    if (mixed) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st[kk][r] += half_bits_to_float(mrow[min(key0 + kk * 32 + crow(r, half), M - 1)]) * kLog2e;
    }
}

// ============================================================== forward
struct FwdArgs16 {
    const float *q;
    const __bf16 *k16, *v16;        // bf16 swizzled [B,Hkv,Mp,DKP] / [B,Hkv,Mp,DVP], rows >= M zero
    const uint16_t *mask;
    const uint8_t *map;
    float *O, *lse;                 // O [DV,H,N,B], lse [N,H,B]
    int B, H, Hkv, N, M, Mp, DK, DV, nqb, nkb, vecK, vecV;
    float scale;
};

template <int DKP, int DVP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_bf16_kernel(FwdArgs16 p)
{
    using VL = RowTile<DVP>;
    __shared__ __attribute__((aligned(16))) __bf16 sK[2 * kQBK * DKP];
    __shared__ __attribute__((aligned(16))) __bf16 sV[2 * kQBK * DVP];
    __shared__ int sList[kQList];
    __shared__ int sCount[kQW + 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int HB = p.H * p.B;
    const int nqt = (p.N + kQBQ - 1) / kQBQ;
    const int qt = nqt - 1 - (int)(blockIdx.x / HB);  // latest queries first: most keys under a causal mask
    const int hb = blockIdx.x % HB;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int q0 = qt * kQBQ;
    const int myq = q0 + 32 * w + l32;  // this lane's query (C-layout column of S^T and O^T)
    const bool qok = myq < p.N;
    const size_t hrow = (size_t)p.N * (h + p.H * b);
    const size_t kvrow = (size_t)p.Mp * (g + p.Hkv * b);
    const rsrc_t rk = make_rsrc(p.k16 + kvrow * DKP, (uint32_t)(p.Mp * DKP) * 2u);
    const rsrc_t rv = make_rsrc(p.v16 + kvrow * DVP, (uint32_t)(p.Mp * DVP) * 2u);

    bf16x8 qf[DKP / 16];
    load_q_operand<DKP>(qf, p.q + (hrow + (qok ? myq : 0)) * p.DK, qok, p.DK, p.vecK, half);
    f32x16 oacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) oacc[i] = zero16();
    float m_run = -INFINITY, l_part = 0.f;   // running max (log2 units), this half's running sum
    const float sl2 = p.scale * kLog2e;
    const uint16_t *mrow = p.mask + (size_t)p.M * min(myq, p.N - 1);

    stream_key_steps<DKP, DVP>(
        rk, rv, sK, sV, sList, sCount, (p.M + kQBK - 1) / kQBK, tid, lane, w,
        [&](int s) {
            return tile_class(p.map, p.nqb, p.nkb, q0 / kMapTile, kQBQ / kMapTile, s * (kQBK / kMapTile),
                              kQBK / kMapTile);
        },
        [&](int s, int cls, const __bf16 *Kb, const __bf16 *Vb) {
            const int key0 = s * kQBK;
            f32x16 st[2];
            st[0] = st_tile<DKP>(Kb, qf, 0, l32, half);
            st[1] = st_tile<DKP>(Kb, qf, 1, l32, half);
            const int lim = qok ? min(cls == kTileCausal ? myq : INT_MAX, p.M - 1) : -1;
            scale_and_mask(st, key0, lim, cls == kTileMixed, mrow, p.M, sl2, half);

            // ---- running max and sum; the two lane halves hold the same query
            float mloc = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, st[kk][r]);
            mloc = swap_halves_max(mloc);
            const float m_new = fmaxf(m_run, mloc);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // all -inf so far: P = 0
            const float alpha = fast_exp2(m_run - m_use);
            float lsum = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(st[kk][r] - m_use);
                    st[kk][r] = e;
                    lsum += e;
                }
            l_part = l_part * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int i = 0; i < DVP / 32; ++i) oacc[i] *= alpha;

            // ---- O^T += V^T P^T: A = V^T by transposing reads (key rows 16u + 4*half
            // (+8) of the sub-tile), B = P^T (lane = query, keys in operand order)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float pv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) pv[i] = st[kk][8 * u + i];
                    const bf16x8 pb = to_bf16x8(pv);
                    bf16x8 av[DVP / 32];
#pragma unroll
                    for (int dt = 0; dt < DVP / 32; ++dt)
                        av[dt] = tile_col8<VL>(Vb, kk * 32 + 16 * u + 4 * half, 8, dt * 32, lane);
#pragma unroll
                    for (int dt = 0; dt < DVP / 32; ++dt) oacc[dt] = mfma_bf16(av[dt], pb, oacc[dt]);
                }
        });

    // ---- normalise and store O [DV,H,N,B] and the natural-log LSE [N,H,B]
    const float l = swap_halves_sum(l_part);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (qok) {
        float *orow = p.O + (size_t)p.DV * (h + p.H * (myq + (size_t)p.N * b));
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
        if (half == 0) p.lse[hrow + myq] = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    }
}

template <int DKP, int DVP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void dq_bf16_kernel(DqArgs p)
{
    using KL = RowTile<DKP>;
    using VL = RowTile<DVP>;
    __shared__ __attribute__((aligned(16))) __bf16 sK[2 * kQBK * DKP];
    __shared__ __attribute__((aligned(16))) __bf16 sV[2 * kQBK * DVP];
    __shared__ int sList[kQList];
    __shared__ int sCount[kQW + 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int HB = p.H * p.B;
    const int nqt = (p.N + kQBQ - 1) / kQBQ;
    const int qt = nqt - 1 - (int)(blockIdx.x / HB);  // latest queries first: most keys under a causal mask
    const int hb = blockIdx.x % HB;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int q0 = qt * kQBQ;
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
    load_q_operand<DKP>(qf, p.q + (hrow + (qok ? myq : 0)) * p.DK, qok, p.DK, p.vecK, half);
    {
        const __bf16 *orow = p.dO16 + (hrow + (qok ? myq : 0)) * DVP;
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
    const uint16_t *mrow = p.mask + (size_t)p.M * min(myq, p.N - 1);

    stream_key_steps<DKP, DVP>(
        rk, rv, sK, sV, sList, sCount, (p.M + kQBK - 1) / kQBK, tid, lane, w,
        [&](int s) {
            return tile_class(p.map, p.nqb, p.nkb, q0 / kMapTile, kQBQ / kMapTile, s * (kQBK / kMapTile),
                              kQBK / kMapTile);
        },
        [&](int s, int cls, const __bf16 *Kb, const __bf16 *Vb) {
            const int key0 = s * kQBK;
            // ---- S^T = K Q^T and dP^T = V dO^T for two 32-key sub-tiles (lane = query)
            f32x16 st[2], pt[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                st[kk] = st_tile<DKP>(Kb, qf, kk, l32, half);
                pt[kk] = zero16();
                bf16x8 av[DVP / 16];
#pragma unroll
                for (int t = 0; t < DVP / 16; ++t)
                    av[t] = *reinterpret_cast<const bf16x8 *>(&Vb[VL::off(kk * 32 + l32, 16 * t + 8 * half)]);
#pragma unroll
                for (int t = 0; t < DVP / 16; ++t) pt[kk] = mfma_bf16(av[t], of[t], pt[kk]);
            }

            // ---- P and dS; keys past M and (causal steps) keys after the query get -inf
            const int lim = min(cls == kTileCausal ? myq : INT_MAX, p.M - 1);
            scale_and_mask(st, key0, lim, cls == kTileMixed, mrow, p.M, sl2, half);
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
        });

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
        hipLaunchKernelGGL((dq_bf16_kernel<DKP, DVP>), dim3(ceil_div(a.N, kQBQ) * a.H * a.B), dim3(kQNT), 0, s, a);
        return hipGetLastError();
    }
}

template <int DKP, int DVP, bool BF16>
hipError_t run_fwd16(const FwdArgs16 &a, hipStream_t s)
{
    if constexpr (!BF16) {
        return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((fwd_bf16_kernel<DKP, DVP>), dim3(ceil_div(a.N, kQBQ) * a.H * a.B), dim3(kQNT), 0, s, a);
        return hipGetLastError();
    }
}
}  // namespace

hipError_t launch_forward_bf16(const float *q, const __bf16 *k16, const __bf16 *v16, const uint16_t *mask,
                               const uint8_t *map, float scale, float *O, float *lse, int Mp, const Dims &d,
                               hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    FwdArgs16 a;
    a.q = q; a.k16 = k16; a.v16 = v16; a.mask = mask; a.map = map; a.O = O; a.lse = lse;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.Mp = Mp; a.DK = d.DK; a.DV = d.DV;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile);
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0);
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_fwd16, a, s, hd, true);
}

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
