// fab_bwd.hip -- key-block-outer attention backward (gfx950).
//
// A work-group owns one block of BC keys of one (batch, query head) and keeps
// its dK and dV in registers while it walks over the query tiles that see the
// block (the mask's block map drops the tiles that are all -inf).  For each
// query tile it recomputes S = scale Q K^T (+ mask) and P = exp(S - LSE) from
// the row log-sum-exp of the forward, then forms, as in the labml "Flash
// Attention" page ("Backward pass"):
//     dV += P^T dO,   dP = dO V^T,   dS = P o (dP - D),   dK += scale dS^T Q
// with D = rowsum(dO o O) from the prep kernel.  The products run on the
// matrix cores: bf16 operands with f32 accumulation (v_mfma_f32_32x32x16_bf16)
// or f32 operands (v_mfma_f32_32x32x2_f32).
//
// dQ = scale dS K: in bf16 mode a separate query-block-outer kernel
// (fab_qouter.hip) recomputes S and dP by query blocks and writes each dQ row
// once; in f32 mode this kernel adds every key block's share with f32 atomics
// into the result blob.
//
// Wave layout: wave w owns keys 32w..32w+31 of the block.  S and dP come out of
// the matrix core with one key per lane (the C layout, see fab_common.h), which
// is exactly the A-operand layout of P^T and dS^T for dV and dK.
#include <algorithm>

#include "fab_common.h"
#include "fab_launch.h"

namespace fab {

struct BwdArgs {
    const float *q, *k, *v, *dO;
    const __bf16 *dO16;               // bf16 mode: d as [B][H][N][DVP]
    const uint16_t *mask;
    const uint8_t *map;
    const float *lse, *delta;
    float *dq, *dk, *dv;
    int B, H, Hkv, N, M, DK, DV;
    int part_heads, nqb, nkb, vecK, vecV;
    float scale;
};

// ============================================================== bf16 mode
template <int DKP, int DVP>
struct B16Cfg {
    static constexpr int W = 4, NT = 64 * W;
    static constexpr int BC = 32 * W;   // keys per work-group (32 per wave)
    static constexpr int BR = 32;       // queries per step
    using QL = RowTile<DKP>;            // layout of Q tiles and of the K block
    using OL = RowTile<DVP>;            // layout of dO tiles
    static constexpr int QCN = BR * DKP / 4, OCN = BR * DVP / 8;   // 16-byte chunks of a Q / dO tile
    static constexpr int QCH = (QCN + NT - 1) / NT;   // f32x4 chunks of a Q tile per thread
    static constexpr int OCH = (OCN + NT - 1) / NT;   // 16-byte chunks of a bf16 dO tile per thread
    static constexpr int LIST = 2048;                 // live query tiles listed at a time
};

template <int DKP, int DVP>
struct B16Tile {
    u32x4 q[B16Cfg<DKP, DVP>::QCH];   // f32 Q (4 floats per chunk)
    u32x4 o[B16Cfg<DKP, DVP>::OCH];   // bf16 dO (8 per chunk)
    float lse, del;
};

// Per-(batch, head) views of the query-side tensors.
struct B16Head {
    rsrc_t q, o, lse, del;
    const float *qp;   // plain pointer to Q for the head-dim-padded (checked) loads
};

// Global loads of query tile rows q0..q0+BR-1 into registers.  Rows at or past N
// read as zero through the buffer bounds; EXACT (DK == DKP) needs no other
// check, otherwise the Q columns past DK are zero-filled explicitly.
template <int DKP, int DVP, bool EXACT>
__device__ __forceinline__ void b16_load(B16Tile<DKP, DVP> &t, const B16Head &hd, int q0, int N, int DK,
                                         int vecK, int tid)
{
    using C = B16Cfg<DKP, DVP>;
#pragma unroll
    for (int i = 0; i < C::QCH; ++i) {
        const int c = tid + C::NT * i;
        if (C::QCN % C::NT != 0 && c >= C::QCN) break;
        const int n = q0 + c / (DKP / 4), col = 4 * (c % (DKP / 4));
        if constexpr (EXACT) {
            t.q[i] = buf_load16(hd.q, (uint32_t)(n * DK + col) * 4u);
        } else {
            const f32x4 x = n < N ? load_row4(hd.qp + (size_t)n * DK, col, DK, vecK) : f32x4{0.f, 0.f, 0.f, 0.f};
            t.q[i] = __builtin_bit_cast(u32x4, x);
        }
    }
#pragma unroll
    for (int i = 0; i < C::OCH; ++i) {
        const int c = tid + C::NT * i;
        if (C::OCN % C::NT != 0 && c >= C::OCN) break;
        const int n = q0 + c / (DVP / 8), col = 8 * (c % (DVP / 8));
        t.o[i] = buf_load16(hd.o, (uint32_t)(n * DVP + col) * 2u);
    }
    if (tid < C::BR) {
        t.lse = buf_load_f32(hd.lse, (uint32_t)(q0 + tid) * 4u);   // 0 past N: harmless, Q = dO = 0 there
        t.del = buf_load_f32(hd.del, (uint32_t)(q0 + tid) * 4u);
    }
}

template <int DKP, int DVP>
__device__ __forceinline__ void b16_store(const B16Tile<DKP, DVP> &t, __bf16 *sQ, __bf16 *sO, float *sL,
                                          float *sD, int tid)
{
    using C = B16Cfg<DKP, DVP>;
#pragma unroll
    for (int i = 0; i < C::QCH; ++i) {
        const int c = tid + C::NT * i;
        if (C::QCN % C::NT != 0 && c >= C::QCN) break;
        *reinterpret_cast<bf16x4 *>(&sQ[C::QL::off(c / (DKP / 4), 4 * (c % (DKP / 4)))]) =
            to_bf16x4(__builtin_bit_cast(f32x4, t.q[i]));
    }
#pragma unroll
    for (int i = 0; i < C::OCH; ++i) {
        const int c = tid + C::NT * i;
        if (C::OCN % C::NT != 0 && c >= C::OCN) break;
        *reinterpret_cast<u32x4 *>(&sO[C::OL::off(c / (DVP / 8), 8 * (c % (DVP / 8)))]) = t.o[i];
    }
    if (tid < C::BR) {
        // log2 units; an all-masked row (LSE = -inf) becomes +inf so that P = 0
        sL[tid] = (t.lse == -INFINITY) ? INFINITY : t.lse * kLog2e;
        sD[tid] = t.del;
    }
}

// One query tile against the key block: S, dP, P, dS, dV and dK.
// The causal rule is applied as "query >= thr" (thr = INT_MIN when the tile
// is not causal); masked adds the additive mask values read from memory.
template <int DKP, int DVP>
__device__ __forceinline__ void b16_step(const BwdArgs &p, const __bf16 *Qb, const __bf16 *Ob, const float *sLb,
                                         const float *sDb, const __bf16 *sK, const bf16x8 *vf,
                                         f32x16 *dkacc, f32x16 *dvacc, int q0, int thr, bool masked, bool fast,
                                         int mykey, float kbias, float sl2, int w, int lane)
{
    using C = B16Cfg<DKP, DVP>;
    using QL = typename C::QL;
    using OL = typename C::OL;
    const int half = lane >> 5, l32 = lane & 31;

    // ---- S = Q K^T and dP = dO V^T (lane = key, rows = queries)
    f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
    for (int t0 = 0; t0 < DKP / 16; t0 += 8) {
        constexpr int T = DKP / 16 < 8 ? DKP / 16 : 8;
        bf16x8 bk[T], a[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t >= DKP / 16) break;
            bk[t] = *reinterpret_cast<const bf16x8 *>(&sK[QL::off(32 * w + l32, 16 * (t0 + t) + 8 * half)]);
            a[t] = *reinterpret_cast<const bf16x8 *>(&Qb[QL::off(l32, 16 * (t0 + t) + 8 * half)]);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t >= DKP / 16) break;
            sacc = mfma_bf16(a[t], bk[t], sacc);
        }
    }
#pragma unroll
    for (int t0 = 0; t0 < DVP / 16; t0 += 8) {
        constexpr int T = DVP / 16 < 8 ? DVP / 16 : 8;
        bf16x8 a[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t >= DVP / 16) break;
            a[t] = *reinterpret_cast<const bf16x8 *>(&Ob[OL::off(l32, 16 * (t0 + t) + 8 * half)]);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t >= DVP / 16) break;
            pacc = mfma_bf16(a[t], vf[t0 + t], pacc);
        }
    }

    // ---- P = exp(scale S + mask - LSE) and dS = P o (dP - D), in f32; a tile with
    // every key visible (fast) folds the scale into the exponent
    const float mul = fast ? sl2 : 1.f;
    if (!fast) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = sacc[r] * sl2 + kbias;
            sacc[r] = (q0 + crow(r, half) >= thr) ? x : -INFINITY;
        }
    }
    if (masked) {
        const uint16_t *mcol = p.mask + min(mykey, p.M - 1);   // clamped: always in bounds
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int n = min(q0 + crow(r, half), p.N - 1);
            sacc[r] += half_bits_to_float(mcol[(size_t)p.M * n]) * kLog2e;
        }
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int qr = 8 * r4 + 4 * half;
        const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(&sLb[qr]);
        const f32x4 del4 = *reinterpret_cast<const f32x4 *>(&sDb[qr]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int r = 4 * r4 + c;
            const float P = fast_exp2(__builtin_fmaf(sacc[r], mul, -lse4[c]));
            sacc[r] = P;
            pacc[r] = P * (pacc[r] - del4[c]);
        }
    }

    // ---- the bf16 A operands of dV and dK
    bf16x8 pa[2], da[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float pv[8], dv8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pv[i] = sacc[8 * u + i];
            dv8[i] = pacc[8 * u + i];
        }
        pa[u] = to_bf16x8(pv);
        da[u] = to_bf16x8(dv8);
    }

    // ---- dV += P^T dO and dK += dS^T Q (lane = head-dim column, rows = keys);
    // query rows of slots 0-3 are 16u + 4*half + 0..3, slots 4-7 are 8 further
    {
        bf16x8 bo[DVP / 32][2];
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int u = 0; u < 2; ++u) bo[dt][u] = tile_col8<OL>(Ob, 16 * u + 4 * half, 8, dt * 32, lane);
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int u = 0; u < 2; ++u) dvacc[dt] = mfma_bf16(pa[u], bo[dt][u], dvacc[dt]);
    }
    {
        bf16x8 bq[DKP / 32][2];
#pragma unroll
        for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
            for (int u = 0; u < 2; ++u) bq[dt][u] = tile_col8<QL>(Qb, 16 * u + 4 * half, 8, dt * 32, lane);
#pragma unroll
        for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
            for (int u = 0; u < 2; ++u) dkacc[dt] = mfma_bf16(da[u], bq[dt][u], dkacc[dt]);
    }
}

template <int DKP, int DVP, bool EXACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_bf16_kernel(BwdArgs p)
{
    using C = B16Cfg<DKP, DVP>;
    using QL = typename C::QL;
    using OL = typename C::OL;
    constexpr int BC = C::BC, BR = C::BR, NT = C::NT, W = C::W;
    __shared__ __attribute__((aligned(16))) __bf16 sK[BC * QL::kLd];         // K block, row-major
    __shared__ __attribute__((aligned(16))) __bf16 sQ[2][BR * QL::kLd];      // Q tiles (double buffer)
    __shared__ __attribute__((aligned(16))) __bf16 sO[2][BR * OL::kLd];      // dO tiles
    __shared__ __attribute__((aligned(16))) float sL[2][BR];                 // LSE (log2 units)
    __shared__ __attribute__((aligned(16))) float sD[2][BR];                 // D
    __shared__ int sList[C::LIST];                                           // live tiles: 4*index + class
    __shared__ int sCount[W + 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int HB = p.H * p.B;
    const int j = blockIdx.x / HB, hb = blockIdx.x % HB;  // key block slowest: heaviest first when causal
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int key0 = j * BC;
    const int mykey = key0 + 32 * w + l32;  // this lane's key in the C layout of S and dP
    const bool keyok = mykey < p.M;
    const float kbias = keyok ? 0.f : -INFINITY;  // keys past M never get weight
    const float *kh = p.k + (size_t)p.DK * p.M * (g + p.Hkv * b);
    const float *vh = p.v + (size_t)p.DV * p.M * (g + p.Hkv * b);
    const size_t hrow = (size_t)p.N * (h + p.H * b);  // first row of this (batch, head)
    B16Head hd;
    hd.qp = p.q + hrow * p.DK;
    hd.q = make_rsrc(hd.qp, (uint32_t)(p.N * p.DK) * 4u);
    hd.o = make_rsrc(p.dO16 + hrow * DVP, (uint32_t)(p.N * DVP) * 2u);
    hd.lse = make_rsrc(p.lse + hrow, (uint32_t)p.N * 4u);
    hd.del = make_rsrc(p.delta + hrow, (uint32_t)p.N * 4u);
    const int nqt = (p.N + BR - 1) / BR;
    const float sl2 = p.scale * kLog2e;

    // ---- the key block: bf16 rows in LDS (B operand of S = Q K^T), and the B
    // operand of dP = dO V^T in registers (lane = key)
    for (int c = tid; c < BC * (DKP / 4); c += NT) {
        const int r = c / (DKP / 4), col = 4 * (c % (DKP / 4));
        const int key = key0 + r;
        const f32x4 x = key < p.M ? load_row4(kh + (size_t)p.DK * key, col, p.DK, p.vecK)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<bf16x4 *>(&sK[QL::off(r, col)]) = to_bf16x4(x);
    }
    bf16x8 vf[DVP / 16];
    {
        const float *vr = vh + (size_t)p.DV * (keyok ? mykey : 0);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DVP / 16; ++t) {
            const f32x4 lo = keyok ? load_row4(vr, 16 * t + 8 * half, p.DV, p.vecV) : z;
            const f32x4 hi = keyok ? load_row4(vr, 16 * t + 8 * half + 4, p.DV, p.vecV) : z;
            vf[t] = __builtin_shufflevector(to_bf16x4(lo), to_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    f32x16 dkacc[DKP / 32], dvacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DKP / 32; ++i) dkacc[i] = zero16();
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) dvacc[i] = zero16();

    for (int seg = 0; seg < nqt; seg += C::LIST) {
        // ---- ordered list of the live query tiles of this segment (block map)
        const int count = build_live_list<W>(sList, sCount, seg, min(seg + C::LIST, nqt), tid, lane, w, [&](int it) {
            return tile_class(p.map, p.nqb, p.nkb, it * (BR / kMapTile), BR / kMapTile, key0 / kMapTile,
                              BC / kMapTile);
        });
        if (count == 0) continue;

        // ---- first live tile into buffer 0
        {
            B16Tile<DKP, DVP> t;
            b16_load<DKP, DVP, EXACT>(t, hd, (sList[0] >> 2) * BR, p.N, p.DK, p.vecK, tid);
            b16_store<DKP, DVP>(t, sQ[0], sO[0], sL[0], sD[0], tid);
        }
        __syncthreads();

        int buf = 0;
        for (int li = 0; li < count; ++li) {
            const int e = sList[li];
            const int it = e >> 2, cls = e & 3;
            const int q0 = it * BR;
            const bool more = li + 1 < count;
            // prefetch the next live tile into registers (the current one again when
            // there is none); stored to the other buffer after this step's products
            B16Tile<DKP, DVP> nt;
            b16_load<DKP, DVP, EXACT>(nt, hd, (more ? (sList[li + 1] >> 2) : it) * BR, p.N, p.DK, p.vecK, tid);

            b16_step<DKP, DVP>(p, sQ[buf], sO[buf], sL[buf], sD[buf], sK, vf, dkacc, dvacc, q0,
                               cls == kTileCausal ? mykey : INT_MIN, cls == kTileMixed,
                               cls == kTileFree && key0 + BC <= p.M, mykey, kbias, sl2, w, lane);
            if (more) b16_store<DKP, DVP>(nt, sQ[buf ^ 1], sO[buf ^ 1], sL[buf ^ 1], sD[buf ^ 1], tid);
            __syncthreads();  // next tile staged; every wave is done with this one
            buf ^= 1;
        }
    }

    // ---- store dK (scaled) and dV of this key block
    const int hdd = p.part_heads ? h : g, Hd = p.part_heads ? p.H : p.Hkv;
    float *dkb = p.dk + (size_t)p.DK * p.M * (hdd + Hd * b);
    float *dvb = p.dv + (size_t)p.DV * p.M * (hdd + Hd * b);
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

// ============================================================== f32 mode
// f32 operands: every matrix-core operand is one float per lane, so transposed
// operands are plain strided LDS reads and no transposed copies are needed.
template <int DKP, int DVP>
struct F32Cfg {
    static constexpr int W = (DKP + DVP <= 128) ? 4 : 2;
    static constexpr int NT = 64 * W;
    static constexpr int BC = 32 * W;   // keys per work-group
    static constexpr int BR = 32;       // queries per step
    static constexpr int LK = DKP + 4, LV = DVP + 4, LQ = DKP + 4, LO = DVP + 4, LS = BC + 4;
};

template <int DKP, int DVP>
__global__ __launch_bounds__((F32Cfg<DKP, DVP>::NT), 1) void bwd_f32_kernel(BwdArgs p)
{
    using C = F32Cfg<DKP, DVP>;
    constexpr int BC = C::BC, BR = C::BR, W = C::W, NT = C::NT;
    constexpr int LK = C::LK, LV = C::LV, LQ = C::LQ, LO = C::LO, LS = C::LS;
    __shared__ __attribute__((aligned(16))) float sK[BC * LK];
    __shared__ __attribute__((aligned(16))) float sV[BC * LV];
    __shared__ __attribute__((aligned(16))) float sQ[BR * LQ];
    __shared__ __attribute__((aligned(16))) float sO[BR * LO];
    __shared__ __attribute__((aligned(16))) float sS[BR * LS];   // dS: [query][key]
    __shared__ __attribute__((aligned(16))) float sL[BR];
    __shared__ __attribute__((aligned(16))) float sD[BR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int HB = p.H * p.B;
    const int j = blockIdx.x / HB, hb = blockIdx.x % HB;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int key0 = j * BC;
    const int mykey = key0 + 32 * w + l32;
    const bool keyok = mykey < p.M;
    const float *kh = p.k + (size_t)p.DK * p.M * (g + p.Hkv * b);
    const float *vh = p.v + (size_t)p.DV * p.M * (g + p.Hkv * b);
    const float *qh = p.q + (size_t)p.DK * p.N * (h + p.H * b);
    const size_t dstride = (size_t)p.DV * p.H;                       // d row stride
    const float *dh = p.dO + (size_t)p.DV * h + dstride * p.N * b;    // row n at + n*dstride
    float *dqh = p.dq + (size_t)p.DK * p.N * (h + p.H * b);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

    for (int c = tid; c < BC * (DKP / 4); c += NT) {
        const int r = c / (DKP / 4), col = 4 * (c % (DKP / 4));
        const int key = key0 + r;
        *reinterpret_cast<f32x4 *>(&sK[r * LK + col]) =
            key < p.M ? load_row4(kh + (size_t)p.DK * key, col, p.DK, p.vecK) : z;
    }
    for (int c = tid; c < BC * (DVP / 4); c += NT) {
        const int r = c / (DVP / 4), col = 4 * (c % (DVP / 4));
        const int key = key0 + r;
        *reinterpret_cast<f32x4 *>(&sV[r * LV + col]) =
            key < p.M ? load_row4(vh + (size_t)p.DV * key, col, p.DV, p.vecV) : z;
    }

    f32x16 dkacc[DKP / 32], dvacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DKP / 32; ++i) dkacc[i] = zero16();
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) dvacc[i] = zero16();
    const float sl2 = p.scale * kLog2e;
    const int nqt = (p.N + BR - 1) / BR;

    for (int it = 0; it < nqt; ++it) {
        const int cls = tile_class(p.map, p.nqb, p.nkb, it * (BR / kMapTile), BR / kMapTile,
                                   key0 / kMapTile, BC / kMapTile);
        if (cls == kTileSkip) continue;
        const int q0 = it * BR;
        __syncthreads();  // the previous step is done with sQ, sO, sS
        for (int c = tid; c < BR * (DKP / 4); c += NT) {
            const int r = c / (DKP / 4), col = 4 * (c % (DKP / 4));
            const int n = q0 + r;
            *reinterpret_cast<f32x4 *>(&sQ[r * LQ + col]) =
                n < p.N ? load_row4(qh + (size_t)p.DK * n, col, p.DK, p.vecK) : z;
        }
        for (int c = tid; c < BR * (DVP / 4); c += NT) {
            const int r = c / (DVP / 4), col = 4 * (c % (DVP / 4));
            const int n = q0 + r;
            *reinterpret_cast<f32x4 *>(&sO[r * LO + col]) =
                n < p.N ? load_row4(dh + dstride * n, col, p.DV, p.vecV) : z;
        }
        if (tid < BR) {
            const int n = q0 + tid;
            float L = -INFINITY, Dl = 0.f;
            if (n < p.N) {
                L = p.lse[n + p.N * (h + p.H * b)];
                Dl = p.delta[n + p.N * (h + p.H * b)];
            }
            sL[tid] = (L == -INFINITY) ? INFINITY : L * kLog2e;
            sD[tid] = Dl;
        }
        __syncthreads();

        // ---- S = Q K^T, dP = dO V^T (k index = half*(D/2) + t)
        f32x16 sacc = zero16(), pacc = zero16();
        {
            const float *kr = &sK[(32 * w + l32) * LK + half * (DKP / 2)];
            const float *vr = &sV[(32 * w + l32) * LV + half * (DVP / 2)];
            const float *qr = &sQ[l32 * LQ + half * (DKP / 2)];
            const float *orr = &sO[l32 * LO + half * (DVP / 2)];
#pragma unroll
            for (int t = 0; t < DKP / 2; t += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(qr + t);
                const f32x4 bk = *reinterpret_cast<const f32x4 *>(kr + t);
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc = mfma_f32(a[i], bk[i], sacc);
            }
#pragma unroll
            for (int t = 0; t < DVP / 2; t += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(orr + t);
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(vr + t);
#pragma unroll
                for (int i = 0; i < 4; ++i) pacc = mfma_f32(a[i], bv[i], pacc);
            }
        }
        // ---- P and dS
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int qr = 8 * r4 + 4 * half;
            const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(&sL[qr]);
            const f32x4 del4 = *reinterpret_cast<const f32x4 *>(&sD[qr]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = 4 * r4 + c, n = q0 + qr + c;
                float x = sacc[r] * sl2;
                if (cls == kTileCausal) {
                    x = (mykey <= n) ? x : -INFINITY;
                } else if (cls == kTileMixed) {
                    if (n < p.N && keyok) x += half_bits_to_float(p.mask[mykey + (size_t)p.M * n]) * kLog2e;
                }
                const float P = keyok ? fast_exp2(x - lse4[c]) : 0.f;
                sacc[r] = P;
                pacc[r] = P * (pacc[r] - del4[c]);
            }
        }
        // ---- dV += P^T dO, dK += dS^T Q
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int qr = crow(u, half);
#pragma unroll
            for (int dt = 0; dt < DVP / 32; ++dt)
                dvacc[dt] = mfma_f32(sacc[u], sO[qr * LO + dt * 32 + l32], dvacc[dt]);
#pragma unroll
            for (int dt = 0; dt < DKP / 32; ++dt)
                dkacc[dt] = mfma_f32(pacc[u], sQ[qr * LQ + dt * 32 + l32], dkacc[dt]);
        }
        // ---- dS to LDS [query][key]
#pragma unroll
        for (int r = 0; r < 16; ++r) sS[crow(r, half) * LS + 32 * w + l32] = pacc[r];
        __syncthreads();
        // ---- dQ tiles (32 queries x 32 dims), round-robin over the waves
        for (int dt = w; dt < DKP / 32; dt += W) {
            f32x16 acc = zero16();
#pragma unroll
            for (int t = 0; t < BC / 2; t += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sS[l32 * LS + half * (BC / 2) + t]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc = mfma_f32(a[i], sK[(half * (BC / 2) + t + i) * LK + dt * 32 + l32], acc);
            }
            const int col = dt * 32 + l32;
            if (col < p.DK)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = q0 + crow(r, half);
                    if (n < p.N) unsafeAtomicAdd(dqh + col + (size_t)p.DK * n, acc[r] * p.scale);
                }
        }
    }

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

// ============================================================== launcher
namespace {
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int DKP, int DVP, bool BF16>
hipError_t run_bwd(const BwdArgs &a, hipStream_t s)
{
    if constexpr (BF16) {
        using C = B16Cfg<DKP, DVP>;
        const dim3 grid(ceil_div(a.M, C::BC) * a.H * a.B);
        if (a.DK == DKP)
            hipLaunchKernelGGL((bwd_bf16_kernel<DKP, DVP, true>), grid, dim3(C::NT), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_bf16_kernel<DKP, DVP, false>), grid, dim3(C::NT), 0, s, a);
    } else {
        using C = F32Cfg<DKP, DVP>;
        hipLaunchKernelGGL((bwd_f32_kernel<DKP, DVP>), dim3(ceil_div(a.M, C::BC) * a.H * a.B), dim3(C::NT),
                           0, s, a);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_backward(const float *q, const float *k, const float *v, const float *dO,
                           const __bf16 *dO16, const uint16_t *mask, const uint8_t *map,
                           const float *lse, const float *delta, float scale, int bf16, float *dq,
                           float *dk, float *dv, int part_heads, const Dims &d, hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    if (bf16 && !dO16) return hipErrorInvalidValue;
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dO = dO; a.dO16 = dO16; a.mask = mask; a.map = map;
    a.lse = lse; a.delta = delta; a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.DK = d.DK; a.DV = d.DV;
    a.part_heads = part_heads;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile);
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0);
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_bwd, a, s, hd, bf16);
}

}  // namespace fab
