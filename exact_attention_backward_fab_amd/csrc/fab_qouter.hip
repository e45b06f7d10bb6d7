// fab_qouter.hip -- the query-block-outer kernels (gfx950), on the bf16 tiles of
// fab_tiles.h.
//
//   fwd_bf16_kernel        O = softmax(scale S + mask) V and the row LSE by query
//                          blocks, with the running max and running sum of the
//                          labml "Flash Attention" page ("Flash Attention
//                          Optimization"); as the backward's own forward (PREP)
//                          it stores no O but, from the O in registers, the
//                          inputs of the backward kernels: D = rowsum(dO o O),
//                          the bf16 Q and dO tiles and the LSE/D blocks
//   dq_ds_kernel           dQ = scale dS K from the bf16 dS^T tiles the dK/dV
//                          kernel stores: a memory-bound product by pairs of
//                          query steps, each dQ element written once; the same
//                          launch runs the grouped-query reduction of dK and dV
//   dq_bf16_kernel         dQ = scale dS K by query blocks without stored dS (the
//                          shapes whose dS would pass 4 GiB):
//                          a work-group owns 128 queries of one (batch, head) and
//                          streams the key blocks that see them (block map),
//                          recomputing S^T = K Q^T and dP^T = V dO^T on the
//                          matrix cores, P = exp(scale S + mask - LSE), dS = P o
//                          (dP - D) (labml "Flash Attention", "Backward pass"),
//                          and accumulating dQ in registers.  Every dQ element is
//                          written once; no atomics on dQ.  Small grids run each
//                          query block as two work-groups on alternate key steps
//                          whose partial sums meet through a per-block counter.
#include <algorithm>
#include <climits>

#include "fab_common.h"
#include "fab_launch.h"
#include "fab_tiles.h"

namespace fab {

// Work-group shape of the query-block-outer kernels: 4 waves, 32 queries each;
// keys stream through LDS one 64-row tile (a step) at a time.
constexpr int kQW = 4, kQNT = 64 * kQW, kQBQ = 32 * kQW, kQBK = kTR;
constexpr int kQList = 512;   // live key steps listed at a time

// LDS stages of the key stream (K and V tiles of one step each) and work-groups
// per CU: two work-groups (two waves per SIMD, so that one wave's softmax
// arithmetic overlaps the other's matrix-core work) when two stages of each fit
// in half of the 160 KiB, else one; then as many stages as fit, at most 4.
template <int DKP, int DVP, bool MS = false>
struct QStages {
    static constexpr int kK = DKP / 8 * kChunkL;            // bytes of a K tile in LDS
    static constexpr int kKV = (DKP + DVP) / 8 * kChunkL;   // ... and of the K and V tiles
    // with MS the step's mask rows (128 queries x 64 keys, f16) follow, chunk-major:
    // the 16-byte chunk c (keys 8c..8c+7) of row r at byte (c * 128 + r) * 16
    static constexpr int kM = MS ? kQBQ * kQBK * 2 : 0;
    static constexpr int kBytes = kKV + kM;
    static constexpr int kFixed = 4 * kQList + 256;
    static constexpr int Occ = (2 * kBytes + kFixed <= 80 * 1024) ? 2 : 1;
    static constexpr int kFit = (160 * 1024 / Occ - kFixed) / kBytes;
    static constexpr int N = kFit > 4 ? 4 : kFit;
    static_assert(N >= 2, "two LDS stages must fit");
};

// Work-group -> (query tile, head): query_block_work (fab_common.h).
struct QWork {
    int qt, hb;
};
__device__ __forceinline__ QWork qouter_work(int bid, int nqt, int HB, int fold = 0)
{
    QWork r;
    query_block_work(bid, nqt, HB, fold, &r.qt, &r.hb);
    return r;
}

// Work-group -> (query block index for qouter_work, share) of the recompute dQ kernel.
// With split == 2 each query block is run by two work-groups (shares) that take
// alternate live key steps; the shares of a block are 8 work-groups apart, so
// the round-robin dispatch over the XCDs puts them on one XCD, one shortly after
// the other.
struct QShare {
    int unit, share;
};
__device__ __forceinline__ QShare query_share(int bid, int HB, int split)
{
    QShare r{bid, 0};
    if (split == 2) {
        if (HB % 8 == 0) {
            r.unit = (bid & 7) + 8 * (bid >> 4);
            r.share = (bid >> 3) & 1;
        } else {
            r.unit = bid >> 1;
            r.share = bid & 1;
        }
    }
    return r;
}

// Streams the live key steps (block map) of one query block through the LDS
// stages: the K and V tiles of later steps are copied from global memory straight
// into LDS while body(step, class, K tile, V tile) works on the current one.  Each
// wave copies a quarter of the chunk columns; before a step is used every wave
// waits for its own copies of it (vmcnt) and a barrier publishes them; the same
// barrier tells every wave that the stage about to be refilled has been consumed.
// sKV is the stage array and kv_lds its LDS byte address.
// With stride > 1 the work-group takes only the live steps at list positions
// off, off + stride, ... (one share of a query block split over work-groups).
// With ST::kM (mask rows staged) every step also copies the mask rows of the
// work-group's queries q0.. at the step's 64 keys into the stage (mask [N][M],
// M % 8 == 0; rows past N read as zero), and body receives their LDS address.
template <int DKP, int DVP, int W = kQW, typename ST = QStages<DKP, DVP>, typename ClassOf, typename Body>
__device__ __forceinline__ void stream_key_steps(rsrc_t rk, rsrc_t rv, const char *sKV, uint32_t kv_lds, int *sList,
                                                 int *sCount, int nks, int tid, int lane, int w, ClassOf class_of,
                                                 Body body, int off = 0, int stride = 1,
                                                 const uint16_t *mask = nullptr, int N = 0, int q0 = 0, int M = 0)
{
    constexpr int NS = ST::N;
    // chunk columns copied per wave; when a tile has fewer columns than waves, the
    // surplus copies repeat a column (same bytes to the same place) so that every
    // wave issues the same number of copies per step (its vmcnt waits count on it)
    constexpr int KCH = (DKP / 8 + W - 1) / W, VCH = (DVP / 8 + W - 1) / W;
    constexpr int MCH = ST::kM / 1024 / W;   // 1 KiB mask copies per wave: 64 rows of one chunk each
    static_assert(MCH * 1024 * W == ST::kM, "mask copy split");
    const rsrc_t rm = mask_rsrc(MCH ? mask : nullptr, N, M);
    auto issue = [&](int s, int bf) {
        const uint32_t stg = kv_lds + (uint32_t)(bf * ST::kBytes);   // wave-uniform LDS byte address
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = (i * W + w) % (DKP / 8);
            lds_copy16(rk, stg + c * kChunkL, (uint32_t)(s * DKP / 8 + c) * kChunkG + (uint32_t)lane * 16u);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = (i * W + w) % (DVP / 8);
            lds_copy16(rv, stg + ST::kK + c * kChunkL, (uint32_t)(s * DVP / 8 + c) * kChunkG + (uint32_t)lane * 16u);
        }
#pragma unroll
        for (int i = 0; i < MCH; ++i) {
            // copy x: chunk x / 2 of rows 64 (x % 2) + lane
            const int x = i * W + w, c = x >> 1, r = 64 * (x & 1) + lane;
            lds_copy16(rm, stg + ST::kKV + (uint32_t)(c * 128 + 64 * (x & 1)) * 16u,
                       2u * ((uint32_t)(q0 + r) * (uint32_t)M + (uint32_t)(s * kQBK)) + (uint32_t)c * 16u);
        }
    };
    for (int seg = 0; seg < nks; seg += kQList) {
        const int live = build_live_list<W>(sList, sCount, seg, min(seg + kQList, nks), tid, lane, w, class_of);
        const int count = live > off ? (live - off + stride - 1) / stride : 0;   // this share's steps
        if (count == 0) continue;
        const int *list = sList + off;
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            if (i < count) issue(list[stride * i] >> 2, i);
        for (int li = 0; li < count; ++li) {
            wait_vm_steps<KCH + VCH + MCH>(min(count - 1 - li, NS - 2));   // step li has landed (this wave)
            __syncthreads();                                                // ... for every wave; stage li-1 is free
            if (li + NS - 1 < count) issue(list[stride * (li + NS - 1)] >> 2, (li + NS - 1) % NS);
            const int e = list[stride * li];
            const char *stg = sKV + (li % NS) * ST::kBytes;
            body(e >> 2, e & 3, stg, stg + ST::kK, stg + ST::kKV);
        }
        __syncthreads();   // every wave is done with the stages before they are refilled
    }
}

// Per-lane query operands: B operands of S^T = K Q^T (Q rows of f32, bf16 or f16
// elements, fmt, -> bf16) for query row `row` (all zero when !ok).
template <int DKP>
__device__ __forceinline__ void load_q_operand(bf16x8 *qf, const void *q, int64_t row_off, bool ok, int DK, int vecK,
                                               int half, int fmt)
{
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DKP / 16; ++t) {
        const f32x4 lo = ok ? load_row4_any(q, row_off, 16 * t + 8 * half, DK, vecK, fmt) : z;
        const f32x4 hi = ok ? load_row4_any(q, row_off, 16 * t + 8 * half + 4, DK, vecK, fmt) : z;
        qf[t] = __builtin_shufflevector(to_bf16x4(lo), to_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// S^T for both 32-key sub-tiles of a step (and, with VB, dP^T = V dO^T for both
// from the V tile at Vb and the lane's dO operand of): the LDS row operands run R
// products ahead of the matrix cores in a register ring that the scheduling barriers
// hold in place (left to itself the compiler issues each product's reads, waits for
// them and multiplies, one product at a time).
template <int DKP, int DVP, bool VB, int R = 2>
__device__ __forceinline__ void st_pt_pair(const char *Kb, const bf16x8 *qf, const char *Vb, const bf16x8 *of,
                                           int row_off, f32x16 *st, f32x16 *pt)
{
    constexpr int TS = DKP / 16, TP = VB ? DVP / 16 : 0, T = TS > TP ? TS : TP;
    bf16x8 k0[R], k1[R], v0[R], v1[R];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        st[kk] = zero16();
        if (VB) pt[kk] = zero16();
    }
#pragma unroll
    for (int j = 0; j < T + R; ++j) {
        if (j >= R) {
            const int t = j - R;
            if (t < TS) {
                st[0] = mfma_bf16(k0[t % R], qf[t], st[0]);
                st[1] = mfma_bf16(k1[t % R], qf[t], st[1]);
            }
            if (t < TP) {
                pt[0] = mfma_bf16(v0[t % R], of[t], pt[0]);
                pt[1] = mfma_bf16(v1[t % R], of[t], pt[1]);
            }
        }
        if (j < TS) {
            k0[j % R] = lds_row8(Kb + row_off + 2304 * j);
            k1[j % R] = lds_row8(Kb + row_off + 512 + 2304 * j);
        }
        if (j < TP) {
            v0[j % R] = lds_row8(Vb + row_off + 2304 * j);
            v1[j % R] = lds_row8(Vb + row_off + 512 + 2304 * j);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// acc[c] += A(g) * B(g, c) over the four (sub-tile kk, operand half u) groups g = 2 kk + u
// of a step, B by transposing reads of the tile at Tb (column tile c, rows of group g),
// read R products ahead (ring and scheduling barriers as above).  SWAP: the transposed
// operand is the A side (acc += B * A, the product order of O^T += V^T P^T).
template <int NC, bool SWAP, int R = 3>
__device__ __forceinline__ void tr_products(f32x16 *acc, const bf16x8 *a4, const char *Tb, int tr_off)
{
    constexpr int NJ = 4 * NC;
    bf16x8 br[R];
#pragma unroll
    for (int j = 0; j < NJ + R; ++j) {
        if (j >= R) {
            const int i = j - R, g = i / NC, c = i % NC;
            acc[c] = SWAP ? mfma_bf16(br[i % R], a4[g], acc[c]) : mfma_bf16(a4[g], br[i % R], acc[c]);
        }
        if (j < NJ) {
            const int g = j / NC, c = j % NC;
            br[j % R] = lds_tr8(Tb + tr_off + 4608 * c + 512 * (g >> 1) + 256 * (g & 1));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Scaled scores (log2 units) of NT 32-key sub-tiles from key0 on for the lane's
// query myq: keys past lim get -inf; with ALiBi (slope2 != 0, log2 units) the
// bias slope2 (key - myq) is added; MIXED steps add the mask row of the query.  A
// lane's keys come in runs of 4 (slots 4j..4j+3), read as one 8-byte load when
// vecM (M % 4 == 0).
// With mst (mask rows staged in LDS by stream_key_steps), the mask of row mrl of the
// stage is read from there instead of from mrow.
template <int NT, bool AB = false>
__device__ __forceinline__ void scale_and_mask(f32x16 *st, int key0, int lim, bool mixed, const uint16_t *mrow, int M,
                                               bool vecM, float sl2, int half, float slope2 = 0.f, int myq = 0,
                                               const char *mst = nullptr, int mrl = 0)
{
#pragma unroll
    for (int kk = 0; kk < NT; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = st[kk][r] * sl2;
            st[kk][r] = (key0 + kk * 32 + crow(r, half) <= lim) ? x : -INFINITY;
        }
    if (AB && slope2 != 0.f) {   // ALiBi: + slope (key - query), in log2 units
        const float ab = slope2 * (float)(key0 - myq);
#pragma unroll
        for (int kk = 0; kk < NT; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r) st[kk][r] += __builtin_fmaf(slope2, (float)(kk * 32 + crow(r, half)), ab);
    }
    if (mixed && mst) {
#pragma unroll
        for (int kk = 0; kk < NT; ++kk)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                // keys kk*32 + 8 r4 + 4 half.. of the step: chunk 4 kk + r4, bytes 8 half..
                const uint2 x = *reinterpret_cast<const uint2 *>(mst + ((4 * kk + r4) * 128 + mrl) * 16 + 8 * half);
                const uint16_t m4[4] = {(uint16_t)(x.x & 0xFFFFu), (uint16_t)(x.x >> 16), (uint16_t)(x.y & 0xFFFFu),
                                        (uint16_t)(x.y >> 16)};
#pragma unroll
                for (int i = 0; i < 4; ++i) st[kk][4 * r4 + i] += half_bits_to_float(m4[i]) * kLog2e;
            }
    } else if (mixed) {
        uint16_t m[NT][16];
#pragma unroll
        for (int kk = 0; kk < NT; ++kk)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int k0 = key0 + kk * 32 + 8 * r4 + 4 * half;
                if (vecM && k0 + 3 < M) {
                    const uint2 x = *reinterpret_cast<const uint2 *>(mrow + k0);
                    m[kk][4 * r4 + 0] = (uint16_t)(x.x & 0xFFFFu);
                    m[kk][4 * r4 + 1] = (uint16_t)(x.x >> 16);
                    m[kk][4 * r4 + 2] = (uint16_t)(x.y & 0xFFFFu);
                    m[kk][4 * r4 + 3] = (uint16_t)(x.y >> 16);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) m[kk][4 * r4 + i] = mrow[min(k0 + i, M - 1)];
                }
            }
#pragma unroll
        for (int kk = 0; kk < NT; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r) st[kk][r] += half_bits_to_float(m[kk][r]) * kLog2e;
    }
}

// ============================================================== forward
struct FwdArgs16 {
    const void *q;                  // f32, bf16 or f16 elements (in_fmt: kF32, kBF16, kF16; as dO)
    int in_fmt;
    const __bf16 *k16, *v16;        // bf16 [B,Hkv,Mp,DKP] / [B,Hkv,Mp,DVP] in 64-row tiles, rows >= M zero
    const uint16_t *mask;
    const uint8_t *map;
    void *O;                        // O [DV,H,N,B]: f32, or bf16 when o_bf16
    int o_bf16;
    float *lse;                     // lse [N,H,B]
    int B, H, Hkv, N, M, Mp, DK, DV, nqb, nkb, vecK, vecV;
    int causal;                     // causal rule as a flag (no mask, no map)
    float scale;
    const float *alibi;             // per-head ALiBi slopes [H] or NULL
    // The backward's own forward (PREP) writes, instead of O and lse, what the
    // backward kernels read: the bf16 tiles of Q and dO (rows >= N and columns
    // >= DK / DV zero), the LSE/D blocks (D = rowsum(dO o O)), and it zeroes the
    // blob pads (work-group 0) and the dQ split counters.
    const void *dO;                 // [DV,H,N,B]
    __bf16 *q16, *o16;              // tiles [B,H,Np,DKP] / [B,H,Np,DVP]
    float *stats;                   // [B,H,Np/64][128]
    float *blob;
    int64_t pad_lo[3], pad_hi[3];   // the blob's pads, in 16-bit units (zero in every element type)
    int *zero;
    int nzero, Np;
    int fold;                       // the whole grid is resident at once (query_block_work)
};

// MS: the mask rows of every key step are staged in LDS with its K and V tiles
// (a mask is given and M % 8 == 0).  Used where one work-group fills a CU and two
// stages with the mask rows fit (the 192-wide heads): there the MIXED steps would
// otherwise wait on their own mask loads with no other work-group's products to
// hide them.
template <int DKP, int DVP, bool PREP, bool AB, bool MS = false, int KS = 1>
__global__ __launch_bounds__(256, (QStages<DKP, DVP, MS>::Occ))
__attribute__((amdgpu_waves_per_eu(QStages<DKP, DVP, MS>::Occ, QStages<DKP, DVP, MS>::Occ))) void fwd_bf16_kernel(FwdArgs16 p)
{
    using ST = QStages<DKP, DVP, MS>;
    static_assert(KS == 1 || (KS == 2 && !MS), "key split without staged mask rows only");
    constexpr int QWv = kQW / KS, BRv = 32 * QWv;   // 32-query tiles and queries of the work-group
    __shared__ __attribute__((aligned(16))) char sKV[ST::N * ST::kBytes];
    __shared__ int sList[kQList];
    __shared__ int sCount[kQW + 1];

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int row_off = tile_row_off(lane), tr_off = tile_tr_off(lane);
    const uint32_t kv_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)sKV;
    const int qw = KS == 1 ? w : w % QWv, kh = KS == 1 ? 0 : w / QWv;   // query tile, key part of this wave
    const int nqt = (p.N + BRv - 1) / BRv;
    const QWork wk = qouter_work(blockIdx.x, nqt, p.H * p.B, p.fold);   // latest queries first (most keys if causal)
    const int qt = wk.qt, hb = wk.hb;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int q0 = qt * BRv;
    const int myq = q0 + 32 * qw + l32;  // this lane's query (C-layout column of S^T and O^T)
    const bool qok = myq < p.N;
    const size_t hrow = (size_t)p.N * (h + p.H * b);
    const size_t kvrow = (size_t)p.Mp * (g + p.Hkv * b);
    const rsrc_t rk = make_rsrc(p.k16 + kvrow * DKP, (uint32_t)(p.Mp * DKP) * 2u);
    const rsrc_t rv = make_rsrc(p.v16 + kvrow * DVP, (uint32_t)(p.Mp * DVP) * 2u);

    bf16x8 qf[DKP / 16];
    load_q_operand<DKP>(qf, p.q, (int64_t)(hrow + (qok ? myq : 0)) * p.DK, qok, p.DK, p.vecK, half, p.in_fmt);
    const size_t qhead = (size_t)(h + p.H * b) * p.Np;   // PREP: first tile row of this head
    if constexpr (PREP) {
        if (kh == 0 && myq < p.Np) {
            __bf16 *qt16 = p.q16 + qhead * DKP;
#pragma unroll
            for (int t = 0; t < DKP / 16; ++t)
                *reinterpret_cast<bf16x8 *>(qt16 + tile_elem(myq, 16 * t + 8 * half, DKP)) = qf[t];
        }
        for (int i = blockIdx.x * kQNT + tid; i < p.nzero; i += gridDim.x * kQNT) p.zero[i] = 0;
        if (blockIdx.x == 0 && tid < 8)   // pads below 16 bytes: at most 7 16-bit units
            for (int k = 0; k < 3; ++k)
                if (p.pad_lo[k] + tid < p.pad_hi[k]) reinterpret_cast<uint16_t *>(p.blob)[p.pad_lo[k] + tid] = 0;
    }
    f32x16 oacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) oacc[i] = zero16();
    float m_run = -INFINITY, l_part = 0.f;   // reference max (log2 units), this half's running sum
    const float sl2 = p.scale * kLog2e;
    const float slope2 = AB ? p.alibi[h] * kLog2e : 0.f;   // ALiBi, log2 units
    const uint16_t *mrow = p.mask + (size_t)p.M * min(myq, p.N - 1);

    stream_key_steps<DKP, DVP, kQW, ST>(
        rk, rv, sKV, kv_lds, sList, sCount, (p.M + kQBK - 1) / kQBK, tid, lane, w,
        [&](int s) {
            return tile_class<BRv / kMapTile, kQBK / kMapTile>(p.map, p.causal, p.N, p.M, p.nqb, p.nkb, q0 / kMapTile,
                              s * (kQBK / kMapTile));
        },
        [&](int s, int cls, const char *Kb, const char *Vb, const char *Mb) {
            const int key0 = s * kQBK;
            constexpr int NSUB = 2 / KS;   // 32-key sub-tiles of the step this wave takes
            f32x16 st[NSUB];
            if constexpr (KS == 1) {
                st_pt_pair<DKP, DVP, false>(Kb, qf, nullptr, nullptr, row_off, st, nullptr);
            } else {
                // S^T of sub-tile kh only, the K rows read two products ahead
                constexpr int TS = DKP / 16, R = 2;
                bf16x8 kr[R];
                st[0] = zero16();
#pragma unroll
                for (int j = 0; j < TS + R; ++j) {
                    if (j >= R) st[0] = mfma_bf16(kr[(j - R) % R], qf[j - R], st[0]);
                    if (j < TS) kr[j % R] = lds_row8(Kb + row_off + 512 * kh + 2304 * j);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // scores in log2 units = st * mul: a step with every key visible (FREE and
            // inside M) keeps the raw products and folds the scale into the exponent
            float mul = sl2;
            if (!(cls == kTileFree && key0 + kQBK <= p.M && sl2 > 0.f && (!AB || slope2 == 0.f))) {
                const int lim = qok ? min(cls == kTileCausal ? myq : INT_MAX, p.M - 1) : -1;
                scale_and_mask<NSUB, AB>(st, key0 + 32 * kh, lim, cls == kTileMixed, mrow, p.M, (p.M & 3) == 0, sl2, half,
                                     slope2, myq, MS ? Mb : nullptr, 32 * w + l32);
                mul = 1.f;
            }

            // ---- running max and sum; the two lane halves hold the same query.  The
            // reference max m_run moves only when the step's max exceeds it by more
            // than 8 (P <= 2^8 stays exact in f32 and bf16 relative terms; O = Õ / l
            // and LSE = m_run + log2 l do not depend on which reference is used), so
            // most steps skip rescaling the accumulators.
            float mraw = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < NSUB; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, st[kk][r]);
            const float mloc = swap_halves_max(mraw) * mul;
            const bool grow = mloc > m_run + 8.f;   // m_run = -inf: any finite score
            const float m_new = grow ? mloc : m_run;
            if (__any(grow)) {
                const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
                l_part *= alpha;
#pragma unroll
                for (int i = 0; i < DVP / 32; ++i) oacc[i] *= alpha;
            }
            m_run = m_new;
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // all -inf so far: P = 0
            float lsum = 0.f;
#pragma unroll
            for (int kk = 0; kk < NSUB; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(__builtin_fmaf(st[kk][r], mul, -m_use));
                    st[kk][r] = e;
                    lsum += e;
                }
            l_part += lsum;

            // ---- O^T += V^T P^T: A = V^T by transposing reads (key rows 16u + 4*half
            // (+8) of the sub-tile), B = P^T (lane = query, keys in operand order)
            bf16x8 pb4[2 * NSUB];   // index 2 kk + u
#pragma unroll
            for (int kk = 0; kk < NSUB; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float pv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) pv[i] = st[kk][8 * u + i];
                    pb4[2 * kk + u] = to_bf16x8(pv);
                }
            if constexpr (KS == 1) {
                tr_products<DVP / 32, true>(oacc, pb4, Vb, tr_off);
            } else {
                // the two groups (u) of sub-tile kh: V^T rows of that sub-tile by transposing reads
                constexpr int NC = DVP / 32, NJ = 2 * NC, R = 3;
                bf16x8 br[R];
#pragma unroll
                for (int j = 0; j < NJ + R; ++j) {
                    if (j >= R) {
                        const int i = j - R, u = i / NC, c = i % NC;
                        oacc[c] = mfma_bf16(br[i % R], pb4[u], oacc[c]);
                    }
                    if (j < NJ) {
                        const int u = j / NC, c = j % NC;
                        br[j % R] = lds_tr8(Vb + tr_off + 4608 * c + 512 * kh + 256 * u);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        },
        0, 1, p.mask, p.N, q0, p.M);

    // ---- KS = 2: the second key part hands its reference max, sum and O to the first
    // through the stages (no longer read); the first rescales both to the larger max
    if constexpr (KS == 2) {
        constexpr int XO = DVP / 32 * 16;   // O values per lane
        static_assert(QWv * (XO + 2) * 64 * 4 <= ST::N * ST::kBytes, "key-part exchange area");
        float *xch = reinterpret_cast<float *>(sKV) + qw * (XO + 2) * 64;
        __syncthreads();   // every wave is done with the stages
        if (kh == 1) {
#pragma unroll
            for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xch[(dt * 16 + r) * 64 + lane] = oacc[dt][r];
            xch[XO * 64 + lane] = m_run;
            xch[(XO + 1) * 64 + lane] = l_part;
        }
        __syncthreads();
        if (kh == 1) return;
        const float m1 = xch[XO * 64 + lane], l1 = xch[(XO + 1) * 64 + lane];
        const float m = fmaxf(m_run, m1);
        // a part that saw no weight has max -inf and zero sum and O: its factor is 0
        const float a0 = m == -INFINITY ? 0.f : fast_exp2(m_run - m);
        const float a1 = m == -INFINITY ? 0.f : fast_exp2(m1 - m);
        l_part = l_part * a0 + l1 * a1;
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] = oacc[dt][r] * a0 + xch[(dt * 16 + r) * 64 + lane] * a1;
        m_run = m;
    }

    // ---- normalise and store O [DV,H,N,B] and the natural-log LSE [N,H,B]
    const float l = swap_halves_sum(l_part);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if constexpr (PREP) {
        // D = rowsum(dO o O) with O = Õ / l in f32, the bf16 dO row into its tile, and
        // the row's LSE (log2 units; +inf = no weight: all-masked or past N) and D
        if (myq >= p.Np) return;
        const int64_t drow = (int64_t)p.DV * (h + p.H * (min(myq, p.N - 1) + (int64_t)p.N * b));
        __bf16 *ot16 = p.o16 + qhead * DVP;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        float dsum = 0.f;
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c0 = dt * 32 + 8 * r4 + 4 * half;
                const f32x4 dv = qok ? load_row4_any(p.dO, drow, c0, p.DV, p.vecV, p.in_fmt) : z;
#pragma unroll
                for (int i = 0; i < 4; ++i) dsum += dv[i] * (oacc[dt][4 * r4 + i] * inv);
                *reinterpret_cast<bf16x4 *>(ot16 + tile_elem(myq, c0, DVP)) = to_bf16x4(dv);
            }
        dsum = swap_halves_sum(dsum);
        if (half == 0) {
            float *st = p.stats + (qhead / 64 + myq / 64) * kStatsTile + (myq & 63);
            const bool live = qok && l > 0.f;
            st[0] = live ? m_run + log2f(l) : INFINITY;
            st[64] = live ? dsum : 0.f;
        }
        return;
    }
    if (qok) {
        const size_t ooff = (size_t)p.DV * (h + p.H * (myq + (size_t)p.N * b));
        float *orow = static_cast<float *>(p.O) + ooff;
        __bf16 *orow16 = static_cast<__bf16 *>(p.O) + ooff;   // o_bf16: the f32 values rounded to nearest even
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c0 = dt * 32 + 8 * r4 + 4 * half;
                if (c0 >= p.DV) continue;
                f32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = oacc[dt][4 * r4 + i] * inv;
                if (p.o_bf16) {
                    if (p.vecV) {
                        *reinterpret_cast<bf16x4 *>(orow16 + c0) = to_bf16x4(o);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (c0 + i < p.DV) orow16[c0 + i] = (__bf16)o[i];
                    }
                } else if (p.vecV) {
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

// ============================================================== dQ by query blocks
struct DqArgs {
    const __bf16 *q16, *o16;        // bf16 tiles [B,H,Np,DKP] / [B,H,Np,DVP], rows >= N zero
    const float *stats;             // LSE/D blocks [B,H,Np/64][128]
    const __bf16 *k16, *v16;        // bf16 tiles [B,Hkv,Mp,DKP] / [B,Hkv,Mp,DVP], rows >= M zero
    const uint16_t *mask;
    const uint8_t *map;
    float *dq;                      // [DK,N,H,B] slice of the result blob (out_fmt elements)
    int out_fmt;
    float *part;                    // split == 2: per-share dQ partials [blocks][2][4 waves][DKP/2 * 64]
    int *ticket;                    // split == 2: one zeroed counter per query block
    int B, H, Hkv, N, Np, M, Mp, DK, DV, nqb, nkb;
    int causal;                     // causal rule as a flag (no mask, no map)
    int split;                      // work-groups per query block (1 or 2)
    float scale;
    const float *alibi;             // per-head ALiBi slopes [H] or NULL
};

template <int DKP, int DVP, bool AB>
__global__ __launch_bounds__(256, (QStages<DKP, DVP>::Occ))
__attribute__((amdgpu_waves_per_eu(QStages<DKP, DVP>::Occ, QStages<DKP, DVP>::Occ))) void dq_bf16_kernel(DqArgs p)
{
    __shared__ __attribute__((aligned(16))) char sKV[QStages<DKP, DVP>::N * QStages<DKP, DVP>::kBytes];
    __shared__ int sList[kQList];
    __shared__ int sCount[kQW + 1];
    __shared__ int sTicket;

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int row_off = tile_row_off(lane), tr_off = tile_tr_off(lane);
    const uint32_t kv_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)sKV;
    const int nqt = (p.N + kQBQ - 1) / kQBQ, HB = p.H * p.B;
    const QShare sh = query_share(blockIdx.x, HB, p.split);
    const int unit = sh.unit, share = sh.share;
    const QWork wk = qouter_work(unit, nqt, HB);   // latest queries first (most keys if causal)
    const int qt = wk.qt, hb = wk.hb;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int q0 = qt * kQBQ;
    const int myq = q0 + 32 * w + l32;  // this lane's query (C-layout column of S^T and dP^T)
    const size_t hrow = (size_t)p.N * (h + p.H * b);
    const size_t kvrow = (size_t)p.Mp * (g + p.Hkv * b);
    const rsrc_t rk = make_rsrc(p.k16 + kvrow * DKP, (uint32_t)(p.Mp * DKP) * 2u);
    const rsrc_t rv = make_rsrc(p.v16 + kvrow * DVP, (uint32_t)(p.Mp * DVP) * 2u);

    // ---- this lane's query: LSE (log2 units, +inf when all-masked or past N), D,
    // and the B operands Q^T and dO^T of S^T = K Q^T and dP^T = V dO^T (rows past
    // the padded extent Np read as zero with no weight)
    float lse2 = INFINITY, dl = 0.f;
    bf16x8 qf[DKP / 16], of[DVP / 16];
    {
        const bool in = myq < p.Np;
        const size_t qhead = (size_t)(h + p.H * b) * p.Np;
        const __bf16 *qh16 = p.q16 + qhead * DKP;
        const __bf16 *oh16 = p.o16 + qhead * DVP;
        const bf16x8 z = {};
#pragma unroll
        for (int t = 0; t < DKP / 16; ++t)
            qf[t] = in ? *reinterpret_cast<const bf16x8 *>(qh16 + tile_elem(myq, 16 * t + 8 * half, DKP)) : z;
#pragma unroll
        for (int t = 0; t < DVP / 16; ++t)
            of[t] = in ? *reinterpret_cast<const bf16x8 *>(oh16 + tile_elem(myq, 16 * t + 8 * half, DVP)) : z;
        if (in) {
            const float *st = p.stats + (qhead / 64 + myq / 64) * kStatsTile + (myq & 63);
            lse2 = st[0];
            dl = st[64];
        }
    }

    f32x16 dqacc[DKP / 32];
#pragma unroll
    for (int i = 0; i < DKP / 32; ++i) dqacc[i] = zero16();
    const float sl2 = p.scale * kLog2e;
    const float slope2 = AB ? p.alibi[h] * kLog2e : 0.f;   // ALiBi, log2 units
    const uint16_t *mrow = p.mask + (size_t)p.M * min(myq, p.N - 1);

    stream_key_steps<DKP, DVP>(
        rk, rv, sKV, kv_lds, sList, sCount, (p.M + kQBK - 1) / kQBK, tid, lane, w,
        [&](int s) {
            return tile_class<kQBQ / kMapTile, kQBK / kMapTile>(p.map, p.causal, p.N, p.M, p.nqb, p.nkb, q0 / kMapTile,
                              s * (kQBK / kMapTile));
        },
        [&](int s, int cls, const char *Kb, const char *Vb, const char *) {
            const int key0 = s * kQBK;
            // ---- S^T = K Q^T and dP^T = V dO^T for two 32-key sub-tiles (lane = query)
            f32x16 st[2], pt[2];
            st_pt_pair<DKP, DVP, true>(Kb, qf, Vb, of, row_off, st, pt);

            // ---- P and dS; keys past M and (causal steps) keys after the query get -inf;
            // a step with every key visible folds the scale into the exponent
            float mul = sl2;
            if (!(cls == kTileFree && key0 + kQBK <= p.M && (!AB || slope2 == 0.f))) {
                const int lim = min(cls == kTileCausal ? myq : INT_MAX, p.M - 1);
                scale_and_mask<2, AB>(st, key0, lim, cls == kTileMixed, mrow, p.M, (p.M & 3) == 0, sl2, half, slope2,
                                  myq);
                mul = 1.f;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float P = fast_exp2(__builtin_fmaf(st[kk][r], mul, -lse2));
                    pt[kk][r] = P * (pt[kk][r] - dl);
                }

            // ---- dQ += dS K: A = dS (lane = query, keys in operand order), B = K via
            // transposing reads (key rows 16u + 4*half (+8) of the sub-tile)
            bf16x8 da4[4];   // index 2 kk + u
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float d8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) d8[i] = pt[kk][8 * u + i];
                    da4[2 * kk + u] = to_bf16x8(d8);
                }
            tr_products<DKP / 32, false>(dqacc, da4, Kb, tr_off);
        },
        share, p.split);

    // ---- two shares: both publish their partial sums and take the block's ticket;
    // the second to arrive adds the other's partial (a + b = b + a: the result
    // does not depend on which share that is) and stores the block.
    if (p.split == 2) {
        constexpr int PW = DKP / 32 * 16 * 64;   // floats of one wave's partial
        float *mine = p.part + ((size_t)(2 * unit + share) * kQW + w) * PW;
#pragma unroll
        for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                coherent_store(mine + (dt * 16 + r) * 64 + lane, dqacc[dt][r]);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) sTicket = ticket_take(p.ticket + unit);
        __syncthreads();
        if (sTicket == 0) return;   // first share: the other one finishes the block
        const float *other = p.part + ((size_t)(2 * unit + (share ^ 1)) * kQW + w) * PW;
#pragma unroll
        for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dqacc[dt][r] += coherent_load(other + (dt * 16 + r) * 64 + lane);
    }

    // ---- store dQ (scaled): lane = head-dim column, rows = this wave's queries
    const size_t dq0 = hrow * p.DK;   // this head's dQ rows in the result slice (out_fmt elements)
    with_result_width(p.out_fmt, [&](auto w16) {
        constexpr bool W16 = decltype(w16)::value;
#pragma unroll
        for (int dt = 0; dt < DKP / 32; ++dt) {
            const int col = dt * 32 + l32;
            if (col < p.DK)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = q0 + 32 * w + crow(r, half);
                    if (n < p.N) store_as<W16>(p.dq, dq0 + (size_t)n * p.DK + col, dqacc[dt][r] * p.scale, p.out_fmt);
                }
        }
    });
}

// ============================================================== dQ from the stored dS
// dQ = scale dS K as a plain product over the dS^T tiles the dK/dV kernel stored
// (fab_tiles.h, ds_query): a work-group owns the 128 queries of two consecutive
// query steps of one (batch, head) and streams the key blocks that see either of
// them (the block map test of the dK/dV kernel, so exactly the tiles it wrote),
// 64 keys at a time: both steps' dS^T key tiles and the K tile of those keys are
// copied straight into LDS, and both operands are taken by transposing reads
// (keys are the k dimension of the product).  8 waves: wave w owns
// queries 32 (w & 3).. of the pair and the head-dim tiles of parity w >> 2.  Each
// dQ element is written once (zero when no key block is live).
struct DqsArgs {
    const __bf16 *ds;               // dS^T tiles [B,H,ceil(Np/128),nkb128][2 key tiles][2 query steps][64 x 64]
    const __bf16 *k16;              // bf16 tiles [B,Hkv,Mp,DKP], rows >= M zero
    const uint8_t *map;
    float *dq;                      // [DK,N,H,B] slice of the result blob (out_fmt elements)
    int out_fmt;
    int B, H, Hkv, N, Np, M, Mp, DK, nqb, nkb, nkb128;
    int causal;                     // causal rule as a flag (no mask, no map)
    int fold;                       // the whole grid is resident at once (query_block_work)
    float scale;
    // grouped-query reduction run by the work-groups past the dQ grid (nred of them)
    ReduceJob red[2];
    int rk2, ndq, nred;
};

constexpr int kDsW = 8, kDsNT = 64 * kDsW;
constexpr int kDsList = 512;       // live key blocks listed at a time

// LDS stages: the two dS^T key tiles and the K tile of 64 keys.  Two stages and
// two work-groups per CU (16 waves) where they fit: measured on the N=2048 and
// N=8192 causal workloads, a second resident work-group hides the copy latency
// better than deeper staging in one (4 stages, one work-group: 70 / 381 us instead
// of 53 / 256).  Where only one work-group fits (the wide heads), as many stages as
// the LDS holds, at most 4.
template <int DKP>
struct DsStages {
    static constexpr int kCols = 16 + DKP / 8;   // chunk columns: dS^T of step 0, of step 1, K
    static constexpr int kS = 8 * kChunkL;
    static constexpr int kBytes = kCols * kChunkL;
    static constexpr int kFixed = 4 * kDsList + 256;
    static constexpr int Occ = (2 * (2 * kBytes + kFixed) <= 160 * 1024) ? 2 : 1;
    static constexpr int kFit = (160 * 1024 - kFixed) / kBytes;
    static constexpr int N = Occ == 2 ? 2 : (kFit > 4 ? 4 : kFit);
    static_assert(N >= 2, "two LDS stages must fit");
};

template <int DKP>
__global__ __launch_bounds__(kDsNT) __attribute__((amdgpu_waves_per_eu(2 * DsStages<DKP>::Occ, 2 * DsStages<DKP>::Occ)))
void dq_ds_kernel(DqsArgs p)
{
    using ST = DsStages<DKP>;
    constexpr int NS = ST::N;
    // chunk columns copied per wave; when they do not split evenly, surplus copies
    // repeat a column (same bytes to the same place), so that every wave issues the
    // same number of copies per step (its vmcnt waits count on it)
    constexpr int CH = (ST::kCols + kDsW - 1) / kDsW;
    constexpr int NDT = DKP / 32, DT = (NDT + 1) / 2;
    __shared__ __attribute__((aligned(16))) char sSK[NS * ST::kBytes];
    __shared__ int sList[kDsList];
    __shared__ int sCount[kDsW + 1];

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    if ((int)blockIdx.x >= p.ndq) {
        // grouped-query reduction of dK and dV: these work-groups come after the dQ
        // grid and take the CU slots that the short query blocks free
        const int64_t total = p.red[0].items + p.red[1].items;
        for (int64_t i = (int64_t)(blockIdx.x - p.ndq) * kDsNT + tid; i < total; i += (int64_t)p.nred * kDsNT) {
            if (i < p.red[0].items)
                reduce_item(p.red[0], p.rk2, i);
            else
                reduce_item(p.red[1], p.rk2, i - p.red[0].items);
        }
        return;
    }
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;   // wave index (uniform, < 8)
    const int sw = (w >> 1) & 1, qh = w & 1, dh = w >> 2;       // step of the pair, query half, head-dim parity
    const int tr_off = tile_tr_off(lane);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)sSK;
    const int nqt = p.Np / kTR, HB = p.H * p.B;
    const QWork wk = qouter_work(blockIdx.x, (nqt + 1) / 2, HB, p.fold);   // latest queries first (most keys if causal)
    const int it0 = 2 * wk.qt, hb = wk.hb;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int nst = min(2, nqt - it0);                                // steps of this pair inside Np
    const rsrc_t rk = make_rsrc(p.k16 + (size_t)(g + p.Hkv * b) * p.Mp * DKP, (uint32_t)(p.Mp * DKP) * 2u);
    // this pair's dS^T tiles: 2 nkb128 key tiles x 2 query steps of 8 KiB, in that order
    const rsrc_t rs = make_rsrc(p.ds + ((size_t)hb * ((nqt + 1) / 2) + wk.qt) * p.nkb128 * 16384,
                                (uint32_t)p.nkb128 * 32768u);

    // copies of 64-key step ss (key tile ss: the 16 KiB of both query steps' dS^T at
    // 16384 ss.., K tile ss) into stage bf
    auto issue = [&](int ss, int bf) {
        const uint32_t stg = lds0 + (uint32_t)(bf * ST::kBytes);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = (i * kDsW + w) % ST::kCols;
            if (c < 16)   // dS^T: read once, streamed (the K tiles are reused across heads and blocks)
                lds_copy16<true>(rs, stg + c * kChunkL, (uint32_t)(ss * 16 + c) * kChunkG + (uint32_t)lane * 16u);
            else
                lds_copy16(rk, stg + (c - 16 + 16) * kChunkL,
                           (uint32_t)(ss * (DKP / 8) + c - 16) * kChunkG + (uint32_t)lane * 16u);
        }
    };

    f32x16 acc[DT];
#pragma unroll
    for (int j = 0; j < DT; ++j) acc[j] = zero16();

    for (int seg = 0; seg < p.nkb128; seg += kDsList) {
        // a key block is listed when either step sees it; bit s of its class: step s does
        const int count = build_live_list<kDsW>(sList, sCount, seg, min(seg + kDsList, p.nkb128), tid, lane, w,
                                                [&](int kb) {
            int live = 0;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                if (s2 < nst && tile_class<kTR / kMapTile, 128 / kMapTile>(p.map, p.causal, p.N, p.M, p.nqb, p.nkb,
                                                                           (it0 + s2) * (kTR / kMapTile),
                                                                           kb * (128 / kMapTile)) != kTileSkip)
                    live |= 1 << s2;
            return live;
        });
        const int nss = 2 * count;   // two 64-key steps per listed key block
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            if (i < nss) issue(2 * (sList[i >> 1] >> 2) + (i & 1), i);
        for (int li = 0; li < nss; ++li) {
            wait_vm_steps<CH>(min(nss - 1 - li, NS - 2));   // step li has landed (this wave)
            __syncthreads();                                  // ... for every wave; stage li-1 is free
            const int nx = li + NS - 1;
            if (nx < nss) issue(2 * (sList[nx >> 1] >> 2) + (nx & 1), nx % NS);
            // the dS^T tile of a step that does not see this key block was never
            // written: its copy is ignored
            if (!((sList[li >> 1] >> sw) & 1)) continue;
            const char *Sb = sSK + (li % NS) * ST::kBytes + sw * ST::kS;
            const char *Kb = sSK + (li % NS) * ST::kBytes + 2 * ST::kS;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const bf16x8 a = lds_tr8(Sb + tr_off + 4608 * qh + 512 * kk + 256 * u);
                    bf16x8 bk[DT];
#pragma unroll
                    for (int j = 0; j < DT; ++j)
                        if (2 * j + dh < NDT) bk[j] = lds_tr8(Kb + tr_off + 4608 * (2 * j + dh) + 512 * kk + 256 * u);
#pragma unroll
                    for (int j = 0; j < DT; ++j)
                        if (2 * j + dh < NDT) acc[j] = mfma_bf16(a, bk[j], acc[j]);
                }
        }
        __syncthreads();   // every wave is done with the stages before they are refilled
    }

    // ---- store dQ (scaled): lane = head-dim column, slot r = query column
    // crow(r, half) of this wave's 32, in the dS^T column order (ds_query)
    const size_t dq0 = (size_t)p.N * p.DK * hb;   // this head's dQ rows in the result slice (out_fmt elements)
    with_result_width(p.out_fmt, [&](auto w16) {
        constexpr bool W16 = decltype(w16)::value;
#pragma unroll
        for (int j = 0; j < DT; ++j) {
            const int col = (2 * j + dh) * 32 + l32;
            if (2 * j + dh < NDT && col < p.DK)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = (it0 + sw) * kTR + ds_query(32 * qh + crow(r, half));
                    if (n < p.N) store_as<W16>(p.dq, dq0 + (size_t)n * p.DK + col, acc[j][r] * p.scale, p.out_fmt);
                }
        }
    });
}

namespace {
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int DKP, int DVP, bool BF16>
hipError_t run_dq_ds(const DqsArgs &a, hipStream_t s)
{
    if constexpr (!BF16) {
        return hipErrorInvalidValue;
    } else {
        static ResidentCache slots;
        DqsArgs b = a;
        b.ndq = (a.Np / kTR + 1) / 2 * a.H * a.B;
        const int res = slots.get(reinterpret_cast<const void *>(&dq_ds_kernel<DKP>), kDsNT);
        b.fold = b.ndq <= res;
        // one round of reduction work-groups over the chip, fewer for small reductions
        const int64_t items = a.red[0].items + a.red[1].items;
        b.nred = (int)std::min<int64_t>((items + kDsNT - 1) / kDsNT, std::max(res / 2, 1));
        hipLaunchKernelGGL((dq_ds_kernel<DKP>), dim3(b.ndq + b.nred), dim3(kDsNT), 0, s, b);
        return hipGetLastError();
    }
}

template <int DKP, int DVP, bool BF16>
hipError_t run_dq(const DqArgs &a, hipStream_t s)
{
    if constexpr (!BF16) {
        return hipErrorInvalidValue;
    } else {
        const dim3 grid(ceil_div(a.N, kQBQ) * a.H * a.B * a.split);
        if (a.alibi)
            hipLaunchKernelGGL((dq_bf16_kernel<DKP, DVP, true>), grid, dim3(kQNT), 0, s, a);
        else
            hipLaunchKernelGGL((dq_bf16_kernel<DKP, DVP, false>), grid, dim3(kQNT), 0, s, a);
        return hipGetLastError();
    }
}

// One forward variant (PREP: the backward's own forward; MS: mask rows staged in
// LDS), ALiBi or not; the ALiBi instantiation shares the plain one's occupancy query.
template <int DKP, int DVP, bool PREP, bool MS>
void launch_fwd16_variant(FwdArgs16 b, int grid, hipStream_t s)
{
    static ResidentCache slots;
    const int res = slots.get(reinterpret_cast<const void *>(&fwd_bf16_kernel<DKP, DVP, PREP, false, MS>), kQNT);
    // each 32-query tile's keys split over two waves (64-query work-groups, twice as
    // many) where the plain grid fills at most half of the resident slots: causal MHA
    // N=1024, 64-wide heads, forward 27.7 -> 23.2 us.  Only the kernels that never
    // stage mask rows (two work-groups per CU) split, so that a mask and the causal
    // flag, which may differ in MS, still take the same path and give the same bits.
    if constexpr (!MS && QStages<DKP, DVP>::Occ == 2) {
        if (2 * grid <= res) {
            const int grid2 = ceil_div(b.N, kQBQ / 2) * b.H * b.B;
            b.fold = grid2 <= res;
            if (b.alibi)
                hipLaunchKernelGGL((fwd_bf16_kernel<DKP, DVP, PREP, true, MS, 2>), dim3(grid2), dim3(kQNT), 0, s, b);
            else
                hipLaunchKernelGGL((fwd_bf16_kernel<DKP, DVP, PREP, false, MS, 2>), dim3(grid2), dim3(kQNT), 0, s, b);
            return;
        }
    }
    b.fold = grid <= res;
    if (b.alibi)
        hipLaunchKernelGGL((fwd_bf16_kernel<DKP, DVP, PREP, true, MS>), dim3(grid), dim3(kQNT), 0, s, b);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<DKP, DVP, PREP, false, MS>), dim3(grid), dim3(kQNT), 0, s, b);
}

template <int DKP, int DVP, bool BF16>
hipError_t run_fwd16(const FwdArgs16 &a, hipStream_t s)
{
    if constexpr (!BF16) {
        return hipErrorInvalidValue;
    } else {
        const int grid = ceil_div(a.N, kQBQ) * a.H * a.B;
        // stage the mask rows: one work-group per CU, rows of whole 16-byte chunks, two
        // stages with the mask rows fit
        constexpr bool kMs = QStages<DKP, DVP>::Occ == 1 &&
                             2 * (QStages<DKP, DVP>::kKV + kQBQ * kQBK * 2) + QStages<DKP, DVP>::kFixed <= 160 * 1024;
        bool ms = false;
        if constexpr (kMs) ms = a.mask && a.M % 8 == 0;
        if (ms) {
            if constexpr (kMs) {
                if (a.dO)
                    launch_fwd16_variant<DKP, DVP, true, true>(a, grid, s);
                else
                    launch_fwd16_variant<DKP, DVP, false, true>(a, grid, s);
            }
        } else if (a.dO) {
            launch_fwd16_variant<DKP, DVP, true, false>(a, grid, s);
        } else {
            launch_fwd16_variant<DKP, DVP, false, false>(a, grid, s);
        }
        return hipGetLastError();
    }
}
}  // namespace

hipError_t launch_forward_bf16(const void *q, const __bf16 *k16, const __bf16 *v16, const uint16_t *mask,
                               const uint8_t *map, float scale, void *O, float *lse, int Mp, const Dims &d,
                               hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    FwdArgs16 a = {};
    a.q = q; a.k16 = k16; a.v16 = v16; a.mask = mask; a.map = map; a.O = O; a.o_bf16 = d.o_bf16; a.lse = lse;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.Mp = Mp; a.DK = d.DK; a.DV = d.DV;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile); a.causal = d.causal; a.alibi = d.alibi;
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0); a.in_fmt = d.in_fmt;
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_fwd16, a, s, hd, true);
}

hipError_t launch_forward_prep_bf16(const void *q, const __bf16 *k16, const __bf16 *v16, const uint16_t *mask,
                                    const uint8_t *map, float scale, const void *dO, __bf16 *q16, __bf16 *o16,
                                    float *stats, float *blob, int64_t nq, int64_t off_k, int64_t nk, int64_t off_v,
                                    int64_t nv, int64_t total, int *zero, int nzero, int Np, int Mp, const Dims &d,
                                    hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd) || !dO || !q16 || !o16 || !stats) return hipErrorInvalidValue;
    FwdArgs16 a = {};
    a.q = q; a.k16 = k16; a.v16 = v16; a.mask = mask; a.map = map;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.Mp = Mp; a.DK = d.DK; a.DV = d.DV;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile); a.causal = d.causal; a.alibi = d.alibi;
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0); a.in_fmt = d.in_fmt;
    a.scale = scale;
    a.dO = dO; a.q16 = q16; a.o16 = o16; a.stats = stats; a.blob = blob;
    const int u = d.out_fmt == kF32 ? 2 : 1;   // 16-bit units per blob element
    a.pad_lo[0] = u * nq; a.pad_hi[0] = u * off_k;
    a.pad_lo[1] = u * (off_k + nk); a.pad_hi[1] = u * off_v;
    a.pad_lo[2] = u * (off_v + nv); a.pad_hi[2] = u * total;
    a.zero = zero; a.nzero = nzero; a.Np = Np;
    FAB_DISPATCH_HEAD_DIMS(run_fwd16, a, s, hd, true);
}

hipError_t launch_dq(const __bf16 *q16, const __bf16 *o16, const float *stats, const __bf16 *k16, const __bf16 *v16,
                     const uint16_t *mask, const uint8_t *map, float scale, float *dq, float *part, int *ticket,
                     int Np, int Mp, const Dims &d, hipStream_t s)
{
    static_assert(kQBQ == kDqBlock, "dQ query block");
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    DqArgs a;
    a.q16 = q16; a.o16 = o16; a.stats = stats; a.k16 = k16; a.v16 = v16; a.mask = mask; a.map = map;
    a.dq = dq; a.out_fmt = d.out_fmt; a.part = part; a.ticket = ticket; a.split = dq_split(d);
    if (a.split == 2 && (!part || !ticket)) return hipErrorInvalidValue;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.Np = Np; a.M = d.M; a.Mp = Mp; a.DK = d.DK; a.DV = d.DV;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile); a.causal = d.causal; a.alibi = d.alibi;
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_dq, a, s, hd, true);
}

hipError_t launch_dq_from_ds(const __bf16 *ds, const __bf16 *k16, const uint8_t *map, float scale, float *dq, int Np,
                             int Mp, const float *pk, float *dk, const float *pv, float *dv, int upg, const Dims &d,
                             hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd) || !ds || !dq_from_ds(d, Np, hd.dk, hd.dv)) return hipErrorInvalidValue;
    DqsArgs a;
    a.ds = ds; a.k16 = k16; a.map = map; a.dq = dq; a.out_fmt = d.out_fmt;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.Np = Np; a.M = d.M; a.Mp = Mp; a.DK = d.DK;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile); a.nkb128 = ceil_div(d.M, 128);
    a.causal = d.causal;
    a.scale = scale;
    if (pk) {
        a.rk2 = gqa_reduce_jobs(pk, dk, pv, dv, d, upg, a.red);
    } else {
        a.rk2 = 1;
        a.red[0] = a.red[1] = ReduceJob{nullptr, nullptr, 0, 0, 0};
    }
    FAB_DISPATCH_HEAD_DIMS(run_dq_ds, a, s, hd, true);
}

}  // namespace fab
