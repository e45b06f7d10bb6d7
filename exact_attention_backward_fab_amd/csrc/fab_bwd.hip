// fab_bwd.hip -- key-block-outer attention backward (gfx950).
//
// A work-group owns one block of BC keys of one (batch, query head) and keeps
// its dK and dV in registers while it walks over the query tiles that see the
// block (the mask's block map drops the tiles that are all -inf).  For each
// query tile it recomputes S = scale Q K^T (+ mask) and P = exp(S - LSE) from
// the row log-sum-exp of the forward, then forms, as in the labml "Flash
// Attention" page ("Backward pass"):
//     dV += P^T dO,   dP = dO V^T,   dS = P o (dP - D),   dK += scale dS^T Q
// with D = rowsum(dO o O) from the prep (bf16: the backward's forward or the
// pack launch).  The products run on the
// matrix cores: bf16 operands with f32 accumulation (v_mfma_f32_32x32x16_bf16)
// or f32 operands (v_mfma_f32_32x32x2_f32).
//
// dQ = scale dS K: in bf16 mode this kernel stores the bf16 dS^T operands of
// its dK product, and a query-outer kernel (fab_qouter.hip) forms dQ from them
// as a plain product, writing each dQ row once (for shapes whose dS would pass
// 4 GiB a query-outer kernel recomputes S and dP instead); in
// f32 mode this kernel adds every key block's share with f32 atomics into the
// result blob.
//
// Wave layout: a wave owns 32 keys of the block (the bf16 kernel: 8 waves, 4
// key sub-blocks x 2 query halves of each 64-query step; the f32 and the wide-head
// bf16 kernels: 4 waves, all queries of a step).  S and dP come out of the matrix
// core with one key per lane (the C layout, see fab_common.h), which is exactly
// the A-operand layout of P^T and dS^T for dV and dK.
#include <algorithm>

#include "fab_common.h"
#include "fab_launch.h"
#include "fab_tiles.h"

namespace fab {

struct BwdArgs {
    const float *q, *k, *v, *dO;
    const uint16_t *mask;
    const uint8_t *map;
    const float *lse, *delta;
    float *dq, *dk, *dv;
    int B, H, Hkv, N, M, DK, DV;
    int part_heads, nqb, nkb, vecK, vecV;
    int qsplit;                     // work-groups per (key block, query head) on interleaved live query steps
    int causal;                     // causal rule as a flag (no mask, no map)
    float scale;
    const float *alibi;             // per-head ALiBi slopes [H] or NULL
};

// ============================================================== bf16 mode
// Inputs are the bf16 tiles of fab_tiles.h: Q and dO per query head ([B,H,Np,*]),
// K and V per key/value head ([B,Hkv,Mp,*]), and the per-query LSE/D blocks.  A
// work-group owns 128 keys (32 per wave, one per lane in the C layout of S and
// dP); its K and V rows are B operands held in registers.  The query tiles that
// see the block stream through LDS 64 queries at a time: the Q tile, the dO tile
// and the LSE/D block of a step are copied from global memory straight into LDS
// (several stages ahead), and every product reads its LDS operand as a per-lane
// base plus a constant offset.
struct KvArgs {
    const __bf16 *q16, *o16;          // bf16 tiles [B,H,Np,DKP] / [B,H,Np,DVP]
    const float *stats;               // LSE/D blocks [B,H,Np/64][128]
    const __bf16 *k16, *v16;          // bf16 tiles [B,Hkv,Mp,DKP] / [B,Hkv,Mp,DVP]
    const uint16_t *mask;
    const uint8_t *map;
    float *dk, *dv;
    // dS^T of every visited (key block, query step) pair for the dQ product, or
    // NULL: 64-key x 64-query bf16 tiles in the layout of fab_tiles.h (rows = keys;
    // the 16-byte chunk c = 4 qq + 2 u + half holds the 8 queries of one
    // matrix-core operand, see ds_query in fab_tiles.h), ordered
    // [B,H,ceil(Np/128)][nkb128][2 key tiles][2 query steps]: the two query steps
    // of a pair sit side by side, so the dQ product reads one contiguous stream.
    // Pairs the block map skips are not written.
    __bf16 *ds;
    uint32_t ds_bytes;              // extent of ds (below 4 GiB)
    int ds_cached;                  // dS^T stores through the caches (small totals, read back from them)
    int B, H, Hkv, N, Np, M, Mp, DK, DV;
    int hpw;                        // query heads of one group per work-group (1 or 2), summed in registers
    int qsplit;                     // work-groups per (key block, head unit) on interleaved query steps (8-wave kernel)
    int out_fmt;                    // element type of the result blob (dk, dv when not partials)
    int part_heads, nqb, nkb, nkb128;
    int causal;                     // causal rule as a flag (no mask, no map)
    float scale;
    const float *alibi;             // per-head ALiBi slopes [H] or NULL
};

// 8 waves, two per SIMD: wave w owns keys 32 (w & 3).. of the block and the
// 32-query half (w >> 2) of every 64-query step; the two halves' dK/dV are summed
// through LDS at the end.
constexpr int kKW = 8, kKNT = 64 * kKW;
constexpr int kKBC = 128;        // keys per work-group
constexpr int kKBR = kTR;        // queries per step
constexpr int kKList = 512;      // live query steps listed at a time

// LDS stages: the Q tile, the dO tile and the LSE/D block of one step each.
template <int DKP, int DVP>
struct KStages {
    static constexpr int kQ = DKP / 8 * kChunkL, kO = DVP / 8 * kChunkL, kS = kStatsTile * 4;
    static constexpr int kBytes = kQ + kO + kS;
    static constexpr int kKV = 2 * (kQ + kO);   // the block's K and V rows: two 64-row tiles each
    static constexpr int kFit = (160 * 1024 - 4 * kKList - 256 - kKV) / kBytes;
    static constexpr int N = kFit > 4 ? 4 : kFit;
    static_assert(N >= 2, "two LDS stages must fit");
};

template <int DKP, int DVP, bool AB, bool O16>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_bf16_kernel(KvArgs p)
{
    using ST = KStages<DKP, DVP>;
    constexpr int NS = ST::N;
    // chunk columns copied per wave; when a tile has fewer columns than 2 per wave,
    // the surplus copies repeat a column (same bytes to the same place) so that
    // every wave issues the same number of copies per step (its vmcnt waits count on it)
    constexpr int QCH = (DKP / 8 + kKW - 1) / kKW, OCH = (DVP / 8 + kKW - 1) / kKW;
    constexpr int PER = QCH + OCH + 1;                         // copies per wave and step
    static_assert((DKP > DVP ? DKP : DVP) / 32 * 16 * 64 * 4 * 4 <= NS * ST::kBytes, "dK/dV exchange area");
    __shared__ __attribute__((aligned(16))) char sQO[NS * ST::kBytes];
    __shared__ __attribute__((aligned(16))) char sKV[ST::kKV];   // K tiles, then V tiles of the block
    __shared__ int sList[kKList];
    __shared__ int sCount[kKW + 1];

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int kw = w & 3, qq = w >> 2;                         // key sub-block, query half
    const int row_off = tile_row_off(lane), tr_off = tile_tr_off(lane);
    const uint32_t qo_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)sQO;

    // ---- work-group -> (key block, head unit of hpw query heads of one group, query
    // split): first key blocks first (under a causal mask they see the most queries);
    // units dealt to the XCDs in contiguous ranges, the splits of a unit side by side
    const int qs = p.qsplit;
    const int hpu = p.H / p.hpw, HU = hpu * p.B * qs;
    int kb, hus;
    if (HU % 8 == 0) {
        const int xcd = blockIdx.x % 8, jj = blockIdx.x / 8, per = HU / 8;
        kb = jj / per;
        hus = xcd * per + jj % per;
    } else {
        kb = blockIdx.x / HU;
        hus = blockIdx.x % HU;
    }
    const int split = hus % qs, hu = hus / qs;   // this work-group takes live steps split, split + qs, ...
    const int hp = hu % hpu, b = hu / hpu, g = hp * p.hpw / (p.H / p.Hkv);
    const int key0 = kb * kKBC;
    const int mykey = key0 + 32 * kw + l32;  // this lane's key in the C layout of S and dP
    const float kbias = mykey < p.M ? 0.f : -INFINITY;  // keys past M never get weight
    const float sl2 = p.scale * kLog2e;
    const rsrc_t rmask = mask_rsrc(p.mask, p.N, p.M);
    const rsrc_t rds = make_rsrc(p.ds, p.ds_bytes);   // the dS^T tiles (p.ds: dq_from_ds shapes only)

    // ---- the block's K and V rows (B operands of S = Q K^T and dP = dO V^T, one key
    // per lane) into LDS: 2 tiles of each, copied by chunk columns
    {
        const rsrc_t rk = make_rsrc(p.k16 + (size_t)(g + p.Hkv * b) * p.Mp * DKP, (uint32_t)(p.Mp * DKP) * 2u);
        const rsrc_t rv = make_rsrc(p.v16 + (size_t)(g + p.Hkv * b) * p.Mp * DVP, (uint32_t)(p.Mp * DVP) * 2u);
        const uint32_t kv_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)sKV;
        // rows past Mp read as zero (buffer bounds); chunk column c of tile tt
        for (int c = w; c < 2 * (DKP / 8); c += kKW) {
            const int tt = c / (DKP / 8), cc = c - tt * (DKP / 8);
            lds_copy16(rk, kv_lds + tt * ST::kQ + cc * kChunkL,
                       (uint32_t)((key0 / 64 + tt) * DKP / 8 + cc) * kChunkG + (uint32_t)lane * 16u);
        }
        for (int c = w; c < 2 * (DVP / 8); c += kKW) {
            const int tt = c / (DVP / 8), cc = c - tt * (DVP / 8);
            lds_copy16(rv, kv_lds + 2 * ST::kQ + tt * ST::kO + cc * kChunkL,
                       (uint32_t)((key0 / 64 + tt) * DVP / 8 + cc) * kChunkG + (uint32_t)lane * 16u);
        }
        // not waited for here: the waits of the first step (and the map reads of the
        // live list) cover these older copies, so their latency overlaps
    }
    // this lane's key row in the K and V tiles: tile kw / 2, row 32 (kw & 1) + l32
    const char *Krow = sKV + (kw >> 1) * ST::kQ + 512 * (kw & 1) + row_off;
    const char *Vrow = sKV + 2 * ST::kQ + (kw >> 1) * ST::kO + 512 * (kw & 1) + row_off;
    f32x16 dkacc[DKP / 32], dvacc[DVP / 32];
#pragma unroll
    for (int i = 0; i < DKP / 32; ++i) dkacc[i] = zero16();
#pragma unroll
    for (int i = 0; i < DVP / 32; ++i) dvacc[i] = zero16();

    // the current head's Q and dO tiles and LSE/D blocks
    rsrc_t rq, ro, rs;
    auto set_head = [&](int hb) {
        const size_t qhead = (size_t)hb * p.Np;   // first tile row of this head
        rq = make_rsrc(p.q16 + qhead * DKP, (uint32_t)(p.Np * DKP) * 2u);
        ro = make_rsrc(p.o16 + qhead * DVP, (uint32_t)(p.Np * DVP) * 2u);
        rs = make_rsrc(p.stats + qhead / 64 * kStatsTile, (uint32_t)(p.Np / 64 * kStatsTile) * 4u);
    };

    // copies of query step it into stage bf: Q and dO chunk columns split over the
    // waves, lanes 0-7 of each wave copy a quarter of the LSE/D block
    auto issue = [&](int it, int bf) {
        const uint32_t stg = qo_lds + (uint32_t)(bf * ST::kBytes);
#pragma unroll
        for (int i = 0; i < QCH; ++i) {
            const int c = (i * kKW + w) % (DKP / 8);
            lds_copy16(rq, stg + c * kChunkL, (uint32_t)(it * DKP / 8 + c) * kChunkG + (uint32_t)lane * 16u);
        }
#pragma unroll
        for (int i = 0; i < OCH; ++i) {
            const int c = (i * kKW + w) % (DVP / 8);
            lds_copy16(ro, stg + ST::kQ + c * kChunkL, (uint32_t)(it * DVP / 8 + c) * kChunkG + (uint32_t)lane * 16u);
        }
        if (lane < 4)
            lds_copy16(rs, stg + ST::kQ + ST::kO + w * 64,
                       (uint32_t)(it * kStatsTile * 4 + w * 64) + (uint32_t)lane * 16u);
    };

    const int nqt = p.Np / kKBR;
    for (int hh = 0; hh < p.hpw; ++hh) {
        const int hb = hp * p.hpw + hh + p.H * b;   // this head (h + H b)
        set_head(hb);
        const float slope2 = AB ? p.alibi[hb % p.H] * kLog2e : 0.f;   // ALiBi, log2 units
        for (int seg = 0; seg < nqt; seg += kKList) {
            const int count = build_live_list<kKW>(sList, sCount, seg, min(seg + kKList, nqt), tid, lane, w, [&](int it) {
                return tile_class<kKBR / kMapTile, kKBC / kMapTile>(p.map, p.causal, p.N, p.M, p.nqb, p.nkb, it * (kKBR / kMapTile),
                                  key0 / kMapTile);
            });
            // this work-group's share of the live steps: list entries split + qs li
            const int mine = count > split ? (count - split + qs - 1) / qs : 0;
            if (mine == 0) continue;
    #pragma unroll
            for (int i = 0; i < NS - 1; ++i)
                if (i < mine) issue(sList[split + qs * i] >> 2, i);
            for (int li = 0; li < mine; ++li) {
                wait_vm_steps<PER>(min(mine - 1 - li, NS - 2));   // step li has landed (this wave)
                __syncthreads();                                   // ... for every wave; stage li-1 is free
                if (li + NS - 1 < mine) issue(sList[split + qs * (li + NS - 1)] >> 2, (li + NS - 1) % NS);
                const int e = sList[split + qs * li];
                const int it = e >> 2, cls = e & 3;
                const int q0 = it * kKBR;
                const char *Qb = sQO + (li % NS) * ST::kBytes;
                const char *Ob = Qb + ST::kQ;
                const float *Sb = reinterpret_cast<const float *>(Ob + ST::kO);

                const int qb = q0 + 32 * qq;   // first query of this wave's half

                // ---- S = Q K^T and dP = dO V^T for this wave's 32 queries (lane = key)
                f32x16 sacc = zero16(), pacc = zero16();
                {
                    // the LDS operands run R products ahead of the matrix cores (a ring of
                    // registers; the scheduling barriers keep the compiler from folding it back
                    // into read-wait-multiply pairs), S and dP products alternating
                    constexpr int TS = DKP / 16, TP = DVP / 16, T = TS > TP ? TS : TP, R = 2;
                    bf16x8 qa[R], ka[R], oa[R], va[R];
                    const char *Qrow = Qb + row_off + 512 * qq, *Orow = Ob + row_off + 512 * qq;
    #pragma unroll
                    for (int t = 0; t < T + R; ++t) {
                        if (t >= R) {
                            const int u = t - R;
                            if (u < TS) sacc = mfma_bf16(qa[u % R], ka[u % R], sacc);
                            if (u < TP) pacc = mfma_bf16(oa[u % R], va[u % R], pacc);
                        }
                        if (t < TS) { qa[t % R] = lds_row8(Qrow + 2304 * t); ka[t % R] = lds_row8(Krow + 2304 * t); }
                        if (t < TP) { oa[t % R] = lds_row8(Orow + 2304 * t); va[t % R] = lds_row8(Vrow + 2304 * t); }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }

                // ---- P = exp(scale S + mask - LSE) and dS = P o (dP - D), in f32; a step with
                // every key visible folds the scale into the exponent
                const bool fast = cls == kTileFree && key0 + kKBC <= p.M && (!AB || slope2 == 0.f);
                const float mul = fast ? sl2 : 1.f;
                if (!fast) {
                    const int thr = cls == kTileCausal ? mykey : INT_MIN;   // causal: query >= key
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float x = sacc[r] * sl2 + kbias;
                        sacc[r] = (qb + crow(r, half) >= thr) ? x : -INFINITY;
                    }
                    if (AB && slope2 != 0.f) {   // ALiBi: + slope (key - query)
                        const float ab = slope2 * (float)(mykey - qb);
    #pragma unroll
                        for (int r = 0; r < 16; ++r) sacc[r] += __builtin_fmaf(-slope2, (float)crow(r, half), ab);
                    }
                    if (cls == kTileMixed)   // this lane's 16 mask entries, all loads in flight at once
                        add_mask_column(sacc, rmask, mykey, qb, half, p.N, p.M);
                }
    #pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int qr = 32 * qq + 8 * r4 + 4 * half;
                    const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(Sb + qr);
                    const f32x4 del4 = *reinterpret_cast<const f32x4 *>(Sb + 64 + qr);
    #pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = 4 * r4 + c;
                        const float P = fast_exp2(__builtin_fmaf(sacc[r], mul, -lse4[c]));
                        sacc[r] = P;
                        pacc[r] = P * (pacc[r] - del4[c]);
                    }
                }

                // ---- dV += P^T dO and dK += dS^T Q (lane = head-dim column, rows = keys):
                // A = P^T / dS^T in operand order, B = dO / Q by transposing reads
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
                if (p.ds) {
                    // the dS^T operands of this step, for dQ = scale dS K: stored before the
                    // products so that the stores complete behind them (the next step's
                    // vmcnt wait counts them too); streaming stores, which leave the L2 to
                    // the Q and dO tiles this kernel re-reads, unless the tiles are few
                    // enough to be read back from the caches by the dQ launch
                    const uint32_t t = 2u * (uint32_t)(((((size_t)hb * ((nqt + 1) / 2) + (it >> 1)) * p.nkb128 + kb) * 4 +
                                                         (kw >> 1) * 2 + (it & 1)) * 4096 +
                                                        (4 * qq + half) * 512 + (32 * (kw & 1) + l32) * 8);
                    buf_store16(rds, t, da[0], p.ds_cached);
                    buf_store16(rds, t + 2048u, da[1], p.ds_cached);
                }
                {
                    // the transposed operands of both halves' dV and dK products in one
                    // sequence, read R2 products ahead
                    constexpr int NV = DVP / 32, NK = DKP / 32, NJ = 2 * (NV + NK), R2 = 3;
                    bf16x8 br[R2];
    #pragma unroll
                    for (int j = 0; j < NJ + R2; ++j) {
                        if (j >= R2) {
                            const int i = j - R2, u = i / (NV + NK), c = i % (NV + NK);
                            if (c < NV) dvacc[c] = mfma_bf16(pa[u], br[i % R2], dvacc[c]);
                            else dkacc[c - NV] = mfma_bf16(da[u], br[i % R2], dkacc[c - NV]);
                        }
                        if (j < NJ) {
                            const int u = j / (NV + NK), c = j % (NV + NK);
                            br[j % R2] = c < NV ? lds_tr8(Ob + tr_off + 4608 * c + 512 * qq + 256 * u)
                                                : lds_tr8(Qb + tr_off + 4608 * (c - NV) + 512 * qq + 256 * u);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            __syncthreads();   // every wave is done with the stages before they are refilled
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the K/V copies, also with no live step

    // ---- sum the two query halves: waves 4-7 hand their accumulators to waves 0-3
    // through LDS, dK then dV (the stream ended with a barrier: the stage memory is free)
    {
        float *xch = reinterpret_cast<float *>(sQO) + kw * ((DKP > DVP ? DKP : DVP) / 2) * 64;
        if (qq == 1) {
#pragma unroll
            for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xch[(16 * dt + r) * 64 + lane] = dkacc[dt][r];
        }
        __syncthreads();
        if (qq == 0) {
#pragma unroll
            for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) dkacc[dt][r] += xch[(16 * dt + r) * 64 + lane];
        }
        __syncthreads();
        if (qq == 1) {
#pragma unroll
            for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xch[(16 * dt + r) * 64 + lane] = dvacc[dt][r];
        }
        __syncthreads();
        if (qq == 1) return;
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) dvacc[dt][r] += xch[(16 * dt + r) * 64 + lane];
    }

    // ---- store dK (scaled) and dV of this key block: per unit (head unit x query
    // split; partials) or, when a unit covers the whole group, into the result
    const int hdd = p.part_heads ? hp * qs + split : g, Hd = p.part_heads ? hpu * qs : p.Hkv;
    // O16: the result slices hold 16-bit elements (p.out_fmt); partials are always f32
    const size_t dk0 = (size_t)p.DK * p.M * (hdd + Hd * b), dv0 = (size_t)p.DV * p.M * (hdd + Hd * b);
#pragma unroll
    for (int dt = 0; dt < DKP / 32; ++dt) {
        const int col = dt * 32 + l32;
        if (col < p.DK)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * kw + crow(r, half);
                if (key < p.M) store_as<O16>(p.dk, dk0 + col + (size_t)p.DK * key, dkacc[dt][r] * p.scale, p.out_fmt);
            }
    }
#pragma unroll
    for (int dt = 0; dt < DVP / 32; ++dt) {
        const int col = dt * 32 + l32;
        if (col < p.DV)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * kw + crow(r, half);
                if (key < p.M) store_as<O16>(p.dv, dv0 + col + (size_t)p.DV * key, dvacc[dt][r], p.out_fmt);
            }
    }
}

// 4-wave variant for the large head dims (K and V rows of the block in registers,
// one wave per SIMD): wave w owns keys 32w.. of the block and both 32-query halves
// of every step.  For the 256-wide heads the dK/dV columns are split over two
// work-groups per (key block, head) (kW4ColSplit): each forms the whole S and dP
// but accumulates half of the dK and dV columns, so that the accumulators fit the
// registers beside the K and V rows.
constexpr int kKW4 = 4, kKNT4 = 64 * kKW4;
template <int DKP, int DVP>
constexpr int kW4ColSplit = DKP + DVP > 384 ? 2 : 1;


// LDS stages of the 4-wave kernel: the Q tile, the dO tile and the LSE/D block of
// one step each, and with MS the step's mask rows (64 queries x the block's 128
// keys, f16, 256-byte rows).
template <int DKP, int DVP, bool MS = false>
struct KStages4 {
    static constexpr int kQ = DKP / 8 * kChunkL, kO = DVP / 8 * kChunkL, kS = kStatsTile * 4;
    static constexpr int kM = MS ? kTR * kKBC * 2 : 0;
    static constexpr int kBytes = kQ + kO + kS + kM;
    static constexpr int kFit = (160 * 1024 - 4 * kKList - 256) / kBytes;
    static constexpr int N = kFit > 4 ? 4 : kFit;
    static_assert(N >= 2, "two LDS stages must fit");
};

// MS: the mask rows of every step are copied into the LDS stage with the Q and dO
// tiles (mask given, M % 8 == 0), so a MIXED step reads its mask from LDS instead of
// waiting on 32 global loads with nothing else in flight (one wave per SIMD).
template <int DKP, int DVP, bool AB, bool MS, bool O16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_bf16_w4_kernel(KvArgs p)
{
    using ST = KStages4<DKP, DVP, MS>;
    constexpr int NS = ST::N;
    constexpr int QCH = DKP / 8 / kKW4, OCH = DVP / 8 / kKW4;   // chunk columns copied per wave
    static_assert(QCH * 8 * kKW4 == DKP && OCH * 8 * kKW4 == DVP, "tile copy split");
    constexpr int MCH = MS ? kTR * kKBC * 2 / 1024 / kKW4 : 0;   // 1 KiB mask copies per wave (4 rows each)
    constexpr int PER = QCH + OCH + 1 + MCH;                     // copies per wave and step
    __shared__ __attribute__((aligned(16))) char sQO[NS * ST::kBytes];
    __shared__ int sList[kKList];
    __shared__ int sCount[kKW4 + 1];

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int row_off = tile_row_off(lane), tr_off = tile_tr_off(lane);
    const uint32_t qo_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)sQO;

    // ---- work-group -> (key block, head, column part): first key blocks first (under
    // a causal mask they see the most queries); heads dealt to the XCDs in contiguous
    // ranges
    constexpr int CS = kW4ColSplit<DKP, DVP>;
    constexpr int NVC = DVP / 32 / CS, NKC = DKP / 32 / CS;   // dV, dK column tiles of this work-group
    const int cs = blockIdx.x % CS, bid = blockIdx.x / CS;
    const int HB = p.H * p.B;
    int kb, hb;
    if (HB % 8 == 0) {
        const int xcd = bid % 8, jj = bid / 8, per = HB / 8;
        kb = jj / per;
        hb = xcd * per + jj % per;
    } else {
        kb = bid / HB;
        hb = bid % HB;
    }
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int key0 = kb * kKBC;
    const int mykey = key0 + 32 * w + l32;  // this lane's key in the C layout of S and dP
    const float kbias = mykey < p.M ? 0.f : -INFINITY;  // keys past M never get weight
    const float sl2 = p.scale * kLog2e;
    const float slope2 = AB ? p.alibi[h] * kLog2e : 0.f;   // ALiBi, log2 units
    const rsrc_t rmask = mask_rsrc(p.mask, p.N, p.M);
    const rsrc_t rds = make_rsrc(p.ds, p.ds_bytes);   // the dS^T tiles (p.ds: dq_from_ds shapes only)

    // ---- this lane's K and V rows: B operands of S = Q K^T and dP = dO V^T
    bf16x8 kf[DKP / 16], vf[DVP / 16];
    {
        const __bf16 *kh = p.k16 + (size_t)(g + p.Hkv * b) * p.Mp * DKP;
        const __bf16 *vh = p.v16 + (size_t)(g + p.Hkv * b) * p.Mp * DVP;
        const bool in = mykey < p.Mp;
        const bf16x8 z = {};
#pragma unroll
        for (int t = 0; t < DKP / 16; ++t)
            kf[t] = in ? *reinterpret_cast<const bf16x8 *>(kh + tile_elem(mykey, 16 * t + 8 * half, DKP)) : z;
#pragma unroll
        for (int t = 0; t < DVP / 16; ++t)
            vf[t] = in ? *reinterpret_cast<const bf16x8 *>(vh + tile_elem(mykey, 16 * t + 8 * half, DVP)) : z;
    }
    f32x16 dkacc[NKC], dvacc[NVC];
#pragma unroll
    for (int i = 0; i < NKC; ++i) dkacc[i] = zero16();
#pragma unroll
    for (int i = 0; i < NVC; ++i) dvacc[i] = zero16();

    const size_t qhead = (size_t)(h + p.H * b) * p.Np;   // first tile row of this head
    const rsrc_t rq = make_rsrc(p.q16 + qhead * DKP, (uint32_t)(p.Np * DKP) * 2u);
    const rsrc_t ro = make_rsrc(p.o16 + qhead * DVP, (uint32_t)(p.Np * DVP) * 2u);
    const rsrc_t rs = make_rsrc(p.stats + qhead / 64 * kStatsTile, (uint32_t)(p.Np / 64 * kStatsTile) * 4u);

    // copies of query step it into stage bf: Q and dO chunk columns split over the
    // waves, lanes 0-7 of each wave copy a quarter of the LSE/D block
    auto issue = [&](int it, int bf) {
        const uint32_t stg = qo_lds + (uint32_t)(bf * ST::kBytes);
#pragma unroll
        for (int i = 0; i < QCH; ++i) {
            const int c = i * kKW4 + w;
            lds_copy16(rq, stg + c * kChunkL, (uint32_t)(it * DKP / 8 + c) * kChunkG + (uint32_t)lane * 16u);
        }
#pragma unroll
        for (int i = 0; i < OCH; ++i) {
            const int c = i * kKW4 + w;
            lds_copy16(ro, stg + ST::kQ + c * kChunkL, (uint32_t)(it * DVP / 8 + c) * kChunkG + (uint32_t)lane * 16u);
        }
        if (lane < 8)
            lds_copy16(rs, stg + ST::kQ + ST::kO + w * 128,
                       (uint32_t)(it * kStatsTile * 4 + w * 128) + (uint32_t)lane * 16u);
        if constexpr (MS) {
            // mask rows it*64 + 4c + lane/16, bytes 16 (lane%16).. of keys key0..key0+127;
            // rows past N read as zero (buffer bounds)
#pragma unroll
            for (int i = 0; i < MCH; ++i) {
                const int c = i * kKW4 + w, row = it * kKBR + 4 * c + (lane >> 4);
                lds_copy16(rmask, stg + ST::kQ + ST::kO + ST::kS + c * 1024,
                           2u * ((uint32_t)row * (uint32_t)p.M + (uint32_t)key0) + (uint32_t)(lane & 15) * 16u);
            }
        }
    };

    const int nqt = p.Np / kKBR;
    for (int seg = 0; seg < nqt; seg += kKList) {
        const int count = build_live_list<kKW4>(sList, sCount, seg, min(seg + kKList, nqt), tid, lane, w, [&](int it) {
            return tile_class<kKBR / kMapTile, kKBC / kMapTile>(p.map, p.causal, p.N, p.M, p.nqb, p.nkb, it * (kKBR / kMapTile),
                              key0 / kMapTile);
        });
        if (count == 0) continue;
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            if (i < count) issue(sList[i] >> 2, i);
        for (int li = 0; li < count; ++li) {
            wait_vm_steps<PER>(min(count - 1 - li, NS - 2));   // step li has landed (this wave)
            __syncthreads();                                    // ... for every wave; stage li-1 is free
            if (li + NS - 1 < count) issue(sList[li + NS - 1] >> 2, (li + NS - 1) % NS);
            const int e = sList[li];
            const int it = e >> 2, cls = e & 3;
            const int q0 = it * kKBR;
            const char *Qb = sQO + (li % NS) * ST::kBytes;
            const char *Ob = Qb + ST::kQ;
            const float *Sb = reinterpret_cast<const float *>(Ob + ST::kO);

            // ---- S = Q K^T and dP = dO V^T for two 32-query sub-tiles (lane = key); the Q
            // and dO row operands run R products ahead of the matrix cores (a register ring
            // held in place by scheduling barriers), S and dP products alternating
            f32x16 sacc[2], pacc[2];
            {
                constexpr int TS = DKP / 16, TP = DVP / 16, T = TS > TP ? TS : TP, R = 3, NJ = 2 * T;
                bf16x8 qa[R], oa[R];
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    sacc[qq] = zero16();
                    pacc[qq] = zero16();
                }
#pragma unroll
                for (int j = 0; j < NJ + R; ++j) {
                    if (j >= R) {
                        const int i = j - R, qq = i / T, t = i % T;
                        if (t < TS) sacc[qq] = mfma_bf16(qa[i % R], kf[t], sacc[qq]);
                        if (t < TP) pacc[qq] = mfma_bf16(oa[i % R], vf[t], pacc[qq]);
                    }
                    if (j < NJ) {
                        const int qq = j / T, t = j % T;
                        if (t < TS) qa[j % R] = lds_row8(Qb + row_off + 512 * qq + 2304 * t);
                        if (t < TP) oa[j % R] = lds_row8(Ob + row_off + 512 * qq + 2304 * t);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // ---- P = exp(scale S + mask - LSE) and dS = P o (dP - D), in f32; a step with
            // every key visible folds the scale into the exponent
            const bool fast = cls == kTileFree && key0 + kKBC <= p.M && (!AB || slope2 == 0.f);
            const float mul = fast ? sl2 : 1.f;
            if (!fast) {
                const int thr = cls == kTileCausal ? mykey : INT_MIN;   // causal: query >= key
#pragma unroll
                for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float x = sacc[qq][r] * sl2 + kbias;
                        sacc[qq][r] = (q0 + 32 * qq + crow(r, half) >= thr) ? x : -INFINITY;
                    }
                if (AB && slope2 != 0.f) {   // ALiBi: + slope (key - query)
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq) {
                        const float ab = slope2 * (float)(mykey - q0 - 32 * qq);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            sacc[qq][r] += __builtin_fmaf(-slope2, (float)crow(r, half), ab);
                    }
                }
                if (cls == kTileMixed) {
                    if constexpr (MS) {
                        // this lane's key column of the step's mask rows in LDS
                        const _Float16 *mcol = reinterpret_cast<const _Float16 *>(Sb + 128) + 32 * w + l32;
#pragma unroll
                        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                sacc[qq][r] += (float)mcol[(32 * qq + crow(r, half)) * kKBC] * kLog2e;
                    } else {
#pragma unroll
                        for (int qq = 0; qq < 2; ++qq)
                            add_mask_column(sacc[qq], rmask, mykey, q0 + 32 * qq, half, p.N, p.M);
                    }
                }
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int qr = 32 * qq + 8 * r4 + 4 * half;
                    const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(Sb + qr);
                    const f32x4 del4 = *reinterpret_cast<const f32x4 *>(Sb + 64 + qr);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = 4 * r4 + c;
                        const float P = fast_exp2(__builtin_fmaf(sacc[qq][r], mul, -lse4[c]));
                        sacc[qq][r] = P;
                        pacc[qq][r] = P * (pacc[qq][r] - del4[c]);
                    }
                }

            // ---- dV += P^T dO and dK += dS^T Q (lane = head-dim column, rows = keys):
            // A = P^T / dS^T in operand order, B = dO / Q by transposing reads
            bf16x8 pa4[4], da4[4];   // index 2 qq + u
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float pv[8], dv8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        pv[i] = sacc[qq][8 * u + i];
                        dv8[i] = pacc[qq][8 * u + i];
                    }
                    const bf16x8 pa = to_bf16x8(pv), da = to_bf16x8(dv8);
                    pa4[2 * qq + u] = pa;
                    da4[2 * qq + u] = da;
                    if (p.ds && cs == 0) {
                        // the dS^T operands of this step for dQ = scale dS K, in the tile
                        // layout and with the stores bwd_bf16_kernel uses
                        const uint32_t t = 2u * (uint32_t)(((((size_t)hb * ((nqt + 1) / 2) + (it >> 1)) * p.nkb128 + kb) * 4 +
                                                             (w >> 1) * 2 + (it & 1)) * 4096 +
                                                            (4 * qq + half) * 512 + u * 1024 + (32 * (w & 1) + l32) * 8);
                        buf_store16(rds, t, da, p.ds_cached);
                    }
                }
            {
                // the transposed operands of the four (half, u) groups' dV and dK products in
                // one sequence (this work-group's column tiles), read R2 products ahead
                constexpr int NV = NVC, NK = NKC, NC = NV + NK, NJ = 4 * NC, R2 = 4;
                const char *Obc = Ob + tr_off + 4608 * NV * cs, *Qbc = Qb + tr_off + 4608 * NK * cs;
                bf16x8 br[R2];
#pragma unroll
                for (int j = 0; j < NJ + R2; ++j) {
                    if (j >= R2) {
                        const int i = j - R2, gq = i / NC, c = i % NC;
                        if (c < NV) dvacc[c] = mfma_bf16(pa4[gq], br[i % R2], dvacc[c]);
                        else dkacc[c - NV] = mfma_bf16(da4[gq], br[i % R2], dkacc[c - NV]);
                    }
                    if (j < NJ) {
                        const int gq = j / NC, c = j % NC, qq = gq >> 1, u = gq & 1;
                        br[j % R2] = c < NV ? lds_tr8(Obc + 4608 * c + 512 * qq + 256 * u)
                                            : lds_tr8(Qbc + 4608 * (c - NV) + 512 * qq + 256 * u);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __syncthreads();   // every wave is done with the stages before they are refilled
    }

    // ---- store dK (scaled) and dV of this key block (this work-group's columns)
    const int hdd = p.part_heads ? h : g, Hd = p.part_heads ? p.H : p.Hkv;
    // O16: the result slices hold 16-bit elements (p.out_fmt); partials are always f32
    const size_t dk0 = (size_t)p.DK * p.M * (hdd + Hd * b), dv0 = (size_t)p.DV * p.M * (hdd + Hd * b);
#pragma unroll
    for (int dt = 0; dt < NKC; ++dt) {
        const int col = (NKC * cs + dt) * 32 + l32;
        if (col < p.DK)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * w + crow(r, half);
                if (key < p.M) store_as<O16>(p.dk, dk0 + col + (size_t)p.DK * key, dkacc[dt][r] * p.scale, p.out_fmt);
            }
    }
#pragma unroll
    for (int dt = 0; dt < NVC; ++dt) {
        const int col = (NVC * cs + dt) * 32 + l32;
        if (col < p.DV)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * w + crow(r, half);
                if (key < p.M) store_as<O16>(p.dv, dv0 + col + (size_t)p.DV * key, dvacc[dt][r], p.out_fmt);
            }
    }
}

// ============================================================== f32 mode
// f32 operands: every matrix-core operand is one float per lane, so transposed
// operands are plain strided LDS reads and no transposed copies are needed.
// A work-group has KW x QH waves: KW sub-blocks of 32 keys times QH halves of
// 32 queries of each step (the query halves of one key sub-block add their dK,
// dV through LDS at the end).  4 x 1 for the small head dims, 2 x 2 for
// 128 / 128 (every SIMD busy; the LDS just fits), 2 x 1 for the 192-wide ones,
// 1 x 1 for 256 / 256 (the K, V, Q and dO rows of one sub-block fill the LDS).
template <int DKP, int DVP>
struct F32Cfg {
    static constexpr int KW = (DKP + DVP <= 128) ? 4 : (DKP + DVP <= 384) ? 2 : 1;
    static constexpr int QH = (DKP + DVP == 256) ? 2 : 1;
    // column split: where KW x QH waves would leave SIMDs of the CU idle (the wide
    // heads, whose K, V, Q and dO rows fill the LDS for one work-group), CS waves share
    // each (key sub-block, query half): each forms the same S and dP and owns 1/CS of
    // the dK and dV column tiles, so all four SIMDs multiply
    static constexpr int CS = KW * QH >= 4 ? 1 : 4 / (KW * QH);
    static_assert((DKP / 32) % CS == 0 && (DVP / 32) % CS == 0, "column split");
    static constexpr int W = KW * QH * CS;
    static constexpr int NT = 64 * W;
    static constexpr int BC = 32 * KW;  // keys per work-group
    static_assert(BC == f32_keys_per_wg(DKP, DVP), "f32 key block");
    static constexpr int BR = 32 * QH;  // queries per step
    static constexpr int LK = DKP + 4, LV = DVP + 4, LQ = DKP + 4, LO = DVP + 4, LS = BC + 4;
};

template <int DKP, int DVP, bool AB>
__global__ __launch_bounds__((F32Cfg<DKP, DVP>::NT), 1) void bwd_f32_kernel(BwdArgs p)
{
    using C = F32Cfg<DKP, DVP>;
    constexpr int BC = C::BC, BR = C::BR, W = C::W, NT = C::NT, KW = C::KW, QH = C::QH, CS = C::CS;
    constexpr int NKT = DKP / 32 / CS, NVT = DVP / 32 / CS;   // dK, dV column tiles of a wave
    constexpr int LK = C::LK, LV = C::LV, LQ = C::LQ, LO = C::LO, LS = C::LS;
    __shared__ __attribute__((aligned(16))) float sK[BC * LK];
    __shared__ __attribute__((aligned(16))) float sV[BC * LV];
    __shared__ __attribute__((aligned(16))) float sQ[BR * LQ];
    __shared__ __attribute__((aligned(16))) float sO[BR * LO];
    __shared__ __attribute__((aligned(16))) float sS[BR * LS];   // dS: [query][key]
    __shared__ __attribute__((aligned(16))) float sL[BR];
    __shared__ __attribute__((aligned(16))) float sD[BR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int wl = w % (KW * QH), cs = w / (KW * QH);                  // (key sub-block, query half), column part
    const int kw = QH == 1 ? wl : wl % KW, qq = QH == 1 ? 0 : wl / KW;   // key sub-block, query half
    const int HB = p.H * p.B, qs = p.qsplit;
    const int split = blockIdx.x % qs, jhb = blockIdx.x / qs;   // this work-group takes live steps split, split + qs, ...
    const int j = jhb / HB, hb = jhb % HB;
    const int h = hb % p.H, b = hb / p.H, g = h / (p.H / p.Hkv);
    const int key0 = j * BC;
    const int mykey = key0 + 32 * kw + l32;
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

    f32x16 dkacc[NKT], dvacc[NVT];
#pragma unroll
    for (int i = 0; i < NKT; ++i) dkacc[i] = zero16();
#pragma unroll
    for (int i = 0; i < NVT; ++i) dvacc[i] = zero16();
    const float sl2 = p.scale * kLog2e;
    const float slope2 = AB ? p.alibi[h] * kLog2e : 0.f;   // ALiBi, log2 units
    const rsrc_t rmask = mask_rsrc(p.mask, p.N, p.M);
    const int nqt = (p.N + BR - 1) / BR;

    // Live query steps only.  Where the registers allow it (PF: head dims up to 128,
    // and the wide heads, whose column parts split the accumulators), the rows of the
    // next live step are loaded into registers while the current step computes and
    // written to LDS at the top of the next one.
    auto next_live = [&](int from, int *c) {
        for (int i = from; i < nqt; ++i) {
            *c = tile_class<BR / kMapTile, BC / kMapTile>(p.map, p.causal, p.N, p.M, p.nqb, p.nkb,
                                                          i * (BR / kMapTile), key0 / kMapTile);
            if (*c != kTileSkip) return i;
        }
        return nqt;
    };
    constexpr int PQ = BR * (DKP / 4) / NT, PO = BR * (DVP / 4) / NT;
    constexpr bool PF = (DKP + DVP <= 256 || CS > 1) && PQ * NT == BR * (DKP / 4) && PO * NT == BR * (DVP / 4);
    f32x4 pq[PF ? PQ : 1], po[PF ? PO : 1];
    float pl = INFINITY, pd = 0.f;
    auto fetch = [&](int step) {
        const int q0 = step * BR;
#pragma unroll
        for (int i = 0; i < PQ; ++i) {
            const int c = tid + i * NT, r = c / (DKP / 4), col = 4 * (c % (DKP / 4)), n = q0 + r;
            pq[i] = n < p.N ? load_row4(qh + (size_t)p.DK * n, col, p.DK, p.vecK) : z;
        }
#pragma unroll
        for (int i = 0; i < PO; ++i) {
            const int c = tid + i * NT, r = c / (DVP / 4), col = 4 * (c % (DVP / 4)), n = q0 + r;
            po[i] = n < p.N ? load_row4(dh + dstride * n, col, p.DV, p.vecV) : z;
        }
        if (tid < BR) {
            const int n = q0 + tid;
            float L = -INFINITY, Dl = 0.f;
            if (n < p.N) {
                L = p.lse[n + p.N * (h + p.H * b)];
                Dl = p.delta[n + p.N * (h + p.H * b)];
            }
            pl = (L == -INFINITY) ? INFINITY : L * kLog2e;
            pd = Dl;
        }
    };
    // this work-group's live steps: every qs-th, from the split-th on
    auto next_mine = [&](int from, int *c, int skip) {
        int i = next_live(from, c);
        for (int k = 0; k < skip && i < nqt; ++k) i = next_live(i + 1, c);
        return i;
    };
    int cls = kTileSkip;
    int it = next_mine(0, &cls, split);
    if constexpr (PF)
        if (it < nqt) fetch(it);
    while (it < nqt) {
        const int q0 = it * BR;
        int ncls = kTileSkip;
        const int nx = next_mine(it + 1, &ncls, qs - 1);
        __syncthreads();  // the previous step is done with sQ, sO, sS
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < PQ; ++i) {
                const int c = tid + i * NT, r = c / (DKP / 4), col = 4 * (c % (DKP / 4));
                *reinterpret_cast<f32x4 *>(&sQ[r * LQ + col]) = pq[i];
            }
#pragma unroll
            for (int i = 0; i < PO; ++i) {
                const int c = tid + i * NT, r = c / (DVP / 4), col = 4 * (c % (DVP / 4));
                *reinterpret_cast<f32x4 *>(&sO[r * LO + col]) = po[i];
            }
            if (tid < BR) {
                sL[tid] = pl;
                sD[tid] = pd;
            }
            if (nx < nqt) fetch(nx);
        } else {
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
        }
        __syncthreads();

        // ---- S = Q K^T, dP = dO V^T (k index = half*(D/2) + t)
        f32x16 sacc = zero16(), pacc = zero16();
        {
            const float *kr = &sK[(32 * kw + l32) * LK + half * (DKP / 2)];
            const float *vr = &sV[(32 * kw + l32) * LV + half * (DVP / 2)];
            const float *qr = &sQ[(32 * qq + l32) * LQ + half * (DKP / 2)];
            const float *orr = &sO[(32 * qq + l32) * LO + half * (DVP / 2)];
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
        // ---- P and dS (scores in log2 units; a MIXED step adds the lane's mask column with
        // all 16 loads in flight at once -- rows past N carry no weight through their LSE)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] *= sl2;
        if (cls == kTileMixed) add_mask_column(sacc, rmask, mykey, q0 + 32 * qq, half, p.N, p.M);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int qr = 32 * qq + 8 * r4 + 4 * half;
            const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(&sL[qr]);
            const f32x4 del4 = *reinterpret_cast<const f32x4 *>(&sD[qr]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = 4 * r4 + c, n = q0 + qr + c;
                float x = sacc[r];
                if (AB && slope2 != 0.f) x += slope2 * (float)(mykey - n);
                if (cls == kTileCausal) x = (mykey <= n) ? x : -INFINITY;
                const float P = keyok ? fast_exp2(x - lse4[c]) : 0.f;
                sacc[r] = P;
                pacc[r] = P * (pacc[r] - del4[c]);
            }
        }
        // ---- dV += P^T dO, dK += dS^T Q (this wave's column tiles)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int qr = 32 * qq + crow(u, half);
#pragma unroll
            for (int dt = 0; dt < NVT; ++dt)
                dvacc[dt] = mfma_f32(sacc[u], sO[qr * LO + (NVT * cs + dt) * 32 + l32], dvacc[dt]);
#pragma unroll
            for (int dt = 0; dt < NKT; ++dt)
                dkacc[dt] = mfma_f32(pacc[u], sQ[qr * LQ + (NKT * cs + dt) * 32 + l32], dkacc[dt]);
        }
        // ---- dS to LDS [query][key] (the column parts hold the same dS: part 0 writes it)
        if (cs == 0)
#pragma unroll
            for (int r = 0; r < 16; ++r) sS[(32 * qq + crow(r, half)) * LS + 32 * kw + l32] = pacc[r];
        __syncthreads();
        // ---- dQ tiles (32 queries x 32 dims), round-robin over the waves
        for (int tt = w; tt < QH * (DKP / 32); tt += W) {
            const int qt = tt / (DKP / 32), dt = tt - qt * (DKP / 32);
            f32x16 acc = zero16();
#pragma unroll
            for (int t = 0; t < BC / 2; t += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sS[(32 * qt + l32) * LS + half * (BC / 2) + t]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc = mfma_f32(a[i], sK[(half * (BC / 2) + t + i) * LK + dt * 32 + l32], acc);
            }
            const int col = dt * 32 + l32;
            if (col < p.DK)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = q0 + 32 * qt + crow(r, half);
                    if (n < p.N) unsafeAtomicAdd(dqh + col + (size_t)p.DK * n, acc[r] * p.scale);
                }
        }
        it = nx;
        cls = ncls;
    }

    // ---- the second query half hands its dK, dV to the first through the K and V
    // rows, which are no longer read (sK holds KW x dK tiles, sV KW x dV tiles)
    if constexpr (QH == 2) {
        static_assert(CS == 1, "query halves and column parts are not combined");
        static_assert(KW * (DKP / 32) * 1024 <= BC * LK && KW * (DVP / 32) * 1024 <= BC * LV,
                      "dK/dV exchange area");
        float *xk = sK + kw * (DKP / 32) * 1024;
        float *xv = sV + kw * (DVP / 32) * 1024;
        __syncthreads();   // every wave is done with sK and sV
        if (qq == 1) {
#pragma unroll
            for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xk[(dt * 16 + r) * 64 + lane] = dkacc[dt][r];
#pragma unroll
            for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xv[(dt * 16 + r) * 64 + lane] = dvacc[dt][r];
        }
        __syncthreads();
        if (qq == 1) return;
#pragma unroll
        for (int dt = 0; dt < DKP / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) dkacc[dt][r] += xk[(dt * 16 + r) * 64 + lane];
#pragma unroll
        for (int dt = 0; dt < DVP / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) dvacc[dt][r] += xv[(dt * 16 + r) * 64 + lane];
    }

    const int hd = p.part_heads ? h * qs + split : g, Hd = p.part_heads ? p.H * qs : p.Hkv;
    float *dkb = p.dk + (size_t)p.DK * p.M * (hd + Hd * b);
    float *dvb = p.dv + (size_t)p.DV * p.M * (hd + Hd * b);
#pragma unroll
    for (int dt = 0; dt < NKT; ++dt) {
        const int col = (NKT * cs + dt) * 32 + l32;
        if (col < p.DK)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * kw + crow(r, half);
                if (key < p.M) dkb[col + (size_t)p.DK * key] = dkacc[dt][r] * p.scale;
            }
    }
#pragma unroll
    for (int dt = 0; dt < NVT; ++dt) {
        const int col = (NVT * cs + dt) * 32 + l32;
        if (col < p.DV)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * kw + crow(r, half);
                if (key < p.M) dvb[col + (size_t)p.DV * key] = dvacc[dt][r];
            }
    }
}

// ============================================================== launchers
namespace {
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int DKP, int DVP, bool BF16>
hipError_t run_bwd_f32(const BwdArgs &a, hipStream_t s)
{
    if constexpr (BF16) {
        return hipErrorInvalidValue;
    } else {
        using C = F32Cfg<DKP, DVP>;
        if (a.alibi)
            hipLaunchKernelGGL((bwd_f32_kernel<DKP, DVP, true>), dim3(ceil_div(a.M, C::BC) * a.H * a.B * a.qsplit),
                               dim3(C::NT), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_f32_kernel<DKP, DVP, false>), dim3(ceil_div(a.M, C::BC) * a.H * a.B * a.qsplit),
                               dim3(C::NT), 0, s, a);
        return hipGetLastError();
    }
}

// The kernel instance for the result's element width: 16-bit only when the kernel
// itself writes a 16-bit result (partials stay f32).
inline void launch_o16(const KvArgs &a, void (*k32)(KvArgs), void (*k16)(KvArgs), dim3 grid, int nt, hipStream_t s)
{
    hipLaunchKernelGGL((!a.part_heads && a.out_fmt != kF32) ? k16 : k32, grid, dim3(nt), 0, s, a);
}

template <int DKP, int DVP, bool BF16>
hipError_t run_bwd_bf16(const KvArgs &a, hipStream_t s)
{
    if constexpr (!BF16) {
        return hipErrorInvalidValue;
    } else if constexpr (DKP + DVP <= 256) {
        const dim3 grid(ceil_div(a.M, kKBC) * (a.H / a.hpw) * a.B * a.qsplit);
        if (a.alibi)
            launch_o16(a, bwd_bf16_kernel<DKP, DVP, true, false>, bwd_bf16_kernel<DKP, DVP, true, true>, grid, kKNT, s);
        else
            launch_o16(a, bwd_bf16_kernel<DKP, DVP, false, false>, bwd_bf16_kernel<DKP, DVP, false, true>, grid, kKNT, s);
        return hipGetLastError();
    } else {
        const dim3 grid(ceil_div(a.M, kKBC) * a.H * a.B * kW4ColSplit<DKP, DVP>);
        // mask rows staged in LDS (16-byte aligned rows), where two stages with them fit
        constexpr bool kMsFits = 2 * (KStages4<DKP, DVP>::kBytes + kTR * kKBC * 2) + 4 * kKList + 256 <= 160 * 1024;
        const bool ms = kMsFits && a.mask && a.M % 8 == 0;
        if constexpr (kMsFits) {
            if (ms) {
                if (a.alibi)
                    launch_o16(a, bwd_bf16_w4_kernel<DKP, DVP, true, true, false>, bwd_bf16_w4_kernel<DKP, DVP, true, true, true>, grid,
                               kKNT4, s);
                else
                    launch_o16(a, bwd_bf16_w4_kernel<DKP, DVP, false, true, false>, bwd_bf16_w4_kernel<DKP, DVP, false, true, true>, grid,
                               kKNT4, s);
                return hipGetLastError();
            }
        }
        if (a.alibi)
            launch_o16(a, bwd_bf16_w4_kernel<DKP, DVP, true, false, false>, bwd_bf16_w4_kernel<DKP, DVP, true, false, true>, grid,
                               kKNT4, s);
        else
            launch_o16(a, bwd_bf16_w4_kernel<DKP, DVP, false, false, false>, bwd_bf16_w4_kernel<DKP, DVP, false, false, true>, grid,
                               kKNT4, s);
        return hipGetLastError();
    }
}
}  // namespace

hipError_t launch_backward_f32(const float *q, const float *k, const float *v, const float *dO,
                               const uint16_t *mask, const uint8_t *map, const float *lse, const float *delta,
                               float scale, float *dq, float *dk, float *dv, int part_heads, const Dims &d,
                               hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dO = dO; a.mask = mask; a.map = map;
    a.lse = lse; a.delta = delta; a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.M = d.M; a.DK = d.DK; a.DV = d.DV;
    a.part_heads = part_heads;
    a.qsplit = f32_query_splits(d, hd.dk, hd.dv);
    if (a.qsplit > 1 && !part_heads) return hipErrorInvalidValue;   // the splits' partials need the reduction
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile); a.causal = d.causal; a.alibi = d.alibi;
    a.vecK = (d.DK % 4 == 0); a.vecV = (d.DV % 4 == 0);
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_bwd_f32, a, s, hd, false);
}

hipError_t launch_backward_bf16(const __bf16 *q16, const __bf16 *o16, const float *stats, const __bf16 *k16,
                                const __bf16 *v16, const uint16_t *mask, const uint8_t *map, float scale, float *dk,
                                float *dv, __bf16 *ds, int part_heads, int Np, int Mp, const Dims &d, hipStream_t s)
{
    HeadDims hd;
    if (!pick_head_dims(d.DK, d.DV, &hd)) return hipErrorInvalidValue;
    if (ds && !dq_from_ds(d, Np, hd.dk, hd.dv)) return hipErrorInvalidValue;
    KvArgs a;
    a.q16 = q16; a.o16 = o16; a.stats = stats; a.k16 = k16; a.v16 = v16; a.mask = mask; a.map = map;
    a.dk = dk; a.dv = dv; a.ds = ds; a.nkb128 = ceil_div(d.M, 128);
    // dS^T totals up to 64 MiB stay in the caches between the two launches (the dQ
    // launch reads them back from there); larger ones are streamed past the L2
    a.ds_bytes = ds ? (uint32_t)ds_bytes(d, Np) : 0u;
    a.out_fmt = d.out_fmt;
    a.ds_cached = ds && ds_bytes(d, Np) <= ((int64_t)64 << 20);
    a.hpw = bwd_heads_per_wg(d, hd.dk, hd.dv);
    a.qsplit = bwd_query_splits(d, hd.dk, hd.dv);
    // partials only while a unit (head unit x query split) is smaller than its group
    if (part_heads != (bwd_units_per_group(d, hd.dk, hd.dv) > 1 ? 1 : 0)) return hipErrorInvalidValue;
    a.B = d.B; a.H = d.H; a.Hkv = d.Hkv; a.N = d.N; a.Np = Np; a.M = d.M; a.Mp = Mp; a.DK = d.DK; a.DV = d.DV;
    a.part_heads = part_heads;
    a.nqb = ceil_div(d.N, kMapTile); a.nkb = ceil_div(d.M, kMapTile); a.causal = d.causal; a.alibi = d.alibi;
    a.scale = scale;
    FAB_DISPATCH_HEAD_DIMS(run_bwd_bf16, a, s, hd, true);
}

}  // namespace fab
