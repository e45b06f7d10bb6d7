// fab_api.cpp -- the C ABI of libfab (see include/fab.h): argument
// validation, result-blob layout, workspace carving and the launch sequence.
// No HIP call is made before every argument has been checked, so the
// validation paths run on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/fab.h"
#include "fab_launch.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int kMaxHeadDim = 256;
constexpr size_t kWsAlign = 256;

int64_t pad4(int64_t n) { return (n + 3) / 4 * 4; }
int64_t pad8(int64_t n) { return (n + 7) / 8 * 8; }
size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
    fab::Dims d;
    int64_t nq, nk, nv, nrow, nO, off_k, off_v, total;   // blob offsets and length in its elements
    int esize;                                            // bytes of one blob element (4, or 2 for 16-bit)
    // workspace offsets (bytes) and total
    size_t ws_map, ws_k16, ws_v16, ws_fwd, ws_lse, ws_O, ws_delta, ws_q16, ws_o16, ws_stats, ws_dqp, ws_tick, ws_ds,
        ws_pk, ws_pv, ws_bytes;
    int dkp, dvp;  // padded head dims of the kernels
    int np;        // query rows per head of the bf16 Q / dO tiles
    int mp;        // key rows per head of the bf16 K / V copies
    bool gqa;
    bool ds;       // bf16 mode: dQ from the stored dS^T tiles (else the recompute kernel)
    int upg;       // dK/dV partials per key/value head (1: none, the kernels write the result)
    bool part;     // dK/dV go through per-unit partials and the grouped-query reduction
};

// Blob layout [dQ | pad | dK | pad | dV | pad] for elements of fmt: every slice
// starts on a 16-byte boundary (4 f32 or 8 16-bit elements).
void set_blob_layout(Plan *pl, int fmt)
{
    const bool h = fmt != fab::kF32;
    auto pad = h ? pad8 : pad4;
    pl->esize = h ? 2 : 4;
    pl->d.out_fmt = fmt;
    pl->off_k = pad(pl->nq);
    pl->off_v = pl->off_k + pad(pl->nk);
    pl->total = pl->off_v + pad(pl->nv);
}

// Shape checks: the asserts of "Function ggml_flash_attn_back" restated for the
// ggmlR layouts (q [DK,N,H,B], k [DK,M,Hkv,B], v [DV,M,Hkv,B], d [DV,H,N,B]),
// plus the limits of these kernels.
int check_shape(const fab_shape *s, Plan *pl)
{
    if (!s) return fail(FAB_E_INVAL, "shape is NULL");
    if (s->B < 0 || s->N < 0 || s->M < 0)
        return fail(FAB_E_INVAL, "B, N and M must be >= 0 (got B=%lld N=%lld M=%lld)",
                    (long long)s->B, (long long)s->N, (long long)s->M);
    if (s->H < 1 || s->Hkv < 1 || s->DK < 1 || s->DV < 1)
        return fail(FAB_E_INVAL, "H, Hkv, DK and DV must be >= 1");
    if (s->H % s->Hkv != 0)
        return fail(FAB_E_INVAL, "H (%lld) must be a multiple of Hkv (%lld)", (long long)s->H,
                    (long long)s->Hkv);
    if (s->DK > kMaxHeadDim || s->DV > kMaxHeadDim)
        return fail(FAB_E_UNSUPPORTED, "head dims above %d are not supported (DK=%lld DV=%lld)",
                    kMaxHeadDim, (long long)s->DK, (long long)s->DV);
    // element counts, computed with overflow guards
    const double fq = (double)s->DK * s->N * s->H * s->B;
    const double fk = (double)s->DK * s->M * s->H * s->B;  // per-head dK partials bound nk
    const double fv = (double)s->DV * s->M * s->H * s->B;
    const double fo = (double)s->DV * s->N * s->H * s->B;
    const double fm = (double)s->M * s->N;
    if (fq > kMaxElems || fk > kMaxElems || fv > kMaxElems || fo > kMaxElems || fm > kMaxElems)
        return fail(FAB_E_UNSUPPORTED, "a tensor exceeds 2^31-1 elements");
    pl->d = fab::Dims{(int)s->B, (int)s->H, (int)s->Hkv, (int)s->N, (int)s->M, (int)s->DK, (int)s->DV};
    pl->nq = s->DK * s->N * s->H * s->B;
    pl->nk = s->DK * s->M * s->Hkv * s->B;
    pl->nv = s->DV * s->M * s->Hkv * s->B;
    pl->nO = s->DV * s->H * s->N * s->B;
    pl->nrow = s->N * s->H * s->B;
    set_blob_layout(pl, fab::kF32);
    if ((double)pl->total > kMaxElems) return fail(FAB_E_UNSUPPORTED, "result blob exceeds 2^31-1 floats");
    pl->gqa = s->H > s->Hkv;
    fab::HeadDims hd;
    if (!fab::pick_head_dims((int)s->DK, (int)s->DV, &hd)) return fail(FAB_E_UNSUPPORTED, "head dims");
    pl->dkp = hd.dk;
    pl->dvp = hd.dv;
    pl->mp = (int)((s->M + fab::kPackRows - 1) / fab::kPackRows * fab::kPackRows);
    pl->np = (int)((s->N + fab::kPackRows - 1) / fab::kPackRows * fab::kPackRows);
    // one head's bf16 tiles are addressed with 32-bit offsets: keep them below 2 GiB
    const double head_elems = (double)std::max(pl->mp, pl->np) * std::max(pl->dkp, pl->dvp);
    if (head_elems >= (double)(1 << 30))
        return fail(FAB_E_UNSUPPORTED, "one head's rows exceed the kernels' 32-bit tile addressing (N or M too large)");
    return FAB_OK;
}

// Workspace carving (256-byte aligned sub-buffers, in this order):
//   map        u8 block map of the mask                       (mask given)
//   k16, v16   bf16 K / V rows, Mp per head, swizzled chunks   (bf16 mode)
//   lse, O     forward recompute                               (O, lse not given, f32 mode)
//   delta      f32 D = rowsum(dO o O) [N,H,B]                  (backward, f32 mode)
//   q16, o16   bf16 Q / dO tiles, Np rows per head             (backward, bf16 mode)
//   stats      LSE / D blocks [B][H][Np/64][128]               (backward, bf16 mode)
//   dqp, tick  dQ partials of split query blocks and counters  (backward, bf16 mode, dQ by recompute, few blocks)
//   ds         bf16 dS^T tiles [B,H,Np/64,ceil(M/128)][128x64]  (backward, bf16 mode, dQ from dS)
//   pk, pv     dK / dV partials per head unit                  (backward, H > Hkv * hpw)
// ws_fwd is the end of the part the forward alone uses.
void plan_workspace(Plan *pl, int mode, int has_mask, int have_o_lse)
{
    const fab::Dims &d = pl->d;
    size_t off = 0;
    const int64_t nqb = (d.N + 31) / 32, nkb = (d.M + 31) / 32;
    pl->ws_map = off;
    if (has_mask) off = align_up(off + (size_t)(nqb * nkb));
    pl->ws_k16 = off;
    pl->ws_v16 = off;
    if (mode == FAB_MODE_BF16) {
        const size_t kvrows = (size_t)pl->mp * d.Hkv * d.B;
        off = align_up(off + 2 * kvrows * pl->dkp);
        pl->ws_v16 = off;
        off = align_up(off + 2 * kvrows * pl->dvp);
    }
    pl->ws_fwd = off;
    pl->ws_lse = off;
    pl->ws_O = off;
    if (!have_o_lse && mode == FAB_MODE_F32) {   // bf16: the backward's own forward stores no O
        off = align_up(off + sizeof(float) * (size_t)pl->nrow);
        pl->ws_O = off;
        off = align_up(off + sizeof(float) * (size_t)pl->nO);
    }
    pl->ws_delta = off;
    if (mode == FAB_MODE_F32) off = align_up(off + sizeof(float) * (size_t)pl->nrow);
    pl->ws_q16 = off;
    pl->ws_o16 = off;
    pl->ws_stats = off;
    if (mode == FAB_MODE_BF16) {
        const size_t qrows = (size_t)pl->np * d.H * d.B;
        off = align_up(off + 2 * qrows * pl->dkp);
        pl->ws_o16 = off;
        off = align_up(off + 2 * qrows * pl->dvp);
        pl->ws_stats = off;
        off = align_up(off + sizeof(float) * qrows / 64 * 128);
    }
    pl->ds = mode == FAB_MODE_BF16 && fab::dq_from_ds(d, pl->np, pl->dkp, pl->dvp);
    pl->upg = mode == FAB_MODE_BF16 ? fab::bwd_units_per_group(d, pl->dkp, pl->dvp)
                                    : fab::f32_units_per_group(d, pl->dkp, pl->dvp);
    pl->part = pl->upg > 1;
    pl->ws_dqp = off;
    pl->ws_tick = off;
    pl->ws_ds = off;
    if (pl->ds) {
        off = align_up(off + (size_t)fab::ds_bytes(d, pl->np));
    } else if (mode == FAB_MODE_BF16) {
        off = align_up(off + sizeof(float) * (size_t)fab::dq_part_floats(d, pl->dkp));
        pl->ws_tick = off;
        off = align_up(off + sizeof(int) * (size_t)fab::dq_split_blocks(d));
    }
    pl->ws_pk = off;
    pl->ws_pv = off;
    if (pl->part) {   // one partial per unit (head unit x query split)
        off = align_up(off + sizeof(float) * (size_t)d.DK * d.M * ((size_t)d.Hkv * pl->upg) * d.B);
        pl->ws_pv = off;
        off = align_up(off + sizeof(float) * (size_t)d.DV * d.M * ((size_t)d.Hkv * pl->upg) * d.B);
    }
    pl->ws_bytes = off;
}

int check_mode(int mode)
{
    if (mode != FAB_MODE_F32 && mode != FAB_MODE_BF16) return fail(FAB_E_INVAL, "unknown mode %d", mode);
    return FAB_OK;
}

// Splits the FAB_CAUSAL, FAB_BF16_INPUTS, FAB_F16_INPUTS, FAB_BF16_O, FAB_BF16_BLOB and
// FAB_F16_BLOB flags off the mode argument and checks the rest; *in_fmt receives the
// storage of q, k, v and d, *out_fmt (when given) the blob's element type.  Without
// out_fmt (the forward, which writes no blob) the blob flags are FAB_E_INVAL.
int take_mode(int *mode, bool *causal, int *in_fmt, bool *o_bf16 = nullptr, int *out_fmt = nullptr)
{
    *causal = (*mode & FAB_CAUSAL) != 0;
    const bool ib = (*mode & FAB_BF16_INPUTS) != 0, ih = (*mode & FAB_F16_INPUTS) != 0;
    const bool ob = (*mode & FAB_BF16_O) != 0;
    const bool bb = (*mode & FAB_BF16_BLOB) != 0, hb = (*mode & FAB_F16_BLOB) != 0;
    if (o_bf16) *o_bf16 = ob;
    *mode &= ~(FAB_CAUSAL | FAB_BF16_INPUTS | FAB_F16_INPUTS | FAB_BF16_O | FAB_BF16_BLOB | FAB_F16_BLOB);
    const int rc = check_mode(*mode);
    if (rc != FAB_OK) return rc;
    if (ib && ih) return fail(FAB_E_INVAL, "FAB_BF16_INPUTS and FAB_F16_INPUTS are exclusive");
    if (ib && *mode != FAB_MODE_BF16) return fail(FAB_E_INVAL, "FAB_BF16_INPUTS needs FAB_MODE_BF16");
    if (ih && *mode != FAB_MODE_BF16) return fail(FAB_E_INVAL, "FAB_F16_INPUTS needs FAB_MODE_BF16");
    if (ob && *mode != FAB_MODE_BF16) return fail(FAB_E_INVAL, "FAB_BF16_O needs FAB_MODE_BF16");
    if ((bb || hb) && !out_fmt) return fail(FAB_E_INVAL, "FAB_BF16_BLOB / FAB_F16_BLOB apply to the backward only");
    if (bb && hb) return fail(FAB_E_INVAL, "FAB_BF16_BLOB and FAB_F16_BLOB are exclusive");
    if ((bb || hb) && *mode != FAB_MODE_BF16) return fail(FAB_E_INVAL, "FAB_BF16_BLOB / FAB_F16_BLOB need FAB_MODE_BF16");
    *in_fmt = ib ? fab::kBF16 : (ih ? fab::kF16 : fab::kF32);
    if (out_fmt) *out_fmt = bb ? fab::kBF16 : (hb ? fab::kF16 : fab::kF32);
    return FAB_OK;
}

int check_ptr(const void *p, int64_t elems, const char *name)
{
    if (elems == 0) return FAB_OK;
    if (!p) return fail(FAB_E_INVAL, "%s is NULL", name);
    if (!aligned16(p)) return fail(FAB_E_ALIGN, "%s is not 16-byte aligned", name);
    return FAB_OK;
}

// ALiBi slopes: a device array of H floats, or NULL for none.
int check_alibi(const float *alibi)
{
    if (alibi && (reinterpret_cast<uintptr_t>(alibi) & 3u) != 0)
        return fail(FAB_E_ALIGN, "alibi is not 4-byte aligned");
    return FAB_OK;
}

int check_ws(const void *ws, size_t ws_bytes, size_t need)
{
    if (need == 0) return FAB_OK;
    if (!ws) return fail(FAB_E_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if ((reinterpret_cast<uintptr_t>(ws) & (kWsAlign - 1)) != 0)
        return fail(FAB_E_ALIGN, "workspace is not %zu-byte aligned", kWsAlign);
    if (ws_bytes < need) return fail(FAB_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return FAB_OK;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(FAB_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FAB_TRY(x)                 \
    do {                           \
        const int rc__ = (x);      \
        if (rc__ != FAB_OK) return rc__; \
    } while (0)

#define FAB_HIP(call, what)                        \
    do {                                           \
        const hipError_t e__ = (call);             \
        if (e__ != hipSuccess) return hip_fail(e__, what); \
    } while (0)

// ---------------------------------------------------------------- measurement hooks
enum Kid { kMap = 0, kFwd, kPrep, kBwd, kRed, kPack, kDq, kNumKid };
const char *const kKidNames[kNumKid] = {"block_map", "forward", "prep", "backward", "gqa_reduce", "pack", "dq"};

struct ProfRec {
    int kid;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event()
{
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Brackets one launch with events when profiling is on.
struct ProfScope {
    int kid;
    hipStream_t s;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(int k, hipStream_t st) : kid(k), s(st)
    {
        if (!g_prof_on) return;
        std::lock_guard<std::mutex> lk(g_prof_mu);
        a = prof_event();
        b = prof_event();
        if (a) (void)hipEventRecord(a, s);
    }
    ~ProfScope()
    {
        if (!a || !b) return;
        (void)hipEventRecord(b, s);
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof_recs.push_back(ProfRec{kid, a, b});
    }
};

#define FAB_LAUNCH(kid, call, what)             \
    do {                                        \
        ProfScope ps__(kid, s);                 \
        FAB_HIP(call, what);                    \
    } while (0)

// The bf16 tiles of Q (when q16 is given), K and V (bf16 mode), one launch.
// (and the block map of the mask when map is given: the same launch)
int launch_pack(const Plan &pl, const void *q, const void *k, const void *v, __bf16 *q16, __bf16 *k16,
                __bf16 *v16, const uint16_t *mask, uint8_t *map, hipStream_t s)
{
    FAB_LAUNCH(kPack,
               fab::launch_pack_qkv(q16 ? q : nullptr, k, v, q16, k16, v16, mask, map, pl.np, pl.mp, pl.d, s),
               "pack launch");
    return FAB_OK;
}

int launch_fwd(const Plan &pl, int bf16, const void *q, const void *k, const void *v, const __bf16 *k16,
               const __bf16 *v16, const uint16_t *mask, const uint8_t *map, float scale, void *O, float *lse,
               hipStream_t s)
{
    if (bf16)
        FAB_LAUNCH(kFwd, fab::launch_forward_bf16(q, k16, v16, mask, map, scale, O, lse, pl.mp, pl.d, s),
                   "forward launch");
    else
        FAB_LAUNCH(kFwd,
                   fab::launch_forward_f32(static_cast<const float *>(q), static_cast<const float *>(k),
                                           static_cast<const float *>(v), mask, map, scale, static_cast<float *>(O),
                                           lse, pl.d, s),
                   "forward launch");
    return FAB_OK;
}

}  // namespace

int fab::set_error(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

extern "C" {

int fab_profile_enable(int on)
{
    g_err[0] = 0;
    g_prof_on = on != 0;
    return FAB_OK;
}

int fab_profile_reset(void)
{
    g_err[0] = 0;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (ProfRec &r : g_prof_recs) {
        (void)hipEventSynchronize(r.b);
        g_prof_pool.push_back(r.a);
        g_prof_pool.push_back(r.b);
    }
    g_prof_recs.clear();
    return FAB_OK;
}

int fab_profile_read(const char *kernel, double *total_ms, int64_t *launches)
{
    g_err[0] = 0;
    if (!kernel || !total_ms || !launches) return fail(FAB_E_INVAL, "NULL argument");
    int kid = -1;
    for (int i = 0; i < kNumKid; ++i)
        if (std::strcmp(kernel, kKidNames[i]) == 0) kid = i;
    if (kid < 0) return fail(FAB_E_INVAL, "unknown kernel name '%s'", kernel);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    double sum = 0.0;
    int64_t n = 0;
    for (ProfRec &r : g_prof_recs) {
        if (r.kid != kid) continue;
        FAB_HIP(hipEventSynchronize(r.b), "event sync");
        float ms = 0.f;
        FAB_HIP(hipEventElapsedTime(&ms, r.a, r.b), "event elapsed time");
        sum += ms;
        ++n;
    }
    *total_ms = sum;
    *launches = n;
    return FAB_OK;
}

int fab_version(void) { return FAB_VERSION; }

const char *fab_strerror(int status)
{
    switch (status) {
    case FAB_OK: return "ok";
    case FAB_E_INVAL: return "invalid argument";
    case FAB_E_UNSUPPORTED: return "unsupported shape";
    case FAB_E_WORKSPACE: return "workspace missing or too small";
    case FAB_E_ALIGN: return "misaligned pointer";
    case FAB_E_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char *fab_last_error(void) { return g_err; }

int fab_blob_layout(const fab_shape *shape, int64_t *off_q, int64_t *off_k, int64_t *off_v,
                    int64_t *total_floats)
{
    g_err[0] = 0;
    Plan pl;
    FAB_TRY(check_shape(shape, &pl));
    if (off_q) *off_q = 0;
    if (off_k) *off_k = pl.off_k;
    if (off_v) *off_v = pl.off_v;
    if (total_floats) *total_floats = pl.total;
    return FAB_OK;
}

int fab_blob_layout16(const fab_shape *shape, int64_t *off_q, int64_t *off_k, int64_t *off_v,
                      int64_t *total_elems)
{
    g_err[0] = 0;
    Plan pl;
    FAB_TRY(check_shape(shape, &pl));
    set_blob_layout(&pl, fab::kBF16);
    if (off_q) *off_q = 0;
    if (off_k) *off_k = pl.off_k;
    if (off_v) *off_v = pl.off_v;
    if (total_elems) *total_elems = pl.total;
    return FAB_OK;
}

int fab_workspace_bytes(const fab_shape *shape, int mode, int has_mask, int have_o_lse, size_t *bytes)
{
    g_err[0] = 0;
    Plan pl;
    FAB_TRY(check_shape(shape, &pl));
    bool causal;
    int in_fmt, out_fmt;
    FAB_TRY(take_mode(&mode, &causal, &in_fmt, nullptr, &out_fmt));   // the blob's type changes no workspace
    if (!bytes) return fail(FAB_E_INVAL, "bytes is NULL");
    if (causal && has_mask) return fail(FAB_E_INVAL, "a mask and FAB_CAUSAL exclude each other");
    plan_workspace(&pl, mode, has_mask != 0, have_o_lse != 0);
    *bytes = pl.ws_bytes;
    return FAB_OK;
}

int fab_forward_lse_alibi(const fab_shape *shape, const void *q, const void *k, const void *v,
                          const uint16_t *mask, const float *alibi, float scale, int mode, void *O, float *lse,
                          void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    Plan pl;
    FAB_TRY(check_shape(shape, &pl));
    bool causal, o_bf16;
    int in_fmt;
    FAB_TRY(take_mode(&mode, &causal, &in_fmt, &o_bf16));
    if (causal && mask) return fail(FAB_E_INVAL, "a mask and FAB_CAUSAL exclude each other");
    FAB_TRY(check_alibi(alibi));
    pl.d.causal = causal;
    pl.d.in_fmt = in_fmt;
    pl.d.o_bf16 = o_bf16;
    pl.d.alibi = alibi;
    if (!std::isfinite(scale)) return fail(FAB_E_INVAL, "scale is not finite");
    FAB_TRY(check_ptr(q, pl.nq, "q"));
    FAB_TRY(check_ptr(k, pl.nk, "k"));
    FAB_TRY(check_ptr(v, pl.nv, "v"));
    FAB_TRY(check_ptr(O, pl.nO, "O"));
    FAB_TRY(check_ptr(lse, pl.nrow, "lse"));
    if (mask && !aligned16(mask)) return fail(FAB_E_ALIGN, "mask is not 16-byte aligned");
    const bool use_mask = mask && (int64_t)pl.d.M * pl.d.N > 0;
    plan_workspace(&pl, mode, use_mask, 1);
    const size_t need = pl.nrow == 0 ? 0 : pl.ws_fwd;
    FAB_TRY(check_ws(ws, ws_bytes, need));
    if (pl.nrow == 0) return FAB_OK;  // no query rows: nothing to write

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *wsb = static_cast<char *>(ws);
    uint8_t *map = use_mask ? reinterpret_cast<uint8_t *>(wsb + pl.ws_map) : nullptr;
    const int bf16 = mode == FAB_MODE_BF16;
    __bf16 *k16 = bf16 ? reinterpret_cast<__bf16 *>(wsb + pl.ws_k16) : nullptr;
    __bf16 *v16 = bf16 ? reinterpret_cast<__bf16 *>(wsb + pl.ws_v16) : nullptr;
    if (bf16)
        FAB_TRY(launch_pack(pl, q, k, v, nullptr, k16, v16, mask, map, s));
    else if (map)
        FAB_LAUNCH(kMap, fab::launch_block_map(mask, map, pl.d, s), "block map launch");
    FAB_TRY(launch_fwd(pl, bf16, q, k, v, k16, v16, use_mask ? mask : nullptr, map, scale, O, lse, s));
    return FAB_OK;
}

int fab_backward_alibi(const fab_shape *shape, const void *q, const void *k, const void *v,
                       const uint16_t *mask, const float *alibi, const void *d, float scale, int mode,
                       const void *O, const float *lse, void *blob, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    Plan pl;
    FAB_TRY(check_shape(shape, &pl));
    bool causal, o_bf16;
    int in_fmt, out_fmt;
    FAB_TRY(take_mode(&mode, &causal, &in_fmt, &o_bf16, &out_fmt));
    set_blob_layout(&pl, out_fmt);
    if (causal && mask) return fail(FAB_E_INVAL, "a mask and FAB_CAUSAL exclude each other");
    FAB_TRY(check_alibi(alibi));
    pl.d.causal = causal;
    pl.d.in_fmt = in_fmt;
    pl.d.o_bf16 = o_bf16;
    pl.d.alibi = alibi;
    if (!std::isfinite(scale)) return fail(FAB_E_INVAL, "scale is not finite");
    if ((O == nullptr) != (lse == nullptr))
        return fail(FAB_E_INVAL, "O and lse must be given together or both be NULL");
    const bool have = O != nullptr;
    FAB_TRY(check_ptr(q, pl.nq, "q"));
    FAB_TRY(check_ptr(k, pl.nk, "k"));
    FAB_TRY(check_ptr(v, pl.nv, "v"));
    FAB_TRY(check_ptr(d, pl.nO, "d"));
    if (have) {
        FAB_TRY(check_ptr(O, pl.nO, "O"));
        FAB_TRY(check_ptr(lse, pl.nrow, "lse"));
    }
    FAB_TRY(check_ptr(blob, pl.total, "blob"));
    if (mask && !aligned16(mask)) return fail(FAB_E_ALIGN, "mask is not 16-byte aligned");
    const bool use_mask = mask && (int64_t)pl.d.M * pl.d.N > 0;
    plan_workspace(&pl, mode, use_mask, have);
    const bool empty = pl.d.B == 0 || pl.d.N == 0 || pl.d.M == 0;
    FAB_TRY(check_ws(ws, ws_bytes, empty ? 0 : pl.ws_bytes));
    if (pl.total == 0) return FAB_OK;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (empty) {
        // no queries (dK = dV = 0) or no keys (every row all-masked: dQ = 0)
        FAB_HIP(fab::launch_zero(static_cast<float *>(blob), pl.total * pl.esize / 4, s), "zero blob");
        return FAB_OK;
    }
    char *wsb = static_cast<char *>(ws);
    // the blob's slices as the kernels take them: element offsets of the blob's type
    float *const bq = static_cast<float *>(blob);
    float *const bk = reinterpret_cast<float *>(static_cast<char *>(blob) + pl.off_k * pl.esize);
    float *const bv = reinterpret_cast<float *>(static_cast<char *>(blob) + pl.off_v * pl.esize);
    uint8_t *map = use_mask ? reinterpret_cast<uint8_t *>(wsb + pl.ws_map) : nullptr;
    const uint16_t *mk = use_mask ? mask : nullptr;
    const int bf16 = mode == FAB_MODE_BF16;
    __bf16 *k16 = bf16 ? reinterpret_cast<__bf16 *>(wsb + pl.ws_k16) : nullptr;
    __bf16 *v16 = bf16 ? reinterpret_cast<__bf16 *>(wsb + pl.ws_v16) : nullptr;
    __bf16 *q16 = bf16 ? reinterpret_cast<__bf16 *>(wsb + pl.ws_q16) : nullptr;
    if (map && !bf16) FAB_LAUNCH(kMap, fab::launch_block_map(mk, map, pl.d, s), "block map launch");
    __bf16 *o16 = bf16 ? reinterpret_cast<__bf16 *>(wsb + pl.ws_o16) : nullptr;
    float *stats = bf16 ? reinterpret_cast<float *>(wsb + pl.ws_stats) : nullptr;
    float *dqp = bf16 && !pl.ds ? reinterpret_cast<float *>(wsb + pl.ws_dqp) : nullptr;
    int *tick = bf16 && !pl.ds ? reinterpret_cast<int *>(wsb + pl.ws_tick) : nullptr;
    const int ntick = tick ? (int)fab::dq_split_blocks(pl.d) : 0;
    __bf16 *dst = pl.ds ? reinterpret_cast<__bf16 *>(wsb + pl.ws_ds) : nullptr;
    float *delta = reinterpret_cast<float *>(wsb + pl.ws_delta);
    const float *lseu = lse;
    if (bf16 && !have) {
        // the backward's own forward writes the Q and dO tiles and the LSE/D blocks
        // directly (no O, no separate prep pass); dQ is written once by the
        // query-block-outer kernel (only its pad is zeroed)
        FAB_TRY(launch_pack(pl, q, k, v, nullptr, k16, v16, mk, map, s));
        FAB_LAUNCH(kFwd, fab::launch_forward_prep_bf16(q, k16, v16, mk, map, scale, d, q16, o16, stats, bq, pl.nq,
                                                       pl.off_k, pl.nk, pl.off_v, pl.nv, pl.total, tick, ntick, pl.np,
                                                       pl.mp, pl.d, s),
                   "forward launch");
    } else if (bf16) {
        // the bf16 tiles of Q, K, V (and the block map) with the dO tiles and LSE/D
        // blocks of the supplied O and LSE: one launch
        FAB_LAUNCH(kPack,
                   fab::launch_pack_prep_bf16(q, k, v, q16, k16, v16, mk, map, d, O, lse, o16, stats, bq, pl.nq,
                                              pl.off_k, pl.nk, pl.off_v, pl.nv, pl.total, tick, ntick, pl.np, pl.mp,
                                              pl.d, s),
                   "pack and prep launch");
    } else {
        // f32: dQ is accumulated by atomics into a zeroed slice
        const float *Ou = static_cast<const float *>(O);   // f32 mode: O is f32
        if (!have) {
            float *Ow = reinterpret_cast<float *>(wsb + pl.ws_O);
            float *lw = reinterpret_cast<float *>(wsb + pl.ws_lse);
            FAB_TRY(launch_fwd(pl, bf16, q, k, v, k16, v16, mk, map, scale, Ow, lw, s));
            Ou = Ow;
            lseu = lw;
        }
        FAB_LAUNCH(kPrep, fab::launch_prep(static_cast<const float *>(d), Ou, delta, bq, pl.off_k, pl.nk, pl.off_v,
                                           pl.nv, pl.total, pl.d, s),
                   "prep launch");
    }
    float *dk = pl.part ? reinterpret_cast<float *>(wsb + pl.ws_pk) : bk;
    float *dv = pl.part ? reinterpret_cast<float *>(wsb + pl.ws_pv) : bv;
    if (bf16) {
        FAB_LAUNCH(kBwd, fab::launch_backward_bf16(q16, o16, stats, k16, v16, mk, map, scale, dk, dv, dst,
                                                   pl.part ? 1 : 0, pl.np, pl.mp, pl.d, s),
                   "backward launch");
        if (pl.ds)   // with the grouped-query reduction of dK and dV in the same launch
            FAB_LAUNCH(kDq, fab::launch_dq_from_ds(dst, k16, map, scale, bq, pl.np, pl.mp, pl.part ? dk : nullptr,
                                                   bk, pl.part ? dv : nullptr, bv, pl.upg,
                                                   pl.d, s),
                       "dQ launch");
        else
            FAB_LAUNCH(kDq, fab::launch_dq(q16, o16, stats, k16, v16, mk, map, scale, bq, dqp, tick, pl.np, pl.mp,
                                           pl.d, s),
                       "dQ launch");
    } else {
        FAB_LAUNCH(kBwd, fab::launch_backward_f32(static_cast<const float *>(q), static_cast<const float *>(k),
                                                  static_cast<const float *>(v), static_cast<const float *>(d), mk,
                                                  map, lseu, delta, scale, bq, dk, dv,
                                                  pl.part ? 1 : 0, pl.d, s),
                   "backward launch");
    }
    if (pl.part && !pl.ds) {
        FAB_LAUNCH(kRed, fab::launch_gqa_reduce(dk, bk, dv, bv, pl.d, pl.upg, s),
                   "dK/dV reduce launch");
    }
    return FAB_OK;
}

int fab_forward_lse(const fab_shape *shape, const void *q, const void *k, const void *v,
                    const uint16_t *mask, float scale, int mode, void *O, float *lse, void *ws,
                    size_t ws_bytes, void *stream)
{
    return fab_forward_lse_alibi(shape, q, k, v, mask, nullptr, scale, mode, O, lse, ws, ws_bytes, stream);
}

int fab_backward(const fab_shape *shape, const void *q, const void *k, const void *v,
                 const uint16_t *mask, const void *d, float scale, int mode, const void *O,
                 const float *lse, void *blob, void *ws, size_t ws_bytes, void *stream)
{
    return fab_backward_alibi(shape, q, k, v, mask, nullptr, d, scale, mode, O, lse, blob, ws, ws_bytes, stream);
}

}  // extern "C"
