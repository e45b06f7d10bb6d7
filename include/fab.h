/*
 * fab.h -- C ABI of libfab: the exact (flash) attention backward on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the one PowerInfer's "Function ggml_flash_attn_back"
 * constructs and the ggmlR test file "tests/testthat/test-flash-attn-back.R"
 * exercises: given q, k, v, an optional additive f16 mask and the upstream
 * gradient d of the attention output, return the gradients of sum(d * attn)
 * with respect to q, k and v, packed into one f32 buffer.  The backward
 * formulas are those of the labml "Flash Attention" page, section "Backward
 * pass" (dV = P^T dO, dP = dO V^T, D = rowsum(dO o O), dS = P o (dP - D),
 * dQ = scale dS K, dK = scale dS^T Q); the forward and its running max/sum
 * are that page's "Forward pass" and "Flash Attention Optimization" sections.
 *
 * Tensor conventions (ggml ne order, ne0 fastest; every tensor contiguous f32,
 * as in the ggmlR test file's header comment of `attn_ref`):
 *     q    [DK, N,   H,   B]   element (c,n,h,b) at c + DK*(n + N*(h + H*b))
 *     k    [DK, M,   Hkv, B]   element (c,m,g,b) at c + DK*(m + M*(g + Hkv*b))
 *     v    [DV, M,   Hkv, B]   element (c,m,g,b) at c + DV*(m + M*(g + Hkv*b))
 *     d, O [DV, H,   N,   B]   element (c,h,n,b) at c + DV*(h + H*(n + N*b))
 *     mask [M,  N]  f16 bits   element (m,n)     at m + M*n, shared by all h, b
 *     lse  [N,  H,   B]        element (n,h,b)   at n + N*(h + H*b)
 * Query head h reads key/value head g = h / (H/Hkv) (grouped-query attention;
 * H must be a multiple of Hkv).  Scores are scale*(q.k) + mask[m,n]: the scale
 * multiplies first, then the mask is added.  A query row whose scores are all
 * -inf is all-masked: its output row, its LSE (-inf) and its dQ row are zero
 * and it contributes nothing to dK and dV.  The mask may hold finite values
 * and -inf; +inf and NaN entries are outside the contract.
 *
 * Result blob (f32), the layout of "Function ggml_flash_attn_back" and the
 * ggmlR test's `fab_grads` unpacker: [dQ | pad | dK | pad | dV | pad] with
 *     off_q = 0, off_k = pad4(nq), off_v = off_k + pad4(nk), total = off_v + pad4(nv)
 * in floats, where nq, nk, nv are the element counts of q, k, v and
 * pad4(x) = ceil(x/4)*4 (16-byte alignment).  Every float of the blob is
 * written; the pads are zero.  A 16-bit blob (FAB_BF16_BLOB, FAB_F16_BLOB) has
 * the same order with pad8 in 16-bit elements (fab_blob_layout16).
 *
 * Ownership and threading: the caller allocates and owns every buffer (inputs,
 * outputs, workspace).  The compute entry points never allocate, free or
 * synchronise device memory; they only enqueue kernels on the caller's stream
 * and keep no state between calls, so calls on different streams with separate
 * workspaces may run concurrently.  Two exceptions hold process-wide state:
 * fab_backward_noalloc works in one static device array per GPU (calls that
 * overlap on one GPU race, see its declaration), and the measurement hooks
 * below create HIP events on first use, keep them until the process ends, and
 * while enabled record them on the caller's stream around every launch (the
 * hooks are meant for one thread at a time).
 *
 * Errors: every entry point validates all arguments before touching the
 * device.  On any error nothing is enqueued and no output byte is written; the
 * return value is a negative fab_status and fab_last_error() describes it
 * (thread-local).  FAB_E_HIP reports a failed kernel launch; faults inside a
 * kernel surface at the caller's next synchronisation of the stream.
 */
#ifndef FAB_H
#define FAB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FAB_VERSION 100  /* 1.0.0 */

/* Problem extents.  B, N, M >= 0 (zero gives an empty problem); H, Hkv, DK,
 * DV >= 1; H % Hkv == 0; DK, DV <= 256; every tensor below 2^31 elements, and
 * one head's rows (N or M, rounded up to 64) times its padded head dim below
 * 2^30 (FAB_E_UNSUPPORTED otherwise). */
typedef struct fab_shape {
    int64_t B, H, Hkv, N, M, DK, DV;
} fab_shape;

/* Arithmetic mode of the dense contractions.
 *   FAB_MODE_F32 : f32 operands on the f32 matrix cores (f32 accumulation).
 *   FAB_MODE_BF16: q, k, v, d and the intermediate P and dS are rounded to
 *                  bf16 (round-to-nearest-even) as matrix-core operands; all
 *                  accumulation, the softmax statistics, D and the scale stay f32. */
typedef enum fab_mode { FAB_MODE_F32 = 0, FAB_MODE_BF16 = 1 } fab_mode;

/* Flag OR-ed into the mode argument of fab_workspace_bytes, fab_forward_lse and
 * fab_backward: the causal rule without a mask tensor -- key m is seen by query
 * n iff m <= n (the boolean `masked` argument of PowerInfer's
 * `ggml_flash_attn_back`; for N != M the same rule as the 0 / -inf f16 mask
 * with entry (n, m) = 0 iff m <= n).  The mask pointer must then be NULL
 * (has_mask = 0), else FAB_E_INVAL; no block map is built and no mask is read. */
#define FAB_CAUSAL 0x100

/* Flag OR-ed into the mode argument: q, k, v and d are bf16 (16-bit bit
 * patterns, the same layouts) instead of f32 -- the storage the bf16 matrix
 * cores read anyway, so the values are those FAB_MODE_BF16 would round f32
 * inputs to, and the results equal those for the f32 inputs holding the same
 * values.  FAB_MODE_BF16 only (FAB_E_INVAL otherwise); O (unless FAB_BF16_O),
 * lse and the blob stay f32. */
#define FAB_BF16_INPUTS 0x200

/* Flag OR-ed into the mode argument: O is bf16 (16-bit bit patterns, layout
 * [DV,H,N,B]) instead of f32 -- written so by fab_forward_lse (the f32 output
 * rounded to nearest even) and read so by fab_backward (D = rowsum(dO o O) from
 * those values, widened exactly).  FAB_MODE_BF16 only (FAB_E_INVAL otherwise);
 * it combines with FAB_BF16_INPUTS or FAB_F16_INPUTS.  lse and the blob stay f32. */
#define FAB_BF16_O 0x400

/* Flag OR-ed into the mode argument: q, k, v and d are IEEE binary16 (f16, the
 * 16-bit storage of the ggmlR reference manual's tensors; same layouts) instead
 * of f32.  Each value is widened exactly to f32 and then handled as an f32 input
 * (rounded to bf16 for the matrix cores; D = rowsum(dO o O) from the widened dO),
 * so the results equal those for the f32 inputs holding the same values.
 * FAB_MODE_BF16 only, and not together with FAB_BF16_INPUTS (FAB_E_INVAL
 * otherwise); O (unless FAB_BF16_O), lse and the blob stay f32. */
#define FAB_F16_INPUTS 0x800

/* Flags OR-ed into the mode argument of fab_backward (and its ALiBi and
 * allocation-free forms) and fab_workspace_bytes: the result blob holds bf16
 * (FAB_BF16_BLOB) or IEEE f16 (FAB_F16_BLOB) elements instead of f32 -- each the
 * f32 gradient the kernels accumulate, rounded to nearest even once at the
 * store (half-precision storage of gradients, as the ggmlR package description on
 * its ggml_flash_attn_back page names half precision among the package's features).
 * The blob then follows fab_blob_layout16: the same [dQ | pad | dK | pad | dV |
 * pad] order with each slice padded to 16 bytes (8 elements), pads zero.  Every
 * accumulation, including the grouped-query sums of dK and dV, stays f32, so the
 * 16-bit blob is element for element the rounding of the f32 blob.  The
 * workspace is unchanged.  FAB_MODE_BF16 only, exclusive of each other, and
 * FAB_E_INVAL in fab_forward_lse (which writes no blob). */
#define FAB_BF16_BLOB 0x1000
#define FAB_F16_BLOB 0x2000

typedef enum fab_status {
    FAB_OK = 0,
    FAB_E_INVAL = -1,        /* bad shape, NULL pointer, bad scale or mode */
    FAB_E_UNSUPPORTED = -2,  /* valid but outside what the kernels handle (DK/DV > 256, size) */
    FAB_E_WORKSPACE = -3,    /* workspace missing or smaller than fab_workspace_bytes() */
    FAB_E_ALIGN = -4,        /* a pointer is not 16-byte aligned (workspace: 256-byte) */
    FAB_E_HIP = -5           /* a HIP launch or runtime call failed */
} fab_status;

/* Host only.  Blob offsets and total length, in floats (see above).
 * Returns FAB_OK or FAB_E_INVAL. */
int fab_blob_layout(const fab_shape *shape, int64_t *off_q, int64_t *off_k, int64_t *off_v,
                    int64_t *total_floats);

/* Host only.  The same for a 16-bit blob (FAB_BF16_BLOB, FAB_F16_BLOB):
 * offsets and total length in 16-bit elements, each slice padded to a multiple
 * of 8 elements.  Returns FAB_OK or FAB_E_INVAL. */
int fab_blob_layout16(const fab_shape *shape, int64_t *off_q, int64_t *off_k, int64_t *off_v,
                      int64_t *total_elems);

/* Host only.  Workspace bytes that fab_forward_lse (have_o_lse ignored) or
 * fab_backward need for this shape, mode and mask presence.  have_o_lse != 0
 * means the caller will pass O and lse to fab_backward.  *bytes is written on
 * FAB_OK.  In bf16 mode the backward's workspace holds the bf16 dS of every
 * (query, key) pair, 2 * B * H * ceil(N/128)*128 * ceil(M/128)*128 bytes, as long
 * as that is below 4 GiB (e.g. 2.1 GB for B=1, H=16, N=M=8192); larger shapes
 * compute dQ without it. */
int fab_workspace_bytes(const fab_shape *shape, int mode, int has_mask, int have_o_lse,
                        size_t *bytes);

/* Forward with row log-sum-exp (labml "Flash Attention": "Forward pass" and the
 * running max/sum of "Flash Attention Optimization").
 *   q, k, v   device, f32 (bf16 with FAB_BF16_INPUTS, f16 with FAB_F16_INPUTS), layouts
 *             above (read only)
 *   mask      device f16 bits [M,N] or NULL for no mask (read only)
 *   scale     finite f32 softmax scale
 *   mode      fab_mode, optionally | FAB_CAUSAL (then mask must be NULL)
 *             | FAB_BF16_INPUTS or FAB_F16_INPUTS, FAB_BF16_O (FAB_MODE_BF16 only)
 *   O         device f32 (bf16 with FAB_BF16_O) [DV,H,N,B] (written):
 *             softmax(scale*q.k + mask) v
 *   lse       device f32 [N,H,B] (written): natural-log log-sum-exp of the row's
 *             scores, -inf for an all-masked row
 *   ws        device workspace of ws_bytes >= fab_workspace_bytes(.., have_o_lse=1)
 *   stream    hipStream_t of the caller (NULL = default stream) */
int fab_forward_lse(const fab_shape *shape, const void *q, const void *k, const void *v,
                    const uint16_t *mask, float scale, int mode, void *O, float *lse, void *ws,
                    size_t ws_bytes, void *stream);

/* The attention backward ("Function ggml_flash_attn_back"; ggmlR
 * `fab_grads`): gradients of sum(d * attn(q,k,v)) packed into blob.
 *   q, k, v, mask, scale, mode  as for fab_forward_lse
 *   d         device f32 (bf16 / f16 with FAB_BF16_INPUTS / FAB_F16_INPUTS) [DV,H,N,B]: upstream gradient
 *             of the attention output
 *   O, lse    either both NULL (the forward is recomputed internally, the
 *             pages' semantics) or both given: the output and row LSE of the
 *             same forward (as written by fab_forward_lse; O f32, or bf16 with
 *             FAB_BF16_O); exactly one NULL is FAB_E_INVAL
 *   blob      device f32, total_floats of fab_blob_layout (written in full); with
 *             FAB_BF16_BLOB / FAB_F16_BLOB 16-bit elements, total_elems of
 *             fab_blob_layout16
 *   ws        device workspace, ws_bytes >= fab_workspace_bytes(.., have_o_lse)
 *   stream    hipStream_t of the caller */
int fab_backward(const fab_shape *shape, const void *q, const void *k, const void *v,
                 const uint16_t *mask, const void *d, float scale, int mode, const void *O,
                 const float *lse, void *blob, void *ws, size_t ws_bytes, void *stream);

/* ALiBi: fab_forward_lse and fab_backward with a linear per-head bias on the
 * scores.  The ggmlR test file names ALiBi only through `max_bias`, in its block
 * "the graph builder rejects attention features it cannot differentiate", and
 * gives no score function; the reading taken here: the caller passes one slope
 * per query head, and the score of query n at key m becomes
 *     scale * (q . k) + alibi[h] * (m - n) + mask[m, n]
 * (the bias after the scale, next to the mask; softmax, LSE and the backward
 * formulas unchanged).  ggml's geometric slopes (from max_bias) or any others are
 * the caller's choice.
 *   alibi   device f32 [H] (read only, 4-byte aligned) or NULL: then these calls
 *           are exactly fab_forward_lse / fab_backward.  Finite slopes only.
 * Every other argument, the workspace and the errors are as for fab_forward_lse /
 * fab_backward; O and lse passed to fab_backward_alibi must come from the forward
 * with the same slopes. */
int fab_forward_lse_alibi(const fab_shape *shape, const void *q, const void *k, const void *v,
                          const uint16_t *mask, const float *alibi, float scale, int mode, void *O, float *lse,
                          void *ws, size_t ws_bytes, void *stream);
int fab_backward_alibi(const fab_shape *shape, const void *q, const void *k, const void *v,
                       const uint16_t *mask, const float *alibi, const void *d, float scale, int mode,
                       const void *O, const float *lse, void *blob, void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: fab_backward
 * (same arguments, kernels and results, same validation and error codes) with
 * its workspace taken from a fixed array of FAB_NOALLOC_SCRATCH_BYTES inside the
 * library instead of a caller's buffer.  The call allocates and frees nothing;
 * the array is device memory that each GPU the library runs on holds from the
 * time the library's code is loaded on it until the process ends.  The caller
 * still passes every input and the blob.
 *   Limit: shapes whose fab_workspace_bytes(.., has_mask = mask != NULL,
 *   have_o_lse = O != NULL) exceeds FAB_NOALLOC_SCRATCH_BYTES return
 *   FAB_E_UNSUPPORTED (nothing enqueued); e.g. B=2, H=8, N=M=1024, D=64 in bf16
 *   mode needs about 56 MiB.
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *   last call's contents (the kernels write every workspace byte they read, so
 *   nothing needs to start at zero).  Calls that overlap on one GPU -- on two
 *   streams, or from two threads without ordering -- race on the array and give
 *   undefined results; calls ordered on one stream are safe. */
#define FAB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fab_backward_noalloc(const fab_shape *shape, const void *q, const void *k, const void *v,
                         const uint16_t *mask, const void *d, float scale, int mode, const void *O,
                         const float *lse, void *blob, void *stream);

/* Measurement hooks (they compute nothing).  While enabled, every kernel
 * launch made by fab_forward_lse and fab_backward is bracketed by a pair of
 * HIP events recorded on the caller's stream.  fab_profile_read waits for the
 * recorded events of one kernel -- "block_map" (f32 mode), "forward", "prep"
 * (f32 mode), "pack" (bf16 copies of k and v, the block map of the mask, and with
 * O and lse supplied also of q and the prep of d), "backward" (dK, dV; f32 mode
 * also dQ), "dq" (bf16 mode's dQ, with the
 * grouped-query reduction of dK and dV when dQ comes from the stored dS) or
 * "gqa_reduce" -- and returns their summed
 * duration in milliseconds and the
 * number of launches since the last fab_profile_reset.  The events are created
 * by the library on first use and kept for reuse; only one thread should use
 * the hooks at a time.  Returns FAB_OK, FAB_E_INVAL (unknown kernel name or
 * NULL output) or FAB_E_HIP. */
int fab_profile_enable(int on);
int fab_profile_reset(void);
int fab_profile_read(const char *kernel, double *total_ms, int64_t *launches);

/* Measurement hook (computes nothing of the attention): the sustained rate of the
 * bf16 matrix cores on this GPU.  A fully resident grid in which every wave
 * runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 products
 * (32x32x16x2 flops each) is timed with two HIP events on `stream` (after a
 * short warm-up launch); *tflops receives the rate and *clock_ghz the shader
 * clock over the run (s_memtime cycles per 100 MHz s_memrealtime tick, averaged
 * over 64 work-groups).  The chip lowers its clock under this load, so the rate
 * is the practical ceiling of dense bf16 products, below the published peak.
 * scratch: device memory of at least fab_probe_scratch_bytes() bytes, owned by
 * the caller, overwritten.  Synchronises `stream`; creates and destroys two
 * events.  iters in [1, 2^24].  Returns FAB_OK, FAB_E_INVAL or FAB_E_HIP. */
size_t fab_probe_scratch_bytes(void);
int fab_measure_mfma_loop(void *scratch, size_t scratch_bytes, int iters, double *tflops, double *clock_ghz,
                          void *stream);

/* Static text for a status code. */
const char *fab_strerror(int status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char *fab_last_error(void);
/* FAB_VERSION of the library. */
int fab_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FAB_H */
