"""Python binding of libfab, the exact attention backward for AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfab.so`` (built in-tree by ``build.py``).  PyTorch supplies
device memory and the stream; no attention arithmetic happens here.  If the
library is missing the import of this module's compute entry points fails
loudly; there is no fallback.

Tensors use ggml ne order stored C-contiguous with the shape reversed (see
include/fab.h): q (B,H,N,DK), k (B,Hkv,M,DK), v (B,Hkv,M,DV), d and O
(B,N,H,DV), lse (B,H,N), mask (N,M) int16/uint16 f16 bit patterns or float16.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfab.so")

FAB_MODE_F32 = 0
FAB_MODE_BF16 = 1
FAB_CAUSAL = 0x100   # flag: the causal rule (key m seen by query n iff m <= n) without a mask
FAB_BF16_INPUTS = 0x200   # flag: q, k, v, d are bf16 (bf16 mode only)
FAB_F16_INPUTS = 0x800    # flag: q, k, v, d are f16 (bf16 mode only)
FAB_BF16_O = 0x400        # flag: O is bf16 (bf16 mode only)
FAB_BF16_BLOB = 0x1000    # flag: the result blob is bf16 (bf16 mode, backward only)
FAB_F16_BLOB = 0x2000     # flag: the result blob is f16 (bf16 mode, backward only)
MODES = {"f32": FAB_MODE_F32, "bf16": FAB_MODE_BF16, FAB_MODE_F32: FAB_MODE_F32,
         FAB_MODE_BF16: FAB_MODE_BF16}

FAB_OK = 0
FAB_E_INVAL = -1
FAB_E_UNSUPPORTED = -2
FAB_E_WORKSPACE = -3
FAB_E_ALIGN = -4
FAB_E_HIP = -5

# every symbol include/fab.h declares
EXPORTS = ("fab_blob_layout", "fab_blob_layout16", "fab_workspace_bytes", "fab_forward_lse", "fab_backward",
           "fab_forward_lse_alibi", "fab_backward_alibi", "fab_backward_noalloc", "fab_profile_enable", "fab_profile_reset", "fab_profile_read",
           "fab_probe_scratch_bytes", "fab_measure_mfma_loop", "fab_strerror", "fab_last_error", "fab_version")
KERNELS = ("block_map", "forward", "prep", "pack", "backward", "dq", "gqa_reduce")


class FabShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "H", "Hkv", "N", "M", "DK", "DV")]


class FabError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libfab error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libfab.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python exact_attention_backward_fab_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        SP = ctypes.POINTER(FabShape)
        L.fab_blob_layout.restype = I
        L.fab_blob_layout.argtypes = [SP, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                      ctypes.POINTER(I64), ctypes.POINTER(I64)]
        L.fab_blob_layout16.restype = I
        L.fab_blob_layout16.argtypes = [SP, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                        ctypes.POINTER(I64), ctypes.POINTER(I64)]
        L.fab_workspace_bytes.restype = I
        L.fab_workspace_bytes.argtypes = [SP, I, I, I, ctypes.POINTER(SZ)]
        L.fab_forward_lse.restype = I
        L.fab_forward_lse.argtypes = [SP, P, P, P, P, ctypes.c_float, I, P, P, P, SZ, P]
        L.fab_backward.restype = I
        L.fab_backward.argtypes = [SP, P, P, P, P, P, ctypes.c_float, I, P, P, P, P, SZ, P]
        L.fab_forward_lse_alibi.restype = I
        L.fab_forward_lse_alibi.argtypes = [SP, P, P, P, P, P, ctypes.c_float, I, P, P, P, SZ, P]
        L.fab_backward_alibi.restype = I
        L.fab_backward_alibi.argtypes = [SP, P, P, P, P, P, P, ctypes.c_float, I, P, P, P, P, SZ, P]
        L.fab_backward_noalloc.restype = I
        L.fab_backward_noalloc.argtypes = [SP, P, P, P, P, P, ctypes.c_float, I, P, P, P, P]
        L.fab_strerror.restype = ctypes.c_char_p
        L.fab_strerror.argtypes = [I]
        L.fab_last_error.restype = ctypes.c_char_p
        L.fab_last_error.argtypes = []
        L.fab_version.restype = I
        L.fab_version.argtypes = []
        L.fab_profile_enable.restype = I
        L.fab_profile_enable.argtypes = [I]
        L.fab_profile_reset.restype = I
        L.fab_profile_reset.argtypes = []
        L.fab_profile_read.restype = I
        L.fab_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(I64)]
        L.fab_probe_scratch_bytes.restype = SZ
        L.fab_probe_scratch_bytes.argtypes = []
        L.fab_measure_mfma_loop.restype = I
        L.fab_measure_mfma_loop.argtypes = [P, SZ, I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), P]
        _lib = L
    return _lib


def _check(rc):
    if rc != FAB_OK:
        raise FabError(rc, lib().fab_last_error().decode() or lib().fab_strerror(rc).decode())


@dataclass(frozen=True)
class Shape:
    B: int
    H: int
    Hkv: int
    N: int
    M: int
    DK: int
    DV: int

    def c(self):
        return FabShape(self.B, self.H, self.Hkv, self.N, self.M, self.DK, self.DV)


def shape_of(q, k, v):
    B, H, N, DK = q.shape
    Bk, Hkv, M, DKk = k.shape
    DV = v.shape[-1]
    return Shape(B, H, Hkv, N, M, DK, DV)


def _blob_dtypes():
    import torch
    return (torch.float32, torch.bfloat16, torch.float16)


def blob_layout(shape: Shape, dtype=None):
    """(off_q, off_k, off_v, total) of the packed [dQ | dK | dV] blob, in elements of
    dtype: float32 (None; fab_blob_layout) or bfloat16 / float16 (fab_blob_layout16)."""
    if dtype is not None and dtype not in _blob_dtypes():
        raise TypeError(f"blob dtype must be float32, bfloat16 or float16, got {dtype}")
    f32 = dtype is None or dtype == _blob_dtypes()[0]
    fn = lib().fab_blob_layout if f32 else lib().fab_blob_layout16
    o = [ctypes.c_int64() for _ in range(4)]
    _check(fn(ctypes.byref(shape.c()), *[ctypes.byref(x) for x in o]))
    return tuple(x.value for x in o)


def _mode(mode, causal, inputs=None, bf16_o=False, blob=None):
    """The mode argument: mode | causal flag | input storage flag (inputs: the torch dtype
    of q, k, v, d; float32 needs no flag) | bf16 O flag | blob flag (blob: the torch
    dtype of the result blob; float32 needs no flag)."""
    import torch
    flag = {torch.bfloat16: FAB_BF16_INPUTS, torch.float16: FAB_F16_INPUTS}.get(inputs, 0) if inputs is not None else 0
    bflag = {torch.bfloat16: FAB_BF16_BLOB, torch.float16: FAB_F16_BLOB}.get(blob, 0) if blob is not None else 0
    return MODES[mode] | (FAB_CAUSAL if causal else 0) | flag | (FAB_BF16_O if bf16_o else 0) | bflag


def workspace_bytes(shape: Shape, mode="f32", has_mask=False, have_o_lse=False, causal=False) -> int:
    n = ctypes.c_size_t()
    _check(lib().fab_workspace_bytes(ctypes.byref(shape.c()), _mode(mode, causal), int(bool(has_mask)),
                                     int(bool(have_o_lse)), ctypes.byref(n)))
    return n.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _mask_arg(mask):
    if mask is None:
        return None
    import torch
    if mask.dtype == torch.float16:
        mask = mask.view(torch.int16)
    if mask.dtype not in (torch.int16, torch.uint16):
        raise TypeError("mask must hold f16 bit patterns (float16, int16 or uint16)")
    return mask


def _input_dtype(*ts):
    """float32, bfloat16 or float16, the same for every input tensor."""
    import torch
    dt = ts[0].dtype
    if dt not in (torch.float32, torch.bfloat16, torch.float16) or any(t.dtype != dt for t in ts):
        raise TypeError("q, k, v (and d) must all be float32, all bfloat16 or all float16, got "
                        + ", ".join(str(t.dtype) for t in ts))
    return dt


def _check_tensor(t, name, shape, dtypes=None):
    """dtype, shape and contiguity of one tensor argument (the C ABI cannot check them:
    it receives a bare pointer and reads or writes exactly the extent the shape implies)."""
    import torch
    dtypes = dtypes or (torch.float32,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(x) for x in dtypes)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_devices(device, **tensors):
    """Every given tensor on the one GPU device the call runs on."""
    if device.type != "cuda":
        raise ValueError(f"the tensors must be on a GPU device, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_mask(mask, s):
    mask = _mask_arg(mask)
    if mask is not None:
        import torch
        _check_tensor(mask, "mask", (s.N, s.M), (torch.int16, torch.uint16))
    return mask


def _check_alibi(alibi, s):
    """Per-query-head ALiBi slopes: float32 (H,), contiguous, or None."""
    if alibi is not None:
        _check_tensor(alibi, "alibi", (s.H,))
    return alibi


def _check_ws(ws, need):
    """A caller's workspace: contiguous, at least `need` bytes; returns its byte size."""
    if not ws.is_contiguous():
        raise ValueError("ws must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"ws has {nbytes} bytes, {need} needed")
    return nbytes


def alloc_workspace(shape: Shape, mode, has_mask, have_o_lse, device, causal=False):
    import torch
    n = workspace_bytes(shape, mode, has_mask, have_o_lse, causal)
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device), n


def _on_stream(stream):
    """Context in which the call's own buffers are allocated: the stream its kernels
    run on, so that the caching allocator does not hand them to other work while those
    kernels may still use them."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def forward_lse(q, k, v, scale, mask=None, mode="f32", O=None, lse=None, ws=None, stream=None, causal=False,
                alibi=None, o_bf16=False):
    """O (B,N,H,DV) and the natural-log row LSE (B,H,N) of softmax(scale*q.k + mask) v.
    causal=True applies the causal rule without a mask (mask must be None).  q, k, v
    are float32, or bfloat16 or float16 (all three; mode "bf16").  alibi: float32 (H,) per-head
    slopes, adding alibi[h] * (m - n) to the score of query n at key m, or None.  O is
    float32, or bfloat16 (mode "bf16": a given bfloat16 O, or o_bf16=True)."""
    import torch
    s = shape_of(q, k, v)
    dev = q.device
    in_dt = _input_dtype(q, k, v)
    _check_tensor(q, "q", (s.B, s.H, s.N, s.DK), (q.dtype,))
    _check_tensor(k, "k", (s.B, s.Hkv, s.M, s.DK), (q.dtype,))
    _check_tensor(v, "v", (s.B, s.Hkv, s.M, s.DV), (q.dtype,))
    mask = _check_mask(mask, s)
    alibi = _check_alibi(alibi, s)
    if O is not None:
        _check_tensor(O, "O", (s.B, s.N, s.H, s.DV), (torch.float32, torch.bfloat16))
        o_bf16 = O.dtype == torch.bfloat16
    if lse is not None:
        _check_tensor(lse, "lse", (s.B, s.H, s.N))
    if ws is not None:
        nbytes = _check_ws(ws, workspace_bytes(s, mode, mask is not None, True, causal))
    _check_devices(dev, k=k, v=v, mask=mask, alibi=alibi, O=O, lse=lse, ws=ws)
    with _on_stream(stream):
        if O is None:
            O = torch.empty((s.B, s.N, s.H, s.DV), dtype=torch.bfloat16 if o_bf16 else torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((s.B, s.H, s.N), dtype=torch.float32, device=dev)
        if ws is None:
            ws, nbytes = alloc_workspace(s, mode, mask is not None, True, dev, causal)
        _check(lib().fab_forward_lse_alibi(ctypes.byref(s.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(alibi),
                                           float(scale), _mode(mode, causal, in_dt, o_bf16), _ptr(O), _ptr(lse),
                                           _ptr(ws), nbytes, _stream_handle(stream)))
    return O, lse


def backward(q, k, v, d, scale, mask=None, mode="f32", O=None, lse=None, blob=None, ws=None,
             stream=None, causal=False, alibi=None, blob_dtype=None):
    """The packed blob [dQ | pad | dK | pad | dV | pad] of d sum(d * attn) / d(q, k, v):
    float32, or (mode "bf16") bfloat16 / float16 elements rounded from the f32 result --
    the dtype of a given blob, else blob_dtype (default float32).
    causal=True applies the causal rule without a mask (mask must be None).  q, k, v, d
    are float32, or bfloat16 or float16 (all four; mode "bf16").  O (B,N,H,DV) and lse (B,H,N),
    (float32, or bfloat16 as forward_lse wrote it) are both given (from forward_lse,
    with the same alibi) or both None.
    alibi: float32 (H,) per-head ALiBi slopes or None (see forward_lse)."""
    import torch
    s = shape_of(q, k, v)
    dev = q.device
    in_dt = _input_dtype(q, k, v, d)
    _check_tensor(q, "q", (s.B, s.H, s.N, s.DK), (q.dtype,))
    _check_tensor(k, "k", (s.B, s.Hkv, s.M, s.DK), (q.dtype,))
    _check_tensor(v, "v", (s.B, s.Hkv, s.M, s.DV), (q.dtype,))
    _check_tensor(d, "d", (s.B, s.N, s.H, s.DV), (q.dtype,))
    mask = _check_mask(mask, s)
    alibi = _check_alibi(alibi, s)
    if (O is None) != (lse is None):
        raise ValueError("O and lse must be given together or both be None")
    o_bf16 = False
    if O is not None:
        _check_tensor(O, "O", (s.B, s.N, s.H, s.DV), (torch.float32, torch.bfloat16))
        _check_tensor(lse, "lse", (s.B, s.H, s.N))
        o_bf16 = O.dtype == torch.bfloat16
    if blob is not None and blob_dtype is not None and blob.dtype != blob_dtype:
        raise TypeError(f"blob is {blob.dtype} but blob_dtype is {blob_dtype}")
    bdt = blob.dtype if blob is not None else (blob_dtype or torch.float32)
    total = blob_layout(s, bdt)[3]
    if blob is not None:
        _check_tensor(blob, "blob", None, _blob_dtypes())
        if blob.numel() < total:
            raise ValueError(f"blob has {blob.numel()} elements, {total} needed")
    if ws is not None:
        nbytes = _check_ws(ws, workspace_bytes(s, mode, mask is not None, O is not None, causal))
    _check_devices(dev, k=k, v=v, d=d, mask=mask, alibi=alibi, O=O, lse=lse, blob=blob, ws=ws)
    with _on_stream(stream):
        if blob is None:
            blob = torch.empty(max(total, 8), dtype=bdt, device=dev)
        if ws is None:
            ws, nbytes = alloc_workspace(s, mode, mask is not None, O is not None, dev, causal)
        _check(lib().fab_backward_alibi(ctypes.byref(s.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(alibi),
                                        _ptr(d), float(scale), _mode(mode, causal, in_dt, o_bf16, bdt), _ptr(O),
                                        _ptr(lse), _ptr(blob), _ptr(ws), nbytes, _stream_handle(stream)))
    return blob


NOALLOC_SCRATCH_BYTES = 64 << 20   # FAB_NOALLOC_SCRATCH_BYTES of include/fab.h


def backward_noalloc(q, k, v, d, scale, blob, mask=None, mode="f32", O=None, lse=None, stream=None,
                     causal=False):
    """backward() through fab_backward_noalloc: the library's fixed scratch array serves
    as the workspace, so the call allocates nothing; the caller passes the blob (float32,
    or in mode "bf16" bfloat16 / float16, at least blob_layout(shape, blob.dtype)[3]
    elements).  Shapes needing more than NOALLOC_SCRATCH_BYTES
    of workspace raise FabError (FAB_E_UNSUPPORTED)."""
    import torch
    s = shape_of(q, k, v)
    dev = q.device
    in_dt = _input_dtype(q, k, v, d)
    _check_tensor(q, "q", (s.B, s.H, s.N, s.DK), (q.dtype,))
    _check_tensor(k, "k", (s.B, s.Hkv, s.M, s.DK), (q.dtype,))
    _check_tensor(v, "v", (s.B, s.Hkv, s.M, s.DV), (q.dtype,))
    _check_tensor(d, "d", (s.B, s.N, s.H, s.DV), (q.dtype,))
    mask = _check_mask(mask, s)
    if (O is None) != (lse is None):
        raise ValueError("O and lse must be given together or both be None")
    if O is not None:
        _check_tensor(O, "O", (s.B, s.N, s.H, s.DV))
        _check_tensor(lse, "lse", (s.B, s.H, s.N))
    _check_tensor(blob, "blob", None, _blob_dtypes())
    total = blob_layout(s, blob.dtype)[3]
    if blob.numel() < total:
        raise ValueError(f"blob has {blob.numel()} elements, {total} needed")
    _check_devices(dev, k=k, v=v, d=d, mask=mask, O=O, lse=lse, blob=blob)
    _check(lib().fab_backward_noalloc(ctypes.byref(s.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(d),
                                      float(scale), _mode(mode, causal, in_dt, blob=blob.dtype), _ptr(O), _ptr(lse), _ptr(blob),
                                      _stream_handle(stream)))
    return blob


def unpack(blob, shape: Shape):
    """Views dq (B,H,N,DK), dk (B,Hkv,M,DK), dv (B,Hkv,M,DV) into the blob at the padded
    offsets of its dtype."""
    s = shape
    _, off_k, off_v, _ = blob_layout(s, blob.dtype)
    nq, nk, nv = s.DK * s.N * s.H * s.B, s.DK * s.M * s.Hkv * s.B, s.DV * s.M * s.Hkv * s.B
    dq = blob[0:nq].view(s.B, s.H, s.N, s.DK)
    dk = blob[off_k:off_k + nk].view(s.B, s.Hkv, s.M, s.DK)
    dv = blob[off_v:off_v + nv].view(s.B, s.Hkv, s.M, s.DV)
    return dq, dk, dv


def profile_enable(on=True):
    """Bracket every kernel launch with HIP events (measurement only)."""
    _check(lib().fab_profile_enable(int(bool(on))))


def profile_reset():
    _check(lib().fab_profile_reset())


def profile_read():
    """{kernel: (total_ms, launches)} since the last reset (waits for the events)."""
    out = {}
    for name in KERNELS:
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        _check(lib().fab_profile_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)))
        out[name] = (ms.value, n.value)
    return out


def measure_mfma_loop(iters=20000, device=None):
    """(TFLOP/s, shader GHz) of a loop of dense bf16 32x32x16 products on every SIMD:
    the practical ceiling of the matrix cores on this GPU (measurement only)."""
    import torch
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    n = lib().fab_probe_scratch_bytes()
    scratch = torch.empty(n, dtype=torch.uint8, device=dev)
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(lib().fab_measure_mfma_loop(ctypes.c_void_p(scratch.data_ptr()), n, int(iters), ctypes.byref(tf),
                                           ctypes.byref(ghz), ctypes.c_void_p(stream)))
    return tf.value, ghz.value
