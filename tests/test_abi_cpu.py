"""CPU-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol include/fab.h declares, computes the blob layout of "Function
ggml_flash_attn_back" / the ggmlR unpacker, and rejects bad arguments before any
device work (the ggmlR test file's principle that unsupported input must be
refused rather than answered wrongly)."""
import ctypes
import math
import os
import re

import pytest
import torch

import exact_attention_backward_fab_amd as fab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "fab.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fab_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = fab.lib()
    declared = header_functions()
    assert set(declared) == set(fab.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.fab_version() == 100


def test_strerror_covers_every_status():
    L = fab.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.fab_strerror(code).decode() not in ("", "unknown status")
    assert L.fab_strerror(-99).decode() == "unknown status"


def _ds_bytes(s):
    # bf16 dS of every (query, key) pair, both extents rounded up to 128
    return 2 * s.B * s.H * (-(-s.N // 128) * 128) * (-(-s.M // 128) * 128)


def test_bf16_workspace_holds_ds_within_its_limit():
    """bf16 mode with head dims up to 128 keeps the bf16 dS tiles in the backward's
    workspace while they fit 4 GiB (every head-dim pair); f32 mode and larger shapes
    compute dQ without them (the header's statement of fab_workspace_bytes)."""
    s = fab.Shape(1, 16, 4, 8192, 8192, 128, 128)
    bf, f32 = fab.workspace_bytes(s, "bf16", False, True), fab.workspace_bytes(s, "f32", False, True)
    assert bf >= _ds_bytes(s) > f32
    # odd extents: one query step and a partial key block still take whole 128 x 128 blocks
    small = fab.Shape(1, 2, 1, 37, 29, 3, 5)
    assert fab.workspace_bytes(small, "bf16", False, True) >= _ds_bytes(small)
    # 192-wide heads: the tiles too
    wide = fab.Shape(1, 8, 8, 4096, 4096, 192, 128)
    assert fab.workspace_bytes(wide, "bf16", False, True) >= _ds_bytes(wide)
    # past 4 GiB of tiles: recompute
    big = fab.Shape(1, 40, 8, 8192, 8192, 128, 128)
    assert _ds_bytes(big) > 4 << 30
    assert fab.workspace_bytes(big, "bf16", False, True) < _ds_bytes(big)
    # exactly 4 GiB of tiles in one row of 131072 key blocks (a buffer resource covers
    # below 2^32 bytes): recompute
    edge = fab.Shape(1, 1, 1, 127, (1 << 24) - 64, 32, 32)
    assert _ds_bytes(edge) == 4 << 30
    assert fab.workspace_bytes(edge, "bf16", False, True) < 4 << 30


@pytest.mark.parametrize("shape", [
    fab.Shape(2, 4, 2, 2, 4, 3, 5), fab.Shape(1, 2, 1, 3, 5, 3, 5), fab.Shape(1, 1, 1, 1, 1, 1, 1),
    fab.Shape(1, 32, 8, 2048, 2048, 128, 128), fab.Shape(4, 16, 16, 512, 4096, 192, 128),
    fab.Shape(0, 2, 1, 3, 5, 3, 5), fab.Shape(1, 2, 1, 0, 5, 3, 5)])
def test_blob_layout_matches_the_pages_padding(shape):
    s = shape
    nq, nk, nv = s.DK * s.N * s.H * s.B, s.DK * s.M * s.Hkv * s.B, s.DV * s.M * s.Hkv * s.B
    pad = lambda n: int(math.ceil(n * 4 / 16) * 16 / 4)
    assert fab.blob_layout(s) == (0, pad(nq), pad(nq) + pad(nk), pad(nq) + pad(nk) + pad(nv))


@pytest.mark.parametrize("shape", [
    fab.Shape(2, 4, 2, 2, 4, 3, 5), fab.Shape(1, 2, 1, 3, 5, 3, 5), fab.Shape(1, 1, 1, 1, 1, 1, 1),
    fab.Shape(1, 32, 8, 2048, 2048, 128, 128), fab.Shape(1, 3, 3, 7, 9, 5, 3),
    fab.Shape(0, 2, 1, 3, 5, 3, 5), fab.Shape(1, 2, 1, 0, 5, 3, 5)])
def test_blob_layout16_pads_each_slice_to_16_bytes(shape):
    """A 16-bit blob keeps the [dQ | pad | dK | pad | dV | pad] order with each slice
    padded to 16 bytes = 8 elements."""
    s = shape
    nq, nk, nv = s.DK * s.N * s.H * s.B, s.DK * s.M * s.Hkv * s.B, s.DV * s.M * s.Hkv * s.B
    pad8 = lambda n: -(-n // 8) * 8
    want = (0, pad8(nq), pad8(nq) + pad8(nk), pad8(nq) + pad8(nk) + pad8(nv))
    assert fab.blob_layout(s, torch.bfloat16) == want
    assert fab.blob_layout(s, torch.float16) == want
    assert fab.blob_layout(s, torch.float32) == fab.blob_layout(s)
    o = [ctypes.c_int64() for _ in range(4)]
    assert fab.lib().fab_blob_layout16(ctypes.byref(s.c()), *[ctypes.byref(x) for x in o]) == fab.FAB_OK
    assert tuple(x.value for x in o) == want
    with pytest.raises(TypeError):
        fab.blob_layout(s, torch.int32)


def test_blob_flags_change_no_workspace_and_stay_out_of_the_forward():
    s = fab.Shape(1, 8, 2, 300, 400, 64, 64)
    L = fab.lib()
    for has_mask in (0, 1):
        for have in (0, 1):
            base = fab.workspace_bytes(s, "bf16", has_mask, have)
            for flag in (fab.FAB_BF16_BLOB, fab.FAB_F16_BLOB):
                n = ctypes.c_size_t()
                assert L.fab_workspace_bytes(ctypes.byref(s.c()), fab.FAB_MODE_BF16 | flag, has_mask, have,
                                             ctypes.byref(n)) == fab.FAB_OK
                assert n.value == base
    n = ctypes.c_size_t()
    assert L.fab_workspace_bytes(ctypes.byref(s.c()), fab.FAB_MODE_F32 | fab.FAB_BF16_BLOB, 0, 0,
                                 ctypes.byref(n)) == fab.FAB_E_INVAL
    P = ctypes.c_void_p
    sh = fab.FabShape(*GOOD)
    for flag in (fab.FAB_BF16_BLOB, fab.FAB_F16_BLOB):
        rc = L.fab_forward_lse(ctypes.byref(sh), P(FAKE), P(FAKE), P(FAKE), None, 0.5, fab.FAB_MODE_BF16 | flag,
                               P(FAKE), P(FAKE), P(FAKE), 1 << 40, None)
        assert rc == fab.FAB_E_INVAL and "backward" in L.fab_last_error().decode()


def test_workspace_grows_with_what_must_be_recomputed():
    s = fab.Shape(1, 8, 2, 300, 400, 64, 64)
    base = fab.workspace_bytes(s, "bf16", False, True)
    assert fab.workspace_bytes(s, "bf16", True, True) > base      # mask block map
    # bf16: the backward's own forward writes the tiles the backward reads, no O;
    # f32: the internal O and LSE need room
    assert fab.workspace_bytes(s, "bf16", False, False) == base
    assert fab.workspace_bytes(s, "f32", False, False) > fab.workspace_bytes(s, "f32", False, True)
    # with a grid of at least one dK/dV work-group per CU: partials only for grouped-query
    # heads; on smaller grids the query splits of the dK/dV kernel have partials too
    big = fab.Shape(1, 8, 2, 300, 4096, 64, 64)
    big_mha = fab.Shape(1, 8, 8, 300, 4096, 64, 64)
    assert fab.workspace_bytes(big_mha, "bf16", False, True) < fab.workspace_bytes(big, "bf16", False, True)
    small_mha = fab.Shape(1, 8, 8, 300, 400, 64, 64)
    partials = 2 * 4 * 64 * 400 * 8 * 4   # dK and dV, f32, 4 query splits of 8 heads
    assert fab.workspace_bytes(small_mha, "bf16", False, True) >= partials


FAKE = 1 << 20   # a 256-byte aligned address that is never dereferenced: every call below fails validation


def call_bwd(shape, q=FAKE, k=FAKE, v=FAKE, mask=None, d=FAKE, scale=0.5, mode=0, O=None, lse=None,
             blob=FAKE, ws=FAKE, ws_bytes=1 << 40):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    L = fab.lib()
    return L.fab_backward(ctypes.byref(fab.FabShape(*shape)), P(q), P(k), P(v), P(mask), P(d),
                          float(scale), mode, P(O), P(lse), P(blob), P(ws), ws_bytes, None)


GOOD = (1, 4, 2, 8, 8, 16, 16)


@pytest.mark.parametrize("shape,kw,code", [
    ((1, 3, 2, 8, 8, 16, 16), {}, fab.FAB_E_INVAL),          # H % Hkv != 0
    ((1, 4, 2, -1, 8, 16, 16), {}, fab.FAB_E_INVAL),         # negative N
    ((1, 0, 1, 8, 8, 16, 16), {}, fab.FAB_E_INVAL),          # no heads
    ((1, 4, 2, 8, 8, 0, 16), {}, fab.FAB_E_INVAL),           # DK = 0
    ((1, 4, 2, 8, 8, 257, 16), {}, fab.FAB_E_UNSUPPORTED),   # head dim above the kernels' range (256)
    ((1, 4, 2, 8, 8, 16, 257), {}, fab.FAB_E_UNSUPPORTED),
    ((1 << 20, 64, 64, 1024, 1024, 128, 128), {}, fab.FAB_E_UNSUPPORTED),  # beyond 2^31 elements
    ((1, 1, 1, 8, 5_700_000, 192, 32), {}, fab.FAB_E_UNSUPPORTED),  # one head's tiles beyond 2 GiB
    (GOOD, {"mode": 7}, fab.FAB_E_INVAL),
    (GOOD, {"scale": float("nan")}, fab.FAB_E_INVAL),
    (GOOD, {"scale": float("inf")}, fab.FAB_E_INVAL),
    (GOOD, {"q": None}, fab.FAB_E_INVAL),
    (GOOD, {"d": None}, fab.FAB_E_INVAL),
    (GOOD, {"blob": None}, fab.FAB_E_INVAL),
    (GOOD, {"O": FAKE}, fab.FAB_E_INVAL),                    # O without lse
    (GOOD, {"lse": FAKE}, fab.FAB_E_INVAL),                  # lse without O
    (GOOD, {"k": FAKE + 4}, fab.FAB_E_ALIGN),
    (GOOD, {"mask": FAKE + 2}, fab.FAB_E_ALIGN),
    (GOOD, {"ws": FAKE + 16}, fab.FAB_E_ALIGN),
    (GOOD, {"ws": None}, fab.FAB_E_WORKSPACE),
    (GOOD, {"ws_bytes": 16}, fab.FAB_E_WORKSPACE),
    (GOOD, {"mode": fab.FAB_CAUSAL, "mask": FAKE}, fab.FAB_E_INVAL),         # mask and causal flag
    (GOOD, {"mode": fab.FAB_MODE_BF16 | 0x4000}, fab.FAB_E_INVAL),          # unknown flag bit
    (GOOD, {"mode": fab.FAB_MODE_F32 | fab.FAB_BF16_BLOB}, fab.FAB_E_INVAL),   # 16-bit blob needs bf16 mode
    (GOOD, {"mode": fab.FAB_MODE_F32 | fab.FAB_F16_BLOB}, fab.FAB_E_INVAL),
    (GOOD, {"mode": fab.FAB_MODE_BF16 | fab.FAB_BF16_BLOB | fab.FAB_F16_BLOB}, fab.FAB_E_INVAL),  # one blob type
    (GOOD, {"mode": fab.FAB_MODE_BF16 | fab.FAB_F16_BLOB, "blob": FAKE + 8}, fab.FAB_E_ALIGN),  # 16-byte aligned
    (GOOD, {"mode": fab.FAB_MODE_F32 | fab.FAB_F16_INPUTS}, fab.FAB_E_INVAL),   # f16 inputs need bf16 mode
    (GOOD, {"mode": fab.FAB_MODE_BF16 | fab.FAB_F16_INPUTS | fab.FAB_BF16_INPUTS}, fab.FAB_E_INVAL),  # one input storage
    (GOOD, {"mode": fab.FAB_MODE_F32 | fab.FAB_BF16_O, "O": FAKE, "lse": FAKE}, fab.FAB_E_INVAL),  # bf16 O needs bf16 mode
    (GOOD, {"mode": fab.FAB_MODE_F32 | fab.FAB_BF16_INPUTS}, fab.FAB_E_INVAL),  # bf16 inputs need bf16 mode
])
def test_backward_rejects_bad_arguments_before_device_work(shape, kw, code):
    assert call_bwd(shape, **kw) == code
    assert fab.lib().fab_last_error().decode() != ""


def test_causal_flag_workspace():
    # the causal flag needs no block map: the same workspace as no mask; with a
    # mask it is rejected
    s = fab.Shape(1, 8, 2, 300, 400, 64, 64)
    for mode in ("f32", "bf16"):
        assert fab.workspace_bytes(s, mode, False, False, causal=True) == fab.workspace_bytes(s, mode, False, False)
        assert fab.workspace_bytes(s, mode, True, False) > fab.workspace_bytes(s, mode, False, False, causal=True)
    with pytest.raises(fab.FabError) as e:
        fab.workspace_bytes(s, "bf16", True, False, causal=True)
    assert e.value.code == fab.FAB_E_INVAL


def test_forward_rejects_bad_arguments():
    L = fab.lib()
    P = ctypes.c_void_p
    sh = fab.FabShape(1, 4, 2, 8, 8, 16, 16)
    rc = L.fab_forward_lse(ctypes.byref(sh), P(FAKE), P(FAKE), P(FAKE), None, 0.5, 0, None, P(FAKE),
                           P(FAKE), 1 << 30, None)
    assert rc == fab.FAB_E_INVAL   # O is NULL
    rc = L.fab_forward_lse(ctypes.byref(sh), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 0.5, 0, P(FAKE),
                           P(FAKE), None, 0, None)
    assert rc == fab.FAB_E_WORKSPACE   # a mask needs its block map workspace
    assert L.fab_blob_layout(None, None, None, None, None) == fab.FAB_E_INVAL


def test_noalloc_rejects_before_device_work():
    """fab_backward_noalloc checks the shape, the mode and its fixed scratch size on the
    host before any HIP call (here, without a GPU, it must return the error code)."""
    L = fab.lib()
    P = ctypes.c_void_p
    big = fab.FabShape(1, 32, 8, 2048, 2048, 128, 128)   # ~370 MB of bf16 workspace
    rc = L.fab_backward_noalloc(ctypes.byref(big), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), 0.1,
                                fab.FAB_MODE_BF16 | fab.FAB_CAUSAL, P(FAKE), P(FAKE), P(FAKE), None)
    assert rc == fab.FAB_E_UNSUPPORTED
    assert "scratch" in L.fab_last_error().decode()
    bad = fab.FabShape(1, 3, 2, 8, 8, 16, 16)              # H % Hkv != 0
    rc = L.fab_backward_noalloc(ctypes.byref(bad), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), 0.1, 0, None, None,
                                P(FAKE), None)
    assert rc == fab.FAB_E_INVAL
    assert fab.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_alibi_entry_points_reject_a_misaligned_slope_array():
    L = fab.lib()
    P = ctypes.c_void_p
    sh = fab.FabShape(*GOOD)
    rc = L.fab_backward_alibi(ctypes.byref(sh), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE + 2), P(FAKE), 0.5, 0,
                              None, None, P(FAKE), P(FAKE), 1 << 40, None)
    assert rc == fab.FAB_E_ALIGN and "alibi" in L.fab_last_error().decode()
    rc = L.fab_forward_lse_alibi(ctypes.byref(sh), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE + 1), 0.5, 0, P(FAKE),
                                 P(FAKE), P(FAKE), 1 << 40, None)
    assert rc == fab.FAB_E_ALIGN


def test_mfma_probe_rejects_bad_arguments_before_device_work():
    L = fab.lib()
    P = ctypes.c_void_p
    n = L.fab_probe_scratch_bytes()
    assert n >= 2048 * 512 * 4
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    assert L.fab_measure_mfma_loop(None, n, 10, ctypes.byref(tf), ctypes.byref(ghz), None) == fab.FAB_E_INVAL
    assert L.fab_measure_mfma_loop(P(FAKE), n - 1, 10, ctypes.byref(tf), ctypes.byref(ghz), None) == fab.FAB_E_INVAL
    assert "scratch" in L.fab_last_error().decode()
    assert L.fab_measure_mfma_loop(P(FAKE), n, 0, ctypes.byref(tf), ctypes.byref(ghz), None) == fab.FAB_E_INVAL
