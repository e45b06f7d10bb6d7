"""GPU parity: the HIP path (through the C ABI) against the f64 CPU oracle.

Bar, per gradient tensor over the unpadded slice: max|gpu - oracle| / max|oracle|
<= 1e-4 in f32 mode and <= 2e-2 in bf16 mode; blob pads exactly 0; no NaN/inf;
the exact-zero sets (all-masked query rows, keys no query attends to) exactly 0.
Small problems are compared element by element against the full oracle; the
five workloads at full size are compared on sampled rows and keys the oracle
computes one by one, and through sums that hold at any size.
"""
import math
import time

import numpy as np
import pytest

import fab_inputs as fi
from fab_inputs import Shape, make_qkvd, random_mask, causal_mask, padding64_mask, F16_NEG_INF

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    return torch, torch.device("cuda:0")


def fabmod():
    import exact_attention_backward_fab_amd as fab
    fab.lib()
    return fab


def to_dev(torch, dev, a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def rel_err(got, ref, den=None):
    """max|got - ref| / max|ref|; den overrides the denominator (used when ref is
    identically zero by cancellation, e.g. a single key, where a relative error is
    undefined and the scale of the other gradients is used instead)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den is None:
        den = np.max(np.abs(ref)) if ref.size else 0.0
    return err / den if den > 0 else err


def structural_zeros(s, mask):
    """Boolean masks of the entries that are zero by structure, not by cancellation:
    dQ rows of all-masked query rows (every score -inf), and dK/dV rows of keys
    that no query attends to."""
    dead_rows = np.zeros(s.N, bool)
    dead_keys = np.zeros(s.M, bool) if s.N > 0 else np.ones(s.M, bool)
    if mask is not None and s.N > 0 and s.M > 0:
        inf = mask == F16_NEG_INF
        dead_rows = inf.all(axis=1)
        dead_keys = inf.all(axis=0)
    return dead_rows, dead_keys


def run_gpu(torch, dev, s, q, k, v, d, mask, scale, mode, with_o_lse=False):
    fab = fabmod()
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    tm = to_dev(torch, dev, mask)
    fs = fab.Shape(*s.astuple())
    O = lse = None
    if with_o_lse:
        O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode=mode)
    total = fab.blob_layout(fs)[3]
    blob = torch.full((total + 64,), float("nan"), dtype=torch.float32, device=dev)  # guard band after
    fab.backward(t[0], t[1], t[2], t[3], scale, mask=tm, mode=mode, O=O, lse=lse, blob=blob[:total]
                 if total else blob[:4])
    torch.cuda.synchronize()
    out = blob.cpu().numpy()
    assert np.all(np.isnan(out[total:])), "write past the end of the blob"
    return out[:total]


def check_blob(s, blob, ref, mode, tag="", mask=None):
    """ref: dict with dq, dk, dv (oracle, f64)."""
    fab = fabmod()
    _, off_k, off_v, total = fab.blob_layout(fab.Shape(*s.astuple()))
    nq, nk, nv = ref["dq"].size, ref["dk"].size, ref["dv"].size
    assert np.all(np.isfinite(blob)), f"{tag}: non-finite values in the blob"
    assert np.all(blob[nq:off_k] == 0) and np.all(blob[off_k + nk:off_v] == 0) and \
        np.all(blob[off_v + nv:total] == 0), f"{tag}: pads not zero"
    scale_all = max(float(np.max(np.abs(ref[n]))) if ref[n].size else 0.0 for n in ("dq", "dk", "dv"))
    dead_rows, dead_keys = structural_zeros(s, mask)
    errs = {}
    for name, lo, n in (("dq", 0, nq), ("dk", off_k, nk), ("dv", off_v, nv)):
        got = blob[lo:lo + n].reshape(ref[name].shape)
        den = None if (ref[name].size and np.max(np.abs(ref[name])) > 0) else scale_all
        errs[name] = rel_err(got, ref[name], den)
        # zeros by structure are exact zeros in the GPU result too
        z = got[:, :, dead_rows, :] if name == "dq" else got[:, :, dead_keys, :]
        assert np.all(z == 0), f"{tag}: {name} non-zero where it is zero by structure"
        assert np.all(ref[name][:, :, dead_rows if name == "dq" else dead_keys, :] == 0)
    for name, e in errs.items():
        assert e <= TOL[mode], f"{tag}: {name} max-rel error {e:.3e} > {TOL[mode]} ({errs})"
    return errs


def oracle_full(s, q, k, v, d, mask, scale):
    from oracle import oracle as orc
    return orc.backward(s, q, k, v, mask, d, scale)


# ---------------------------------------------------------------- small, full oracle

SMALL = [
    # name, shape, mask kind, seed
    ("p3_single_head", Shape(1, 1, 1, 3, 5, 4, 4), None, 11),
    ("p3_causal", Shape(1, 1, 1, 3, 4, 4, 4), "causal", 12),
    ("p3_gqa_batch", Shape(2, 4, 2, 2, 3, 4, 4), None, 13),
    ("p3_packing", Shape(2, 4, 2, 2, 4, 3, 5), None, 31),
    ("odd_pad_mask", Shape(1, 2, 1, 37, 29, 3, 5), "random", 41),
    ("ragged_d64_random", Shape(2, 4, 2, 200, 300, 64, 64), "random", 42),
    ("ragged_d128_causal_gqa", Shape(1, 4, 1, 333, 333, 128, 128), "causal", 43),
    ("d192_128_padding", Shape(1, 2, 2, 130, 260, 192, 128), "padding", 44),
    ("d40_72_nomask", Shape(1, 3, 1, 70, 90, 40, 72), None, 45),
    ("d192_192_random", Shape(1, 2, 1, 65, 97, 192, 192), "random", 46),
    # M % 8 == 0: the 4-wave kernel copies each step's mask rows into LDS (rows past
    # N=100 read as zero, the last key block runs past M)
    ("d192_128_random_staged_mask", Shape(1, 2, 2, 100, 264, 192, 128), "random", 50),
    # 256-wide heads (the pair 256 / 256): the 4-wave dK/dV kernel splits the dK/dV
    # columns over two work-groups, each forming the whole S and dP; the f32 kernel
    # runs one 32-key sub-block per work-group
    ("d256_random_gqa", Shape(1, 4, 2, 100, 264, 256, 256), "random", 55),
    ("d200_256_causal_batch", Shape(2, 2, 1, 130, 130, 200, 256), "causal", 56),
    ("d64_256_padding", Shape(1, 2, 2, 70, 300, 64, 256), "padding", 57),
    ("one_key", Shape(1, 2, 1, 17, 1, 16, 16), None, 47),
    ("one_query", Shape(1, 2, 2, 1, 130, 64, 64), "random", 48),
    ("workload1", fi.WORKLOADS[1].shape, None, 1),
    # 192-wide heads with many (batch, head, query-step) blocks: the 4-wave dK/dV
    # kernel (mask rows staged in LDS, M % 8 == 0) and dQ from its stored dS
    ("d192_528_query_blocks", Shape(1, 33, 3, 2000, 200, 192, 128), "causal", 49),
    # 16 key blocks x 64 (batch, head) pairs = 1024 work-groups: the bf16 dK/dV kernel
    # takes two query heads of a group per work-group; with 2 heads per group a unit is
    # the whole group (dK/dV straight into the result), with 4 two partials per group
    ("two_heads_per_wg_group_of_2", Shape(4, 16, 8, 100, 2048, 64, 64), "random", 50),
    ("two_heads_per_wg_group_of_4", Shape(2, 32, 8, 70, 2048, 128, 128), None, 51),
    # 128 key blocks x 10 heads: two heads per work-group, 5 head units (not a multiple
    # of the 8 XCDs: the plain work-group order)
    ("two_heads_per_wg_5_units", Shape(1, 10, 5, 64, 16384, 64, 64), "random", 53),
    # two heads per work-group (64 key blocks x 16 heads = 1024) with a deep query loop:
    # each work-group walks 16 query steps of 64 for each of its two heads, so every dK/dV
    # element accumulates 2 x 1024 queries in registers before it is stored
    ("two_heads_per_wg_deep_query_loop", Shape(1, 16, 4, 1024, 8192, 64, 64), None, 54),
]


def small_mask(kind, s, seed):
    if kind is None:
        return None
    if kind == "causal":
        return causal_mask(s.N, s.M)
    if kind == "padding":
        m = np.zeros((s.N, s.M), np.uint16)
        m[:, (3 * s.M) // 4:] = F16_NEG_INF
        m[::7, :] = F16_NEG_INF
        return m
    return random_mask(s.N, s.M, seed, p_inf=0.3, full_rows=2, full_cols=3)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("name,s,mkind,seed", SMALL, ids=[c[0] for c in SMALL])
def test_small_against_full_oracle(torch_dev, name, s, mkind, seed, mode):
    torch, dev = torch_dev
    print(f"[parity] {name} {mode} {s}", flush=True)
    q, k, v, d = make_qkvd(s, seed)
    mask = small_mask(mkind, s, seed)
    scale = float(np.float32(1.0 / math.sqrt(s.DK)))
    ref = oracle_full(s, q, k, v, d, mask, scale)
    blob = run_gpu(torch, dev, s, q, k, v, d, mask, scale, mode)
    check_blob(s, blob, ref, mode, tag=f"{name}/{mode}", mask=mask)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_forward_output_and_lse(torch_dev, mode):
    torch, dev = torch_dev
    fab = fabmod()
    from oracle import oracle as orc
    s = Shape(2, 4, 2, 150, 170, 64, 96)
    q, k, v, _ = make_qkvd(s, 61)
    mask = random_mask(s.N, s.M, 61, p_inf=0.3, full_rows=2, full_cols=2)
    scale = 0.125
    O_ref, lse_ref = orc.forward(s, q, k, v, mask, scale)
    O, lse = fab.forward_lse(to_dev(torch, dev, q), to_dev(torch, dev, k), to_dev(torch, dev, v), scale,
                             mask=to_dev(torch, dev, mask), mode=mode)
    O, lse = O.cpu().numpy(), lse.cpu().numpy()
    assert rel_err(O, O_ref) <= TOL[mode]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse), ~fin)
    assert np.max(np.abs(lse[fin] - lse_ref[fin])) <= (1e-5 if mode == "f32" else 2e-2)
    dead = ~fin   # (B,H,N)
    for b in range(s.B):
        for h in range(s.H):
            assert np.all(O[b, dead[b, h], h, :] == 0)


def test_route_agreement_supplied_vs_recomputed_forward(torch_dev):
    # the ggmlR test's "two routes agree to 1e-5" check, for O/LSE supplied by the
    # caller vs recomputed inside the backward
    torch, dev = torch_dev
    s = Shape(1, 4, 2, 190, 210, 64, 64)
    q, k, v, d = make_qkvd(s, 71)
    mask = random_mask(s.N, s.M, 71, p_inf=0.2, full_rows=1, full_cols=1)
    a = run_gpu(torch, dev, s, q, k, v, d, mask, 0.125, "f32", with_o_lse=False)
    b = run_gpu(torch, dev, s, q, k, v, d, mask, 0.125, "f32", with_o_lse=True)
    assert rel_err(a, b) <= 1e-5


def test_bf16_repeat_is_bitwise_stable(torch_dev):
    # the same inputs and workspace three times: bf16 mode has no order-dependent
    # sums (dQ blocks split over two work-groups add their halves with a + b = b + a;
    # the split counters are re-zeroed on every call), so the blobs are identical
    torch, dev = torch_dev
    fab = fabmod()
    s = Shape(1, 8, 2, 700, 700, 128, 128)
    q, k, v, d = make_qkvd(s, 91)
    mask = causal_mask(s.N, s.M)
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    tm = to_dev(torch, dev, mask)
    fs = fab.Shape(*s.astuple())
    ws, _ = fab.alloc_workspace(fs, "bf16", True, False, dev)
    outs = []
    for _ in range(3):
        blob = fab.backward(t[0], t[1], t[2], t[3], 0.1, mask=tm, mode="bf16", ws=ws)
        torch.cuda.synchronize()
        outs.append(blob.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    ref = oracle_full(s, q, k, v, d, mask, 0.1)
    check_blob(s, outs[0], ref, "bf16", tag="repeat", mask=mask)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_autograd_grads_are_views_of_one_blob(torch_dev, mode):
    # [RT] "autodiff views address their own slice of the packed buffer": through
    # torch.autograd, the three gradients are views of one blob at its padded
    # offsets, and they match the oracle
    torch, dev = torch_dev
    fab = fabmod()
    from exact_attention_backward_fab_amd.autograd import attention
    s = Shape(2, 4, 2, 150, 170, 64, 48)
    q, k, v, d = make_qkvd(s, 101)
    mask = random_mask(s.N, s.M, 101, p_inf=0.3, full_rows=1, full_cols=1)
    scale = 0.125
    tq, tk, tv = [to_dev(torch, dev, x).requires_grad_(True) for x in (q, k, v)]
    O = attention(tq, tk, tv, mask=to_dev(torch, dev, mask), scale=scale, mode=mode)
    gq, gk, gv = torch.autograd.grad(O, (tq, tk, tv), grad_outputs=to_dev(torch, dev, d))
    base = gq.untyped_storage().data_ptr()
    assert gk.untyped_storage().data_ptr() == base and gv.untyped_storage().data_ptr() == base
    _, off_k, off_v, _ = fab.blob_layout(fab.Shape(*s.astuple()))
    assert (gq.storage_offset(), gk.storage_offset(), gv.storage_offset()) == (0, off_k, off_v)
    ref = oracle_full(s, q, k, v, d, mask, scale)
    for name, g in (("dq", gq), ("dk", gk), ("dv", gv)):
        assert rel_err(g.cpu().numpy(), ref[name]) <= TOL[mode], name


CAUSAL_FLAG = [
    ("square_gqa", Shape(1, 4, 2, 333, 333, 128, 128), 51),
    ("n_gt_m", Shape(2, 2, 1, 300, 130, 64, 64), 52),
    ("n_lt_m", Shape(1, 3, 3, 97, 260, 40, 72), 53),
    ("d192", Shape(1, 2, 1, 200, 200, 192, 128), 54),
]


@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("name,s,seed", CAUSAL_FLAG, ids=[c[0] for c in CAUSAL_FLAG])
def test_causal_flag_equals_causal_mask(torch_dev, name, s, seed, mode):
    # FAB_CAUSAL (no mask tensor, no block map) against the oracle on the explicit
    # 0 / -inf causal mask, and bit for bit against the library's own masked path
    # (f32 mode: dK and dV bit for bit, dQ up to the order of its atomics)
    torch, dev = torch_dev
    fab = fabmod()
    print(f"[parity] causal flag {name} {mode} {s}", flush=True)
    q, k, v, d = make_qkvd(s, seed)
    mask = causal_mask(s.N, s.M)
    scale = float(np.float32(1.0 / math.sqrt(s.DK)))
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    flag = fab.backward(*t, scale, mode=mode, causal=True)
    masked = fab.backward(*t, scale, mask=to_dev(torch, dev, mask), mode=mode)
    O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mode=mode, causal=True)
    torch.cuda.synchronize()
    flag = flag[:fab.blob_layout(fab.Shape(*s.astuple()))[3]].cpu().numpy()
    ref = oracle_full(s, q, k, v, d, mask, scale)
    check_blob(s, flag, ref, mode, tag=f"causal flag {name}/{mode}", mask=mask)
    masked = masked[:flag.size].cpu().numpy()
    if mode == "bf16":
        assert np.array_equal(flag.view(np.uint32), masked.view(np.uint32))
    else:   # f32 mode: dQ is summed by atomics in any order, dK and dV in a fixed one
        off_k = fab.blob_layout(fab.Shape(*s.astuple()))[1]
        assert np.abs(flag[:off_k] - masked[:off_k]).max() <= 1e-6 * np.abs(masked[:off_k]).max()
        assert np.array_equal(flag[off_k:].view(np.uint32), masked[off_k:].view(np.uint32))
    from oracle import oracle as orc
    O_ref, _ = orc.forward(s, q, k, v, mask, scale)
    assert rel_err(O.cpu().numpy(), O_ref) <= TOL[mode]


BF16_IN = [
    ("gqa_causal", Shape(1, 4, 2, 333, 333, 128, 128), "causal", 61),
    ("random_mask", Shape(2, 2, 1, 150, 170, 64, 64), "random", 62),
    ("d192_padding", Shape(1, 2, 2, 130, 260, 192, 128), "padding", 63),
    ("odd_dims", Shape(1, 3, 1, 70, 90, 40, 72), None, 64),
]


@pytest.mark.parametrize("store", ["bf16", "f16"])
@pytest.mark.parametrize("supplied", [False, True], ids=["own_forward", "o_lse_supplied"])
@pytest.mark.parametrize("name,s,mkind,seed", BF16_IN, ids=[c[0] for c in BF16_IN])
def test_16bit_inputs_equal_f32_inputs_of_the_same_values(torch_dev, name, s, mkind, seed, supplied, store):
    # FAB_BF16_INPUTS / FAB_F16_INPUTS: q, k, v, d stored as bf16 (the values bf16 mode
    # rounds to anyway) or as f16 (widened exactly, then rounded like f32 inputs) give
    # bit for bit the result of the f32 inputs holding the same values, and that
    # result matches the oracle on those values
    torch, dev = torch_dev
    fab = fabmod()
    print(f"[parity] {store} inputs {name} supplied={supplied} {s}", flush=True)
    q, k, v, d = make_qkvd(s, seed)
    mask = small_mask(mkind, s, seed)
    tm = to_dev(torch, dev, mask)
    scale = float(np.float32(1.0 / math.sqrt(s.DK)))
    dt16 = torch.bfloat16 if store == "bf16" else torch.float16
    t16 = [to_dev(torch, dev, x).to(dt16) for x in (q, k, v, d)]
    t32 = [x.float() for x in t16]
    outs = []
    for t in (t16, t32):
        O = lse = None
        if supplied:
            O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode="bf16")
        outs.append(fab.backward(*t, scale, mask=tm, mode="bf16", O=O, lse=lse))
        if supplied:
            outs.append(torch.cat([O.flatten(), lse.flatten()]))
    torch.cuda.synchronize()
    for a, b in zip(outs[:len(outs) // 2], outs[len(outs) // 2:]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    qr, kr, vr, dr = (x.cpu().numpy() for x in t32)
    ref = oracle_full(s, qr, kr, vr, dr, mask, scale)
    total = fab.blob_layout(fab.Shape(*s.astuple()))[3]
    check_blob(s, outs[0][:total].cpu().numpy(), ref, "bf16", tag=f"{store} inputs {name}", mask=mask)


@pytest.mark.parametrize("inputs16", [False, True], ids=["f32_inputs", "bf16_inputs"])
@pytest.mark.parametrize("name,s,mkind,seed", BF16_IN, ids=[c[0] for c in BF16_IN])
def test_bf16_o_equals_f32_o_of_the_same_values(torch_dev, name, s, mkind, seed, inputs16):
    # FAB_BF16_O: fab_forward_lse writes O as bf16 -- the f32 O rounded to nearest even,
    # bit for bit -- and fab_backward reading that bf16 O gives bit for bit the result of
    # the f32 O holding the same values; the result matches the oracle
    torch, dev = torch_dev
    fab = fabmod()
    print(f"[parity] bf16 O {name} inputs16={inputs16} {s}", flush=True)
    q, k, v, d = make_qkvd(s, seed)
    mask = small_mask(mkind, s, seed)
    tm = to_dev(torch, dev, mask)
    scale = float(np.float32(1.0 / math.sqrt(s.DK)))
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    if inputs16:
        t = [x.to(torch.bfloat16) for x in t]
    O32, lse32 = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode="bf16")
    O16, lse16 = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode="bf16", o_bf16=True)
    assert O16.dtype == torch.bfloat16
    assert torch.equal(O16.view(torch.int16), O32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(lse16.view(torch.int32), lse32.view(torch.int32))
    b16 = fab.backward(*t, scale, mask=tm, mode="bf16", O=O16, lse=lse16)
    b32 = fab.backward(*t, scale, mask=tm, mode="bf16", O=O16.float(), lse=lse16)
    torch.cuda.synchronize()
    assert torch.equal(b16.view(torch.int32), b32.view(torch.int32))
    qr, kr, vr, dr = (x.float().cpu().numpy() for x in t)
    ref = oracle_full(s, qr, kr, vr, dr, mask, scale)
    total = fab.blob_layout(fab.Shape(*s.astuple()))[3]
    check_blob(s, b16[:total].cpu().numpy(), ref, "bf16", tag=f"bf16 O {name}", mask=mask)


@pytest.mark.parametrize("supplied", [False, True], ids=["own_forward", "o_lse_supplied"])
@pytest.mark.parametrize("name,s,mkind,seed", [
    ("causal_d64", Shape(1, 4, 2, 333, 333, 64, 64), "causal", 61),
    ("random_d128", Shape(2, 2, 1, 200, 300, 128, 128), "random", 62),
], ids=["causal_d64", "random_d128"])
def test_bf16_stale_workspace_is_not_read(torch_dev, name, s, mkind, seed, supplied):
    """bf16 mode stores dS^T only for the (key block, query step) pairs the block
    map does not skip, and the dQ product reads only those: a workspace full of NaN
    bit patterns (0xFF bytes) gives the oracle's result, identical to a zeroed one."""
    torch, dev = torch_dev
    fab = fabmod()
    q, k, v, d = make_qkvd(s, seed)
    mask = small_mask(mkind, s, seed)
    scale = float(np.float32(1 / math.sqrt(s.DK)))
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    tm = to_dev(torch, dev, mask)
    O = lse = None
    if supplied:
        O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode="bf16")
    blobs = []
    for fill in (255, 0):
        ws, _ = fab.alloc_workspace(fab.Shape(*s.astuple()), "bf16", True, supplied, dev)
        ws.fill_(fill)
        blobs.append(fab.backward(t[0], t[1], t[2], t[3], scale, mask=tm, mode="bf16", O=O, lse=lse, ws=ws))
    torch.cuda.synchronize()
    b0, b1 = (x.cpu().numpy() for x in blobs)
    assert np.array_equal(b0, b1)
    check_blob(s, b0, oracle_full(s, q, k, v, d, mask, scale), "bf16", name, mask)


def test_caller_stream_is_used(torch_dev):
    # every launch goes to the stream the caller passes: the same call on a side
    # stream (inputs written there, nothing synchronised in between) gives the same blob
    torch, dev = torch_dev
    fab = fabmod()
    s = Shape(1, 4, 2, 300, 300, 64, 64)
    q, k, v, d = make_qkvd(s, 71)
    mask = to_dev(torch, dev, causal_mask(s.N, s.M))
    ref = fab.backward(*[to_dev(torch, dev, x) for x in (q, k, v, d)], 0.125, mask=mask, mode="bf16")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        t = [torch.from_numpy(x).to(dev, non_blocking=False) for x in (q, k, v, d)]
        out = fab.backward(*t, 0.125, mask=mask, mode="bf16", stream=side)
    side.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


def test_side_stream_that_is_not_current_keeps_its_buffers(torch_dev):
    # a stream passed without being made current: the call's own workspace and blob
    # belong to that stream, so memory allocated and filled on the current stream
    # right after the call (before any synchronisation) cannot take them over while
    # the call's kernels still run
    torch, dev = torch_dev
    fab = fabmod()
    s = Shape(1, 4, 2, 300, 300, 64, 64)
    q, k, v, d = make_qkvd(s, 73)
    mask = to_dev(torch, dev, causal_mask(s.N, s.M))
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    ref = fab.backward(*t, 0.125, mask=mask, mode="bf16").clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = fab.backward(*t, 0.125, mask=mask, mode="bf16", stream=side)
    junk = [torch.full((1 << 22,), float("nan"), device=dev) for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("mode", ["bf16", "f32"])
def test_graph_capture_replays(torch_dev, mode):
    # fab_backward captured into a graph (no memset nodes: every zeroing is a
    # kernel) and replayed three times with eager work and synchronisation in
    # between; every replay matches the eager result (bf16 mode bit for bit, f32
    # mode up to the order of its dQ atomics)
    torch, dev = torch_dev
    fab = fabmod()
    s = Shape(1, 4, 2, 257, 300, 64, 64)
    q, k, v, d = make_qkvd(s, 72)
    mask = to_dev(torch, dev, random_mask(s.N, s.M, 72, p_inf=0.3, full_rows=1, full_cols=1))
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    fs = fab.Shape(*s.astuple())
    ws, _ = fab.alloc_workspace(fs, mode, True, False, dev)
    blob = torch.empty(fab.blob_layout(fs)[3], device=dev)
    eager = fab.backward(*t, 0.125, mask=mask, mode=mode, ws=ws).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            fab.backward(*t, 0.125, mask=mask, mode=mode, blob=blob, ws=ws, stream=cap)
    torch.cuda.synchronize()
    for rep in range(3):
        blob.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if mode == "bf16":
            assert torch.equal(blob.view(torch.int32), eager.view(torch.int32)), rep
        else:
            assert torch.allclose(blob, eager, rtol=1e-5, atol=1e-6 * float(eager.abs().max())), rep
        # eager work between replays
        _ = fab.backward(*t, 0.125, mask=mask, mode=mode)
        torch.cuda.synchronize()


def test_d_ones_closed_form_on_gpu(torch_dev):
    # d = ones: every component of dV[:, m] equals the summed attention weight of key m
    torch, dev = torch_dev
    s = Shape(2, 4, 2, 96, 128, 32, 48)
    q, k, v, _ = make_qkvd(s, 32)
    d = np.ones(s.d_shape, np.float32)
    blob = run_gpu(torch, dev, s, q, k, v, d, None, 1 / math.sqrt(s.DK), "f32")
    fab = fabmod()
    _, off_k, off_v, _ = fab.blob_layout(fab.Shape(*s.astuple()))
    dv = blob[off_v:off_v + s.DV * s.M * s.Hkv * s.B].reshape(s.v_shape)
    assert np.max(np.abs(dv - dv[..., :1])) <= 1e-5 * np.max(np.abs(dv))
    rk2 = s.H // s.Hkv
    assert np.allclose(dv[..., 0].sum(axis=2), rk2 * s.N, rtol=1e-4)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_all_masked_everything_gives_zero_blob(torch_dev, mode):
    torch, dev = torch_dev
    s = Shape(1, 2, 1, 40, 70, 32, 32)
    q, k, v, d = make_qkvd(s, 81)
    mask = np.full((s.N, s.M), F16_NEG_INF, np.uint16)
    blob = run_gpu(torch, dev, s, q, k, v, d, mask, 0.2, mode)
    assert np.all(blob == 0)


@pytest.mark.parametrize("s", [Shape(1, 2, 1, 0, 5, 8, 8), Shape(1, 2, 1, 5, 0, 8, 8),
                               Shape(0, 2, 1, 5, 5, 8, 8)], ids=["N0", "M0", "B0"])
def test_empty_extents(torch_dev, s):
    torch, dev = torch_dev
    q, k, v, d = make_qkvd(s, 3)
    blob = run_gpu(torch, dev, s, q, k, v, d, None, 0.3, "f32")
    assert np.all(blob == 0)


# ---------------------------------------------------------------- the five workloads at full size

_cache = {}


def workload(wid):
    if wid not in _cache:
        _cache[wid] = fi.workload_inputs(wid)
    return _cache[wid]


def sample_ids(s, wid, rng):
    """Rows (n + N*(h + H*b)) and keys (m + M*(g + Hkv*b)) the oracle evaluates one by one.
    Keys cover the whole key range of several groups: the tile edges 0, 63, 64, 127, 128,
    the middle, the last key and random ones -- under the causal rule key m is seen by
    every query from m on, so the first keys carry the deepest dK/dV accumulation."""
    R = s.B * s.H * s.N
    rows = list(rng.choice(R, 24, replace=False)) + [0, R - 1]
    fixed = [0, 63, 64, 127, 128, s.M // 2 - 1, s.M // 2, s.M - 129, s.M - 1]
    fixed = [m for m in fixed if 0 <= m < s.M]
    ngroups = 2 if wid == 4 else 3
    keys = []
    for gb in rng.choice(s.Hkv * s.B, min(ngroups, s.Hkv * s.B), replace=False):
        ms = fixed + list(rng.choice(s.M, 6, replace=False))
        keys += [int(m + s.M * gb) for m in ms]
    return np.array(rows, dtype=np.int64), np.array(sorted(set(keys)), dtype=np.int64)


def test_bf16_large_shape_recomputes_dq(torch_dev):
    """Head dims up to 128 whose bf16 dS tiles would pass 4 GiB (here 5.4 GB; the tiles
    are dense over all pairs, whatever the mask) take dQ from the recompute kernel, the
    grouped-query reduction as its own launch, and (groups of 10, 4608 work-groups) two
    query heads per dK/dV work-group.  A causal mask with M > N keeps the oracle cheap:
    sampled rows, keys just below N and keys past N (exactly zero), and sums that hold
    at any size."""
    torch, dev = torch_dev
    from oracle import oracle as orc
    fab = fabmod()
    s = Shape(1, 40, 4, 4096, 16384, 64, 64)
    print(f"[parity] large recompute {s}", flush=True)
    assert 2 * s.B * s.H * s.N * s.M > 4 << 30
    q, k, v, d = make_qkvd(s, 52)
    mask = causal_mask(s.N, s.M)
    scale = float(np.float32(1 / math.sqrt(s.DK)))
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    blob = fab.backward(*t, scale, mask=to_dev(torch, dev, mask), mode="bf16")
    torch.cuda.synchronize()
    blob = blob.cpu().numpy()
    _, off_k, off_v, total = fab.blob_layout(fab.Shape(*s.astuple()))
    nq, nk, nv = q.size, k.size, v.size
    assert np.all(np.isfinite(blob))
    dq = blob[:nq].reshape(s.q_shape)
    dk = blob[off_k:off_k + nk].reshape(s.k_shape)
    dv = blob[off_v:off_v + nv].reshape(s.v_shape)
    assert np.all(dk[:, :, s.N:] == 0) and np.all(dv[:, :, s.N:] == 0)   # keys no query sees
    rng = np.random.default_rng(152)
    rows = np.concatenate([rng.choice(s.B * s.H * s.N, 24, replace=False), [0, s.B * s.H * s.N - 1]])
    keys = [int(m + s.M * g) for g in range(s.Hkv) for m in rng.choice(np.arange(s.N - 256, s.N), 3, replace=False)]
    keys += [s.N + 5, s.M - 1]
    rdq, rdk, rdv = orc.backward_sampled(s, q, k, v, mask, d, scale, rows, keys)
    gdq = np.stack([dq[r // (s.N * s.H), (r // s.N) % s.H, r % s.N] for r in rows])
    gdk = np.stack([dk[r // (s.M * s.Hkv), (r // s.M) % s.Hkv, r % s.M] for r in keys])
    gdv = np.stack([dv[r // (s.M * s.Hkv), (r // s.M) % s.Hkv, r % s.M] for r in keys])
    for name, got, ref in (("dq", gdq, rdq), ("dk", gdk, rdk), ("dv", gdv, rdv)):
        e = rel_err(got, ref)
        print(f"  sampled {name} max-rel {e:.3e}", flush=True)
        assert e <= TOL["bf16"], name
    # sum_m dK[:, m] = 0 per group; sum_m dV[:, m] = the group's sum of d over all rows
    tol = TOL["bf16"]
    dk_sum = dk.astype(np.float64).sum(axis=2)
    assert np.max(np.abs(dk_sum) / np.abs(dk.astype(np.float64)).sum(axis=2)) <= tol
    rk2 = s.H // s.Hkv
    expect = d.astype(np.float64).sum(axis=1).reshape(s.B, s.Hkv, rk2, s.DV).sum(axis=2)
    got = dv.astype(np.float64).sum(axis=2)
    assert np.max(np.abs(got - expect)) <= tol * np.max(np.abs(dv.astype(np.float64)).sum(axis=2))


WL_CASES = [(1, "f32"), (2, "f32"), (2, "bf16"), (3, "bf16"), (3, "f32"), (4, "bf16"), (5, "f32"), (5, "bf16")]
_oracle_cache = {}


def sampled_oracle(wid, s, q, k, v, mask, d, scale):
    if wid not in _oracle_cache:
        from oracle import oracle as orc
        rows, keys = sample_ids(s, wid, np.random.default_rng(100 + wid))
        t0 = time.perf_counter()
        ref = orc.backward_sampled(s, q, k, v, mask, d, scale, rows, keys)
        print(f"  oracle: {len(rows)} rows, {len(keys)} keys in {time.perf_counter() - t0:.1f} s", flush=True)
        _oracle_cache[wid] = (rows, keys, ref)
    return _oracle_cache[wid]


@pytest.mark.parametrize("route", ["o_lse_supplied", "own_forward"])
@pytest.mark.parametrize("wid,mode", WL_CASES, ids=[f"w{w}-{m}" for w, m in WL_CASES])
def test_workload_full_size(torch_dev, wid, mode, route):
    """Each workload at full size in both routes of fab_backward: O and LSE from a prior
    fab_forward_lse (the benchmark's headline call) and O = lse = NULL (the forward inside
    the call: in bf16 mode the forward kernel writes the tiles, LSE/D blocks and pads the
    backward reads)."""
    torch, dev = torch_dev
    from oracle import oracle as orc
    s, q, k, v, d, mask, scale = workload(wid)
    print(f"[parity] workload {wid} {mode} {route} {s}", flush=True)
    fab = fabmod()
    fs = fab.Shape(*s.astuple())
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    tm = to_dev(torch, dev, mask)
    O = lse = None
    if route == "o_lse_supplied":
        O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode=mode)
    blob = fab.backward(t[0], t[1], t[2], t[3], scale, mask=tm, mode=mode, O=O, lse=lse)
    torch.cuda.synchronize()
    blob = blob.cpu().numpy()
    del t, O, lse
    _, off_k, off_v, total = fab.blob_layout(fs)
    nq, nk, nv = q.size, k.size, v.size
    assert np.all(np.isfinite(blob))
    assert np.all(blob[nq:off_k] == 0) and np.all(blob[off_k + nk:off_v] == 0) and np.all(blob[off_v + nv:] == 0)
    dq = blob[:nq].reshape(s.q_shape)
    dk = blob[off_k:off_k + nk].reshape(s.k_shape)
    dv = blob[off_v:off_v + nv].reshape(s.v_shape)
    tol = TOL[mode]

    dead_rows, dead_keys = structural_zeros(s, mask)
    assert np.all(dq[:, :, dead_rows, :] == 0)
    assert np.all(dk[:, :, dead_keys, :] == 0) and np.all(dv[:, :, dead_keys, :] == 0)
    if wid in (1, 2):
        key = ("full", wid)
        if key not in _oracle_cache:
            _oracle_cache[key] = orc.backward(s, q, k, v, mask, d, scale)
        ref = _oracle_cache[key]
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = rel_err(got, ref[name])
            print(f"  {name} max-rel {e:.3e}", flush=True)
            assert e <= tol, name
        return

    rows, keys, (rdq, rdk, rdv) = sampled_oracle(wid, s, q, k, v, mask, d, scale)
    gdq = np.stack([dq[r // (s.N * s.H), (r // s.N) % s.H, r % s.N] for r in rows])
    gdk = np.stack([dk[r // (s.M * s.Hkv), (r // s.M) % s.Hkv, r % s.M] for r in keys])
    gdv = np.stack([dv[r // (s.M * s.Hkv), (r // s.M) % s.Hkv, r % s.M] for r in keys])
    for name, got, ref in (("dq", gdq, rdq), ("dk", gdk, rdk), ("dv", gdv, rdv)):
        e = rel_err(got, ref)
        print(f"  sampled {name} max-rel {e:.3e}", flush=True)
        assert e <= tol, name

    # sums that hold at any size: a common shift of all keys leaves every softmax row
    # unchanged, so sum_m dK[:, m] = 0; and sum_m dV[:, m] = sum of d over the live
    # query rows of the group
    live = None
    if mask is not None:
        live = np.array([np.any(mask[n] != F16_NEG_INF) for n in range(s.N)])
    rk2 = s.H // s.Hkv
    dk_sum = dk.astype(np.float64).sum(axis=2)
    dk_abs = np.abs(dk.astype(np.float64)).sum(axis=2)
    assert np.max(np.abs(dk_sum) / np.maximum(dk_abs, 1e-30)) <= tol
    d64 = d.astype(np.float64)
    if live is not None:
        d64 = d64 * live[None, :, None, None]
    expect = d64.sum(axis=1).reshape(s.B, s.Hkv, rk2, s.DV).sum(axis=2)
    got = dv.astype(np.float64).sum(axis=2)
    assert np.max(np.abs(got - expect)) <= tol * np.max(np.abs(dv.astype(np.float64)).sum(axis=2))
    if wid == 5:
        # keys past the padding cut and all-masked query rows are exactly zero
        assert np.all(dk[:, :, 3072:] == 0) and np.all(dv[:, :, 3072:] == 0)
        assert np.all(dq[:, :, ::64, :] == 0)
