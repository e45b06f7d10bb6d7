"""GPU checks of the 16-bit result blob (FAB_BF16_BLOB, FAB_F16_BLOB).

The kernels accumulate every gradient in f32 whatever the blob's type, and round
once at the store, so a 16-bit blob must be, element for element and bit for bit,
the f32 blob of the same call rounded to nearest even (torch's own f32 -> bf16 /
f16 conversion).  Each case runs both and compares them over the unpadded slices
of every route: the 8-wave dK/dV kernel writing the result itself (one or two
heads per work-group) or through per-unit partials and the grouped-query sum, the
4-wave kernel (192- and 256-wide heads), dQ from the stored dS or from the
recompute kernel, the backward's own forward or a supplied O and LSE, 16-bit
inputs and ALiBi slopes.  The pads read as 16-bit zeros, nothing past the blob's
end is written, and on small shapes the 16-bit values also meet the oracle's bf16
bar directly.
"""
import math

import numpy as np
import pytest

from fab_inputs import Shape, make_qkvd, random_mask, causal_mask, F16_NEG_INF

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2      # the bf16-mode bar of the oracle parity tests (max|err| / max|ref|)
GUARD = 64           # elements after the blob that must stay untouched
SENTINEL = 0x7FC1    # a 16-bit pattern the kernels never write (a NaN in both formats)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    return torch, torch.device("cuda:0")


def fabmod():
    import exact_attention_backward_fab_amd as fab
    fab.lib()
    return fab


def dtype16(torch, store):
    return torch.bfloat16 if store == "bf16" else torch.float16


def mask_of(kind, s, seed):
    if kind in (None, "causal_flag"):
        return None
    if kind == "causal":
        return causal_mask(s.N, s.M)
    return random_mask(s.N, s.M, seed, p_inf=0.3, full_rows=2, full_cols=3)


def to_dev(torch, dev, a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def slopes(H):
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], np.float32)


def blob16_of(torch, dev, fab, fs, dt):
    """A 16-bit blob of the layout's length plus a guard band, every element SENTINEL."""
    total = fab.blob_layout(fs, dt)[3]
    raw = torch.full((total + GUARD,), SENTINEL, dtype=torch.int16, device=dev)
    return raw.view(dt), total


def check_against_f32(torch, fab, fs, b16, total16, b32, dt, tag):
    """b16 (with guard band) against the f32 blob b32 of the same call."""
    _, k16, v16, t16 = fab.blob_layout(fs, dt)
    _, k32, v32, _ = fab.blob_layout(fs)
    assert t16 == total16
    nq = fs.DK * fs.N * fs.H * fs.B
    nk = fs.DK * fs.M * fs.Hkv * fs.B
    nv = fs.DV * fs.M * fs.Hkv * fs.B
    bits16 = b16.view(torch.int16)
    for name, lo16, lo32, n in (("dq", 0, 0, nq), ("dk", k16, k32, nk), ("dv", v16, v32, nv)):
        want = b32[lo32:lo32 + n].to(dt).view(torch.int16)
        got = bits16[lo16:lo16 + n]
        bad = (got != want).nonzero().flatten()
        if bad.numel():
            ex = [(int(i), float(b32[lo32 + i]), hex(int(got[i]) & 0xFFFF), hex(int(want[i]) & 0xFFFF))
                  for i in bad[:6].tolist()]
            raise AssertionError(f"{tag}: {name} differs from the rounded f32 result at {bad.numel()} "
                                 f"elements (index, f32 value, stored bits, rounded bits): {ex}")
    for lo, hi in ((nq, k16), (k16 + nk, v16), (v16 + nv, t16)):
        assert hi - lo < 8
        assert bool((bits16[lo:hi] == 0).all()), f"{tag}: pad [{lo}, {hi}) not zero"
    assert bool((bits16[t16:] == SENTINEL).all()), f"{tag}: write past the end of the blob"


def oracle_check(s, b16, fab, fs, dt, q, k, v, d, mask, scale, alibi, tag):
    from oracle import oracle as orc
    ref = orc.backward(s, q, k, v, mask, d, scale,
                       **({"alibi": alibi.astype(np.float64)} if alibi is not None else {}))
    _, off_k, off_v, _ = fab.blob_layout(fs, dt)
    got = b16.float().cpu().numpy()
    scale_all = max(float(np.max(np.abs(ref[n]))) if ref[n].size else 0.0 for n in ("dq", "dk", "dv"))
    for name, lo in (("dq", 0), ("dk", off_k), ("dv", off_v)):
        r = ref[name]
        g = got[lo:lo + r.size].reshape(r.shape).astype(np.float64)
        den = np.max(np.abs(r)) if r.size and np.max(np.abs(r)) > 0 else scale_all
        e = np.max(np.abs(g - r)) / den if r.size else 0.0
        assert e <= BF16_TOL, f"{tag}: {name} max-rel error {e:.3e} against the oracle"


CASES = [
    # name, shape, mask kind, seed, supplied O/LSE, inputs (f32 / bf16 / f16), ALiBi, oracle check
    ("odd_pads_random", Shape(1, 3, 1, 37, 29, 3, 5), "random", 41, False, "f32", False, True),
    ("gqa_d64_random", Shape(2, 4, 2, 200, 300, 64, 64), "random", 42, False, "f32", False, True),
    ("mha_d128_causal_flag", Shape(1, 4, 4, 333, 333, 128, 128), "causal_flag", 43, False, "f32", False, False),
    ("d40_72_supplied", Shape(1, 3, 1, 70, 90, 40, 72), None, 45, True, "f32", False, True),
    ("d192_128_staged_mask", Shape(1, 2, 2, 100, 264, 192, 128), "random", 50, False, "f32", False, False),
    ("d192_192_f16_inputs", Shape(1, 2, 1, 65, 97, 192, 192), "random", 46, True, "f16", False, False),
    ("d256_gqa_alibi", Shape(1, 4, 2, 100, 264, 256, 256), "random", 55, False, "bf16", True, True),
    # two query heads of a group of 2 per work-group: dK/dV straight into the result
    ("two_heads_per_wg_group_of_2", Shape(4, 16, 8, 100, 2048, 64, 64), "random", 50, False, "f32", False, False),
    # a grid that fills the chip without query splits: one head per unit, no partials
    ("mha_d128_full_grid", Shape(1, 16, 16, 1024, 2048, 128, 128), "causal_flag", 60, True, "bf16", False, False),
]


@pytest.mark.parametrize("store", ["bf16", "f16"])
@pytest.mark.parametrize("name,s,mkind,seed,supplied,inputs,use_alibi,with_oracle", CASES,
                         ids=[c[0] for c in CASES])
def test_16bit_blob_is_the_rounded_f32_blob(torch_dev, name, s, mkind, seed, supplied, inputs, use_alibi,
                                            with_oracle, store):
    torch, dev = torch_dev
    fab = fabmod()
    print(f"[blob16] {name} {store} {s}", flush=True)
    dt = dtype16(torch, store)
    fs = fab.Shape(*s.astuple())
    q, k, v, d = make_qkvd(s, seed)
    mask = mask_of(mkind, s, seed)
    causal = mkind == "causal_flag"
    scale = float(np.float32(1.0 / math.sqrt(s.DK)))
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    if inputs != "f32":
        t = [x.to(torch.bfloat16 if inputs == "bf16" else torch.float16) for x in t]
    tm = to_dev(torch, dev, mask)
    al = slopes(s.H) if use_alibi else None
    ta = to_dev(torch, dev, al)
    O = lse = None
    if supplied:
        O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode="bf16", causal=causal, alibi=ta)
    b32 = fab.backward(*t, scale, mask=tm, mode="bf16", O=O, lse=lse, causal=causal, alibi=ta)
    b16, total16 = blob16_of(torch, dev, fab, fs, dt)
    out = fab.backward(*t, scale, mask=tm, mode="bf16", O=O, lse=lse, causal=causal, alibi=ta, blob=b16)
    assert out.data_ptr() == b16.data_ptr() and out.dtype == dt
    torch.cuda.synchronize()
    check_against_f32(torch, fab, fs, b16, total16, b32, dt, f"{name} {store}")
    if with_oracle:
        qr, kr, vr, dr = (x.float().cpu().numpy() for x in t)
        oracle_check(s, b16[:total16], fab, fs, dt, qr, kr, vr, dr, mask, scale, al, f"{name} {store}")


@pytest.mark.parametrize("store", ["bf16", "f16"])
def test_16bit_blob_from_the_recompute_dq_route(torch_dev, store):
    """Head dims up to 128 whose dS tiles would pass 4 GiB take dQ from the recompute
    kernel (query blocks shared by two work-groups) and the grouped-query sum as a
    launch of its own; its 16-bit stores are those of the f32 result, rounded."""
    torch, dev = torch_dev
    fab = fabmod()
    s = Shape(1, 40, 4, 4096, 16384, 64, 64)
    assert 2 * s.B * s.H * s.N * s.M > 4 << 30
    print(f"[blob16] recompute dQ {store} {s}", flush=True)
    dt = dtype16(torch, store)
    fs = fab.Shape(*s.astuple())
    g = torch.Generator(device=dev)
    g.manual_seed(5207)
    t = [torch.rand(sh, generator=g, device=dev) * 2 - 1
         for sh in (s.q_shape, s.k_shape, s.v_shape, s.d_shape)]
    scale = 0.125
    b32 = fab.backward(*t, scale, mode="bf16", causal=True)
    b16, total16 = blob16_of(torch, dev, fab, fs, dt)
    fab.backward(*t, scale, mode="bf16", causal=True, blob=b16)
    torch.cuda.synchronize()
    check_against_f32(torch, fab, fs, b16, total16, b32, dt, f"recompute {store}")


@pytest.mark.parametrize("store", ["bf16", "f16"])
@pytest.mark.parametrize("s", [Shape(1, 2, 1, 0, 5, 8, 8), Shape(1, 2, 1, 5, 0, 8, 8), Shape(0, 2, 1, 5, 5, 8, 8),
                               Shape(1, 2, 1, 5, 0, 3, 5)], ids=["N0", "M0", "B0", "M0_odd"])
def test_16bit_blob_of_empty_extents_is_zero(torch_dev, s, store):
    torch, dev = torch_dev
    fab = fabmod()
    dt = dtype16(torch, store)
    fs = fab.Shape(*s.astuple())
    q, k, v, d = make_qkvd(s, 3)
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    b16, total16 = blob16_of(torch, dev, fab, fs, dt)
    fab.backward(*t, 0.3, mode="bf16", blob=b16)
    torch.cuda.synchronize()
    bits = b16.view(torch.int16)
    assert bool((bits[:total16] == 0).all())
    assert bool((bits[total16:] == SENTINEL).all())


def test_16bit_blob_of_all_masked_rows_is_zero(torch_dev):
    torch, dev = torch_dev
    fab = fabmod()
    s = Shape(1, 2, 1, 40, 70, 32, 32)
    fs = fab.Shape(*s.astuple())
    q, k, v, d = make_qkvd(s, 81)
    mask = np.full((s.N, s.M), F16_NEG_INF, np.uint16)
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    b16, total16 = blob16_of(torch, dev, fab, fs, torch.bfloat16)
    fab.backward(*t, 0.2, mask=to_dev(torch, dev, mask), mode="bf16", blob=b16)
    torch.cuda.synchronize()
    assert bool((b16.view(torch.int16)[:total16] == 0).all())


def test_16bit_blob_unpacks_and_passes_through_noalloc(torch_dev):
    """unpack() reads the 16-bit offsets, and fab_backward_noalloc writes the same
    16-bit blob as fab_backward."""
    torch, dev = torch_dev
    fab = fabmod()
    s = Shape(1, 4, 2, 150, 170, 64, 64)
    fs = fab.Shape(*s.astuple())
    q, k, v, d = make_qkvd(s, 77)
    t = [to_dev(torch, dev, x) for x in (q, k, v, d)]
    a = fab.backward(*t, 0.125, mode="bf16", causal=True, blob_dtype=torch.float16)
    b, _ = blob16_of(torch, dev, fab, fs, torch.float16)
    fab.backward_noalloc(*t, 0.125, b, mode="bf16", causal=True)
    f = fab.backward(*t, 0.125, mode="bf16", causal=True)
    torch.cuda.synchronize()
    total = fab.blob_layout(fs, torch.float16)[3]
    assert a.dtype == torch.float16 and a.numel() >= total
    assert torch.equal(a[:total].view(torch.int16), b[:total].view(torch.int16))
    for x16, x32 in zip(fab.unpack(a, fs), fab.unpack(f, fs)):
        assert x16.dtype == torch.float16 and x16.shape == x32.shape
        assert torch.equal(x16.view(torch.int16), x32.to(torch.float16).view(torch.int16))


def test_bf16_autograd_stays_bf16_end_to_end(torch_dev):
    """attention() on bfloat16 inputs: O is the bf16-stored forward output, and the
    gradients are bf16 views of one bf16 blob at its 16-bit offsets, bit for bit the
    direct calls (forward with FAB_BF16_O, backward with bf16 d and FAB_BF16_BLOB)."""
    torch, dev = torch_dev
    fab = fabmod()
    from exact_attention_backward_fab_amd.autograd import attention
    s = Shape(2, 4, 2, 150, 170, 64, 48)
    fs = fab.Shape(*s.astuple())
    q, k, v, d = make_qkvd(s, 102)
    mask = random_mask(s.N, s.M, 102, p_inf=0.3, full_rows=1, full_cols=1)
    tm = to_dev(torch, dev, mask)
    t = [to_dev(torch, dev, x).to(torch.bfloat16) for x in (q, k, v, d)]
    tq, tk, tv = [x.clone().requires_grad_(True) for x in t[:3]]
    O = attention(tq, tk, tv, mask=tm, scale=0.125, mode="bf16")
    assert O.dtype == torch.bfloat16
    gq, gk, gv = torch.autograd.grad(O, (tq, tk, tv), grad_outputs=t[3])
    O_ref, lse_ref = fab.forward_lse(t[0], t[1], t[2], 0.125, mask=tm, mode="bf16", o_bf16=True)
    blob = fab.backward(*t, 0.125, mask=tm, mode="bf16", O=O_ref, lse=lse_ref, blob_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O_ref.view(torch.int16))
    base = gq.untyped_storage().data_ptr()
    assert gk.untyped_storage().data_ptr() == base and gv.untyped_storage().data_ptr() == base
    _, off_k, off_v, _ = fab.blob_layout(fs, torch.bfloat16)
    assert (gq.storage_offset(), gk.storage_offset(), gv.storage_offset()) == (0, off_k, off_v)
    for g, r in zip((gq, gk, gv), fab.unpack(blob, fs)):
        assert g.dtype == torch.bfloat16 and torch.equal(g.view(torch.int16), r.view(torch.int16))
