"""GPU parity of the ALiBi entry points (fab_forward_lse_alibi, fab_backward_alibi)
against the f64 oracle with the same per-head slopes.  The ggmlR test file names
ALiBi only to show its graph builder refusing `max_bias`; the reading implemented and
tested here: the score of query n at key m gains slope_h * (m - n) after the scale.

Bar as everywhere: per gradient tensor max|gpu - oracle| / max|oracle| <= 1e-4 (f32
mode) and <= 2e-2 (bf16 mode); exact zeros where the mask fixes them.  Slopes of zero
give bit for bit the result without slopes (the bias vanishes; the same arithmetic
runs)."""
import math

import numpy as np
import pytest

from fab_inputs import Shape, make_qkvd, causal_mask, random_mask, F16_NEG_INF

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _mask(kind, s, seed):
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


def _slopes(H):
    # ggml-like geometric slopes for most heads, one zero and one negative slope
    s = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]
    if H > 1:
        s[1] = 0.0
    if H > 2:
        s[2] = -0.05
    return np.array(s, np.float32)


CASES = [
    # name, shape, mask kind, seed
    ("causal_gqa_d128", Shape(1, 4, 2, 333, 333, 128, 128), "causal", 501),
    ("random_mask_d64", Shape(2, 4, 2, 200, 300, 64, 64), "random", 502),
    ("d192_128_padding", Shape(1, 3, 3, 130, 260, 192, 128), "padding", 503),
    ("odd_dims_nomask", Shape(1, 3, 1, 70, 90, 40, 72), None, 504),
    # 256-wide heads: the 4-wave dK/dV kernel with its columns split over two work-groups
    ("d256_random_gqa", Shape(1, 4, 2, 90, 200, 256, 256), "random", 506),
    ("two_heads_per_wg", Shape(2, 32, 8, 70, 2048, 128, 128), None, 505),
]


@pytest.mark.parametrize("supplied", [False, True], ids=["own_forward", "o_lse_supplied"])
@pytest.mark.parametrize("mode", ["f32", "bf16"])
@pytest.mark.parametrize("name,s,mkind,seed", CASES, ids=[c[0] for c in CASES])
def test_alibi_against_oracle(name, s, mkind, seed, mode, supplied):
    import torch
    import exact_attention_backward_fab_amd as fab
    from oracle import oracle as orc
    dev = torch.device("cuda:0")
    print(f"[alibi] {name} {mode} supplied={supplied} {s}", flush=True)
    q, k, v, d = make_qkvd(s, seed)
    mask = _mask(mkind, s, seed)
    slopes = _slopes(s.H)
    scale = float(np.float32(1 / math.sqrt(s.DK)))
    t = [torch.from_numpy(x).to(dev) for x in (q, k, v, d)]
    tm = None if mask is None else torch.from_numpy(mask.view(np.int16)).to(dev)
    ta = torch.from_numpy(slopes).to(dev)
    O = lse = None
    if supplied:
        O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode=mode, alibi=ta)
    fs = fab.Shape(*s.astuple())
    total = fab.blob_layout(fs)[3]
    blob = torch.full((total + 64,), float("nan"), device=dev)
    fab.backward(*t, scale, mask=tm, mode=mode, O=O, lse=lse, blob=blob[:total], alibi=ta)
    torch.cuda.synchronize()
    got = blob.cpu().numpy()
    assert np.all(np.isnan(got[total:]))
    got = got[:total]
    assert np.all(np.isfinite(got))
    ref = orc.backward(s, q, k, v, mask, d, scale, alibi=slopes.astype(np.float64))
    _, off_k, off_v, _ = fab.blob_layout(fs)
    for nm, lo in (("dq", 0), ("dk", off_k), ("dv", off_v)):
        n = ref[nm].size
        e = np.max(np.abs(got[lo:lo + n] - ref[nm].ravel())) / np.max(np.abs(ref[nm]))
        print(f"  {nm} max-rel {e:.3e}", flush=True)
        assert e <= TOL[mode], nm
    if supplied:
        Og, lg = O.cpu().numpy(), lse.cpu().numpy()
        assert np.max(np.abs(Og - ref["O"])) / np.max(np.abs(ref["O"])) <= TOL[mode]
        fin = np.isfinite(ref["lse"])
        assert np.array_equal(np.isneginf(lg), ~fin)
        # the bias makes the LSE large (up to slope * M): bound its error relative to its size
        lerr = np.abs(lg[fin] - ref["lse"][fin]) / np.maximum(1.0, np.abs(ref["lse"][fin]))
        assert np.max(lerr) <= (1e-5 if mode == "f32" else 2e-2)
    if mask is not None:
        dead = (mask == F16_NEG_INF).all(axis=1)
        dq = got[:q.size].reshape(s.q_shape)
        assert np.all(dq[:, :, dead, :] == 0)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_alibi_causal_flag_equals_causal_mask(mode):
    import torch
    import exact_attention_backward_fab_amd as fab
    dev = torch.device("cuda:0")
    s = Shape(1, 4, 2, 300, 257, 64, 64)
    q, k, v, d = make_qkvd(s, 506)
    t = [torch.from_numpy(x).to(dev) for x in (q, k, v, d)]
    ta = torch.from_numpy(_slopes(s.H)).to(dev)
    tm = torch.from_numpy(causal_mask(s.N, s.M).view(np.int16)).to(dev)
    a = fab.backward(*t, 0.125, mode=mode, causal=True, alibi=ta)
    b = fab.backward(*t, 0.125, mask=tm, mode=mode, alibi=ta)
    torch.cuda.synchronize()
    if mode == "bf16":
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    else:   # the dQ atomics of f32 mode add in any order; dK and dV are summed in a fixed one
        off_k = fab.blob_layout(fab.Shape(*s.astuple()))[1]
        assert float((a[:off_k] - b[:off_k]).abs().max()) <= 1e-6 * float(b[:off_k].abs().max())
        assert torch.equal(a[off_k:].view(torch.int32), b[off_k:].view(torch.int32))


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_zero_slopes_equal_no_slopes_bit_for_bit(mode):
    import torch
    import exact_attention_backward_fab_amd as fab
    dev = torch.device("cuda:0")
    s = Shape(1, 4, 2, 333, 333, 128, 128)
    q, k, v, d = make_qkvd(s, 507)
    t = [torch.from_numpy(x).to(dev) for x in (q, k, v, d)]
    tm = torch.from_numpy(causal_mask(s.N, s.M).view(np.int16)).to(dev)
    z = torch.zeros(s.H, device=dev)
    a = fab.backward(*t, 0.1, mask=tm, mode=mode, alibi=z)
    b = fab.backward(*t, 0.1, mask=tm, mode=mode)
    torch.cuda.synchronize()
    if mode == "bf16":
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    else:   # the dQ atomics of f32 mode add in any order
        assert float((a - b).abs().max()) <= 1e-6 * float(b.abs().max())


def test_alibi_through_autograd():
    import torch
    from exact_attention_backward_fab_amd.autograd import attention
    from oracle import oracle as orc
    dev = torch.device("cuda:0")
    s = Shape(2, 4, 2, 150, 170, 64, 48)
    q, k, v, d = make_qkvd(s, 508)
    slopes = _slopes(s.H)
    tq, tk, tv = [torch.from_numpy(x).to(dev).requires_grad_(True) for x in (q, k, v)]
    O = attention(tq, tk, tv, scale=0.125, mode="f32", alibi=torch.from_numpy(slopes).to(dev))
    gq, gk, gv = torch.autograd.grad(O, (tq, tk, tv), grad_outputs=torch.from_numpy(d).to(dev))
    ref = orc.backward(s, q, k, v, None, d, 0.125, alibi=slopes.astype(np.float64))
    for nm, g in (("dq", gq), ("dk", gk), ("dv", gv)):
        assert np.max(np.abs(g.cpu().numpy() - ref[nm])) / np.max(np.abs(ref[nm])) <= 1e-4, nm
