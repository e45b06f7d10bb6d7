"""Pins for the f64 CPU oracle: each checks it against something other than itself.

Sources of the pins:
  * ggmlR "tests/testthat/test-flash-attn-back.R": its finite-difference checks
    (`num_grad`, eps = 1e-3, tolerance 2e-2) on the single-head, causal-mask and
    grouped-query shapes, the packing-layout test and its "a key no query attends
    to gets no gradient" remark.  R is not available, so the same shapes are
    drawn with numpy's generator seeded with the test's seed numbers; the values
    differ from R's.
  * labml "Flash Attention", section "Backward pass": D_i = dO_i . O_i = sum_j
    P_ij dP_ij, so each row of dS sums to zero.
  * Closed forms (one key, uniform attention, d = ones), structural identities
    (grouped-query = repeated keys/values, mask shift invariance, a masked key =
    a deleted key) and an independent library implementation (torch autograd in
    float64).
A plausible slip in the oracle (a dropped D term, a wrong sign, a swapped head
map, the mask added before the scale, a transposed layout) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

from fab_inputs import Shape, make_qkvd, causal_mask, random_mask, F16_NEG_INF
from oracle import oracle as orc


def rel_max(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a - b)))


def r_all_equal_rel(target, current):
    """Mean relative difference as R's all.equal reports it (testthat's tolerance)."""
    target = np.asarray(target).ravel()
    current = np.asarray(current).ravel()
    xy = np.mean(np.abs(target - current))
    xn = np.mean(np.abs(target))
    return xy / xn if xn > 0 else xy


# ---------------------------------------------------------------- f16 decode

def test_half_decode_matches_numpy_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- finite differences

def _golden_cases():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ggmlr_fd_cases.json")
    with open(path) as f:
        spec = json.load(f)
    out = []
    for c in spec["cases"]:
        if c.get("d") == "ones":
            continue
        out.append((c["name"], Shape(c["B"], c["H"], c["Hkv"], c["N"], c["M"], c["DK"], c["DV"]),
                    c["seed"], None if c["mask"] == "none" else c["mask"]))
    return out


P3_CASES = _golden_cases() + [
    # odd shapes that force slice padding, and a random mixed mask
    ("odd_pad", Shape(1, 2, 1, 3, 5, 3, 5), 41, None),
    ("odd_mixed_mask", Shape(1, 2, 1, 4, 6, 3, 5), 42, "random"),
]


def _mask_for(kind, N, M, seed):
    if kind is None:
        return None
    if kind == "causal":
        return causal_mask(N, M)
    return random_mask(N, M, seed, p_inf=0.25, full_rows=1, full_cols=1)


@pytest.mark.parametrize("name,shape,seed,mkind", P3_CASES, ids=[c[0] for c in P3_CASES])
def test_backward_matches_central_differences(name, shape, seed, mkind):
    q, k, v, d = make_qkvd(shape, seed)
    mask = _mask_for(mkind, shape.N, shape.M, seed)
    scale = 1.0 / math.sqrt(shape.DK)
    g = orc.backward(shape, q, k, v, mask, d, scale)
    for nm, an in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        fd = orc.num_grad(shape, q, k, v, mask, d, scale, nm, eps=1e-3)
        # the pages' tolerance, as testthat applies it, and as a max-relative bound
        assert r_all_equal_rel(fd, an) < 2e-2, nm
        assert rel_max(an, fd) < 2e-2, nm
        # f64 central differences are accurate to O(eps^2): a much tighter bound holds
        assert np.max(np.abs(an - fd)) < 1e-5, nm
        assert np.all(np.isfinite(an))


# ---------------------------------------------------------------- invariants

def test_dS_rows_sum_to_zero_via_identical_keys():
    # With every key equal to c, dQ_i = scale * (sum_j dS_ij) * c, which the row-sum
    # identity (sum_j P_ij (dP_ij - D_i) = 0) makes zero.
    s = Shape(1, 2, 1, 5, 7, 6, 4)
    q, k, v, d = make_qkvd(s, 5)
    k[:] = k[:, :, :1, :]
    mask = random_mask(s.N, s.M, 3, p_inf=0.3, full_rows=0, full_cols=0)
    g = orc.backward(s, q, k, v, mask, d, 0.7)
    assert np.max(np.abs(g["dq"])) < 1e-13
    # without identical keys dQ is clearly non-zero (so the test has teeth)
    q, k, v, d = make_qkvd(s, 5)
    assert np.max(np.abs(orc.backward(s, q, k, v, mask, d, 0.7)["dq"])) > 1e-3


def test_sum_of_dK_over_keys_is_zero():
    # A common shift of every key moves each row's scores by a constant, which the
    # softmax ignores; so the gradient summed over keys vanishes.
    s = Shape(2, 4, 2, 9, 11, 5, 3)
    q, k, v, d = make_qkvd(s, 6)
    mask = random_mask(s.N, s.M, 6, p_inf=0.2)
    g = orc.backward(s, q, k, v, mask, d, 0.45)
    assert np.max(np.abs(g["dk"].sum(axis=2))) < 1e-12
    assert np.max(np.abs(g["dk"])) > 1e-3


def test_unattended_key_gets_exactly_zero_gradient():
    s = Shape(1, 1, 1, 3, 4, 4, 4)
    q, k, v, d = make_qkvd(s, 12)
    mask = causal_mask(s.N, s.M)   # key 3 is seen by no query when N = 3
    g = orc.backward(s, q, k, v, mask, d, 0.5)
    assert np.all(g["dk"][0, 0, 3, :] == 0.0)
    assert np.all(g["dv"][0, 0, 3, :] == 0.0)
    assert np.all(np.abs(g["dk"][0, 0, :3, :]) > 0)


def test_all_masked_row_gives_zero_output_and_gradient():
    s = Shape(1, 2, 2, 5, 6, 3, 4)
    q, k, v, d = make_qkvd(s, 21)
    mask = np.zeros((s.N, s.M), dtype=np.uint16)
    mask[2, :] = F16_NEG_INF
    g = orc.backward(s, q, k, v, mask, d, 0.6)
    assert np.all(g["O"][0, 2] == 0.0)
    assert np.all(g["dq"][0, :, 2, :] == 0.0)
    assert np.all(np.isneginf(g["lse"][0, :, 2]))
    # the row contributes nothing to dK/dV: changing its upstream gradient changes nothing
    d2 = d.copy()
    d2[0, 2] = 123.0
    g2 = orc.backward(s, q, k, v, mask, d2, 0.6)
    assert np.array_equal(g2["dk"], g["dk"]) and np.array_equal(g2["dv"], g["dv"])
    # a fully -inf mask gives an all-zero result
    g3 = orc.backward(s, q, k, v, np.full_like(mask, F16_NEG_INF), d, 0.6)
    for key in ("dq", "dk", "dv", "O"):
        assert np.all(g3[key] == 0.0)


def test_D_equals_rowsum_dO_times_O():
    s = Shape(1, 2, 1, 6, 8, 4, 5)
    q, k, v, d = make_qkvd(s, 8)
    g = orc.backward(s, q, k, v, None, d, 0.5)
    D = np.einsum("bnhc,bnhc->bhn", d.astype(np.float64), g["O"])
    assert np.max(np.abs(D - g["D"])) < 1e-13


# ---------------------------------------------------------------- closed forms

def test_d_ones_gives_dV_equal_to_summed_attention():
    s = Shape(2, 4, 2, 5, 6, 3, 4)
    q, k, v, _ = make_qkvd(s, 32)
    mask = random_mask(s.N, s.M, 32, p_inf=0.2, full_rows=1, full_cols=0)
    d = np.ones(s.d_shape, dtype=np.float32)
    g = orc.backward(s, q, k, v, mask, d, 0.5)
    dv = g["dv"]
    # every dv component is the same number: sum of attention weights
    assert np.max(np.abs(dv - dv[..., :1])) < 1e-13
    # summed over keys, each live row contributes sum_m P = 1; rk2 heads per group
    live = np.array([np.any(mask[n] != F16_NEG_INF) for n in range(s.N)]).sum()
    rk2 = s.H // s.Hkv
    assert np.allclose(dv[..., 0].sum(axis=2), rk2 * live, rtol=0, atol=1e-12)


def test_single_key_closed_form():
    s = Shape(1, 4, 2, 3, 1, 5, 3)
    q, k, v, d = make_qkvd(s, 77)
    g = orc.backward(s, q, k, v, None, d, 0.9)
    rk2 = s.H // s.Hkv
    assert np.max(np.abs(g["dq"])) < 1e-15
    assert np.max(np.abs(g["dk"])) < 1e-15
    for gi in range(s.Hkv):
        expect = d[0, :, gi * rk2:(gi + 1) * rk2, :].astype(np.float64).sum(axis=(0, 1))
        assert np.allclose(g["dv"][0, gi, 0], expect, atol=1e-13)
        for h in range(gi * rk2, (gi + 1) * rk2):
            assert np.allclose(g["O"][0, :, h, :], v[0, gi, 0].astype(np.float64), atol=1e-15)


def test_zero_queries_give_uniform_attention_closed_form():
    s = Shape(1, 1, 1, 4, 6, 3, 5)
    q, k, v, d = make_qkvd(s, 9)
    q[:] = 0
    scale = 0.8
    g = orc.backward(s, q, k, v, None, d, scale)
    k64, v64, d64 = (x.astype(np.float64) for x in (k[0, 0], v[0, 0], d[0, :, 0]))
    M = s.M
    assert np.allclose(g["O"][0, :, 0], np.tile(v64.mean(axis=0), (s.N, 1)), atol=1e-14)
    assert np.allclose(g["dv"][0, 0], np.tile(d64.sum(axis=0) / M, (M, 1)), atol=1e-14)
    vbar = v64.mean(axis=0)
    for n in range(s.N):
        dS = (d64[n] @ v64.T - d64[n] @ vbar) / M
        assert np.allclose(g["dq"][0, 0, n], scale * dS @ k64, atol=1e-14)
    assert np.max(np.abs(g["dk"])) == 0.0


def test_lse_matches_direct_log_sum_exp():
    s = Shape(1, 2, 1, 4, 7, 5, 3)
    q, k, v, _ = make_qkvd(s, 17)
    mask = random_mask(s.N, s.M, 17, p_inf=0.3, full_rows=1, full_cols=0)
    scale = 0.6
    _, lse = orc.forward(s, q, k, v, mask, scale)
    mk = mask.view(np.float16).astype(np.float64)
    for h in range(s.H):
        S = scale * q[0, h].astype(np.float64) @ k[0, 0].astype(np.float64).T + mk
        with np.errstate(divide="ignore"):
            direct = np.log(np.sum(np.exp(S), axis=1))   # no max trick
        assert np.allclose(lse[0, h], direct, rtol=0, atol=1e-13, equal_nan=False) or \
            np.array_equal(np.isneginf(lse[0, h]), np.isneginf(direct))
        fin = np.isfinite(direct)
        assert np.allclose(lse[0, h][fin], direct[fin], atol=1e-13)
        assert np.array_equal(np.isneginf(lse[0, h]), ~fin)


# ---------------------------------------------------------------- structure

def test_gqa_equals_repeated_kv_mha():
    s = Shape(2, 6, 2, 5, 7, 4, 3)
    q, k, v, d = make_qkvd(s, 13)
    mask = random_mask(s.N, s.M, 13, p_inf=0.2)
    g = orc.backward(s, q, k, v, mask, d, 0.5)
    rk2 = s.H // s.Hkv
    s_mha = Shape(s.B, s.H, s.H, s.N, s.M, s.DK, s.DV)
    k_rep = np.repeat(k, rk2, axis=1)   # head h reads group h // rk2
    v_rep = np.repeat(v, rk2, axis=1)
    gm = orc.backward(s_mha, q, k_rep, v_rep, mask, d, 0.5)
    assert np.max(np.abs(g["dq"] - gm["dq"])) < 1e-14
    assert np.max(np.abs(g["O"] - gm["O"])) < 1e-14
    dk_sum = gm["dk"].reshape(s.B, s.Hkv, rk2, s.M, s.DK).sum(axis=2)
    dv_sum = gm["dv"].reshape(s.B, s.Hkv, rk2, s.M, s.DV).sum(axis=2)
    assert np.max(np.abs(g["dk"] - dk_sum)) < 1e-13
    assert np.max(np.abs(g["dv"] - dv_sum)) < 1e-13


def test_mask_row_shift_invariance():
    s = Shape(1, 2, 1, 4, 6, 3, 4)
    q, k, v, d = make_qkvd(s, 23)
    mask = random_mask(s.N, s.M, 23, p_inf=0.2, full_rows=0, full_cols=0)
    g = orc.backward(s, q, k, v, mask, d, 0.5)
    m2 = mask.view(np.float16).copy()
    fin = np.isfinite(m2[1])
    m2[1, fin] = (m2[1, fin].astype(np.float32) + np.float32(0.5)).astype(np.float16)
    # the shift must be exact in f16 for the identity to be exact
    assert np.array_equal(m2[1, fin].astype(np.float64),
                          mask.view(np.float16)[1, fin].astype(np.float64) + 0.5)
    g2 = orc.backward(s, q, k, v, m2.view(np.uint16), d, 0.5)
    for key in ("dq", "dk", "dv", "O"):
        assert np.max(np.abs(g[key] - g2[key])) < 1e-13


def test_masked_key_equals_deleted_key():
    s = Shape(1, 2, 1, 4, 6, 3, 4)
    q, k, v, d = make_qkvd(s, 29)
    mask = np.zeros((s.N, s.M), dtype=np.uint16)
    mask[:, 2] = F16_NEG_INF
    g = orc.backward(s, q, k, v, mask, d, 0.5)
    keep = [m for m in range(s.M) if m != 2]
    s2 = Shape(s.B, s.H, s.Hkv, s.N, s.M - 1, s.DK, s.DV)
    g2 = orc.backward(s2, q, np.ascontiguousarray(k[:, :, keep]), np.ascontiguousarray(v[:, :, keep]),
                      None, d, 0.5)
    assert np.max(np.abs(g["dq"] - g2["dq"])) < 1e-14
    assert np.max(np.abs(g["dk"][:, :, keep] - g2["dk"])) < 1e-14
    assert np.max(np.abs(g["dv"][:, :, keep] - g2["dv"])) < 1e-14
    assert np.all(g["dk"][:, :, 2] == 0) and np.all(g["dv"][:, :, 2] == 0)


def test_scale_is_applied_before_the_mask():
    # with scale 2 and mask value 1, the score is 2*q.k + 1, not 2*(q.k + 1)
    s = Shape(1, 1, 1, 1, 2, 1, 1)
    q = np.ones(s.q_shape, np.float32)
    k = np.array([0.0, 0.0], np.float32).reshape(s.k_shape)
    v = np.array([0.0, 1.0], np.float32).reshape(s.v_shape)
    mask = np.array([[0.0, 1.0]], np.float16).view(np.uint16)
    O, lse = orc.forward(s, q, k, v, mask, 2.0)
    p1 = math.exp(1.0) / (1.0 + math.exp(1.0))
    assert abs(O[0, 0, 0, 0] - p1) < 1e-15
    assert abs(lse[0, 0, 0] - math.log(1 + math.e)) < 1e-15


def test_against_torch_float64_autograd():
    torch = pytest.importorskip("torch")
    s = Shape(2, 4, 2, 19, 23, 7, 5)
    q, k, v, d = make_qkvd(s, 99)
    mask = random_mask(s.N, s.M, 99, p_inf=0.3, full_rows=0, full_cols=1)
    scale = 0.37
    g = orc.backward(s, q, k, v, mask, d, scale)
    rk2 = s.H // s.Hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    tm = torch.tensor(mask.view(np.float16).astype(np.float64))
    kr = tk.repeat_interleave(rk2, dim=1)
    vr = tv.repeat_interleave(rk2, dim=1)
    S = scale * torch.matmul(tq, kr.transpose(-1, -2)) + tm      # (B,H,N,M)
    P = torch.softmax(S, dim=-1)
    O = torch.matmul(P, vr)                                        # (B,H,N,DV)
    td = torch.tensor(d, dtype=torch.float64).permute(0, 2, 1, 3)  # (B,N,H,DV) -> (B,H,N,DV)
    (O * td).sum().backward()
    assert np.max(np.abs(tq.grad.numpy() - g["dq"])) < 1e-12
    assert np.max(np.abs(tk.grad.numpy() - g["dk"])) < 1e-12
    assert np.max(np.abs(tv.grad.numpy() - g["dv"])) < 1e-12
    assert np.max(np.abs(O.detach().permute(0, 2, 1, 3).numpy() - g["O"])) < 1e-13


# ---------------------------------------------------------------- packing

@pytest.mark.parametrize("shape", [Shape(2, 4, 2, 2, 4, 3, 5), Shape(1, 2, 1, 3, 5, 3, 5),
                                   Shape(1, 1, 1, 1, 1, 1, 1), Shape(3, 3, 1, 7, 5, 2, 3)])
def test_blob_layout_and_packing(shape):
    s = shape
    nq, nk, nv = s.DK * s.N * s.H * s.B, s.DK * s.M * s.Hkv * s.B, s.DV * s.M * s.Hkv * s.B
    pad = lambda n: int(math.ceil(n * 4 / 16) * 16 / 4)     # the ggmlR unpacker's pad()
    off = orc.blob_layout(s)
    assert off == (0, pad(nq), pad(nq) + pad(nk), pad(nq) + pad(nk) + pad(nv))
    assert all(o % 4 == 0 for o in off)
    assert nq <= off[1] and off[1] + nk <= off[2] and off[2] + nv <= off[3]
    q, k, v, d = make_qkvd(s, 31)
    g = orc.backward(s, q, k, v, None, d, 1 / math.sqrt(s.DK))
    blob = orc.pack(s, g["dq"], g["dk"], g["dv"])
    assert blob.size == off[3]
    assert np.array_equal(blob[:nq], g["dq"].ravel())
    assert np.array_equal(blob[off[1]:off[1] + nk], g["dk"].ravel())
    assert np.array_equal(blob[off[2]:off[2] + nv], g["dv"].ravel())
    assert np.all(blob[nq:off[1]] == 0) and np.all(blob[off[1] + nk:off[2]] == 0)
    assert np.all(blob[off[2] + nv:] == 0)


def test_padding_actually_fires_on_odd_shape():
    s = Shape(1, 2, 1, 3, 5, 3, 5)
    assert orc.blob_layout(s) == (0, 20, 36, 64)   # nq=18->20, nk=15->16, nv=25->28


# ---------------------------------------------------------------- sampled path

def test_sampled_backward_equals_full_backward():
    s = Shape(2, 4, 2, 37, 41, 6, 5)
    q, k, v, d = make_qkvd(s, 55)
    mask = random_mask(s.N, s.M, 55, p_inf=0.3, full_rows=2, full_cols=2)
    g = orc.backward(s, q, k, v, mask, d, 0.41)
    rng = np.random.default_rng(0)
    rows = rng.choice(s.B * s.H * s.N, 20, replace=False)
    keys = rng.choice(s.B * s.Hkv * s.M, 20, replace=False)
    dq, dk, dv = orc.backward_sampled(s, q, k, v, mask, d, 0.41, rows, keys)
    for i, r in enumerate(rows):
        n, h, b = r % s.N, (r // s.N) % s.H, r // (s.N * s.H)
        assert np.array_equal(dq[i], g["dq"][b, h, n])
    for i, r in enumerate(keys):
        m, gg, b = r % s.M, (r // s.M) % s.Hkv, r // (s.M * s.Hkv)
        assert np.max(np.abs(dk[i] - g["dk"][b, gg, m])) < 1e-14
        assert np.max(np.abs(dv[i] - g["dv"][b, gg, m])) < 1e-14


def test_empty_extents():
    # no keys: every row is all-masked -> zero output, zero dQ
    s = Shape(1, 2, 1, 3, 0, 4, 4)
    q, k, v, d = make_qkvd(s, 1)
    g = orc.backward(s, q, k, v, None, d, 0.5)
    assert np.all(g["dq"] == 0) and np.all(g["O"] == 0)
    # no queries: dK = dV = 0
    s = Shape(1, 2, 1, 0, 3, 4, 4)
    q, k, v, d = make_qkvd(s, 1)
    g = orc.backward(s, q, k, v, None, d, 0.5)
    assert np.all(g["dk"] == 0) and np.all(g["dv"] == 0)


def test_thread_count_does_not_change_the_result():
    s = Shape(1, 4, 2, 33, 29, 8, 6)
    q, k, v, d = make_qkvd(s, 3)
    a = orc.backward(s, q, k, v, None, d, 0.3, nthreads=1)
    b = orc.backward(s, q, k, v, None, d, 0.3, nthreads=7)
    for key in a:
        assert np.array_equal(a[key], b[key])


# ---------------------------------------------------------------- ALiBi (per-head linear bias)
# The ggmlR test file names ALiBi only through `max_bias`, in the block "the graph
# builder rejects attention features it cannot differentiate"; the reading taken here
# is a caller-given slope per query head and the bias slope_h * (m - n) added to the
# score after the scale, next to the mask.  The pins below restate that definition by
# routes that do not go through the oracle's ALiBi code.

def _alibi_mask_bits(slope, N, M, extra=None):
    """f16 bits of slope * (m - n) (+ extra, f16 bits or None): the bias as an additive mask."""
    n = np.arange(N)[:, None]
    m = np.arange(M)[None, :]
    bias = slope * (m - n).astype(np.float64)
    assert np.array_equal(bias.astype(np.float16).astype(np.float64), bias), "bias must be exact in f16"
    if extra is not None:
        e = extra.view(np.float16).astype(np.float64)
        bias = np.where(np.isneginf(e), -np.inf, bias + e)
        assert np.array_equal(bias.astype(np.float16).astype(np.float64), bias)
    return bias.astype(np.float16).view(np.uint16)


def test_alibi_single_head_equals_the_additive_mask_of_its_bias():
    # H = 1: the ALiBi bias slope * (m - n) is an additive mask, so the oracle with the
    # slope and no mask equals the oracle with that mask and no slope (exactly: every
    # bias value is an f16 number, and 0 is added in place of the other term)
    s = Shape(2, 1, 1, 7, 11, 5, 3)
    q, k, v, d = make_qkvd(s, 401)
    a = orc.backward(s, q, k, v, None, d, 0.6, alibi=[0.25])
    b = orc.backward(s, q, k, v, _alibi_mask_bits(0.25, s.N, s.M), d, 0.6)
    for name in ("dq", "dk", "dv", "O", "lse"):
        assert np.max(np.abs(a[name] - b[name])) <= 1e-13 * (1 + np.max(np.abs(b[name]))), name
    # with a causal mask on top: the bias and the mask add
    cm = causal_mask(s.N, s.M)
    a = orc.backward(s, q, k, v, cm, d, 0.6, alibi=[-0.5])
    b = orc.backward(s, q, k, v, _alibi_mask_bits(-0.5, s.N, s.M, cm), d, 0.6)
    for name in ("dq", "dk", "dv", "O", "lse"):
        assert np.max(np.abs(a[name] - b[name])) <= 1e-13 * (1 + np.max(np.abs(b[name]))), name


def test_alibi_slope_belongs_to_the_query_head():
    # grouped-query heads with different slopes: each query head h, run alone (H = 1,
    # its key/value head, its slope as a mask) gives the same O and dQ as in the
    # full problem; dK/dV of a group are the sums over its heads
    s = Shape(1, 4, 2, 6, 9, 4, 4)
    slopes = [0.5, -0.25, 0.125, 1.0]
    q, k, v, d = make_qkvd(s, 402)
    full = orc.backward(s, q, k, v, None, d, 0.5, alibi=slopes)
    rk2 = s.H // s.Hkv
    dk = np.zeros_like(full["dk"])
    dv = np.zeros_like(full["dv"])
    for h in range(s.H):
        g = h // rk2
        s1 = Shape(1, 1, 1, s.N, s.M, s.DK, s.DV)
        one = orc.backward(s1, q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1],
                           _alibi_mask_bits(slopes[h], s.N, s.M), d[:, :, h:h + 1], 0.5)
        assert np.max(np.abs(one["dq"][0, 0] - full["dq"][0, h])) <= 1e-13
        assert np.max(np.abs(one["O"][0, :, 0] - full["O"][0, :, h])) <= 1e-13
        dk[:, g] += one["dk"][:, 0]
        dv[:, g] += one["dv"][:, 0]
    assert np.max(np.abs(dk - full["dk"])) <= 1e-12
    assert np.max(np.abs(dv - full["dv"])) <= 1e-12


def test_alibi_uniform_scores_closed_form():
    # q = 0: the scores are the bias alone, slope * (m - n); the softmax of a row is that
    # of slope * m (the -n term is the same for every key of the row), so
    #   P[m] = exp(slope m) / sum exp(slope m'),  O_n = sum_m P[m] v_m for every n,
    #   LSE_n = log sum_m exp(slope (m - n)),  dV[:, m] = P[m] sum_n d_n
    s = Shape(1, 1, 1, 5, 8, 3, 4)
    _, k, v, d = make_qkvd(s, 403)
    q = np.zeros(s.q_shape, np.float32)
    slope = 0.75
    r = orc.backward(s, q, k, v, None, d, 0.9, alibi=[slope])
    m = np.arange(s.M)
    P = np.exp(slope * m) / np.exp(slope * m).sum()
    O = P @ v[0, 0].astype(np.float64)
    for n in range(s.N):
        assert np.allclose(r["O"][0, n, 0], O, rtol=0, atol=1e-14)
        assert abs(r["lse"][0, 0, n] - math.log(np.exp(slope * (m - n)).sum())) <= 1e-13
    dsum = d[0, :, 0].astype(np.float64).sum(axis=0)
    assert np.allclose(r["dv"][0, 0], P[:, None] * dsum[None, :], rtol=0, atol=1e-13)


@pytest.mark.parametrize("shape,seed,causal", [
    (Shape(1, 1, 1, 3, 5, 4, 4), 11, False),
    (Shape(1, 1, 1, 3, 4, 4, 4), 12, True),
    (Shape(2, 4, 2, 2, 3, 4, 4), 13, False),
], ids=["single_head", "causal", "gqa_batch"])
def test_alibi_backward_matches_central_differences(shape, seed, causal):
    # the ggmlR test's num_grad check (eps = 1e-3) of the backward against the forward,
    # with per-head slopes: the bias enters the gradient only through P
    s = shape
    q, k, v, d = make_qkvd(s, seed)
    mask = causal_mask(s.N, s.M) if causal else None
    slopes = [0.5 - 0.3 * h for h in range(s.H)]
    g = orc.backward(s, q, k, v, mask, d, 0.5, alibi=slopes)
    for name, an in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        fd = orc.num_grad(s, q, k, v, mask, d, 0.5, name, alibi=slopes)
        assert r_all_equal_rel(fd, an) <= 2e-2
        assert np.max(np.abs(an - fd)) <= 1e-6, name


def test_alibi_against_torch_float64_autograd():
    torch = pytest.importorskip("torch")
    s = Shape(2, 4, 2, 9, 13, 6, 5)
    q, k, v, d = make_qkvd(s, 404)
    mask = random_mask(s.N, s.M, 404, p_inf=0.2, full_rows=0, full_cols=1)
    slopes = np.array([0.3, -0.2, 0.05, 0.6])
    scale = 0.4
    g = orc.backward(s, q, k, v, mask, d, scale, alibi=slopes)
    rk2 = s.H // s.Hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    tm = torch.tensor(mask.view(np.float16).astype(np.float64))
    rel = torch.arange(s.M, dtype=torch.float64)[None, :] - torch.arange(s.N, dtype=torch.float64)[:, None]
    bias = torch.tensor(slopes)[:, None, None] * rel[None]                          # (H, N, M)
    S = scale * torch.matmul(tq, tk.repeat_interleave(rk2, 1).transpose(-1, -2)) + bias + tm
    O = torch.matmul(torch.softmax(S, -1), tv.repeat_interleave(rk2, 1))
    (O * torch.tensor(d, dtype=torch.float64).permute(0, 2, 1, 3)).sum().backward()
    assert np.max(np.abs(tq.grad.numpy() - g["dq"])) < 1e-12
    assert np.max(np.abs(tk.grad.numpy() - g["dk"])) < 1e-12
    assert np.max(np.abs(tv.grad.numpy() - g["dv"])) < 1e-12
