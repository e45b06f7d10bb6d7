"""GPU parity sweep: seeded random configurations against the full f64 oracle.

Each case draws, from one seeded generator, a shape (batch, grouped-query ratio,
ragged N and M down to 1, head dims 1..256 with tile edges such as 31/32/33,
127/128/129 and 191/192/193 favoured, DK != DV), a mask (none, random with
all-masked rows and key columns, the causal rule as a tensor or as FAB_CAUSAL, a
padding mask), the mode and, where the mode allows, the storage options (16-bit
q, k, v, d; O and LSE supplied, with O as bf16; a bf16 or f16 result blob) and
ALiBi slopes.  Every element of dQ, dK and dV is compared with the oracle on the
values the library actually read (16-bit inputs widened): max|gpu - oracle| /
max|oracle| within 1e-4 (f32 mode) or 2e-2 (bf16 mode), the zeros that structure
fixes (all-masked query rows, keys no query sees) exact, the blob's pads zero and
nothing written past its end.
"""
import math

import numpy as np
import pytest

from fab_inputs import Shape, make_qkvd, random_mask, causal_mask, F16_NEG_INF

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
EDGE_DIMS = [1, 2, 3, 4, 5, 8, 16, 31, 32, 33, 40, 63, 64, 65, 72, 96, 127, 128, 129, 160, 191, 192, 193, 200,
             255, 256]
N_CASES = 96


def draw_cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.choice([1, 1, 2]))
        Hkv = int(rng.choice([1, 2, 3]))
        H = Hkv * int(rng.choice([1, 2, 4]))
        ext = lambda: int(rng.choice([1, int(rng.integers(2, 80)), int(rng.integers(80, 260)),
                                      int(rng.integers(260, 700))], p=[0.08, 0.32, 0.45, 0.15]))
        N, M = ext(), ext()
        DK = int(rng.choice(EDGE_DIMS)) if rng.random() < 0.7 else int(rng.integers(1, 257))
        DV = DK if rng.random() < 0.5 else int(rng.choice(EDGE_DIMS))
        mkind = str(rng.choice(["none", "random", "causal", "causal_flag", "padding"]))
        mode = "bf16" if rng.random() < 0.6 else "f32"
        alibi = bool(rng.random() < 0.3)
        inputs, supplied, o16, blob = "f32", bool(rng.random() < 0.4), False, "f32"
        if mode == "bf16":
            inputs = str(rng.choice(["f32", "f32", "bf16", "f16"]))
            o16 = supplied and bool(rng.random() < 0.5)
            blob = str(rng.choice(["f32", "f32", "bf16", "f16"]))
        cases.append((f"c{i:02d}", Shape(B, H, Hkv, N, M, DK, DV), mkind, 500 + i, mode, inputs, supplied, o16,
                      blob, alibi))
    return cases


CASES = draw_cases(N_CASES)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    return torch, torch.device("cuda:0")


def to_dev(torch, dev, a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def mask_of(kind, s, seed):
    if kind in ("none", "causal_flag"):
        return None
    if kind == "causal":
        return causal_mask(s.N, s.M)
    if kind == "padding":
        m = np.zeros((s.N, s.M), np.uint16)
        m[:, (3 * s.M) // 4 + 1:] = F16_NEG_INF
        m[::5, :] = F16_NEG_INF
        return m
    return random_mask(s.N, s.M, seed, p_inf=0.3, full_rows=1, full_cols=2)


@pytest.mark.parametrize("name,s,mkind,seed,mode,inputs,supplied,o16,blob,alibi", CASES, ids=[c[0] for c in CASES])
def test_random_configuration_against_full_oracle(torch_dev, name, s, mkind, seed, mode, inputs, supplied, o16,
                                                  blob, alibi):
    run_case(torch_dev, name, s, mkind, seed, mode, inputs, supplied, o16, blob, alibi)


SHARED = CASES[::4]


@pytest.fixture(scope="module")
def dirty_workspace(torch_dev):
    """One workspace for every case below, large enough for each, all bytes 0xFF (NaN
    patterns) at the start and left as each call leaves it for the next."""
    torch, dev = torch_dev
    import exact_attention_backward_fab_amd as fab
    need = max(fab.workspace_bytes(fab.Shape(*c[1].astuple()), c[4], c[2] not in ("none", "causal_flag"), c[6],
                                   c[2] == "causal_flag") for c in SHARED)
    return torch.full((need + 256,), 255, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("name,s,mkind,seed,mode,inputs,supplied,o16,blob,alibi", SHARED, ids=[c[0] for c in SHARED])
def test_random_configuration_in_a_shared_dirty_workspace(torch_dev, dirty_workspace, name, s, mkind, seed, mode,
                                                          inputs, supplied, o16, blob, alibi):
    # every call writes each workspace byte it reads: a workspace that an earlier call of
    # another shape (or the initial NaN fill) left behind changes nothing
    run_case(torch_dev, name, s, mkind, seed, mode, inputs, supplied, o16, blob, alibi, ws=dirty_workspace)


def run_case(torch_dev, name, s, mkind, seed, mode, inputs, supplied, o16, blob, alibi, ws=None):
    torch, dev = torch_dev
    import exact_attention_backward_fab_amd as fab
    from oracle import oracle as orc
    print(f"[sweep] {name} {s} mask={mkind} mode={mode} inputs={inputs} supplied={supplied} o16={o16} "
          f"blob={blob} alibi={alibi} shared_ws={ws is not None}", flush=True)
    q, k, v, d = make_qkvd(s, seed)
    mask = mask_of(mkind, s, seed)
    causal = mkind == "causal_flag"
    scale = float(np.float32(1.0 / math.sqrt(s.DK)))
    slopes = (np.array([2.0 ** (-4.0 * (h + 1) / s.H) for h in range(s.H)], np.float32) if alibi else None)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    t = [to_dev(torch, dev, x).to(dt[inputs]) for x in (q, k, v, d)]
    tm = to_dev(torch, dev, mask)
    ta = to_dev(torch, dev, slopes)
    O = lse = None
    if supplied:
        O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode=mode, causal=causal, alibi=ta, o_bf16=o16)
    fs = fab.Shape(*s.astuple())
    bdt = dt[blob]
    _, off_k, off_v, total = fab.blob_layout(fs, bdt)
    # the blob and a guard band after it, every element a NaN pattern the kernels never write
    sentinel = 0x7FC0DEAD if blob == "f32" else 0x7FC1
    raw = torch.full((total + 64,), sentinel, dtype=torch.int32 if blob == "f32" else torch.int16, device=dev)
    out = raw.view(bdt)
    fab.backward(*t, scale, mask=tm, mode=mode, O=O, lse=lse, causal=causal, alibi=ta, blob=out, ws=ws)
    torch.cuda.synchronize()
    bits = raw.cpu().numpy()
    assert np.all(bits[total:] == sentinel), f"{name}: write past the end of the blob"
    got = out[:total].float().cpu().numpy().astype(np.float64)
    nq, nk, nv = q.size, k.size, v.size
    assert np.all(bits[nq:off_k] == 0) and np.all(bits[off_k + nk:off_v] == 0) and \
        np.all(bits[off_v + nv:total] == 0), f"{name}: pads not zero"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"

    # the oracle on the values the library read: 16-bit inputs widened exactly
    qr, kr, vr, dr = (x.float().cpu().numpy() for x in t)
    omask = causal_mask(s.N, s.M) if causal else mask
    kw = {"alibi": slopes.astype(np.float64)} if alibi else {}
    ref = orc.backward(s, qr, kr, vr, omask, dr, scale, **kw)
    scale_all = max(float(np.max(np.abs(ref[n]))) if ref[n].size else 0.0 for n in ("dq", "dk", "dv"))
    dead_rows = np.zeros(s.N, bool)
    dead_keys = np.zeros(s.M, bool)
    if omask is not None:
        inf = omask == F16_NEG_INF
        dead_rows, dead_keys = inf.all(axis=1), inf.all(axis=0)
    errs = {}
    for nm, lo, n in (("dq", 0, nq), ("dk", off_k, nk), ("dv", off_v, nv)):
        r = ref[nm]
        g = got[lo:lo + n].reshape(r.shape)
        den = float(np.max(np.abs(r))) if r.size and np.max(np.abs(r)) > 0 else scale_all
        errs[nm] = float(np.max(np.abs(g - r)) / den) if r.size and den > 0 else float(np.max(np.abs(g - r), initial=0))
        z = g[:, :, dead_rows, :] if nm == "dq" else g[:, :, dead_keys, :]
        assert np.all(z == 0), f"{name}: {nm} non-zero where it is zero by structure"
    print(f"  max-rel {errs}", flush=True)
    for nm, e in errs.items():
        assert e <= TOL[mode], f"{name}: {nm} max-rel error {e:.3e} > {TOL[mode]} ({errs})"
