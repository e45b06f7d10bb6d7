"""fab_backward_noalloc (the allocation-free variant of fab_backward) through the
C ABI: two calls in a row on the library's one scratch array, the second with a
smaller input, each equal to fab_backward with a caller workspace (bit for bit in
bf16 mode, whose kernels sum in a fixed order; up to the order of the dQ atomics in
f32 mode) and within the parity bar of the oracle."""
import math

import numpy as np
import pytest

from fab_inputs import Shape, make_qkvd, random_mask, causal_mask

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = [
    # (shape, mask kind, seed): the larger first, then a smaller one on the same array
    (Shape(2, 8, 4, 700, 900, 64, 64), "random", 201),
    (Shape(1, 4, 2, 150, 170, 128, 128), "causal", 202),
]


def _mask(kind, s, seed):
    return causal_mask(s.N, s.M) if kind == "causal" else random_mask(s.N, s.M, seed, p_inf=0.3, full_rows=2,
                                                                       full_cols=2)


@pytest.mark.parametrize("supplied", [False, True], ids=["own_forward", "o_lse_supplied"])
@pytest.mark.parametrize("mode", ["bf16", "f32"])
def test_noalloc_matches_backward_on_two_calls(mode, supplied):
    import torch
    import exact_attention_backward_fab_amd as fab
    from oracle import oracle as orc
    dev = torch.device("cuda:0")
    for s, kind, seed in CASES:
        print(f"[noalloc] {mode} supplied={supplied} {s}", flush=True)
        q, k, v, d = make_qkvd(s, seed)
        mask = _mask(kind, s, seed)
        scale = float(np.float32(1 / math.sqrt(s.DK)))
        t = [torch.from_numpy(x).to(dev) for x in (q, k, v, d)]
        tm = torch.from_numpy(mask.view(np.int16)).to(dev)
        fs = fab.Shape(*s.astuple())
        assert fab.workspace_bytes(fs, mode, True, supplied) <= fab.NOALLOC_SCRATCH_BYTES
        O = lse = None
        if supplied:
            O, lse = fab.forward_lse(t[0], t[1], t[2], scale, mask=tm, mode=mode)
        total = fab.blob_layout(fs)[3]
        blob = torch.full((total + 64,), float("nan"), device=dev)
        fab.backward_noalloc(*t, scale, blob[:total], mask=tm, mode=mode, O=O, lse=lse)
        ref_blob = fab.backward(*t, scale, mask=tm, mode=mode, O=O, lse=lse)
        torch.cuda.synchronize()
        got = blob.cpu().numpy()
        assert np.all(np.isnan(got[total:])), "write past the end of the blob"
        got = got[:total]
        want = ref_blob.cpu().numpy()[:total]
        if mode == "bf16":
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        else:
            assert np.max(np.abs(got - want)) <= 1e-5 * np.max(np.abs(want))
        ref = orc.backward(s, q, k, v, mask, d, scale)
        _, off_k, off_v, _ = fab.blob_layout(fs)
        for name, lo in (("dq", 0), ("dk", off_k), ("dv", off_v)):
            n = ref[name].size
            e = np.max(np.abs(got[lo:lo + n] - ref[name].ravel())) / np.max(np.abs(ref[name]))
            assert e <= TOL[mode], (name, e)


def test_noalloc_refuses_a_shape_beyond_its_array():
    import torch
    import exact_attention_backward_fab_amd as fab
    dev = torch.device("cuda:0")
    s = Shape(1, 32, 8, 2048, 2048, 128, 128)
    assert fab.workspace_bytes(fab.Shape(*s.astuple()), "bf16", True, True) > fab.NOALLOC_SCRATCH_BYTES
    t = [torch.zeros(sh, device=dev) for sh in (s.q_shape, s.k_shape, s.v_shape, s.d_shape)]
    blob = torch.zeros(fab.blob_layout(fab.Shape(*s.astuple()))[3], device=dev)
    with pytest.raises(fab.FabError) as e:
        fab.backward_noalloc(*t, 0.1, blob, causal=True, mode="bf16")
    assert e.value.code == fab.FAB_E_UNSUPPORTED and "scratch" in str(e.value)
