"""Plant mistakes in copies of the oracle source and check that the pins catch them.

Each mutant is a one-line change to oracle/fab_oracle.c of the kind the pins are
meant to catch: a wrong sign or a dropped term in dS (labml "Flash Attention",
section "Backward pass"), a wrong grouped-query head map or the mask added before
the scale (ggmlR test file's `attn_ref`), a missing scale, a transposed layout, and
for the ALiBi bias a flipped sign, the key/value head's slope in place of the query
head's, and the bias added before the scale.
The unmodified source must pass the same checks.
"""
import math
import os
import subprocess

import numpy as np
import pytest

from fab_inputs import Shape, make_qkvd, random_mask
from oracle import oracle as orc

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "fab_oracle.c")

MUTANTS = {
    "none": None,
    "dS_sign": ("double dS = P * (dP - j->D[row]);", "double dS = P * (dP + j->D[row]);"),
    "dS_drop_D": ("double dS = pbuf[m] * (dpbuf[m] - D);", "double dS = pbuf[m] * dpbuf[m];"),
    "head_map": ("int64_t g = h / (s->H / s->Hkv);", "int64_t g = h % s->Hkv;"),
    # the mask added before the scale: scale * (q.k + mask)
    "mask_before_scale": ("        acc += fab_oracle_half_to_double(mask[m + s->M * n]);\n    return acc;",
                          "        acc += scale * fab_oracle_half_to_double(mask[m + s->M * n]);\n    return acc;"),
    "dk_no_scale": ("kacc[i] += j->scale * dS * qr[i];", "kacc[i] += dS * qr[i];"),
    "d_layout": ("{ return dv + s->DV * (h + s->H * (n + s->N * b)); }",
                 "{ return dv + s->DV * (n + s->N * (h + s->H * b)); }"),
    "mask_transposed": ("mask[m + s->M * n]", "mask[n + s->N * m]"),
    # ALiBi: the bias of query n at key m is slope_h * (m - n), after the scale
    "alibi_sign": ("acc += alibi[h] * (double)(m - n);", "acc += alibi[h] * (double)(n - m);"),
    "alibi_head_is_kv_head": ("acc += alibi[h] * (double)(m - n);", "acc += alibi[g] * (double)(m - n);"),
    "alibi_before_scale": ("    acc *= scale;\n    if (alibi)\n        acc += alibi[h] * (double)(m - n);",
                           "    if (alibi)\n        acc += alibi[h] * (double)(m - n);\n    acc *= scale;"),
}


def _build(tmp_path, name, mut):
    src = open(SRC).read()
    if mut is not None:
        old, new = mut
        assert src.count(old) >= 1, name
        src = src.replace(old, new)
    c = tmp_path / f"m_{name}.c"
    so = tmp_path / f"m_{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-pthread", "-o", str(so), str(c),
                    "-lm"], check=True)
    return str(so)


def _pins_pass():
    """A compact subset of the pins: central differences and the torch f64 cross-check."""
    torch = pytest.importorskip("torch")
    s = Shape(1, 4, 2, 3, 5, 3, 4)          # N != M and DK != DV so layout slips show
    q, k, v, d = make_qkvd(s, 101)
    mask = random_mask(s.N, s.M, 101, p_inf=0.2, full_rows=0, full_cols=0)
    mask[0, :] = np.float16(0.5).view(np.uint16)   # finite, non-zero mask entries
    mask[0, 0] = np.float16(-1.25).view(np.uint16)
    scale = 0.7
    try:
        g = orc.backward(s, q, k, v, mask, d, scale)
    except AssertionError:
        return False
    for nm, an in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        fd = orc.num_grad(s, q, k, v, mask, d, scale, nm)
        if np.max(np.abs(an - fd)) > 1e-5:
            return False
    slopes = np.array([0.3, -0.2, 0.05, 0.6])
    ga = orc.backward(s, q, k, v, mask, d, scale, alibi=slopes)
    rk2 = s.H // s.Hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    tm = torch.tensor(mask.view(np.float16).astype(np.float64))
    S = scale * torch.matmul(tq, tk.repeat_interleave(rk2, 1).transpose(-1, -2)) + tm
    O = torch.matmul(torch.softmax(S, -1), tv.repeat_interleave(rk2, 1))
    (O * torch.tensor(d, dtype=torch.float64).permute(0, 2, 1, 3)).sum().backward()
    ok = (np.max(np.abs(tq.grad.numpy() - g["dq"])) < 1e-12 and
          np.max(np.abs(tk.grad.numpy() - g["dk"])) < 1e-12 and
          np.max(np.abs(tv.grad.numpy() - g["dv"])) < 1e-12)
    # the same with per-head ALiBi slopes (bias slope_h * (m - n) after the scale)
    tq.grad = tk.grad = tv.grad = None
    rel = torch.arange(s.M, dtype=torch.float64)[None, :] - torch.arange(s.N, dtype=torch.float64)[:, None]
    S = scale * torch.matmul(tq, tk.repeat_interleave(rk2, 1).transpose(-1, -2)) + \
        torch.tensor(slopes)[:, None, None] * rel[None] + tm
    O = torch.matmul(torch.softmax(S, -1), tv.repeat_interleave(rk2, 1))
    (O * torch.tensor(d, dtype=torch.float64).permute(0, 2, 1, 3)).sum().backward()
    return ok and (np.max(np.abs(tq.grad.numpy() - ga["dq"])) < 1e-12 and
                   np.max(np.abs(tk.grad.numpy() - ga["dk"])) < 1e-12 and
                   np.max(np.abs(tv.grad.numpy() - ga["dv"])) < 1e-12)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    so = _build(tmp_path, name, MUTANTS[name])
    prev = orc.use_library(so)
    try:
        ok = _pins_pass()
    finally:
        orc.restore_library(prev)
    if name == "none":
        assert ok, "the unmodified oracle must pass"
    else:
        assert not ok, f"planted mistake {name} went unnoticed"
