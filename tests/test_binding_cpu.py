"""CPU-side checks of the Python binding: every tensor it hands to the C ABI as a bare
pointer is checked first (dtype, shape, contiguity, extent, device), because the
library reads and writes exactly the extent the shape implies and cannot see a
wrong-sized buffer.  These checks run before any device work, so CPU tensors reach
them; a call whose tensors pass every check but live on the CPU is refused too."""
import pytest
import torch

import exact_attention_backward_fab_amd as fab

S = fab.Shape(1, 4, 2, 8, 12, 16, 16)


def inputs(dtype=torch.float32):
    q = torch.zeros(S.B, S.H, S.N, S.DK, dtype=dtype)
    k = torch.zeros(S.B, S.Hkv, S.M, S.DK, dtype=dtype)
    v = torch.zeros(S.B, S.Hkv, S.M, S.DV, dtype=dtype)
    d = torch.zeros(S.B, S.N, S.H, S.DV, dtype=dtype)
    return q, k, v, d


def good_o_lse():
    return torch.zeros(S.B, S.N, S.H, S.DV), torch.zeros(S.B, S.H, S.N)


def total():
    return fab.blob_layout(S)[3]


BAD = [
    ("mask_shape", dict(mask=torch.zeros(S.M, S.N, dtype=torch.int16)), ValueError, "mask"),
    ("mask_broadcast", dict(mask=torch.zeros(1, S.M, dtype=torch.int16).expand(S.N, S.M)), ValueError, "mask"),
    ("mask_dtype", dict(mask=torch.zeros(S.N, S.M, dtype=torch.float32)), TypeError, "mask"),
    ("o_shape", dict(O=torch.zeros(S.B, S.H, S.N, S.DV), lse=torch.zeros(S.B, S.H, S.N)), ValueError, "O"),
    ("o_dtype", dict(O=torch.zeros(S.B, S.N, S.H, S.DV, dtype=torch.float64), lse=torch.zeros(S.B, S.H, S.N)),
     TypeError, "O"),
    ("lse_shape", dict(O=torch.zeros(S.B, S.N, S.H, S.DV), lse=torch.zeros(S.B, S.N, S.H + 1)), ValueError, "lse"),
    ("o_without_lse", dict(O=torch.zeros(S.B, S.N, S.H, S.DV)), ValueError, "lse"),
    ("lse_without_o", dict(lse=torch.zeros(S.B, S.H, S.N)), ValueError, "lse"),
    ("blob_short", dict(blob=torch.zeros(16)), ValueError, "blob"),
    ("blob_dtype", dict(blob=torch.zeros(10_000, dtype=torch.float64)), TypeError, "blob"),
    ("blob16_short", dict(blob=torch.zeros(16, dtype=torch.bfloat16)), ValueError, "blob"),
    ("blob_dtype_arg", dict(blob_dtype=torch.int32), TypeError, "blob"),
    ("blob_dtype_mismatch", dict(blob=torch.zeros(10_000), blob_dtype=torch.bfloat16), TypeError, "blob"),
    ("blob_strided", dict(blob=torch.zeros(20_000)[::2]), ValueError, "blob"),
    ("ws_strided", dict(ws=torch.zeros(1 << 20, dtype=torch.uint8)[::2]), ValueError, "ws"),
    ("ws_short", dict(ws=torch.zeros(16, dtype=torch.uint8)), ValueError, "ws"),
    ("alibi_shape", dict(alibi=torch.zeros(S.H + 1)), ValueError, "alibi"),
    ("alibi_dtype", dict(alibi=torch.zeros(S.H, dtype=torch.float64)), TypeError, "alibi"),
    ("cpu_tensors", dict(), ValueError, "GPU"),
]


@pytest.mark.parametrize("name,kw,exc,word", BAD, ids=[b[0] for b in BAD])
def test_backward_checks_every_pointer_argument(name, kw, exc, word):
    q, k, v, d = inputs()
    with pytest.raises(exc) as e:
        fab.backward(q, k, v, d, 0.25, mode="bf16", **kw)
    assert word in str(e.value)


def test_forward_checks_its_outputs_and_mask():
    q, k, v, _ = inputs()
    with pytest.raises(ValueError, match="O"):
        fab.forward_lse(q, k, v, 0.25, O=torch.zeros(S.B, S.N, S.H, S.DV + 1))
    with pytest.raises(ValueError, match="lse"):
        fab.forward_lse(q, k, v, 0.25, lse=torch.zeros(S.B, S.H, S.N)[:, :, :-1])
    with pytest.raises(ValueError, match="mask"):
        fab.forward_lse(q, k, v, 0.25, mask=torch.zeros(S.N, S.M + 1, dtype=torch.int16))
    with pytest.raises(ValueError, match="GPU"):
        fab.forward_lse(q, k, v, 0.25)


def test_inputs_of_mixed_dtype_or_shape_are_refused():
    q, k, v, d = inputs()
    with pytest.raises(TypeError):
        fab.backward(q, k.double(), v, d, 0.25)
    with pytest.raises(TypeError):
        fab.backward(q.half(), k.half(), v.bfloat16(), d.half(), 0.25, mode="bf16")
    with pytest.raises(ValueError, match="d has shape"):
        fab.backward(q, k, v, d.transpose(1, 2).contiguous(), 0.25)
    with pytest.raises(ValueError, match="contiguous"):
        fab.backward(q.transpose(2, 3).contiguous().transpose(2, 3), k, v, d, 0.25)


def test_float16_inputs_pass_the_checks_and_set_the_flag():
    """float16 q, k, v, d are accepted (bf16 mode); the mode argument carries
    FAB_F16_INPUTS, bfloat16 inputs FAB_BF16_INPUTS; the call then stops at the device check."""
    q, k, v, d = (x.half() for x in inputs())
    with pytest.raises(ValueError, match="GPU"):
        fab.backward(q, k, v, d, 0.25, mode="bf16")
    assert fab._mode("bf16", False, torch.float16) == fab.FAB_MODE_BF16 | fab.FAB_F16_INPUTS
    assert fab._mode("bf16", True, torch.bfloat16) == fab.FAB_MODE_BF16 | fab.FAB_CAUSAL | fab.FAB_BF16_INPUTS
    assert fab._mode("f32", False, torch.float32) == fab.FAB_MODE_F32


def test_autograd_refuses_float16_inputs():
    from exact_attention_backward_fab_amd.autograd import attention
    q, k, v, _ = inputs(torch.float16)
    with pytest.raises(TypeError, match="float16"):
        attention(q, k, v, mode="bf16")
