"""The matrix-core measurement hook on the GPU: a loop of dense bf16 products reports
a rate below the published dense peak (2.5 PFLOP/s) and a plausible shader clock."""
import pytest
import torch

import exact_attention_backward_fab_amd as fab


@pytest.mark.gpu
def test_mfma_loop_rate_and_clock_are_plausible():
    tf, ghz = fab.measure_mfma_loop(iters=2000)
    print(f"[probe] mfma loop {tf:.1f} TFLOP/s at {ghz:.2f} GHz", flush=True)
    assert 200.0 < tf < 2600.0
    assert 0.5 < ghz < 3.0
    # the rate follows the clock: at most 1024 flops per cycle per SIMD on 1024 SIMDs
    assert tf <= 1024 * 1024 * ghz * 1e9 / 1e12 * 1.05
