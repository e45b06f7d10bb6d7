"""f64 CPU oracle for the exact attention backward.

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline leg may import anything from this package.  It shares no code with the
HIP library under exact_attention_backward_fab_amd/.
"""
