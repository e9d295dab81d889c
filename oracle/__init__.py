"""CPU oracle for Compressed Sparse Attention (CSA) and its HCA variant.

TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library imports, links or runs
this package; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
kernels.  See ``csa_oracle.py`` for the definitions and their sources.
"""
from .csa_oracle import (  # noqa: F401
    NEG_INF,
    append_block,
    attend,
    csa_reference,
    e2m1_scaled_to_e4m3,
    e2m1_to_e4m3,
    e2m1_value,
    e4m3_value,
    e8m0_value,
    fp4_dequantize,
    from_bf16_bits,
    hca_attend,
    swa_attend,
    index_scores,
    merge_attention,
    mx4_dequantize,
    mx4_quantize,
    pool,
    round_to_bf16,
    topk_select,
    visible_count,
)
