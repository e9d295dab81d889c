"""Seeded synthetic inputs for the CSA / HCA attention path.

This package only draws random numbers and stores them in the storage
formats the path consumes (fp32, bf16 bit patterns, FP4 E2M1 codes with
fp32 or E8M0 block scales).  It holds none of the method's arithmetic: no pooling,
no scoring, no selection, no attention.  Both the CPU oracle (``oracle/``)
and the GPU library's tests / benchmark take their inputs from here.
"""
from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
from .generate import (  # noqa: F401
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    fp4_quantize,
    make_inputs,
    make_swa_inputs,
    mx4_quantize,
    SWA_DECODE,
)
