"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package only draws random numbers and stores them in the dtypes the kernels read
(float32, bfloat16 bit patterns, OCP fp8 E4M3FN bytes).  It holds none of the attention
method's arithmetic: no metadata, no scores, no selection, no softmax.
"""
from .encode import f64_to_bf16_bits, f64_to_e4m3fn_bytes  # noqa: F401
from .workloads import (WORKLOADS, Workload, make_inputs, stream_inputs, query_inputs,  # noqa: F401
                        rerange_buffer, score_rows)
