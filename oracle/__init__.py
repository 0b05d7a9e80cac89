"""CPU oracle for MoE token layout, dispatch and combine (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its binding) never
does; it shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, gcc -O2 -ffp-contract=off);
this module builds it with gcc if needed and wraps it with ctypes and NumPy.
"""
from .oracle import (  # noqa: F401
    build_oracle, lib_path, ceil_div, round_up4, num_max_pretrain,
    num_max_infer, validate_num_max, check_capacity, layout, dispatch,
    dispatch_rows, combine, combine_tokens, f32_to_bf16, run_pipeline,
    combine_backward, dispatch_backward, topk_from_routing_map, dispatch_scaled,
    grouped_gemm, grouped_gemm_at, f64_to_bf16, run_layer,
)
