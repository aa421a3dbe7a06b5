"""CPU oracle for the dropless MoE expert-MLP layer (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product path (the HIP library and its binding) never touches it.
"""
from .oracle import (  # noqa: F401
    build,
    capacity_plan,
    layer_bwd,
    layer_fwd,
    layer_fwd_mxfp8,
    dx_weights_mxfp8,
    dx_mxfp8,
    lib_path,
    mx_scale_cols,
    pairs_from_plan,
    pairs_from_topk,
    router_bwd,
    router_logits,
    permute,
    quantize_mxfp8,
    route_topk,
    set_threads,
    threads,
    token_round,
)
