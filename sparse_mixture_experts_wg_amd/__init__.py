"""Mixtral sparse mixture-of-experts feed-forward layer on MI355X (gfx950).

The layer (Mixtral of Experts pages): router logits x . W_g over E experts, the
top-2 experts per token with a softmax over their two logits, and
y = sum_k w_k * W2_k(silu(W1_k x) * (W3_k x)). It runs as hand-written HIP
kernels in libmoe.so behind the C ABI of include/moe.h; this package is the
Python binding (torch tensors in, torch tensors out).
"""
from .binding import (  # noqa: F401
    BF16, F32, FLAG_DOWN_PARTIALS, NOALLOC_SCRATCH_BYTES, PATH_AUTO, PATH_STREAM, PATH_TILED,
    MoeError, Problem, block_forward, block_workspace_bytes, capacity_rows, combine,
    combine_residual, down_parts, expert_down, expert_gate_up, expert_gate_up_rows,
    expert_swiglu, expert_workspace_bytes, forward, forward_noalloc, forward_workspace_bytes,
    header_functions, last_error, lib, permute, problem, resolve_path, rmsnorm, route,
    status_string,
)

__all__ = [
    "Problem", "problem", "route", "permute", "expert_gate_up", "expert_gate_up_rows", "expert_down", "expert_swiglu",
    "combine", "forward", "forward_noalloc", "expert_workspace_bytes", "forward_workspace_bytes", "resolve_path",
    "down_parts", "capacity_rows", "rmsnorm", "combine_residual", "block_forward", "block_workspace_bytes",
    "MoeError", "status_string", "last_error", "header_functions",
]
