"""Switch-Transformer MoE layer forward on MI355X (gfx950): HIP kernels behind a C ABI.

The layer: fp32 router, softmax, top-1 argmax (top-k option, lowest index
wins ties), capacity with overflow dropped to the residual path, expert-major
dispatch, grouped-GEMM expert FFN (ReLU or SwiGLU), gate-scaled combine and
the auxiliary load-balancing loss.  Entry points mirror include/moe.h.
"""
from .api import (ForwardPlan, capacity, combine, combine_backward, dispatch, dispatch_backward,  # noqa: F401
                  dispatch_priority, dispatch_reroute, expert_ffn, expert_ffn_backward, forward, forward_policy,
                  router,
                  router_backward, router_noalloc, workspace_bytes)
from ._lib import MoEError, LIB_PATH  # noqa: F401
