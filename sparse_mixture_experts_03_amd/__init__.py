"""MI355X (gfx950) sparse Mixture-of-Experts layer forward.

The layer runs in the HIP kernels of libmoe_mi355x.so (C ABI: include/moe.h);
this package only marshals torch tensors into that ABI.  `MoELayerForward`
allocates outputs and workspace with torch and calls `moe_forward`.
"""
from . import binding
from .binding import (ACT_GELU, ACT_SILU, ACT_SWIGLU, BF16, CAPACITY_DROP, CAPACITY_REROUTE, F32, GEMM_AUTO, GEMM_STREAMING, GEMM_TILED, INT4_G128,
                      MoeConfig, MoeError, config,
                      moe_combine, moe_forward, moe_forward_no_alloc, moe_grouped_gemm, moe_permute, moe_router, moe_router_encoder,
                      moe_router_stats,
                      moe_router_stats_workspace_size, moe_router_workspace_size, moe_workspace_size)

__all__ = ["binding", "BF16", "F32", "INT4_G128", "GEMM_AUTO", "GEMM_STREAMING", "GEMM_TILED", "CAPACITY_DROP",
           "CAPACITY_REROUTE", "ACT_GELU", "ACT_SILU", "ACT_SWIGLU", "MoeConfig",
           "MoeError", "config", "moe_forward", "moe_forward_no_alloc", "moe_router", "moe_permute", "moe_grouped_gemm", "moe_combine",
           "moe_workspace_size", "moe_router_workspace_size", "moe_router_stats", "moe_router_stats_workspace_size",
           "moe_router_encoder",
           "MoELayerForward"]


class MoELayerForward:
    """Holds the output and workspace buffers for one layer configuration and
    runs the whole forward pass on the current stream.  Inputs must already be
    device tensors in the layouts of include/moe.h."""

    def __init__(self, cfg, device="cuda"):
        import torch
        self.cfg = cfg
        act = torch.float32 if cfg.act_dtype == F32 else torch.bfloat16
        self.y = torch.empty((cfg.T, cfg.d), dtype=act, device=device)
        self.expert_ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=device)
        self.gate_weights = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=device)
        self.counts = torch.empty((cfg.E,), dtype=torch.int32, device=device)
        nbytes = moe_workspace_size(cfg)
        self.workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)

    def __call__(self, x, Wg, bias, W1, W2, W1_scales=None, W2_scales=None, stream=None, W_in=None, b_in=None):
        moe_forward(self.cfg, x, Wg, bias, W1, W1_scales, W2, W2_scales, self.y, self.expert_ids,
                    self.gate_weights, self.counts, self.workspace, stream=stream, W_in=W_in, b_in=b_in)
        return self.y, self.expert_ids, self.gate_weights, self.counts
