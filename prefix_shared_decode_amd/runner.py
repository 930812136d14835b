"""Device-memory plumbing around one plan: workspace allocation and upload.

``DecodeStep`` owns a plan and a torch uint8 workspace on the current GPU;
calling it launches the fused kernel on the current (or given) stream.
"""

from __future__ import annotations

from . import _lib


class DecodeStep:
    def __init__(self, cfg, batch, stream=None, **plan_opts):
        import torch

        self.plan = _lib.psa_build_plan(cfg, batch, **plan_opts)
        self.info = self.plan.info()
        nbytes = max(int(self.info["workspace_bytes"]), 256)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        _lib.psa_plan_upload(self.plan, self.workspace, stream)
        # the plan's pinned staging buffer must outlive the copy
        (stream or torch.cuda.current_stream()).synchronize()

    def __call__(self, q, k_pool, v_pool, out, out_m=None, out_l=None, stream=None):
        _lib.psa_decode_attention(self.plan, q, k_pool, v_pool, out, self.workspace, out_m, out_l, stream)
