"""Device-side plumbing for one expert-projection workload.

Uploads a synthetic problem's arrays to device memory, allocates the outputs
and the workspace, and runs the hot path through the C ABI: route/group, the
expert projection and (where the workload has one) the gate-weighted combine.
No arithmetic happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def _bf16_tensor(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


class DeviceProblem:
    """A synthetic MoEProblem resident in device memory, with its output buffers."""

    def __init__(self, p, device="cuda:0", path=B.MXFP4_PATH_AUTO):
        self.p = p
        self.device = torch.device(device)
        self.path = path
        dev = self.device
        self.blocks = torch.from_numpy(np.ascontiguousarray(p.blocks)).to(dev)
        self.scales = torch.from_numpy(np.ascontiguousarray(p.scales)).to(dev)
        self.bias = _bf16_tensor(p.bias, dev)
        self.x = _bf16_tensor(p.x, dev)
        self.logits = _bf16_tensor(p.logits, dev) if p.logits is not None else None
        self.ids_in = torch.from_numpy(np.ascontiguousarray(p.ids_in, dtype=np.int32)).to(dev) if p.ids_in is not None else None
        T, k, N, E = p.T, p.k, p.N, p.E
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=dev) if p.logits is not None else None
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        self.sorted_rows = torch.empty((T * k,), dtype=torch.int32, device=dev)
        self.error_word = torch.zeros((1,), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, k, N), dtype=torch.float32, device=dev)
        # the gated activation of a gate/up projection (even N): bf16 [T, k, N / 2]
        self.act = torch.zeros((T, k, N // 2), dtype=torch.bfloat16, device=dev) if N % 2 == 0 else None
        self.y = torch.empty((T, N), dtype=torch.float32, device=dev) if (p.combine and self.gates is not None) else None
        self.set_path(path)

    def set_path(self, path):
        self.path = path
        p = self.p
        nbytes = B.mxfp4_expert_proj_workspace_size(p.E, p.N, p.T, p.k, p.K, p.x_per_slot, path)
        self.workspace = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=self.device) if nbytes else None

    def route_group(self, stream=None):
        p = self.p
        B.mxfp4_moe_route_group(self.logits, self.ids_in, p.T, p.E, p.k, self.topk_ids, self.gates, self.offsets,
                                self.sorted_rows, self.error_word, stream)

    def expert_proj(self, stream=None, blocks=None, scales=None):
        p = self.p
        B.mxfp4_expert_proj(self.blocks if blocks is None else blocks, self.scales if scales is None else scales,
                            self.bias, p.E, p.N, p.K, self.x, p.x_per_slot, p.T, p.k, self.offsets,
                            self.sorted_rows, self.out, self.path, self.workspace, stream)

    def expert_proj_swiglu(self, stream=None, blocks=None, scales=None):
        p = self.p
        B.mxfp4_expert_proj_swiglu(self.blocks if blocks is None else blocks,
                                   self.scales if scales is None else scales, self.bias, p.E, p.N, p.K, self.x,
                                   p.x_per_slot, p.T, p.k, self.offsets, self.sorted_rows, self.act, self.path,
                                   self.workspace, stream)

    def combine(self, stream=None):
        if self.y is not None:
            p = self.p
            B.moe_combine(self.out, self.gates, p.T, p.k, p.N, self.y, stream)

    def decode(self, stream=None, blocks=None, scales=None):
        """One token from logits: routing, grouping and the projection in one launch."""
        p = self.p
        B.mxfp4_moe_decode(self.logits, p.E, p.k, self.blocks if blocks is None else blocks,
                           self.scales if scales is None else scales, self.bias, p.N, p.K, self.x, p.x_per_slot,
                           self.topk_ids, self.gates, self.offsets, self.sorted_rows, self.out, self.error_word,
                           stream)

    def decode_swiglu(self, stream=None, blocks=None, scales=None):
        """One token from logits through the gated activation: routing, grouping, the
        gate/up projection and the activation in one launch."""
        p = self.p
        B.mxfp4_moe_decode_swiglu(self.logits, p.E, p.k, self.blocks if blocks is None else blocks,
                                  self.scales if scales is None else scales, self.bias, p.N, p.K, self.x,
                                  self.topk_ids, self.gates, self.offsets, self.sorted_rows, self.act,
                                  self.error_word, stream)

    def decode_batch(self, stream=None, blocks=None, scales=None):
        """Up to 64 tokens from logits: routing, grouping and the projection (GEMV
        path) in one launch."""
        p = self.p
        B.mxfp4_moe_decode_batch(self.logits, p.T, p.E, p.k, self.blocks if blocks is None else blocks,
                                 self.scales if scales is None else scales, self.bias, p.N, p.K, self.x,
                                 p.x_per_slot, self.topk_ids, self.gates, self.offsets, self.sorted_rows, self.out,
                                 self.error_word, stream)

    def decode_batch_swiglu(self, stream=None, blocks=None, scales=None):
        """Up to 64 tokens from logits through the gated activation in one launch."""
        p = self.p
        B.mxfp4_moe_decode_batch_swiglu(self.logits, p.T, p.E, p.k, self.blocks if blocks is None else blocks,
                                        self.scales if scales is None else scales, self.bias, p.N, p.K, self.x,
                                        self.topk_ids, self.gates, self.offsets, self.sorted_rows, self.act,
                                        self.error_word, stream)

    def proj_combine(self, stream=None, blocks=None, scales=None, with_out=True):
        """One token (T = 1): every slot's projection and the combine in one launch,
        from the routing already in topk_ids and gates."""
        p = self.p
        assert p.T == 1 and self.y is not None
        B.mxfp4_expert_proj_combine(self.blocks if blocks is None else blocks,
                                    self.scales if scales is None else scales, self.bias, p.E, p.N, p.K, self.x,
                                    p.x_per_slot, p.k, self.topk_ids, self.gates, self.y,
                                    out=self.out if with_out else None, stream=stream)

    def proj_combine_routed(self, stream=None, blocks=None, scales=None):
        """Any T: the projection and the gate-weighted combine (fused into the
        grouped GEMM), from the routing already in topk_ids, gates, offsets and
        sorted_rows."""
        p = self.p
        assert self.y is not None
        B.mxfp4_expert_proj_combine_routed(self.blocks if blocks is None else blocks,
                                           self.scales if scales is None else scales, self.bias, p.E, p.N, p.K,
                                           self.x, p.x_per_slot, p.T, p.k, self.topk_ids, self.gates, self.offsets,
                                           self.sorted_rows, self.out, self.y, self.path, self.workspace, stream)

    def run_fused(self, stream=None):
        """route_group, then the projection with the combine fused in."""
        self.route_group(stream)
        self.proj_combine_routed(stream)

    def run_dense(self, stream=None):
        """The dense-routing form (a validation mode): every expert on every token,
        weighed by the dense router weights, through the same kernels.  Returns
        y [T, N] f32 (gate/up-style problems: one input per token)."""
        p = self.p
        assert p.logits is not None and not p.x_per_slot
        T, E, N = p.T, p.E, p.N
        dev = self.device
        probs = torch.empty((T, E), dtype=torch.float32, device=dev)
        B.mxfp4_moe_dense_route(self.logits, T, E, p.k, probs, stream)
        all_ids = torch.arange(E, dtype=torch.int32, device=dev).repeat(T, 1).contiguous()
        ids = torch.empty((T, E), dtype=torch.int32, device=dev)
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        rows = torch.empty((T * E,), dtype=torch.int32, device=dev)
        B.mxfp4_moe_route_group(None, all_ids, T, E, E, ids, None, offsets, rows, None, stream)
        out = torch.empty((T, E, N), dtype=torch.float32, device=dev)
        nbytes = B.mxfp4_expert_proj_workspace_size(E, N, T, E, p.K, False, self.path)
        ws = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=dev) if nbytes else None
        B.mxfp4_expert_proj(self.blocks, self.scales, self.bias, E, N, p.K, self.x, False, T, E, offsets, rows, out,
                            self.path, ws, stream)
        y = torch.empty((T, N), dtype=torch.float32, device=dev)
        B.moe_combine(out, probs, T, E, N, y, stream)
        torch.cuda.synchronize(dev)
        return probs.cpu().numpy(), y.cpu().numpy()

    def run(self, stream=None):
        self.route_group(stream)
        self.expert_proj(stream)
        self.combine(stream)

    def run_decode(self, stream=None):
        self.decode(stream)
        self.combine(stream)

    def results(self):
        torch.cuda.synchronize(self.device)
        r = {
            "ids": self.topk_ids.cpu().numpy(),
            "offsets": self.offsets.cpu().numpy(),
            "sorted_rows": self.sorted_rows.cpu().numpy(),
            "error_word": int(self.error_word.cpu().item()),
            "out": self.out.cpu().numpy(),
        }
        r["gates"] = self.gates.cpu().numpy() if self.gates is not None else None
        r["y"] = self.y.cpu().numpy() if self.y is not None else None
        r["act"] = self.act.view(torch.int16).cpu().numpy().view(np.uint16) if self.act is not None else None
        return r
