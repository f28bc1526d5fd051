"""Shared helpers of the GPU parity tests: run the HIP path through the
C-ABI binding and the oracle on the same seeded inputs."""

import sys

import numpy as np

from dropless_grouped_gemm_router_amd import binding as B
from dropless_grouped_gemm_router_amd.inputs import Problem, make_inputs
from oracle import oracle

# Normwise relative-error bars: fp32 storage, and bf16 storage with fp32 accumulation.
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def pid(p: Problem) -> str:
    """Test id of a problem."""
    return (f"T{p.tokens}E{p.experts}k{p.top_k}d{p.d_model}h{p.d_hidden}s{p.d_shared}{p.dtype}"
            f"bm{p.block_m}" + (f"skew{p.skew}" if p.skew else "")
            + (f"cap{p.capacity}" if p.capacity else ""))


def keep_of(p: Problem, idx):
    """[T, k] flags of the slots capacity routing keeps (None: dropless),
    from the oracle's permutation."""
    if not p.capacity:
        return None
    r = oracle.permute(idx, p.experts, p.block_m, capacity=p.capacity)
    return oracle.keep_mask(r, p.tokens, p.top_k)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


class Case:
    """One problem: generated inputs, device copies and device buffers."""

    def __init__(self, p: Problem, seed=0, training=False, inputs=None):
        import torch
        self.p = p
        self.inputs = inputs if inputs is not None else make_inputs(p, seed=seed, with_grad_out=training)
        self.v = {n: t.value for n, t in self.inputs.items()}
        self.dev = B.device_inputs(self.inputs)
        self.buf = B.allocate(p, training=training)
        self.training = training
        # the caller-owned second stream moe_forward and moe_bwd may fork onto
        self.side = torch.cuda.Stream()
        torch.cuda.synchronize()

    def weights(self):
        return {n: self.dev[n] for n in self.dev if n not in ("x", "grad_out")}

    def forward(self):
        import torch
        out = B.forward(self.p, self.dev["x"], self.weights(), self.buf, training=self.training)
        torch.cuda.synchronize()
        return out

    def routing_np(self):
        r = self.buf.routing
        n = int(r["num_tiles"].cpu().item())
        return dict(topk_idx=r["topk_idx"].cpu().numpy(), topk_w=r["topk_w"].cpu().numpy(),
                    offsets=r["expert_offsets"].cpu().numpy(), perm=r["perm"].cpu().numpy(),
                    inv_perm=r["inv_perm"].cpu().numpy(), tiles=r["tiles"][:n].cpu().numpy(),
                    num_tiles=n)

    def shared(self):
        v = self.v
        return (v.get("ws_gate"), v.get("ws_up"), v.get("ws_down"))
