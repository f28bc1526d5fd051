"""The allocation-free permute (moe_permute_static) against moe_permute,
through the C ABI (GPU): two calls in a row, the second on a smaller
problem, each bit-exact against the workspace entry point's routing state
and against the oracle's permutation. The second call reuses the fixed
device scratch the first one left behind."""

import numpy as np
import pytest

from dropless_grouped_gemm_router_amd import binding as B
from dropless_grouped_gemm_router_amd.inputs import Problem
from oracle import oracle

from gpu_util import Case, note

pytestmark = pytest.mark.gpu

KEYS = ("expert_offsets", "perm", "inv_perm", "num_tiles")


def _static_vs_workspace(p: Problem, seed: int):
    import torch
    note(f"permute_static {p}")
    c = Case(p, seed=seed)
    B.moe_route(p, c.dev["x"], c.dev["w_router"], c.buf.routing)
    B.moe_permute(p, c.buf.routing, c.buf.workspace)
    torch.cuda.synchronize()
    ref = {k: c.buf.routing[k].clone() for k in KEYS}
    n = int(ref["num_tiles"].item())
    ref_tiles = c.buf.routing["tiles"][:n].clone()
    # scribble over the outputs, then the allocation-free call
    for k in KEYS + ("tiles",):
        c.buf.routing[k].fill_(-7)
    B.moe_permute_static(p, c.buf.routing)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(c.buf.routing[k], ref[k]), k
    assert torch.equal(c.buf.routing["tiles"][:n], ref_tiles)
    idx = c.buf.routing["topk_idx"].cpu().numpy()
    r = oracle.permute(idx, p.experts, p.block_m, capacity=p.capacity)
    assert np.array_equal(c.buf.routing["perm"].cpu().numpy(), r["perm"])
    assert np.array_equal(c.buf.routing["inv_perm"].cpu().numpy(), r["inv_perm"])
    assert np.array_equal(c.buf.routing["tiles"][:n].cpu().numpy(), r["tiles"])


def test_permute_static_two_calls_second_smaller():
    # 131072 tokens x top-8 at 64 experts: 256 blocks x 64 experts of counts
    # (64 KiB of the scratch); then a smaller, ragged, skewed problem with
    # capacity routing that reads fewer of the entries the first call wrote
    _static_vs_workspace(Problem(131072, 64, 8, 128, 64, 0, "bf16", 256), seed=3)
    _static_vs_workspace(Problem(5001, 16, 3, 128, 64, 0, "bf16", 64, skew=0.9, capacity=700),
                         seed=4)


def test_permute_static_largest_fitting_problem():
    # exactly the 1 MiB of counts the scratch holds: 4096 blocks x 64 experts
    _static_vs_workspace(Problem((1 << 24) // 8, 64, 8, 128, 64, 0, "bf16", 128), seed=5)
