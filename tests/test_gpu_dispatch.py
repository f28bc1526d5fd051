"""Dispatch variants of the whole forward (moe_forward: gather, sorted,
fused_gsum; kernel_gmm_gpu.json "layer" suite, field "dispatch") through the
C ABI (GPU). The variants change where token rows are gathered and where the
combine runs, never the arithmetic or its order, so each must reproduce the
staged calls (moe_route, moe_permute, moe_ffn_fwd, moe_combine) bit for bit;
the staged calls are checked against the oracle elsewhere, and the output is
also checked against the oracle here."""

import numpy as np
import pytest

from dropless_grouped_gemm_router_amd import binding as B
from dropless_grouped_gemm_router_amd.inputs import Problem, WORKLOADS
from oracle import oracle

from gpu_util import TOL, Case, keep_of, note, pid, to_np

pytestmark = pytest.mark.gpu

DISPATCHES = ["gather", "sorted", "fused_gsum"]

CASES = [
    # bf16, block_m 256: the wide engine's fused epilogue; 1500 = 5 * 256 + 220
    # leaves a ragged last token tile.
    Problem(1500, 8, 2, 256, 128, 128, "bf16", 256),
    # d_model 384 is not a multiple of 256: the shared down GEMM (and its
    # fused epilogue) runs on the four-wave 256 x 128 tile.
    Problem(517, 16, 4, 384, 192, 128, "bf16", 128),
    # fp32: the register-staged engine's four-column fused epilogue
    Problem(517, 16, 4, 256, 192, 128, "fp32", 64),
    # odd top_k, narrow shared expert
    Problem(700, 8, 5, 512, 128, 64, "bf16", 256),
    # top_k 10 > 8 and no shared expert: fused_gsum runs as gather
    Problem(300, 16, 10, 256, 128, 128, "bf16", 64),
    Problem(300, 8, 2, 256, 128, 0, "bf16", 64),
    Problem(1, 4, 2, 128, 64, 64, "bf16", 32),
    Problem(3000, 64, 8, 256, 128, 128, "bf16", 256, skew=0.9),
    # capacity routing: dropped slots are left out of every variant's combine
    Problem(3000, 64, 8, 256, 128, 128, "bf16", 256, skew=0.9, capacity=300),
    Problem(517, 16, 4, 384, 192, 128, "bf16", 128, capacity=100),
]


def bits_equal(a, b) -> bool:
    import torch
    return a.shape == b.shape and torch.equal(a.contiguous().view(torch.uint8),
                                              b.contiguous().view(torch.uint8))


def run_variant(c: Case, dispatch, training=False):
    import torch
    buf = B.allocate(c.p, training=training, dispatch=dispatch)
    B.forward_dispatch(c.p, dispatch, c.dev["x"], c.weights(), buf, training=training,
                       side_stream=c.side)
    torch.cuda.synchronize()
    return buf


def assert_same_forward(ref: B.Buffers, got: B.Buffers, n_tiles: int, training=False):
    for k in ("topk_idx", "topk_w", "expert_offsets", "perm", "inv_perm", "num_tiles"):
        assert bits_equal(ref.routing[k], got.routing[k]), k
    assert bits_equal(ref.routing["tiles"][:n_tiles], got.routing["tiles"][:n_tiles])
    # every row of a kept slot (rows of slots dropped by capacity routing are
    # never written)
    rows = ref.routing["inv_perm"]
    rows = rows[rows >= 0].long()
    assert bits_equal(ref.y_sorted[rows], got.y_sorted[rows])
    assert bits_equal(ref.out, got.out)
    if training:
        assert bits_equal(ref.saved, got.saved)


@pytest.mark.parametrize("p", CASES, ids=pid)
@pytest.mark.parametrize("dispatch", DISPATCHES)
def test_dispatch_matches_staged_and_oracle(p, dispatch):
    note(f"dispatch {dispatch} {p}")
    c = Case(p, seed=11)
    c.forward()
    n_tiles = int(c.buf.routing["num_tiles"].cpu().item())
    got = run_variant(c, dispatch)
    assert_same_forward(c.buf, got, n_tiles)
    # routing from the oracle, not from the device: indices bit-exact,
    # weights to fp32 rounding, the output from the oracle's own routing
    _, idx, w = oracle.route(c.v["x"], c.v["w_router"], p.top_k)
    assert np.array_equal(got.routing["topk_idx"].cpu().numpy(), idx)
    assert np.max(np.abs(got.routing["topk_w"].cpu().numpy() - w)) < 2e-6
    r = oracle.permute(idx, p.experts, p.block_m, capacity=p.capacity)
    assert np.array_equal(got.routing["perm"].cpu().numpy(), r["perm"])
    assert np.array_equal(got.routing["inv_perm"].cpu().numpy(), r["inv_perm"])
    ref = oracle.forward_rows(c.v["x"], c.v["w_gate"], c.v["w_up"], c.v["w_down"], idx, w,
                              *c.shared(), keep=keep_of(p, idx))
    assert oracle.rel_err(to_np(got.out), ref) < TOL[p.dtype]


@pytest.mark.parametrize("dispatch", ["sorted", "fused_gsum"])
def test_dispatch_training_saves_the_same_activations(dispatch):
    """With a saved buffer the variants write the activations moe_bwd reads,
    identical to the staged forward's, so the backward is unchanged."""
    p = Problem(1000, 16, 4, 256, 128, 128, "bf16", 128)
    c = Case(p, seed=4, training=True)
    c.forward()
    n_tiles = int(c.buf.routing["num_tiles"].cpu().item())
    got = run_variant(c, dispatch, training=True)
    assert_same_forward(c.buf, got, n_tiles, training=True)


def test_dispatch_repeat_is_deterministic():
    """Two fused_gsum calls into the same buffers give identical bits."""
    import torch
    p = Problem(2000, 8, 2, 512, 128, 256, "bf16", 256)
    c = Case(p, seed=2)
    buf = B.allocate(p, dispatch="fused_gsum")
    B.forward_dispatch(p, "fused_gsum", c.dev["x"], c.weights(), buf)
    torch.cuda.synchronize()
    first = buf.out.clone()
    B.forward_dispatch(p, "fused_gsum", c.dev["x"], c.weights(), buf)
    torch.cuda.synchronize()
    assert bits_equal(first, buf.out)


def test_dispatch_full_size_workload():
    """The 131072-token, 64-expert, top-8 workload with its 1024-wide shared
    expert: every variant equals the staged forward on every output element;
    a sample of rows against the oracle."""
    import torch
    name, p, _ = WORKLOADS[3]
    note(f"dispatch full size: {name}")
    c = Case(p, seed=0)
    c.forward()
    n_tiles = int(c.buf.routing["num_tiles"].cpu().item())
    for dispatch in DISPATCHES:
        note(f"dispatch full size: {dispatch}")
        got = run_variant(c, dispatch)
        assert_same_forward(c.buf, got, n_tiles)
        if dispatch == "fused_gsum":
            _, idx, w = oracle.route(c.v["x"], c.v["w_router"], p.top_k)
            assert np.array_equal(got.routing["topk_idx"].cpu().numpy(), idx)
            rng = np.random.default_rng(5)
            rows = np.unique(np.concatenate([[0, p.tokens - 1],
                                             rng.choice(p.tokens, 126, replace=False)]))
            ref = oracle.forward_rows(c.v["x"], c.v["w_gate"], c.v["w_up"], c.v["w_down"], idx,
                                      w, *c.shared(), rows=rows)
            assert oracle.rel_err(to_np(got.out[rows.tolist()]), ref) < TOL[p.dtype]
        del got
        torch.cuda.empty_cache()
