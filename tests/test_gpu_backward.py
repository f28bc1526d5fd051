"""HIP train-step backward vs the oracle, through the C ABI (GPU)."""

import numpy as np
import pytest

from dropless_grouped_gemm_router_amd import binding as B
from dropless_grouped_gemm_router_amd.inputs import Problem, WORKLOADS
from oracle import oracle

from gpu_util import TOL, Case, keep_of, note, pid, to_np

pytestmark = pytest.mark.gpu

GRAD_NAMES = ["w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"]


def run_bwd(c: Case, side=True):
    """Staged forward with saved activations, then moe_bwd, by default with
    a second stream for the shared expert's backward."""
    import torch
    c.forward()
    gx, g = B.backward(c.p, c.dev["x"], c.weights(), c.dev["grad_out"], c.buf,
                       side_stream=c.side if side else None)
    torch.cuda.synchronize()
    return gx, g


def check_grads(c: Case, gx, g, nthreads=0):
    p, v = c.p, c.v
    idx = c.buf.routing["topk_idx"].cpu().numpy()
    _, idx_ref, w = oracle.route(v["x"], v["w_router"], p.top_k, nthreads)
    assert np.array_equal(idx, idx_ref)
    ref = oracle.backward(v["x"], v["w_router"], v["w_gate"], v["w_up"], v["w_down"],
                          v["grad_out"], idx_ref, w, *c.shared(), nthreads=nthreads,
                          keep=keep_of(p, idx_ref))
    errs = {"x": oracle.rel_err(to_np(gx), ref["x"])}
    for n in GRAD_NAMES:
        if n in g:
            errs[n] = oracle.rel_err(to_np(g[n]), ref[n])
    note(f"grad rel errs: " + ", ".join(f"{k} {e:.2e}" for k, e in errs.items()))
    for n, e in errs.items():
        assert e < TOL[p.dtype], (n, e)
    return ref


SMALL = [
    Problem(300, 8, 2, 256, 128, 0, "bf16", 64),
    Problem(300, 8, 2, 256, 128, 0, "fp32", 64),
    Problem(517, 16, 4, 256, 256, 128, "bf16", 128),
    Problem(517, 16, 4, 256, 128, 128, "fp32", 32),
    Problem(3, 4, 2, 128, 128, 128, "bf16", 32),
    Problem(200, 5, 5, 128, 128, 0, "fp32", 64),
    Problem(1000, 64, 8, 128, 128, 256, "bf16", 128),
    Problem(1500, 8, 2, 256, 128, 128, "bf16", 256),
    Problem(700, 4, 2, 256, 256, 128, "fp32", 256),
    Problem(2000, 64, 8, 256, 128, 128, "bf16", 128, skew=0.9),
    # experts averaging >= 512 rows at block_m 128: the gate/up dgrad runs on
    # a 256-row tile list derived from the offsets (capacity-clipped too)
    Problem(20000, 8, 2, 256, 128, 128, "bf16", 128),
    Problem(20000, 8, 2, 256, 128, 0, "bf16", 64, capacity=4000),
    # the largest d_model the library takes, and every expert selected
    Problem(64, 8, 2, 8192, 128, 0, "bf16", 64),
    Problem(300, 64, 64, 128, 128, 128, "bf16", 64),
    # capacity routing: dropped slots give no expert gradient but still a
    # router gradient
    Problem(1500, 8, 2, 256, 128, 128, "bf16", 256, capacity=300),
    Problem(517, 16, 4, 256, 128, 128, "fp32", 32, capacity=100),
    Problem(2000, 64, 8, 256, 128, 128, "bf16", 128, skew=0.9, capacity=200),
    Problem(300, 8, 2, 256, 128, 0, "bf16", 64, capacity=1),
    # odd top_k for the k-specialised gathers (combine backward, dx)
    Problem(400, 6, 3, 128, 128, 0, "bf16", 64, capacity=150),
    Problem(300, 12, 7, 128, 128, 128, "fp32", 64),
]


@pytest.mark.parametrize("p", SMALL, ids=pid)
def test_backward_small_elementwise(p):
    note(f"backward small {p}")
    c = Case(p, seed=11, training=True)
    gx, g = run_bwd(c)
    check_grads(c, gx, g)


def test_top1_router_gradient_exactly_zero():
    p = Problem(150, 8, 1, 128, 128, 0, "bf16", 64)
    c = Case(p, seed=2, training=True)
    gx, g = run_bwd(c)
    assert bool((g["w_router"] == 0).all())
    check_grads(c, gx, g)


def test_backward_deterministic():
    p = Problem(700, 16, 4, 256, 128, 128, "bf16", 64)
    c = Case(p, seed=4, training=True)
    gx, g = run_bwd(c)
    a = {n: t.clone() for n, t in g.items()}
    ax = gx.clone()
    gx2, g2 = run_bwd(c)
    assert bool((ax == gx2).all())
    for n in a:
        assert bool((a[n] == g2[n]).all()), n


def test_backward_side_stream_same_bits():
    """moe_bwd with and without a second stream: the same kernels in another
    order across two streams, so identical gradients bit for bit."""
    p = Problem(1500, 16, 4, 256, 128, 256, "bf16", 128)
    c = Case(p, seed=6, training=True)
    gx, g = run_bwd(c, side=True)
    a = {n: t.clone() for n, t in g.items()}
    ax = gx.clone()
    gx2, g2 = run_bwd(c, side=False)
    assert bool((ax == gx2).all())
    for n in a:
        assert bool((a[n] == g2[n]).all()), n


def test_zero_tokens_zeroes_weight_grads():
    import torch
    p = Problem(0, 8, 2, 256, 128, 128, "bf16", 64)
    f32 = dict(dtype=torch.float32, device="cuda")
    g = dict(w_router=torch.ones((256, 8), **f32), w_gate=torch.ones((8, 256, 128), **f32),
             w_up=torch.ones((8, 256, 128), **f32), w_down=torch.ones((8, 128, 256), **f32),
             ws_gate=torch.ones((256, 128), **f32), ws_up=torch.ones((256, 128), **f32),
             ws_down=torch.ones((128, 256), **f32))
    B.moe_bwd(p, None, {}, {}, None, None, None, None, g, None, workspace_bytes=0)
    torch.cuda.synchronize()
    for n, t in g.items():
        assert bool((t == 0).all()), n


def test_train_workload_full_size():
    """The train-step workload (16384 tokens, E64 top-8, d512 h128, shared
    1024) at full size: every gradient element against the oracle."""
    name, p, _ = WORKLOADS[4]
    note(f"workload 4: {name}")
    c = Case(p, seed=0, training=True)
    gx, g = run_bwd(c)
    check_grads(c, gx, g)


def test_backward_maxtok_shape_elementwise():
    """The max-token train-step shape (kernel_gmm_gpu.json "maxtok" suite:
    E=8, top-2, d_model 512, d_hidden 1024, bf16) at 3000 tokens: every
    element of every gradient and of dx against the oracle."""
    p = Problem(3000, 8, 2, 512, 1024, 0, "bf16", 128)
    note(f"backward maxtok shape {p}")
    c = Case(p, seed=13, training=True)
    gx, g = run_bwd(c)
    check_grads(c, gx, g)


LARGE_TOKENS = 2228224  # T*k*d_model = 2,281,701,376 > 2^31 elements per slot buffer


@pytest.mark.timeout(900)
def test_train_step_past_2e31_elements_sampled():
    """The max-token shape at 2,228,224 tokens: y_sorted, dY and the per-slot
    dX hold more than 2^31 elements and the saved gate/up activations more
    than 2^33, so every slot-indexed address needs 64 bits. Routing and the
    permutation bit-exact on every token; out and dx on sampled tokens,
    among them tokens whose slots sit at the far end of the sorted rows.
    Tokens are generated in full; grad_out is a seeded 131072-token block
    repeated (it is indexed by token, below 2^31 elements)."""
    import dataclasses

    import torch

    from dropless_grouped_gemm_router_amd.inputs import Tensor, make_inputs

    p = Problem(LARGE_TOKENS, 8, 2, 512, 1024, 0, "bf16", 128)
    note(f"train step past 2^31 elements: {p}: generating inputs")
    inp = make_inputs(p, seed=0)
    blk = make_inputs(dataclasses.replace(p, tokens=131072), seed=0, with_grad_out=True,
                      names=["grad_out"])["grad_out"]
    reps = -(-p.tokens // 131072)
    inp["grad_out"] = Tensor(stored=np.tile(blk.stored, (reps, 1))[:p.tokens],
                             value=np.tile(blk.value, (reps, 1))[:p.tokens])
    c = Case(p, training=True, inputs=inp)
    note("forward + backward on the GPU")
    gx, g = run_bwd(c)
    note("oracle routing of every token")
    v = c.v
    _, idx, w = oracle.route(v["x"], v["w_router"], p.top_k)
    got = c.routing_np()
    assert np.array_equal(got["topk_idx"], idx)
    assert np.max(np.abs(got["topk_w"] - w)) < 2e-6
    r = oracle.permute(idx, p.experts, p.block_m)
    assert np.array_equal(got["offsets"], r["offsets"])
    assert np.array_equal(got["perm"], r["perm"])
    assert np.array_equal(got["inv_perm"], r["inv_perm"])
    assert got["num_tiles"] == r["num_tiles"] and np.array_equal(got["tiles"], r["tiles"])
    S = p.tokens * p.top_k
    far = r["perm"][[S - 1, S - 2, S - 777, S // 2 + 5, (1 << 31) // p.d_model + 3]] // p.top_k
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, p.tokens - 1], far,
                                     rng.choice(p.tokens, 120, replace=False)]))
    note(f"oracle on {rows.size} sampled tokens")
    ref = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w, rows=rows)
    err = oracle.rel_err(to_np(c.buf.out[rows.tolist()]), ref)
    # dx of a token depends on that token alone (dropless): the oracle's
    # backward over the sampled tokens gives their rows exactly
    gref = oracle.backward(v["x"][rows], v["w_router"], v["w_gate"], v["w_up"], v["w_down"],
                           v["grad_out"][rows], idx[rows], w[rows])
    ex = oracle.rel_err(to_np(gx[rows.tolist()]), gref["x"])
    note(f"out rel err {err:.3e}, dx rel err {ex:.3e}")
    assert err < TOL[p.dtype] and ex < TOL[p.dtype]
    assert bool(torch.isfinite(g["w_gate"]).all()) and bool(torch.isfinite(g["w_down"]).all())
