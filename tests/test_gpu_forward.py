"""HIP forward path vs the oracle, through the C ABI (GPU)."""

import numpy as np
import pytest

from dropless_grouped_gemm_router_amd.inputs import Problem, WORKLOADS
from oracle import oracle

from gpu_util import TOL, Case, keep_of, note, pid, to_np

pytestmark = pytest.mark.gpu


def check_routing(c: Case, nthreads=0):
    """Routing ints bit-exact; weights to fp32 rounding."""
    p, v = c.p, c.v
    _, idx, w = oracle.route(v["x"], v["w_router"], p.top_k, nthreads)
    g = c.routing_np()
    assert np.array_equal(g["topk_idx"], idx)
    assert np.max(np.abs(g["topk_w"] - w)) < 2e-6
    r = oracle.permute(idx, p.experts, p.block_m, capacity=p.capacity)
    assert np.array_equal(g["offsets"], r["offsets"])
    assert np.array_equal(g["perm"], r["perm"])
    assert np.array_equal(g["inv_perm"], r["inv_perm"])
    assert g["num_tiles"] == r["num_tiles"]
    assert np.array_equal(g["tiles"], r["tiles"])
    return idx, w, r


SMALL = [
    # tokens, E, k, d, h, hs, dtype, bm  -- several tiles and ragged tails
    Problem(300, 8, 2, 256, 128, 0, "bf16", 64),
    Problem(300, 8, 2, 256, 128, 0, "fp32", 64),
    Problem(517, 16, 4, 256, 192, 128, "bf16", 128),
    Problem(517, 16, 4, 256, 192, 128, "fp32", 32),
    Problem(1, 4, 2, 128, 64, 64, "bf16", 32),
    Problem(97, 1, 1, 128, 64, 0, "bf16", 128),
    Problem(200, 5, 5, 128, 64, 0, "fp32", 64),
    Problem(1000, 64, 8, 128, 64, 64, "bf16", 128),
    Problem(1500, 8, 2, 256, 128, 128, "bf16", 256),
    Problem(700, 4, 2, 256, 256, 0, "fp32", 256),
    # bf16, block_m 256, three 256-column tiles of d_model in the down GEMM
    Problem(900, 16, 4, 768, 128, 0, "bf16", 256),
    # skewed routing (uneven expert loads, nearly empty experts)
    Problem(3000, 64, 8, 256, 128, 128, "bf16", 256, skew=0.9),
    Problem(3000, 64, 8, 256, 128, 0, "bf16", 64, skew=0.9),
    # 64 experts and more than 65536 tokens: the router's 8-lane x 8-expert
    # layout in 512-thread workgroups; 66000 leaves a ragged last pass
    Problem(66000, 64, 8, 128, 64, 0, "bf16", 256),
    # experts averaging >= 512 rows at block_m < 256: the down GEMM runs on
    # a 256-row tile list derived from the offsets (capacity-clipped too)
    Problem(20000, 8, 2, 256, 128, 0, "bf16", 64),
    Problem(20000, 8, 2, 256, 128, 128, "bf16", 128, capacity=4000),
    # the largest d_model the library takes (K = 8192 in the gate/up GEMM,
    # the router streamed through LDS in chunks) and every expert selected
    # (top_k = E = 64: the combine past eight ranks)
    Problem(64, 8, 2, 8192, 64, 0, "bf16", 64),
    Problem(64, 8, 2, 8192, 64, 0, "fp32", 64),
    Problem(300, 64, 64, 128, 64, 64, "bf16", 64),
    # capacity routing: the busier experts drop their last slots
    Problem(1500, 8, 2, 256, 128, 128, "bf16", 256, capacity=300),
    Problem(517, 16, 4, 256, 192, 128, "fp32", 32, capacity=100),
    Problem(3000, 64, 8, 256, 128, 0, "bf16", 64, skew=0.9, capacity=375),
    Problem(3000, 64, 8, 256, 128, 128, "bf16", 256, skew=0.9, capacity=300),
    Problem(300, 8, 2, 256, 128, 0, "bf16", 128, capacity=1),
]


@pytest.mark.parametrize("p", SMALL, ids=pid)
def test_forward_small_elementwise(p):
    note(f"forward small {p}")
    c = Case(p, seed=7)
    out = c.forward()
    idx, w, r = check_routing(c)
    keep = keep_of(p, idx)
    ref, y = oracle.forward_rows(c.v["x"], c.v["w_gate"], c.v["w_up"], c.v["w_down"], idx, w,
                                 *c.shared(), want_y=True, keep=keep)
    # sorted expert outputs: row inv_perm[s] holds the unweighted output of
    # flat slot s (kept slots only; rows of dropped ones are never written)
    kept = r["inv_perm"] >= 0
    if p.capacity:
        assert not kept.all()
    import torch
    ys = to_np(c.buf.y_sorted[torch.from_numpy(r["inv_perm"][kept].astype(np.int64)).cuda()])
    assert oracle.rel_err(ys, y[kept]) < TOL[p.dtype]
    if p.d_shared:
        sref = oracle.forward_rows(c.v["x"], c.v["w_gate"], c.v["w_up"], c.v["w_down"], idx,
                                   np.zeros_like(w), *c.shared())
        assert oracle.rel_err(to_np(c.buf.shared_out), sref) < TOL[p.dtype]
    assert oracle.rel_err(to_np(out), ref) < TOL[p.dtype]
    assert np.all(np.isfinite(to_np(out)))


@pytest.mark.parametrize("p", [Problem(777, 8, 2, 256, 128, 128, "bf16", 64),
                               Problem(2000, 8, 2, 512, 128, 128, "bf16", 256)],
                         ids=["bm64", "bm256"])
def test_forward_deterministic(p):
    c = Case(p, seed=3)
    a = c.forward().clone()
    ya = c.buf.y_sorted.clone()
    b = c.forward()
    assert bool((a.view(-1).view(dtype=__import__("torch").int16) ==
                 b.view(-1).view(dtype=__import__("torch").int16)).all())
    assert bool((ya == c.buf.y_sorted).all())


def _route_only(p: Problem, seed: int, wr: np.ndarray = None):
    """moe_route on generated tokens (and an optional replacement router);
    returns the device routing and the oracle's (indices, weights)."""
    import torch
    from dropless_grouped_gemm_router_amd import binding as B
    c = Case(p, seed=seed)
    if wr is not None:
        c.v["w_router"] = wr
        c.dev["w_router"] = torch.from_numpy(wr).cuda()
    B.moe_route(p, c.dev["x"], c.dev["w_router"], c.buf.routing)
    torch.cuda.synchronize()
    _, idx, w = oracle.route(c.v["x"], c.v["w_router"], p.top_k)
    return c.routing_np(), idx, w


# Every router lane layout: (L lanes x P experts x R tokens per lane) by
# experts and batch size, and the chunked kernel for routers too wide for LDS
# (64 experts at d_model 768, 32 at 1280, 8 at 5120).
ROUTE_LAYOUTS = [
    Problem(66000, 64, 8, 128, 64, 0, "bf16", 256),
    Problem(40000, 64, 8, 128, 64, 0, "bf16", 256),
    Problem(3000, 64, 8, 128, 64, 0, "bf16", 256),
    Problem(3000, 64, 8, 128, 64, 0, "fp32", 256),
    Problem(3000, 32, 4, 256, 64, 0, "bf16", 256),
    Problem(3000, 16, 4, 256, 64, 0, "bf16", 256),
    Problem(3000, 8, 2, 256, 64, 0, "bf16", 256),
    Problem(3000, 8, 2, 128, 64, 0, "fp32", 256),
    Problem(66000, 8, 2, 128, 64, 0, "bf16", 256),
    Problem(66000, 8, 2, 128, 64, 0, "fp32", 256),
    Problem(3000, 4, 2, 256, 64, 0, "bf16", 256),
    Problem(3000, 2, 1, 256, 64, 0, "bf16", 256),
    Problem(3000, 64, 8, 768, 64, 0, "bf16", 256),
    Problem(3000, 64, 8, 768, 64, 0, "fp32", 256),
    Problem(3000, 32, 4, 1280, 64, 0, "bf16", 256),
    Problem(1000, 8, 2, 5120, 64, 0, "bf16", 256),
]


@pytest.mark.parametrize("p", ROUTE_LAYOUTS, ids=pid)
def test_route_layouts(p):
    note(f"route layout {p}")
    g, idx, w = _route_only(p, seed=13)
    assert np.array_equal(g["topk_idx"], idx)
    assert np.max(np.abs(g["topk_w"] - w)) < 2e-6


@pytest.mark.parametrize("p", ROUTE_LAYOUTS, ids=pid)
def test_route_exact_ties(p):
    """Duplicated router columns give equal logits for every token: the
    lower expert index must rank first, whether the tied experts sit in one
    lane, in two lanes of a token's group, or far apart. The tied columns
    are scaled up so they are usually among the top k."""
    note(f"route ties {p}")
    rng = np.random.default_rng(17)
    E, d = p.experts, p.d_model
    wr = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    for e0 in range(0, E, 16):
        for dup in (1, 4, 8, 9):
            if e0 + dup < E:
                wr[:, e0 + dup] = wr[:, e0]
        wr[:, e0] *= 3.0
        for dup in (1, 4, 8, 9):
            if e0 + dup < E:
                wr[:, e0 + dup] = wr[:, e0]
    g, idx, w = _route_only(p, seed=19, wr=wr)
    if p.top_k > 1:
        # the ties were actually exercised
        assert np.any((idx[:, :-1] + 1 == idx[:, 1:]) & (idx[:, :-1] % 16 == 0))
    assert np.array_equal(g["topk_idx"], idx)
    assert np.max(np.abs(g["topk_w"] - w)) < 2e-6


@pytest.mark.parametrize("p", [Problem(3000, 64, 8, 128, 64, 0, "bf16", 256),
                               Problem(66000, 64, 8, 128, 64, 0, "bf16", 256),
                               Problem(3000, 64, 8, 768, 64, 0, "bf16", 256),
                               Problem(500, 5, 3, 128, 64, 0, "fp32", 64)], ids=pid)
def test_route_zero_router(p):
    """An all-zero router: every logit is +0, so every token takes experts
    0..k-1 in that order with weights exactly 1/k."""
    g, idx, w = _route_only(p, seed=23, wr=np.zeros((p.d_model, p.experts), np.float32))
    assert np.array_equal(g["topk_idx"], np.tile(np.arange(p.top_k, dtype=np.int32), (p.tokens, 1)))
    assert np.all(g["topk_w"] == np.float32(1.0) / np.float32(p.top_k))
    assert np.array_equal(g["topk_idx"], idx)


def test_permute_scan_long_chunks():
    """More than 16384 (expert, block) counts: each thread of the one-workgroup
    scan takes a chunk longer than its sixteen-entry register batch (the
    scan's third path). Routing and the permutation bit-exact."""
    import torch
    from dropless_grouped_gemm_router_amd import binding as B
    p = Problem(139264, 64, 8, 128, 64, 0, "bf16", 128)  # 272 blocks x 64 experts
    note(f"long scan chunks: {p}")
    c = Case(p, seed=7)
    B.moe_route(p, c.dev["x"], c.dev["w_router"], c.buf.routing)
    B.moe_permute(p, c.buf.routing, c.buf.workspace)
    torch.cuda.synchronize()
    check_routing(c)


def test_skewed_routing_empty_experts():
    """A router that sends every token to experts 0 and 1: two experts with
    every slot (many tiles each), the rest empty."""
    import torch
    p = Problem(700, 8, 2, 128, 64, 0, "bf16", 32)
    c = Case(p, seed=5)
    wr = np.zeros((128, 8), np.float32)
    wr[:, 0] = 1.0
    wr[:, 1] = 0.5
    c.inputs["w_router"].stored = wr
    c.inputs["w_router"].value = wr
    c.v["w_router"] = wr
    c.dev["w_router"] = torch.from_numpy(wr).cuda()
    # make x positive so experts 0, 1 always lead
    xs = np.abs(c.v["x"]).astype(np.float32)
    from dropless_grouped_gemm_router_amd.inputs import f32_to_bf16_bits, bf16_bits_to_f32
    bits = f32_to_bf16_bits(xs)
    c.v["x"] = bf16_bits_to_f32(bits).reshape(xs.shape)
    c.dev["x"] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    out = c.forward()
    idx, w, r = check_routing(c)
    assert np.all(idx[:, 0] == 0) and np.all(idx[:, 1] == 1)
    assert r["num_tiles"] == 2 * ((700 + 31) // 32)
    ref = oracle.forward_rows(c.v["x"], c.v["w_gate"], c.v["w_up"], c.v["w_down"], idx, w)
    assert oracle.rel_err(to_np(out), ref) < TOL["bf16"]


def test_zero_tokens_is_noop():
    import torch
    from dropless_grouped_gemm_router_amd import binding as B
    p = Problem(0, 8, 2, 256, 128, 0, "bf16", 64)
    B.moe_route(p, None, None, {})
    B.moe_permute(p, {}, None, workspace_bytes=0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_workload_full_size_sampled(cfg):
    """The measured workloads at full size: routing and permutation bit-exact
    on every token, outputs on a sample of rows."""
    name, p, _ = WORKLOADS[cfg]
    note(f"workload {cfg}: {name}")
    c = Case(p, seed=0)
    out = c.forward()
    idx, w, r = check_routing(c, nthreads=0)
    rng = np.random.default_rng(cfg)
    rows = np.unique(np.concatenate([[0, p.tokens - 1], rng.choice(p.tokens, 254, replace=False)]))
    ref = oracle.forward_rows(c.v["x"], c.v["w_gate"], c.v["w_up"], c.v["w_down"], idx, w,
                              *c.shared(), rows=rows)
    got = to_np(out[rows.tolist()])
    err = oracle.rel_err(got, ref)
    note(f"workload {cfg}: out rel err {err:.3e}")
    assert err < TOL[p.dtype]
