"""Pins of the CPU oracle against things other than itself: a dense
every-expert-masked brute force (numpy float64), finite differences, closed
forms and special cases, a constructed permutation, invariants and the
pages' parameter count. CPU only."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

from dropless_grouped_gemm_router_amd.inputs import Problem, make_inputs
from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ brute force
# Dense formulation (the pages' "dense:auto:sorted" routing, kernel_gmm_gpu.json
# layer suite): every expert is evaluated on every token and masked by the
# renormalised top-k weight, which is zero for experts not kept.

def bf_select(logits, k):
    """Independent selection loop: k rounds of 'largest value, lowest index'."""
    T, E = logits.shape
    sel = np.empty((T, k), np.int64)
    for t in range(T):
        taken = set()
        for i in range(k):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or logits[t, e] > logits[t, best]:
                    best = e
            sel[t, i] = best
            taken.add(best)
    return sel


def bf_mask_weights(logits64, sel):
    """Dense [T,E] weights: softmax over all E, zero the non-kept, divide by the kept sum."""
    T, E = logits64.shape
    p = softmax(logits64, axis=1)
    m = np.zeros((T, E))
    for t in range(T):
        m[t, sel[t]] = 1.0
    q = p * m
    return q / q.sum(axis=1, keepdims=True)


def bf_ffn(x, wg, wu, wd):
    a = x @ wg
    b = x @ wu
    return ((a * expit(a)) * b) @ wd


def bf_forward(x, wr, wg, wu, wd, sel, ws=None, logits64=None, keep=None):
    x = x.astype(np.float64)
    if logits64 is None:
        logits64 = x @ wr.astype(np.float64)
    W = bf_mask_weights(logits64, sel)
    if keep is not None:
        # capacity routing: a dropped slot's expert contributes nothing, the
        # kept weights stay as they are
        for t, i in zip(*np.nonzero(~keep)):
            W[t, sel[t, i]] = 0.0
    out = np.zeros((x.shape[0], wd.shape[2]))
    for e in range(wg.shape[0]):
        out += W[:, e:e + 1] * bf_ffn(x, wg[e].astype(np.float64), wu[e].astype(np.float64),
                                      wd[e].astype(np.float64))
    if ws is not None:
        out += bf_ffn(x, *[w.astype(np.float64) for w in ws])
    return out


def tiny_problem(T, E, k, d, h, hs, dtype, seed):
    p = Problem(T, E, k, d, h, hs, dtype, 4)
    inp = make_inputs(p, seed=seed, with_grad_out=True)
    return p, {n: t.value for n, t in inp.items()}


def shared_of(v):
    if "ws_gate" in v:
        return (v["ws_gate"], v["ws_up"], v["ws_down"])
    return None


GRID = [
    # T, E, k, d, h, hs, dtype
    (1, 1, 1, 4, 3, 0, "fp32"),
    (7, 2, 1, 8, 5, 0, "fp32"),
    (13, 2, 2, 8, 4, 3, "bf16"),
    (33, 4, 2, 16, 8, 0, "bf16"),
    (67, 8, 2, 16, 6, 5, "fp32"),
    (40, 8, 4, 12, 8, 0, "bf16"),
    (19, 64, 8, 32, 4, 6, "bf16"),
    (25, 5, 5, 8, 3, 0, "fp32"),
]


# ----------------------------------------------------------------- pins

def test_param_count_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "pages_params.json")))
    for c in g["cases"]:
        assert oracle.param_count(c["experts"], c["d_model"], c["d_hidden"], c["shared"]) == c["params"]


def test_param_count_equals_generated_tensor_sizes():
    p = Problem(3, 4, 2, 6, 5, 7, "fp32", 4)
    inp = make_inputs(p, seed=1)
    assert sum(t.value.size for t in inp.values()) == oracle.param_count(4, 6, 5, 7) + 3 * 6


@pytest.mark.parametrize("T,E,k,d,h,hs,dtype", GRID)
def test_logits_within_fp32_bound_of_exact_dot(T, E, k, d, h, hs, dtype):
    _, v = tiny_problem(T, E, k, d, h, hs, dtype, seed=3)
    logits, _, _ = oracle.route(v["x"], v["w_router"], k)
    x64, w64 = v["x"].astype(np.float64), v["w_router"].astype(np.float64)
    exact = x64 @ w64
    # Sequential fused multiply-add chain: |err| <= d * u * sum|x_j w_j| (u = 2^-24).
    bound = d * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64)) + 1e-30
    assert np.all(np.abs(logits.astype(np.float64) - exact) <= bound)


@pytest.mark.parametrize("T,E,k,d,h,hs,dtype", GRID)
def test_forward_matches_dense_brute_force(T, E, k, d, h, hs, dtype):
    _, v = tiny_problem(T, E, k, d, h, hs, dtype, seed=11)
    logits, idx, w = oracle.route(v["x"], v["w_router"], k)
    sel = bf_select(logits.astype(np.float64), k)
    assert np.array_equal(sel, idx)
    Wd = bf_mask_weights(logits.astype(np.float64), sel)
    assert np.allclose(np.take_along_axis(Wd, sel, 1), w, rtol=1e-13, atol=0)
    out = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w,
                              *(shared_of(v) or (None, None, None)))
    ref = bf_forward(v["x"], v["w_router"], v["w_gate"], v["w_up"], v["w_down"], sel, shared_of(v),
                     logits64=logits.astype(np.float64))
    assert oracle.rel_err(out, ref) < 1e-12


def test_forward_rows_subset_equals_full():
    _, v = tiny_problem(20, 4, 2, 8, 5, 3, "bf16", seed=5)
    _, idx, w = oracle.route(v["x"], v["w_router"], 2)
    full, y = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w,
                                  *shared_of(v), want_y=True)
    rows = [19, 0, 7, 7]
    sub = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w, *shared_of(v),
                              rows=rows)
    assert np.array_equal(sub, full[rows])
    # y per flat slot is the unweighted expert FFN of the token
    x64 = v["x"].astype(np.float64)
    for t in (0, 13):
        for i in range(2):
            e = idx[t, i]
            ref = bf_ffn(x64[t:t + 1], v["w_gate"][e].astype(np.float64),
                         v["w_up"][e].astype(np.float64), v["w_down"][e].astype(np.float64))[0]
            assert np.allclose(y[t * 2 + i], ref, rtol=1e-12, atol=1e-14)


def test_zero_router_tie_break():
    """All logits +0.0: experts 0..k-1 in index order, weights exactly 1/k."""
    _, v = tiny_problem(9, 6, 3, 8, 4, 0, "fp32", seed=2)
    logits, idx, w = oracle.route(v["x"], np.zeros_like(v["w_router"]), 3)
    assert np.all(logits == 0)
    assert np.array_equal(idx, np.tile(np.arange(3, dtype=np.int32), (9, 1)))
    assert np.all(w == 1.0 / 3.0)
    out = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w)
    x64 = v["x"].astype(np.float64)
    ref = sum(bf_ffn(x64, *(v[n][e].astype(np.float64) for n in ("w_gate", "w_up", "w_down")))
              for e in range(3)) / 3.0
    assert oracle.rel_err(out, ref) < 1e-13


def test_duplicate_logits_lowest_index_wins():
    """Identical router columns give bit-identical logits; the lower index ranks first."""
    rng = np.random.default_rng(0)
    T, d, E, k = 50, 16, 8, 4
    x = rng.standard_normal((T, d)).astype(np.float32)
    base = rng.standard_normal((d, 3)).astype(np.float32)
    wr = base[:, [0, 1, 0, 2, 1, 0, 2, 2]].copy()  # duplicated columns
    logits, idx, _ = oracle.route(x, wr, k)
    for t in range(T):
        assert logits[t, 0] == logits[t, 2] == logits[t, 5]
    assert np.array_equal(idx, bf_select(logits.astype(np.float64), k))


def test_k_equals_E_is_plain_softmax_mixture():
    _, v = tiny_problem(15, 4, 4, 8, 5, 0, "fp32", seed=8)
    logits, idx, w = oracle.route(v["x"], v["w_router"], 4)
    out = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w)
    x64 = v["x"].astype(np.float64)
    p = softmax(logits.astype(np.float64), axis=1)
    ref = sum(p[:, e:e + 1] * bf_ffn(x64, *(v[n][e].astype(np.float64)
                                            for n in ("w_gate", "w_up", "w_down"))) for e in range(4))
    assert oracle.rel_err(out, ref) < 1e-13
    # selection lists every expert, in descending-logit order
    assert np.all(np.sort(idx, axis=1) == np.arange(4))


def test_single_expert_is_textbook_swiglu():
    _, v = tiny_problem(11, 1, 1, 8, 6, 0, "bf16", seed=4)
    _, idx, w = oracle.route(v["x"], v["w_router"], 1)
    assert np.all(idx == 0) and np.all(w == 1.0)
    out = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w)
    x = v["x"].astype(np.float64)
    a = x @ v["w_gate"][0].astype(np.float64)
    b = x @ v["w_up"][0].astype(np.float64)
    ref = (a / (1 + np.exp(-a)) * b) @ v["w_down"][0].astype(np.float64)
    assert oracle.rel_err(out, ref) < 1e-13


def test_identical_experts_route_invariant():
    _, v = tiny_problem(12, 4, 2, 8, 5, 0, "fp32", seed=6)
    for n in ("w_gate", "w_up", "w_down"):
        v[n] = np.repeat(v[n][:1], 4, axis=0)
    _, idx, w = oracle.route(v["x"], v["w_router"], 2)
    out = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w)
    x = v["x"].astype(np.float64)
    ref = bf_ffn(x, v["w_gate"][0].astype(np.float64), v["w_up"][0].astype(np.float64),
                 v["w_down"][0].astype(np.float64))
    assert oracle.rel_err(out, ref) < 1e-13
    g = oracle.backward(v["x"], v["w_router"], v["w_gate"], v["w_up"], v["w_down"], v["grad_out"],
                        idx, w)
    assert np.max(np.abs(g["w_router"])) < 1e-12 * max(1.0, np.max(np.abs(g["w_gate"])))


def test_top1_router_gradient_is_exactly_zero():
    _, v = tiny_problem(10, 4, 1, 8, 5, 0, "fp32", seed=9)
    _, idx, w = oracle.route(v["x"], v["w_router"], 1)
    assert np.all(w == 1.0)
    g = oracle.backward(v["x"], v["w_router"], v["w_gate"], v["w_up"], v["w_down"], v["grad_out"],
                        idx, w)
    assert np.all(g["w_router"] == 0.0)
    # with a zero router, dx has no router term either: compare against no-router FD below
    zero = oracle.backward(v["x"], np.zeros_like(v["w_router"]), v["w_gate"], v["w_up"],
                           v["w_down"], v["grad_out"], idx, w)
    assert np.array_equal(zero["x"], g["x"])


@pytest.mark.parametrize("T,E,k", [(12, 4, 1), (30, 8, 2), (16, 5, 3)])
def test_constructed_permutation(T, E, k):
    """x[t] has a single spike at column t mod E and W_r = I: token t's
    logits are +1 at expert t mod E and +0 elsewhere, so it keeps t mod E
    and then the lowest other indices."""
    d = E + 3
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), np.arange(T) % E] = 1.0
    wr = np.zeros((d, E), np.float32)
    wr[np.arange(E), np.arange(E)] = 1.0
    _, idx, _ = oracle.route(x, wr, k)
    want = np.empty((T, k), np.int64)
    for t in range(T):
        top = t % E
        rest = [e for e in range(E) if e != top][: k - 1]
        want[t] = [top] + rest
    assert np.array_equal(idx, want)
    bm = 3
    r = oracle.permute(idx, E, bm)
    counts = np.bincount(want.ravel(), minlength=E)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    # closed form of the sorted order: experts ascending, flat slots ascending
    flat = [s for e in range(E) for s in range(T * k) if want.ravel()[s] == e]
    assert np.array_equal(r["perm"], np.array(flat))
    assert r["num_tiles"] == sum(math.ceil(c / bm) for c in counts)


def check_permutation_invariants(idx, E, bm, r):
    T, k = idx.shape
    S = T * k
    perm, inv = r["perm"], r["inv_perm"]
    assert np.array_equal(np.sort(perm), np.arange(S))
    assert np.array_equal(inv[perm], np.arange(S))
    ex = idx.ravel()[perm]
    assert np.all(np.diff(ex) >= 0)
    for e in range(E):
        seg = perm[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ex[r["offsets"][e]:r["offsets"][e + 1]] == e)
    assert r["counts"].sum() == S
    assert all(len(set(row)) == k for row in idx.tolist())
    covered = np.zeros(S, np.int64)
    for e, r0, rows in r["tiles"]:
        assert 1 <= rows <= bm
        assert r["offsets"][e] <= r0 and r0 + rows <= r["offsets"][e + 1]
        covered[r0:r0 + rows] += 1
    assert np.all(covered == 1)
    assert r["num_tiles"] == sum(math.ceil(c / bm) for c in r["counts"])


@pytest.mark.parametrize("T,E,k,bm", [(1, 1, 1, 32), (67, 8, 2, 4), (300, 64, 8, 32), (129, 7, 3, 64)])
def test_permutation_invariants(T, E, k, bm):
    rng = np.random.default_rng(T + E)
    x = rng.standard_normal((T, 8)).astype(np.float32)
    wr = rng.standard_normal((8, E)).astype(np.float32)
    _, idx, w = oracle.route(x, wr, k)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    check_permutation_invariants(idx, E, bm, oracle.permute(idx, E, bm))


def test_permute_rejects_bad_index():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 5]], np.int32), 4, 32)


# ------------------------------------------------------ capacity routing
# kernel_gmm_gpu.json records with "routing": "capacity" (the pages define
# neither the capacity nor the drop rule): an expert keeps its first C slots
# in flat slot order t*k + i.

def bf_keep(sel, E, C):
    """Independent drop rule: a slot's position within its expert is the
    running count of that expert over the flat slots up to it (cumulative
    one-hot sums); capacity C keeps positions < C (C = 0: every slot)."""
    T, k = sel.shape
    flat = sel.reshape(-1)
    onehot = np.zeros((T * k, E), np.int64)
    onehot[np.arange(T * k), flat] = 1
    pos = np.cumsum(onehot, axis=0)[np.arange(T * k), flat] - 1
    return (pos < C).reshape(T, k) if C > 0 else np.ones((T, k), bool)


@pytest.mark.parametrize("T,E,k,bm,C", [(67, 8, 2, 4, 9), (300, 64, 8, 32, 30), (129, 7, 3, 64, 1),
                                        (50, 4, 2, 8, 25), (40, 5, 5, 16, 13)])
def test_capacity_permute_matches_cumulative_count(T, E, k, bm, C):
    rng = np.random.default_rng(T + C)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    full = oracle.permute(idx, E, bm)
    r = oracle.permute(idx, E, bm, capacity=C)
    keep = oracle.keep_mask(r, T, k)
    assert np.array_equal(keep, bf_keep(idx, E, C))
    # the sorted order is the dropless one; dropped slots lose their row
    assert np.array_equal(r["perm"], full["perm"]) and np.array_equal(r["offsets"], full["offsets"])
    flat_keep = keep.reshape(-1)
    assert np.array_equal(r["inv_perm"][flat_keep], full["inv_perm"][flat_keep])
    assert np.all(r["inv_perm"][~flat_keep] == -1)
    # tiles cover exactly each expert's first min(count, C) rows, in block_m pieces
    kept = np.minimum(r["counts"], C)
    assert kept.sum() == flat_keep.sum()
    expect = [(e, r["offsets"][e] + q, min(bm, kept[e] - q)) for e in range(E)
              for q in range(0, kept[e], bm)]
    assert r["num_tiles"] == len(expect)
    assert np.array_equal(r["tiles"], np.array(expect, np.int32).reshape(-1, 3))


def test_capacity_at_least_the_largest_load_is_dropless():
    _, v = tiny_problem(40, 8, 2, 12, 6, 4, "bf16", seed=9)
    _, idx, w = oracle.route(v["x"], v["w_router"], 2)
    full = oracle.permute(idx, 8, 4)
    C = int(full["counts"].max())
    r = oracle.permute(idx, 8, 4, capacity=C)
    for n in ("perm", "inv_perm", "offsets", "tiles"):
        assert np.array_equal(r[n], full[n])
    keep = oracle.keep_mask(r, 40, 2)
    assert keep.all()
    a = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w, *shared_of(v), keep=keep)
    b = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w, *shared_of(v))
    assert np.array_equal(a, b)
    r1 = oracle.permute(idx, 8, 4, capacity=C - 1)
    assert not oracle.keep_mask(r1, 40, 2).all()


@pytest.mark.parametrize("T,E,k,d,h,hs,dtype,C", [(33, 4, 2, 16, 8, 0, "bf16", 10),
                                                  (67, 8, 2, 16, 6, 5, "fp32", 12),
                                                  (40, 8, 4, 12, 8, 0, "bf16", 15),
                                                  (19, 64, 8, 32, 4, 6, "bf16", 2)])
def test_capacity_forward_matches_dense_brute_force(T, E, k, d, h, hs, dtype, C):
    _, v = tiny_problem(T, E, k, d, h, hs, dtype, seed=13)
    logits, idx, w = oracle.route(v["x"], v["w_router"], k)
    sel = bf_select(logits.astype(np.float64), k)
    keep = bf_keep(sel, E, C)
    assert not keep.all()
    out, y = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w,
                                 *(shared_of(v) or (None, None, None)), want_y=True, keep=keep)
    ref = bf_forward(v["x"], v["w_router"], v["w_gate"], v["w_up"], v["w_down"], sel, shared_of(v),
                     logits64=logits.astype(np.float64), keep=keep)
    assert oracle.rel_err(out, ref) < 1e-12
    assert np.all(y[~keep.reshape(-1)] == 0.0)


def test_capacity_zero_router_closed_form():
    """All-zero router: every token picks experts 0..k-1 with weight 1/k, so
    with capacity C exactly tokens 0..C-1 reach the experts and the rest get
    the shared expert alone."""
    T, E, k, C = 10, 4, 2, 6
    _, v = tiny_problem(T, E, k, 8, 5, 3, "fp32", seed=2)
    wr = np.zeros_like(v["w_router"])
    _, idx, w = oracle.route(v["x"], wr, k)
    r = oracle.permute(idx, E, 4, capacity=C)
    keep = oracle.keep_mask(r, T, k)
    assert keep[:C].all() and not keep[C:].any()
    out = oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w, *shared_of(v),
                              keep=keep)
    x = v["x"].astype(np.float64)
    sh = bf_ffn(x, *[a.astype(np.float64) for a in shared_of(v)])
    ex = sum(bf_ffn(x, v["w_gate"][e].astype(np.float64), v["w_up"][e].astype(np.float64),
                    v["w_down"][e].astype(np.float64)) for e in range(k)) / k
    ref = sh.copy()
    ref[:C] += ex[:C]
    assert oracle.rel_err(out, ref) < 1e-12


# ------------------------------------------------------ finite differences

def fd_loss(v, sel, hs, keep=None):
    """L = sum(out * G) through the dense brute force, selection (and any
    capacity drops) frozen, logits in double."""
    out = bf_forward(v["x"], v["w_router"], v["w_gate"], v["w_up"], v["w_down"], sel,
                     shared_of(v) if hs else None, keep=keep)
    return float(np.sum(out * v["grad_out"].astype(np.float64)))


@pytest.mark.parametrize("T,E,k,d,h,hs,C", [(3, 2, 1, 4, 3, 0, 0), (4, 3, 2, 5, 4, 2, 0),
                                            (5, 4, 2, 8, 6, 3, 0), (2, 4, 4, 6, 2, 0, 0),
                                            (6, 3, 2, 5, 4, 2, 3), (5, 2, 2, 4, 3, 0, 3)])
def test_gradients_match_central_differences(T, E, k, d, h, hs, C):
    _, v = tiny_problem(T, E, k, d, h, hs, "fp32", seed=21)
    v = {n: a.astype(np.float64) for n, a in v.items()}
    logits, idx, w = oracle.route(v["x"].astype(np.float32), v["w_router"].astype(np.float32), k)
    sel = idx.astype(np.int64)
    keep = bf_keep(sel, E, C) if C else None
    if C:
        assert not keep.all()
    g = oracle.backward(v["x"], v["w_router"], v["w_gate"], v["w_up"], v["w_down"], v["grad_out"],
                        idx, w, *(shared_of(v) if hs else (None, None, None)), keep=keep)
    eps = 1e-6
    names = ["x", "w_router", "w_gate", "w_up", "w_down"] + (["ws_gate", "ws_up", "ws_down"] if hs else [])
    for n in names:
        base = v[n]
        fd = np.empty_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = base[mi]
            base[mi] = old + eps
            lp = fd_loss(v, sel, hs, keep)
            base[mi] = old - eps
            lm = fd_loss(v, sel, hs, keep)
            base[mi] = old
            fd[mi] = (lp - lm) / (2 * eps)
        # the oracle's weights come from fp32 logits, the brute force from double ones
        assert oracle.rel_err(g[n], fd) < 2e-6, n


# ------------------------------------------------------ statistical sanity

def test_routing_statistics_in_pages_band():
    """Plausibility only (not parity): the pages report max_expert_frac
    0.128-0.136 and no empty experts at 4096 tokens, E=8, top-2
    (kernel_gmm_gpu.json, layer-suite records)."""
    p = Problem(4096, 8, 2, 512, 1024, 0, "fp32")
    inp = make_inputs(p, seed=0, names=["x", "w_router"])
    _, idx, _ = oracle.route(inp["x"].value, inp["w_router"].value, 2)
    c = np.bincount(idx.ravel(), minlength=8)
    frac = c.max() / idx.size
    assert 0.125 < frac < 0.16 and np.all(c > 0)
