"""libmoe on the host, no GPU: the library loads and exports every symbol
include/moe.h declares, host-side helpers, and every argument check, all of
which run before any HIP call."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

from dropless_grouped_gemm_router_amd import binding as B
from dropless_grouped_gemm_router_amd.inputs import Problem, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = B.load()
    names = declared_functions()
    assert len(names) == 17
    assert sorted(B.EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in B.moe_version()


def test_stage_probe_library_loads():
    """The wide engine's stage-loop probe (bench.py --stage-probe) is a
    library of its own, built beside libmoe; it rejects bad configurations
    on the host before touching a GPU."""
    lib = ctypes.CDLL(os.path.join(ROOT, "dropless_grouped_gemm_router_amd", "libmoe_probe.so"))
    fn = lib.moe_stage_probe
    fn.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    ms = ctypes.c_float(0.0)
    assert fn(11, 4096, 0, 0, 256, 16, 1, ctypes.byref(ms)) == -1     # no such mode
    assert fn(3, 100, 0, 0, 256, 16, 1, ctypes.byref(ms)) == -1       # region under one tile
    assert fn(3, (1 << 20) + 1, 0, 0, 256, 16, 1, ctypes.byref(ms)) == -1
    assert fn(3, 4096, 0, 2, 256, 16, 1, ctypes.byref(ms)) == -1      # no such data kind
    assert fn(3, 4096, 0, 0, 0, 16, 1, ctypes.byref(ms)) == -1
    assert fn(3, 4096, 0, 0, 256, 16, 1, None) == -1
    st = lib.moe_store_probe
    st.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    assert st(3, 1, ctypes.byref(ms)) == -1      # no such store order
    assert st(0, 0, ctypes.byref(ms)) == -1
    assert st(0, 1, None) == -1


def test_param_count_and_tiles():
    p = Problem(4096, 8, 2, 512, 1024, 0, "fp32", 64)
    assert B.moe_param_count(p) == 12587008  # gpu_nn.json, moe suite, "params"
    assert B.moe_max_tiles(p) == 8192 // 64 + 8
    p3 = WORKLOADS[3][1]
    assert B.moe_param_count(p3) == 3 * 64 * 512 * 128 + 512 * 64 + 3 * 512 * 1024
    assert B.moe_max_tiles(p3) == 131072 * 8 // p3.block_m + 64


@pytest.mark.parametrize("kw,code", [
    (dict(experts=0), B.MOE_ERR_INVALID),
    (dict(top_k=0), B.MOE_ERR_INVALID),
    (dict(top_k=9), B.MOE_ERR_INVALID),
    (dict(tokens=-1), B.MOE_ERR_INVALID),
    (dict(dtype=7), B.MOE_ERR_INVALID),
    (dict(d_shared=-64), B.MOE_ERR_INVALID),
    (dict(capacity=-1), B.MOE_ERR_INVALID),
    (dict(capacity=1), B.MOE_OK),
    (dict(experts=65, top_k=2), B.MOE_ERR_UNSUPPORTED),
    (dict(block_m=48), B.MOE_ERR_UNSUPPORTED),
    (dict(block_m=512), B.MOE_ERR_UNSUPPORTED),
    (dict(block_m=256), B.MOE_OK),
    (dict(d_model=500), B.MOE_ERR_UNSUPPORTED),
    (dict(d_hidden=100), B.MOE_ERR_UNSUPPORTED),
    (dict(d_shared=96), B.MOE_ERR_UNSUPPORTED),
    (dict(tokens=1 << 30, top_k=2), B.MOE_ERR_UNSUPPORTED),
    # tokens * top_k would overflow int64: rejected without forming it
    (dict(tokens=(1 << 62) + 1, top_k=8), B.MOE_ERR_UNSUPPORTED),
    (dict(tokens=(1 << 31) // 2 - 1, top_k=2), B.MOE_OK),
    (dict(), B.MOE_OK),
    (dict(tokens=0), B.MOE_OK),
])
def test_check_problem(kw, code):
    base = dict(tokens=10, experts=8, top_k=2, d_model=256, d_hidden=128, d_shared=0,
                dtype=B.MOE_BF16, block_m=64)
    base.update(kw)
    p = B.moe_problem(**base)
    assert B.load().moe_check_problem(ctypes.byref(p)) == code
    if code != B.MOE_OK:
        assert B.load().moe_workspace_bytes(ctypes.byref(p), 1) == 0
        assert B.load().moe_max_tiles(ctypes.byref(p)) == 0
        assert B.load().moe_param_count(ctypes.byref(p)) == -1


class FakeTensor:
    """Host stand-in with an arbitrary (never dereferenced) address."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def fake_routing(base=0x10000000):
    return {n: FakeTensor(base + i * 0x100000) for i, n in enumerate(
        ["topk_idx", "topk_w", "expert_offsets", "perm", "inv_perm", "tiles", "num_tiles"])}


def fake_weights(base=0x20000000, shared=True):
    names = ["w_router", "w_gate", "w_up", "w_down"] + (["ws_gate", "ws_up", "ws_down"] if shared else [])
    return {n: FakeTensor(base + i * 0x100000) for i, n in enumerate(names)}


P = Problem(100, 8, 2, 256, 128, 128, "bf16", 64)


def expect(code, fn, *a, **k):
    with pytest.raises(B.MoeError) as e:
        fn(*a, **k)
    assert e.value.status == code


def test_route_argument_errors():
    r = fake_routing()
    expect(B.MOE_ERR_INVALID, B.moe_route, P, None, FakeTensor(0x3000), r, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_route, P, FakeTensor(0x3008), FakeTensor(0x3000), r, stream=0)
    r2 = dict(r, topk_idx=None)
    expect(B.MOE_ERR_INVALID, B.moe_route, P, FakeTensor(0x3000), FakeTensor(0x3000), r2, stream=0)
    bad = Problem(100, 8, 9, 256, 128, 0, "bf16", 64)
    expect(B.MOE_ERR_INVALID, B.moe_route, bad, FakeTensor(0x3000), FakeTensor(0x3000), r, stream=0)
    # zero tokens: a successful no-op, pointers unused
    B.moe_route(Problem(0, 8, 2, 256, 128, 0, "bf16", 64), None, None, {}, stream=0)


def test_permute_argument_errors():
    r = fake_routing()
    need = B.moe_workspace_bytes(P)
    ws = FakeTensor(0x40000000)
    expect(B.MOE_ERR_WORKSPACE, B.moe_permute, P, r, ws, workspace_bytes=0, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_permute, P, r, FakeTensor(0x40000010), workspace_bytes=need,
           stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_permute, P, dict(r, perm=None), ws, workspace_bytes=need,
           stream=0)
    B.moe_permute(Problem(0, 8, 2, 256, 128, 0, "bf16", 64), {}, None, workspace_bytes=0, stream=0)


def test_permute_static_argument_errors():
    """The allocation-free permute checks everything on the host before it
    touches the device: bad pointers, and problems whose per-block counts
    would not fit its fixed 1 MiB scratch (64 experts x ceil(S / 4096)
    blocks x 4 bytes)."""
    r = fake_routing()
    expect(B.MOE_ERR_INVALID, B.moe_permute_static, P, dict(r, inv_perm=None), stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_permute_static, P, dict(r, tiles=FakeTensor(0x40000002)),
           stream=0)
    # 64 experts: 4096 blocks of 4096 slots fit, one more does not
    fits = Problem((1 << 24) // 8, 64, 8, 128, 64, 0, "bf16", 256)
    over = Problem((1 << 24) // 8 + 1, 64, 8, 128, 64, 0, "bf16", 256)
    assert fits.tokens * fits.top_k == 4096 * 4096
    expect(B.MOE_ERR_TOO_LARGE, B.moe_permute_static, over, r, stream=0)
    assert "fixed scratch" in B.status_string(B.MOE_ERR_TOO_LARGE)
    B.moe_permute_static(Problem(0, 8, 2, 256, 128, 0, "bf16", 64), {}, stream=0)


def test_ffn_and_combine_argument_errors():
    r, w = fake_routing(), fake_weights()
    ws = FakeTensor(0x40000000)
    need = B.moe_workspace_bytes(P)
    y, sh, out = FakeTensor(0x50000000), FakeTensor(0x51000000), FakeTensor(0x52000000)
    x = FakeTensor(0x53000000)
    expect(B.MOE_ERR_WORKSPACE, B.moe_ffn_fwd, P, x, w, r, y, sh, None, ws, workspace_bytes=need - 1,
           stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_ffn_fwd, P, x, fake_weights(shared=False), r, y, sh, None, ws,
           workspace_bytes=need, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_ffn_fwd, P, x, w, r, y, None, None, ws, workspace_bytes=need,
           stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_ffn_fwd, P, x, w, r, y, sh, FakeTensor(0x60000010), ws,
           workspace_bytes=need, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_combine, P, y, dict(r, inv_perm=None), sh, out, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_combine, P, y, r, FakeTensor(0x51000004), out, stream=0)


def test_forward_workspace_sizes():
    es = 2
    T, S, d = P.tokens, P.tokens * P.top_k, P.d_model
    base = B.moe_workspace_bytes(P)
    g = B.moe_forward_workspace_bytes(P, "gather")
    s = B.moe_forward_workspace_bytes(P, "sorted")
    f = B.moe_forward_workspace_bytes(P, "fused_gsum")
    # gather stages the shared output after the permute/FFN area, sorted also
    # the expert-ordered token copy, fused_gsum neither.
    assert g >= base + T * d * es
    assert s >= g + S * d * es
    assert base <= f < g
    # no shared expert or top_k > 8: fused_gsum needs what gather needs
    p0 = Problem(100, 8, 2, 256, 128, 0, "bf16", 64)
    assert B.moe_forward_workspace_bytes(p0, "fused_gsum") == B.moe_forward_workspace_bytes(p0, "gather")
    p9 = Problem(100, 16, 9, 256, 128, 128, "bf16", 64)
    assert B.moe_forward_workspace_bytes(p9, "fused_gsum") == B.moe_forward_workspace_bytes(p9, "gather")
    # training keeps the hidden activations in the saved buffer instead
    assert T * d * es < B.moe_forward_workspace_bytes(P, "gather", training=True) < g
    assert B.moe_forward_workspace_bytes(P, 3) == 0
    assert B.moe_forward_workspace_bytes(Problem(100, 8, 2, 500, 128, 0, "bf16", 64), 0) == 0


def test_forward_argument_errors():
    r, w = fake_routing(), fake_weights()
    ws = FakeTensor(0x40000000)
    y, out, x = FakeTensor(0x50000000), FakeTensor(0x52000000), FakeTensor(0x53000000)
    for disp in ("gather", "sorted", "fused_gsum"):
        need = B.moe_forward_workspace_bytes(P, disp)
        expect(B.MOE_ERR_WORKSPACE, B.moe_forward, P, disp, x, w, r, y, None, out, ws,
               workspace_bytes=need - 1, stream=0)
        expect(B.MOE_ERR_INVALID, B.moe_forward, P, disp, x, w, dict(r, tiles=None), y, None, out,
               ws, workspace_bytes=need, stream=0)
        expect(B.MOE_ERR_INVALID, B.moe_forward, P, disp, x, w, r, y, None, None, ws,
               workspace_bytes=need, stream=0)
        expect(B.MOE_ERR_INVALID, B.moe_forward, P, disp, x, fake_weights(shared=False), r, y, None,
               out, ws, workspace_bytes=need, stream=0)
        expect(B.MOE_ERR_INVALID, B.moe_forward, P, disp, x, w, r, y, FakeTensor(0x60000010), out,
               ws, workspace_bytes=need, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_forward, P, 3, x, w, r, y, None, out, ws,
           workspace_bytes=1 << 40, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_forward, P, -1, x, w, r, y, None, out, ws,
           workspace_bytes=1 << 40, stream=0)
    B.moe_forward(Problem(0, 8, 2, 256, 128, 0, "bf16", 64), "fused_gsum", None, {}, {}, None, None,
                  None, None, workspace_bytes=0, stream=0)


def test_bwd_argument_errors():
    r, w = fake_routing(), fake_weights()
    g = {n: FakeTensor(0x70000000 + i * 0x100000) for i, n in
         enumerate(["w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"])}
    a = [FakeTensor(0x50000000), FakeTensor(0x54000000), FakeTensor(0x55000000),
         FakeTensor(0x56000000)]
    x = FakeTensor(0x53000000)
    ws = FakeTensor(0x40000000)
    need = B.moe_workspace_bytes(P, training=True)
    expect(B.MOE_ERR_INVALID, B.moe_bwd, P, x, w, r, a[0], a[1], a[2], a[3], dict(g, ws_up=None),
           ws, workspace_bytes=need, stream=0)
    expect(B.MOE_ERR_INVALID, B.moe_bwd, P, x, w, r, a[0], None, a[2], a[3], g, ws,
           workspace_bytes=need, stream=0)
    assert need > B.moe_workspace_bytes(P, training=False)
    expect(B.MOE_ERR_WORKSPACE, B.moe_bwd, P, x, w, r, a[0], a[1], a[2], a[3], g, ws,
           workspace_bytes=need - 1, stream=0)
    # y_sorted: required in fp32, not read (may be NULL) in bf16
    p32 = Problem(100, 8, 2, 256, 128, 128, "fp32", 64)
    need32 = B.moe_workspace_bytes(p32, training=True)
    expect(B.MOE_ERR_INVALID, B.moe_bwd, p32, x, w, r, None, a[1], a[2], a[3], g, ws,
           workspace_bytes=need32, stream=0)
    expect(B.MOE_ERR_WORKSPACE, B.moe_bwd, P, x, w, r, None, a[1], a[2], a[3], g, ws,
           workspace_bytes=need - 1, stream=0)
    # the backward tiles hidden widths by 128
    p64 = Problem(100, 8, 2, 256, 192, 128, "bf16", 64)
    expect(B.MOE_ERR_UNSUPPORTED, B.moe_bwd, p64, x, w, r, a[0], a[1], a[2], a[3], g, ws,
           workspace_bytes=need, stream=0)


def test_buffer_layouts_match_pages_argument_bytes():
    """The stage inputs have the byte sizes the pages' 'pieces' records
    report: storage-dtype tokens with an fp32 router, storage-dtype sorted
    rows [T*k, d] and weights, fp32 combine weights."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_arg_bytes.json")))
    for c in g["cases"]:
        dt = "fp32" if c["dtype"] == "float32" else "bf16"
        p = Problem(c["tokens"], 8, 2, 512, 1024, 0, dt, 64)
        b = B.allocate(p, device="cpu")
        es = 4 if dt == "fp32" else 2
        x_bytes = p.tokens * p.d_model * es
        w_bytes = 3 * p.experts * p.d_model * p.d_hidden * es
        if c["piece"] == "route":
            got = x_bytes + p.d_model * p.experts * 4  # w_router is fp32
        elif c["piece"] == "experts_grouped_swiglu":
            got = b.y_sorted.numel() * b.y_sorted.element_size() + w_bytes
        else:
            got = (b.y_sorted.numel() * b.y_sorted.element_size()
                   + b.routing["topk_w"].numel() * b.routing["topk_w"].element_size())
        assert got == int(round(c["xla_arg_mb"] * 2 ** 20)), c


@pytest.mark.parametrize("p", [Problem(100, 8, 2, 256, 128, 128, "bf16", 64),
                               Problem(300, 8, 2, 512, 1024, 0, "bf16", 128),
                               Problem(77, 5, 3, 128, 128, 64, "fp32", 32)])
def test_train_footprint_equals_allocation(p):
    """The max-token measurement's footprint model counts exactly what a train
    step allocates: the generated inputs with grad_out and every buffer of
    binding.allocate(training=True)."""
    import bench
    from dropless_grouped_gemm_router_amd.inputs import make_inputs
    b = B.allocate(p, device="cpu", training=True)
    tensors = [b.y_sorted, b.out, b.workspace, b.saved, b.grad_x] + list(b.routing.values())
    tensors += list(b.grads.values()) + ([b.shared_out] if p.d_shared else [])
    got = sum(t.numel() * t.element_size() for t in tensors)
    es = 2 if p.dtype == "bf16" else 4
    got += sum(t.value.size * (4 if n == "w_router" else es)
               for n, t in make_inputs(p, seed=0, with_grad_out=True).items())
    assert bench.train_footprint(B, p) == got


def test_training_workspace_for_narrow_shared_width():
    """d_shared 64 is below the backward's 128-column tile: moe_bwd rejects
    it, but sizing the training forward's workspace must still work."""
    p = Problem(77, 5, 3, 128, 128, 64, "bf16", 32)
    assert B.moe_workspace_bytes(p, True) >= B.moe_workspace_bytes(p, False) > 0


def test_kernel_source_hash_ignores_comments_only():
    """The stored FETCH/WRITE counters stay valid across comment edits and go
    stale on any code change: the hash strips comments (not string or
    character literals that hold comment markers) and blank lines."""
    import bench
    a = 'int a = 1;  // note\n/* block\n comment */ const char* s = "//x/*y*/";\n\nchar c = \'/\';\n'
    b = 'int a = 1;\nconst char* s = "//x/*y*/";\nchar c = \'/\';   // other note\n'
    assert bench.strip_comments(a) == 'int a = 1;\n const char* s = "//x/*y*/";\nchar c = \'/\';'
    assert bench.strip_comments(b) == 'int a = 1;\nconst char* s = "//x/*y*/";\nchar c = \'/\';'
    assert bench.strip_comments("x = 2; // y\n") != bench.strip_comments("x = 3; // y\n")
    assert "gemm_dgrad.h" in bench.KERNEL_SOURCES
    assert len(bench.kernel_source_hash()) == 16
