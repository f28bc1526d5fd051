"""Streams and graphs around the C ABI (GPU): moe_forward and moe_bwd fork the
shared expert onto the caller's second stream and join it back with events
made for the call. Concurrent callers, each with its own pair of streams,
must get the same bits as a lone call, and the whole train step must replay
from a captured HIP graph with the results of eager calls, replay after
replay."""

import threading

import pytest

from dropless_grouped_gemm_router_amd import binding as B
from dropless_grouped_gemm_router_amd.inputs import Problem, make_inputs

from gpu_util import Case, note

pytestmark = pytest.mark.gpu


def bits_equal(a, b) -> bool:
    import torch
    return a.shape == b.shape and torch.equal(a.contiguous().view(torch.uint8),
                                              b.contiguous().view(torch.uint8))


def test_concurrent_host_threads_match_lone_calls():
    """Two host threads, each on its own stream with its own buffers, call
    moe_forward repeatedly at the same time (ctypes releases the GIL)."""
    import torch
    probs = [Problem(3000, 16, 4, 256, 128, 256, "bf16", 256),
             Problem(2000, 8, 2, 512, 128, 128, "bf16", 128)]
    cases = [Case(p, seed=20 + i) for i, p in enumerate(probs)]
    refs = []
    for c in cases:
        buf = B.allocate(c.p, dispatch="gather")
        B.forward_dispatch(c.p, "gather", c.dev["x"], c.weights(), buf)
        torch.cuda.synchronize()
        refs.append(buf.out.clone())
    bufs = [B.allocate(c.p, dispatch="gather") for c in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    sides = [torch.cuda.Stream() for _ in cases]
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(6):
                    B.forward_dispatch(cases[i].p, "gather", cases[i].dev["x"], cases[i].weights(),
                                       bufs[i], side_stream=sides[i])
            streams[i].synchronize()
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for ref, buf in zip(refs, bufs):
        assert bits_equal(ref, buf.out)


def test_back_to_back_forwards_use_their_own_weights():
    """moe_forward packs the routed weights into the workspace on the second
    stream, and the routed GEMMs wait for that. Calls in a row on one stream
    and one workspace, alternating two weight sets with no synchronisation
    in between, must each give the bits of a lone call with their weights:
    a call's pack may neither overtake the previous call's GEMMs nor be
    overtaken by its own."""
    import torch
    p = Problem(3000, 16, 4, 256, 128, 256, "bf16", 256)
    cases = [Case(p, seed=31), Case(p, seed=32)]
    refs = []
    for c in cases:
        buf = B.allocate(p, dispatch="gather")
        B.forward_dispatch(p, "gather", c.dev["x"], c.weights(), buf)
        torch.cuda.synchronize()
        refs.append(buf.out.clone())
    assert not bits_equal(refs[0], refs[1])
    buf = B.allocate(p, dispatch="gather")
    side = torch.cuda.Stream()
    outs = []
    for i in range(6):
        c = cases[i % 2]
        B.forward_dispatch(p, "gather", c.dev["x"], c.weights(), buf, side_stream=side)
        outs.append(buf.out.clone())  # the current stream, after the call
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert bits_equal(refs[i % 2], o), f"call {i}"


def test_late_fork_gives_one_stream_bits():
    """From 65536 tokens on, moe_forward packs and permutes on the caller's
    stream and forks the shared expert only then. Two weight sets
    alternating on one workspace (forward and train step) must give the
    bits of one-stream calls."""
    import torch
    p = Problem(65536, 16, 2, 256, 128, 256, "bf16", 256)
    cases = [Case(p, seed=41, training=True), Case(p, seed=42, training=True)]
    refs = []
    for c in cases:
        buf = B.allocate(p, training=True, dispatch="gather")
        B.forward_dispatch(p, "gather", c.dev["x"], c.weights(), buf, training=True)
        B.backward(p, c.dev["x"], c.weights(), c.dev["grad_out"], buf)
        torch.cuda.synchronize()
        refs.append([buf.out.clone(), buf.grad_x.clone()] + [t.clone() for t in buf.grads.values()])
    assert not bits_equal(refs[0][0], refs[1][0])
    buf = B.allocate(p, training=True, dispatch="gather")
    side = torch.cuda.Stream()
    for i in range(4):
        c = cases[i % 2]
        B.forward_dispatch(p, "gather", c.dev["x"], c.weights(), buf, training=True,
                           side_stream=side)
        B.backward(p, c.dev["x"], c.weights(), c.dev["grad_out"], buf, side_stream=side)
        got = [buf.out.clone(), buf.grad_x.clone()] + [t.clone() for t in buf.grads.values()]
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(refs[i % 2], got)):
            assert bits_equal(a, b), f"call {i}, output {j}"


def test_train_step_replays_from_a_hip_graph():
    """Forward (with saved activations) and backward captured once, replayed
    on new token values; every replay equals the eager step bit for bit."""
    import torch
    p = Problem(1500, 8, 2, 256, 128, 128, "bf16", 128)
    c = Case(p, seed=31, training=True)
    w = c.weights()
    x_buf = c.dev["x"].clone()
    g_buf = c.dev["grad_out"].clone()
    buf = B.allocate(p, training=True, dispatch="gather")
    side = torch.cuda.Stream()

    def step():
        B.forward_dispatch(p, "gather", x_buf, w, buf, training=True, side_stream=side)
        B.backward(p, x_buf, w, g_buf, buf, side_stream=side)

    def snapshot():
        return [buf.out.clone(), buf.grad_x.clone()] + [t.clone() for t in buf.grads.values()]

    # Warm up on a stream of its own, then capture.
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for seed in (41, 42, 43):
        note(f"graph replay, inputs seed {seed}")
        fresh = B.device_inputs(make_inputs(p, seed=seed, with_grad_out=True))
        x_buf.copy_(fresh["x"])
        g_buf.copy_(fresh["grad_out"])
        torch.cuda.synchronize()
        step()  # eager, between replays
        torch.cuda.synchronize()
        eager = snapshot()
        graph.replay()
        torch.cuda.synchronize()
        replayed = snapshot()
        for a, b in zip(eager, replayed):
            assert bits_equal(a, b)


def test_kernel_timer_mode_gives_the_same_bits():
    """With libmoe's kernel timer on, moe_forward and moe_bwd ignore the
    second stream and run the shared expert's part on the caller's stream
    (so every recorded duration is a kernel's own): the same kernels in
    issue order, so the same bits as the two-stream call, and every kernel
    of the step is recorded."""
    import torch
    p = Problem(1500, 8, 2, 256, 128, 128, "bf16", 128)
    c = Case(p, seed=37, training=True)
    w = c.weights()
    buf = B.allocate(p, training=True, dispatch="gather")

    def step():
        B.forward_dispatch(p, "gather", c.dev["x"], w, buf, training=True, side_stream=c.side)
        B.backward(p, c.dev["x"], w, c.dev["grad_out"], buf, side_stream=c.side)
        torch.cuda.synchronize()
        return [buf.out.clone(), buf.grad_x.clone()] + [t.clone() for t in buf.grads.values()]

    plain = step()
    B.moe_trace_enable(True)
    try:
        timed = step()
        kern = B.moe_trace_summary()
    finally:
        B.moe_trace_enable(False)
    for a, b in zip(plain, timed):
        assert bits_equal(a, b)
    for name in ("route", "gemm_gate_up", "gemm_down", "shared_gate_up", "shared_down", "combine",
                 "bwd_down_dgrad", "bwd_router_dl", "bwd_shared_down_dgrad", "bwd_wgrad_gate_up",
                 "bwd_dx"):
        assert name in kern and kern[name]["count"] >= 1, name
