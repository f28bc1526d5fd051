"""Python front of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding. It
shares no code with the HIP path; only the seeded input generator
(``dropless_grouped_gemm_router_amd.inputs``, which holds no layer arithmetic)
feeds both.

Every function takes the *stored* input values widened exactly to fp32
(``Tensor.value``) and returns float64 results (fp32 logits, int32 indices).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over tokens / experts)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fvisibility=hidden",
               "-ffp-contract=off", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.oracle_param_count.restype = i64
        lib.oracle_param_count.argtypes = [i64, i64, i64, i64]
        lib.oracle_max_threads.restype = i32
        lib.oracle_route.restype = i32
        lib.oracle_route.argtypes = [i64, i32, i32, i32, P, P, P, P, P, i32]
        lib.oracle_permute.restype = i64
        lib.oracle_permute.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P]
        lib.oracle_forward_rows.restype = i32
        lib.oracle_forward_rows.argtypes = [i64, P, i32, i32, i32, i32, i32] + [P] * 10 + [P, P, i32]
        lib.oracle_backward.restype = i32
        lib.oracle_backward.argtypes = [i64, i32, i32, i32, i32, i32] + [P] * 12 + [P] * 8 + [i32]
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def param_count(E: int, d: int, h: int, hs: int = 0) -> int:
    return int(_load().oracle_param_count(E, d, h, hs))


def route(x: np.ndarray, w_router: np.ndarray, k: int, nthreads: int = 0):
    """Returns (logits fp32 [T,E], topk_idx int32 [T,k], topk_w float64 [T,k])."""
    x = _f32(x)
    wr = _f32(w_router)
    T, d = x.shape
    E = wr.shape[1]
    logits = np.empty((T, E), np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _load().oracle_route(T, d, E, k, _p(x), _p(wr), _p(logits), _p(idx), _p(w), nthreads)
    return logits, idx, w


def max_tiles(T: int, k: int, E: int, bm: int) -> int:
    return (T * k + bm - 1) // bm + E


def permute(topk_idx: np.ndarray, E: int, bm: int, capacity: int = 0) -> Dict[str, np.ndarray]:
    """Stable grouping by expert and the tile list; with capacity > 0 each
    expert keeps its first ``capacity`` slots (inv_perm -1 for the others)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    S = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(S, np.int32)
    inv = np.empty(S, np.int32)
    tiles = np.empty((max_tiles(T, k, E, bm), 3), np.int32)
    n = _load().oracle_permute(T, k, E, bm, int(capacity), _p(idx), _p(counts), _p(offsets),
                               _p(perm), _p(inv), _p(tiles))
    if n < 0:
        raise ValueError("expert index out of range")
    return dict(counts=counts, offsets=offsets, perm=perm, inv_perm=inv, tiles=tiles[:n].copy(),
                num_tiles=int(n))


def keep_mask(perm: Dict[str, np.ndarray], T: int, k: int) -> np.ndarray:
    """[T, k] flags of the slots a capacity-routed permute kept."""
    return (perm["inv_perm"] >= 0).reshape(T, k)


def _keep(keep, T, k):
    return None if keep is None else np.ascontiguousarray(np.asarray(keep).reshape(T, k), np.uint8)


def forward_rows(x, w_gate, w_up, w_down, topk_idx, topk_w, ws_gate=None, ws_up=None,
                 ws_down=None, rows: Optional[Sequence[int]] = None, want_y: bool = False,
                 nthreads: int = 0, keep=None):
    """Output rows (float64). ``rows`` selects tokens (default: all);
    ``keep`` ([T, k] flags) marks the slots capacity routing kept."""
    x = _f32(x)
    T, d = x.shape
    E, _, h = w_gate.shape
    k = topk_idx.shape[1]
    hs = 0 if ws_gate is None else ws_gate.shape[1]
    wg, wu, wd = _f32(w_gate), _f32(w_up), _f32(w_down)
    wsg = _f32(ws_gate) if hs else None
    wsu = _f32(ws_up) if hs else None
    wsd = _f32(ws_down) if hs else None
    idx = np.ascontiguousarray(topk_idx, np.int32)
    w = np.ascontiguousarray(topk_w, np.float64)
    if rows is None:
        n, rows_arr = T, None
    else:
        rows_arr = np.ascontiguousarray(rows, np.int64)
        n = rows_arr.size
    out = np.empty((n, d), np.float64)
    y = np.empty((n * k, d), np.float64) if want_y else None
    kp = _keep(keep, T, k)
    _load().oracle_forward_rows(n, _p(rows_arr), d, E, k, h, hs, _p(x), _p(wg), _p(wu), _p(wd),
                                _p(wsg), _p(wsu), _p(wsd), _p(idx), _p(w), _p(kp), _p(out), _p(y),
                                nthreads)
    return (out, y) if want_y else out


def backward(x, w_router, w_gate, w_up, w_down, grad_out, topk_idx, topk_w, ws_gate=None,
             ws_up=None, ws_down=None, nthreads: int = 0, keep=None) -> Dict[str, np.ndarray]:
    """Gradients of sum(out * grad_out) (float64), selection (and, with
    ``keep``, the capacity drops) held fixed."""
    x = _f32(x)
    T, d = x.shape
    E, _, h = w_gate.shape
    k = topk_idx.shape[1]
    hs = 0 if ws_gate is None else ws_gate.shape[1]
    wr, wg, wu, wd = _f32(w_router), _f32(w_gate), _f32(w_up), _f32(w_down)
    wsg = _f32(ws_gate) if hs else None
    wsu = _f32(ws_up) if hs else None
    wsd = _f32(ws_down) if hs else None
    G = _f32(grad_out)
    idx = np.ascontiguousarray(topk_idx, np.int32)
    w = np.ascontiguousarray(topk_w, np.float64)
    g = dict(
        x=np.empty((T, d)), w_router=np.empty((d, E)), w_gate=np.empty((E, d, h)),
        w_up=np.empty((E, d, h)), w_down=np.empty((E, h, d)))
    if hs:
        g.update(ws_gate=np.empty((d, hs)), ws_up=np.empty((d, hs)), ws_down=np.empty((hs, d)))
    _load().oracle_backward(
        T, d, E, k, h, hs, _p(x), _p(wr), _p(wg), _p(wu), _p(wd), _p(wsg), _p(wsu), _p(wsd), _p(G),
        _p(idx), _p(w), _p(_keep(keep, T, k)), _p(g["x"]), _p(g["w_router"]), _p(g["w_gate"]),
        _p(g["w_up"]),
        _p(g["w_down"]), _p(g.get("ws_gate")), _p(g.get("ws_up")), _p(g.get("ws_down")), nthreads)
    return g


def rel_err(a: np.ndarray, ref: np.ndarray) -> float:
    """Normwise relative difference max|a - ref| / max|ref| (0 when both are 0)."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(a - ref))) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def layer_forward(inputs: Dict, k: int, rows=None, nthreads: int = 0):
    """Route all tokens, then compute the requested output rows. ``inputs``
    maps tensor names to ``Tensor`` objects from the input generator."""
    v = {n: t.value for n, t in inputs.items()}
    logits, idx, w = route(v["x"], v["w_router"], k, nthreads)
    out = forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w, v.get("ws_gate"),
                       v.get("ws_up"), v.get("ws_down"), rows=rows, nthreads=nthreads)
    return dict(logits=logits, topk_idx=idx, topk_w=w, out=out)
