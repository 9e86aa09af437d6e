"""fp64 CPU oracle of the multi-LoRA batched adapter path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library: the
arithmetic lives in ``lora_oracle.c`` (plain fp64 loops, built with gcc), and
this module only converts inputs to float64 and marshals pointers.

Inputs arrive either as float32 arrays or as uint16 bf16 bit patterns; both
convert to float64 exactly.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, dense-matrix agreement, numpy library routines, finite
differences, adjoint identities, brute-force grouping) and by the hand-worked
fixtures in ``tests/golden/``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liblora_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, IEEE fp64 (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-std=c99", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # LORA_ORACLE_LIB: another build of lora_oracle.c (the sanitizer test builds one
    # with AddressSanitizer and UndefinedBehaviorSanitizer and runs the pins on it)
    path = os.environ.get("LORA_ORACLE_LIB") or _LIB
    if path == _LIB and not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(path)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    f64pp = ctypes.POINTER(f64p)
    lib.oracle_segments.argtypes = [i32p, ctypes.c_int64, ctypes.c_int32, i32p, i32p, i32p, i32p]
    lib.oracle_segments.restype = None
    lib.oracle_forward.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, f64p, i32p,
                                   ctypes.c_int32, i32p, f64p, f64pp, f64pp, f64p, f64p,
                                   ctypes.c_int32]
    lib.oracle_forward.restype = None
    lib.oracle_backward.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, f64p, f64p,
                                    i32p, ctypes.c_int32, i32p, f64p, f64pp, f64pp, f64p, f64pp,
                                    f64pp, f64p, f64p, ctypes.c_int32]
    lib.oracle_backward.restype = None
    lib.oracle_adamw.argtypes = [ctypes.c_int64, f64p, f64p, f64p, f64p] + [ctypes.c_double] * 6 + [ctypes.c_int32]
    lib.oracle_adamw.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def threads() -> int:
    return int(_load().oracle_threads())


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored elements to float64 ('bf16' bit patterns or 'f32')."""
    if dtype == "bf16":
        u = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _p64(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr_table(mats: Sequence[Optional[np.ndarray]]):
    f64p = ctypes.POINTER(ctypes.c_double)
    arr = (f64p * max(1, len(mats)))()
    for i, m in enumerate(mats):
        arr[i] = _p64(m) if m is not None else f64p()
    return arr


def segments(ids: np.ndarray, num_adapters: int):
    """(counts [A], offsets [A+1], perm [n_valid], err) of the row grouping."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T = ids.shape[0]
    counts = np.zeros(num_adapters, dtype=np.int32)
    offsets = np.zeros(num_adapters + 1, dtype=np.int32)
    perm = np.full(max(T, 1), -1, dtype=np.int32)
    err = np.zeros(1, dtype=np.int32)
    lib.oracle_segments(_p32(ids), T, num_adapters, _p32(counts), _p32(offsets), _p32(perm), _p32(err))
    return counts, offsets, perm[: int(offsets[-1])].copy(), int(err[0])


def forward(x: np.ndarray, ids: np.ndarray, ranks: np.ndarray, scales: np.ndarray,
            A: List[np.ndarray], B: List[np.ndarray], y0: np.ndarray):
    """y = y0 + per-row low-rank delta; returns (y [T, d_out], v [T, r_max]) in float64."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.array(y0, dtype=np.float64, order="C", copy=True)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    scales = np.ascontiguousarray(scales, dtype=np.float64)
    A = [np.ascontiguousarray(m, dtype=np.float64) for m in A]
    B = [np.ascontiguousarray(m, dtype=np.float64) for m in B]
    T, d_in = x.shape
    d_out = y.shape[1]
    r_max = max(1, int(ranks.max()) if ranks.size else 1)
    v = np.zeros((T, r_max), dtype=np.float64)
    lib.oracle_forward(T, d_in, d_out, _p64(x), _p32(ids), len(A), _p32(ranks), _p64(scales),
                       _ptr_table(A), _ptr_table(B), _p64(y), _p64(v), r_max)
    return y, v


def backward(x: np.ndarray, dy: np.ndarray, ids: np.ndarray, ranks: np.ndarray,
             scales: np.ndarray, A: List[np.ndarray], B: List[np.ndarray],
             dx0: Optional[np.ndarray] = None, dA0=None, dB0=None):
    """Gradients over the given fine-tuning rows.

    Returns (dx [T, d_in], dA list, dB list, g [T, r_max], v [T, r_max]) in float64;
    dx, dA, dB start from dx0 / dA0 / dB0 (zeros when None) and accumulate.
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    scales = np.ascontiguousarray(scales, dtype=np.float64)
    A = [np.ascontiguousarray(m, dtype=np.float64) for m in A]
    B = [np.ascontiguousarray(m, dtype=np.float64) for m in B]
    T, d_in = x.shape
    d_out = dy.shape[1]
    nA = len(A)
    dx = np.zeros((T, d_in)) if dx0 is None else np.array(dx0, dtype=np.float64, order="C", copy=True)
    dA = [np.zeros_like(m) if dA0 is None else np.array(dA0[i], dtype=np.float64, order="C", copy=True)
          for i, m in enumerate(A)]
    dB = [np.zeros_like(m) if dB0 is None else np.array(dB0[i], dtype=np.float64, order="C", copy=True)
          for i, m in enumerate(B)]
    r_max = max(1, int(ranks.max()) if ranks.size else 1)
    g = np.zeros((T, r_max))
    v = np.zeros((T, r_max))
    lib.oracle_backward(T, d_in, d_out, _p64(x), _p64(dy), _p32(ids), nA, _p32(ranks), _p64(scales),
                        _ptr_table(A), _ptr_table(B), _p64(dx), _ptr_table(dA), _ptr_table(dB),
                        _p64(g), _p64(v), r_max)
    return dx, dA, dB, g, v


def adamw(w: np.ndarray, grad: np.ndarray, m: np.ndarray, v: np.ndarray, *, lr: float, beta1: float,
          beta2: float, eps: float, weight_decay: float, step: int, grad_scale: float = 1.0):
    """One AdamW step; returns new (w, m, v) float64 arrays of w's shape (inputs untouched)."""
    lib = _load()
    w = np.array(w, dtype=np.float64, order="C", copy=True)
    m = np.array(m, dtype=np.float64, order="C", copy=True)
    v = np.array(v, dtype=np.float64, order="C", copy=True)
    g = np.ascontiguousarray(grad, dtype=np.float64)
    if not (w.shape == m.shape == v.shape == g.shape):
        raise ValueError("w, grad, m, v must have one shape")
    lib.oracle_adamw(w.size, _p64(w), _p64(g), _p64(m), _p64(v), lr, beta1, beta2, eps, weight_decay,
                     grad_scale, int(step))
    return w, m, v


def from_workload(wl) -> dict:
    """Decode a workload's stored elements to float64 (duck-typed; no import of the generator)."""
    dt = wl.dtype
    out = {
        "x": to_f64(wl.x, dt),
        "y0": to_f64(wl.y0, dt),
        "A": [to_f64(m, dt) for m in wl.A],
        "B": [to_f64(m, dt) for m in wl.B],
        "ids": np.asarray(wl.ids, dtype=np.int32),
        "ranks": np.asarray(wl.ranks, dtype=np.int32),
        "scales": np.asarray(wl.scales, dtype=np.float64),
    }
    if getattr(wl, "dy", None) is not None:
        out["dy"] = to_f64(wl.dy, dt)
    return out
