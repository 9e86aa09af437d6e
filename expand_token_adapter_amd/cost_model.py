"""Cost model of this library's own calls, fitted to measurements.

A co-serving scheduler prices a batch before dispatching it.  DeltaServe's
latency model (section 3.3, Equation I) is linear in the batch composition,
with a term gamma * T_ft for the fine-tuning tokens and a fixed per-step
overhead c, its coefficients seeded by offline profiling; the adapter-caching
page models the adapters' overhead as linear in the number of adapters and
fits its constants to profiled data by non-linear least squares.  This module
does the same for the LoRA delta itself: for each entry point,

    t = c + k_t * T + k_row * T (d_in + d_out) + k_w * sum_{a in U} r_a (d_in + d_out)
          + k_r * sum_t r_{a(t)} + k_a * |U| + k_tile * sum_{a in U} ceil(n_a / 16)
          + k_g * sum_t ceil(r_{a(t)} / 16) (d_in + d_out)

(U = adapters with at least one row, n_a = rows of adapter a; T = rows, the
segment build's work; T (d_in + d_out) = row elements read and written;
sum_U r_a (d_in + d_out) = weight elements read; sum_t r = the rank-wide
intermediate per row; |U| = per-adapter work starts; sum_U ceil(n_a / 16) =
16-row tiles, each a chain of dependent loads in the kernels that walk
them; sum_t ceil(r / 16) (d_in + d_out) = row elements once per 16-rank group,
as the backward's token contraction reads them), with non-negative coefficients fitted by bounded least squares on
relative residuals, so that a 10 us and a 1 ms call weigh alike.

Each entry point has one model per kernel route the library takes: the
backward's streaming route is ``backward_stream``; the split forward on
decode batches (at most 32 rows per adapter: the 16-row-tile shrink and
expand) is ``forward_decode``; ``forward_fused`` is
``lora_forward`` without v, whose one-launch kernels are the 16-row-tile
decode kernel (``forward_fused_decode``: bf16 decode batches with r_max <=
16) or the 64-row-tile kernel (``forward_fused``); with v, ``lora_forward``
runs the split kernels on decode batches and at r_max <= 16, priced as the
split forward of the same batch (``route``).

``features`` and ``fit`` / ``predict`` run on the host; ``calibrate`` times the
library's calls on synthetic batches on the GPU (random ids, ranks and
weights; no dataset).  ``python -m expand_token_adapter_amd.cost_model``
calibrates, fits and prints the coefficients and the fit's relative errors.
"""
from __future__ import annotations

import argparse
import json
from typing import Dict, Iterable, List, Sequence, Tuple

import numpy as np

FEATURES = ("const", "rows", "row_elems", "weight_elems", "rank_rows", "adapters", "tiles16", "group_elems")
OPS = ("segments", "forward", "forward_fused", "backward")

# The terms each model entry is fitted with (the others stay zero): the
# segment build handles rows and adapters only; the forwards read rows and
# weights; the two-pass backward also re-reads rows per 16-rank group.
_OP_FEATURES = {
    "segments": ("const", "rows", "adapters", "tiles16"),
    "forward": ("const", "row_elems", "weight_elems", "rank_rows", "adapters", "tiles16"),
    "forward_decode": ("const", "row_elems", "weight_elems", "rank_rows", "adapters", "tiles16"),
    "forward_fused": ("const", "row_elems", "weight_elems", "rank_rows", "adapters", "tiles16"),
    "forward_fused_decode": ("const", "row_elems", "weight_elems", "tiles16"),
    "backward": ("const", "row_elems", "weight_elems", "rank_rows", "adapters", "tiles16", "group_elems"),
    "backward_stream": ("const", "row_elems", "weight_elems", "rank_rows", "adapters", "tiles16"),
}


DECODE_ROWS_PER_ADAPTER = 32  # the library's decode-batch bound: T <= 32 x (adapters in the table)


def route(op: str, ranks: Sequence[int], d_in: int, d_out: int, r_max: int = 0, T: int = -1,
          with_v: bool = False) -> str:
    """The model entry of a bf16 call, as the library routes it.  r_max
    defaults to max(ranks); T is the call's row count (-1: not a decode batch).
    - backward: 'backward_stream' (one pass over dY) when r_max <= 16 and
      d_out >= 2 d_in, else 'backward';
    - forward (lora_shrink + lora_expand_add): 'forward_decode' on decode
      batches (T <= 32 x len(ranks): the 16-row-tile kernels), else 'forward';
    - forward_fused (lora_forward): 'forward_fused_decode' on decode batches
      with r_max <= 16; else, with v given, the split kernels on decode
      batches or at r_max <= 16 (priced as the split forward); else
      'forward_fused' (the 64-row-tile kernel);
    - the others: one model each."""
    r = r_max or (max(ranks) if len(ranks) else 0)
    decode = 0 <= T <= DECODE_ROWS_PER_ADAPTER * len(ranks)
    if op == "backward":
        if r <= 16 and d_out >= 2 * d_in:
            return "backward_stream"
    if op == "forward_fused":
        if decode and r <= 16:
            return "forward_fused_decode"
        if with_v and (decode or r <= 16):
            op = "forward"
    if op == "forward" and decode:
        return "forward_decode"
    return op


def features(ids: Sequence[int], ranks: Sequence[int], d_in: int, d_out: int) -> np.ndarray:
    """The model's features of one call over rows with adapter ids `ids` (-1: no adapter)."""
    ids = np.asarray(ids, dtype=np.int64)
    ranks = np.asarray(ranks, dtype=np.int64)
    valid = ids[(ids >= 0) & (ids < len(ranks))]
    used, counts = np.unique(valid, return_counts=True)
    T = ids.size
    return np.array([1.0,
                     float(T),
                     float(T) * (d_in + d_out),
                     float(ranks[used].sum()) * (d_in + d_out),
                     float(ranks[valid].sum()),
                     float(used.size),
                     float(((counts + 15) // 16).sum()),
                     float(((ranks[valid] + 15) // 16).sum()) * (d_in + d_out)])


def fit(X: np.ndarray, t: np.ndarray) -> np.ndarray:
    """Non-negative coefficients minimising sum ((X c - t) / t)^2 (bounded least squares)."""
    from scipy.optimize import least_squares

    X = np.asarray(X, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    if X.ndim != 2 or X.shape[0] != t.size or X.shape[0] < X.shape[1]:
        raise ValueError("need at least as many samples as features")
    scale = np.maximum(np.abs(X).max(axis=0), 1e-30)  # columns brought to O(1)
    A = X / scale / t[:, None]
    x0 = np.full(X.shape[1], 1.0 / X.shape[1])
    res = least_squares(lambda c: A @ c - 1.0, x0, bounds=(0.0, np.inf), method="trf", x_scale="jac")
    return res.x / scale


class CostModel:
    """Fitted coefficients per entry point; predict(op, ...) returns seconds."""

    def __init__(self, coef: Dict[str, Sequence[float]]):
        self.coef = {op: np.asarray(c, dtype=np.float64) for op, c in coef.items()}

    def predict(self, op: str, ids, ranks, d_in: int, d_out: int, r_max: int = 0, with_v: bool = False) -> float:
        key = route(op, ranks, d_in, d_out, r_max, T=len(ids), with_v=with_v)
        return float(features(ids, ranks, d_in, d_out) @ self.coef[key if key in self.coef else op])

    def to_json(self) -> str:
        return json.dumps({op: {f: float(v) for f, v in zip(FEATURES, c)} for op, c in self.coef.items()})

    @classmethod
    def from_json(cls, text: str) -> "CostModel":
        d = json.loads(text)
        return cls({op: [d[op][f] for f in FEATURES] for op in d})


def relative_errors(model: CostModel, samples: List[dict]) -> Dict[str, np.ndarray]:
    out: Dict[str, List[float]] = {}
    for s in samples:
        p = float(np.asarray(s["features"]) @ model.coef[s["op"]])
        out.setdefault(s["op"], []).append(p / s["seconds"] - 1.0)
    return {op: np.asarray(v) for op, v in out.items()}


def fit_samples(samples: List[dict]) -> CostModel:
    coef = {}
    for op in sorted({s["op"] for s in samples}):
        rows = [s for s in samples if s["op"] == op]
        cols = [FEATURES.index(f) for f in _OP_FEATURES.get(op, FEATURES)]
        X = np.array([s["features"] for s in rows])
        c = np.zeros(len(FEATURES))
        c[cols] = fit(X[:, cols], np.array([s["seconds"] for s in rows]))
        coef[op] = c
    return CostModel(coef)


# ------------------------------------------------------------------ calibration (GPU)

def default_shapes() -> List[Tuple[int, int, int, Tuple[int, ...], str]]:
    """(T, d_in, d_out, ranks of the adapters, id distribution) of the calibration batches."""
    shapes = []
    for d_in, d_out in ((4096, 4096), (4096, 14336), (8192, 8192)):
        for T in (64, 512, 2048, 8192):
            for ranks, dist in (((16,) * 64, "uniform"), ((8, 16, 32, 64) * 8, "uniform"), ((16,), "one"),
                                ((8, 16, 32, 64, 128) * 32, "zipf")):
                shapes.append((T, d_in, d_out, ranks, dist))
    return shapes


def _ids(rng, T: int, n_adapters: int, dist: str) -> np.ndarray:
    if dist == "one":
        return np.zeros(T, dtype=np.int32)
    if dist == "zipf":
        p = np.arange(1, n_adapters + 1, dtype=np.float64) ** -1.1
        return rng.choice(n_adapters, size=T, p=p / p.sum()).astype(np.int32)
    return rng.integers(0, n_adapters, size=T).astype(np.int32)


def calibrate(shapes=None, reps: int = 10, ops: Iterable[str] = OPS, seed: int = 0, progress=None) -> List[dict]:
    """Time the library's calls on synthetic bf16 batches; returns samples {op, features, seconds, shape}."""
    import torch
    import expand_token_adapter_amd as lb

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(seed)
    ops = tuple(ops)
    samples: List[dict] = []
    for k, (T, d_in, d_out, ranks, dist) in enumerate(shapes or default_shapes()):
        ranks = list(ranks)
        ids_np = _ids(rng, T, len(ranks), dist)
        A = [torch.randn((r, d_in), device=dev, dtype=torch.bfloat16) * 0.02 for r in ranks]
        B = [torch.randn((d_out, r), device=dev, dtype=torch.bfloat16) * 0.02 for r in ranks]
        table = lb.AdapterTable(A, B, [2.0] * len(ranks))
        ids = torch.from_numpy(ids_np).to(dev)
        x = torch.randn((T, d_in), device=dev, dtype=torch.bfloat16)
        y = torch.randn((T, d_out), device=dev, dtype=torch.bfloat16)
        dy = torch.randn((T, d_out), device=dev, dtype=torch.bfloat16)
        dx = torch.zeros((T, d_in), device=dev, dtype=torch.bfloat16)
        v = torch.zeros((T, (table.r_max + 7) // 8 * 8), device=dev, dtype=torch.float32)
        seg = lb.Segments(T, len(ranks), dev)
        lb.lora_segments_build(ids, len(ranks), out=seg)
        ws = torch.empty(lb.lora_shrink_workspace_bytes(torch.bfloat16, T, d_in, table.r_max), dtype=torch.uint8,
                         device=dev)
        bws = torch.empty(lb.lora_backward_workspace_bytes(torch.bfloat16, T, d_in, d_out, table.r_max),
                          dtype=torch.uint8, device=dev)
        dA = [torch.zeros(a.shape, device=dev, dtype=torch.float32) for a in A]
        dB = [torch.zeros(b.shape, device=dev, dtype=torch.float32) for b in B]
        grads = lb.GradTable(dA, dB)
        calls = {
            "segments": lambda: lb.lora_segments_build(ids, len(ranks), out=seg),
            "forward": lambda: (lb.lora_shrink(x, table, seg, v=v, ws=ws), lb.lora_expand_add(v, table, seg, y)),
            "forward_fused": lambda: lb.lora_forward(x, table, seg, y),  # without v: one launch
            "backward": lambda: lb.lora_backward(x, dy, table, grads, seg, dx=dx, v_saved=v, ws=bws),
        }
        feats = features(ids_np, ranks, d_in, d_out)
        for op in ops:
            f = calls[op]
            f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) * 1e-3 / reps
            samples.append({"op": route(op, ranks, d_in, d_out, T=T), "features": feats.tolist(), "seconds": sec,
                            "shape": {"T": T, "d_in": d_in, "d_out": d_out, "adapters": len(ranks), "dist": dist}})
        if progress:
            progress(k, T, d_in, d_out, len(ranks), dist)
        del A, B, table, x, y, dy, dx, v, ws, bws, dA, dB, grads
    return samples


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--samples-out", help="write the measured samples (JSON)")
    ap.add_argument("--model-out", help="write the fitted coefficients (JSON)")
    args = ap.parse_args(argv)
    samples = calibrate(reps=args.reps, progress=lambda k, *s: print(f"shape {k}: {s}", flush=True))
    model = fit_samples(samples)
    if args.samples_out:
        with open(args.samples_out, "w") as f:
            json.dump(samples, f)
    if args.model_out:
        with open(args.model_out, "w") as f:
            f.write(model.to_json())
    errs = relative_errors(model, samples)
    for op in model.coef:
        e = np.abs(errs[op])
        print(json.dumps({"op": op, "coef": dict(zip(FEATURES, model.coef[op].tolist())),
                          "median_abs_rel_err": float(np.median(e)), "max_abs_rel_err": float(e.max()),
                          "samples": int(e.size)}), flush=True)


if __name__ == "__main__":
    main()
