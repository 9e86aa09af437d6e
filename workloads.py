"""Seeded synthetic inputs for the multi-LoRA batched adapter path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP library
(``expand_token_adapter_amd``) are fed from it, and it imports neither.

Shapes follow the workloads the pages describe:
  * LoRA factors A in R^{r x k} and B in R^{d x r} (DeltaServe, section 2.2;
    MOLT, section 2.1), stored row-major: A_a is [r_a, d_in], B_a is [d_out, r_a].
  * rank 16 with alpha 32 for the tuned adapter (DeltaServe, section 4.1), so the
    per-adapter scale is 32/16 = 2.0 throughout;
  * heterogeneous adapter ranks and up to A_max = 320 resident adapters
    (Data-Driven Optimization of GPU efficiency for Distributed LLM-Adapter
    Serving, adapter caching discussion);
  * a mixed batch of decode rows, prefill segments and fine-tuning rows routed
    to a reserved adapter (DeltaServe, section 3.2, "Mixed forward batch").

Draw order (fixed, so a seed pins every array): adapter ids / segment shapes,
then ranks, then every A_a, then every B_a, then x, then y0, then dY.
Values are drawn in fp32 (``standard_normal(dtype=float32)`` times the stated
standard deviation).  bf16 workloads round each fp32 draw once,
round-to-nearest-even, and store the 16-bit patterns as ``uint16``.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional

import numpy as np

__all__ = ["Workload", "config", "custom", "fp32_to_bf16_bits", "CONFIG_NAMES"]

CONFIG_NAMES = {
    1: "tiny-fp32-fwd-bwd",
    2: "decode-64x-r16-4096",
    3: "mixed-coserve-32x-4096to14336",
    4: "ft-step-r16-5120",
    5: "decode-zipf-320x-8192",
}


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


@dataclasses.dataclass
class Workload:
    """One synthetic batch.

    Element arrays (A, B, x, y0, dy) hold ``uint16`` bf16 bit patterns when
    ``dtype == "bf16"`` and ``float32`` values when ``dtype == "f32"``.
    ``ft_rows`` are the batch rows that also run the backward; they form one
    contiguous range ``[ft_start, ft_start + len(ft_rows))`` and ``dy`` has one
    row per fine-tuning row, in that order.
    """

    name: str
    dtype: str
    d_in: int
    d_out: int
    ids: np.ndarray  # int32 [T]; -1 = row without an adapter
    ranks: np.ndarray  # int32 [A]
    scales: np.ndarray  # float32 [A]
    A: List[np.ndarray]  # [r_a, d_in]
    B: List[np.ndarray]  # [d_out, r_a]
    x: np.ndarray  # [T, d_in]
    y0: np.ndarray  # [T, d_out]
    ft_start: int = 0
    ft_count: int = 0
    dy: Optional[np.ndarray] = None  # [ft_count, d_out]

    @property
    def T(self) -> int:
        return int(self.ids.shape[0])

    @property
    def num_adapters(self) -> int:
        return int(self.ranks.shape[0])

    @property
    def r_max(self) -> int:
        return int(self.ranks.max())

    @property
    def ft_ids(self) -> np.ndarray:
        return self.ids[self.ft_start:self.ft_start + self.ft_count]

    def manifest(self) -> dict:
        """SHA-256 of every array, for result files."""
        h = {}
        for key in ("ids", "ranks", "scales", "x", "y0"):
            h[key] = hashlib.sha256(np.ascontiguousarray(getattr(self, key)).tobytes()).hexdigest()
        ha = hashlib.sha256()
        for m in self.A:
            ha.update(np.ascontiguousarray(m).tobytes())
        h["A"] = ha.hexdigest()
        hb = hashlib.sha256()
        for m in self.B:
            hb.update(np.ascontiguousarray(m).tobytes())
        h["B"] = hb.hexdigest()
        if self.dy is not None:
            h["dy"] = hashlib.sha256(np.ascontiguousarray(self.dy).tobytes()).hexdigest()
        return h


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if dtype == "bf16":
        return fp32_to_bf16_bits(v)
    return v


def custom(
    ids,
    ranks,
    d_in: int,
    d_out: int,
    dtype: str = "bf16",
    seed: int = 0,
    scales=None,
    ft_start: int = 0,
    ft_count: int = 0,
    w_std: float = 0.02,
    name: str = "custom",
    rng: Optional[np.random.Generator] = None,
) -> Workload:
    """Draw A, B, x, y0 (and dY for ``ft_count`` rows) for given ids and ranks."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    if scales is None:
        scales = np.full(ranks.shape[0], 2.0, dtype=np.float32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    if rng is None:
        rng = np.random.default_rng(seed)
    T = int(ids.shape[0])
    A = [_draw(rng, (int(r), d_in), w_std, dtype) for r in ranks]
    B = [_draw(rng, (d_out, int(r)), w_std, dtype) for r in ranks]
    x = _draw(rng, (T, d_in), 1.0, dtype)
    y0 = _draw(rng, (T, d_out), 1.0, dtype)
    dy = _draw(rng, (ft_count, d_out), 1.0, dtype) if ft_count > 0 else None
    return Workload(name, dtype, d_in, d_out, ids, ranks, scales, A, B, x, y0,
                    ft_start, ft_count, dy)


def config(index: int, seed: int = 0) -> Workload:
    """The five synthetic workloads, by number (1..5)."""
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[index]
    if index == 1:
        # 64 rows in 4 contiguous segments of 16; backward on segment 0.
        ids = np.repeat(np.arange(4, dtype=np.int32), 16)
        ranks = np.full(4, 8, dtype=np.int32)
        return custom(ids, ranks, 256, 256, "f32", rng=rng, ft_start=0, ft_count=16, name=name)
    if index == 2:
        # 256 decode rows, adapter id uniform over 64 adapters of rank 16.
        ids = rng.integers(0, 64, size=256).astype(np.int32)
        ranks = np.full(64, 16, dtype=np.int32)
        return custom(ids, ranks, 4096, 4096, "bf16", rng=rng, name=name)
    if index == 3:
        # [128 decode rows, id ~ U{1..31}] [8 prefill segments, length ~ U{128..1024},
        # one id ~ U{1..31} each] [2 fine-tuning segments x 1024 rows on reserved id 0].
        dec_ids = rng.integers(1, 32, size=128)
        lens = rng.integers(128, 1025, size=8)
        seg_ids = rng.integers(1, 32, size=8)
        parts = [dec_ids]
        for length, sid in zip(lens, seg_ids):
            parts.append(np.full(int(length), sid))
        parts.append(np.zeros(2 * 1024, dtype=np.int64))
        ids = np.concatenate(parts).astype(np.int32)
        ranks = rng.choice(np.array([8, 16, 32, 64]), size=32).astype(np.int32)
        T = ids.shape[0]
        return custom(ids, ranks, 4096, 14336, "bf16", rng=rng,
                      ft_start=T - 2048, ft_count=2048, name=name)
    if index == 4:
        # 4 sequences x 1024 rows, one adapter of rank 16; backward on every row.
        ids = np.zeros(4096, dtype=np.int32)
        ranks = np.array([16], dtype=np.int32)
        return custom(ids, ranks, 5120, 5120, "bf16", rng=rng, ft_start=0, ft_count=4096, name=name)
    if index == 5:
        # 2048 decode rows; P(id = k-1) proportional to k^-1.1 for k = 1..320.
        k = np.arange(1, 321, dtype=np.float64)
        p = k ** -1.1
        p /= p.sum()
        ids = rng.choice(320, size=2048, p=p).astype(np.int32)
        ranks = rng.choice(np.array([8, 16, 32, 64, 128]), size=320).astype(np.int32)
        return custom(ids, ranks, 8192, 8192, "bf16", rng=rng, name=name)
    raise ValueError(f"no config {index}")
