"""Multi-LoRA batched adapter kernels for AMD MI355X (gfx950).

Python binding of the C ABI (include/lora_batch.h).  Each function has the
name of the C entry point it calls, takes torch tensors that live on the GPU,
and only marshals pointers, sizes and the current HIP stream: every step of
the computation runs in the HIP kernels of liblora_batch.so.  PyTorch supplies
device memory and streams.

    seg = lora_segments_build(ids, num_adapters)         # group rows by adapter
    v = lora_shrink(x, table, seg)                       # v = A_a x    (fp32)
    lora_expand_add(v, table, seg, y)                    # y += s_a B_a v
    lora_backward(x_ft, dy, table, grads, seg_ft, dx)    # dX, dA, dB  (+=)
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _abi
from ._abi import LORA_BF16, LORA_F32, LORA_MAX_RANK, LoraError

__all__ = [
    "AdapterTable", "GradTable", "Segments", "LoraError",
    "lora_segments_build", "lora_segments_build_batch", "lora_shrink", "lora_shrink_noalloc", "lora_expand_add",
    "lora_forward",
    "lora_forward_multi", "lora_backward", "lora_backward_preemptible", "lora_adamw_step",
    "lora_abi_version", "lora_status_string",
    "lora_segments_workspace_bytes", "lora_shrink_workspace_bytes", "lora_backward_workspace_bytes",
    "lora_segments_sched_elems",
]

_DTYPES = {torch.bfloat16: LORA_BF16, torch.float32: LORA_F32}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"element type must be bfloat16 or float32, got {t.dtype}")
    return _DTYPES[t.dtype]


# The current stream's raw handle, without building a torch Stream object per
# call (that costs about as much as the rest of a call's marshalling); the
# public query where this PyTorch build lacks the raw one.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev: torch.device) -> int:
    if _raw_stream is not None:
        return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


def _on_gpu(*ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _rows(t: torch.Tensor, name: str):
    """(pointer, rows, cols, pitch) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return t.data_ptr(), t.shape[0], t.shape[1], t.stride(0)


def _check_batch(name: str, adapters: "AdapterTable", seg: "Segments", T: int, *, x=None, y=None,
                 v=None, r_max: int = 0) -> None:
    """Raise ValueError unless the arguments of one compute call describe one batch.

    The C side sizes its offsets and strides from T, the adapter count, the
    dtype and r_max; arguments from different batches would make the kernels
    index outside the buffers, so they are rejected here, before any enqueue."""
    if seg.T != T:
        raise ValueError(f"{name}: the segments were built for {seg.T} rows, the call has {T}")
    if seg.num_adapters != len(adapters):
        raise ValueError(f"{name}: the segments were built for {seg.num_adapters} adapters, "
                         f"the table has {len(adapters)}")
    if x is not None:
        if x.dtype != adapters.dtype:
            raise ValueError(f"{name}: x is {x.dtype}, the adapters are {adapters.dtype}")
        if x.shape[1] != adapters.d_in:
            raise ValueError(f"{name}: x has {x.shape[1]} columns, the adapters' d_in is {adapters.d_in}")
        if x.device != adapters.device:
            raise ValueError(f"{name}: x and the adapters are on different devices")
    if y is not None:
        if y.dtype != adapters.dtype:
            raise ValueError(f"{name}: y is {y.dtype}, the adapters are {adapters.dtype}")
        if y.shape[1] != adapters.d_out:
            raise ValueError(f"{name}: y has {y.shape[1]} columns, the adapters' d_out is {adapters.d_out}")
        if y.shape[0] != T:
            raise ValueError(f"{name}: y has {y.shape[0]} rows, the call has {T}")
        if y.device != adapters.device:
            raise ValueError(f"{name}: y and the adapters are on different devices")
    if v is not None:
        if v.dtype != torch.float32:
            raise ValueError(f"{name}: v must be float32")
        if v.dim() != 2 or v.shape[0] != T:
            raise ValueError(f"{name}: v must have one row per row of the call ({T})")
        if v.shape[1] < (r_max + 7) // 8 * 8:
            raise ValueError(f"{name}: v needs at least round_up(r_max, 8) = {(r_max + 7) // 8 * 8} columns")
        if v.device != adapters.device:
            raise ValueError(f"{name}: v and the adapters are on different devices")


def lora_abi_version() -> int:
    return _abi.load().lora_abi_version()


def lora_status_string(status: int) -> str:
    return _abi.status_string(status)


def lora_segments_workspace_bytes(T: int, num_adapters: int) -> int:
    return _abi.load().lora_segments_workspace_bytes(T, num_adapters)


def lora_shrink_workspace_bytes(dtype: torch.dtype, T: int, d_in: int, r_max: int) -> int:
    return _abi.load().lora_shrink_workspace_bytes(_DTYPES[dtype], T, d_in, r_max)


def lora_backward_workspace_bytes(dtype: torch.dtype, T_ft: int, d_in: int, d_out: int, r_max: int) -> int:
    return _abi.load().lora_backward_workspace_bytes(_DTYPES[dtype], T_ft, d_in, d_out, r_max)


def lora_segments_sched_elems(T: int, num_adapters: int) -> int:
    return _abi.load().lora_segments_sched_elems(T, num_adapters)


class AdapterTable:
    """Device-resident table of adapters (lora_adapter structs).

    A[a]: [r_a, d_in] and B[a]: [d_out, r_a] tensors on the GPU (kept alive
    by this object); scales[a] multiplies adapter a's delta.
    """

    def __init__(self, A: Sequence[torch.Tensor], B: Sequence[torch.Tensor], scales: Sequence[float]):
        if not (len(A) == len(B) == len(scales)) or len(A) == 0:
            raise ValueError("A, B and scales must have the same nonzero length")
        self.A = list(A)
        self.B = list(B)
        self.scales = [float(s) for s in scales]
        self.dtype = self.A[0].dtype
        self.device = self.A[0].device
        _on_gpu(*self.A, *self.B)
        ranks = []
        host = (_abi.LoraAdapter * len(A))()
        for i, (a, b, s) in enumerate(zip(self.A, self.B, self.scales)):
            if a.dtype != self.dtype or b.dtype != self.dtype or not a.is_contiguous() or not b.is_contiguous():
                raise ValueError("adapter weights must share one dtype and be contiguous")
            if a.dim() != 2 or b.dim() != 2 or b.shape[1] != a.shape[0]:
                raise ValueError("A must be [r, d_in] and B [d_out, r]")
            if a.shape[1] != self.A[0].shape[1] or b.shape[0] != self.B[0].shape[0]:
                raise ValueError("every A must have the same d_in and every B the same d_out")
            if a.device != self.device or b.device != self.device:
                raise ValueError("adapter weights must live on one device")
            host[i] = _abi.LoraAdapter(a.data_ptr(), b.data_ptr(), a.shape[0], s)
            ranks.append(int(a.shape[0]))
        self.ranks = ranks
        self.r_max = max(ranks)
        self.d_in = int(self.A[0].shape[1])
        self.d_out = int(self.B[0].shape[0])
        raw = bytes(host)
        self.table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(self.device)

    def __len__(self) -> int:
        return len(self.A)

    @property
    def ptr(self) -> int:
        return self.table.data_ptr()


class GradTable:
    """Device-resident table of fp32 gradient targets (lora_adapter_grad structs).

    dA[a]: [r_a, d_in], dB[a]: [d_out, r_a] float32 GPU tensors, or None for
    adapters that are not trained.
    """

    def __init__(self, dA: Sequence[Optional[torch.Tensor]], dB: Sequence[Optional[torch.Tensor]]):
        if len(dA) != len(dB) or len(dA) == 0:
            raise ValueError("dA and dB must have the same nonzero length")
        self.dA = list(dA)
        self.dB = list(dB)
        host = (_abi.LoraAdapterGrad * len(dA))()
        device = None
        for i, (ga, gb) in enumerate(zip(self.dA, self.dB)):
            if (ga is None) != (gb is None):
                raise ValueError("dA and dB must both be given or both be None")
            if ga is None:
                continue
            _on_gpu(ga, gb)
            if ga.dtype != torch.float32 or gb.dtype != torch.float32:
                raise TypeError("gradients are float32")
            if not ga.is_contiguous() or not gb.is_contiguous():
                raise ValueError("gradients must be contiguous")
            device = ga.device
            host[i] = _abi.LoraAdapterGrad(ga.data_ptr(), gb.data_ptr())
        if device is None:
            raise ValueError("at least one adapter needs gradient buffers")
        self.table = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8).to(device)

    @property
    def ptr(self) -> int:
        return self.table.data_ptr()


class Segments:
    """Output of lora_segments_build: rows grouped by adapter (device tensors)."""

    def __init__(self, T: int, num_adapters: int, device: torch.device):
        lib = _abi.load()
        self.T = T
        self.num_adapters = num_adapters
        i32 = dict(dtype=torch.int32, device=device)
        self.counts = torch.zeros(num_adapters, **i32)
        self.offsets = torch.zeros(num_adapters + 1, **i32)
        self.perm = torch.zeros(max(T, 1), **i32)
        self.err = torch.zeros(1, **i32)
        self.sched = torch.zeros(max(1, lib.lora_segments_sched_elems(T, num_adapters)), **i32)
        self.ws = torch.empty(max(1, lib.lora_segments_workspace_bytes(T, num_adapters)), dtype=torch.uint8,
                              device=device)
        self._c = _abi.LoraSegments(self.counts.data_ptr(), self.offsets.data_ptr(), self.perm.data_ptr(),
                                    self.err.data_ptr(), self.sched.data_ptr())

    @property
    def c(self) -> _abi.LoraSegments:
        """The C struct of device pointers (the tensors are allocated once, so it is built once)."""
        return self._c


def lora_segments_build(adapter_ids: torch.Tensor, num_adapters: int, out: Optional[Segments] = None) -> Segments:
    """Group rows by adapter id (-1 = no adapter).  Returns (or refills) a Segments."""
    _on_gpu(adapter_ids)
    if adapter_ids.dtype != torch.int32 or adapter_ids.dim() != 1 or not adapter_ids.is_contiguous():
        raise ValueError("adapter_ids must be a contiguous 1-D int32 tensor")
    T = int(adapter_ids.shape[0])
    seg = out if out is not None else Segments(T, num_adapters, adapter_ids.device)
    if seg.T != T or seg.num_adapters != num_adapters:
        raise ValueError("Segments buffers were sized for another batch")
    st = _abi.load().lora_segments_build(adapter_ids.data_ptr(), T, num_adapters, seg.c, seg.ws.data_ptr(),
                                         seg.ws.numel(), _stream(adapter_ids.device))
    _abi.check("lora_segments_build", st)
    return seg


def lora_segments_build_batch(jobs, num_adapters: int) -> list:
    """Several lora_segments_build calls in one enqueue: jobs = [(adapter_ids, out Segments or None), ...]
    on one device; the one-workgroup builds share launches.  Returns the Segments, in order."""
    segs, raw = [], []
    for ids, out in jobs:
        _on_gpu(ids)
        if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
            raise ValueError("adapter_ids must be a contiguous 1-D int32 tensor")
        T = int(ids.shape[0])
        seg = out if out is not None else Segments(T, num_adapters, ids.device)
        if seg.T != T or seg.num_adapters != num_adapters:
            raise ValueError("Segments buffers were sized for another batch")
        segs.append(seg)
        raw.append(_abi.LoraSegmentsJob(ids.data_ptr(), T, seg.c, seg.ws.data_ptr(), seg.ws.numel()))
    if not segs:
        return segs
    arr = (_abi.LoraSegmentsJob * len(raw))(*raw)
    st = _abi.load().lora_segments_build_batch(ctypes.addressof(arr), len(raw), num_adapters,
                                               _stream(jobs[0][0].device))
    _abi.check("lora_segments_build_batch", st)
    return segs


def lora_shrink(x: torch.Tensor, adapters: AdapterTable, seg: Segments, v: Optional[torch.Tensor] = None,
                r_max: Optional[int] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """v[t, :r_a] = A_a x_t (fp32) for every row with an adapter; returns v [T, r_max]."""
    _on_gpu(x)
    px, T, d_in, ldx = _rows(x, "x")
    r_max = adapters.r_max if r_max is None else r_max
    if v is None:
        v = torch.zeros((T, (r_max + 7) // 8 * 8), dtype=torch.float32, device=x.device)
    pv, _, _, ldv = _rows(v, "v")
    _check_batch("lora_shrink", adapters, seg, T, x=x, v=v, r_max=r_max)
    lib = _abi.load()
    if ws is None:  # a caller's workspace is size-checked by the library (LORA_ERR_WORKSPACE)
        ws = torch.empty(max(lib.lora_shrink_workspace_bytes(_dtype_code(x), T, d_in, r_max), 1),
                         dtype=torch.uint8, device=x.device)
    st = lib.lora_shrink(_dtype_code(x), px, ldx, T, d_in, adapters.ptr, len(adapters), r_max, seg.c,
                         pv, ldv, ws.data_ptr(), ws.numel(), _stream(x.device))
    _abi.check("lora_shrink", st)
    return v


def lora_shrink_noalloc(x: torch.Tensor, adapters: AdapterTable, seg: Segments, v: torch.Tensor,
                        r_max: Optional[int] = None) -> torch.Tensor:
    """lora_shrink into the caller's v with the library's static device scratch as its
    workspace: neither the library nor this binding allocates anything.  Calls that
    overlap on one GPU share that scratch and must be ordered by the caller."""
    _on_gpu(x, v)
    px, T, d_in, ldx = _rows(x, "x")
    r_max = adapters.r_max if r_max is None else r_max
    pv, _, _, ldv = _rows(v, "v")
    _check_batch("lora_shrink_noalloc", adapters, seg, T, x=x, v=v, r_max=r_max)
    st = _abi.load().lora_shrink_noalloc(_dtype_code(x), px, ldx, T, d_in, adapters.ptr, len(adapters), r_max, seg.c,
                                         pv, ldv, _stream(x.device))
    _abi.check("lora_shrink_noalloc", st)
    return v


def lora_expand_add(v: torch.Tensor, adapters: AdapterTable, seg: Segments, y: torch.Tensor,
                    r_max: Optional[int] = None) -> torch.Tensor:
    """y[t] += s_a B_a v[t, :r_a] in place; returns y."""
    _on_gpu(v, y)
    pv, T, _, ldv = _rows(v, "v")
    py, Ty, d_out, ldy = _rows(y, "y")
    if Ty != T:
        raise ValueError("v and y must have the same number of rows")
    r_max = adapters.r_max if r_max is None else r_max
    _check_batch("lora_expand_add", adapters, seg, T, y=y, v=v, r_max=r_max)
    st = _abi.load().lora_expand_add(_dtype_code(y), pv, ldv, T, d_out, adapters.ptr, len(adapters), r_max,
                                     seg.c, py, ldy, _stream(y.device))
    _abi.check("lora_expand_add", st)
    return y


def lora_forward(x: torch.Tensor, adapters: AdapterTable, seg: Segments, y: torch.Tensor,
                 v: Optional[torch.Tensor] = None, r_max: Optional[int] = None) -> torch.Tensor:
    """y[t] += s_a B_a A_a x[t] without a workspace; v, if given, receives A_a x[t].

    The library picks the kernels: one launch on rank-16 decode batches; with v
    given on other decode batches or at r_max <= 16, the split calls' kernels
    (bit-equal to lora_shrink + lora_expand_add); otherwise one 64-row-tile launch.
    """
    _on_gpu(x, y, v)
    px, T, d_in, ldx = _rows(x, "x")
    py, Ty, d_out, ldy = _rows(y, "y")
    if Ty != T:
        raise ValueError("x and y must have the same number of rows")
    if y.dtype != x.dtype:
        raise ValueError("x and y must have the same element type")
    pv, ldv = 0, 0
    if v is not None:
        pv, Tv, _, ldv = _rows(v, "v")
        if Tv != T or v.dtype != torch.float32:
            raise ValueError("v must be fp32 with one row per row of x")
    r_max = adapters.r_max if r_max is None else r_max
    _check_batch("lora_forward", adapters, seg, T, x=x, y=y, v=v, r_max=r_max)
    st = _abi.load().lora_forward(_dtype_code(x), px, ldx, T, d_in, d_out, adapters.ptr, len(adapters), r_max,
                                  seg.c, py, ldy, pv or None, ldv, _stream(x.device))
    _abi.check("lora_forward", st)
    return y


def lora_forward_multi(x: torch.Tensor, slices, seg: Segments, r_max: Optional[int] = None) -> None:
    """Several projections of the same x: slices = [(adapters, y[, v]), ...] (1..3 entries).

    For every slice, y[t] += s_a B_a A_a x[t] with that slice's adapter table (same adapter ids),
    bit-equal to lora_forward of that slice alone with the same arguments; the slices that
    lora_forward would run in one launch share one launch (x read once per tile).
    """
    entries = [tuple(e) + (None,) * (3 - len(e)) for e in slices]
    if not 1 <= len(entries) <= _abi.LORA_MAX_SLICES:
        raise ValueError(f"1 to {_abi.LORA_MAX_SLICES} slices")
    _on_gpu(x)
    px, T, d_in, ldx = _rows(x, "x")
    arr = (_abi.LoraSlice * len(entries))()
    n_adapters = len(entries[0][0])
    for i, (table, y, v) in enumerate(entries):
        _on_gpu(y, v)
        py, Ty, d_out, ldy = _rows(y, "y")
        if Ty != T or y.dtype != x.dtype:
            raise ValueError("every y must have x's rows and element type")
        if len(table) != n_adapters:
            raise ValueError("every slice's adapter table must have the same number of entries")
        pv, ldv = 0, 0
        if v is not None:
            pv, Tv, _, ldv = _rows(v, "v")
            if Tv != T or v.dtype != torch.float32:
                raise ValueError("v must be fp32 with one row per row of x")
        arr[i] = _abi.LoraSlice(table.ptr, py, ldy, pv or None, ldv, d_out, 0)
    if r_max is None:
        r_max = max(e[0].r_max for e in entries)
    for table, y, v in entries:
        _check_batch("lora_forward_multi", table, seg, T, x=x, y=y, v=v, r_max=r_max)
    st = _abi.load().lora_forward_multi(_dtype_code(x), px, ldx, T, d_in, arr, len(entries), n_adapters, r_max,
                                        seg.c, _stream(x.device))
    _abi.check("lora_forward_multi", st)


def lora_backward(x: torch.Tensor, dy: torch.Tensor, adapters: AdapterTable, grads: GradTable, seg_ft: Segments,
                  dx: Optional[torch.Tensor] = None, v_saved: Optional[torch.Tensor] = None,
                  r_max: Optional[int] = None, ws: Optional[torch.Tensor] = None) -> None:
    """Accumulate dX (if given), dA and dB of the fine-tuning rows x / dy."""
    _backward("lora_backward", x, dy, adapters, grads, seg_ft, dx, v_saved, r_max, ws, ())


def lora_backward_preemptible(x: torch.Tensor, dy: torch.Tensor, adapters: AdapterTable, grads: GradTable,
                              seg_ft: Segments, grant: torch.Tensor, status: torch.Tensor,
                              dx: Optional[torch.Tensor] = None, v_saved: Optional[torch.Tensor] = None,
                              r_max: Optional[int] = None, ws: Optional[torch.Tensor] = None) -> None:
    """lora_backward that yields while grant[0] == 0; status[0] becomes 0 (ran) or 1 (yielded, outputs untouched).

    grant: int32 tensor on the GPU, or in pinned host memory (``pin_memory=True``), which the
    host may change while the call is queued: the device reads it when the call's gates run."""
    if not status.is_cuda or status.dtype != torch.int32 or status.numel() < 1:
        raise ValueError("status must be an int32 tensor on the GPU")
    if grant.dtype != torch.int32 or grant.numel() < 1:
        raise ValueError("grant must be an int32 tensor")
    if grant.is_cuda:
        grant_ptr = grant.data_ptr()
    elif grant.is_pinned():
        grant_ptr = _abi.host_device_pointer(grant.data_ptr())
    else:
        raise ValueError("grant must be on the GPU or in pinned host memory")
    _backward("lora_backward_preemptible", x, dy, adapters, grads, seg_ft, dx, v_saved, r_max, ws,
              (grant_ptr, status.data_ptr()))


def _backward(fn, x, dy, adapters, grads, seg_ft, dx, v_saved, r_max, ws, extra) -> None:
    _on_gpu(x, dy, dx, v_saved)
    px, T, d_in, ldx = _rows(x, "x")
    pdy, Td, d_out, lddy = _rows(dy, "dy")
    if Td != T:
        raise ValueError("x and dy must have the same number of rows")
    pdx, lddx = 0, 0
    if dx is not None:
        pdx, Tx, _, lddx = _rows(dx, "dx")
        if Tx != T or dx.dtype != x.dtype:
            raise ValueError("dx must match x")
    pvs, ldv = 0, 0
    if v_saved is not None:
        pvs, _, _, ldv = _rows(v_saved, "v_saved")
    if len(grads.dA) != len(adapters):
        raise ValueError("the gradient table must have one entry per adapter")
    r_max = adapters.r_max if r_max is None else r_max
    _check_batch(fn, adapters, seg_ft, T, x=x, v=v_saved, r_max=r_max)
    if dy.dtype != adapters.dtype or dy.shape[1] != adapters.d_out or dy.device != adapters.device:
        raise ValueError(f"{fn}: dy must be {adapters.dtype} with d_out = {adapters.d_out} columns on the adapters' device")
    for i, (ga, gb) in enumerate(zip(grads.dA, grads.dB)):
        if ga is None:
            continue
        if tuple(ga.shape) != tuple(adapters.A[i].shape) or tuple(gb.shape) != tuple(adapters.B[i].shape):
            raise ValueError(f"{fn}: gradient entry {i} must have the shapes of A[{i}] and B[{i}]")
        if ga.device != adapters.device or gb.device != adapters.device:
            raise ValueError(f"{fn}: gradient entry {i} is on another device")
    lib = _abi.load()
    if ws is None:  # a caller's workspace is size-checked by the library (LORA_ERR_WORKSPACE)
        ws = torch.empty(max(lib.lora_backward_workspace_bytes(_dtype_code(x), T, d_in, d_out, r_max), 1),
                         dtype=torch.uint8, device=x.device)
    st = getattr(lib, fn)(_dtype_code(x), px, ldx, pdy, lddy, pdx or None, lddx, T, d_in, d_out, adapters.ptr,
                          grads.ptr, len(adapters), r_max, seg_ft.c, pvs or None, ldv, ws.data_ptr(), ws.numel(),
                          *extra, _stream(x.device))
    _abi.check(fn, st)


def lora_adamw_step(tensors, *, step: int, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                    weight_decay: float = 0.01, grad_scale: float = 1.0, zero_grad: bool = False) -> None:
    """One AdamW step over a list of (w, grad, m, v[, master]) tensors (in place, one launch).

    w: bfloat16 or float32 weights (all entries one element type); grad, m, v and the
    optional master copy: float32 with w's element count, contiguous.
    """
    entries = [tuple(e) + (None,) * (5 - len(e)) for e in tensors]
    if len(entries) > _abi.LORA_ADAMW_MAX_TENSORS:
        raise ValueError(f"at most {_abi.LORA_ADAMW_MAX_TENSORS} tensors per step")
    arr = (_abi.LoraAdamwTensor * max(1, len(entries)))()
    dtype = None
    dev = None
    for i, (w, grad, m, v, master) in enumerate(entries):
        _on_gpu(w, grad, m, v, master)
        code = _dtype_code(w)
        if dtype is not None and code != dtype:
            raise ValueError("all weights of one step must share their element type")
        dtype, dev = code, w.device
        for name, t in (("w", w), ("grad", grad), ("m", m), ("v", v), ("master", master)):
            if t is None and name != "master":
                raise ValueError(f"{name} is required")
            if t is not None and (not t.is_contiguous() or t.numel() != w.numel()):
                raise ValueError(f"{name} must be contiguous with w's element count")
            if t is not None and name != "w" and t.dtype != torch.float32:
                raise ValueError(f"{name} must be float32")
        arr[i] = _abi.LoraAdamwTensor(w.data_ptr(), master.data_ptr() if master is not None else None,
                                      grad.data_ptr(), m.data_ptr(), v.data_ptr(), w.numel())
    hp = _abi.LoraAdamwParams(lr, betas[0], betas[1], eps, weight_decay, grad_scale, int(step), int(bool(zero_grad)))
    stream = _stream(dev) if dev is not None else 0
    st = _abi.load().lora_adamw_step(LORA_BF16 if dtype is None else dtype, arr, len(entries), hp, stream or None)
    _abi.check("lora_adamw_step", st)
