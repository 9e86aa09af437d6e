"""Shared helpers of the GPU tests: move a synthetic workload to the GPU, run
the HIP path through the C-ABI binding, and run the oracle on the same
inputs.  Tolerances: bf16 max|err| <= 2e-2 * max|ref|, fp32 <= 1e-5 * max|ref|,
applied per output tensor; integer outputs must match exactly."""
from __future__ import annotations

import numpy as np
import torch

import expand_token_adapter_amd as lb
import oracle

TOL = {"bf16": 2e-2, "f32": 1e-5}


def to_dev(a: np.ndarray, dtype: str, dev) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def rel_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.detach().double().cpu().numpy()
    denom = float(np.max(np.abs(want))) if want.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(g))) if g.size else 0.0
    return float(np.max(np.abs(g - want)) / denom)


class GpuCase:
    """A workload resident on the GPU plus its adapter table."""

    def __init__(self, wl, dev=None, y0_zero: bool = False):
        self.wl = wl
        self.dev = dev or torch.device("cuda:0")
        dt = wl.dtype
        self.A = [to_dev(a, dt, self.dev) for a in wl.A]
        self.B = [to_dev(b, dt, self.dev) for b in wl.B]
        self.table = lb.AdapterTable(self.A, self.B, wl.scales.tolist())
        self.ids = torch.from_numpy(np.ascontiguousarray(wl.ids)).to(self.dev)
        self.x = to_dev(wl.x, dt, self.dev)
        self.y0 = torch.zeros_like(to_dev(wl.y0, dt, self.dev)) if y0_zero else to_dev(wl.y0, dt, self.dev)
        self.y0_zero = y0_zero

    def forward(self, fused: bool = False, with_v: bool = True):
        """Split path (lora_shrink + lora_expand_add) or lora_forward (with_v=False:
        no v output, so lora_forward runs one of its one-launch kernels)."""
        y = self.y0.clone()
        seg = lb.lora_segments_build(self.ids, self.wl.num_adapters)
        if fused:
            v = torch.zeros((self.wl.T, (self.table.r_max + 7) // 8 * 8), dtype=torch.float32, device=self.dev)
            lb.lora_forward(self.x, self.table, seg, y, v=v if with_v else None)
        else:
            v = lb.lora_shrink(self.x, self.table, seg)
            lb.lora_expand_add(v, self.table, seg, y)
        torch.cuda.synchronize()
        return y, v, seg

    def backward(self, v_saved=None, dx0=None, dA0=None, dB0=None, with_dx=True, grant=None, status=None,
                 r_max=None, grads_none=()):
        """lora_backward, or lora_backward_preemptible when a grant word is given.

        r_max: passed to the call (None: the table's); grads_none: adapters given no
        gradient entry."""
        wl = self.wl
        s, n = wl.ft_start, wl.ft_count
        dev = self.dev
        dA = [torch.zeros(a.shape, dtype=torch.float32, device=dev) if dA0 is None
              else torch.from_numpy(dA0[i]).float().to(dev) for i, a in enumerate(wl.A)]
        dB = [torch.zeros(b.shape, dtype=torch.float32, device=dev) if dB0 is None
              else torch.from_numpy(dB0[i]).float().to(dev) for i, b in enumerate(wl.B)]
        grads = lb.GradTable([None if i in grads_none else t for i, t in enumerate(dA)],
                             [None if i in grads_none else t for i, t in enumerate(dB)])
        seg_ft = lb.lora_segments_build(self.ids[s:s + n].contiguous(), wl.num_adapters)
        dx = None
        if with_dx:
            dx = torch.zeros((n, wl.d_in), dtype=self.x.dtype, device=dev) if dx0 is None else to_dev(dx0, wl.dtype, dev)
        dy = to_dev(wl.dy, wl.dtype, dev)
        if grant is None:
            lb.lora_backward(self.x[s:s + n], dy, self.table, grads, seg_ft, dx=dx, v_saved=v_saved, r_max=r_max)
        else:
            lb.lora_backward_preemptible(self.x[s:s + n], dy, self.table, grads, seg_ft, grant, status, dx=dx,
                                         v_saved=v_saved, r_max=r_max)
        torch.cuda.synchronize()
        return dx, dA, dB, seg_ft

    # ---------------------------------------------------------------- oracle
    def oracle_forward(self):
        ref = oracle.from_workload(self.wl)
        y0 = np.zeros_like(ref["y0"]) if self.y0_zero else ref["y0"]
        return oracle.forward(ref["x"], ref["ids"], ref["ranks"], ref["scales"], ref["A"], ref["B"], y0)

    def oracle_backward(self, dx0=None, dA0=None, dB0=None):
        wl = self.wl
        ref = oracle.from_workload(wl)
        s, n = wl.ft_start, wl.ft_count
        dx0f = None if dx0 is None else oracle.to_f64(dx0, wl.dtype)
        return oracle.backward(ref["x"][s:s + n], ref["dy"], ref["ids"][s:s + n], ref["ranks"], ref["scales"],
                               ref["A"], ref["B"], dx0=dx0f, dA0=dA0, dB0=dB0)
