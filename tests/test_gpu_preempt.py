"""GPU tests of the preemptible backward (lora_backward_preemptible).

The grant word is set from the host (a host-to-device copy) before each call.
Granted, the call must produce exactly what lora_backward produces (the same
kernels run in the same order); withdrawn, it must leave dA, dB and dX
bit-identical to their values before the call and report status 1; re-issued
after a yield, it must produce what a single granted call produces.
"""
import functools

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_helpers import GpuCase

_config = functools.lru_cache(maxsize=None)(workloads.config)


def _initial(wl, seed):
    """Nonzero starting values of dX (element type), dA and dB (fp32)."""
    rng = np.random.default_rng(seed)
    n = wl.ft_count
    dx0 = rng.standard_normal((n, wl.d_in)).astype(np.float32)
    if wl.dtype == "bf16":
        dx0 = workloads.fp32_to_bf16_bits(dx0)
    dA0 = [rng.standard_normal(a.shape).astype(np.float32) for a in wl.A]
    dB0 = [rng.standard_normal(b.shape).astype(np.float32) for b in wl.B]
    return dx0, dA0, dB0


def _word(v):
    w = torch.empty(1, dtype=torch.int32, device="cuda:0")
    w.copy_(torch.tensor([v], dtype=torch.int32))  # set from the host
    return w


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved_v"])
@pytest.mark.parametrize("cfg", [1, 4])
def test_granted_call_equals_lora_backward(cfg, saved):
    c = GpuCase(_config(cfg))
    wl = c.wl
    s, n = wl.ft_start, wl.ft_count
    v_saved = c.forward()[1][s:s + n] if saved else None
    dx0, dA0, dB0 = _initial(wl, 5)
    dx_r, dA_r, dB_r, _ = c.backward(v_saved, dx0, dA0, dB0)
    status = _word(7)
    dx, dA, dB, _ = c.backward(v_saved, dx0, dA0, dB0, grant=_word(1), status=status)
    assert status.item() == 0
    assert torch.equal(dx, dx_r) and _same(dA, dA_r) and _same(dB, dB_r)
    assert not torch.equal(dA[int(wl.ft_ids[0])], torch.from_numpy(dA0[int(wl.ft_ids[0])]).cuda())


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved_v"])
@pytest.mark.parametrize("cfg", [1, 4])
def test_withdrawn_grant_leaves_outputs_untouched(cfg, saved):
    c = GpuCase(_config(cfg))
    wl = c.wl
    s, n = wl.ft_start, wl.ft_count
    v_saved = c.forward()[1][s:s + n] if saved else None
    dx0, dA0, dB0 = _initial(wl, 6)
    status = _word(7)
    dx, dA, dB, seg_ft = c.backward(v_saved, dx0, dA0, dB0, grant=_word(0), status=status)
    assert status.item() == 1
    from gpu_helpers import to_dev
    assert torch.equal(dx, to_dev(dx0, wl.dtype, dx.device))
    assert _same(dA, [torch.from_numpy(a).cuda() for a in dA0])
    assert _same(dB, [torch.from_numpy(b).cuda() for b in dB0])
    assert seg_ft.err.item() == 0


def test_reissued_after_yield_equals_one_granted_call():
    c = GpuCase(_config(4))
    wl = c.wl
    s, n = wl.ft_start, wl.ft_count
    import expand_token_adapter_amd as lb
    dev = c.dev
    dA = [torch.zeros(a.shape, dtype=torch.float32, device=dev) for a in wl.A]
    dB = [torch.zeros(b.shape, dtype=torch.float32, device=dev) for b in wl.B]
    grads = lb.GradTable(dA, dB)
    seg_ft = lb.lora_segments_build(c.ids[s:s + n].contiguous(), wl.num_adapters)
    dx = torch.zeros((n, wl.d_in), dtype=c.x.dtype, device=dev)
    from gpu_helpers import to_dev
    dy = to_dev(wl.dy, wl.dtype, dev)
    grant, status = _word(0), _word(7)
    lb.lora_backward_preemptible(c.x[s:s + n], dy, c.table, grads, seg_ft, grant, status, dx=dx)
    torch.cuda.synchronize()
    assert status.item() == 1 and not dx.any().item()
    grant.copy_(torch.tensor([1], dtype=torch.int32))  # granted again, from the host
    lb.lora_backward_preemptible(c.x[s:s + n], dy, c.table, grads, seg_ft, grant, status, dx=dx)
    torch.cuda.synchronize()
    assert status.item() == 0
    dx_r, dA_r, dB_r, _ = c.backward()
    assert torch.equal(dx, dx_r) and _same(dA, dA_r) and _same(dB, dB_r)


# ---------------------------------------------------------------- grant word in pinned host memory

def _pinned_word(v):
    w = torch.empty(1, dtype=torch.int32, pin_memory=True)
    w[0] = v
    return w


def _queued_call(c, grant_value_at_enqueue, grant_value_later):
    """Enqueue lora_backward_preemptible behind a long bounded spin kernel, then change
    the pinned host grant word while the spin still runs (checked with an event that
    completes only when the spin has ended, i.e. before the call's first gate runs)."""
    import expand_token_adapter_amd as lb
    from gpu_helpers import to_dev
    wl = c.wl
    s, n = wl.ft_start, wl.ft_count
    dev = c.dev
    dx0, dA0, dB0 = _initial(wl, 8)
    dA = [torch.from_numpy(a).to(dev) for a in dA0]
    dB = [torch.from_numpy(b).to(dev) for b in dB0]
    grads = lb.GradTable(dA, dB)
    seg_ft = lb.lora_segments_build(c.ids[s:s + n].contiguous(), wl.num_adapters)
    dx = to_dev(dx0, wl.dtype, dev)
    dy = to_dev(wl.dy, wl.dtype, dev)
    grant, status = _pinned_word(grant_value_at_enqueue), _word(7)
    torch.cuda.synchronize()
    spun = torch.cuda.Event()
    torch.cuda._sleep(400_000_000)  # bounded: a few hundred ms of clock cycles
    spun.record()
    lb.lora_backward_preemptible(c.x[s:s + n], dy, c.table, grads, seg_ft, grant, status, dx=dx)
    grant[0] = grant_value_later  # from the host, while the call is queued
    still_spinning = not spun.query()
    torch.cuda.synchronize()
    assert still_spinning, "the spin ended before the grant changed: the test did not test a queued call"
    return dx, dA, dB, status, (dx0, dA0, dB0)


def test_pinned_grant_withdrawn_while_queued_yields():
    c = GpuCase(_config(4))
    dx, dA, dB, status, (dx0, dA0, dB0) = _queued_call(c, 1, 0)
    from gpu_helpers import to_dev
    assert status.item() == 1
    assert torch.equal(dx, to_dev(dx0, c.wl.dtype, dx.device))
    assert _same(dA, [torch.from_numpy(a).cuda() for a in dA0])
    assert _same(dB, [torch.from_numpy(b).cuda() for b in dB0])


def test_pinned_grant_given_while_queued_runs():
    c = GpuCase(_config(4))
    dx, dA, dB, status, (dx0, dA0, dB0) = _queued_call(c, 0, 1)
    assert status.item() == 0
    dx_r, dA_r, dB_r, _ = c.backward(None, dx0, dA0, dB0)
    assert torch.equal(dx, dx_r) and _same(dA, dA_r) and _same(dB, dB_r)
