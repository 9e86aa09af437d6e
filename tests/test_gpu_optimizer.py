"""GPU parity of the AdamW step (lora_adamw_step) against the fp64 oracle.

Bars: fp32 results (master weights, moments, fp32 weights) within
max|err| <= 1e-5 * max|ref| per tensor; bf16 weights equal the round-to-
nearest-even of the GPU's own fp32 master bit for bit, and, without a
master, within one bf16 unit in the last place of the oracle's value rounded
the same way (the rounding decision is taken on an fp32 value on the GPU and
on the fp64 value in the oracle).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import expand_token_adapter_amd as lb

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
DEV = "cuda:0"


def _f32(**hp):
    # the C ABI carries the hyper-parameters as fp32: the oracle gets the same values
    return {k: float(np.float32(v)) for k, v in hp.items()}


def _bf16_to_f64(bits):
    return oracle.to_f64(np.asarray(bits, np.uint16), "bf16")


def _gpu_bf16(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _rel(gpu, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _shapes():
    # dA / dB of two adapters (ranks 3 and 16) plus an odd-sized tensor with a
    # partial group of 8 and one spanning several workgroups
    return [(3, 40), (72, 3), (16, 4096), (4096, 16), (1001,)]


def _tensors(rng, dtype):
    out = []
    for shp in _shapes():
        w = (rng.standard_normal(shp) * 0.02).astype(np.float32)
        out.append(w)
    return out


def test_adamw_bf16_with_master_matches_oracle_over_steps():
    rng = np.random.default_rng(0)
    ws = _tensors(rng, "bf16")
    master = [torch.tensor(w, device=DEV) for w in ws]
    wb = [_gpu_bf16(workloads.fp32_to_bf16_bits(w)) for w in ws]
    m = [torch.zeros(w.shape, dtype=torch.float32, device=DEV) for w in ws]
    v = [torch.zeros(w.shape, dtype=torch.float32, device=DEV) for w in ws]
    ref = [(w.astype(np.float64), np.zeros(w.shape), np.zeros(w.shape)) for w in ws]
    for step in range(1, 4):
        grads = [(rng.standard_normal(w.shape) * (0.5 + step)).astype(np.float32) for w in ws]
        g = [torch.tensor(x, device=DEV) for x in grads]
        lb.lora_adamw_step([(wb[i], g[i], m[i], v[i], master[i]) for i in range(len(ws))], step=step,
                           lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                           weight_decay=HP["weight_decay"], grad_scale=0.25)
        ref = [oracle.adamw(r[0], gr, r[1], r[2], step=step, grad_scale=0.25, **_f32(**HP))
               for r, gr in zip(ref, grads)]
        torch.cuda.synchronize()
        for i in range(len(ws)):
            assert _rel(master[i].cpu().numpy(), ref[i][0]) <= 1e-5, (step, i)
            assert _rel(m[i].cpu().numpy(), ref[i][1]) <= 1e-5, (step, i)
            assert _rel(v[i].cpu().numpy(), ref[i][2]) <= 1e-5, (step, i)
            # w is the RNE rounding of the GPU's own master, bit for bit
            np.testing.assert_array_equal(_bits(wb[i]), workloads.fp32_to_bf16_bits(master[i].cpu().numpy()))
            # the gradient is left in place without zero_grad
            np.testing.assert_array_equal(g[i].cpu().numpy(), grads[i])


def test_adamw_bf16_without_master_within_one_ulp():
    rng = np.random.default_rng(1)
    ws = _tensors(rng, "bf16")
    bits = [workloads.fp32_to_bf16_bits(w) for w in ws]
    wb = [_gpu_bf16(b) for b in bits]
    m = [torch.zeros(w.shape, dtype=torch.float32, device=DEV) for w in ws]
    v = [torch.zeros(w.shape, dtype=torch.float32, device=DEV) for w in ws]
    grads = [(rng.standard_normal(w.shape)).astype(np.float32) for w in ws]
    g = [torch.tensor(x, device=DEV) for x in grads]
    lb.lora_adamw_step([(wb[i], g[i], m[i], v[i]) for i in range(len(ws))], step=1, zero_grad=True,
                       lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"], weight_decay=HP["weight_decay"])
    torch.cuda.synchronize()
    for i in range(len(ws)):
        rw, rm, rv = oracle.adamw(_bf16_to_f64(bits[i]), grads[i], np.zeros(ws[i].shape), np.zeros(ws[i].shape),
                                  step=1, **_f32(**HP))
        want = workloads.fp32_to_bf16_bits(rw.astype(np.float32))
        got = _bits(wb[i])
        ulp = np.abs(_bf16_to_f64(want)) * 2.0 ** -7  # one bf16 unit in the last place (upper bound)
        assert np.all(np.abs(_bf16_to_f64(got) - _bf16_to_f64(want)) <= ulp), i
        assert np.mean(got == want) >= 0.999, i
        assert _rel(m[i].cpu().numpy(), rm) <= 1e-5 and _rel(v[i].cpu().numpy(), rv) <= 1e-5
        assert not g[i].any().item()  # zero_grad


def test_adamw_fp32_weights_from_a_nonzero_state():
    rng = np.random.default_rng(2)
    shapes = _shapes()
    w0 = [rng.standard_normal(s) for s in shapes]
    m0 = [rng.standard_normal(s) * 0.1 for s in shapes]
    v0 = [np.abs(rng.standard_normal(s)) * 0.01 for s in shapes]
    grads = [rng.standard_normal(s) for s in shapes]
    to = lambda a: torch.tensor(np.asarray(a, np.float32), device=DEV)
    w, m, v, g = [to(a) for a in w0], [to(a) for a in m0], [to(a) for a in v0], [to(a) for a in grads]
    f32 = lambda a: np.asarray(a, np.float32).astype(np.float64)
    lb.lora_adamw_step([(w[i], g[i], m[i], v[i]) for i in range(len(shapes))], step=7, lr=3e-3, betas=(0.8, 0.99),
                       eps=1e-6, weight_decay=0.1)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        rw, rm, rv = oracle.adamw(f32(w0[i]), f32(grads[i]), f32(m0[i]), f32(v0[i]), step=7,
                                  **_f32(lr=3e-3, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.1))
        assert _rel(w[i].cpu().numpy(), rw) <= 1e-5, i
        assert _rel(m[i].cpu().numpy(), rm) <= 1e-5, i
        assert _rel(v[i].cpu().numpy(), rv) <= 1e-5, i


def test_adamw_empty_calls_and_empty_entries_change_nothing():
    lb.lora_adamw_step([], step=1)
    w = torch.ones(16, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(0, dtype=torch.float32, device=DEV)
    ew = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(16, dtype=torch.float32, device=DEV)
    m = torch.zeros(16, dtype=torch.float32, device=DEV)
    v = torch.zeros(16, dtype=torch.float32, device=DEV)
    lb.lora_adamw_step([(ew, e, e, e), (w, g, m, v)], step=1, lr=0.0, weight_decay=0.0)
    torch.cuda.synchronize()
    assert torch.equal(w, torch.ones_like(w))  # lr = 0: weights unchanged
    assert torch.allclose(m, torch.full_like(m, 1.0 - np.float32(0.9)))
