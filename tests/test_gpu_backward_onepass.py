"""GPU parity of the streaming backward (bf16, trained adapters of rank <= 16).

With r_max <= 16 and d_out >= 2 d_in a bf16 backward computes g = B^T dy and
dB from one read of dY (partials per 256-column slice, dB tiles cut between
workgroups added in workgroup order); other shapes take the two-pass
backward, which the full-size fine-tuning workload (5120 -> 5120) exercises
here with the same r_max.  Each case is compared with the fp64 oracle at the usual
bar (max|err| <= 2e-2 * max|ref| per tensor): ragged ranks (1, 5, 12, 16), a
window shared by several adapters, a column slice cut by d_out, pairs cut
between workgroups, many small adapters, saved and recomputed v, nonzero
initial buffers, the two fine-tuning workloads at full size, bad entries and
adapters without gradient entries.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_helpers import TOL, GpuCase, rel_err, to_dev
    import expand_token_adapter_amd as lb

oracle.set_threads(16)
_config = functools.lru_cache(maxsize=None)(workloads.config)
TOLB = 2e-2  # the bf16 bar of every GPU parity test


def _ft16(seed=3, d_in=264, d_out=1032):
    """Four adapters (ranks 16, 5, 12, 1) over 299 rows: long runs, a mixed
    stretch, a one-row adapter; d_out leaves a last column slice of 8."""
    rng = np.random.default_rng(seed)
    ids = np.concatenate([np.full(70, 1), rng.integers(0, 4, size=45), np.full(150, 2), np.full(1, 3),
                          np.full(33, 0)]).astype(np.int32)
    return workloads.custom(ids, [16, 5, 12, 1], d_in, d_out, "bf16", seed=seed, name="ft16",
                            scales=[2.0, -0.5, 1.5, 3.0], ft_start=0, ft_count=int(ids.shape[0]))


def _check(case, r_max=16, v_saved=None, init=False, with_dx=True, skip=(), grads_none=()):
    """Run the backward and compare with the oracle; adapters in `skip` are
    bad entries: their dA / dB and dX rows must stay as they were."""
    wl = case.wl
    rng = np.random.default_rng(99)
    dx0 = dA0 = dB0 = None
    if init:
        dx0 = workloads.fp32_to_bf16_bits(rng.standard_normal((wl.ft_count, wl.d_in)).astype(np.float32))
        dA0 = [rng.standard_normal(a.shape).astype(np.float32).astype(np.float64) for a in wl.A]
        dB0 = [rng.standard_normal(b.shape).astype(np.float32).astype(np.float64) for b in wl.B]
    dx, dA, dB, seg_ft = case.backward(v_saved=v_saved, dx0=dx0, dA0=dA0, dB0=dB0, with_dx=with_dx, r_max=r_max,
                                       grads_none=grads_none)
    dx_ref, dA_ref, dB_ref, _, _ = case.oracle_backward(dx0=dx0, dA0=dA0, dB0=dB0)
    ids = wl.ids[wl.ft_start:wl.ft_start + wl.ft_count]
    errs = {}
    if with_dx:
        keep = ~np.isin(ids, list(skip))
        got = dx.detach()[torch.from_numpy(keep).to(dx.device)]
        errs["dx"] = rel_err(got, dx_ref[keep])
        if skip:
            before = to_dev(dx0, "bf16", dx.device) if init else torch.zeros_like(dx)
            rows = torch.from_numpy(~keep).to(dx.device)
            assert torch.equal(dx[rows], before[rows]), "rows of a bad entry were written"
    for a in sorted(set(ids.tolist())):
        if a in skip or a in grads_none:
            continue
        errs[f"dA{a}"] = rel_err(dA[a], dA_ref[a])
        errs[f"dB{a}"] = rel_err(dB[a], dB_ref[a])
    for a in skip:
        want = torch.from_numpy(dB0[a]).float() if init else torch.zeros(dB[a].shape)
        assert torch.equal(dB[a].cpu(), want) and torch.equal(dA[a].cpu(), torch.from_numpy(dA0[a]).float()
                                                                  if init else torch.zeros(dA[a].shape))
    bad = {k: v for k, v in errs.items() if not v <= TOLB}
    assert not bad, f"backward errors above {TOLB}: {bad}"
    return errs, int(seg_ft.err.item()), (dx, dA, dB)


@pytest.mark.parametrize("init", [False, True])
@pytest.mark.parametrize("saved", [False, True])
def test_one_pass_small(saved, init):
    case = GpuCase(_ft16())
    v = case.forward()[1] if saved else None
    errs, err, _ = _check(case, v_saved=v, init=init)
    assert err == 0, errs


def test_one_pass_without_dx():
    case = GpuCase(_ft16(seed=4, d_in=64, d_out=256))
    errs, err, _ = _check(case, with_dx=False)
    assert err == 0


def test_one_pass_pairs_cut_between_workgroups():
    """One adapter, 3000 rows x 2056 columns: 9 slices x 94 windows spread
    over 256 workgroups, so most (adapter, slice) pairs are cut."""
    ids = np.zeros(3000, dtype=np.int32)
    wl = workloads.custom(ids, [16], 128, 2056, "bf16", seed=5, name="ft16-cut", ft_start=0, ft_count=3000)
    errs, err, _ = _check(GpuCase(wl))
    assert err == 0


def test_one_pass_many_small_adapters():
    """300 adapters with 1-3 rows each (ranks 1..16): workgroups hold many
    whole pairs; ids in random order."""
    rng = np.random.default_rng(6)
    counts = rng.integers(1, 4, size=300)
    ids = np.repeat(np.arange(300, dtype=np.int32), counts)
    rng.shuffle(ids)
    ranks = rng.integers(1, 17, size=300)
    wl = workloads.custom(ids, ranks, 136, 520, "bf16", seed=6, name="ft16-many", ft_start=0,
                          ft_count=int(ids.shape[0]))
    errs, err, _ = _check(GpuCase(wl))
    assert err == 0


def test_one_pass_deterministic_and_close_to_two_pass():
    case = GpuCase(_ft16(seed=7))
    a = case.backward(r_max=16)
    b = case.backward(r_max=16)
    assert torch.equal(a[0], b[0])
    for x, y in zip(a[1] + a[2], b[1] + b[2]):
        assert torch.equal(x, y)
    two = case.backward(r_max=64)  # the two-pass backward
    for x, y in zip(a[1] + a[2], two[1] + two[2]):
        scale = float(y.abs().max()) or 1.0
        assert float((x - y).abs().max()) <= 2e-3 * scale


@pytest.mark.parametrize("idx", [3, 4])
def test_one_pass_configs_full_size(idx):
    wl = _config(idx)
    ft_ranks = {int(wl.ranks[a]) for a in set(wl.ids[wl.ft_start:wl.ft_start + wl.ft_count].tolist())}
    assert max(ft_ranks) <= 16
    print(f"one-pass backward {wl.name} T_ft={wl.ft_count}", flush=True)
    case = GpuCase(wl)
    v = None
    if idx == 3:
        v = case.forward()[1][wl.ft_start:wl.ft_start + wl.ft_count]
    errs, err, _ = _check(case, v_saved=v)
    print(errs, flush=True)
    assert err == 0


def test_one_pass_bad_entry_is_skipped_and_counted():
    """Adapter 2 (rank 20 > r_max = 16) is a bad entry: its rows' dX and its
    gradients stay as they were, the others are exact, err counts it."""
    rng = np.random.default_rng(8)
    ids = np.concatenate([np.full(40, 0), np.full(50, 2), rng.integers(0, 3, size=30), np.full(20, 1)])
    wl = workloads.custom(ids.astype(np.int32), [16, 7, 20], 96, 264, "bf16", seed=8, name="ft16-bad",
                          ft_start=0, ft_count=int(ids.shape[0]))
    errs, err, _ = _check(GpuCase(wl), init=True, skip=(2,))
    assert err > 0


def test_one_pass_adapter_without_gradients():
    """Adapter 1 has no gradient entry: its dA / dB are not written, its rows
    still receive dX, the call counts it."""
    case = GpuCase(_ft16(seed=9))
    errs, err, (dx, dA, dB) = _check(case, grads_none=(1,))
    assert err > 0 and "dx" in errs
