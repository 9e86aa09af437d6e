"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: segment outputs bit-exact; y, dX, dA, dB within max|err| <= 2e-2 *
max|ref| (bf16) or 1e-5 * max|ref| (fp32) per tensor; the same rule on the
delta alone (base output zero), so the check sees the low-rank term itself.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_helpers import TOL, GpuCase, rel_err
    import expand_token_adapter_amd as lb

oracle.set_threads(16)
_config = functools.lru_cache(maxsize=None)(workloads.config)


def _ids_case(kind, T, A, rng):
    if kind == "random":
        return rng.integers(-1, A, size=T)
    if kind == "sorted":
        return np.sort(rng.integers(0, A, size=T))
    if kind == "reverse":
        return np.sort(rng.integers(0, A, size=T))[::-1]
    if kind == "same":
        return np.full(T, A - 1)
    if kind == "none":
        return np.full(T, -1)
    if kind == "zipf":
        p = np.arange(1, A + 1, dtype=float) ** -1.1
        return rng.choice(A, size=T, p=p / p.sum())
    if kind == "bad":
        return rng.integers(-4, A + 4, size=T)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["random", "sorted", "reverse", "same", "none", "zipf", "bad"])
# (6000, 1500) and (70001, 7) take the three-kernel path; the others the one-workgroup path
@pytest.mark.parametrize("T,A", [(1, 1), (255, 3), (257, 64), (2048, 320), (10368, 32), (65536, 1024),
                                 (6000, 1500), (70001, 7)])
def test_segments_bit_exact(kind, T, A):
    rng = np.random.default_rng(T * 7919 + A)
    ids = np.ascontiguousarray(_ids_case(kind, T, A, rng), dtype=np.int32)
    seg = lb.lora_segments_build(torch.from_numpy(ids).cuda(), A)
    torch.cuda.synchronize()
    counts, offsets, perm, err = oracle.segments(ids, A)
    assert np.array_equal(seg.counts.cpu().numpy(), counts)
    assert np.array_equal(seg.offsets.cpu().numpy(), offsets)
    n = int(offsets[-1])
    assert np.array_equal(seg.perm.cpu().numpy()[:n], perm)
    assert int(seg.err.item()) == err
    _check_tile_records(seg.sched.cpu().numpy(), counts, offsets, T, A)


def _check_tile_records(sched, counts, offsets, T, A):
    """The scheduling records the compute kernels walk, bit for bit: a header
    (16-row tiles, 64-row tiles, active adapters), the active adapters in
    ascending order, then per active adapter its rows in runs of 16 and of 64
    consecutive sorted positions, as (adapter, first position, rows)."""
    active = [a for a in range(A) if counts[a] > 0]

    def tiles(n):
        return [(a, int(offsets[a]) + j, min(n, int(counts[a]) - j)) for a in active for j in range(0, counts[a], n)]

    t16, t64 = tiles(16), tiles(64)
    assert list(sched[:3]) == [len(t16), len(t64), len(active)]
    off16 = 4 + (A + 3) // 4 * 4
    off64 = off16 + 4 * ((T + 15) // 16 + A)
    assert list(sched[4:4 + len(active)]) == active
    for off, want in ((off16, t16), (off64, t64)):
        got = sched[off:off + 4 * len(want)].reshape(-1, 4)[:, :3]
        assert np.array_equal(got, np.array(want, dtype=np.int64).reshape(-1, 3)), off


def test_segments_build_batch_matches_single_builds():
    """One batched call == one lora_segments_build per job, bit for bit, and the oracle;
    covers a three-kernel job, an empty job, bad ids and more jobs than one launch holds."""
    rng = np.random.default_rng(5)
    A = 32
    cases = [rng.integers(-1, A, size=8185), rng.integers(0, A, size=2048), rng.integers(-1, A, size=70001),
             np.zeros(0), rng.integers(-4, A + 4, size=300)]
    cases += [rng.integers(-1, A, size=int(n)) for n in rng.integers(1, 3000, size=6)]
    ids = [torch.from_numpy(np.ascontiguousarray(c, dtype=np.int32)).cuda() for c in cases]
    batch = lb.lora_segments_build_batch([(t, None) for t in ids], A)
    singles = [lb.lora_segments_build(t, A) for t in ids]
    torch.cuda.synchronize()
    assert len(batch) == len(cases)
    for c, b, one in zip(cases, batch, singles):
        for name in ("counts", "offsets", "err", "sched"):
            assert torch.equal(getattr(b, name), getattr(one, name)), name
        counts, offsets, perm, err = oracle.segments(np.ascontiguousarray(c, dtype=np.int32), A)
        n = int(offsets[-1])
        assert np.array_equal(b.counts.cpu().numpy(), counts)
        assert np.array_equal(b.offsets.cpu().numpy(), offsets)
        assert np.array_equal(b.perm.cpu().numpy()[:n], perm)
        assert np.array_equal(one.perm.cpu().numpy()[:n], perm)
        if len(c):
            assert int(b.err.item()) == err
            _check_tile_records(b.sched.cpu().numpy(), counts, offsets, len(c), A)


def _check_forward(case, tol, fused=False):
    y, v, seg = case.forward(fused=fused)
    y_ref, v_ref = case.oracle_forward()
    assert int(seg.err.item()) == 0
    e = rel_err(y, y_ref)
    assert e <= tol, f"y max|err|/max|ref| = {e:.3e} > {tol}"
    ranks = case.wl.ranks
    ids = case.wl.ids
    vg = v.double().cpu().numpy()
    mask = np.zeros_like(v_ref, dtype=bool)
    for t in np.nonzero(ids >= 0)[0]:
        mask[t, :ranks[ids[t]]] = True
    ev = float(np.max(np.abs(vg[:, :v_ref.shape[1]][mask] - v_ref[mask])) / np.max(np.abs(v_ref[mask])))
    assert ev <= tol, f"v max|err|/max|ref| = {ev:.3e}"
    # rows without an adapter are untouched, bit for bit
    none = ids < 0
    if none.any():
        assert torch.equal(y[torch.from_numpy(none).cuda()], case.y0[torch.from_numpy(none).cuda()])
    return y, e


def _small_mixed(dtype, seed=0):
    """Several tiles, a ragged tail, ragged ranks (incl. ones not a multiple of 8 or 16)."""
    rng = np.random.default_rng(seed)
    parts = [rng.integers(-1, 7, size=37), np.full(130, 3), np.full(77, 6), rng.integers(0, 7, size=19)]
    ids = np.concatenate(parts).astype(np.int32)
    ranks = [8, 24, 5, 40, 128, 16, 64]
    return workloads.custom(ids, ranks, 328, 200, dtype, seed=seed, name="small-mixed",
                            scales=[2.0, 0.5, 1.0, -1.5, 2.0, 3.0, 0.25])


def _small_decode(dtype, seed=0, d_out=1032):
    """Few rows per adapter (the 16-row-tile kernels for bf16): 40 adapters with ranks
    1..128 (several not a multiple of 8 or 16), rows without adapters, 1..16-row tiles,
    and 1032 output columns (two 1024-column ranges, the second one ragged)."""
    rng = np.random.default_rng(100 + seed)
    A = 40
    ranks = [8, 24, 5, 40, 128, 16, 64, 1, 12, 32, 96, 8, 16, 72, 3, 48, 128, 20, 56, 8] * 2
    ids = np.concatenate([rng.integers(-1, A, size=260), np.full(19, 7), np.full(33, 4)]).astype(np.int32)
    ids = ids[rng.permutation(len(ids))]
    scales = rng.choice([2.0, 0.5, -1.25, 3.0], size=A)
    return workloads.custom(ids, ranks, 328, d_out, dtype, seed=seed, name="small-decode", scales=scales)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("y0_zero", [False, True])
@pytest.mark.parametrize("d_out", [1032, 200])
def test_forward_small_decode(dtype, y0_zero, d_out):
    case = GpuCase(_small_decode(dtype, d_out=d_out), y0_zero=y0_zero)
    _check_forward(case, TOL[dtype])


def test_forward_decode_deterministic_and_b_zero_identity():
    wl = _small_decode("bf16")
    case = GpuCase(wl, y0_zero=True)
    y1, v1, _ = case.forward()
    y2, v2, _ = case.forward()
    assert torch.equal(y1, y2) and torch.equal(v1, v2)
    wl0 = _small_decode("bf16")
    wl0.B = [np.zeros_like(b) for b in wl0.B]
    c0 = GpuCase(wl0)
    y, _, _ = c0.forward()
    assert torch.equal(y, c0.y0)
    # columns r_a .. round_up(r_a, 8) - 1 of v are zero
    for a, r in enumerate(wl.ranks):
        rows = torch.from_numpy(wl.ids == a).cuda()
        hi = (r + 7) // 8 * 8
        if rows.any() and hi > r:
            assert not v1[rows][:, r:hi].any()


def test_forward_decode_bad_table_entries_are_skipped_and_counted():
    wl = _small_decode("bf16")
    case = GpuCase(wl)
    y = case.y0.clone()
    seg = lb.lora_segments_build(case.ids, wl.num_adapters)
    v = lb.lora_shrink(case.x, case.table, seg, r_max=64)
    lb.lora_expand_add(v, case.table, seg, y, r_max=64)
    torch.cuda.synchronize()
    assert int(seg.err.item()) > 0
    big = torch.from_numpy(np.isin(wl.ids, [a for a, r in enumerate(wl.ranks) if r > 64])).cuda()
    assert torch.equal(y[big], case.y0[big])
    ok = torch.from_numpy(wl.ids == 3).cuda()  # rank 40
    assert not torch.equal(y[ok], case.y0[ok])


def _long_rows_r64(seed=0):
    """Long row groups (more than 32 rows per adapter) with ranks 5..64
    (several not a multiple of 8 or 16): the split-K shrink and its reduce,
    with d_in = 264 (a ragged last slice) and rows without adapters."""
    rng = np.random.default_rng(400 + seed)
    parts = [np.full(70, 1), rng.integers(-1, 8, size=41), np.full(130, 4), np.full(33, 7), np.full(96, 2),
             rng.integers(0, 8, size=37)]
    ids = np.concatenate(parts).astype(np.int32)
    ranks = [8, 24, 5, 40, 64, 16, 64, 33]
    assert len(ids) > 32 * len(ranks)
    return workloads.custom(ids, ranks, 264, 200, "bf16", seed=seed, name="long-rows-r64",
                            scales=[2.0, 0.5, 1.0, -1.5, 2.0, 3.0, 0.25, -0.75])


@pytest.mark.parametrize("y0_zero", [False, True])
def test_forward_long_rows_ranks_to_64(y0_zero):
    case = GpuCase(_long_rows_r64(), y0_zero=y0_zero)
    _check_forward(case, TOL["bf16"])


def _many_decode(seed=0, A=600, T=2000, d_out=2056):
    """Many adapters with few rows each and a Zipf-like head (an adapter with
    hundreds of rows, several with tens): enough 16-row tiles x rank blocks for
    the shrink's cost-balanced plan and enough tiles x chunks for the expand's;
    ranks 1..128, d_in = 264 (a ragged K group), rows without adapters."""
    rng = np.random.default_rng(200 + seed)
    k = np.arange(1, A + 1, dtype=np.float64)
    p = k ** -1.1
    ids = rng.choice(A, size=T, p=p / p.sum()).astype(np.int32)
    ids[rng.random(T) < 0.03] = -1
    ranks = rng.choice(np.array([1, 5, 8, 12, 16, 24, 32, 40, 64, 72, 96, 128]), size=A).astype(np.int32)
    scales = rng.choice([2.0, 0.5, -1.25, 3.0], size=A)
    return workloads.custom(ids, ranks, 264, d_out, "bf16", seed=seed, name="many-decode", scales=scales)


@pytest.mark.parametrize("y0_zero", [False, True])
def test_forward_decode_balanced_plans(y0_zero):
    """Shrink and expand both in their cost-balanced modes (parity with the oracle)."""
    case = GpuCase(_many_decode(), y0_zero=y0_zero)
    _check_forward(case, TOL["bf16"])


def test_forward_decode_balanced_bad_entries_are_skipped_and_counted():
    """r_max = 64 makes the adapters of rank 72..128 bad entries: the plans give
    them no work and count them; every other row matches the oracle."""
    wl = _many_decode(seed=1)
    case = GpuCase(wl)
    y = case.y0.clone()
    seg = lb.lora_segments_build(case.ids, wl.num_adapters)
    v = lb.lora_shrink(case.x, case.table, seg, r_max=64)
    lb.lora_expand_add(v, case.table, seg, y, r_max=64)
    torch.cuda.synchronize()
    ranks = np.asarray(wl.ranks)
    bad_ids = [a for a in range(wl.num_adapters) if ranks[a] > 64]
    used_bad = set(np.unique(wl.ids[np.isin(wl.ids, bad_ids)]).tolist())
    assert used_bad and int(seg.err.item()) > 0
    bad = np.isin(wl.ids, bad_ids)
    assert torch.equal(y[torch.from_numpy(bad).cuda()], case.y0[torch.from_numpy(bad).cuda()])
    y_ref, _ = case.oracle_forward()
    good = ~bad
    e = rel_err(y[torch.from_numpy(good).cuda()], y_ref[good])
    assert e <= TOL["bf16"], e


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("y0_zero", [False, True])
def test_forward_small_mixed(dtype, y0_zero):
    case = GpuCase(_small_mixed(dtype), y0_zero=y0_zero)
    _check_forward(case, TOL[dtype])


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("y0_zero", [False, True])
def test_forward_configs_full_size(idx, y0_zero):
    wl = _config(idx)
    print(f"forward {wl.name} T={wl.T} y0_zero={y0_zero}", flush=True)
    case = GpuCase(wl, y0_zero=y0_zero)
    _check_forward(case, TOL[wl.dtype])


def test_forward_b_zero_is_bit_exact_identity():
    wl = _small_mixed("bf16")
    wl.B = [np.zeros_like(b) for b in wl.B]
    case = GpuCase(wl)
    y, _, _ = case.forward()
    assert torch.equal(y, case.y0)


def test_forward_deterministic_and_linear_in_scale():
    wl = _small_mixed("f32")
    case = GpuCase(wl, y0_zero=True)
    y1, _, _ = case.forward()
    y2, _, _ = case.forward()
    assert torch.equal(y1, y2)
    wl2 = _small_mixed("f32")
    wl2.scales = wl2.scales * 2
    y3, _, _ = GpuCase(wl2, y0_zero=True).forward()
    torch.testing.assert_close(y3, 2 * y1, rtol=1e-6, atol=1e-6)


def test_forward_bad_table_entries_are_skipped_and_counted():
    wl = _small_mixed("bf16")
    case = GpuCase(wl)
    # adapter 2: rank above r_max passed to the call -> skipped, err counted
    y = case.y0.clone()
    seg = lb.lora_segments_build(case.ids, wl.num_adapters)
    v = lb.lora_shrink(case.x, case.table, seg, r_max=64)
    lb.lora_expand_add(v, case.table, seg, y, r_max=64)
    torch.cuda.synchronize()
    assert int(seg.err.item()) > 0
    rows128 = torch.from_numpy(wl.ids == 4).cuda()  # rank-128 adapter exceeds r_max=64
    assert torch.equal(y[rows128], case.y0[rows128])
    ok = torch.from_numpy(wl.ids == 3).cuda()
    assert not torch.equal(y[ok], case.y0[ok])


# ------------------------------------------------------------------ fused forward

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("y0_zero", [False, True])
def test_fused_forward_small_mixed(dtype, y0_zero):
    """Ranks 5..128 (one to four 32-rank steps, rows that are not 16-byte units), ragged tiles."""
    case = GpuCase(_small_mixed(dtype), y0_zero=y0_zero)
    _check_forward(case, TOL[dtype], fused=True)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("y0_zero", [False, True])
def test_fused_forward_configs_full_size(idx, y0_zero):
    wl = _config(idx)
    print(f"fused forward {wl.name} T={wl.T} y0_zero={y0_zero}", flush=True)
    case = GpuCase(wl, y0_zero=y0_zero)
    _check_forward(case, TOL[wl.dtype], fused=True)


def test_fused_forward_matches_split_path_and_is_deterministic():
    wl = _small_mixed("bf16")
    case = GpuCase(wl, y0_zero=True)
    yf, vf, _ = case.forward(fused=True)
    yf2, vf2, _ = case.forward(fused=True)
    assert torch.equal(yf, yf2) and torch.equal(vf, vf2)
    ys, vs, _ = case.forward()
    assert rel_err(yf, ys.double().cpu().numpy()) <= TOL["bf16"]
    assert rel_err(vf, vs.double().cpu().numpy()) <= 1e-5  # both fp32 sums of the same bf16 products
    # columns r_a .. round_up(r_a, 8) - 1 of v are zero, as lora_shrink writes them
    for a, r in enumerate(wl.ranks):
        rows = torch.from_numpy(wl.ids == a).cuda()
        hi = (r + 7) // 8 * 8
        if rows.any() and hi > r:
            assert not vf[rows][:, r:hi].any()


def test_fused_forward_b_zero_is_bit_exact_identity():
    wl = _small_mixed("bf16")
    wl.B = [np.zeros_like(b) for b in wl.B]
    case = GpuCase(wl)
    y, _, _ = case.forward(fused=True)
    assert torch.equal(y, case.y0)


def test_fused_forward_bad_table_entries_are_skipped_and_counted():
    wl = _small_mixed("bf16")
    case = GpuCase(wl)
    y = case.y0.clone()
    seg = lb.lora_segments_build(case.ids, wl.num_adapters)
    lb.lora_forward(case.x, case.table, seg, y, r_max=64)
    torch.cuda.synchronize()
    assert int(seg.err.item()) > 0
    rows128 = torch.from_numpy(wl.ids == 4).cuda()  # rank-128 adapter exceeds r_max=64
    assert torch.equal(y[rows128], case.y0[rows128])
    ok = torch.from_numpy(wl.ids == 3).cuda()
    assert not torch.equal(y[ok], case.y0[ok])


def test_empty_batch_is_a_no_op():
    wl = _small_mixed("bf16")
    case = GpuCase(wl)
    ids = torch.zeros(0, dtype=torch.int32, device="cuda")
    seg = lb.lora_segments_build(ids, wl.num_adapters)
    x = case.x[:0]
    v = lb.lora_shrink(x, case.table, seg)
    y = case.y0[:0].clone()
    lb.lora_expand_add(v, case.table, seg, y)
    lb.lora_forward(x, case.table, seg, y)
    torch.cuda.synchronize()
    assert v.shape[0] == 0


# ------------------------------------------------------------------ backward

def _check_backward(case, tol, v_saved=None, init=False, with_dx=True):
    wl = case.wl
    rng = np.random.default_rng(99)
    dx0 = dA0 = dB0 = None
    if init:
        dx_init = rng.standard_normal((wl.ft_count, wl.d_in)).astype(np.float32)
        dx0 = workloads.fp32_to_bf16_bits(dx_init) if wl.dtype == "bf16" else dx_init
        dA0 = [rng.standard_normal(a.shape) .astype(np.float32).astype(np.float64) for a in wl.A]
        dB0 = [rng.standard_normal(b.shape).astype(np.float32).astype(np.float64) for b in wl.B]
    dx, dA, dB, seg_ft = case.backward(v_saved=v_saved, dx0=dx0, dA0=dA0, dB0=dB0, with_dx=with_dx)
    dx_ref, dA_ref, dB_ref, _, _ = case.oracle_backward(dx0=dx0, dA0=dA0, dB0=dB0)
    assert int(seg_ft.err.item()) == 0
    errs = {}
    if with_dx:
        errs["dx"] = rel_err(dx, dx_ref)
    used = sorted(set(wl.ft_ids.tolist()))
    for a in used:
        errs[f"dA{a}"] = rel_err(dA[a], dA_ref[a])
        errs[f"dB{a}"] = rel_err(dB[a], dB_ref[a])
    for a in range(wl.num_adapters):
        if a not in used and not init:
            assert not dA[a].any() and not dB[a].any()
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"backward errors above {tol}: {bad}"
    return errs


def _small_ft(dtype, seed=1):
    """Fine-tuning rows of three adapters (ragged ranks), several windows and a ragged tail."""
    rng = np.random.default_rng(seed)
    ids = np.concatenate([np.full(70, 1), rng.integers(0, 3, size=45), np.full(150, 2)]).astype(np.int32)
    T = ids.shape[0]
    return workloads.custom(ids, [16, 40, 8], 264, 392, dtype, seed=seed, name="small-ft",
                            scales=[2.0, -0.5, 1.5], ft_start=0, ft_count=T)


def _small_ft_wide(dtype, seed=2):
    """Ranks 64 / 128 / 32 / 24 (two rank groups, a rank that is not a power of two),
    row lengths that leave partial 64-wide chunks."""
    rng = np.random.default_rng(seed)
    ids = np.concatenate([rng.integers(0, 4, size=29), np.full(97, 1), np.full(40, 3), np.full(33, 0)])
    ids = ids.astype(np.int32)
    T = ids.shape[0]
    return workloads.custom(ids, [64, 128, 32, 24], 320, 136, dtype, seed=seed, name="small-ft-wide",
                            scales=[2.0, 0.75, -1.0, 1.25], ft_start=0, ft_count=T)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_small(dtype):
    _check_backward(GpuCase(_small_ft(dtype)), TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_wide_ranks(dtype):
    _check_backward(GpuCase(_small_ft_wide(dtype)), TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_wide_ranks(dtype):
    _check_forward(GpuCase(_small_ft_wide(dtype)), TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_accumulates_into_nonzero_buffers(dtype):
    _check_backward(GpuCase(_small_ft(dtype)), TOL[dtype], init=True)


def test_backward_without_dx_and_with_saved_v():
    case = GpuCase(_small_ft("bf16"))
    y, v, _ = case.forward()
    _check_backward(case, TOL["bf16"], v_saved=v, with_dx=False)


@pytest.mark.parametrize("idx", [1, 3, 4])
def test_backward_configs_full_size(idx):
    wl = _config(idx)
    print(f"backward {wl.name} T_ft={wl.ft_count}", flush=True)
    case = GpuCase(wl)
    errs = _check_backward(case, TOL[wl.dtype])
    print(errs, flush=True)


def test_backward_config3_saved_v_matches_recompute():
    wl = _config(3)
    case = GpuCase(wl)
    _, v, _ = case.forward()
    s, n = wl.ft_start, wl.ft_count
    _check_backward(case, TOL["bf16"], v_saved=v[s:s + n])


def test_backward_deterministic():
    case = GpuCase(_small_ft("bf16"))
    a = case.backward()
    b = case.backward()
    assert torch.equal(a[0], b[0])
    for x, y in zip(a[1] + a[2], b[1] + b[2]):
        assert torch.equal(x, y)
