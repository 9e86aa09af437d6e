"""GPU parity of lora_forward's routes.  Its decode route (bf16, r_max <= 16,
at most 32 rows per adapter): one 16-wave workgroup per (16-row tile, column
range), v = A x over d_in in registers, then y += s B v.  With v given and a
decode batch or r_max <= 16 otherwise, the call runs the split calls' kernels
(bit-equal to lora_shrink + lora_expand_add); without v, the 64-row-tile
kernel.

Each case is compared with the fp64 oracle at the usual bar (max|err| <=
2e-2 * max|ref| for y and v): ragged ranks (1, 3, 5, 8, 12, 16), rows without
adapters, adapters with one row and with several 16-row tiles, d_in below one
32-element step per wave, not a multiple of 32, and large enough for several
rounds of loads per wave, d_out with a ragged last chunk and below one chunk;
y0 as drawn and y0 = 0; agreement with the split calls; bad table entries;
B = 0.
"""
import numpy as np
import pytest
import torch

import functools

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_helpers import TOL, GpuCase, rel_err
    import expand_token_adapter_amd as lb

RANKS = [1, 5, 8, 12, 16, 3, 16, 8]


def _dec16(seed=0, d_in=264, d_out=1032, A=48, T=320):
    """Few rows per adapter (T <= 32 A): random ids with rows of id -1, plus
    one adapter with 40 rows (three 16-row tiles) and one with a single row."""
    rng = np.random.default_rng(300 + seed)
    ids = rng.integers(-1, A, size=T - 41).astype(np.int32)
    ids = np.concatenate([ids, np.full(40, 2, dtype=np.int32), np.full(1, A - 1, dtype=np.int32)])
    ids = ids[rng.permutation(len(ids))]
    ranks = [RANKS[a % len(RANKS)] for a in range(A)]
    scales = rng.choice([2.0, 0.5, -1.25, 3.0], size=A)
    wl = workloads.custom(ids, ranks, d_in, d_out, "bf16", seed=seed, name="dec16", scales=scales)
    assert wl.T <= 32 * A and max(ranks) <= 16
    return wl


def _check(case):
    y, v, seg = case.forward(fused=True)
    y_ref, v_ref = case.oracle_forward()
    assert int(seg.err.item()) == 0
    e = rel_err(y, y_ref)
    assert e <= TOL["bf16"], f"y max|err|/max|ref| = {e:.3e}"
    wl = case.wl
    mask = np.zeros_like(v_ref, dtype=bool)
    for t in np.nonzero(wl.ids >= 0)[0]:
        mask[t, :wl.ranks[wl.ids[t]]] = True
    vg = v.double().cpu().numpy()[:, :v_ref.shape[1]]
    ev = float(np.max(np.abs(vg[mask] - v_ref[mask])) / np.max(np.abs(v_ref[mask])))
    assert ev <= TOL["bf16"], f"v max|err|/max|ref| = {ev:.3e}"
    none = torch.from_numpy(wl.ids < 0).cuda()
    assert torch.equal(y[none], case.y0[none]), "rows without an adapter were written"
    return y, v


@pytest.mark.parametrize("y0_zero", [False, True])
@pytest.mark.parametrize("d_in,d_out", [(264, 1032), (24, 200), (4104, 72), (8192, 4096)])
def test_fused_decode_matches_oracle(d_in, d_out, y0_zero):
    print(f"fused decode d_in={d_in} d_out={d_out} y0_zero={y0_zero}", flush=True)
    _check(GpuCase(_dec16(d_in=d_in, d_out=d_out), y0_zero=y0_zero))


def test_fused_decode_matches_split_calls_and_is_deterministic():
    wl = _dec16(seed=1, d_in=520, d_out=1032)
    case = GpuCase(wl, y0_zero=True)
    yf, vf, _ = case.forward(fused=True)
    yf2, vf2, _ = case.forward(fused=True)
    assert torch.equal(yf, yf2) and torch.equal(vf, vf2)
    ys, vs, _ = case.forward()
    assert rel_err(yf, ys.double().cpu().numpy()) <= TOL["bf16"]
    assert rel_err(vf, vs.double().cpu().numpy()) <= 1e-5  # fp32 sums of the same bf16 products
    for a, r in enumerate(wl.ranks):
        rows = torch.from_numpy(wl.ids == a).cuda()
        hi = (r + 7) // 8 * 8
        if rows.any() and hi > r:
            assert not vf[rows][:, r:hi].any()


def test_fused_decode_bad_entries_are_skipped_and_counted():
    """r_max = 8 makes the rank-12 and rank-16 adapters bad entries: their rows
    keep y0, the call counts them, every other row matches the oracle."""
    wl = _dec16(seed=2)
    case = GpuCase(wl)
    y = case.y0.clone()
    seg = lb.lora_segments_build(case.ids, wl.num_adapters)
    lb.lora_forward(case.x, case.table, seg, y, r_max=8)
    torch.cuda.synchronize()
    assert int(seg.err.item()) > 0
    ranks = np.asarray(wl.ranks)
    bad = np.isin(wl.ids, np.nonzero(ranks > 8)[0])
    badt = torch.from_numpy(bad).cuda()
    assert torch.equal(y[badt], case.y0[badt])
    y_ref, _ = case.oracle_forward()
    e = rel_err(y[~badt], y_ref[~bad])
    assert e <= TOL["bf16"], e


def test_fused_decode_b_zero_is_bit_exact_identity():
    wl = _dec16(seed=3)
    wl.B = [np.zeros_like(b) for b in wl.B]
    case = GpuCase(wl)
    y, _, _ = case.forward(fused=True)
    assert torch.equal(y, case.y0)


def test_fused_decode_one_tile_many_ranges():
    """Two adapters, 17 rows (two tiles, the second of one row), d_out of 40
    chunks: two column ranges per tile, one or two chunks per wave."""
    ids = np.array([0] * 16 + [1], dtype=np.int32)
    wl = workloads.custom(ids, [16, 7], 96, 2560, "bf16", seed=4, name="dec16-ranges", scales=[1.5, -2.0])
    _check(GpuCase(wl))


_config = functools.lru_cache(maxsize=None)(workloads.config)


def _zipf64(seed=5):
    """Decode batch with ranks up to 64 (at most 32 rows per adapter)."""
    rng = np.random.default_rng(500 + seed)
    k = np.arange(1, 81, dtype=np.float64)
    ids = rng.choice(80, size=600, p=(k ** -1.1) / (k ** -1.1).sum()).astype(np.int32)
    ids[rng.random(600) < 0.05] = -1
    ranks = rng.choice(np.array([8, 12, 16, 32, 40, 64]), size=80).astype(np.int32)
    return workloads.custom(ids, ranks, 264, 520, "bf16", seed=seed, name="zipf64")


def _long16(seed=6):
    """Long row groups (more than 32 rows per adapter) at ranks <= 16."""
    rng = np.random.default_rng(600 + seed)
    ids = np.concatenate([np.full(300, 0), rng.integers(-1, 3, size=50), np.full(200, 2)]).astype(np.int32)
    return workloads.custom(ids, [16, 5, 12], 200, 328, "bf16", seed=seed, name="long16")


@pytest.mark.parametrize("make", [_zipf64, _long16])
def test_forward_with_v_runs_the_split_kernels_bit_for_bit(make):
    wl = make()
    case = GpuCase(wl, y0_zero=False)
    yf, vf, seg = case.forward(fused=True)
    ys, vs, _ = case.forward()
    assert int(seg.err.item()) == 0
    assert torch.equal(yf, ys) and torch.equal(vf[:, :vs.shape[1]], vs)
    y_ref, _ = case.oracle_forward()
    assert rel_err(yf, y_ref) <= TOL["bf16"]


@pytest.mark.parametrize("make", [_zipf64, _long16])
def test_forward_without_v_runs_one_launch_and_matches_oracle(make):
    case = GpuCase(make(), y0_zero=True)
    y, _, seg = case.forward(fused=True, with_v=False)
    y_ref, _ = case.oracle_forward()
    assert int(seg.err.item()) == 0
    assert rel_err(y, y_ref) <= TOL["bf16"]


@pytest.mark.parametrize("idx", [4, 5])
def test_forward_without_v_configs_full_size(idx):
    """The 64-row-tile one-launch kernel on the fine-tuning and many-adapter
    workloads (with v given, lora_forward runs the split kernels there)."""
    wl = _config(idx)
    print(f"lora_forward without v {wl.name} T={wl.T}", flush=True)
    case = GpuCase(wl, y0_zero=True)
    y, _, seg = case.forward(fused=True, with_v=False)
    y_ref, _ = case.oracle_forward()
    assert int(seg.err.item()) == 0
    assert rel_err(y, y_ref) <= TOL["bf16"]
