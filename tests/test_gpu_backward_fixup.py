"""GPU parity of the backward's contraction when one tile is cut over many
workgroups.

The contraction's workgroups take equal ranges of (tile, 32-row window)
units; a tile whose windows span several workgroups leaves one partial tile
per workgroup, and the fix-up adds them in workgroup order after finding the
run of workgroups that hold the tile (records read 64 workgroups at a time).
Narrow matrices over many rows make a handful of tiles span every
workgroup: with 32768 fine-tuning rows and 64 input columns the dA tile's
1024 windows fall four to a workgroup over all 256, so the run is read in
four batches of records.  Both routes are covered: d_out = 64 takes the
two-pass backward (the dB tile is cut the same way), d_out = 128 the
streaming one (rank <= 16, d_out >= 2 d_in).  Each result is compared with
the fp64 oracle at the bf16 bar (max|err| <= 2e-2 max|ref|) and a repeated
call must be bit-equal (the partial tiles are summed in a fixed order).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_helpers import GpuCase, rel_err

oracle.set_threads(16)
TOLB = 2e-2


@pytest.mark.parametrize("d_out", [64, 128])
@pytest.mark.parametrize("saved", [False, True])
def test_tile_cut_over_every_workgroup(d_out, saved):
    T = 32768
    rng = np.random.default_rng(11)
    # one long adapter, then a short ragged-rank one: the first tiles span all
    # workgroups, the last ones start inside a workgroup's range
    ids = np.concatenate([np.zeros(T - 300, dtype=np.int32), rng.integers(0, 2, size=300).astype(np.int32)])
    wl = workloads.custom(ids, [16, 7], 64, d_out, "bf16", seed=11, name=f"ft-narrow-{d_out}", ft_start=0,
                          ft_count=T)
    print(f"backward {wl.name} T_ft={T} saved={saved}", flush=True)
    case = GpuCase(wl)
    v = case.forward()[1] if saved else None
    dx, dA, dB, seg_ft = case.backward(v_saved=v, r_max=16)
    again = case.backward(v_saved=v, r_max=16)
    assert torch.equal(dx, again[0])
    for x, y in zip(dA + dB, again[1] + again[2]):
        assert torch.equal(x, y)
    dx_ref, dA_ref, dB_ref, _, _ = case.oracle_backward()
    errs = {"dx": rel_err(dx, dx_ref)}
    for a in (0, 1):
        errs[f"dA{a}"] = rel_err(dA[a], dA_ref[a])
        errs[f"dB{a}"] = rel_err(dB[a], dB_ref[a])
    print(errs, flush=True)
    assert int(seg_ft.err.item()) == 0
    bad = {k: v for k, v in errs.items() if not v <= TOLB}
    assert not bad, f"backward errors above {TOLB}: {bad}"
