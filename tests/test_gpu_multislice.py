"""GPU parity of the multi-slice fused forward (lora_forward_multi).

Several projections read one x, each with its own adapter table (same ids).
Every slice's y must match the fp64 oracle of that slice alone (the bf16 /
fp32 bars of the forward), and equal bit for bit what lora_forward computes
for the slice alone with the same arguments (v given or not): the per-slice
routes, arithmetic and sum order do not change.  Each slice's v matches the
oracle.  Slices given v on a decode batch with r_max > 16 run the split
kernels while the others share one launch; that mix is a case of its own.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import expand_token_adapter_amd as lb
    from gpu_helpers import TOL, rel_err, to_dev

DEV = "cuda:0"


def _slices(ids, d_in, d_outs, rank_sets, dtype, seed):
    """One workload per slice with the same ids; x is taken from slice 0."""
    return [workloads.custom(ids, ranks, d_in, d_out, dtype, seed=seed + 17 * q)
            for q, (d_out, ranks) in enumerate(zip(d_outs, rank_sets))]


def _run(wls, dtype, with_v, multi=True, bad=None):
    """with_v: one bool for every slice, or one per slice."""
    if isinstance(with_v, bool):
        with_v = [with_v] * len(wls)
    x = to_dev(wls[0].x, dtype, DEV)
    ids = torch.from_numpy(np.ascontiguousarray(wls[0].ids)).to(DEV)
    n_ad = wls[0].num_adapters
    tables, ys, vs = [], [], []
    for q, wl in enumerate(wls):
        A = [to_dev(a, dtype, DEV) for a in wl.A]
        B = [to_dev(b, dtype, DEV) for b in wl.B]
        ranks = list(wl.ranks)
        scales = wl.scales.tolist()
        t = lb.AdapterTable(A, B, scales)
        if bad is not None and bad[0] == q:
            # an invalid entry: rank 0 (bytes 16..19 of the 24-byte record {A, B, rank, scale})
            t.table[24 * bad[1] + 16:24 * bad[1] + 20] = 0
        tables.append(t)
        ys.append(to_dev(wl.y0, dtype, DEV))
        rm = max(int(r) for w in wls for r in w.ranks)
        vs.append(torch.zeros((wl.T, (rm + 7) // 8 * 8), dtype=torch.float32, device=DEV) if with_v[q] else None)
    seg = lb.lora_segments_build(ids, n_ad)
    r_max = max(t.r_max for t in tables)
    if multi:
        lb.lora_forward_multi(x, [(tables[q], ys[q], vs[q]) for q in range(len(wls))], seg, r_max=r_max)
    else:
        for q in range(len(wls)):
            lb.lora_forward(x, tables[q], seg, ys[q], v=vs[q], r_max=r_max)
    torch.cuda.synchronize()
    return ys, vs, seg


CASES = {
    # name: (T, adapters, d_in, d_outs, rank sets per slice, id kind)
    "qkv_decode": (200, 12, 512, (512, 128, 128), ((16,) * 12, (16,) * 12, (16,) * 12), "uniform"),
    "qkv_mixed_ranks": (300, 6, 256, (384, 64, 64), ((8, 16, 32, 8, 16, 32), (8,) * 6, (32, 16, 8, 32, 16, 8)), "long"),
    "gate_up": (150, 5, 512, (1024, 1024), ((16, 64, 8, 48, 24), (16, 64, 8, 48, 24)), "uniform"),
    # ranks <= 16, few rows per adapter: the 16-row-tile decode kernel (bf16), ragged ranks and d_out
    "qkv_decode_ragged": (180, 10, 264, (520, 136, 72), ((16, 5, 12, 1, 8, 16, 3, 9, 16, 7), (8,) * 10,
                                                         (1, 16, 4, 12, 16, 8, 2, 16, 5, 10)), "uniform"),
    "gate_up_decode": (96, 24, 1024, (1032, 1032), ((16, 8) * 12, (8, 16) * 12), "uniform"),
}


def _ids(kind, T, A, rng):
    if kind == "long":  # runs of one adapter (prefill-like tiles) plus rows without an adapter
        return np.sort(rng.integers(-1, A, size=T)).astype(np.int32)
    return rng.integers(-1, A, size=T).astype(np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_multi_slice_matches_oracle_and_single_slices(case, dtype):
    T, A, d_in, d_outs, rank_sets, kind = CASES[case]
    ids = _ids(kind, T, A, np.random.default_rng(3))
    wls = _slices(ids, d_in, d_outs, rank_sets, dtype, seed=5)
    ys, vs, seg = _run(wls, dtype, with_v=True)
    assert seg.err.item() == 0
    x0 = oracle.to_f64(wls[0].x, dtype)
    for q, wl in enumerate(wls):
        ref = oracle.from_workload(wl)
        y_ref, v_ref = oracle.forward(x0, ref["ids"], ref["ranks"], ref["scales"], ref["A"], ref["B"], ref["y0"])
        assert rel_err(ys[q], y_ref) <= TOL[dtype], (case, q)
        y_d, _ = oracle.forward(x0, ref["ids"], ref["ranks"], ref["scales"], ref["A"], ref["B"],
                                np.zeros_like(ref["y0"]))
        got_d = ys[q].double().cpu().numpy() - ref["y0"]
        assert np.max(np.abs(got_d - y_d)) <= TOL[dtype] * max(np.max(np.abs(y_d)), 1e-30) + \
            (np.max(np.abs(ref["y0"])) * 2.0 ** -8 if dtype == "bf16" else 0.0), (case, q)
        rows = ids >= 0
        for t in np.nonzero(rows)[0][:64]:
            r = int(wl.ranks[ids[t]])
            np.testing.assert_allclose(vs[q][t, :r].double().cpu().numpy(), v_ref[t, :r], rtol=1e-4,
                                       atol=1e-4 * max(np.max(np.abs(v_ref)), 1e-30))
    ys1, vs1, _ = _run(wls, dtype, with_v=True, multi=False)
    for q in range(len(wls)):
        assert torch.equal(ys[q], ys1[q]), (case, q)
        assert torch.equal(vs[q], vs1[q]), (case, q)
    ys0, _, _ = _run(wls, dtype, with_v=False)
    ys01, _, _ = _run(wls, dtype, with_v=False, multi=False)
    for q in range(len(wls)):
        assert torch.equal(ys0[q], ys01[q]), (case, q)


@pytest.mark.parametrize("case,with_v", [("gate_up", [True, False]), ("gate_up", [False, True]),
                                         ("qkv_decode_ragged", [True, False, True]),
                                         ("qkv_mixed_ranks", [False, True, False])])
def test_multi_slice_some_slices_with_v(case, with_v):
    """gate_up is a decode batch (150 rows, 5 adapters) with ranks to 64: the
    slices given v run the split kernels, the others one 64-row-tile launch;
    qkv_decode_ragged (ranks <= 16) runs every slice in the 16-row-tile launch
    and qkv_mixed_ranks (long row groups, ranks to 32) in the 64-row-tile one.
    Each slice equals lora_forward of that slice alone with the same
    arguments, bit for bit, and the oracle."""
    T, A, d_in, d_outs, rank_sets, kind = CASES[case]
    ids = _ids(kind, T, A, np.random.default_rng(6))
    wls = _slices(ids, d_in, d_outs, rank_sets, "bf16", seed=11)
    ys, vs, seg = _run(wls, "bf16", with_v=with_v)
    ys1, vs1, _ = _run(wls, "bf16", with_v=with_v, multi=False)
    assert seg.err.item() == 0
    x0 = oracle.to_f64(wls[0].x, "bf16")
    for q, wl in enumerate(wls):
        assert torch.equal(ys[q], ys1[q]), q
        if with_v[q]:
            assert torch.equal(vs[q], vs1[q]), q
        ref = oracle.from_workload(wl)
        y_ref, _ = oracle.forward(x0, ref["ids"], ref["ranks"], ref["scales"], ref["A"], ref["B"], ref["y0"])
        assert rel_err(ys[q], y_ref) <= TOL["bf16"], q


def test_multi_slice_bad_entry_skips_only_its_slice():
    T, A, d_in, d_outs, rank_sets, kind = CASES["qkv_decode"]
    ids = _ids(kind, T, A, np.random.default_rng(4))
    wls = _slices(ids, d_in, d_outs, rank_sets, "bf16", seed=9)
    ys, _, seg = _run(wls, "bf16", with_v=False, bad=(1, 3))
    ys1, _, _ = _run(wls, "bf16", with_v=False, multi=False)
    # a decode batch of rank-16 adapters (200 rows, 12 adapters): the 16-row-tile
    # kernel counts the bad entry once per 16-row tile of its adapter
    tiles_of_3 = (int((ids == 3).sum()) + 15) // 16
    assert seg.err.item() == tiles_of_3
    assert torch.equal(ys[0], ys1[0]) and torch.equal(ys[2], ys1[2])
    y0 = to_dev(wls[1].y0, "bf16", DEV)
    rows3 = torch.from_numpy(ids == 3).to(DEV)
    assert torch.equal(ys[1][rows3], y0[rows3])            # adapter 3's rows untouched in slice 1
    assert torch.equal(ys[1][~rows3], ys1[1][~rows3])      # every other row as computed alone
