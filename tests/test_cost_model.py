"""Host tests of the cost model: its features against a brute-force count, and
its fit against coefficients it must recover."""
import numpy as np
import pytest

from expand_token_adapter_amd import cost_model as cm


def test_features_by_brute_force():
    ids = [0, 2, 2, -1, 5, 2, 0]      # 5 is out of range: no adapter
    ranks = [4, 8, 16]
    d_in, d_out = 24, 40
    f = cm.features(ids, ranks, d_in, d_out)
    rows = [i for i in ids if 0 <= i < len(ranks)]
    used = sorted(set(rows))
    tiles = sum(-(-rows.count(a) // 16) for a in used)
    groups = sum(-(-ranks[i] // 16) for i in rows) * (d_in + d_out)
    want = [1.0, len(ids), len(ids) * (d_in + d_out), sum(ranks[a] for a in used) * (d_in + d_out),
            sum(ranks[i] for i in rows), len(used), tiles, groups]
    assert f.tolist() == want
    assert cm.features([], ranks, d_in, d_out).tolist() == [1.0] + [0.0] * 7
    # tiles: 17 rows of one adapter and 16 of another are 2 + 1 tiles of 16 rows
    assert cm.features([0] * 17 + [1] * 16, [4, 4], 8, 8)[6] == 3.0
    # rank groups: ranks 16 and 17 are one and two groups of 16
    assert cm.features([0, 1], [16, 17], 8, 8)[7] == 3 * 16


def _design(rng, n):
    # feature columns with the magnitudes of real calls
    T = rng.integers(16, 8192, size=n)
    d = rng.choice([4096, 8192, 18432], size=n)
    return np.stack([np.ones(n), T, T * d, rng.integers(16, 4096, size=n) * d, T * rng.integers(8, 64, size=n),
                     rng.integers(1, 320, size=n), T // 16 + rng.integers(1, 320, size=n),
                     T * rng.integers(1, 8, size=n) * d], axis=1).astype(np.float64)


def test_fit_recovers_exact_coefficients():
    rng = np.random.default_rng(0)
    X = _design(rng, 60)
    c = np.array([8e-6, 1e-10, 2.5e-13, 2.6e-13, 1e-11, 3e-8, 2e-9, 5e-14])
    got = cm.fit(X, X @ c)
    np.testing.assert_allclose(got, c, rtol=1e-5)


def test_fit_with_noise_and_a_zero_coefficient():
    rng = np.random.default_rng(1)
    X = _design(rng, 200)
    c = np.array([5e-6, 0.0, 3e-13, 0.0, 2e-11, 1e-8, 1e-9, 0.0])
    t = X @ c * (1.0 + 0.01 * rng.standard_normal(200))
    got = cm.fit(X, t)
    assert np.all(got >= 0.0)
    np.testing.assert_allclose(got[[0, 2, 4]], c[[0, 2, 4]], rtol=0.1)
    assert got[3] * X[:, 3].max() < 0.05 * t.min()   # the absent term stays negligible
    rel = X @ got / t - 1.0
    assert np.median(np.abs(rel)) < 0.02


def test_fit_needs_enough_samples():
    with pytest.raises(ValueError):
        cm.fit(np.ones((3, 8)), np.ones(3))


def test_model_json_round_trip_and_predict():
    m = cm.CostModel({"forward": [1e-6, 1e-10, 1e-12, 2e-12, 3e-11, 4e-9, 5e-9, 1e-13]})
    m2 = cm.CostModel.from_json(m.to_json())
    ids, ranks = [0, 1, 1], [8, 16]
    assert m2.predict("forward", ids, ranks, 64, 32) == pytest.approx(m.predict("forward", ids, ranks, 64, 32))
    f = cm.features(ids, ranks, 64, 32)
    assert m.predict("forward", ids, ranks, 64, 32) == pytest.approx(float(f @ m.coef["forward"]))


def test_route_follows_the_library_routes():
    r16, mixed = [16] * 64, [8, 16, 32, 64] * 8
    # backward: streaming at r_max <= 16 and d_out >= 2 d_in
    assert cm.route("backward", r16, 4096, 14336) == "backward_stream"
    assert cm.route("backward", r16, 4096, 4096) == "backward"
    assert cm.route("backward", mixed, 4096, 14336) == "backward"
    assert cm.route("backward", mixed, 4096, 14336, r_max=16) == "backward_stream"
    # lora_forward: decode batches (T <= 32 per adapter of the table) at r_max <= 16
    # take the 16-row-tile kernel, with or without v
    for with_v in (False, True):
        assert cm.route("forward_fused", r16, 4096, 4096, T=2048, with_v=with_v) == "forward_fused_decode"
        assert cm.route("forward_fused", r16, 4096, 4096, T=2049, with_v=with_v) == \
            ("forward" if with_v else "forward_fused")
    # with v: the split kernels on decode batches of any rank and at r_max <= 16
    assert cm.route("forward_fused", mixed, 4096, 4096, T=1024, with_v=True) == "forward_decode"
    assert cm.route("forward_fused", mixed, 4096, 4096, T=1024) == "forward_fused"
    assert cm.route("forward_fused", mixed, 4096, 4096, T=1025, with_v=True) == "forward_fused"
    assert cm.route("forward_fused", [16], 4096, 4096, T=4096, with_v=True) == "forward"
    assert cm.route("forward_fused", [16], 4096, 4096, T=4096) == "forward_fused"
    # the split forward: its decode route (16-row tiles) has its own entry
    assert cm.route("forward", mixed, 4096, 4096, T=1) == "forward_decode"
    assert cm.route("forward", mixed, 4096, 4096, T=1024) == "forward_decode"
    assert cm.route("forward", mixed, 4096, 4096, T=1025) == "forward"
    assert cm.route("forward", mixed, 4096, 4096) == "forward"  # T unknown: not a decode batch
    assert cm.route("segments", r16, 4096, 4096, T=1) == "segments"


def test_predict_uses_the_routed_entry():
    c = lambda k: [k * 1e-6] + [0.0] * 7
    m = cm.CostModel({"forward": c(1), "forward_fused": c(2), "forward_fused_decode": c(3), "forward_decode": c(4)})
    ids = [0, 1, 1]
    assert m.predict("forward_fused", ids, [16, 16], 64, 32) == pytest.approx(3e-6)
    assert m.predict("forward_fused", ids, [64, 64], 64, 32) == pytest.approx(2e-6)
    assert m.predict("forward_fused", ids, [64, 64], 64, 32, with_v=True) == pytest.approx(4e-6)
    assert m.predict("forward", ids, [64, 64], 64, 32) == pytest.approx(4e-6)
    assert m.predict("forward", list(range(2)) * 40, [64, 64], 64, 32) == pytest.approx(1e-6)
