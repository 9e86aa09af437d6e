"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to something independent: a hand-worked example,
a closed form, an explicit dense matrix, a numpy library routine, a finite
difference, an adjoint identity, or a brute-force / library sort.  Shapes use
d_in != d_out and ranks > 1 so that a transposed operand, a dropped scale, a
wrong sign or a wrong index fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, T=9, d_in=5, d_out=7, ranks=(1, 2, 3), scales=(2.0, 0.5, -1.25), with_none=True):
    rng = np.random.default_rng(seed)
    A = [rng.standard_normal((r, d_in)) for r in ranks]
    B = [rng.standard_normal((d_out, r)) for r in ranks]
    x = rng.standard_normal((T, d_in))
    y0 = rng.standard_normal((T, d_out))
    lo = -1 if with_none else 0
    ids = rng.integers(lo, len(ranks), size=T).astype(np.int32)
    return x, ids, np.array(ranks, np.int32), np.array(scales, np.float64), A, B, y0


# ----------------------------------------------------------------- hand-worked

def test_golden_handworked_forward_backward_segments():
    with open(os.path.join(GOLDEN, "handworked_lora.json")) as f:
        gd = json.load(f)
    ad = gd["adapters"]
    A = [np.array(a["A"], float) for a in ad]
    B = [np.array(a["B"], float) for a in ad]
    ranks = np.array([a["rank"] for a in ad], np.int32)
    scales = np.array([a["scale"] for a in ad], float)
    fw = gd["forward"]
    y, v = oracle.forward(np.array(fw["x"], float), np.array(fw["ids"], np.int32), ranks, scales,
                          A, B, np.array(fw["y0"], float))
    np.testing.assert_array_equal(y, np.array(fw["y"], float))
    np.testing.assert_array_equal(v, np.array(fw["v"], float))
    bw = gd["backward"]
    dx, dA, dB, g, _ = oracle.backward(np.array(bw["x"], float), np.array(bw["dy"], float),
                                        np.array(bw["ids"], np.int32), ranks, scales, A, B)
    np.testing.assert_array_equal(dx, np.array(bw["dx"], float))
    np.testing.assert_array_equal(dA[0], np.array(bw["dA"], float))
    np.testing.assert_array_equal(dB[0], np.array(bw["dB"], float))
    np.testing.assert_array_equal(g[:, :2], np.array(bw["g"], float))
    assert not dA[1].any() and not dB[1].any()
    for sg in gd["segments"]:
        counts, offsets, perm, err = oracle.segments(np.array(sg["ids"], np.int32), sg["num_adapters"])
        assert counts.tolist() == sg["counts"]
        assert offsets.tolist() == sg["offsets"]
        assert perm.tolist() == sg["perm"]
        assert err == sg["err"]


# --------------------------------------------------------------------- forward

def test_b_zero_gives_base_output_exactly():
    x, ids, ranks, scales, A, B, y0 = _rand_case(1)
    Bz = [np.zeros_like(b) for b in B]
    y, _ = oracle.forward(x, ids, ranks, scales, A, Bz, y0)
    assert np.array_equal(y, y0)


def test_linear_in_scale():
    x, ids, ranks, scales, A, B, y0 = _rand_case(2)
    y0s, _ = oracle.forward(x, ids, ranks, np.zeros_like(scales), A, B, y0)
    assert np.array_equal(y0s, y0)
    y1, _ = oracle.forward(x, ids, ranks, scales, A, B, y0)
    y2, _ = oracle.forward(x, ids, ranks, 2 * scales, A, B, y0)
    np.testing.assert_allclose(y2 - y0, 2 * (y1 - y0), rtol=1e-12, atol=1e-13)
    # the delta of every row with an adapter is nonzero, so the scale is really used
    assert np.all(np.abs(y1 - y0)[ids >= 0].max(axis=1) > 0)


def test_dense_effective_weight_agreement():
    """y_t = (W0 + s_a B_a A_a) x_t with the dense effective weight formed first."""
    x, ids, ranks, scales, A, B, _ = _rand_case(3, T=11)
    rng = np.random.default_rng(33)
    W0 = rng.standard_normal((7, 5))
    y0 = x @ W0.T
    y, _ = oracle.forward(x, ids, ranks, scales, A, B, y0)
    for t in range(x.shape[0]):
        a = ids[t]
        W = W0 if a < 0 else W0 + scales[a] * (B[a] @ A[a])
        np.testing.assert_allclose(y[t], W @ x[t], rtol=1e-12, atol=1e-12)


def test_single_adapter_matches_numpy_matmul():
    rng = np.random.default_rng(4)
    T, d_in, d_out, r, s = 37, 24, 40, 6, 1.75
    A = rng.standard_normal((r, d_in))
    B = rng.standard_normal((d_out, r))
    x = rng.standard_normal((T, d_in))
    y0 = rng.standard_normal((T, d_out))
    y, v = oracle.forward(x, np.zeros(T, np.int32), np.array([r], np.int32), np.array([s]), [A], [B], y0)
    np.testing.assert_allclose(y, y0 + s * (x @ A.T @ B.T), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v[:, :r], x @ A.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("i,j", [(0, 0), (3, 5), (4, 1)])
def test_rank1_unit_vectors_closed_form(i, j):
    """A = e_i^T, B = e_j gives delta y_j = s x_i and no other change."""
    rng = np.random.default_rng(5)
    T, d_in, d_out, s = 6, 5, 7, 3.0
    A = np.zeros((1, d_in)); A[0, i] = 1.0
    B = np.zeros((d_out, 1)); B[j, 0] = 1.0
    x = rng.standard_normal((T, d_in))
    y0 = rng.standard_normal((T, d_out))
    y, _ = oracle.forward(x, np.zeros(T, np.int32), np.array([1], np.int32), np.array([s]), [A], [B], y0)
    expect = y0.copy()
    expect[:, j] += s * x[:, i]
    np.testing.assert_array_equal(y, expect)


def test_row_permutation_equivariance():
    x, ids, ranks, scales, A, B, y0 = _rand_case(6, T=13)
    p = np.random.default_rng(66).permutation(13)
    y, v = oracle.forward(x, ids, ranks, scales, A, B, y0)
    yp, vp = oracle.forward(x[p], ids[p], ranks, scales, A, B, y0[p])
    assert np.array_equal(yp, y[p])
    assert np.array_equal(vp, v[p])


def test_rows_without_adapter_and_bad_ids_unchanged():
    x, ids, ranks, scales, A, B, y0 = _rand_case(7, T=10)
    ids = ids.copy()
    ids[0], ids[1], ids[2] = -1, 3, -7
    y, _ = oracle.forward(x, ids, ranks, scales, A, B, y0)
    assert np.array_equal(y[:3], y0[:3])
    _, _, _, err = oracle.segments(ids, 3)
    assert err == 2


# -------------------------------------------------------------------- backward

def _loss(x, dy, ids, ranks, scales, A, B):
    y, _ = oracle.forward(x, ids, ranks, scales, A, B, np.zeros((x.shape[0], dy.shape[1])))
    return float(np.sum(dy * y))


def test_finite_differences_of_inner_product_loss():
    """L = sum_t <dy_t, y_t> is affine in each of A, B, x: central differences are exact."""
    rng = np.random.default_rng(8)
    T, d_in, d_out = 12, 9, 11
    ranks = np.array([3, 2, 4], np.int32)
    scales = np.array([2.0, -0.75, 1.5])
    A = [rng.standard_normal((r, d_in)) for r in ranks]
    B = [rng.standard_normal((d_out, r)) for r in ranks]
    x = rng.standard_normal((T, d_in))
    dy = rng.standard_normal((T, d_out))
    ids = rng.integers(-1, 3, size=T).astype(np.int32)
    dx, dA, dB, _, _ = oracle.backward(x, dy, ids, ranks, scales, A, B)
    h = 1e-3
    for a in range(3):
        for k in range(ranks[a]):
            for i in range(d_in):
                Ap = [m.copy() for m in A]; Am = [m.copy() for m in A]
                Ap[a][k, i] += h; Am[a][k, i] -= h
                fd = (_loss(x, dy, ids, ranks, scales, Ap, B) - _loss(x, dy, ids, ranks, scales, Am, B)) / (2 * h)
                assert abs(fd - dA[a][k, i]) <= 1e-8 * (1 + abs(fd))
        for j in range(d_out):
            for k in range(ranks[a]):
                Bp = [m.copy() for m in B]; Bm = [m.copy() for m in B]
                Bp[a][j, k] += h; Bm[a][j, k] -= h
                fd = (_loss(x, dy, ids, ranks, scales, A, Bp) - _loss(x, dy, ids, ranks, scales, A, Bm)) / (2 * h)
                assert abs(fd - dB[a][j, k]) <= 1e-8 * (1 + abs(fd))
    for t in range(T):
        for i in range(d_in):
            xp = x.copy(); xm = x.copy()
            xp[t, i] += h; xm[t, i] -= h
            fd = (_loss(xp, dy, ids, ranks, scales, A, B) - _loss(xm, dy, ids, ranks, scales, A, B)) / (2 * h)
            assert abs(fd - dx[t, i]) <= 1e-8 * (1 + abs(fd))
    # rows without an adapter get no input gradient
    assert not dx[ids < 0].any()


def test_adjoint_identities():
    """<dy, J d> = <J^T dy, d> for perturbations of x, A and B."""
    rng = np.random.default_rng(9)
    T, d_in, d_out = 15, 10, 6
    ranks = np.array([2, 5], np.int32)
    scales = np.array([1.5, -2.0])
    A = [rng.standard_normal((r, d_in)) for r in ranks]
    B = [rng.standard_normal((d_out, r)) for r in ranks]
    x = rng.standard_normal((T, d_in))
    dy = rng.standard_normal((T, d_out))
    ids = rng.integers(0, 2, size=T).astype(np.int32)
    dx, dA, dB, _, _ = oracle.backward(x, dy, ids, ranks, scales, A, B)
    z = np.zeros((T, d_out))
    # x direction: J dx_dir = s B A dx_dir
    dxd = rng.standard_normal(x.shape)
    Jd, _ = oracle.forward(dxd, ids, ranks, scales, A, B, z)
    assert np.isclose(np.sum(dy * Jd), np.sum(dx * dxd), rtol=1e-12)
    # A direction: y is linear in A, so J dA_dir = forward with A replaced by the direction
    dAd = [rng.standard_normal(m.shape) for m in A]
    Jd, _ = oracle.forward(x, ids, ranks, scales, dAd, B, z)
    assert np.isclose(np.sum(dy * Jd), sum(np.sum(g * d) for g, d in zip(dA, dAd)), rtol=1e-12)
    dBd = [rng.standard_normal(m.shape) for m in B]
    Jd, _ = oracle.forward(x, ids, ranks, scales, A, dBd, z)
    assert np.isclose(np.sum(dy * Jd), sum(np.sum(g * d) for g, d in zip(dB, dBd)), rtol=1e-12)


def test_single_adapter_backward_matches_numpy_closed_form():
    rng = np.random.default_rng(10)
    T, d_in, d_out, r, s = 33, 20, 28, 5, 2.0
    A = rng.standard_normal((r, d_in))
    B = rng.standard_normal((d_out, r))
    X = rng.standard_normal((T, d_in))
    dY = rng.standard_normal((T, d_out))
    dx, dA, dB, g, v = oracle.backward(X, dY, np.zeros(T, np.int32), np.array([r], np.int32),
                                       np.array([s]), [A], [B])
    np.testing.assert_allclose(dA[0], s * (dY @ B).T @ X, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dB[0], s * dY.T @ (X @ A.T), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dx, s * (dY @ B) @ A, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g[:, :r], dY @ B, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v[:, :r], X @ A.T, rtol=1e-12, atol=1e-12)


def test_backward_additive_over_row_sets_and_accumulates():
    rng = np.random.default_rng(11)
    T, d_in, d_out = 20, 8, 12
    ranks = np.array([4, 3], np.int32)
    scales = np.array([2.0, 0.5])
    A = [rng.standard_normal((r, d_in)) for r in ranks]
    B = [rng.standard_normal((d_out, r)) for r in ranks]
    x = rng.standard_normal((T, d_in))
    dy = rng.standard_normal((T, d_out))
    ids = rng.integers(0, 2, size=T).astype(np.int32)
    dx, dA, dB, _, _ = oracle.backward(x, dy, ids, ranks, scales, A, B)
    s1 = slice(0, 9)
    s2 = slice(9, T)
    dx1, dA1, dB1, _, _ = oracle.backward(x[s1], dy[s1], ids[s1], ranks, scales, A, B)
    dx2, dA2, dB2, _, _ = oracle.backward(x[s2], dy[s2], ids[s2], ranks, scales, A, B, dA0=dA1, dB0=dB1)
    for a in range(2):
        np.testing.assert_allclose(dA2[a], dA[a], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dB2[a], dB[a], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.vstack([dx1, dx2]), dx, rtol=1e-12, atol=1e-12)
    # += semantics for dx
    dx0 = rng.standard_normal(dx.shape)
    dxa, _, _, _, _ = oracle.backward(x, dy, ids, ranks, scales, A, B, dx0=dx0)
    np.testing.assert_allclose(dxa, dx0 + dx, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------------- segments

def _segments_by_sort(ids, A):
    valid = [t for t in range(len(ids)) if 0 <= ids[t] < A]
    perm = sorted(valid, key=lambda t: (ids[t], t))
    counts = np.bincount(np.asarray([ids[t] for t in valid], dtype=np.int64), minlength=A)[:A]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    err = sum(1 for t in range(len(ids)) if ids[t] != -1 and not (0 <= ids[t] < A))
    return counts, offsets, perm, err


@pytest.mark.parametrize("kind", ["random", "sorted", "reverse", "same", "none", "zipf", "bad", "empty"])
def test_segments_match_library_sort(kind):
    rng = np.random.default_rng(12)
    A, T = 37, 1000
    if kind == "random":
        ids = rng.integers(-1, A, size=T)
    elif kind == "sorted":
        ids = np.sort(rng.integers(0, A, size=T))
    elif kind == "reverse":
        ids = np.sort(rng.integers(0, A, size=T))[::-1]
    elif kind == "same":
        ids = np.full(T, 5)
    elif kind == "none":
        ids = np.full(T, -1)
    elif kind == "zipf":
        p = np.arange(1, A + 1, dtype=float) ** -1.1
        ids = rng.choice(A, size=T, p=p / p.sum())
    elif kind == "bad":
        ids = rng.integers(-3, A + 3, size=T)
    else:
        ids = np.zeros(0)
    ids = np.asarray(ids, dtype=np.int32)
    counts, offsets, perm, err = oracle.segments(ids, A)
    c2, o2, p2, e2 = _segments_by_sort(ids.tolist(), A)
    assert counts.tolist() == list(c2)
    assert offsets.tolist() == list(o2)
    assert perm.tolist() == p2
    assert err == e2
    # invariants
    assert np.all(np.diff(offsets) >= 0)
    if perm.size:
        assert np.all(np.diff(ids[perm]) >= 0)
        assert len(set(perm.tolist())) == perm.size


# ------------------------------------------------------------- AdamW step
#
# The optimizer step is Adam with decoupled weight decay (AdamW), lr 1e-3 and
# weight decay 0.01 (DeltaServe, section 4.1).  Pins: torch's own AdamW in
# float64 on the CPU (an independent implementation of the same published
# algorithm), the closed form of the first step, pure decay for zero
# gradients, and invariance to the gradient's scale when eps vanishes.

ADAMW_HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_adamw_matches_torch_adamw_fp64_over_several_steps():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    w0 = rng.standard_normal((3, 7)) * 0.02
    grads = [rng.standard_normal((3, 7)) * (0.1 + k) for k in range(5)]
    p = torch.nn.Parameter(torch.tensor(w0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=ADAMW_HP["lr"], betas=(ADAMW_HP["beta1"], ADAMW_HP["beta2"]),
                            eps=ADAMW_HP["eps"], weight_decay=ADAMW_HP["weight_decay"])
    w, m, v = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    for k, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        w, m, v = oracle.adamw(w, g, m, v, step=k, **ADAMW_HP)
        st = opt.state[p]
        np.testing.assert_allclose(w, p.detach().numpy(), rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-18)


def test_adamw_first_step_closed_form():
    # m = v = 0 before step 1: m_hat = g, v_hat = g^2, so
    # w1 = w0 - lr (wd w0 + g / (|g| + eps)).
    rng = np.random.default_rng(12)
    w0 = rng.standard_normal(50)
    g = rng.standard_normal(50) * 3.0
    lr, wd, eps = 2e-3, 0.05, 1e-6
    w, m, v = oracle.adamw(w0, g, np.zeros(50), np.zeros(50), lr=lr, beta1=0.8, beta2=0.99, eps=eps,
                           weight_decay=wd, step=1)
    np.testing.assert_allclose(w, w0 - lr * (wd * w0 + g / (np.abs(g) + eps)), rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(m, 0.2 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.01 * g * g, rtol=1e-14)


def test_adamw_zero_gradient_is_pure_decay():
    rng = np.random.default_rng(13)
    w0 = rng.standard_normal(20)
    w, m, v = w0.copy(), np.zeros(20), np.zeros(20)
    for k in range(1, 6):
        w, m, v = oracle.adamw(w, np.zeros(20), m, v, step=k, **ADAMW_HP)
    decay = 1.0 - ADAMW_HP["lr"] * ADAMW_HP["weight_decay"]
    np.testing.assert_allclose(w, w0 * decay ** 5, rtol=1e-14)
    assert not m.any() and not v.any()


def test_adamw_is_invariant_to_gradient_scale_when_eps_vanishes():
    rng = np.random.default_rng(14)
    w0 = rng.standard_normal(30)
    gs = [rng.standard_normal(30) for _ in range(3)]
    hp = dict(ADAMW_HP, eps=1e-300)
    a = (w0.copy(), np.zeros(30), np.zeros(30))
    b = (w0.copy(), np.zeros(30), np.zeros(30))
    for k, g in enumerate(gs, start=1):
        a = oracle.adamw(a[0], g, a[1], a[2], step=k, **hp)
        b = oracle.adamw(b[0], 1e3 * g, b[1], b[2], step=k, grad_scale=1e-3 * 7.0, **hp)
        # b sees 7 g: Adam's update does not depend on the gradient's scale
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12)
