"""Seeded input generator: determinism and the shapes of the five workloads."""
import numpy as np
import pytest

import workloads


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 0.0], dtype=np.float32)
    bits = workloads.fp32_to_bf16_bits(vals)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    assert back[1] == 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: rounds to even (1 + 2^-6)
    assert back[2] == np.float32(1 + 2 ** -6)
    assert back[0] == 1.0 and back[3] == -2.5 and back[5] == 0.0
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_same_seed_same_bytes():
    a = workloads.config(2, seed=0).manifest()
    b = workloads.config(2, seed=0).manifest()
    c = workloads.config(2, seed=1).manifest()
    assert a == b
    assert a["x"] != c["x"]


@pytest.mark.parametrize("idx", [1, 2, 4])
def test_config_shapes_small(idx):
    wl = workloads.config(idx)
    exp = {1: (64, 256, 256, 4, "f32", 16), 2: (256, 4096, 4096, 64, "bf16", 0),
           4: (4096, 5120, 5120, 1, "bf16", 4096)}[idx]
    T, d_in, d_out, nA, dt, nft = exp
    assert wl.T == T and wl.d_in == d_in and wl.d_out == d_out
    assert wl.num_adapters == nA and wl.dtype == dt and wl.ft_count == nft
    assert wl.x.shape == (T, d_in) and wl.y0.shape == (T, d_out)
    for a in range(nA):
        assert wl.A[a].shape == (wl.ranks[a], d_in)
        assert wl.B[a].shape == (d_out, wl.ranks[a])
    assert np.all(wl.scales == 2.0)
    if idx == 1:
        assert wl.ids.tolist() == sum([[a] * 16 for a in range(4)], [])
        assert np.all(wl.ranks == 8)
    if idx == 2:
        assert wl.ids.min() >= 0 and wl.ids.max() < 64 and np.all(wl.ranks == 16)


def test_config3_structure():
    wl = workloads.config(3)
    T = wl.T
    assert wl.d_in == 4096 and wl.d_out == 14336
    assert 128 + 8 * 128 + 2048 <= T <= 128 + 8 * 1024 + 2048
    assert np.all(wl.ids[:128] >= 1) and np.all(wl.ids[:128] <= 31)
    assert np.all(wl.ids[T - 2048:] == 0) and wl.ft_start == T - 2048 and wl.ft_count == 2048
    assert wl.dy.shape == (2048, 14336)
    assert set(wl.ranks.tolist()) <= {8, 16, 32, 64} and wl.num_adapters == 32
    mid = wl.ids[128:T - 2048]
    # 8 prefill segments, each one adapter id in 1..31
    assert np.count_nonzero(np.diff(mid)) <= 7 and mid.min() >= 1


def test_config5_zipf():
    wl = workloads.config(5)
    assert wl.T == 2048 and wl.num_adapters == 320 and wl.d_in == 8192
    assert set(wl.ranks.tolist()) <= {8, 16, 32, 64, 128}
    counts = np.bincount(wl.ids, minlength=320)
    # the most popular id carries about a fifth of the rows; ~250 distinct ids
    assert 300 <= counts[0] <= 520
    assert 200 <= np.count_nonzero(counts) <= 300
