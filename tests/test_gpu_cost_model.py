"""The cost model's calibration runs the library's calls on the GPU and fits them."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from expand_token_adapter_amd import cost_model as cm


def test_calibrate_and_fit_small_set():
    shapes = [(T, 1024, 2048, ranks, dist) for T in (64, 512, 2048)
              for ranks, dist in (((16,) * 8, "uniform"), ((8, 16, 32, 64), "zipf"), ((16,), "one"))]
    samples = cm.calibrate(shapes, reps=3)
    assert len(samples) == len(shapes) * len(cm.OPS)
    assert all(s["seconds"] > 0 and np.isfinite(s["seconds"]) for s in samples)
    model = cm.fit_samples(samples)
    for op in cm.OPS:
        assert np.all(model.coef[op] >= 0)
        assert model.predict(op, [0, 1, 1], [8, 16], 1024, 2048) > 0
