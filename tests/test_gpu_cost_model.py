"""The cost model on the GPU: calibrate on one set of batch shapes, predict a
disjoint held-out set, and hold the split forward and the backward to a
median |relative error| of at most 15 % (DeltaServe section 3.3 prices a
batch with a model of this kind before dispatching it); the two-pass
backward (ranks above 16, or dY no wider than 2 d_in) to 20 %: its time is
not monotone in the row count on these shapes (e.g. 16 adapters of ranks
8-64, 2048 -> 4096: about 97 us at 512 rows and 88 us at 2048 rows), which
no model over these features follows more closely.

The shapes cover the routes of each entry point: decode-sized batches
(at most 32 rows per adapter) take the 16-row-tile split forward (its own
model entry, 'forward_decode'), larger ones the 64-row one ('forward'); rank-16 tables with d_out >= 2 d_in take the streaming backward
(its own model entry, 'backward_stream'), the others the two-pass one;
lora_forward without v runs the 16-row-tile decode kernel on rank-16 decode
batches ('forward_fused_decode') and the 64-row-tile kernel elsewhere
('forward_fused').  Those two and the segment build are fitted and reported
but not held to the bound (their time is set by latency chains; see the fit
summary under profiles/)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from expand_token_adapter_amd import cost_model as cm

_FAMILIES = (((16,) * 32, "uniform"), ((8, 16, 32, 64) * 4, "uniform"), ((16,), "one"),
             ((8, 16, 32, 64, 128) * 16, "zipf"))
TRAIN = [(T, d_in, d_out, ranks, dist) for d_in, d_out in ((2048, 2048), (1024, 4096), (2048, 8192), (4096, 4096))
         for T in (128, 1024, 4096) for ranks, dist in _FAMILIES]
HELD = [(T, d_in, d_out, ranks, dist) for d_in, d_out in ((2048, 4096), (4096, 8192))
        for T in (512, 2048) for ranks, dist in _FAMILIES]
BOUND = {"forward": 0.15, "forward_decode": 0.20, "backward_stream": 0.15, "backward": 0.20}


def _key(s):
    sh = s["shape"]
    return (sh["T"], sh["d_in"], sh["d_out"], sh["adapters"], sh["dist"])


def test_calibrate_fit_and_held_out_accuracy():
    samples = cm.calibrate(TRAIN + HELD, reps=5)
    assert len(samples) == (len(TRAIN) + len(HELD)) * len(cm.OPS)
    assert all(s["seconds"] > 0 and np.isfinite(s["seconds"]) for s in samples)
    held_keys = {(T, di, do, len(r), dist) for T, di, do, r, dist in HELD}
    train = [s for s in samples if _key(s) not in held_keys]
    held = [s for s in samples if _key(s) in held_keys]
    model = cm.fit_samples(train)
    assert set(model.coef) >= {"segments", "forward", "forward_decode", "forward_fused", "forward_fused_decode",
                               "backward", "backward_stream"}
    for op in model.coef:
        assert np.all(model.coef[op] >= 0)
    errs = cm.relative_errors(model, held)
    med = {op: float(np.median(np.abs(e))) for op, e in errs.items()}
    print({op: (round(med[op], 3), round(float(np.max(np.abs(errs[op]))), 3)) for op in errs}, flush=True)
    assert set(errs) >= {"forward", "forward_decode", "backward", "backward_stream"}
    for op, bound in BOUND.items():
        assert med[op] <= bound, (op, med[op], errs[op].round(3).tolist())
