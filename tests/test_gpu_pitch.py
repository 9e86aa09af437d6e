"""Row pitches larger than the row length (views of wider buffers) on every
compute entry point: the results equal those of contiguous buffers bit for
bit (the work split depends on the shapes, never on the pitches), no element
of an input's padding reaches a result (the padding holds NaN), and no
element of an output's padding is written."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import expand_token_adapter_amd as lb
    from gpu_helpers import to_dev

DEV = "cuda:0"


def _case_decode16():
    # a bf16 decode batch of rank <= 16 adapters (at most 32 rows per adapter):
    # the 16-row-tile shrink and expand and the one-launch decode forward; the
    # fine-tuning rows (rank 16, d_out >= 2 d_in) take the streaming backward
    rng = np.random.default_rng(19)
    ids = np.concatenate([rng.integers(-1, 40, size=150), np.full(48, 7)]).astype(np.int32)
    ranks = [16, 5, 8, 12, 1, 16, 3, 16] * 5
    return workloads.custom(ids, ranks, 136, 520, "bf16", seed=21, ft_start=len(ids) - 48, ft_count=48,
                            name="pitch-decode16")


def _case(dtype):
    # rows without an adapter, ragged runs, ranks that are not multiples of 8;
    # the fine-tuning rows (rank 40) close the batch
    rng = np.random.default_rng(17)
    ids = np.concatenate([rng.integers(-1, 5, size=70), np.full(90, 3), rng.integers(0, 5, size=33),
                          np.full(80, 1)]).astype(np.int32)
    return workloads.custom(ids, [8, 40, 5, 16, 24], 320, 136, dtype, seed=9, ft_start=len(ids) - 80, ft_count=80,
                            name="pitch")


class _Buffers:
    """Contiguous tensors, or views with a wider row pitch whose padding holds NaN."""

    def __init__(self, pitched: bool):
        self.pitched = pitched
        self.padded = []

    def like(self, t: torch.Tensor, pad: int = 24) -> torch.Tensor:
        if not self.pitched:
            return t.clone()
        big = torch.full((t.shape[0], t.shape[1] + pad), float("nan"), dtype=t.dtype, device=t.device)
        big[:, :t.shape[1]] = t
        self.padded.append((big, t.shape[1]))
        return big[:, :t.shape[1]]

    def padding_untouched(self) -> bool:
        return all(bool(torch.isnan(big[:, n:]).all().item()) for big, n in self.padded)


def _run(wl, dtype, pitched):
    dev = torch.device(DEV)
    table = lb.AdapterTable([to_dev(a, dtype, dev) for a in wl.A], [to_dev(b, dtype, dev) for b in wl.B],
                            wl.scales.tolist())
    ids = torch.from_numpy(wl.ids).to(dev)
    s, n, A = wl.ft_start, wl.ft_count, wl.num_adapters
    seg = lb.lora_segments_build(ids, A)
    seg_ft = lb.lora_segments_build(ids[s:s + n].contiguous(), A)
    buf = _Buffers(pitched)
    x = buf.like(to_dev(wl.x, dtype, dev))
    dy = buf.like(to_dev(wl.dy, dtype, dev))
    y0 = to_dev(wl.y0, dtype, dev)
    v0 = torch.zeros((wl.T, (table.r_max + 7) // 8 * 8), dtype=torch.float32, device=dev)
    out = {}

    y, v = buf.like(y0), buf.like(v0, pad=16)
    lb.lora_shrink(x, table, seg, v=v)
    lb.lora_expand_add(v, table, seg, y)
    out["split y"], out["split v"] = y, v

    yf, vf = buf.like(y0), buf.like(v0, pad=8)
    lb.lora_forward(x, table, seg, yf, v=vf)
    out["fused y"], out["fused v"] = yf, vf

    y1, y2, v1 = buf.like(y0), buf.like(y0, pad=8), buf.like(v0, pad=8)
    lb.lora_forward_multi(x, [(table, y1, v1), (table, y2)], seg)
    out["multi y1"], out["multi y2"], out["multi v1"] = y1, y2, v1

    for mode in ("saved v", "recomputed v"):
        dA = [torch.zeros(a.shape, dtype=torch.float32, device=dev) for a in table.A]
        dB = [torch.zeros(b.shape, dtype=torch.float32, device=dev) for b in table.B]
        dx = buf.like(torch.zeros((n, wl.d_in), dtype=y0.dtype, device=dev))
        lb.lora_backward(x[s:s + n], dy, table, lb.GradTable(dA, dB), seg_ft, dx=dx,
                         v_saved=v[s:s + n] if mode == "saved v" else None)
        out[f"dx, {mode}"] = dx
        for a in range(A):
            out[f"dA[{a}], {mode}"], out[f"dB[{a}], {mode}"] = dA[a], dB[a]
    torch.cuda.synchronize()
    assert seg.err.item() == 0 and seg_ft.err.item() == 0
    return {k: t.clone() for k, t in out.items()}, buf


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pitched_views_match_contiguous_buffers_bit_for_bit(dtype):
    wl = _case(dtype)
    want, _ = _run(wl, dtype, pitched=False)
    got, buf = _run(wl, dtype, pitched=True)
    assert buf.padding_untouched()
    assert want["dA[1], saved v"].abs().sum().item() > 0  # the fine-tuning adapter received gradients
    for k in want:
        assert torch.equal(got[k], want[k]), k


def test_pitched_views_on_the_decode_routes_bit_for_bit():
    wl = _case_decode16()
    want, _ = _run(wl, "bf16", pitched=False)
    got, buf = _run(wl, "bf16", pitched=True)
    assert buf.padding_untouched()
    assert want["dA[7], saved v"].abs().sum().item() > 0
    for k in want:
        assert torch.equal(got[k], want[k]), k
