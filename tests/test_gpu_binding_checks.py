"""The Python binding rejects arguments that do not describe one batch, on the
host, before anything is enqueued (ValueError): the C side would otherwise
size offsets and strides from the wrong T, adapter count, dtype or rank and
the kernels would index outside the buffers."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import expand_token_adapter_amd as lb

DEV = "cuda:0"


def _table(A=3, d_in=64, d_out=96, r=8, dtype=torch.bfloat16):
    As = [torch.randn(r, d_in, device=DEV).to(dtype) for _ in range(A)]
    Bs = [torch.randn(d_out, r, device=DEV).to(dtype) for _ in range(A)]
    return lb.AdapterTable(As, Bs, [1.0] * A)


def _ids(T, A):
    return torch.from_numpy(np.arange(T, dtype=np.int32) % A).to(DEV)


def test_adapter_table_rejects_mixed_shapes():
    A1 = torch.zeros(8, 64, device=DEV, dtype=torch.bfloat16)
    A2 = torch.zeros(8, 72, device=DEV, dtype=torch.bfloat16)
    B = torch.zeros(96, 8, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lb.AdapterTable([A1, A2], [B, B], [1.0, 1.0])
    with pytest.raises(ValueError):
        lb.AdapterTable([A1, A1], [B, torch.zeros(104, 8, device=DEV, dtype=torch.bfloat16)], [1.0, 1.0])


def test_forward_calls_reject_mismatched_batches():
    t = _table()
    T = 40
    x = torch.randn(T, 64, device=DEV).bfloat16()
    y = torch.randn(T, 96, device=DEV).bfloat16()
    seg = lb.lora_segments_build(_ids(T, 3), 3)
    seg_other_T = lb.lora_segments_build(_ids(T + 8, 3), 3)
    seg_other_A = lb.lora_segments_build(_ids(T, 2), 2)
    for s in (seg_other_T, seg_other_A):
        with pytest.raises(ValueError):
            lb.lora_shrink(x, t, s)
        with pytest.raises(ValueError):
            lb.lora_forward(x, t, s, y)
    with pytest.raises(ValueError):  # x columns != d_in
        lb.lora_shrink(torch.randn(T, 72, device=DEV).bfloat16(), t, seg)
    with pytest.raises(ValueError):  # x dtype != the adapters'
        lb.lora_shrink(x.float(), t, seg)
    v = lb.lora_shrink(x, t, seg)
    with pytest.raises(ValueError):  # y columns != d_out
        lb.lora_expand_add(v, t, seg, torch.randn(T, 104, device=DEV).bfloat16())
    with pytest.raises(ValueError):  # y dtype
        lb.lora_expand_add(v, t, seg, y.float())
    with pytest.raises(ValueError):  # v not fp32
        lb.lora_expand_add(v.bfloat16(), t, seg, y)
    with pytest.raises(ValueError):  # v narrower than round_up(r_max, 8)
        lb.lora_expand_add(v[:, :4], t, seg, y)
    with pytest.raises(ValueError):  # v rows != T
        lb.lora_shrink(x, t, seg, v=torch.zeros(T - 1, 8, device=DEV))
    with pytest.raises(ValueError):  # a slice whose table has another d_in
        lb.lora_forward_multi(x, [(t, y), (_table(d_in=72), y)], seg)
    torch.cuda.synchronize()


def test_backward_rejects_mismatched_batches():
    t = _table()
    T = 24
    x = torch.randn(T, 64, device=DEV).bfloat16()
    dy = torch.randn(T, 96, device=DEV).bfloat16()
    seg = lb.lora_segments_build(_ids(T, 3), 3)
    good = lb.GradTable([torch.zeros(8, 64, device=DEV) for _ in range(3)],
                        [torch.zeros(96, 8, device=DEV) for _ in range(3)])
    wrong = lb.GradTable([torch.zeros(8, 64, device=DEV) for _ in range(3)],
                         [torch.zeros(96, 4, device=DEV) for _ in range(3)])
    with pytest.raises(ValueError):
        lb.lora_backward(x, dy, t, wrong, seg)
    with pytest.raises(ValueError):  # dy columns != d_out
        lb.lora_backward(x, torch.randn(T, 104, device=DEV).bfloat16(), t, good, seg)
    with pytest.raises(ValueError):  # dy dtype
        lb.lora_backward(x, dy.float(), t, good, seg)
    with pytest.raises(ValueError):  # segments of another row count
        lb.lora_backward(x, dy, t, good, lb.lora_segments_build(_ids(T + 1, 3), 3))
    with pytest.raises(ValueError):  # saved v of another row count
        lb.lora_backward(x, dy, t, good, seg, v_saved=torch.zeros(T + 1, 8, device=DEV))
    grant = torch.ones(1, dtype=torch.int32)  # host memory that is not pinned
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        lb.lora_backward_preemptible(x, dy, t, good, seg, grant, status)
    lb.lora_backward(x, dy, t, good, seg)  # the consistent call runs
    torch.cuda.synchronize()
    assert int(seg.err.item()) == 0
