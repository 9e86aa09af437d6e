"""lora_shrink_noalloc (static device scratch, no allocation) against
lora_shrink (caller's workspace) through the C ABI: bit-identical v on two
calls in a row, the second with a smaller batch, and sizes beyond the static
scratch rejected on the host."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import expand_token_adapter_amd as lb
    from expand_token_adapter_amd import _abi
    from gpu_helpers import to_dev


def _case(wl, dev):
    A = [to_dev(a, wl.dtype, dev) for a in wl.A]
    B = [to_dev(b, wl.dtype, dev) for b in wl.B]
    table = lb.AdapterTable(A, B, wl.scales.tolist())
    x = to_dev(wl.x, wl.dtype, dev)
    seg = lb.lora_segments_build(torch.from_numpy(wl.ids).to(dev), wl.num_adapters)
    return table, x, seg


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_shrink_equals_lora_shrink_twice(dtype):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(31)
    big = workloads.custom(rng.integers(-1, 6, size=3000).astype(np.int32), [8, 24, 5, 64, 128, 16], 1032, 40,
                           dtype, seed=31, name="noalloc-big")
    small = workloads.custom(rng.integers(0, 3, size=77).astype(np.int32), [16, 40, 8], 264, 24, dtype, seed=32,
                             name="noalloc-small")
    for wl in (big, small):  # two calls in a row, the second smaller
        table, x, seg = _case(wl, dev)
        width = (table.r_max + 7) // 8 * 8
        v_ref = torch.full((wl.T, width), -3.0, dtype=torch.float32, device=dev)
        v_na = v_ref.clone()
        lb.lora_shrink(x, table, seg, v=v_ref)
        lb.lora_shrink_noalloc(x, table, seg, v_na)
        torch.cuda.synchronize()
        assert int(seg.err.item()) == 0
        assert torch.equal(v_na, v_ref), wl.name


def test_noalloc_rejects_sizes_beyond_the_scratch():
    dev = torch.device("cuda:0")
    lib = _abi.load()
    T, d_in, r_max = 1 << 16, 8192, 128  # 16 slices x 65536 rows x 128 ranks x 4 B = 512 MiB of partials
    assert lib.lora_shrink_workspace_bytes(_abi.LORA_BF16, T, d_in, r_max) > _abi.LORA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((8, d_in), dtype=torch.bfloat16, device=dev)  # never read: rejected first
    v = torch.zeros((8, r_max), dtype=torch.float32, device=dev)
    seg = lb.Segments(T, 4, dev)
    table = lb.AdapterTable([torch.zeros((r_max, d_in), dtype=torch.bfloat16, device=dev)] * 4,
                            [torch.zeros((16, r_max), dtype=torch.bfloat16, device=dev)] * 4, [1.0] * 4)
    st = lib.lora_shrink_noalloc(_abi.LORA_BF16, x.data_ptr(), d_in, T, d_in, table.ptr, 4, r_max, seg.c,
                                 v.data_ptr(), r_max, None)
    assert st == _abi.LORA_ERR_TOO_LARGE
    assert "static scratch" in _abi.status_string(st)
