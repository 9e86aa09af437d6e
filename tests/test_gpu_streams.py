"""Two independent steps (segment build, shrink, expand-add, backward) with
their own buffers and workspaces, run concurrently on two streams, give the
same bits as the same steps run one after the other: the library keeps no
state between calls, and every call works on the caller's stream only."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import expand_token_adapter_amd as lb
    from gpu_helpers import to_dev


def _state(seed, dev):
    rng = np.random.default_rng(seed)
    ids = np.concatenate([rng.integers(-1, 6, size=150), np.full(200, 4), rng.integers(0, 6, size=60),
                          np.full(128, 2)]).astype(np.int32)
    wl = workloads.custom(ids, [16, 8, 64, 24, 32, 40], 512, 384, "bf16", seed=seed, ft_start=len(ids) - 128,
                          ft_count=128, name=f"streams-{seed}")
    table = lb.AdapterTable([to_dev(a, "bf16", dev) for a in wl.A], [to_dev(b, "bf16", dev) for b in wl.B],
                            wl.scales.tolist())
    st = {"wl": wl, "table": table, "x": to_dev(wl.x, "bf16", dev), "y0": to_dev(wl.y0, "bf16", dev),
          "dy": to_dev(wl.dy, "bf16", dev), "ids": torch.from_numpy(wl.ids).to(dev)}
    s, n = wl.ft_start, wl.ft_count
    st["ft_ids"] = st["ids"][s:s + n].contiguous()
    st["seg"] = lb.Segments(wl.T, wl.num_adapters, dev)
    st["seg_ft"] = lb.Segments(n, wl.num_adapters, dev)
    st["ws"] = torch.empty(lb.lora_shrink_workspace_bytes(torch.bfloat16, wl.T, wl.d_in, table.r_max),
                           dtype=torch.uint8, device=dev)
    st["bws"] = torch.empty(lb.lora_backward_workspace_bytes(torch.bfloat16, n, wl.d_in, wl.d_out, table.r_max),
                            dtype=torch.uint8, device=dev)
    st["y"] = st["y0"].clone()
    st["v"] = torch.zeros((wl.T, (table.r_max + 7) // 8 * 8), dtype=torch.float32, device=dev)
    st["dx"] = torch.zeros((n, wl.d_in), dtype=torch.bfloat16, device=dev)
    st["dA"] = [torch.zeros(a.shape, dtype=torch.float32, device=dev) for a in table.A]
    st["dB"] = [torch.zeros(b.shape, dtype=torch.float32, device=dev) for b in table.B]
    st["grads"] = lb.GradTable(st["dA"], st["dB"])
    return st


def _reset(st):
    st["y"].copy_(st["y0"])
    st["v"].zero_()
    st["dx"].zero_()
    for t in st["dA"] + st["dB"]:
        t.zero_()


def _step(st):
    wl = st["wl"]
    s, n = wl.ft_start, wl.ft_count
    lb.lora_segments_build_batch([(st["ids"], st["seg"]), (st["ft_ids"], st["seg_ft"])], wl.num_adapters)
    lb.lora_shrink(st["x"], st["table"], st["seg"], v=st["v"], ws=st["ws"])
    lb.lora_expand_add(st["v"], st["table"], st["seg"], st["y"])
    lb.lora_backward(st["x"][s:s + n], st["dy"], st["table"], st["grads"], st["seg_ft"], dx=st["dx"],
                     v_saved=st["v"][s:s + n], ws=st["bws"])


def _results(st):
    return [t.clone() for t in [st["y"], st["v"], st["dx"]] + st["dA"] + st["dB"]]


def test_concurrent_streams_match_sequential_calls():
    dev = torch.device("cuda:0")
    sts = [_state(seed, dev) for seed in (31, 32)]
    for st in sts:
        _reset(st)
        _step(st)
    torch.cuda.synchronize()
    want = [_results(st) for st in sts]
    for st in sts:
        assert st["seg"].err.item() == 0 and st["seg_ft"].err.item() == 0
    streams = [torch.cuda.Stream(device=dev) for _ in sts]  # default priority
    for rep in range(3):
        for st in sts:
            _reset(st)
        torch.cuda.synchronize()
        for st, strm in zip(sts, streams):
            with torch.cuda.stream(strm):
                _step(st)
        torch.cuda.synchronize()
        for k, st in enumerate(sts):
            for i, (a, b) in enumerate(zip(_results(st), want[k])):
                assert torch.equal(a, b), (rep, k, i)
