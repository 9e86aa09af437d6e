"""A captured HIP graph of one step (batched segment build, shrink, expand-add,
lora_forward without and with v, backward with saved v) replays to the eager results, bit for bit, on every
replay, with eager work and synchronisations between the replays.  The kernels
clear their own scratch (no memset nodes are recorded) and every reduction runs
in a fixed order, so a replay must reproduce the eager step exactly."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import expand_token_adapter_amd as lb
    from gpu_helpers import to_dev


def _mixed():
    rng = np.random.default_rng(21)
    ids = np.concatenate([rng.integers(-1, 5, size=60), np.full(150, 2), rng.integers(0, 5, size=40),
                          np.full(96, 0)]).astype(np.int32)
    return workloads.custom(ids, [8, 16, 40, 24, 64], 320, 448, "bf16", seed=3, ft_start=len(ids) - 96,
                            ft_count=96, name="graph-mixed")


def _decode16():
    # at most 32 rows per adapter, ranks <= 16: the 16-row-tile shrink and
    # expand, the one-launch decode forward and the streaming backward
    rng = np.random.default_rng(23)
    ids = np.concatenate([rng.integers(-1, 24, size=120), np.full(40, 3)]).astype(np.int32)
    return workloads.custom(ids, [16, 8, 5, 16, 12, 1] * 4, 200, 456, "bf16", seed=5, ft_start=len(ids) - 40,
                            ft_count=40, name="graph-decode16")


def _decode64():
    # at most 32 rows per adapter, ranks to 64: lora_forward without v runs the
    # 64-row-tile kernel, with v the 16-row-tile shrink and expand
    rng = np.random.default_rng(29)
    ids = np.concatenate([rng.integers(-1, 12, size=180), np.full(48, 5)]).astype(np.int32)
    return workloads.custom(ids, [16, 64, 8, 40, 24, 33] * 2, 264, 328, "bf16", seed=7, ft_start=len(ids) - 48,
                            ft_count=48, name="graph-decode64")


@pytest.mark.parametrize("kind", ["mixed", "decode16", "decode64"])
def test_graph_replays_match_eager_step(kind):
    wl = {"mixed": _mixed, "decode16": _decode16, "decode64": _decode64}[kind]()
    dev = torch.device("cuda:0")
    s, n = wl.ft_start, wl.ft_count
    A = [to_dev(a, "bf16", dev) for a in wl.A]
    B = [to_dev(b, "bf16", dev) for b in wl.B]
    table = lb.AdapterTable(A, B, wl.scales.tolist())
    x = to_dev(wl.x, "bf16", dev)
    y0 = to_dev(wl.y0, "bf16", dev)
    dy = to_dev(wl.dy, "bf16", dev)
    ids = torch.from_numpy(wl.ids).to(dev)
    ft_ids = ids[s:s + n].contiguous()
    y = y0.clone()
    yf = y0.clone()  # lora_forward's output (without v)
    yfv = y0.clone()  # lora_forward's output with v
    v = torch.zeros((wl.T, (table.r_max + 7) // 8 * 8), dtype=torch.float32, device=dev)
    vf = torch.zeros_like(v)
    dx = torch.zeros((n, wl.d_in), dtype=torch.bfloat16, device=dev)
    dA = [torch.zeros(a.shape, dtype=torch.float32, device=dev) for a in A]
    dB = [torch.zeros(b.shape, dtype=torch.float32, device=dev) for b in B]
    grads = lb.GradTable(dA, dB)
    seg = lb.Segments(wl.T, wl.num_adapters, dev)
    seg_ft = lb.Segments(n, wl.num_adapters, dev)
    ws = torch.empty(lb.lora_shrink_workspace_bytes(torch.bfloat16, wl.T, wl.d_in, table.r_max), dtype=torch.uint8,
                     device=dev)
    bws = torch.empty(lb.lora_backward_workspace_bytes(torch.bfloat16, n, wl.d_in, wl.d_out, table.r_max),
                      dtype=torch.uint8, device=dev)

    def reset():
        # stale values everywhere: columns past round_up(r_a, 8) and rows
        # without an adapter are left unchanged by design, the rest rewritten
        v.fill_(-1.0)
        vf.fill_(-1.0)
        y.copy_(y0)
        yf.copy_(y0)
        yfv.copy_(y0)
        dx.zero_()
        for t in dA + dB:
            t.zero_()

    def step():
        lb.lora_segments_build_batch([(ids, seg), (ft_ids, seg_ft)], wl.num_adapters)
        lb.lora_shrink(x, table, seg, v=v, ws=ws)
        lb.lora_expand_add(v, table, seg, y)
        lb.lora_forward(x, table, seg, yf)
        lb.lora_forward(x, table, seg, yfv, v=vf)
        lb.lora_backward(x[s:s + n], dy, table, grads, seg_ft, dx=dx, v_saved=v[s:s + n], ws=bws)

    reset()
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in [y, yf, yfv, v, vf, dx] + dA + dB]
    assert seg.err.item() == 0 and seg_ft.err.item() == 0

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        reset()
        step()  # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for k in range(3):
        reset()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [y, yf, yfv, v, vf, dx] + dA + dB
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), (k, i)
        assert seg.err.item() == 0 and seg_ft.err.item() == 0


def test_graph_of_multi_slice_forward_preemptible_backward_and_adamw():
    """q/k/v forward in one launch, the grant-gated backward of the trained
    adapter and its AdamW step, captured once.  The grant word is read by the
    kernels at replay time: a replay with the grant withdrawn yields (status 1,
    gradients untouched) and the next granted replay matches the eager step."""
    rng = np.random.default_rng(5)
    ids = np.concatenate([rng.integers(-1, 4, size=90), np.full(64, 1)]).astype(np.int32)
    s, n = 90, 64
    ranks = [16, 8, 32, 24]
    wls = [workloads.custom(ids, ranks, 256, d_out, "bf16", seed=11 + i, ft_start=s, ft_count=n, name=f"slice{i}")
           for i, d_out in enumerate((256, 64, 200))]
    dev = torch.device("cuda:0")
    tables, ys0, ys = [], [], []
    for wl in wls:
        tables.append(lb.AdapterTable([to_dev(a, "bf16", dev) for a in wl.A], [to_dev(b, "bf16", dev) for b in wl.B],
                                      wl.scales.tolist()))
        ys0.append(to_dev(wl.y0, "bf16", dev))
        ys.append(ys0[-1].clone())
    q = tables[0]
    x = to_dev(wls[0].x, "bf16", dev)
    dy = to_dev(wls[0].dy, "bf16", dev)
    ids_d = torch.from_numpy(ids).to(dev)
    seg = lb.Segments(len(ids), len(ranks), dev)
    seg_ft = lb.Segments(n, len(ranks), dev)
    v = torch.zeros((len(ids), 32), dtype=torch.float32, device=dev)
    dx = torch.zeros((n, 256), dtype=torch.bfloat16, device=dev)
    dA = [None, torch.zeros(q.A[1].shape, dtype=torch.float32, device=dev), None, None]
    dB = [None, torch.zeros(q.B[1].shape, dtype=torch.float32, device=dev), None, None]
    grads = lb.GradTable(dA, dB)
    w0 = [q.A[1].clone(), q.B[1].clone()]
    mom = [torch.zeros(t.shape, dtype=torch.float32, device=dev) for t in (dA[1], dB[1], dA[1], dB[1])]
    grant = torch.ones(1, dtype=torch.int32, device=dev)
    status = torch.full((1,), 7, dtype=torch.int32, device=dev)

    def reset():
        for y, y0 in zip(ys, ys0):
            y.copy_(y0)
        v.fill_(-1.0)
        dx.zero_()
        for t in (dA[1], dB[1], *mom):
            t.zero_()
        q.A[1].copy_(w0[0])
        q.B[1].copy_(w0[1])
        status.fill_(7)

    def step():
        lb.lora_segments_build_batch([(ids_d, seg), (ids_d[s:s + n].contiguous(), seg_ft)], len(ranks))
        lb.lora_forward_multi(x, [(tables[0], ys[0], v), (tables[1], ys[1]), (tables[2], ys[2])], seg)
        lb.lora_backward_preemptible(x[s:s + n], dy, q, grads, seg_ft, grant, status, dx=dx)
        lb.lora_adamw_step([(q.A[1], dA[1], mom[0], mom[1]), (q.B[1], dB[1], mom[2], mom[3])], step=1)

    def state():
        return [t.clone() for t in (*ys, v, dx, dA[1], dB[1], *mom, q.A[1], q.B[1], status)]

    reset()
    step()
    torch.cuda.synchronize()
    want = state()
    assert status.item() == 0 and seg.err.item() == 0 and seg_ft.err.item() == 0
    assert dA[1].abs().sum().item() > 0 and not torch.equal(q.A[1], w0[0])

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for k, granted in enumerate((1, 0, 1, 1)):
        reset()
        grant.fill_(granted)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = state()
        if granted:
            for i, (a, b) in enumerate(zip(got, want)):
                assert torch.equal(a, b), (k, i)
        else:
            assert status.item() == 1, k
            for i in range(4):  # y of each slice and v: the forward does not depend on the grant
                assert torch.equal(got[i], want[i]), (k, i)
            assert not dx.any().item() and not dA[1].any().item() and not dB[1].any().item(), k
