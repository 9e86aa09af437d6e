"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, answers its pure queries, and rejects bad arguments before touching
the GPU (every call here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

from expand_token_adapter_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_batch.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.SIGNATURES), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert lib.lora_abi_version() == 1
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(_abi.status_string(s), str) and _abi.status_string(s)


def test_struct_sizes_match_header():
    assert ctypes.sizeof(_abi.LoraAdapter) == 24
    assert ctypes.sizeof(_abi.LoraAdapterGrad) == 16
    assert ctypes.sizeof(_abi.LoraSegments) == 40
    assert ctypes.sizeof(_abi.LoraSegmentsJob) == 72
    assert _abi.LoraSegmentsJob.seg.offset == 16 and _abi.LoraSegmentsJob.ws_bytes.offset == 64


def test_struct_layouts_match_header_compiled_by_gcc(tmp_path):
    # sizes and offsets of the header's structs as a C compiler lays them out
    probe = tmp_path / "probe.c"
    probe.write_text("""#include <stdio.h>
#include <stddef.h>
#include "lora_batch.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(lora_adapter), sizeof(lora_adapter_grad), sizeof(lora_segments),
         sizeof(lora_segments_job), sizeof(lora_adamw_tensor), sizeof(lora_adamw_params), sizeof(lora_slice));
  printf("%zu %zu %zu %zu\\n", offsetof(lora_adamw_tensor, n), offsetof(lora_adamw_params, step),
         offsetof(lora_adamw_params, zero_grad), offsetof(lora_segments_job, ws_bytes));
  return 0;
}
""")
    exe = tmp_path / "probe"
    import subprocess
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(probe), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    sizes = [int(v) for v in out]
    assert sizes[:7] == [ctypes.sizeof(t) for t in (_abi.LoraAdapter, _abi.LoraAdapterGrad, _abi.LoraSegments,
                                                      _abi.LoraSegmentsJob, _abi.LoraAdamwTensor,
                                                      _abi.LoraAdamwParams, _abi.LoraSlice)]
    assert sizes[7:] == [_abi.LoraAdamwTensor.n.offset, _abi.LoraAdamwParams.step.offset,
                         _abi.LoraAdamwParams.zero_grad.offset, _abi.LoraSegmentsJob.ws_bytes.offset]


def test_forward_multi_rejects(lib):
    bad, uns = _abi.LORA_ERR_INVALID_ARG, _abi.LORA_ERR_UNSUPPORTED

    def sl(adapters=FAKE, y=FAKE, ldy=512, v=None, ldv=0, d_out=512, reserved=0):
        return _abi.LoraSlice(adapters, y, ldy, v, ldv, d_out, reserved)

    def call(*slices, n=None, r_max=16, T=10, A=4, seg=None):
        arr = (_abi.LoraSlice * max(1, len(slices)))(*slices)
        return lib.lora_forward_multi(0, FAKE, 256, T, 256, arr, len(slices) if n is None else n, A, r_max,
                                      seg or _seg(), None)

    assert call(sl(), n=0) == bad and call(sl(), sl(), sl(), sl()) == bad      # 1..3 slices
    assert lib.lora_forward_multi(0, FAKE, 256, 10, 256, None, 1, 4, 16, _seg(), None) == bad
    assert call(sl(), sl(adapters=None)) == bad and call(sl(), sl(adapters=FAKE + 4)) == bad
    assert call(sl(), sl(d_out=0)) == bad and call(sl(reserved=1)) == bad
    assert call(sl(), sl(y=None)) == bad and call(sl(), sl(ldy=256)) == bad
    assert call(sl(), sl(d_out=260, ldy=264)) == uns                          # d_out not a multiple of 8
    assert call(sl(), sl(v=FAKE, ldv=8)) == bad                               # ldv < r_max
    assert call(sl(), sl(), r_max=72) == uns                                  # several slices above rank 64
    assert call(sl(), r_max=129) == bad and call(sl(), seg=_seg(False)) == bad
    assert call(sl(y=None), sl(y=None), T=0) == 0                             # nothing to do


def test_backward_preemptible_rejects(lib):
    bad = _abi.LORA_ERR_INVALID_ARG
    need = lib.lora_backward_workspace_bytes(0, 64, 256, 512, 16)

    def call(grant=FAKE, status=FAKE, T=64, A=4):
        return lib.lora_backward_preemptible(0, FAKE, 256, FAKE, 512, None, 0, T, 256, 512, FAKE, FAKE, A, 16,
                                             _seg(), None, 0, FAKE, need, grant, status, None)

    assert call(grant=None) == bad and call(status=None) == bad
    assert call(grant=FAKE + 2) == bad and call(status=FAKE + 1) == bad   # not 4-byte aligned
    assert call(A=0) == bad                                                # the backward's own checks follow
    assert call(T=-1) == bad


def test_adamw_rejects_before_touching_the_gpu(lib):
    bad = _abi.LORA_ERR_INVALID_ARG

    def hp(**kw):
        d = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, grad_scale=1.0, step=1, zero_grad=0)
        d.update(kw)
        return _abi.LoraAdamwParams(**d)

    def arr(*ts):
        a = (_abi.LoraAdamwTensor * max(1, len(ts)))(*ts)
        return a

    good = _abi.LoraAdamwTensor(FAKE, None, FAKE, FAKE, FAKE, 1024)
    # nothing to do: no tensors, or only empty ones
    assert lib.lora_adamw_step(0, None, 0, hp(), None) == _abi.LORA_OK
    assert lib.lora_adamw_step(0, arr(_abi.LoraAdamwTensor(None, None, None, None, None, 0)), 1, hp(), None) == 0
    assert lib.lora_adamw_step(2, arr(good), 1, hp(), None) == bad          # dtype
    assert lib.lora_adamw_step(0, None, 1, hp(), None) == bad               # no array
    assert lib.lora_adamw_step(0, arr(good), -1, hp(), None) == bad
    assert lib.lora_adamw_step(0, arr(*[good] * 33), 33, hp(), None) == bad  # more than the maximum
    for t in (_abi.LoraAdamwTensor(None, None, FAKE, FAKE, FAKE, 8), _abi.LoraAdamwTensor(FAKE, None, None, FAKE, FAKE, 8),
              _abi.LoraAdamwTensor(FAKE, None, FAKE, None, FAKE, 8), _abi.LoraAdamwTensor(FAKE, None, FAKE, FAKE, None, 8),
              _abi.LoraAdamwTensor(FAKE + 4, None, FAKE, FAKE, FAKE, 8),
              _abi.LoraAdamwTensor(FAKE, FAKE + 8, FAKE, FAKE, FAKE, 8),
              _abi.LoraAdamwTensor(FAKE, None, FAKE, FAKE, FAKE, -1)):
        assert lib.lora_adamw_step(0, arr(good, t), 2, hp(), None) == bad
    for kw in (dict(lr=-1.0), dict(lr=float("inf")), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0),
               dict(weight_decay=-0.01), dict(grad_scale=float("nan")), dict(step=0), dict(lr=float("nan"))):
        assert lib.lora_adamw_step(0, arr(good), 1, hp(**kw), None) == bad, kw


def test_workspace_queries(lib):
    assert lib.lora_segments_workspace_bytes(0, 4) > 0
    assert lib.lora_segments_workspace_bytes(-1, 4) == 0
    assert lib.lora_segments_workspace_bytes(10, 0) == 0
    a = lib.lora_segments_workspace_bytes(1000, 32)
    b = lib.lora_segments_workspace_bytes(5000, 32)
    assert b > a >= 4 * 1000
    assert lib.lora_backward_workspace_bytes(0, 2048, 4096, 14336, 64) >= 3 * 2048 * 64 * 4
    assert lib.lora_backward_workspace_bytes(0, 16, 256, 256, 0) == 0
    assert lib.lora_backward_workspace_bytes(0, 16, 256, 256, 129) == 0
    assert lib.lora_backward_workspace_bytes(7, 16, 256, 256, 8) == 0
    # split-K partials: one [T, round_up(r_max, 8)] fp32 block per slice of d_in
    # (512 elements for bf16, 256 for fp32)
    assert lib.lora_shrink_workspace_bytes(0, 100, 4096, 20) == 8 * 100 * 24 * 4
    assert lib.lora_shrink_workspace_bytes(1, 100, 4096, 20) == 16 * 100 * 24 * 4
    assert lib.lora_shrink_workspace_bytes(0, 100, 1000, 8) == 2 * 100 * 8 * 4
    assert lib.lora_shrink_workspace_bytes(0, 100, 0, 8) == 0
    assert lib.lora_shrink_workspace_bytes(3, 100, 256, 8) == 0
    # 16-row and 64-row tile records for every row plus one partial tile per adapter
    n = lib.lora_segments_sched_elems(1000, 10)
    assert n >= 4 * ((1000 + 15) // 16 + 10) + 4 * ((1000 + 63) // 64 + 10)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _seg(ok=True):
    p = FAKE if ok else 0
    return _abi.LoraSegments(FAKE, FAKE, FAKE, FAKE, p)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), _abi.LORA_ERR_INVALID_ARG),
    (dict(T=-1), _abi.LORA_ERR_INVALID_ARG),
    (dict(A=0), _abi.LORA_ERR_INVALID_ARG),
    (dict(r_max=0), _abi.LORA_ERR_INVALID_ARG),
    (dict(r_max=129), _abi.LORA_ERR_INVALID_ARG),
    (dict(adapters=0), _abi.LORA_ERR_INVALID_ARG),
    (dict(seg_ok=False), _abi.LORA_ERR_INVALID_ARG),
    (dict(x=0), _abi.LORA_ERR_INVALID_ARG),
    (dict(x=FAKE + 4), _abi.LORA_ERR_INVALID_ARG),
    (dict(ld=100), _abi.LORA_ERR_INVALID_ARG),
    (dict(d=100, ld=100), _abi.LORA_ERR_UNSUPPORTED),
    (dict(ld=260), _abi.LORA_ERR_UNSUPPORTED),
    (dict(v=0), _abi.LORA_ERR_INVALID_ARG),
    (dict(ldv=6), _abi.LORA_ERR_INVALID_ARG),
    (dict(ldv=4), _abi.LORA_ERR_INVALID_ARG),
    (dict(ldv=12, r_max=8), _abi.LORA_ERR_INVALID_ARG),
])
def test_shrink_and_expand_reject_bad_arguments(lib, kw, code):
    a = dict(dtype=0, T=64, A=4, r_max=8, adapters=FAKE, seg_ok=True, x=FAKE, ld=256, d=256, v=FAKE, ldv=8)
    a.update(kw)
    need = lib.lora_shrink_workspace_bytes(0, max(a["T"], 0), max(a["d"], 1), min(max(a["r_max"], 1), 128))
    st = lib.lora_shrink(a["dtype"], a["x"], a["ld"], a["T"], a["d"], a["adapters"], a["A"], a["r_max"],
                         _seg(a["seg_ok"]), a["v"], a["ldv"], FAKE, need, None)
    assert st == code
    st = lib.lora_expand_add(a["dtype"], a["v"], a["ldv"], a["T"], a["d"], a["adapters"], a["A"], a["r_max"],
                             _seg(a["seg_ok"]), a["x"], a["ld"], None)
    assert st == code


def test_zero_rows_is_a_no_op(lib):
    st = lib.lora_shrink(0, 0, 0, 0, 256, FAKE, 4, 8, _seg(), 0, 0, 0, 0, None)
    assert st == _abi.LORA_OK
    st = lib.lora_expand_add(0, 0, 0, 0, 256, FAKE, 4, 8, _seg(), 0, 0, None)
    assert st == _abi.LORA_OK
    st = lib.lora_segments_build(0, 0, 4, _seg(), 0, 0, None)
    assert st == _abi.LORA_OK
    st = lib.lora_backward(0, 0, 0, 0, 0, 0, 0, 0, 256, 256, FAKE, FAKE, 4, 8, _seg(), 0, 0, 0, 0, None)
    assert st == _abi.LORA_OK
    st = lib.lora_forward(0, 0, 0, 0, 256, 256, FAKE, 4, 8, _seg(), 0, 0, 0, 0, None)
    assert st == _abi.LORA_OK


def test_fused_forward_rejects(lib):
    def call(dtype=0, x=FAKE, ldx=256, T=10, d_in=256, d_out=512, A=4, r_max=16, seg=None, y=FAKE, ldy=512,
             v=0, ldv=0):
        return lib.lora_forward(dtype, x, ldx, T, d_in, d_out, FAKE, A, r_max, seg or _seg(), y, ldy, v, ldv, None)

    bad, uns = _abi.LORA_ERR_INVALID_ARG, _abi.LORA_ERR_UNSUPPORTED
    assert call(dtype=2) == bad
    assert call(x=0) == bad and call(y=0) == bad
    assert call(x=FAKE + 8) == bad            # not 16-byte aligned
    assert call(ldx=128) == bad               # ld < d_in
    assert call(d_in=260, ldx=264) == uns     # d_in not a multiple of 8
    assert call(d_out=0) == bad and call(T=-1) == bad and call(A=0) == bad
    assert call(r_max=0) == bad and call(r_max=129) == bad
    assert call(seg=_seg(False)) == bad
    assert call(v=FAKE, ldv=8) == bad         # ldv < r_max
    assert call(v=FAKE, ldv=20) == bad        # ldv not a multiple of 8


def test_segments_build_rejects(lib):
    need = lib.lora_segments_workspace_bytes(100, 4)
    assert lib.lora_segments_build(FAKE, -1, 4, _seg(), FAKE, need, None) == _abi.LORA_ERR_INVALID_ARG
    assert lib.lora_segments_build(FAKE, 100, 0, _seg(), FAKE, need, None) == _abi.LORA_ERR_INVALID_ARG
    assert lib.lora_segments_build(0, 100, 4, _seg(), FAKE, need, None) == _abi.LORA_ERR_INVALID_ARG
    assert lib.lora_segments_build(FAKE, 100, 4, _seg(False), FAKE, need, None) == _abi.LORA_ERR_INVALID_ARG
    assert lib.lora_segments_build(FAKE, 100, 4, _seg(), FAKE, need - 1, None) == _abi.LORA_ERR_WORKSPACE
    assert lib.lora_segments_build(FAKE, 100, 4, _seg(), 0, need, None) == _abi.LORA_ERR_WORKSPACE


def test_segments_build_batch_rejects(lib):
    need = lib.lora_segments_workspace_bytes(100, 4)

    def jobs(*js):
        arr = (_abi.LoraSegmentsJob * len(js))(*js)
        return ctypes.addressof(arr), arr

    good = _abi.LoraSegmentsJob(FAKE, 100, _seg(), FAKE, need)
    assert lib.lora_segments_build_batch(None, 0, 4, None) == _abi.LORA_OK  # nothing to do
    assert lib.lora_segments_build_batch(None, -1, 4, None) == _abi.LORA_ERR_INVALID_ARG
    assert lib.lora_segments_build_batch(None, 2, 4, None) == _abi.LORA_ERR_INVALID_ARG
    # any bad job rejects the whole call before anything is enqueued
    for bad, code in [(_abi.LoraSegmentsJob(FAKE, -1, _seg(), FAKE, need), _abi.LORA_ERR_INVALID_ARG),
                      (_abi.LoraSegmentsJob(0, 100, _seg(), FAKE, need), _abi.LORA_ERR_INVALID_ARG),
                      (_abi.LoraSegmentsJob(FAKE, 100, _seg(False), FAKE, need), _abi.LORA_ERR_INVALID_ARG),
                      (_abi.LoraSegmentsJob(FAKE, 100, _seg(), FAKE, need - 1), _abi.LORA_ERR_WORKSPACE)]:
        ptr, _keep = jobs(good, bad)
        assert lib.lora_segments_build_batch(ptr, 2, 4, None) == code
    ptr, _keep = jobs(good)
    assert lib.lora_segments_build_batch(ptr, 1, 0, None) == _abi.LORA_ERR_INVALID_ARG


def test_shrink_workspace_rejected(lib):
    need = lib.lora_shrink_workspace_bytes(0, 64, 256, 8)
    args = (0, FAKE, 256, 64, 256, FAKE, 4, 8, _seg(), FAKE, 8)
    assert lib.lora_shrink(*args, FAKE, need - 1, None) == _abi.LORA_ERR_WORKSPACE
    assert lib.lora_shrink(*args, 0, need, None) == _abi.LORA_ERR_WORKSPACE
    assert lib.lora_shrink(*args, FAKE + 4, need, None) == _abi.LORA_ERR_WORKSPACE


def test_backward_rejects(lib):
    need = lib.lora_backward_workspace_bytes(0, 16, 256, 256, 8)

    def call(**kw):
        a = dict(dtype=0, x=FAKE, ldx=256, dy=FAKE, lddy=256, dx=FAKE, lddx=256, T=16, d_in=256, d_out=256,
                 adapters=FAKE, grads=FAKE, A=4, r_max=8, seg=_seg(), vs=0, ldv=0, ws=FAKE, wsb=need)
        a.update(kw)
        return lib.lora_backward(a["dtype"], a["x"], a["ldx"], a["dy"], a["lddy"], a["dx"], a["lddx"], a["T"],
                                 a["d_in"], a["d_out"], a["adapters"], a["grads"], a["A"], a["r_max"], a["seg"],
                                 a["vs"], a["ldv"], a["ws"], a["wsb"], None)

    assert call(grads=0) == _abi.LORA_ERR_INVALID_ARG
    assert call(grads=FAKE + 4) == _abi.LORA_ERR_INVALID_ARG
    assert call(dy=0) == _abi.LORA_ERR_INVALID_ARG
    assert call(lddy=100) == _abi.LORA_ERR_INVALID_ARG
    assert call(d_out=100, lddy=100) == _abi.LORA_ERR_UNSUPPORTED
    assert call(dx=FAKE + 2) == _abi.LORA_ERR_INVALID_ARG
    assert call(vs=FAKE, ldv=4) == _abi.LORA_ERR_INVALID_ARG
    assert call(vs=FAKE, ldv=12) == _abi.LORA_ERR_INVALID_ARG
    assert call(wsb=need - 1) == _abi.LORA_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == _abi.LORA_ERR_WORKSPACE
    assert call(seg=_seg(False)) == _abi.LORA_ERR_INVALID_ARG


def test_shrink_noalloc_rejects_before_touching_the_gpu(lib):
    bad = _abi.LORA_ERR_INVALID_ARG
    args = dict(dtype=0, x=FAKE, ldx=256, T=64, d_in=256, adapters=FAKE, A=4, r_max=8, seg=_seg(), v=FAKE, ldv=8)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.lora_shrink_noalloc(a["dtype"], a["x"], a["ldx"], a["T"], a["d_in"], a["adapters"], a["A"],
                                       a["r_max"], a["seg"], a["v"], a["ldv"], None)

    assert call(dtype=3) == bad and call(T=-1) == bad and call(A=0) == bad and call(r_max=129) == bad
    assert call(x=0) == bad and call(x=FAKE + 4) == bad and call(v=0) == bad and call(ldv=4) == bad
    assert call(seg=_seg(False)) == bad
    assert call(d_in=100, ldx=100) == _abi.LORA_ERR_UNSUPPORTED
    assert call(T=0, x=0, v=0) == _abi.LORA_OK                               # nothing to do
    # 16 slices x 2^20 rows x 128 ranks of fp32 partials: beyond the static scratch
    assert call(T=1 << 20, d_in=8192, ldx=8192, r_max=128, ldv=128) == _abi.LORA_ERR_TOO_LARGE
    assert lib.lora_shrink_workspace_bytes(0, 1 << 20, 8192, 128) > _abi.LORA_NOALLOC_SCRATCH_BYTES
