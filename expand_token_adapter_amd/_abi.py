"""ctypes declarations of the C ABI in include/lora_batch.h.

Loads ``liblora_batch.so`` built in-tree by ``build.py``.  There is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# LORA_BATCH_LIB: another build of the library (e.g. one compiled with tuning
# defines by build.build(out=..., defines=...)); the in-tree build otherwise.
LIB_PATH = os.environ.get("LORA_BATCH_LIB") or os.path.join(_PKG, "liblora_batch.so")

LORA_OK = 0
LORA_ERR_INVALID_ARG = -1
LORA_ERR_UNSUPPORTED = -2
LORA_ERR_WORKSPACE = -3
LORA_ERR_HIP = -4
LORA_ERR_TOO_LARGE = -5
LORA_NOALLOC_SCRATCH_BYTES = 32 << 20
LORA_BF16 = 0
LORA_F32 = 1
LORA_MAX_RANK = 128
LORA_ABI_VERSION = 1

# Every function the header declares, with (restype, argtypes).
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_vp = ctypes.c_void_p


class LoraAdapter(ctypes.Structure):
    _fields_ = [("A", _vp), ("B", _vp), ("rank", _i32), ("scale", ctypes.c_float)]


class LoraAdapterGrad(ctypes.Structure):
    _fields_ = [("dA", _vp), ("dB", _vp)]


class LoraSegments(ctypes.Structure):
    _fields_ = [("counts", _vp), ("offsets", _vp), ("perm", _vp), ("err", _vp), ("sched", _vp)]


class LoraAdamwTensor(ctypes.Structure):
    _fields_ = [("w", _vp), ("master", _vp), ("grad", _vp), ("m", _vp), ("v", _vp), ("n", _i64)]


class LoraAdamwParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("grad_scale", ctypes.c_float),
                ("step", _i32), ("zero_grad", _i32)]


LORA_ADAMW_MAX_TENSORS = 32


class LoraSlice(ctypes.Structure):
    _fields_ = [("adapters", _vp), ("y", _vp), ("ldy", _i64), ("v", _vp), ("ldv", _i64), ("d_out", _i32),
                ("reserved", _i32)]


LORA_MAX_SLICES = 3


class LoraSegmentsJob(ctypes.Structure):
    _fields_ = [("adapter_ids", _vp), ("T", _i32), ("seg", LoraSegments), ("ws", _vp), ("ws_bytes", _sz)]


SIGNATURES = {
    "lora_abi_version": (ctypes.c_int, []),
    "lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lora_segments_sched_elems": (_sz, [_i32, _i32]),
    "lora_segments_workspace_bytes": (_sz, [_i32, _i32]),
    "lora_shrink_workspace_bytes": (_sz, [ctypes.c_int, _i32, _i32, _i32]),
    "lora_backward_workspace_bytes": (_sz, [ctypes.c_int, _i32, _i32, _i32, _i32]),
    "lora_segments_build": (ctypes.c_int, [_vp, _i32, _i32, LoraSegments, _vp, _sz, _vp]),
    "lora_segments_build_batch": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "lora_shrink": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i32, _i32, _vp, _i32, _i32, LoraSegments,
                                   _vp, _i64, _vp, _sz, _vp]),
    "lora_shrink_noalloc": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i32, _i32, _vp, _i32, _i32, LoraSegments,
                                           _vp, _i64, _vp]),
    "lora_expand_add": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i32, _i32, _vp, _i32, _i32, LoraSegments,
                                       _vp, _i64, _vp]),
    "lora_forward": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i32, _i32, _i32, _vp, _i32, _i32, LoraSegments,
                                    _vp, _i64, _vp, _i64, _vp]),
    "lora_forward_multi": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i32, _i32, _vp, _i32, _i32, _i32, LoraSegments,
                                          _vp]),
    "lora_adamw_step": (ctypes.c_int, [ctypes.c_int, _vp, _i32, LoraAdamwParams, _vp]),
    "lora_backward": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp,
                                     _vp, _i32, _i32, LoraSegments, _vp, _i64, _vp, _sz, _vp]),
    "lora_backward_preemptible": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32,
                                                 _vp, _vp, _i32, _i32, LoraSegments, _vp, _i64, _vp, _sz, _vp, _vp,
                                                 _vp]),
}

_lib = None


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = status_string(status) if _lib is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python expand_token_adapter_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.lora_abi_version() != LORA_ABI_VERSION:
        raise RuntimeError("liblora_batch.so ABI version mismatch; rebuild it")
    _lib = lib
    return lib


_hip = None


def host_device_pointer(host_ptr: int) -> int:
    """Device address of pinned host memory (hipHostGetDevicePointer of the
    HIP runtime already loaded by this process; never a second copy of it)."""
    global _hip
    load()
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_LAZY)
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    out = ctypes.c_void_p()
    rc = _hip.hipHostGetDevicePointer(ctypes.byref(out), ctypes.c_void_p(host_ptr), 0)
    if rc != 0 or not out.value:
        raise ValueError(f"hipHostGetDevicePointer failed ({rc}): the memory is not pinned host memory")
    return out.value


def status_string(status: int) -> str:
    return load().lora_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != LORA_OK:
        raise LoraError(fn, status)
