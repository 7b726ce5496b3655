"""ctypes binding for libtsoftmax (C-ABI declared in include/tsoftmax.h and
include/tsoftmax_measure.h).

Argument marshalling only: shape/dtype/device checks, output allocation, and
passing raw device pointers and torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels; there is no CPU fallback. If
the library is missing, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsoftmax.so")
# Same sources built without the -inf guard; loaded only by the tests that show
# what the guard changes. Never used by the functions below.
NOGUARD_LIB_PATH = os.path.join(_HERE, "libtsoftmax_noguard.so")

TS_OK = 0
TS_ERR_INVALID_ARGUMENT = 1
TS_ERR_HIP = 2
TS_ERR_OUT_OF_MEMORY = 3
TS_ERR_NOT_RESERVED = 4
TS_ERR_SYNC_TIMEOUT = 5

TS_VARIANT_AUTO = 0
TS_VARIANT_SPLIT = 1
TS_VARIANT_ROWWISE = 2
TS_VARIANT_FUSED = 3
VARIANT_NAMES = {TS_VARIANT_AUTO: "auto", TS_VARIANT_SPLIT: "split",
                 TS_VARIANT_ROWWISE: "rowwise", TS_VARIANT_FUSED: "fused"}
CHUNKS = (1024, 2048, 4096, 8192, 16384)

# name -> (restype, argtypes); the exported C-ABI, in header order
_P, _I64, _I32, _U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
SIGNATURES = {
    "ts_softmax": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "ts_softmax_noalloc": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "ts_softmax_masked": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P]),
    "ts_softmax_variant": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _I32, _I32, _P]),
    "ts_plan": (ctypes.c_int, [_I64, _I64, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "ts_sample": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "ts_softmax_sample": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P]),
    "ts_reserve": (ctypes.c_int, [_I64, _I64, _P]),
    "ts_device_errors": (ctypes.c_int, [_P, ctypes.POINTER(_U32)]),
    "ts_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ts_abi_version": (ctypes.c_int32, []),
    "ts_copy_f32": (ctypes.c_int, [_P, _P, _I64, _P]),
    "ts_debug_set_spin_limit": (ctypes.c_int, [_U32]),
    "ts_debug_set_resident_cap": (ctypes.c_int, [_I64]),
    "ts_device_memory_params": (ctypes.c_int, [_I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
}

_lib = None


class TsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the C ABI and declare its signatures (raises if missing)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m temperature_softmax_vocabulary_amd.build`")
    l = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(l, name)
        fn.restype = res
        fn.argtypes = args
    return l


def lib() -> ctypes.CDLL:
    """Load libtsoftmax.so from the package directory (raises if not built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def ts_status_string(status: int) -> str:
    return lib().ts_status_string(int(status)).decode()


def ts_abi_version() -> int:
    return int(lib().ts_abi_version())


def _check(status: int) -> None:
    if status == TS_OK:
        return
    msg = ts_status_string(status)
    if status == TS_ERR_INVALID_ARGUMENT:
        raise ValueError(msg)
    raise TsError(status, msg)


# torch's raw current-stream and current-device accessors: the same values as
# torch.cuda.current_stream(...).cuda_stream and torch.cuda.current_device(),
# without building Python stream objects (1.9 and 0.3 us a call otherwise).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_raw_device = getattr(torch._C, "_cuda_getDevice", None)
_NO_SWITCH = contextlib.nullcontext()


def _stream_handle(device: torch.device, stream=None) -> int:
    if stream is None:
        if _raw_stream is not None:
            return int(_raw_stream(device.index if device.index is not None else torch.cuda.current_device()))
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _on(device: torch.device):
    """Make `device` the current HIP device for the call (the library keys its
    workspace by the current device); no switch when it already is."""
    cur = _raw_device() if _raw_device is not None else torch.cuda.current_device()
    return _NO_SWITCH if device.index is None or device.index == cur else torch.cuda.device(device)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if isinstance(t, torch.Tensor) and t.is_cuda and t.dtype is dtype and t.dim() == ndim and t.is_contiguous():
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    raise ValueError(f"{name} must be contiguous")


def _softmax_args(logits, temps, out):
    _need(logits, "logits", torch.float32, 2)
    _need(temps, "temps", torch.float32, 1)
    B, V = logits.shape
    if temps.shape[0] != B or temps.device != logits.device:
        raise ValueError("temps must be [B] on the logits' device")
    if out is None:
        out = torch.empty_like(logits)
    else:
        _need(out, "out", torch.float32, 2)
        if tuple(out.shape) != (B, V) or out.device != logits.device:
            raise ValueError("out must be [B, V] on the logits' device")
    return B, V, out


def ts_softmax(logits: torch.Tensor, temps: torch.Tensor, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """probs = softmax(logits[b, :] / temps[b]) on the device (out may be logits)."""
    B, V, out = _softmax_args(logits, temps, out)
    with _on(logits.device):
        _check(lib().ts_softmax(logits.data_ptr(), temps.data_ptr(), B, V, out.data_ptr(),
                                _stream_handle(logits.device, stream)))
    return out


def ts_softmax_noalloc(logits: torch.Tensor, temps: torch.Tensor, out: torch.Tensor,
                       stream=None) -> torch.Tensor:
    """ts_softmax through the entry point that allocates no device memory (its
    scratch is one array per GPU, shared by every call on it: overlapping calls
    race). out is required (it may be logits)."""
    if out is None:
        raise ValueError("ts_softmax_noalloc needs out: it allocates nothing")
    B, V, out = _softmax_args(logits, temps, out)
    with _on(logits.device):
        _check(lib().ts_softmax_noalloc(logits.data_ptr(), temps.data_ptr(), B, V, out.data_ptr(),
                                        _stream_handle(logits.device, stream)))
    return out


def _allowed_arg(allowed, B, V, device):
    if allowed is None:
        return None
    _need(allowed, "allowed", torch.int32 if getattr(allowed, "dtype", None) == torch.int32 else torch.uint32, 2)
    if tuple(allowed.shape) != (B, (V + 31) // 32) or allowed.device != device:
        raise ValueError(f"allowed must be [B, ceil(V/32)] = [{B}, {(V + 31) // 32}] 32-bit words on the device")
    return allowed.data_ptr()


def ts_softmax_masked(logits: torch.Tensor, temps: torch.Tensor, allowed: torch.Tensor,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ts_softmax with an allowed-id bitmask ([B, ceil(V/32)] int32/uint32; bit j%32
    of word j//32 set = id j allowed) applied as -inf while the logits are read."""
    B, V, out = _softmax_args(logits, temps, out)
    with _on(logits.device):
        _check(lib().ts_softmax_masked(logits.data_ptr(), temps.data_ptr(), _allowed_arg(allowed, B, V, logits.device),
                                       B, V, out.data_ptr(), _stream_handle(logits.device, stream)))
    return out


def ts_softmax_variant(logits: torch.Tensor, temps: torch.Tensor, variant: int, chunk: int = 0,
                       out: Optional[torch.Tensor] = None, stream=None,
                       allowed: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ts_softmax (or ts_softmax_masked) with the work split forced (tests and tuning)."""
    B, V, out = _softmax_args(logits, temps, out)
    with _on(logits.device):
        _check(lib().ts_softmax_variant(logits.data_ptr(), temps.data_ptr(), _allowed_arg(allowed, B, V, logits.device),
                                        B, V, out.data_ptr(), int(variant), int(chunk),
                                        _stream_handle(logits.device, stream)))
    return out


def ts_plan(B: int, V: int, device=None) -> Tuple[int, int]:
    """(variant, chunk) the library picks for (B, V) on `device` (host only)."""
    v, c = ctypes.c_int32(), ctypes.c_int32()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with _on(dev):
        _check(lib().ts_plan(int(B), int(V), ctypes.byref(v), ctypes.byref(c)))
    return v.value, c.value


def ts_sample(probs: torch.Tensor, uniforms: torch.Tensor, out_ids: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """Inverse-CDF ids [B, K] (int32) for probs [B, V] and uniforms [B, K]."""
    _need(probs, "probs", torch.float32, 2)
    _need(uniforms, "uniforms", torch.float32, 2)
    B, V = probs.shape
    if uniforms.shape[0] != B or uniforms.device != probs.device:
        raise ValueError("uniforms must be [B, K] on the probs' device")
    K = uniforms.shape[1]
    if out_ids is None:
        out_ids = torch.empty((B, K), dtype=torch.int32, device=probs.device)
    else:
        _need(out_ids, "out_ids", torch.int32, 2)
        if tuple(out_ids.shape) != (B, K) or out_ids.device != probs.device:
            raise ValueError("out_ids must be [B, K] int32 on the probs' device")
    with _on(probs.device):
        _check(lib().ts_sample(probs.data_ptr(), uniforms.data_ptr(), B, V, K, out_ids.data_ptr(),
                               _stream_handle(probs.device, stream)))
    return out_ids


def ts_softmax_sample(logits: torch.Tensor, temps: torch.Tensor, uniforms: torch.Tensor,
                      out_ids: Optional[torch.Tensor] = None, probs_out=False,
                      stream=None, allowed: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Softmax and inverse-CDF draw in one call.

    Returns (ids [B, K] int32, probs [B, V] or None). probs_out: False (do not
    write the probabilities: the draw works from the logits), True (allocate
    them) or a [B, V] float32 tensor (may be `logits` itself)."""
    B, V, _ = _softmax_args(logits, temps, logits)
    _need(uniforms, "uniforms", torch.float32, 2)
    if uniforms.shape[0] != B or uniforms.device != logits.device:
        raise ValueError("uniforms must be [B, K] on the logits' device")
    K = uniforms.shape[1]
    if out_ids is None:
        out_ids = torch.empty((B, K), dtype=torch.int32, device=logits.device)
    else:
        _need(out_ids, "out_ids", torch.int32, 2)
        if tuple(out_ids.shape) != (B, K) or out_ids.device != logits.device:
            raise ValueError("out_ids must be [B, K] int32 on the logits' device")
    if probs_out is True:
        probs = torch.empty_like(logits)
    elif probs_out is False or probs_out is None:
        probs = None
    else:
        _, _, probs = _softmax_args(logits, temps, probs_out)
    with _on(logits.device):
        _check(lib().ts_softmax_sample(logits.data_ptr(), temps.data_ptr(), _allowed_arg(allowed, B, V, logits.device),
                                       uniforms.data_ptr(), B, V, K,
                                       probs.data_ptr() if probs is not None else None, out_ids.data_ptr(),
                                       _stream_handle(logits.device, stream)))
    return out_ids, probs


def ts_reserve(max_B: int, max_V: int, device=None, stream=None) -> None:
    """Pre-allocate the workspace of `stream` (default: current) for B <= max_B, V <= max_V."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with _on(dev):
        _check(lib().ts_reserve(int(max_B), int(max_V), _stream_handle(dev, stream)))


def ts_device_errors(device=None, stream=None) -> int:
    """Synchronise the stream and return (and clear) its device error flags.

    Raises TsError(TS_ERR_SYNC_TIMEOUT) when a fused wait ran out."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    flags = ctypes.c_uint32()
    with _on(dev):
        st = lib().ts_device_errors(_stream_handle(dev, stream), ctypes.byref(flags))
    if st not in (TS_OK,):
        _check(st)
    return flags.value


def ts_copy_f32(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """dst.copy_(src) through the library's streaming copy kernel (bandwidth reference)."""
    if src.dtype != torch.float32 or dst.dtype != torch.float32 or not src.is_contiguous() \
            or not dst.is_contiguous() or src.numel() != dst.numel() or src.device != dst.device:
        raise ValueError("src and dst must be contiguous float32 tensors of equal size on one device")
    with _on(src.device):
        _check(lib().ts_copy_f32(src.data_ptr(), dst.data_ptr(), src.numel(),
                                 _stream_handle(src.device, stream)))
    return dst


def ts_debug_set_spin_limit(polls: int) -> None:
    """Bound (in polls) on a fused kernel's wait; 0 restores the default."""
    _check(lib().ts_debug_set_spin_limit(int(polls)))


def ts_device_memory_params(device=None) -> Tuple[int, int]:
    """(memory clock in kHz, memory bus width in bits) that HIP reports for `device`."""
    idx = torch.cuda.current_device() if device is None else torch.device(device).index or 0
    c, w = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ts_device_memory_params(int(idx), ctypes.byref(c), ctypes.byref(w)))
    return c.value, w.value


def ts_debug_set_resident_cap(workgroups: int) -> None:
    """Bound on the co-resident fused workgroups the planner counts on; 0 removes it."""
    _check(lib().ts_debug_set_resident_cap(int(workgroups)))
