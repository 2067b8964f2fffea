"""ctypes binding of libmxq_roofline.so (include/mxq_roofline.h): plain
streaming kernels -- copy, read only, write only -- that measure the practical
HBM ceiling the codec kernels are compared with.  Measurement only; the codec
never calls them."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxq_roofline.so")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python fp8_quantize_pack_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        L.mxq_ref_copy.argtypes = [vp, vp, i64, i32, vp]
        L.mxq_ref_read.argtypes = [vp, i64, i32, u32, vp, vp]
        L.mxq_ref_fill.argtypes = [vp, i64, u32, i32, vp]
        L.mxq_ref_clock.argtypes = [vp, i32, i32, vp]
        for f in ("mxq_ref_copy", "mxq_ref_read", "mxq_ref_fill", "mxq_ref_clock"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _nbytes(t: torch.Tensor) -> int:
    if not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError("reference kernels take contiguous GPU tensors")
    return t.numel() * t.element_size()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ok(st: int, call: str) -> None:
    if st != 0:
        raise RuntimeError(f"{call} returned status {st}")


def copy(src: torch.Tensor, dst: torch.Tensor, unroll: int = 2) -> None:
    n = _nbytes(src)
    if _nbytes(dst) != n:
        raise ValueError("copy needs equal sizes")
    _ok(lib().mxq_ref_copy(src.data_ptr(), dst.data_ptr(), n, unroll, _stream(src)), "mxq_ref_copy")


def read(src: torch.Tensor, sink: torch.Tensor, unroll: int = 2, magic: int = 0x9E3779B9) -> None:
    _ok(lib().mxq_ref_read(src.data_ptr(), _nbytes(src), unroll, magic, sink.data_ptr(),
                           _stream(src)), "mxq_ref_read")


def fill(dst: torch.Tensor, value: int = 0, unroll: int = 2) -> None:
    _ok(lib().mxq_ref_fill(dst.data_ptr(), _nbytes(dst), value, unroll, _stream(dst)),
        "mxq_ref_fill")


def clock(out: torch.Tensor, iters: int = 4096) -> None:
    """Launch the shader clock probe: out is an int64 GPU tensor of 2 * blocks
    values (blocks workgroups of one wave); read it with clock_mhz."""
    if out.dtype != torch.int64 or out.numel() % 2 or out.numel() == 0:
        raise ValueError("clock probe output: a non-empty int64 tensor of 2 * blocks values")
    _nbytes(out)
    _ok(lib().mxq_ref_clock(out.data_ptr(), out.numel() // 2, iters, _stream(out)), "mxq_ref_clock")


def clock_mhz(out: torch.Tensor) -> float:
    """Mean shader clock in MHz from a clock probe's output (host read)."""
    v = out.view(-1, 2).cpu().double()
    return float(v[:, 0].sum() / v[:, 1].sum() * 100.0)
