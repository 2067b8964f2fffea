"""fp8_quantize_pack_amd -- block-scaled microscaling quantization on MI355X.

A thin ctypes binding over ``libmxq.so`` (HIP kernels for gfx950; C ABI in
``include/mxq.h``).  Every step of every operation runs in the library's
kernels; this module only checks arguments, allocates outputs with
``torch.empty`` and passes device pointers and the current stream.  There is no
CPU fallback: importing fails if the library has not been built.

Two layers, named after the C ABI and after the source pages:

* ``mxq_quantize_mxfp4`` ... ``mxq_quantize_cache``: one-to-one wrappers of the
  C calls taking preallocated torch CUDA tensors (no allocation).
* ``quantize_mxfp4``, ``dequantize_mxfp4``, ``quantize_nvfp4``,
  ``quantize_nvfp4_modelopt``, ``dequantize_nvfp4``, ``quantize_cache``:
  allocate and return new tensors with the dtypes and shapes the pages give
  ("nemo_automodel.components.quantization.mxfp4" / ".nvfp4" and
  "nemo_automodel.components.models.deepseek_v41.quantization").
* ``quantize_mxfp8``, ``dequantize_mxfp8``, ``fake_quantize_fp4_static``:
  ModelOpt's MX real quantization with e4m3 elements and its static
  two-level FP4 quantizer (Model-Optimizer "tensor_quantizer.py").
* ``dequantize_kv_cache``, ``quantize_kv_nvfp4``: the NVFP4 KV cache of
  LongLive's utils/quant.py (paged dequantization; per-head quantization
  with k_smooth).
* ``grouped_mm_mxfp4``, ``grouped_mm_nvfp4``: the grouped expert GEMM over
  packed weights.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

MXQ_F32, MXQ_BF16, MXQ_F16 = 0, 1, 2
FORMATS = {"fp8": 0, "mxfp4": 1, "nvfp4": 2}
NV_MODES = {"row": 0, "given": 1, "tensor": 2}
_DT = {torch.float32: MXQ_F32, torch.bfloat16: MXQ_BF16, torch.float16: MXQ_F16}

MXFP4_BLOCK_SIZE = 32
NVFP4_BLOCK_SIZE = 16

_STATUS = {
    0: "MXQ_OK", 1: "MXQ_E_NULL", 2: "MXQ_E_SHAPE", 3: "MXQ_E_DTYPE",
    4: "MXQ_E_FORMAT", 5: "MXQ_E_BLOCK", 6: "MXQ_E_SIZE", 7: "MXQ_E_LAUNCH",
    8: "MXQ_E_MODE", 9: "MXQ_E_ALIGN", 10: "MXQ_E_SCRATCH",
}


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with "
            "`python fp8_quantize_pack_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.mxq_quantize_mxfp4.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    L.mxq_dequantize_mxfp4.argtypes = [vp, vp, i64, i64, vp, i32, vp]
    L.mxq_quantize_nvfp4.argtypes = [vp, i32, i64, i64, i32, vp, i64, vp, vp, vp, vp, vp]
    L.mxq_dequantize_nvfp4.argtypes = [vp, vp, vp, i64, i64, vp, i32, vp]
    L.mxq_quantize_cache.argtypes = [vp, vp, i32, i64, i64, i32, i32, vp]
    L.mxq_grouped_mm_mxfp4.argtypes = [vp, i32, i64, vp, vp, i64, i64, i64, vp, i32, vp, vp]
    L.mxq_grouped_mm_nvfp4.argtypes = [vp, i32, i64, vp, vp, vp, i64, i64, i64, vp, i32, vp, vp]
    L.mxq_quantize_mxfp8.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    L.mxq_dequantize_mxfp8.argtypes = [vp, vp, i64, i64, vp, i32, vp]
    L.mxq_fake_quantize_fp4_static.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp]
    L.mxq_dequantize_kv_pages_nvfp4.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    L.mxq_quantize_kv_nvfp4.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp, vp, vp]
    L.mxq_quantize_kv_nvfp4_noalloc.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp, vp]
    for f in ("mxq_quantize_mxfp4", "mxq_dequantize_mxfp4", "mxq_quantize_nvfp4",
              "mxq_dequantize_nvfp4", "mxq_quantize_cache", "mxq_grouped_mm_mxfp4",
              "mxq_grouped_mm_nvfp4", "mxq_quantize_mxfp8", "mxq_dequantize_mxfp8",
              "mxq_fake_quantize_fp4_static", "mxq_dequantize_kv_pages_nvfp4",
              "mxq_quantize_kv_nvfp4", "mxq_quantize_kv_nvfp4_noalloc"):
        getattr(L, f).restype = ctypes.c_int
    L.mxq_status_string.argtypes = [ctypes.c_int]
    L.mxq_status_string.restype = ctypes.c_char_p
    L.mxq_abi_version.argtypes = []
    L.mxq_abi_version.restype = ctypes.c_int32
    return L


lib = _load()


class MxqError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = lib.mxq_status_string(status).decode()
        super().__init__(f"{call}: {_STATUS.get(status, status)} ({msg})")


def _check(status: int, call: str) -> None:
    if status == 0:
        return
    if status == 2:
        raise ValueError(str(MxqError(status, call)))
    if status == 3:
        raise TypeError(str(MxqError(status, call)))
    raise MxqError(status, call)


def _ptr(t):
    """Device address of a tensor passed to a C call (host tensors refused)."""
    if t is None:
        return None
    if t.device.type != "cuda" and t.numel():
        raise ValueError("tensors must live on a GPU")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream=None):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream(t.device).cuda_stream


def _dt(t_dtype) -> int:
    if t_dtype not in _DT:
        raise TypeError(f"unsupported floating dtype {t_dtype}")
    return _DT[t_dtype]


def _rows(t: torch.Tensor) -> int:
    k = t.shape[-1] if t.dim() else 1
    return t.numel() // k if k else 0


def _buf(t, nbytes: int, name: str, call: str, at_least: bool = False) -> None:
    """A buffer a C call reads or writes must be one contiguous GPU range of
    exactly the bytes the call touches (at least them, for a scratch word);
    checked before anything is launched, so a short buffer is an error
    instead of an access out of bounds."""
    if t is None:
        raise ValueError(f"{call}: {name} is required")
    have = t.numel() * t.element_size()
    if have < nbytes or (have != nbytes and not at_least):
        raise ValueError(f"{call}: {name} holds {have} bytes, the call needs {nbytes}")
    if not t.is_contiguous():
        raise ValueError(f"{call}: {name} must be contiguous")


def _dev_input(t: torch.Tensor) -> torch.Tensor:
    """Contiguous and 16-byte aligned (copies only when it has to)."""
    if t.device.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    t = t.contiguous()
    if t.data_ptr() % 16:
        t = t.clone()
    return t


# ------------------------------------------------------------------ C ABI layer

def mxq_quantize_mxfp4(x, packed, scales, stream=None) -> None:
    K = x.shape[-1]
    n, c = _rows(x) * K, "mxq_quantize_mxfp4"
    _buf(x, x.numel() * x.element_size(), "x", c)
    _buf(packed, n // 2, "packed", c)
    _buf(scales, n // 32, "scales", c)
    _check(lib.mxq_quantize_mxfp4(_ptr(x), _dt(x.dtype), _rows(x), K,
                                  _ptr(packed), _ptr(scales), _stream(x, stream)),
           "mxq_quantize_mxfp4")


def mxq_dequantize_mxfp4(packed, scales, y, stream=None) -> None:
    K = y.shape[-1]
    n, c = _rows(y) * K, "mxq_dequantize_mxfp4"
    _buf(y, y.numel() * y.element_size(), "y", c)
    _buf(packed, n // 2, "packed", c)
    _buf(scales, n // 32, "scales", c)
    _check(lib.mxq_dequantize_mxfp4(_ptr(packed), _ptr(scales), _rows(y), K,
                                    _ptr(y), _dt(y.dtype), _stream(y, stream)),
           "mxq_dequantize_mxfp4")


def mxq_quantize_nvfp4(x, packed, scales, row_scale, mode="row", given=None,
                       given_stride=1, scratch=None, stream=None) -> None:
    K = x.shape[-1]
    R, c = _rows(x), "mxq_quantize_nvfp4"
    if mode not in NV_MODES:
        raise ValueError(f"unknown NVFP4 mode {mode!r}; expected one of {list(NV_MODES)}")
    _buf(x, x.numel() * x.element_size(), "x", c)
    _buf(packed, R * K // 2, "packed", c)
    _buf(scales, R * K // 16, "scales", c)
    _buf(row_scale, R * 4, "row_scale", c)
    if mode == "given" and R:
        _buf(given, 4 * (R if given_stride else 1), "given", c)
    if mode == "tensor" and R:
        _buf(scratch, 4, "scratch", c, at_least=True)
    _check(lib.mxq_quantize_nvfp4(_ptr(x), _dt(x.dtype), _rows(x), K,
                                  NV_MODES[mode], _ptr(given), given_stride,
                                  _ptr(scratch), _ptr(packed), _ptr(scales),
                                  _ptr(row_scale), _stream(x, stream)),
           "mxq_quantize_nvfp4")


def mxq_dequantize_nvfp4(packed, scales, row_scale, y, stream=None) -> None:
    K = y.shape[-1]
    R, c = _rows(y), "mxq_dequantize_nvfp4"
    _buf(y, y.numel() * y.element_size(), "y", c)
    _buf(packed, R * K // 2, "packed", c)
    _buf(scales, R * K // 16, "scales", c)
    _buf(row_scale, R * 4, "row_scale", c)
    _check(lib.mxq_dequantize_nvfp4(_ptr(packed), _ptr(scales), _ptr(row_scale),
                                    _rows(y), K, _ptr(y), _dt(y.dtype),
                                    _stream(y, stream)),
           "mxq_dequantize_nvfp4")


def mxq_quantize_cache(x, y, fmt, block_size, stream=None) -> None:
    if fmt not in FORMATS:
        raise ValueError(f"unknown cache format {fmt!r}; expected one of {list(FORMATS)}")
    C = x.shape[-1] if x.dim() else 1
    _buf(x, x.numel() * x.element_size(), "x", "mxq_quantize_cache")
    if y.dtype != x.dtype:
        raise TypeError("mxq_quantize_cache: y must have x's dtype")
    _buf(y, x.numel() * x.element_size(), "y", "mxq_quantize_cache")
    _check(lib.mxq_quantize_cache(_ptr(x), _ptr(y), _dt(x.dtype), _rows(x), C,
                                  FORMATS[fmt], int(block_size), _stream(x, stream)),
           "mxq_quantize_cache")


def _gemm_bufs(x, packed, scales, offs, y, transpose, block, call) -> None:
    if x.dim() != 2 or packed.dim() != 3:
        raise ValueError(f"{call}: x must be [tokens, in_dim] and packed [experts, out_dim, "
                         "in_dim // 2]")
    E, N, K = packed.shape[0], packed.shape[1], packed.shape[2] * 2
    din, dout = (N, K) if transpose else (K, N)
    if x.shape[1] != din:
        raise ValueError(f"{call}: x has {x.shape[1]} columns, the weights need {din}")
    T = x.shape[0]
    _buf(x, T * din * x.element_size(), "x", call)
    _buf(packed, E * N * K // 2, "packed", call)
    _buf(scales, E * N * K // block, "scales", call)
    _buf(offs, 4 * E, "offs", call)
    if offs.dtype != torch.int32:
        raise TypeError(f"{call}: offs must be int32")
    _buf(y, T * dout * x.element_size(), "y", call)


def mxq_grouped_mm_mxfp4(x, packed, scales, offs, y, transpose=False, stream=None) -> None:
    _gemm_bufs(x, packed, scales, offs, y, transpose, 32, "mxq_grouped_mm_mxfp4")
    E, N, K = packed.shape[0], packed.shape[1], packed.shape[2] * 2
    _check(lib.mxq_grouped_mm_mxfp4(_ptr(x), _dt(x.dtype), x.shape[0], _ptr(packed), _ptr(scales),
                                    E, N, K, _ptr(offs), int(bool(transpose)), _ptr(y),
                                    _stream(x, stream)),
           "mxq_grouped_mm_mxfp4")


def mxq_grouped_mm_nvfp4(x, packed, scales, row_scale, offs, y, transpose=False,
                         stream=None) -> None:
    _gemm_bufs(x, packed, scales, offs, y, transpose, 16, "mxq_grouped_mm_nvfp4")
    E, N, K = packed.shape[0], packed.shape[1], packed.shape[2] * 2
    _buf(row_scale, 4 * E * N, "row_scale", "mxq_grouped_mm_nvfp4")
    _check(lib.mxq_grouped_mm_nvfp4(_ptr(x), _dt(x.dtype), x.shape[0], _ptr(packed), _ptr(scales),
                                    _ptr(row_scale), E, N, K, _ptr(offs), int(bool(transpose)),
                                    _ptr(y), _stream(x, stream)),
           "mxq_grouped_mm_nvfp4")


def mxq_quantize_mxfp8(x, codes, scales, stream=None) -> None:
    K = x.shape[-1]
    n, c = _rows(x) * K, "mxq_quantize_mxfp8"
    _buf(x, x.numel() * x.element_size(), "x", c)
    _buf(codes, n, "codes", c)
    _buf(scales, n // 32, "scales", c)
    _check(lib.mxq_quantize_mxfp8(_ptr(x), _dt(x.dtype), _rows(x), K, _ptr(codes),
                                  _ptr(scales), _stream(x, stream)),
           "mxq_quantize_mxfp8")


def mxq_dequantize_mxfp8(codes, scales, y, stream=None) -> None:
    K = y.shape[-1]
    n, c = _rows(y) * K, "mxq_dequantize_mxfp8"
    _buf(y, y.numel() * y.element_size(), "y", c)
    _buf(codes, n, "codes", c)
    _buf(scales, n // 32, "scales", c)
    _check(lib.mxq_dequantize_mxfp8(_ptr(codes), _ptr(scales), _rows(y), K, _ptr(y),
                                    _dt(y.dtype), _stream(y, stream)),
           "mxq_dequantize_mxfp8")


def mxq_fake_quantize_fp4_static(x, block_amax, global_amax, y, block_size,
                                 stream=None) -> None:
    K = x.shape[-1]
    n, c = _rows(x) * K, "mxq_fake_quantize_fp4_static"
    _buf(x, x.numel() * x.element_size(), "x", c)
    if y.dtype != x.dtype:
        raise TypeError(f"{c}: y must have x's dtype")
    _buf(y, x.numel() * x.element_size(), "y", c)
    if block_size >= 1 and K % block_size == 0:
        _buf(block_amax, 4 * (n // block_size), "block_amax", c)
    if n:
        _buf(global_amax, 4, "global_amax", c)
    _check(lib.mxq_fake_quantize_fp4_static(_ptr(x), _dt(x.dtype), _rows(x), K,
                                            int(block_size), _ptr(block_amax),
                                            _ptr(global_amax), _ptr(y), _stream(x, stream)),
           "mxq_fake_quantize_fp4_static")


def mxq_dequantize_kv_pages_nvfp4(values_ptrs, scales_ptrs, amax_ptrs, block_tokens, y,
                                  stream=None) -> None:
    """values_ptrs / scales_ptrs / amax_ptrs: int64 device tensors holding one
    device address per cache block; y [blocks * block_tokens, heads, head_dim]
    (a leading batch dim of 1 is allowed)."""
    H, D = y.shape[-2], y.shape[-1]
    nb = values_ptrs.numel()
    c = "mxq_dequantize_kv_pages_nvfp4"
    for t, name in ((values_ptrs, "values_ptrs"), (scales_ptrs, "scales_ptrs"),
                    (amax_ptrs, "amax_ptrs")):
        _buf(t, 8 * nb, name, c)
    _buf(y, nb * int(block_tokens) * H * D * y.element_size(), "y", c)
    _check(lib.mxq_dequantize_kv_pages_nvfp4(_ptr(values_ptrs), _ptr(scales_ptrs), _ptr(amax_ptrs),
                                             nb, int(block_tokens), H, D, _ptr(y), _dt(y.dtype),
                                             _stream(y, stream)),
           "mxq_dequantize_kv_pages_nvfp4")


def mxq_quantize_kv_nvfp4(k, head_amax, packed, scales, row_scale, smooth=True,
                          stream=None) -> None:
    S, H, D = k.shape[-3], k.shape[-2], k.shape[-1]
    S = k.numel() // (H * D) if k.numel() else 0
    c = "mxq_quantize_kv_nvfp4"
    _buf(k, k.numel() * k.element_size(), "k", c)
    _buf(head_amax, 4 * H * KV_AMAX_SLOTS, "head_amax", c)
    _buf(packed, S * H * D // 2, "packed", c)
    _buf(scales, S * H * D // 16, "scales", c)
    _buf(row_scale, 4 * S * H, "row_scale", c)
    _check(lib.mxq_quantize_kv_nvfp4(_ptr(k), _dt(k.dtype), S, H, D, int(bool(smooth)),
                                     _ptr(head_amax), _ptr(packed), _ptr(scales),
                                     _ptr(row_scale), _stream(k, stream)),
           "mxq_quantize_kv_nvfp4")


def mxq_quantize_kv_nvfp4_noalloc(k, packed, scales, row_scale, smooth=True,
                                  stream=None) -> None:
    """mxq_quantize_kv_nvfp4 with the per-head scratch in the library's static
    device array (no workspace argument; at most NOALLOC_KV_MAX_HEADS heads)."""
    S, H, D = k.shape[-3], k.shape[-2], k.shape[-1]
    S = k.numel() // (H * D) if k.numel() else 0
    c = "mxq_quantize_kv_nvfp4_noalloc"
    _buf(k, k.numel() * k.element_size(), "k", c)
    _buf(packed, S * H * D // 2, "packed", c)
    _buf(scales, S * H * D // 16, "scales", c)
    _buf(row_scale, 4 * S * H, "row_scale", c)
    _check(lib.mxq_quantize_kv_nvfp4_noalloc(_ptr(k), _dt(k.dtype), S, H, D, int(bool(smooth)),
                                             _ptr(packed), _ptr(scales), _ptr(row_scale),
                                             _stream(k, stream)),
           c)


NOALLOC_KV_MAX_HEADS = 1024    # MXQ_NOALLOC_KV_MAX_HEADS


# ------------------------------------------------------------------ tensor API

def quantize_mxfp4(weight: torch.Tensor):
    """[..., K] (K % 32 == 0) -> (int8 packed [..., K//2],
    float8_e8m0fnu scales [..., K//32])."""
    K = weight.shape[-1]
    if K % MXFP4_BLOCK_SIZE:
        raise ValueError(f"last dim {K} is not divisible by {MXFP4_BLOCK_SIZE}")
    x = _dev_input(weight)
    packed = torch.empty(*x.shape[:-1], K // 2, dtype=torch.int8, device=x.device)
    scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8, device=x.device)
    mxq_quantize_mxfp4(x, packed, scales)
    return packed, scales.view(torch.float8_e8m0fnu)


def dequantize_mxfp4(packed: torch.Tensor, scales: torch.Tensor,
                     dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """(int8 [..., K//2], e8m0 [..., K//32]) -> [..., K] in dtype."""
    K = packed.shape[-1] * 2
    if (K % MXFP4_BLOCK_SIZE
            or tuple(scales.shape) != (*packed.shape[:-1], K // MXFP4_BLOCK_SIZE)):
        raise ValueError("packed/scales shapes do not describe 32-column blocks")
    p = _dev_input(packed.view(torch.int8))
    s = _dev_input(scales.view(torch.uint8))
    y = torch.empty(*p.shape[:-1], K, dtype=dtype, device=p.device)
    mxq_dequantize_mxfp4(p, s, y)
    return y


def _check_last_dim(k: int) -> None:
    if k % NVFP4_BLOCK_SIZE:
        raise ValueError(f"last dim {k} is not a whole number of "
                         f"{NVFP4_BLOCK_SIZE}-column blocks")


def quantize_nvfp4(weight: torch.Tensor, global_scale: torch.Tensor | None = None):
    """[..., K] -> (uint8 packed [..., K//2], float8_e4m3fn scales [..., K//16],
    float32 row scales [...]).  One scale per row (amax / (6 * 448)) unless
    ``global_scale`` (broadcastable to ``weight.shape[:-1]``) is given."""
    K = weight.shape[-1]
    _check_last_dim(K)
    x = _dev_input(weight)
    lead = tuple(x.shape[:-1])
    packed = torch.empty(*lead, K // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(*lead, K // 16, dtype=torch.uint8, device=x.device)
    row_scale = torch.empty(lead, dtype=torch.float32, device=x.device)
    if global_scale is None:
        mxq_quantize_nvfp4(x, packed, scales, row_scale, mode="row")
    else:
        g = global_scale.to(device=x.device, dtype=torch.float32)
        if g.numel() == 1:
            g, stride = g.reshape(1).contiguous(), 0
        else:
            g, stride = g.expand(lead).contiguous(), 1
        mxq_quantize_nvfp4(x, packed, scales, row_scale, mode="given",
                           given=g, given_stride=stride)
    return packed, scales.view(torch.float8_e4m3fn), row_scale


def quantize_nvfp4_modelopt(weight: torch.Tensor):
    """2-D [out, in] -> (uint8 [out, in//2], float8_e4m3fn [out, in//16],
    float32 scalar tensor scale amax / (6 * 448))."""
    if weight.dim() != 2:
        raise ValueError("quantize_nvfp4_modelopt takes a 2-D [out, in] matrix")
    K = weight.shape[-1]
    _check_last_dim(K)
    x = _dev_input(weight)
    packed = torch.empty(x.shape[0], K // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[0], K // 16, dtype=torch.uint8, device=x.device)
    row_scale = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    scratch = torch.empty(1, dtype=torch.float32, device=x.device)
    mxq_quantize_nvfp4(x, packed, scales, row_scale, mode="tensor", scratch=scratch)
    g = row_scale[0] if x.shape[0] else (scratch[0] * 0)
    return packed, scales.view(torch.float8_e4m3fn), g


def dequantize_nvfp4(packed: torch.Tensor, scales: torch.Tensor,
                     global_scale: torch.Tensor,
                     dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """(uint8/int8 [..., K//2], e4m3 [..., K//16], float32 [...]) -> [..., K]."""
    K = packed.shape[-1] * 2
    _check_last_dim(K)
    if tuple(scales.shape) != (*packed.shape[:-1], K // NVFP4_BLOCK_SIZE):
        raise ValueError("scales do not describe 16-column blocks of packed")
    try:
        torch.broadcast_shapes(tuple(global_scale.shape), tuple(packed.shape[:-1]))
    except RuntimeError:
        raise ValueError("global_scale does not broadcast to one value per row") from None
    p = _dev_input(packed.view(torch.uint8))
    s = _dev_input(scales.view(torch.uint8))
    g = global_scale.to(device=p.device, dtype=torch.float32)
    g = g.expand(p.shape[:-1]).contiguous()
    y = torch.empty(*p.shape[:-1], K, dtype=dtype, device=p.device)
    mxq_dequantize_nvfp4(p, s, g, y)
    return y


def quantize_cache(values: torch.Tensor, format: str, block_size: int) -> torch.Tensor:
    """Quantize/dequantize round trip of [..., channels] in groups of
    ``block_size`` channels; returns a new tensor with the input's shape and
    dtype.  format: 'fp8' | 'mxfp4' | 'nvfp4'."""
    if format not in FORMATS:
        raise ValueError(f"unknown cache format {format!r}")
    if block_size < 1:
        raise ValueError("block_size must be >= 1")
    x = values.contiguous()
    if x.device.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    y = torch.empty_like(x)
    mxq_quantize_cache(x, y, format, block_size)
    return y


def _grouped_mm_shapes(x, packed, scales, offs, block, row_scale=None) -> None:
    if x.dim() != 2 or packed.dim() != 3:
        raise ValueError("x must be [tokens, in_dim] and packed [experts, out_dim, in_dim // 2]")
    E, N, K = packed.shape[0], packed.shape[1], packed.shape[2] * 2
    if tuple(scales.shape) != (E, N, K // block):
        raise ValueError(f"scales must be [{E}, {N}, {K // block}], got {list(scales.shape)}")
    if row_scale is not None and tuple(row_scale.shape) != (E, N):
        raise ValueError(f"row_scale must be [{E}, {N}], got {list(row_scale.shape)}")
    if offs.numel() != E:
        raise ValueError(f"offs must hold one count per expert ({E}), got {offs.numel()}")


def _grouped_mm_out(x: torch.Tensor, packed: torch.Tensor, transpose: bool) -> torch.Tensor:
    N, K = packed.shape[1], packed.shape[2] * 2
    din, dout = (N, K) if transpose else (K, N)
    if x.shape[1] != din:
        raise ValueError(f"x has {x.shape[1]} columns, the weights need {din}")
    return torch.empty(x.shape[0], dout, dtype=x.dtype, device=x.device)


def grouped_mm_mxfp4(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                     offs: torch.Tensor, transpose: bool = False) -> torch.Tensor:
    """Grouped GEMM over MXFP4 expert weights ([mxfp4 page] MXFP4GroupedMM):
    x [tokens, K] grouped by expert (offs: int32 cumulative counts), packed
    [E, N, K // 2], scales [E, N, K // 32]; returns x @ W_e^T [tokens, N], or
    with transpose=True x [tokens, N] @ W_e, [tokens, K] (the backward product).
    Rows outside every group are left uninitialised."""
    _grouped_mm_shapes(x, packed, scales, offs, MXFP4_BLOCK_SIZE)
    x, packed, scales = _dev_input(x), _dev_input(packed), _dev_input(scales)
    offs = _dev_input(offs.to(torch.int32))
    y = _grouped_mm_out(x, packed, transpose)
    mxq_grouped_mm_mxfp4(x, packed, scales.view(torch.uint8), offs, y, transpose)
    return y


def grouped_mm_nvfp4(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                     row_scale: torch.Tensor, offs: torch.Tensor,
                     transpose: bool = False) -> torch.Tensor:
    """Grouped GEMM over NVFP4 expert weights ([nvfp4 page] NVFP4GroupedMM):
    as grouped_mm_mxfp4, with e4m3 scales [E, N, K // 16] and float32
    row_scale [E, N]."""
    _grouped_mm_shapes(x, packed, scales, offs, NVFP4_BLOCK_SIZE, row_scale)
    x, packed, scales = _dev_input(x), _dev_input(packed), _dev_input(scales)
    row_scale = _dev_input(row_scale.to(torch.float32))
    offs = _dev_input(offs.to(torch.int32))
    y = _grouped_mm_out(x, packed, transpose)
    mxq_grouped_mm_nvfp4(x, packed.view(torch.uint8), scales.view(torch.uint8), row_scale, offs,
                         y, transpose)
    return y


MXFP8_BLOCK_SIZE = 32
KV_AMAX_SLOTS = 32          # scratch words per head of mxq_quantize_kv_nvfp4


def quantize_mxfp8(weight: torch.Tensor):
    """[..., K] (K % 32 == 0) -> (float8_e4m3fn codes [..., K],
    float8_e8m0fnu scales [..., K//32]): the MX branch of ModelOpt's real
    quantization with e4m3 elements."""
    K = weight.shape[-1]
    if K % MXFP8_BLOCK_SIZE:
        raise ValueError(f"last dim {K} is not divisible by {MXFP8_BLOCK_SIZE}")
    x = _dev_input(weight)
    codes = torch.empty(*x.shape[:-1], K, dtype=torch.uint8, device=x.device)
    scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8, device=x.device)
    mxq_quantize_mxfp8(x, codes, scales)
    return codes.view(torch.float8_e4m3fn), scales.view(torch.float8_e8m0fnu)


def dequantize_mxfp8(codes: torch.Tensor, scales: torch.Tensor,
                     dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """(e4m3 [..., K], e8m0 [..., K//32]) -> [..., K] in dtype."""
    K = codes.shape[-1]
    if (K % MXFP8_BLOCK_SIZE
            or tuple(scales.shape) != (*codes.shape[:-1], K // MXFP8_BLOCK_SIZE)):
        raise ValueError("codes/scales shapes do not describe 32-column blocks")
    c = _dev_input(codes.view(torch.uint8))
    s = _dev_input(scales.view(torch.uint8))
    y = torch.empty(*c.shape, dtype=dtype, device=c.device)
    mxq_dequantize_mxfp8(c, s, y)
    return y


def fake_quantize_fp4_static(x: torch.Tensor, block_amax: torch.Tensor,
                             global_amax: torch.Tensor, block_size: int = 16) -> torch.Tensor:
    """Static two-level FP4 quantize/dequantize (ModelOpt's
    StaticBlockScaleQuantizer with FP8 block scales): x [..., K], block_amax
    with one float32 per ``block_size`` consecutive columns ([..., K //
    block_size]), global_amax one float32 (a device tensor); returns a new
    tensor with x's shape and dtype."""
    K = x.shape[-1]
    if block_size < 8 or block_size > 1024 or block_size & (block_size - 1):
        raise ValueError("block_size must be a power of two in [8, 1024]")
    if K % block_size:
        raise ValueError(f"last dim {K} is not a whole number of {block_size}-column blocks")
    xi = _dev_input(x)
    a = _dev_input(block_amax.to(device=xi.device, dtype=torch.float32))
    if a.numel() != xi.numel() // block_size:
        raise ValueError("block_amax must hold one value per block")
    g = global_amax.to(device=xi.device, dtype=torch.float32).reshape(1).contiguous()
    y = torch.empty_like(xi)
    mxq_fake_quantize_fp4_static(xi, a, g, y, block_size)
    return y


def _ptr_table(tensors, device) -> torch.Tensor:
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64).to(device)


def dequantize_kv_cache(values, scales, amax, block_tokens: int, num_heads: int,
                        dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Paged NVFP4 KV cache -> [1, blocks * block_tokens, num_heads, head_dim]
    (LongLive's dequantize_kv_cache with row-major scale bytes): values[b]
    uint8 [block_tokens * num_heads, head_dim // 2], scales[b] e4m3
    [block_tokens * num_heads, head_dim // 16], amax[b] one float32, all on
    the GPU; block b's global scale is amax[b] / (6 * 448)."""
    nb = len(values)
    if nb != len(scales) or nb != len(amax):
        raise ValueError("values, scales and amax must list the same blocks")
    if nb == 0:
        raise ValueError("the cache holds no block")
    D = values[0].shape[-1] * 2
    rows = block_tokens * num_heads
    for v, sc, a in zip(values, scales, amax):
        if v.device.type != "cuda" or sc.device.type != "cuda" or a.device.type != "cuda":
            raise ValueError("tensors must live on a GPU")
        if (v.numel() != rows * D // 2 or sc.numel() != rows * D // 16 or a.numel() != 1
                or not (v.is_contiguous() and sc.is_contiguous())
                or v.data_ptr() % 16 or sc.data_ptr() % 16 or a.dtype != torch.float32):
            raise ValueError("every block needs contiguous 16-byte aligned [rows, D/2] codes, "
                             "[rows, D/16] scales and one float32 amax")
    dev = values[0].device
    y = torch.empty(1, nb * block_tokens, num_heads, D, dtype=dtype, device=dev)
    vt, st, at = _ptr_table(values, dev), _ptr_table(scales, dev), _ptr_table(amax, dev)
    mxq_dequantize_kv_pages_nvfp4(vt, st, at, block_tokens, y)
    return y


def quantize_kv_nvfp4(k: torch.Tensor, smooth: bool = True):
    """Per-head NVFP4 of k [..., tokens, heads, head_dim] (LongLive's
    quantize_kv with the default NVFP4 scale rule; smooth=True applies
    k_smooth first).  Returns (uint8 packed [..., head_dim // 2], float8_e4m3fn
    scales [..., head_dim // 16], float32 row scales [..., tokens, heads])."""
    if k.dim() < 3:
        raise ValueError("k must be [..., tokens, heads, head_dim]")
    D = k.shape[-1]
    if D < 16 or D > 512 or D & (D - 1):
        raise ValueError("head_dim must be a power of two in [16, 512]")
    x = _dev_input(k)
    lead = tuple(x.shape[:-1])
    packed = torch.empty(*lead, D // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(*lead, D // 16, dtype=torch.uint8, device=x.device)
    row_scale = torch.empty(lead, dtype=torch.float32, device=x.device)
    head_amax = torch.empty(x.shape[-2] * KV_AMAX_SLOTS, dtype=torch.float32, device=x.device)
    mxq_quantize_kv_nvfp4(x, head_amax, packed, scales, row_scale, smooth)
    return packed, scales.view(torch.float8_e4m3fn), row_scale


def abi_version() -> int:
    return lib.mxq_abi_version()
