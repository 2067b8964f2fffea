"""CPU oracle for block-scaled microscaling quantization.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``fp8_quantize_pack_amd``) never imports it and shares no code with it.

The arithmetic lives in ``mxq_oracle.c`` (plain scalar C, one element at a
time, in the order the source pages state each step; see the header of that
file for the citations and the readings of open points), the grouped GEMM
included.  This module builds it with gcc and marshals torch CPU tensors to it;
it does no arithmetic itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_mxq.so")

CFLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
          "-fexcess-precision=standard", "-fopenmp", "-fPIC", "-shared"]

_DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
_FMT = {"fp8": 0, "mxfp4": 1, "nvfp4": 2}
_MODE = {"row": 0, "given": 1, "tensor": 2}

_lib = None


def build() -> str:
    """Compile the oracle into ``liboracle_mxq.so`` (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if (not os.path.exists(LIB_PATH)
                or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint32]
        L.orc_e2m1_round_mag.restype = ctypes.c_uint32
        L.orc_e2m1_round_mag.argtypes = [ctypes.c_float]
        L.orc_round_binary.restype = ctypes.c_double
        L.orc_round_binary.argtypes = [ctypes.c_double, i32, i32]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint32]
        L.orc_e4m3_encode.restype = ctypes.c_uint32
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e8m0_decode.restype = ctypes.c_double
        L.orc_e8m0_decode.argtypes = [ctypes.c_uint32]
        L.orc_pow2_ceil.restype = ctypes.c_float
        L.orc_pow2_ceil.argtypes = [ctypes.c_float]
        L.orc_floor_log2.restype = i32
        L.orc_floor_log2.argtypes = [ctypes.c_float]
        L.orc_quantize_mxfp4.restype = None
        L.orc_quantize_mxfp4.argtypes = [vp, i32, i64, i64, vp, vp]
        L.orc_dequantize_mxfp4.restype = None
        L.orc_dequantize_mxfp4.argtypes = [vp, vp, i64, i64, vp, i32]
        L.orc_quantize_nvfp4.restype = None
        L.orc_quantize_nvfp4.argtypes = [vp, i32, i64, i64, i32, vp, i64,
                                         vp, vp, vp]
        L.orc_dequantize_nvfp4.restype = None
        L.orc_dequantize_nvfp4.argtypes = [vp, vp, vp, i64, i64, vp, i32]
        L.orc_quantize_cache.restype = None
        L.orc_quantize_cache.argtypes = [vp, vp, i32, i64, i64, i32, i64]
        L.orc_quantize_mxfp8.restype = None
        L.orc_quantize_mxfp8.argtypes = [vp, i32, i64, i64, vp, vp]
        L.orc_dequantize_mxfp8.restype = None
        L.orc_dequantize_mxfp8.argtypes = [vp, vp, i64, i64, vp, i32]
        L.orc_static_block_scale.restype = ctypes.c_float
        L.orc_static_block_scale.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_fake_quantize_fp4_static.restype = None
        L.orc_fake_quantize_fp4_static.argtypes = [vp, i32, i64, i64, i64, vp,
                                                   ctypes.c_float, vp]
        L.orc_dequantize_kv_pages.restype = None
        L.orc_dequantize_kv_pages.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, i32]
        L.orc_k_smooth_row.restype = None
        L.orc_k_smooth_row.argtypes = [vp, i64, i32]
        L.orc_quantize_kv_nvfp4.restype = None
        L.orc_quantize_kv_nvfp4.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp]
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [i32]
        L.orc_max_threads.restype = i32
        L.orc_max_threads.argtypes = []
        L.orc_grouped_mm.restype = None
        L.orc_grouped_mm.argtypes = [vp, i32, i64, vp, i32, i64, i64, i64, vp, i32,
                                     vp, i64, vp, vp]
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads of the oracle's row loops (OpenMP, static schedule over rows;
    the results do not depend on the count)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- helpers

def _cpu(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError("the oracle takes CPU tensors")
    return t.contiguous()


def _rows(shape, K):
    n = 1
    for s in shape[:-1]:
        n *= s
    return n


# ---------------------------------------------------------------- primitives

def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(code)


def e2m1_round_mag(q: float) -> int:
    return lib().orc_e2m1_round_mag(q)


def round_binary(v: float, p: int, emin: int) -> float:
    return lib().orc_round_binary(v, p, emin)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def e4m3_decode(b: int) -> float:
    return lib().orc_e4m3_decode(b)


def e8m0_decode(b: int) -> float:
    return lib().orc_e8m0_decode(b)


def pow2_ceil(v: float) -> float:
    return lib().orc_pow2_ceil(v)


def floor_log2(a: float) -> int:
    return lib().orc_floor_log2(a)


# ---------------------------------------------------------------- operations

def quantize_mxfp4(x: torch.Tensor):
    """[..., K] -> (uint8 packed [..., K//2], uint8 e8m0 scale bytes [..., K//32])."""
    x = _cpu(x)
    K = x.shape[-1]
    assert K % 32 == 0
    R = _rows(x.shape, K)
    packed = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8)
    scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8)
    lib().orc_quantize_mxfp4(x.data_ptr(), _DT[x.dtype], R, K,
                             packed.data_ptr(), scales.data_ptr())
    return packed, scales


def dequantize_mxfp4(packed: torch.Tensor, scales: torch.Tensor,
                     dtype: torch.dtype) -> torch.Tensor:
    packed, scales = _cpu(packed), _cpu(scales)
    K = packed.shape[-1] * 2
    R = _rows(packed.shape, K)
    y = torch.empty(*packed.shape[:-1], K, dtype=dtype)
    lib().orc_dequantize_mxfp4(packed.data_ptr(), scales.data_ptr(), R, K,
                               y.data_ptr(), _DT[dtype])
    return y


def quantize_nvfp4(x: torch.Tensor, mode: str = "row",
                   given: torch.Tensor | None = None):
    """[..., K] -> (uint8 packed [..., K//2], uint8 e4m3 bytes [..., K//16],
    float32 row scales [...]).  mode: 'row' | 'given' | 'tensor'."""
    x = _cpu(x)
    K = x.shape[-1]
    assert K % 16 == 0
    R = _rows(x.shape, K)
    packed = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8)
    scales = torch.empty(*x.shape[:-1], K // 16, dtype=torch.uint8)
    row_scale = torch.empty(*x.shape[:-1], dtype=torch.float32)
    gptr, gstride = None, 0
    if mode == "given":
        given = _cpu(given.to(torch.float32))
        if given.numel() == 1:
            gstride = 0
        else:
            assert given.numel() == R
            gstride = 1
        gptr = given.data_ptr()
    lib().orc_quantize_nvfp4(x.data_ptr(), _DT[x.dtype], R, K, _MODE[mode],
                             gptr, gstride, packed.data_ptr(),
                             scales.data_ptr(), row_scale.data_ptr())
    return packed, scales, row_scale


def dequantize_nvfp4(packed: torch.Tensor, scales: torch.Tensor,
                     row_scale: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    packed, scales = _cpu(packed), _cpu(scales)
    row_scale = _cpu(row_scale.to(torch.float32))
    K = packed.shape[-1] * 2
    R = _rows(packed.shape, K)
    assert row_scale.numel() == R
    y = torch.empty(*packed.shape[:-1], K, dtype=dtype)
    lib().orc_dequantize_nvfp4(packed.data_ptr(), scales.data_ptr(),
                               row_scale.data_ptr(), R, K, y.data_ptr(),
                               _DT[dtype])
    return y


def quantize_cache(x: torch.Tensor, fmt: str, block_size: int) -> torch.Tensor:
    """Quantize/dequantize round trip; same shape and dtype as x."""
    x = _cpu(x)
    C = x.shape[-1]
    R = _rows(x.shape, C)
    y = torch.empty_like(x)
    lib().orc_quantize_cache(x.data_ptr(), y.data_ptr(), _DT[x.dtype], R, C,
                             _FMT[fmt], block_size)
    return y


def quantize_mxfp8(x: torch.Tensor):
    """[..., K] -> (uint8 e4m3 codes [..., K], uint8 e8m0 scale bytes [..., K//32])."""
    x = _cpu(x)
    K = x.shape[-1]
    assert K % 32 == 0
    R = _rows(x.shape, K)
    codes = torch.empty(*x.shape[:-1], K, dtype=torch.uint8)
    scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8)
    lib().orc_quantize_mxfp8(x.data_ptr(), _DT[x.dtype], R, K, codes.data_ptr(),
                             scales.data_ptr())
    return codes, scales


def dequantize_mxfp8(codes: torch.Tensor, scales: torch.Tensor,
                     dtype: torch.dtype) -> torch.Tensor:
    codes, scales = _cpu(codes), _cpu(scales)
    K = codes.shape[-1]
    R = _rows(codes.shape, K)
    y = torch.empty(*codes.shape[:-1], K, dtype=dtype)
    lib().orc_dequantize_mxfp8(codes.data_ptr(), scales.data_ptr(), R, K,
                               y.data_ptr(), _DT[dtype])
    return y


def static_block_scale(a: float, global_amax: float) -> float:
    """Dequantization-side block scale of the static two-level FP4 rule."""
    return lib().orc_static_block_scale(a, global_amax)


def fake_quantize_fp4_static(x: torch.Tensor, block_amax: torch.Tensor,
                             global_amax: float, block: int) -> torch.Tensor:
    """Static two-level FP4 quantize/dequantize; same shape and dtype as x.
    block_amax holds one float32 per `block` consecutive columns."""
    x = _cpu(x)
    K = x.shape[-1]
    assert K % block == 0
    R = _rows(x.shape, K)
    a = _cpu(block_amax.to(torch.float32)).reshape(-1)
    assert a.numel() == R * (K // block)
    y = torch.empty_like(x)
    lib().orc_fake_quantize_fp4_static(x.data_ptr(), _DT[x.dtype], R, K, block,
                                       a.data_ptr(), float(global_amax), y.data_ptr())
    return y


def dequantize_kv_pages(values, scales, amax, block_tokens: int, heads: int,
                        dtype: torch.dtype) -> torch.Tensor:
    """Blocks of a paged NVFP4 KV cache (lists of per-block tensors: uint8
    [block_tokens*heads, D//2], uint8 [block_tokens*heads, D//16], one float
    amax each) -> [1, nblocks*block_tokens, heads, D]."""
    nb = len(values)
    values = [_cpu(v) for v in values]
    scales = [_cpu(s) for s in scales]
    D = values[0].shape[-1] * 2
    vp = (ctypes.c_void_p * nb)(*[v.data_ptr() for v in values])
    sp = (ctypes.c_void_p * nb)(*[s.data_ptr() for s in scales])
    am = _cpu(torch.as_tensor([float(a) for a in amax], dtype=torch.float32))
    y = torch.empty(1, nb * block_tokens, heads, D, dtype=dtype)
    lib().orc_dequantize_kv_pages(ctypes.cast(vp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                                  am.data_ptr(), nb, block_tokens, heads, D,
                                  y.data_ptr(), _DT[dtype])
    return y


def k_smooth(x: torch.Tensor) -> torch.Tensor:
    """k - mean(k, -1) in x's dtype (pairwise binary32 mean, rounded)."""
    x = _cpu(x)
    D = x.shape[-1]
    rows = x.to(torch.float32).reshape(-1, D).contiguous()
    L = lib()
    for r in range(rows.shape[0]):
        L.orc_k_smooth_row(rows[r].data_ptr(), D, _DT[x.dtype])
    return rows.reshape(x.shape).to(x.dtype)


def quantize_kv_nvfp4(k: torch.Tensor, smooth: bool = True):
    """k [S, H, D] (or [1, S, H, D]) -> (uint8 packed [..., D//2], uint8 e4m3
    bytes [..., D//16], float32 row scales [..., S, H]), one NVFP4 global
    scale per head."""
    k = _cpu(k)
    S, H, D = k.shape[-3:]
    lead = k.shape[:-1]
    packed = torch.empty(*lead, D // 2, dtype=torch.uint8)
    scales = torch.empty(*lead, D // 16, dtype=torch.uint8)
    row_scale = torch.empty(*lead, dtype=torch.float32)
    lib().orc_quantize_kv_nvfp4(k.data_ptr(), _DT[k.dtype], S, H, D, int(bool(smooth)),
                                packed.data_ptr(), scales.data_ptr(), row_scale.data_ptr())
    return packed, scales, row_scale


def grouped_mm(x: torch.Tensor, w: torch.Tensor, offs: torch.Tensor, trans: bool,
               rows=None):
    """Grouped GEMM of activations x [T, D_in] with dequantized expert weights
    w [E, N, K] (in the activation dtype), rows grouped by the cumulative
    counts offs [E]: forward (trans False) x @ W_e^T, backward (trans True)
    x @ W_e.  Only the given rows (all by default) are computed.  Returns
    (out, absout) in float64: the sums and the sums of |products|."""
    x, w = _cpu(x).contiguous(), _cpu(w).contiguous()
    offs = _cpu(offs.to(torch.int32)).contiguous()
    T, din = x.shape
    E, N, K = w.shape
    assert din == (N if trans else K) and offs.numel() == E
    rows = torch.arange(T, dtype=torch.int64) if rows is None else _cpu(torch.as_tensor(rows, dtype=torch.int64)).contiguous()
    dout = K if trans else N
    out = torch.empty(rows.numel(), dout, dtype=torch.float64)
    absout = torch.empty_like(out)
    lib().orc_grouped_mm(x.data_ptr(), _DT[x.dtype], T, w.data_ptr(), _DT[w.dtype], E, N, K,
                         offs.data_ptr(), int(bool(trans)), rows.data_ptr(), rows.numel(),
                         out.data_ptr(), absout.data_ptr())
    return out, absout


def store_values(v: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """Round float32 values to dtype through the oracle's store routine."""
    v = _cpu(v.to(torch.float32)).reshape(-1)
    L = lib()
    L.orc_store.restype = None
    L.orc_store.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float]
    y = torch.empty(v.numel(), dtype=dtype)
    for i in range(v.numel()):
        L.orc_store(y.data_ptr(), _DT[dtype], i, float(v[i]))
    return y
