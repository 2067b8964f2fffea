"""Host build of the libmxq per-chunk arithmetic (see mxq_hostmath.cpp)."""
import ctypes
import os
import subprocess

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "mxq_hostmath.cpp")
HDR = os.path.join(ROOT, "fp8_quantize_pack_amd", "csrc", "mxq_device.h")
LIB = os.path.join(HERE, "libmxq_hostmath.so")
CXX = os.environ.get("MXQ_HOST_CXX", "/opt/rocm/llvm/bin/clang++")

_DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
_FMT = {"fp8": 0, "mxfp4": 1, "nvfp4": 2}
_MODE = {"row": 0, "given": 1, "tensor": 2}
_lib = None


def build():
    tmp = LIB + ".tmp"
    subprocess.run([CXX, "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-pthread", "-I", os.path.dirname(HDR), "-o", tmp, SRC],
                   check=True)
    os.replace(tmp, LIB)


def lib():
    global _lib
    if _lib is None:
        newest = max(os.path.getmtime(SRC), os.path.getmtime(HDR))
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < newest:
            build()
        L = ctypes.CDLL(LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.hm_quantize_mxfp4.argtypes = [vp, i32, i64, i64, vp, vp]
        L.hm_dequantize_mxfp4.argtypes = [vp, vp, i64, i64, vp, i32]
        L.hm_quantize_nvfp4.argtypes = [vp, i32, i64, i64, i32, vp, i64, vp, vp, vp]
        L.hm_dequantize_nvfp4.argtypes = [vp, vp, vp, i64, i64, vp, i32]
        L.hm_quantize_cache.argtypes = [vp, vp, i32, i64, i64, i32, i64]
        for f in ("hm_e4m3_encode_pos", "hm_e4m3_round_value", "hm_pow2_ceil", "hm_bf16_rne", "hm_f16_rne"):
            getattr(L, f).argtypes = [vp, i64, vp]
        L.hm_nv_division_stress.argtypes = [i64, ctypes.c_uint64, i32]
        L.hm_nv_division_stress.restype = i64
        L.hm_ceil22_check.argtypes = []
        L.hm_ceil22_check.restype = i64
        L.hm_scale_division_check.argtypes = []
        L.hm_scale_division_check.restype = i64
        L.hm_half_down_check.argtypes = []
        L.hm_half_down_check.restype = i64
        L.hm_rne_model_check.argtypes = []
        L.hm_rne_model_check.restype = i64
        _lib = L
    return _lib


def _rows(t):
    return t.numel() // t.shape[-1]


def quantize_mxfp4(x):
    x = x.contiguous(); K = x.shape[-1]
    p = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8)
    s = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8)
    lib().hm_quantize_mxfp4(x.data_ptr(), _DT[x.dtype], _rows(x), K, p.data_ptr(), s.data_ptr())
    return p, s


def dequantize_mxfp4(p, s, dtype):
    p, s = p.contiguous(), s.contiguous(); K = p.shape[-1] * 2
    y = torch.empty(*p.shape[:-1], K, dtype=dtype)
    lib().hm_dequantize_mxfp4(p.data_ptr(), s.data_ptr(), _rows(p), K, y.data_ptr(), _DT[dtype])
    return y


def quantize_nvfp4(x, mode="row", given=None):
    x = x.contiguous(); K = x.shape[-1]; R = _rows(x)
    p = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8)
    s = torch.empty(*x.shape[:-1], K // 16, dtype=torch.uint8)
    g = torch.empty(*x.shape[:-1], dtype=torch.float32)
    gp, gs = None, 0
    if mode == "given":
        given = given.to(torch.float32).contiguous()
        gs = 0 if given.numel() == 1 else 1
        gp = given.data_ptr()
    lib().hm_quantize_nvfp4(x.data_ptr(), _DT[x.dtype], R, K, _MODE[mode], gp, gs,
                            p.data_ptr(), s.data_ptr(), g.data_ptr())
    return p, s, g


def dequantize_nvfp4(p, s, g, dtype):
    p, s = p.contiguous(), s.contiguous(); g = g.to(torch.float32).contiguous()
    K = p.shape[-1] * 2
    y = torch.empty(*p.shape[:-1], K, dtype=dtype)
    lib().hm_dequantize_nvfp4(p.data_ptr(), s.data_ptr(), g.data_ptr(), _rows(p), K,
                              y.data_ptr(), _DT[dtype])
    return y


def quantize_cache(x, fmt, B):
    x = x.contiguous(); y = torch.empty_like(x)
    lib().hm_quantize_cache(x.data_ptr(), y.data_ptr(), _DT[x.dtype], _rows(x), x.shape[-1],
                            _FMT[fmt], B)
    return y


def apply(fn_name, x, out_dtype):
    x = x.contiguous(); y = torch.empty(x.shape, dtype=out_dtype)
    getattr(lib(), fn_name)(x.data_ptr(), x.numel(), y.data_ptr())
    return y
