"""The C ABI on a machine without a GPU: the library loads, exports every
function include/mxq.h declares, and rejects bad arguments with the documented
status before touching the device (no compute calls are made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="mxq.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_operations():
    names = _declared_functions()
    for n in ("mxq_quantize_mxfp4", "mxq_dequantize_mxfp4", "mxq_quantize_nvfp4",
              "mxq_dequantize_nvfp4", "mxq_quantize_cache", "mxq_grouped_mm_mxfp4",
              "mxq_grouped_mm_nvfp4", "mxq_quantize_mxfp8", "mxq_dequantize_mxfp8",
              "mxq_fake_quantize_fp4_static", "mxq_dequantize_kv_pages_nvfp4",
              "mxq_quantize_kv_nvfp4", "mxq_quantize_kv_nvfp4_noalloc", "mxq_status_string",
              "mxq_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import fp8_quantize_pack_amd as mxq
    for n in _declared_functions():
        assert hasattr(mxq.lib, n), n
    assert mxq.abi_version() == 2


@pytest.fixture(scope="module")
def L():
    import fp8_quantize_pack_amd as mxq
    return mxq.lib


FAKE = 1 << 20     # an aligned non-null address; never dereferenced here


def test_quantize_mxfp4_validation(L):
    f = L.mxq_quantize_mxfp4
    assert f(FAKE, 1, 4, 48, FAKE, FAKE, None) == 2           # K % 32
    assert f(FAKE, 1, -1, 64, FAKE, FAKE, None) == 2          # rows < 0
    assert f(FAKE, 7, 4, 64, FAKE, FAKE, None) == 3           # dtype
    assert f(FAKE, 1, 1 << 40, 1 << 30, FAKE, FAKE, None) == 6  # overflow
    assert f(None, 1, 4, 64, FAKE, FAKE, None) == 1
    assert f(FAKE, 1, 4, 64, None, FAKE, None) == 1
    assert f(FAKE + 2, 1, 4, 64, FAKE, FAKE, None) == 9       # alignment
    assert f(None, 1, 0, 64, None, None, None) == 0           # empty: no launch
    assert f(None, 1, 5, 0, None, None, None) == 0


def test_dequantize_mxfp4_validation(L):
    f = L.mxq_dequantize_mxfp4
    assert f(FAKE, FAKE, 4, 40, FAKE, 1, None) == 2
    assert f(FAKE, FAKE, 4, 64, FAKE, 9, None) == 3
    assert f(FAKE, None, 4, 64, FAKE, 1, None) == 1
    assert f(FAKE, FAKE, 4, 64, FAKE + 8, 1, None) == 9
    assert f(None, None, 0, 64, None, 1, None) == 0


def test_quantize_nvfp4_validation(L):
    f = L.mxq_quantize_nvfp4
    args = lambda **k: dict(dict(x=FAKE, dt=1, rows=4, K=64, mode=0, given=None, gs=1,
                                 scratch=None, p=FAKE, s=FAKE, rs=FAKE, st=None), **k)
    call = lambda a: f(a["x"], a["dt"], a["rows"], a["K"], a["mode"], a["given"], a["gs"],
                       a["scratch"], a["p"], a["s"], a["rs"], a["st"])
    assert call(args(K=40)) == 2                      # not a whole number of 16-col blocks
    assert call(args(dt=5)) == 3
    assert call(args(mode=3)) == 8
    assert call(args(mode=1, given=None)) == 1
    assert call(args(mode=1, given=FAKE, gs=2)) == 2
    assert call(args(mode=2, scratch=None)) == 1
    assert call(args(rs=None)) == 1
    assert call(args(x=FAKE + 4)) == 9
    assert call(args(rows=0, x=None, p=None, s=None, rs=None)) == 0


def test_quantize_cache_validation(L):
    f = L.mxq_quantize_cache
    assert f(FAKE, FAKE, 1, 4, 64, 3, 32, None) == 4   # format
    assert f(FAKE, FAKE, 1, 4, 64, 0, 0, None) == 5    # block size
    assert f(FAKE, FAKE, 4, 4, 64, 0, 32, None) == 3   # dtype
    assert f(None, FAKE, 1, 4, 64, 0, 32, None) == 1
    assert f(None, None, 1, 0, 64, 0, 32, None) == 0
    assert f(FAKE, FAKE, 1, -2, 64, 0, 32, None) == 2


def test_grouped_mm_validation(L):
    f, g = L.mxq_grouped_mm_mxfp4, L.mxq_grouped_mm_nvfp4
    # x, dt, tokens, packed, scales, E, N, K, offs, transpose, y, stream
    ok = dict(x=FAKE, dt=1, T=64, p=FAKE, s=FAKE, E=4, N=256, K=512, offs=FAKE, tr=0, y=FAKE)
    call = lambda **k: f(*[dict(ok, **k)[n] for n in ("x", "dt", "T", "p", "s", "E", "N", "K",
                                                          "offs", "tr", "y")], None)
    assert call(N=200) == 2 and call(K=96) == 2 and call(T=-1) == 2   # N, K multiples of 128
    assert call(dt=0) == 3 and call(dt=2) == 3                         # bfloat16 only
    assert call(tr=2) == 8
    assert call(offs=None) == 1 and call(y=None) == 1
    assert call(x=FAKE + 2) == 9 and call(p=FAKE + 8) == 9
    assert call(T=0, x=None, p=None, s=None, offs=None, y=None) == 0   # empty: no launch
    assert call(E=0) == 0
    assert g(FAKE, 1, 64, FAKE, FAKE, None, 4, 256, 512, FAKE, 0, FAKE, None) == 1  # row_scale


def test_mxfp8_validation(L):
    q, d = L.mxq_quantize_mxfp8, L.mxq_dequantize_mxfp8
    assert q(FAKE, 1, 4, 48, FAKE, FAKE, None) == 2           # K % 32
    assert q(FAKE, 3, 4, 64, FAKE, FAKE, None) == 3
    assert q(FAKE, 1, 1 << 40, 1 << 30, FAKE, FAKE, None) == 6
    assert q(FAKE, 1, 4, 64, FAKE, None, None) == 1
    assert q(FAKE, 1, 4, 64, FAKE + 8, FAKE, None) == 9       # codes alignment
    assert q(None, 1, 0, 64, None, None, None) == 0
    assert d(FAKE, FAKE, 4, 16, FAKE, 1, None) == 2
    assert d(FAKE, FAKE, 4, 64, FAKE, 5, None) == 3
    assert d(None, FAKE, 4, 64, FAKE, 1, None) == 1
    assert d(FAKE, FAKE, 4, 64, FAKE + 2, 1, None) == 9
    assert d(None, None, 3, 0, None, 1, None) == 0


def test_fp4_static_validation(L):
    f = L.mxq_fake_quantize_fp4_static
    # x, dt, rows, K, block, block_amax, global_amax, y, stream
    assert f(FAKE, 1, 4, 64, 12, FAKE, FAKE, FAKE, None) == 5     # not a power of two
    assert f(FAKE, 1, 4, 64, 4, FAKE, FAKE, FAKE, None) == 5      # below 8
    assert f(FAKE, 1, 4, 4096, 2048, FAKE, FAKE, FAKE, None) == 5 # above 1024
    assert f(FAKE, 1, 4, 48, 32, FAKE, FAKE, FAKE, None) == 2     # K % block
    assert f(FAKE, 2 + 5, 4, 64, 16, FAKE, FAKE, FAKE, None) == 3
    assert f(FAKE, 1, 4, 64, 16, FAKE, None, FAKE, None) == 1
    assert f(FAKE, 1, 4, 64, 16, None, FAKE, FAKE, None) == 1
    assert f(FAKE + 4, 1, 4, 64, 16, FAKE, FAKE, FAKE, None) == 9
    assert f(None, 1, 0, 64, 16, None, None, None, None) == 0


def test_kv_validation(L):
    d, q = L.mxq_dequantize_kv_pages_nvfp4, L.mxq_quantize_kv_nvfp4
    # values, scales, amax, nb, bt, H, D, y, ydt, stream
    assert d(FAKE, FAKE, FAKE, 4, 16, 8, 120, FAKE, 1, None) == 2     # D % 16
    assert d(FAKE, FAKE, FAKE, -1, 16, 8, 128, FAKE, 1, None) == 2
    assert d(FAKE, FAKE, FAKE, 4, 16, 8, 128, FAKE, 7, None) == 3
    assert d(None, FAKE, FAKE, 4, 16, 8, 128, FAKE, 1, None) == 1
    assert d(FAKE, FAKE, None, 4, 16, 8, 128, FAKE, 1, None) == 1
    assert d(FAKE, FAKE, FAKE, 4, 16, 8, 128, FAKE + 2, 1, None) == 9
    assert d(FAKE, FAKE, FAKE, 1 << 30, 1 << 20, 1 << 10, 128, FAKE, 1, None) == 6
    assert d(None, None, None, 0, 16, 8, 128, None, 1, None) == 0
    # k, dt, S, H, D, smooth, head_amax, packed, scales, row_scale, stream
    assert q(FAKE, 1, 64, 8, 96, 1, FAKE, FAKE, FAKE, FAKE, None) == 2   # not a power of two
    assert q(FAKE, 1, 64, 8, 8, 1, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert q(FAKE, 1, 64, 8, 1024, 1, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert q(FAKE, 1, 64, 5000, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert q(FAKE, 1, 64, 8, 128, 2, FAKE, FAKE, FAKE, FAKE, None) == 8
    assert q(FAKE, 9, 64, 8, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert q(FAKE, 1, 64, 8, 128, 1, None, FAKE, FAKE, FAKE, None) == 1
    assert q(FAKE + 4, 1, 64, 8, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == 9
    assert q(None, 1, 0, 8, 128, 1, None, None, None, None, None) == 0


def test_status_strings(L):
    for s in range(11):
        assert L.mxq_status_string(s)
    assert L.mxq_status_string(99) == b"unknown status"


def test_python_wrapper_raises_page_errors_on_cpu_tensors():
    import torch
    import fp8_quantize_pack_amd as mxq
    with pytest.raises(ValueError, match="divisible by 32"):
        mxq.quantize_mxfp4(torch.zeros(2, 48))
    with pytest.raises(ValueError, match="16-column blocks"):
        mxq.quantize_nvfp4(torch.zeros(2, 40))
    with pytest.raises(ValueError, match="GPU"):
        mxq.quantize_mxfp4(torch.zeros(2, 64))
    with pytest.raises(ValueError, match="cache format"):
        mxq.quantize_cache(torch.zeros(2, 64), "int4", 32)


def test_python_wrappers_of_the_newer_calls_check_their_arguments():
    import torch
    import fp8_quantize_pack_amd as mxq
    with pytest.raises(ValueError, match="divisible by 32"):
        mxq.quantize_mxfp8(torch.zeros(2, 48))
    with pytest.raises(ValueError, match="32-column blocks"):
        mxq.dequantize_mxfp8(torch.zeros(2, 64, dtype=torch.uint8), torch.zeros(2, 3, dtype=torch.uint8))
    with pytest.raises(ValueError, match="power of two"):
        mxq.fake_quantize_fp4_static(torch.zeros(2, 48), torch.zeros(2, 4), torch.ones(1), 12)
    with pytest.raises(ValueError, match="whole number"):
        mxq.fake_quantize_fp4_static(torch.zeros(2, 48), torch.zeros(2, 4), torch.ones(1), 32)
    with pytest.raises(ValueError, match="power of two"):
        mxq.quantize_kv_nvfp4(torch.zeros(4, 2, 96))
    with pytest.raises(ValueError, match="tokens, heads, head_dim"):
        mxq.quantize_kv_nvfp4(torch.zeros(4, 128))
    with pytest.raises(ValueError, match="same blocks"):
        mxq.dequantize_kv_cache([torch.zeros(4, 64, dtype=torch.uint8)], [], [], 2, 2)
    with pytest.raises(ValueError, match="GPU"):
        mxq.dequantize_kv_cache([torch.zeros(4, 64, dtype=torch.uint8)],
                                [torch.zeros(4, 8, dtype=torch.uint8)], [torch.ones(1)], 2, 2)
    with pytest.raises(ValueError, match="GPU"):
        mxq.quantize_mxfp8(torch.zeros(2, 64))



def test_tensor_api_rejects_mismatched_scale_and_offs_shapes():
    """Short scale arrays, row scales or offs would make a kernel read past
    its allocation; the binding rejects them before anything is launched."""
    import torch
    import fp8_quantize_pack_amd as mxq
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    with pytest.raises(ValueError, match="32-column blocks"):
        mxq.dequantize_mxfp4(u8(8, 32), u8(4, 2))             # fewer scale rows
    with pytest.raises(ValueError, match="32-column blocks"):
        mxq.dequantize_mxfp4(u8(2, 4, 32), u8(8, 2))          # same numel, other shape
    with pytest.raises(ValueError, match="16-column blocks"):
        mxq.dequantize_nvfp4(u8(8, 32), u8(7, 4), torch.ones(8))
    with pytest.raises(ValueError, match="one value per row"):
        mxq.dequantize_nvfp4(u8(8, 32), u8(8, 4), torch.ones(5))
    with pytest.raises(ValueError, match="32-column blocks"):
        mxq.dequantize_mxfp8(u8(8, 64), u8(3, 2))
    x = torch.zeros(64, 256, dtype=torch.bfloat16)
    pk = u8(4, 128, 128)                                      # E=4, N=128, K=256
    offs = torch.full((4,), 64, dtype=torch.int32)
    with pytest.raises(ValueError, match="scales must be"):
        mxq.grouped_mm_mxfp4(x, pk, u8(4, 128, 4), offs)
    with pytest.raises(ValueError, match="one count per expert"):
        mxq.grouped_mm_mxfp4(x, pk, u8(4, 128, 8), offs[:3])
    with pytest.raises(ValueError, match="scales must be"):
        mxq.grouped_mm_nvfp4(x, pk, u8(4, 128, 8), torch.ones(4, 128), offs)
    with pytest.raises(ValueError, match="row_scale must be"):
        mxq.grouped_mm_nvfp4(x, pk, u8(4, 128, 16), torch.ones(4, 64), offs)
    with pytest.raises(ValueError, match="one count per expert"):
        mxq.grouped_mm_nvfp4(x, pk, u8(4, 128, 16), torch.ones(4, 128), offs[:2])


def test_c_abi_wrappers_check_every_buffer_size():
    """The one-to-one wrappers compute the byte count each buffer must hold
    and reject a short or long one before the call (so a caller-allocated
    output that is too small never reaches a kernel)."""
    import torch
    import fp8_quantize_pack_amd as mxq
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    x = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="packed holds 255 bytes"):
        mxq.mxq_quantize_mxfp4(x, u8(255), u8(16))
    with pytest.raises(ValueError, match="scales holds"):
        mxq.mxq_quantize_mxfp4(x, u8(256), u8(15))
    with pytest.raises(ValueError, match="row_scale holds"):
        mxq.mxq_quantize_nvfp4(x, u8(256), u8(32), torch.zeros(7))
    with pytest.raises(ValueError, match="given holds"):
        mxq.mxq_quantize_nvfp4(x, u8(256), u8(32), torch.zeros(8), mode="given",
                               given=torch.ones(4), given_stride=1)
    with pytest.raises(ValueError, match="scratch is required"):
        mxq.mxq_quantize_nvfp4(x, u8(256), u8(32), torch.zeros(8), mode="tensor")
    with pytest.raises(ValueError, match="unknown NVFP4 mode"):
        mxq.mxq_quantize_nvfp4(x, u8(256), u8(32), torch.zeros(8), mode="col")
    with pytest.raises(ValueError, match="scales holds"):
        mxq.mxq_dequantize_nvfp4(u8(256), u8(31), torch.zeros(8), x)
    with pytest.raises(ValueError, match="y holds"):
        mxq.mxq_quantize_cache(x, torch.zeros(8, 63, dtype=torch.bfloat16), "fp8", 32)
    with pytest.raises(TypeError, match="x's dtype"):
        mxq.mxq_quantize_cache(x, torch.zeros(8, 64), "fp8", 32)
    with pytest.raises(ValueError, match="codes holds"):
        mxq.mxq_quantize_mxfp8(x, u8(511), u8(16))
    with pytest.raises(ValueError, match="block_amax holds"):
        mxq.mxq_fake_quantize_fp4_static(x, torch.zeros(31), torch.ones(1), x.clone(), 16)
    with pytest.raises(ValueError, match="head_amax holds"):
        mxq.mxq_quantize_kv_nvfp4(torch.zeros(4, 2, 64, dtype=torch.bfloat16), torch.zeros(63),
                                  u8(256), u8(32), torch.zeros(8))
    with pytest.raises(ValueError, match="must be contiguous"):
        mxq.mxq_quantize_mxfp4(x, u8(512)[::2], u8(16))
    with pytest.raises(ValueError, match="GPU"):
        mxq.mxq_quantize_mxfp4(x, u8(256), u8(16))
    pk = u8(4, 128, 128)
    with pytest.raises(ValueError, match="offs holds"):
        mxq.mxq_grouped_mm_mxfp4(torch.zeros(64, 256, dtype=torch.bfloat16), pk, u8(4, 128, 8),
                                 torch.zeros(3, dtype=torch.int32),
                                 torch.zeros(64, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y holds"):
        mxq.mxq_grouped_mm_nvfp4(torch.zeros(64, 256, dtype=torch.bfloat16), pk, u8(4, 128, 16),
                                 torch.ones(4, 128), torch.zeros(4, dtype=torch.int32),
                                 torch.zeros(64, 256, dtype=torch.bfloat16))


def test_every_header_is_covered():
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == \
        ["mxq.h", "mxq_roofline.h"]


def test_roofline_library_exports_and_validation():
    """The streaming reference kernels (measurement only): every declared
    symbol is exported, and bad arguments return their status before any
    launch."""
    from fp8_quantize_pack_amd import roofline
    L = roofline.lib()
    names = _declared_functions("mxq_roofline.h")
    assert names == ["mxq_ref_clock", "mxq_ref_copy", "mxq_ref_fill", "mxq_ref_read"]
    for n in names:
        assert hasattr(L, n), n
    assert L.mxq_ref_copy(FAKE, FAKE, 24, 2, None) == 2          # not a multiple of 16
    assert L.mxq_ref_copy(FAKE, FAKE, -16, 2, None) == 2
    assert L.mxq_ref_copy(FAKE, FAKE, 64, 3, None) == 5          # unroll
    assert L.mxq_ref_copy(None, FAKE, 64, 2, None) == 1
    assert L.mxq_ref_copy(FAKE, FAKE + 8, 64, 2, None) == 9
    assert L.mxq_ref_copy(None, None, 0, 2, None) == 0           # empty: no launch
    assert L.mxq_ref_read(FAKE, 64, 2, 0, None, None) == 1       # no sink
    assert L.mxq_ref_read(FAKE + 4, 64, 2, 0, FAKE, None) == 9
    assert L.mxq_ref_fill(FAKE, 40, 0, 2, None) == 2
    assert L.mxq_ref_fill(FAKE, 64, 0, 16, None) == 5
    assert L.mxq_ref_clock(None, 4, 16, None) == 1
    assert L.mxq_ref_clock(FAKE + 4, 4, 16, None) == 9
    assert L.mxq_ref_clock(FAKE, 0, 16, None) == 2
    assert L.mxq_ref_clock(FAKE, 65537, 16, None) == 2
    assert L.mxq_ref_clock(FAKE, 4, 0, None) == 2
    assert L.mxq_ref_clock(FAKE, 4, (1 << 24) + 1, None) == 2


def test_noalloc_validation(L):
    f = L.mxq_quantize_kv_nvfp4_noalloc
    # k, dt, S, H, D, smooth, packed, scales, row_scale, stream
    assert f(FAKE, 1, 64, 1025, 128, 1, FAKE, FAKE, FAKE, None) == 10   # beyond the static scratch
    assert f(FAKE, 1, 64, 5000, 128, 1, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 1, 64, 8, 96, 1, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 9, 64, 8, 128, 1, FAKE, FAKE, FAKE, None) == 3
    assert f(FAKE, 1, 64, 8, 128, 2, FAKE, FAKE, FAKE, None) == 8
    assert f(None, 1, 64, 8, 128, 1, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE + 4, 1, 64, 8, 128, 1, FAKE, FAKE, FAKE, None) == 9
    assert f(None, 1, 0, 8, 128, 1, None, None, None, None) == 0
    assert L.mxq_status_string(10) == b"the call needs more than its static device scratch"
