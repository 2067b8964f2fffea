"""GPU parity: libmxq (through its C ABI) against the CPU oracle, bit for bit.

Every shape is compared whole, the full-size workloads included (in the same
launch configuration the bench uses).  Every output buffer sits between guard bands
filled with 0xA5 that must survive the call.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

GUARD = 4096
DEV = "cuda"


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantize_pack_amd  # noqa: F401  (fails loudly when not built)
    yield


def mxq():
    import fp8_quantize_pack_amd as m
    return m


def guarded(shape, dtype):
    """Output tensor with 4 KiB guard bands of 0xA5 on both sides."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    raw = torch.full((GUARD + n + GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    t = raw[GUARD:GUARD + n].view(dtype).view(*shape)
    return raw, t


def check_guard(raw):
    torch.cuda.synchronize()
    assert bool((raw[:GUARD] == 0xA5).all()) and bool((raw[-GUARD:] == 0xA5).all()), "guard band overwritten"


def bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float32,):
        return t.view(torch.int32)
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e8m0fnu, torch.int8):
        return t.view(torch.uint8)
    return t


def assert_same(gpu, ref, what):
    g, r = bits(gpu), bits(ref)
    if not torch.equal(g, r):
        bad = (g != r).nonzero()
        raise AssertionError(f"{what}: {bad.shape[0]} mismatches, first at {bad[:5].tolist()}: "
                             f"gpu={g[tuple(bad[0])].item()} oracle={r[tuple(bad[0])].item()}")


# ------------------------------------------------------------------ runners (C ABI)

def gpu_quantize_mxfp4(x):
    K = x.shape[-1]
    rp, p = guarded((*x.shape[:-1], K // 2), torch.int8)
    rs, s = guarded((*x.shape[:-1], K // 32), torch.uint8)
    mxq().mxq_quantize_mxfp4(x, p, s)
    check_guard(rp); check_guard(rs)
    return p, s


def gpu_dequantize_mxfp4(p, s, dtype):
    K = p.shape[-1] * 2
    ry, y = guarded((*p.shape[:-1], K), dtype)
    mxq().mxq_dequantize_mxfp4(p, s, y)
    check_guard(ry)
    return y


def gpu_quantize_nvfp4(x, mode="row", given=None):
    K = x.shape[-1]
    lead = tuple(x.shape[:-1])
    rp, p = guarded((*lead, K // 2), torch.uint8)
    rs, s = guarded((*lead, K // 16), torch.uint8)
    rg, g = guarded(lead if lead else (1,), torch.float32)
    scratch = torch.zeros(1, dtype=torch.float32, device=DEV)
    stride = 1
    if mode == "given":
        stride = 0 if given.numel() == 1 else 1
        given = given.to(DEV, torch.float32).contiguous()
    mxq().mxq_quantize_nvfp4(x, p, s, g, mode=mode, given=given, given_stride=stride,
                             scratch=scratch)
    check_guard(rp); check_guard(rs); check_guard(rg)
    return p, s, g


def gpu_dequantize_nvfp4(p, s, g, dtype):
    K = p.shape[-1] * 2
    ry, y = guarded((*p.shape[:-1], K), dtype)
    mxq().mxq_dequantize_nvfp4(p, s, g, y)
    check_guard(ry)
    return y


def gpu_quantize_cache(x, fmt, B):
    ry, y = guarded(tuple(x.shape), x.dtype)
    mxq().mxq_quantize_cache(x, y, fmt, B)
    check_guard(ry)
    return y


# ------------------------------------------------------------------ MXFP4

MX_SHAPES = [(3, 5, 96), (257, 1024), (1, 32), (4100, 64)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("shape", MX_SHAPES)
def test_mxfp4_roundtrip_small(shape, dtype):
    say("mxfp4 small", shape, dtype)
    x = synth.moe_mxfp4(shape, seed=sum(shape)).to(dtype)
    po, so = oracle.quantize_mxfp4(x)
    p, s = gpu_quantize_mxfp4(x.to(DEV))
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")
    for odt in (torch.float32, torch.bfloat16, torch.float16):
        yo = oracle.dequantize_mxfp4(po, so, odt)
        y = gpu_dequantize_mxfp4(p, s, odt)
        assert_same(y, yo, f"dequant {odt}")


def test_mxfp4_config1_fp32_with_zero_and_tiny_rows():
    say("mxfp4 fp32 [256,1024] with zero row and 1e-30 row")
    x = synth.mxfp4_fp32()
    po, so = oracle.quantize_mxfp4(x)
    p, s = gpu_quantize_mxfp4(x.to(DEV))
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")
    assert_same(gpu_dequantize_mxfp4(p, s, torch.float32), oracle.dequantize_mxfp4(po, so, torch.float32), "dequant")


def test_mxfp4_exhaustive_bf16_under_every_scale():
    """All bf16 values that fit a block, under each of the 253 e8m0 scales
    (the GPU's IEEE behaviour on subnormals and on midpoints included)."""
    say("mxfp4 exhaustive bf16 x scales")
    bitsv = np.arange(1 << 16, dtype=np.uint32)
    allv = (bitsv << 16).view(np.float32)
    allv = allv[np.isfinite(allv)]
    expo = (allv.view(np.uint32) >> 23) & 0xFF
    rows = []
    for sb in range(253):
        vals = allv[expo <= sb + 2]
        anchor = np.float32(2.0 ** (sb - 125)) if sb > 0 else np.float32(2.0 ** -125)
        vals = np.concatenate([vals, np.zeros((-vals.size) % 31, np.float32)]).reshape(-1, 31)
        rows.append(np.concatenate([np.full((vals.shape[0], 1), anchor, np.float32), vals], 1))
    x = torch.from_numpy(np.concatenate(rows)).to(torch.bfloat16)
    # second layout: the 31 values shifted by one column, so that every value
    # also sits in the other position of its byte (odd <-> even column)
    x2 = torch.cat([x[:, :1], x[:, 2:], x[:, 1:2]], 1)
    for xin in (x, x2):
        po, so = oracle.quantize_mxfp4(xin)
        p, s = gpu_quantize_mxfp4(xin.to(DEV))
        assert_same(s, so, "scales")
        assert_same(p, po, "packed")
        assert_same(gpu_dequantize_mxfp4(p, s, torch.bfloat16),
                    oracle.dequantize_mxfp4(po, so, torch.bfloat16), "dequant")


def test_mxfp4_fp32_planted_midpoints():
    """float32 inputs on, just below and just above every e2m1 midpoint of
    their block's scale (24-bit significands), both byte positions."""
    say("mxfp4 fp32 planted midpoints")
    rng = np.random.default_rng(1)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    n = 4096
    sc = np.exp2(rng.integers(-120, 120, n)).astype(np.float32)
    blk = np.zeros((n, 32), np.float32)
    blk[:, 0] = 6.0 * sc
    for j in range(1, 32):
        m = mids[rng.integers(0, 7, n)]
        d = rng.integers(-3, 4, n)
        v = (m.view(np.uint32).astype(np.int64) + d).astype(np.uint32).view(np.float32)
        blk[:, j] = v * sc * np.where(rng.random(n) < 0.5, -1, 1)
    x = torch.from_numpy(blk)
    po, so = oracle.quantize_mxfp4(x)
    p, s = gpu_quantize_mxfp4(x.to(DEV))
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")


@pytest.mark.parametrize("steps", ["near", "margin"])
@pytest.mark.parametrize("RK", [(512, 256), (128, 1040)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nvfp4_quotients_hugging_decision_boundaries(dtype, RK, steps):
    """Elements placed at m * den and at its neighbouring representable values
    for every e2m1 midpoint m, with arbitrary (given) row scales and power-of-two
    ones (exact ties).  "near": within 2 units of the last place of the input
    dtype; "margin" (float32): 6 to 20 units away."""
    if steps == "margin" and dtype != torch.float32:
        pytest.skip("bfloat16 neighbours are 2^16 float32 units apart")
    say("nvfp4 boundary-hugging quotients", dtype, RK, steps)
    rng = np.random.default_rng(17)
    R, K = RK
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    g = np.where(rng.random(R) < 0.5, np.exp2(rng.integers(-14, -4, R)), rng.random(R) * 1e-3 + 1e-6).astype(np.float32)
    x = np.zeros((R, K), np.float32)
    for r in range(R):
        for b in range(K // 16):
            sigma = np.float32(2.0 ** rng.integers(-3, 6) * (1 + rng.integers(0, 8) / 8))
            den = np.float32(sigma * g[r])
            blk = np.empty(16, np.float32)
            blk[0] = np.float32(6.0 * den)            # block amax 6 * den: block scale = sigma
            m = mids[rng.integers(0, 7, 15)]
            t = (m * den).astype(np.float32)
            if steps == "near":
                step = rng.integers(-2, 3, 15)
            else:
                step = rng.integers(6, 21, 15) * np.where(rng.random(15) < 0.5, -1, 1)
            if dtype == torch.bfloat16:
                tb = torch.from_numpy(t).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int32)
                tb = (tb + step).astype(np.int16)
                t = torch.from_numpy(tb).view(torch.bfloat16).float().numpy()
            else:
                t = (t.view(np.uint32).astype(np.int64) + step).astype(np.uint32).view(np.float32)
            blk[1:] = t * np.where(rng.random(15) < 0.5, -1, 1)
            x[r, 16 * b:16 * b + 16] = blk
    xt = torch.from_numpy(x).to(dtype)
    gt = torch.from_numpy(g)
    po, so, go = oracle.quantize_nvfp4(xt, mode="given", given=gt)
    p, s, gg = gpu_quantize_nvfp4(xt.to(DEV), mode="given", given=gt)
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_mxfp4_dequant_every_byte_every_scale(dtype):
    say("mxfp4 dequant all bytes x scales", dtype)
    p = torch.arange(256, dtype=torch.uint8).repeat(256, 1).view(torch.int8)
    s = torch.arange(256, dtype=torch.uint8).reshape(256, 1).repeat(1, 16)
    yo = oracle.dequantize_mxfp4(p.view(torch.uint8), s, dtype)
    y = gpu_dequantize_mxfp4(p.to(DEV), s.to(DEV), dtype).cpu()
    nan = torch.isnan(yo.float())
    assert torch.equal(nan, torch.isnan(y.float()))
    assert_same(y[~nan], yo[~nan], "dequant")


def test_mxfp4_empty_inputs_launch_nothing():
    say("mxfp4 empty")
    for shape in ((0, 64), (3, 0)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        p, s = mxq().quantize_mxfp4(x)
        assert p.shape == (*shape[:-1], shape[-1] // 2)
        y = mxq().dequantize_mxfp4(p, s, torch.bfloat16)
        assert y.shape == shape


# ------------------------------------------------------------------ NVFP4

# Row lengths cover every segment count a wave holds (1 to 8 with one wave
# per row; 5 to 8 with two and four), full and ragged last segments, and the
# two-pass kernel for rows of more than 32 segments (33024 columns).
NV_SHAPES = [(5, 16), (7, 48), (33, 512), (4, 1008), (3, 1040), (9, 2064), (6, 4096), (3, 5120),
             (2, 6144), (2, 6160), (5, 7168), (2, 8192), (3, 8208), (2, 12288), (2, 14352),
             (2, 16400), (1, 24576), (1, 32768), (1, 33024), (2, 3, 256)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("shape", NV_SHAPES)
def test_nvfp4_row_mode_small(shape, dtype):
    say("nvfp4 row", shape, dtype)
    x = synth.moe_nvfp4(shape, seed=sum(shape)).to(dtype)
    po, so, go = oracle.quantize_nvfp4(x)
    p, s, g = gpu_quantize_nvfp4(x.to(DEV))
    assert_same(g, go, "row scale")
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")
    for odt in (torch.bfloat16, torch.float32, torch.float16):
        assert_same(gpu_dequantize_nvfp4(p, s, g, odt), oracle.dequantize_nvfp4(po, so, go, odt),
                    f"dequant {odt}")


def test_nvfp4_sweep_specials():
    say("nvfp4 sweep specials")
    x = synth.moe_sweep((2, 64, 7168), seed=11, special_frac=0.02)
    po, so, go = oracle.quantize_nvfp4(x)
    p, s, g = gpu_quantize_nvfp4(x.to(DEV))
    assert_same(g, go, "row scale"); assert_same(s, so, "scales"); assert_same(p, po, "packed")
    assert_same(gpu_dequantize_nvfp4(p, s, g, torch.bfloat16),
                oracle.dequantize_nvfp4(po, so, go, torch.bfloat16), "dequant")


# 7168 and 16400 columns take the row kernels with 7 and 5 segments per wave
# (one and four waves a row), which launch at four workgroups per CU
@pytest.mark.parametrize("K", [256, 2064, 7168, 16400])
@pytest.mark.parametrize("kind", ["pow2", "random", "scalar", "edge", "negative", "bounds", "overflow"])
def test_nvfp4_given_scales(kind, K):
    say("nvfp4 given", kind, K)
    rng = np.random.default_rng(3)
    R = 96
    x = torch.from_numpy(rng.standard_normal((R, K)).astype(np.float32)).to(torch.bfloat16)
    if kind == "pow2":
        gv = torch.from_numpy(np.exp2(rng.integers(-12, -2, R)).astype(np.float32))
    elif kind == "random":
        gv = torch.from_numpy((rng.random(R) * 1e-3).astype(np.float32))
    elif kind == "scalar":
        gv = torch.tensor([3.7e-4])
    elif kind == "negative":
        gv = torch.from_numpy(-(rng.random(R) * 1e-3 + 1e-6).astype(np.float32))
    elif kind == "bounds":
        # both sides of 2^-100 and 2^100 (row scales in between need no
        # zero / infinity handling of the block denominators)
        b = np.array([2.0 ** -100, 2.0 ** 100], np.float32)
        gv = torch.from_numpy(np.resize(np.concatenate(
            [b, np.nextafter(b, np.float32(0)), np.nextafter(b, np.float32(np.inf)), b * 2, b / 2]), R))
    elif kind == "overflow":
        # elements near the bfloat16 maximum under small row scales in the
        # per-row fast range: x / (block scale * g) overflows float32 to
        # +-inf (and the block scale clamps at 448), so every such code
        # saturates, with its sign
        x = (x.float() * 1e38).clamp(-3.3e38, 3.3e38).to(torch.bfloat16)
        x[::7, ::5] = 1.0                              # ordinary values beside them
        gv = torch.from_numpy(np.resize(np.array([2.0 ** -100, 1e-20, 1e-5, 3.0], np.float32), R))
    else:
        x[3] = 0
        gv = torch.from_numpy(np.resize(np.array([0.0, 1e-42, 1e30, np.inf, 2.0 ** -126, 3.0, 1e-20, 1e20],
                                                 np.float32), R))
    po, so, go = oracle.quantize_nvfp4(x, mode="given", given=gv)
    p, s, g = gpu_quantize_nvfp4(x.to(DEV), mode="given", given=gv)
    assert_same(g, go, "row scale"); assert_same(s, so, "scales"); assert_same(p, po, "packed")


def test_nvfp4_block_scale_dense_amax():
    """Block maxima a on a dense grid of float32 values (every 64th bit pattern
    from just below 6 * 2^-9 to just above 2688) and around 6 * t for every
    rounding tie t of e4m3, with row scale 1, so that the block scale byte is
    e4m3(RN(a / 6)) across the whole range of the encoder; 1024-column rows."""
    say("nvfp4 dense block amax")
    lo = int(np.float32(6 * 2.0 ** -9 * 0.999).view(np.uint32))
    hi = int(np.float32(2688 * 1.001).view(np.uint32))
    grid = np.arange(lo, hi, 64, dtype=np.uint32)
    e4 = torch.arange(1, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ties = (e4[:-1] + e4[1:]) / 2
    near = (np.float32(6.0) * ties.astype(np.float32)).view(np.uint32).astype(np.int64)
    near = (near[:, None] + np.arange(-6, 7)[None, :]).reshape(-1).astype(np.uint32)
    a = np.concatenate([grid, near]).view(np.float32)
    a = np.resize(a, -(-a.size // 64) * 64)
    c = np.linspace(1.0, -1.0, 16, dtype=np.float32)       # c[0] = 1: element 0 is the amax
    x = torch.from_numpy((a[:, None] * c[None, :]).astype(np.float32).reshape(-1, 1024))
    one = torch.ones(1)
    po, so, go = oracle.quantize_nvfp4(x, mode="given", given=one)
    p, s, g = gpu_quantize_nvfp4(x.to(DEV), mode="given", given=one)
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")


@pytest.mark.parametrize("shape", [(64, 128), (300, 4096), (17, 16), (40, 7168), (6, 16400)])
def test_nvfp4_tensor_mode(shape):
    say("nvfp4 tensor mode", shape)
    x = synth.moe_nvfp4(shape, seed=shape[0])
    po, so, go = oracle.quantize_nvfp4(x, mode="tensor")
    p, s, g = gpu_quantize_nvfp4(x.to(DEV), mode="tensor")
    assert_same(g, go, "row scale"); assert_same(s, so, "scales"); assert_same(p, po, "packed")
    pw, sw, gw = mxq().quantize_nvfp4_modelopt(x.to(DEV))
    assert_same(pw, po, "modelopt packed"); assert_same(sw, so, "modelopt scales")
    assert gw.item() == go[0].item()


def test_nvfp4_zero_rows():
    say("nvfp4 zero rows")
    x = torch.zeros(8, 64, dtype=torch.bfloat16)
    x[3, 5] = 1.0
    po, so, go = oracle.quantize_nvfp4(x)
    p, s, g = gpu_quantize_nvfp4(x.to(DEV))
    assert_same(g, go, "row scale"); assert_same(s, so, "scales"); assert_same(p, po, "packed")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_nvfp4_dequant_every_code_every_scale(dtype):
    say("nvfp4 dequant all codes x scales", dtype)
    rng = np.random.default_rng(8)
    R = 64
    p = torch.arange(256, dtype=torch.uint8).repeat(R, 8)
    s = torch.arange(256, dtype=torch.uint8).repeat(R, 1)
    g = torch.from_numpy(np.concatenate([np.exp2(rng.random(R - 6) * 60 - 40),
                                         [0.0, 1e-40, 3e38, 2.0 ** -126, 1.0, 6e4]]).astype(np.float32))
    yo = oracle.dequantize_nvfp4(p, s, g, dtype)
    y = gpu_dequantize_nvfp4(p.to(DEV), s.to(DEV), g.to(DEV), dtype).cpu()
    nan = torch.isnan(yo.float())
    assert torch.equal(nan, torch.isnan(y.float()))
    assert_same(y[~nan], yo[~nan], "dequant")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("K", [4096, 256])
def test_nvfp4_dequant_all_codes_under_all_scale_bytes(K, dtype):
    """Each of the 256 scale bytes (both zeros, negatives, NaN) over a block
    holding the 16 codes 0..15, under row scales from zero and subnormal to
    huge; rows of 4096 (segment kernel) and of 256 (short-row kernel)."""
    say("nvfp4 dequant codes x scale bytes", K, dtype)
    rng = np.random.default_rng(9)
    R = 48
    blk = torch.tensor([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=torch.uint8)
    p = blk.repeat(R, 256)                                   # [R, 2048]: 256 blocks of codes 0..15
    s = torch.arange(256, dtype=torch.uint8).repeat(R, 1)   # block j has scale byte j
    g = torch.from_numpy(np.concatenate([np.exp2(rng.random(R - 8) * 60 - 40) * rng.choice([-1, 1], R - 8),
                                         [0.0, -0.0, 1e-40, 3e38, 2.0 ** -126, 1.0, -6e4, float("inf")]])
                         .astype(np.float32))
    per = 4096 // K
    p, s, g = p.reshape(R * per, K // 2), s.reshape(R * per, K // 16), g.repeat_interleave(per)
    yo = oracle.dequantize_nvfp4(p, s, g, dtype)
    y = gpu_dequantize_nvfp4(p.to(DEV), s.to(DEV), g.to(DEV), dtype).cpu()
    nan = torch.isnan(yo.float())
    assert torch.equal(nan, torch.isnan(y.float()))
    assert_same(y[~nan], yo[~nan], "dequant")


# ------------------------------------------------------------------ cache

CACHE_CASES = [(512, 32), (128, 32), (512, 16), (120, 32), (100, 16), (96, 7), (64, 64),
               (1024, 512), (40, 8), (24, 256), (24, 1), (30, 3)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("C,B", CACHE_CASES)
def test_cache_small(C, B, fmt, dtype):
    say("cache", fmt, C, B, dtype)
    x = synth.kv_cache((3, 37, C), seed=C * 7 + B).to(dtype)
    x[0, 0] = 0
    x[0, 1] = x[0, 1] * 2.0 ** -125
    x[0, 2, :8] = -0.0
    yo = oracle.quantize_cache(x, fmt, B)
    y = gpu_quantize_cache(x.to(DEV), fmt, B)
    assert_same(y, yo, "qdq")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_cache_unaligned_views(fmt):
    say("cache unaligned", fmt)
    x = synth.kv_cache((5, 129), seed=1)
    xo = x[:, 1:]                           # C = 128, rows start 2 bytes off
    yo = oracle.quantize_cache(xo.contiguous(), fmt, 32)
    xd = x.to(DEV)[:, 1:]
    raw = torch.full((5 * 129 + 64,), 0, dtype=torch.bfloat16, device=DEV)
    ydst = raw[1:1 + 5 * 128].view(5, 128)  # misaligned output
    mxq().mxq_quantize_cache(xd.contiguous()[:, :], ydst, fmt, 32)
    assert_same(ydst, yo, "qdq")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_cache_all_bf16_values(fmt):
    say("cache all bf16 values", fmt)
    bitsv = np.arange(1 << 16, dtype=np.uint32)
    v = (bitsv << 16).view(np.float32)
    v = torch.from_numpy(v[np.isfinite(v)]).to(torch.bfloat16)
    v = v[torch.randperm(v.numel(), generator=torch.Generator().manual_seed(3))]
    v = torch.nn.functional.pad(v, (0, (-v.numel()) % 32)).reshape(-1, 32)
    for B in (32, 16):
        assert_same(gpu_quantize_cache(v.to(DEV), fmt, B), oracle.quantize_cache(v, fmt, B), f"B={B}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_cache_all_f16_values(fmt):
    """Every finite float16 value (subnormals, both zeros, the largest
    magnitudes) in shuffled groups of 32 and 16 through the cache round trip
    with float16 in and out."""
    say("cache all f16 values", fmt)
    v = torch.from_numpy(np.arange(1 << 16, dtype=np.uint16).view(np.float16).copy())
    v = v[torch.isfinite(v)]
    v = v[torch.randperm(v.numel(), generator=torch.Generator().manual_seed(4))]
    v = torch.nn.functional.pad(v, (0, (-v.numel()) % 32)).reshape(-1, 32)
    for B in (32, 16):
        assert_same(gpu_quantize_cache(v.to(DEV), fmt, B), oracle.quantize_cache(v, fmt, B), f"B={B}")


# ------------------------------------------------------------------ full-size workloads (whole tensors)
#
# Every full-size workload is compared whole: every packed byte, scale byte,
# row scale and dequantized element of the GPU result against the oracle on
# the same input.  The oracle's row loops run on all host threads (OpenMP,
# static schedule; its results do not depend on the thread count).

def _cpu(t):
    return t.detach().cpu()


def test_full_c2_mxfp4_moe():
    say("full C2 mxfp4 [32,4096,2048], oracle threads", oracle.max_threads())
    x = synth.moe_mxfp4(synth.SHAPES["c2"], device=DEV).reshape(-1, 2048)
    p, s = mxq().quantize_mxfp4(x)
    y = mxq().dequantize_mxfp4(p, s, torch.bfloat16)
    po, so = oracle.quantize_mxfp4(_cpu(x))
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")
    assert_same(y, oracle.dequantize_mxfp4(po, so, torch.bfloat16), "dequant")
    # idempotence over the whole tensor
    p2, s2 = mxq().quantize_mxfp4(y)
    assert torch.equal(mxq().dequantize_mxfp4(p2, s2, torch.bfloat16).view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("given_half", [False, True])
def test_full_c3_nvfp4_gate_up(given_half):
    say("full C3 nvfp4 [64,3072,4096] given_half=", given_half)
    x = synth.moe_nvfp4(synth.SHAPES["c3"], device=DEV)
    E, N, K = x.shape
    if given_half:
        amax_half = x.float().abs().reshape(E, 2, N // 2, K).amax(dim=(2, 3))
        gvals = (amax_half / 2688.0).reshape(E, 2, 1).expand(E, 2, N // 2).reshape(E, N)
        p, s, g = mxq().quantize_nvfp4(x, global_scale=gvals)
    else:
        p, s, g = mxq().quantize_nvfp4(x)
    y = mxq().dequantize_nvfp4(p, s, g, torch.bfloat16)
    xs = _cpu(x)
    if given_half:
        po, so, go = oracle.quantize_nvfp4(xs, mode="given", given=_cpu(gvals).reshape(-1))
    else:
        po, so, go = oracle.quantize_nvfp4(xs)
    del xs
    assert_same(g, go, "row scale")
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")
    del p, s
    assert_same(y, oracle.dequantize_nvfp4(po, so, go, torch.bfloat16), "dequant")


def test_full_nvfp4_tensor_mode_sweep_chunk():
    """Per-tensor NVFP4 on the workload the bench times for it: one 36-expert
    chunk of the MoE sweep as rows of 4096 (1 GB, the whole-tensor amax pass
    on one workgroup per CU).  Every row scale must be the exact tensor
    maximum (torch's) divided by 2688 and rounded once, and the whole result
    must equal the oracle's tensor mode."""
    say("full nvfp4 tensor mode [129024, 4096]")
    x = synth.c5_chunk(0, synth.C5_CHUNK_EXPERTS, device=DEV).reshape(-1, 4096)
    p, s, g = gpu_quantize_nvfp4(x, mode="tensor")
    amax = x.abs().max().float().cpu().numpy()
    g0 = np.float32(amax) / np.float32(2688.0)
    assert torch.equal(g.cpu(), torch.full_like(g.cpu(), float(g0))), "row scales"
    po, so, go = oracle.quantize_nvfp4(_cpu(x), mode="tensor")
    assert_same(g, go, "row scales vs oracle")
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")


@pytest.mark.parametrize("case,fmt,B", [("c4a", "fp8", 32), ("c4b", "mxfp4", 32), ("c4c", "nvfp4", 16)])
def test_full_c4_cache(case, fmt, B):
    say("full", case, fmt)
    x = synth.kv_cache(synth.SHAPES[case], seed=synth.SEEDS[case], device=DEV)
    y = mxq().quantize_cache(x, fmt, B)
    assert y.shape == x.shape and y.dtype == x.dtype
    assert_same(y, oracle.quantize_cache(_cpu(x), fmt, B), "qdq")


@pytest.mark.parametrize("cid", [c[0] for c in synth.c5_chunks()])
def test_full_c5_chunk_mxfp4_nvfp4(cid):
    """Every chunk of the large sweep (36 experts, about 1 GiB of bf16, the
    last one 4 experts), as the bench processes it: MXFP4 and NVFP4 quantize
    and dequantize, compared whole."""
    _, e0, ne = synth.c5_chunks()[cid]
    say("full C5 chunk", cid, ne, "experts, oracle threads", oracle.max_threads())
    x = synth.c5_chunk(cid, ne, device=DEV)
    xs = _cpu(x)
    # the chunk holds the special blocks the recipe plants
    bmax = xs.reshape(-1, 32).float().abs().amax(-1)
    assert int((bmax == 0).sum()) > 0 and int((bmax > 1e3).sum()) > 0
    assert int(((bmax > 0) & (bmax < 1e-30)).sum()) > 0
    del bmax
    p, s = mxq().quantize_mxfp4(x)
    y = mxq().dequantize_mxfp4(p, s, torch.bfloat16)
    po, so = oracle.quantize_mxfp4(xs)
    assert_same(s, so, "mx scales")
    assert_same(p, po, "mx packed")
    del p, s
    assert_same(y, oracle.dequantize_mxfp4(po, so, torch.bfloat16), "mx dequant")
    del y, po, so
    p, s, g = mxq().quantize_nvfp4(x)
    y = mxq().dequantize_nvfp4(p, s, g, torch.bfloat16)
    po, so, go = oracle.quantize_nvfp4(xs)
    assert_same(g, go, "nv row scale")
    assert_same(s, so, "nv scales")
    assert_same(p, po, "nv packed")
    del p, s, g
    assert_same(y, oracle.dequantize_nvfp4(po, so, go, torch.bfloat16), "nv dequant")
