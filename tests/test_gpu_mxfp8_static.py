"""GPU parity of MXFP8 quantize / dequantize and of the static two-level FP4
fake quantization against the CPU oracle, bit for bit, through the C ABI.

Every shape is compared whole, the full-size workloads included.  Output buffers sit between
0xA5 guard bands that must survive every call."""
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
    print("[gpu-mx8-static]", *a, flush=True)
    sys.stdout.flush()


def mxq():
    import fp8_quantize_pack_amd as m
    return m


def guarded(shape, dtype):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    raw = torch.full((GUARD + n + GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    return raw, raw[GUARD:GUARD + n].view(dtype).view(*shape)


def check_guard(raw):
    torch.cuda.synchronize()
    assert bool((raw[:GUARD] == 0xA5).all()) and bool((raw[-GUARD:] == 0xA5).all()), "guard band overwritten"


def bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    return t


def assert_same(gpu, ref, what):
    g, r = bits(gpu), bits(ref)
    if not torch.equal(g, r):
        bad = (g != r).nonzero()
        raise AssertionError(f"{what}: {bad.shape[0]} mismatches, first at {bad[:5].tolist()}: "
                             f"gpu={g[tuple(bad[0])].item()} oracle={r[tuple(bad[0])].item()}")


def gpu_quantize_mxfp8(x):
    K = x.shape[-1]
    rc, c = guarded((*x.shape[:-1], K), torch.uint8)
    rs, s = guarded((*x.shape[:-1], K // 32), torch.uint8)
    mxq().mxq_quantize_mxfp8(x, c, s)
    check_guard(rc); check_guard(rs)
    return c, s


def gpu_dequantize_mxfp8(c, s, dtype):
    ry, y = guarded(tuple(c.shape), dtype)
    mxq().mxq_dequantize_mxfp8(c, s, y)
    check_guard(ry)
    return y


def gpu_fp4_static(x, a, G, B):
    ry, y = guarded(tuple(x.shape), x.dtype)
    g = torch.tensor([G], dtype=torch.float32, device=DEV)
    mxq().mxq_fake_quantize_fp4_static(x, a.to(DEV, torch.float32).contiguous(), g, y, B)
    check_guard(ry)
    return y


# ------------------------------------------------------------------ MXFP8

MX8_SHAPES = [(3, 5, 96), (257, 1024), (1, 32), (4100, 64), (2, 7168)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("shape", MX8_SHAPES)
def test_mxfp8_small(shape, dtype):
    say("mxfp8 small", shape, dtype)
    x = synth.moe_mxfp4(shape, seed=sum(shape) + 7).to(dtype)
    xf = x.reshape(-1, shape[-1])
    xf[0].zero_()
    if xf.shape[0] > 2:
        xf[1, :32] = -0.0
        xf[2] = xf[2] * 1e-3
    co, so = oracle.quantize_mxfp8(x)
    c, s = gpu_quantize_mxfp8(x.to(DEV))
    assert_same(s, so, "scales")
    assert_same(c, co, "codes")
    for odt in (torch.float32, torch.bfloat16, torch.float16):
        assert_same(gpu_dequantize_mxfp8(c, s, odt), oracle.dequantize_mxfp8(co, so, odt),
                    f"dequant {odt}")


def test_mxfp8_fp32_tiny_rows_and_config1():
    say("mxfp8 fp32 [256,1024] with zero row and 1e-30 row")
    x = synth.mxfp4_fp32()
    co, so = oracle.quantize_mxfp8(x)
    c, s = gpu_quantize_mxfp8(x.to(DEV))
    assert_same(s, so, "scales")
    assert_same(c, co, "codes")
    assert_same(gpu_dequantize_mxfp8(c, s, torch.float32),
                oracle.dequantize_mxfp8(co, so, torch.float32), "dequant")


def test_mxfp8_exhaustive_bf16_under_many_scales():
    """Every bf16 magnitude (both signs) that fits under a block whose amax is
    448 * 2^k, for k spread over the exponent range: every e4m3 decision,
    the subnormal codes, the round-to-zero band and signed zeros."""
    say("mxfp8 exhaustive bf16")
    bitsv = np.arange(0, 0x7F80, dtype=np.uint32)
    mags = (bitsv << 16).view(np.float32)
    rows = []
    for k in list(range(-126, 120, 9)) + [-125, 0, 119]:
        anchor = np.float32(448.0 * 2.0 ** k)
        vals = mags[mags <= anchor]
        vals = np.concatenate([vals, -vals])
        vals = np.concatenate([vals, np.zeros((-vals.size) % 31, np.float32)]).reshape(-1, 31)
        rows.append(np.concatenate([np.full((vals.shape[0], 1), anchor, np.float32), vals], 1))
    x = torch.from_numpy(np.concatenate(rows)).to(torch.bfloat16)
    say("rows", x.shape)
    co, so = oracle.quantize_mxfp8(x)
    c, s = gpu_quantize_mxfp8(x.to(DEV))
    assert_same(s, so, "scales")
    assert_same(c, co, "codes")
    assert_same(gpu_dequantize_mxfp8(c, s, torch.bfloat16),
                oracle.dequantize_mxfp8(co, so, torch.bfloat16), "dequant")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_mxfp8_dequant_every_code_every_scale(dtype):
    say("mxfp8 dequant every code x scale", dtype)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(256, 8)   # [256, 2048]
    scales = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(256, 1).repeat(1, 64)
    y = gpu_dequantize_mxfp8(codes.to(DEV), scales.to(DEV), dtype).cpu()
    yo = oracle.dequantize_mxfp8(codes, scales, dtype)
    # NaN codes (0x7F, 0xFF) and the NaN scale give NaN; neither the pages nor
    # IEEE fix a NaN's sign or payload, so NaNs are compared by position
    nan = torch.isnan(yo.float())
    assert int(nan.sum()) == 255 * 16 + 2048        # two NaN codes x 8 per row, one NaN-scale row
    assert torch.equal(nan, torch.isnan(y.float()))
    assert_same(y[~nan], yo[~nan], "dequant")


def test_mxfp8_empty():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    c = torch.empty(0, 64, dtype=torch.uint8, device=DEV)
    s = torch.empty(0, 2, dtype=torch.uint8, device=DEV)
    mxq().mxq_quantize_mxfp8(x, c, s)
    mxq().mxq_dequantize_mxfp8(c, s, x)
    torch.cuda.synchronize()


def test_full_mxfp8_moe_experts():
    """MXFP8 of the MoE expert weights [32, 4096, 2048] bf16, compared whole."""
    say("full mxfp8 [32,4096,2048], oracle threads", oracle.max_threads())
    x = synth.moe_mxfp4(synth.SHAPES["c2"], device=DEV).reshape(-1, 2048)
    c, s = mxq().quantize_mxfp8(x)
    y = mxq().dequantize_mxfp8(c, s, torch.bfloat16)
    co, so = oracle.quantize_mxfp8(x.cpu())
    assert_same(s.view(torch.uint8), so, "scales")
    assert_same(c.view(torch.uint8), co, "codes")
    assert_same(y, oracle.dequantize_mxfp8(co, so, torch.bfloat16), "dequant")
    # idempotence of the round trip over the whole tensor
    c2, s2 = mxq().quantize_mxfp8(y)
    assert torch.equal(mxq().dequantize_mxfp8(c2, s2, torch.bfloat16).view(torch.int16),
                       y.view(torch.int16))


# ------------------------------------------------------------------ static two-level FP4

def _block_amax(x, B):
    return x.float().abs().reshape(-1, x.shape[-1] // B, B).amax(-1).reshape(*x.shape[:-1], -1)


ST_CASES = [((3, 5, 96), 16), ((257, 1024), 16), ((257, 1024), 32), ((64, 512), 8),
            ((33, 1024), 128), ((1, 16), 16), ((4100, 64), 64)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("shape,B", ST_CASES)
def test_fp4_static_small(shape, B, dtype):
    say("fp4 static small", shape, B, dtype)
    x = synth.moe_nvfp4(shape if len(shape) == 3 else (1, *shape), seed=sum(shape) + B).reshape(shape).to(dtype)
    a = _block_amax(x, B)
    G = float(x.float().abs().max())
    yo = oracle.fake_quantize_fp4_static(x, a, G, B)
    assert_same(gpu_fp4_static(x.to(DEV), a, G, B), yo, "qdq")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fp4_static_calibrated_amax_differs_from_data(dtype):
    """Calibrated amax values that under- and over-shoot the data (saturated
    codes, block amax above the global one, zero amax, a tiny global amax)."""
    say("fp4 static perturbed amax", dtype)
    g = torch.Generator().manual_seed(81)
    x = synth.kv_cache((8, 64, 256), seed=82).reshape(512, 256).to(dtype)
    for B in (16, 32):
        a = _block_amax(x, B) * torch.exp2(torch.rand(512, 256 // B, generator=g) * 4 - 2)
        a[::7] = 0.0
        for G in (float(x.float().abs().max()), float(a.max()) * 0.25, 0.0, 3e-9, 1e6):
            yo = oracle.fake_quantize_fp4_static(x, a, G, B)
            assert_same(gpu_fp4_static(x.to(DEV), a, G, B), yo, f"qdq B={B} G={G}")


def test_fp4_static_fp32_planted_midpoints():
    """float32 elements whose quotient by their block scale lies on, or a few
    ulps around, each e2m1 midpoint: the exactness of the quotient path."""
    say("fp4 static planted midpoints")
    rng = np.random.default_rng(83)
    R, B = 2048, 16
    G = 37.5
    a = (rng.random((R, 1)) * 40 + 0.01).astype(np.float32)
    sp = np.array([oracle.static_block_scale(float(v), G) for v in a[:, 0]], np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    m = mids[rng.integers(0, 7, (R, B))]
    base = (m * sp[:, None]).astype(np.float32)
    d = rng.integers(-3, 4, (R, B))
    x = (base.view(np.uint32).astype(np.int64) + d).astype(np.uint32).view(np.float32)
    x = x * np.where(rng.random((R, B)) < 0.5, -1, 1).astype(np.float32)
    xt = torch.from_numpy(np.ascontiguousarray(x))
    at = torch.from_numpy(a)
    yo = oracle.fake_quantize_fp4_static(xt, at, G, B)
    assert_same(gpu_fp4_static(xt.to(DEV), at, G, B), yo, "qdq")


def test_fp4_static_empty():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    a = torch.empty(0, 4, dtype=torch.float32, device=DEV)
    g = torch.ones(1, device=DEV)
    mxq().mxq_fake_quantize_fp4_static(x, a, g, torch.empty_like(x), 16)
    torch.cuda.synchronize()


def test_full_fp4_static_gate_up_experts():
    """Static NVFP4-style fake quant (block 16) of the fused gate/up experts
    [64, 3072, 4096] bf16 with calibrated amax values, compared whole."""
    say("full fp4 static [64,3072,4096]")
    x = synth.moe_nvfp4(synth.SHAPES["c3"], device=DEV)
    K = x.shape[-1]
    xf = x.reshape(-1, K)
    a = _block_amax(xf, 16)
    G = xf.float().abs().max().reshape(1)
    y = mxq().fake_quantize_fp4_static(xf, a, G, 16)
    yo = oracle.fake_quantize_fp4_static(xf.cpu(), a.cpu(), float(G), 16)
    assert_same(y, yo, "qdq")
