"""Pins of the oracle's MXFP8, static two-level FP4, paged KV-cache and
k_smooth functions against what the pages and mathematics fix.

As in test_oracle_pins.py, no expected value is the oracle compared with
itself: expected values come from torch's CPU float8 casts and float32
arithmetic (library routines), from special cases that reduce to oracle
functions already pinned there (NVFP4 with a given scale, the mxfp4 cache
round trip), from hand-derived closed forms, and from characterising
properties.

Parity unpinned by the pages, for two readings these tests pin the oracle to
without the pages fixing them:
  * static two-level FP4: the pages name the e4m3 fake quantization of the
    block scale (scaled_e4m3 under the per-tensor amax) without printing its
    arithmetic.  The oracle takes it as multiply by 448 / P, cast, divide by
    448 / P.  Most pins use a global amax for which 448 / P is a power of two,
    where every ordering of those steps gives the same bits; only the 1e-8
    floor case and the error bound reach a general P.
  * k_smooth: the pages compute the row mean with torch's mean, whose
    summation order torch does not fix.  The oracle sums pairwise (halves,
    recursively); the pins check that order on hand cases where it matters
    and the bf16 rounding bound that any order meets.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

TINY = torch.finfo(torch.float32).tiny


def _pow2ceil_torch(v: torch.Tensor) -> torch.Tensor:
    m, e = torch.frexp(v)               # v = m * 2^e, m in [0.5, 1)
    return torch.where(m == 0.5, v, torch.ldexp(torch.ones_like(v), e))


# ------------------------------------------------------------------ MXFP8

def _mxfp8_torch(x: torch.Tensor):
    """Block-32 e8m0 scale as the power-of-two ceiling of amax / 448 (floored
    at the smallest normal float), codes through torch's float8 e4m3 cast."""
    R, K = x.shape
    xg = x.float().reshape(R, K // 32, 32)
    a = xg.abs().amax(-1, keepdim=True)
    s = _pow2ceil_torch(torch.clamp_min(a / 448.0, TINY))
    q = xg / s
    assert q.abs().max() <= 448.0        # the scale keeps every quotient in range
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, K)
    _, e = torch.frexp(s)                # s = 2^(e - 1)
    sbytes = (e - 1 + 127).reshape(R, K // 32).to(torch.uint8)
    return codes, sbytes


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_mxfp8_matches_torch_cast_composition(dtype):
    x = synth.moe_mxfp4((24, 256), seed=61).to(dtype)
    x[3].zero_()
    x[5, :32] = -0.0
    codes, sb = oracle.quantize_mxfp8(x)
    want_c, want_s = _mxfp8_torch(x)
    assert torch.equal(sb, want_s)
    assert torch.equal(codes, want_c)


def test_mxfp8_scale_characterisation_all_bf16_amax():
    """Byte b is the smallest with 448 * 2^(b - 127) >= amax, and at least 1
    (exhaustive over positive finite bfloat16 amax values)."""
    bits = torch.arange(1, 0x7F80, dtype=torch.int32)
    a = (bits << 16).view(torch.float32)
    x = torch.zeros(a.numel(), 32, dtype=torch.bfloat16)
    x[:, 7] = a.to(torch.bfloat16)
    _, sb = oracle.quantize_mxfp8(x)
    b = sb[:, 0].to(torch.float64)
    a64 = a.to(torch.float64)
    cap = 448.0 * torch.exp2(b - 127)
    assert bool((cap >= a64).all())
    below = 448.0 * torch.exp2(b - 128)
    assert bool(((below < a64) | (b == 1)).all())
    assert int(b.min()) >= 1 and int(b.max()) <= 254


def test_mxfp8_zero_block_and_signed_zero():
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    x[1, :32] = -0.0
    codes, sb = oracle.quantize_mxfp8(x)
    assert sb.tolist() == [[1, 1], [1, 1]]           # 2^-126: the floor
    assert codes[0].tolist() == [0] * 64
    assert codes[1, :32].tolist() == [0x80] * 32      # sign of zero kept
    y = oracle.dequantize_mxfp8(codes, sb, torch.float32)
    assert torch.equal(torch.signbit(y), torch.signbit(x.float()))
    assert float(y.abs().max()) == 0.0


def test_mxfp8_dequant_closed_form_all_codes():
    """Every code byte under a spread of scale bytes: the e4m3 value (torch's
    decoding) times 2^(b - 127), rounded once to the output dtype."""
    codes = torch.arange(256, dtype=torch.int32).repeat(8).to(torch.uint8).reshape(8, 256)
    sbytes = torch.tensor([0, 1, 100, 127, 128, 160, 247, 254], dtype=torch.uint8)
    sb = sbytes.reshape(8, 1).repeat(1, 8)
    val = codes.view(torch.float8_e4m3fn).to(torch.float64)
    want = val * torch.exp2(sbytes.to(torch.float64) - 127).reshape(8, 1)
    for dt in (torch.float32, torch.bfloat16, torch.float16):
        got = oracle.dequantize_mxfp8(codes, sb, dt)
        w = want.to(torch.float32).to(dt)              # exact product, one rounding
        same = (got == w) | (torch.isnan(got) & torch.isnan(w))
        assert bool(same.all()), dt
    # scale byte 255 is the e8m0 NaN
    y = oracle.dequantize_mxfp8(torch.full((1, 32), 0x38, dtype=torch.uint8),
                                torch.tensor([[255]], dtype=torch.uint8), torch.float32)
    assert bool(torch.isnan(y).all())


def test_mxfp8_roundtrip_representable_and_error_bound():
    """Values that are e4m3 values times a block's own scale come back
    unchanged; everything else within half an e4m3 step (relative 2^-4 in
    the normal range, 2^-10 * s below it)."""
    g = torch.Generator().manual_seed(62)
    bytes_ = torch.randint(0, 0x7F, (16, 128), generator=g, dtype=torch.int32).to(torch.uint8)
    vals = bytes_.view(torch.float8_e4m3fn).float()
    vals[:, ::32] = 448.0                                # amax 448: scale 1
    sign = torch.where(torch.rand(16, 128, generator=g) < 0.5, -1.0, 1.0)
    x = (vals * sign * 2.0 ** 5).to(torch.bfloat16)      # scale 2^5
    codes, sb = oracle.quantize_mxfp8(x)
    assert bool((sb == 132).all())
    assert torch.equal(oracle.dequantize_mxfp8(codes, sb, torch.bfloat16), x)
    z = synth.kv_cache((4, 8, 256), seed=63).reshape(32, 256)
    c2, s2 = oracle.quantize_mxfp8(z)
    y = oracle.dequantize_mxfp8(c2, s2, torch.float32).double()
    s = torch.exp2(s2.double() - 127).repeat_interleave(32, -1)
    err = (y - z.double()).abs()
    bound = torch.maximum(z.double().abs() * 2.0 ** -4, s * 2.0 ** -10)
    assert bool((err <= bound).all())


# ------------------------------------------------------------------ static two-level FP4

def _blocks_amax(x: torch.Tensor, B: int) -> torch.Tensor:
    R, K = x.shape
    return x.float().abs().reshape(R, K // B, B).amax(-1)


@pytest.mark.parametrize("j", [-10, 0, 7])
def test_static_fp4_reduces_to_nvfp4_with_power_of_two_row_scale(j):
    """G = 2688 * 2^j makes 448 / P = 2^-j exact; every later product is then
    exact and the chain is the NVFP4 rule with the given row scale 2^j
    (quantize, then dequantize, both pinned in test_oracle_pins.py)."""
    x = (synth.moe_nvfp4((2, 16, 256), seed=64).reshape(32, 256).float() * 2.0 ** j).to(torch.bfloat16)
    G = 2688.0 * 2.0 ** j
    a = _blocks_amax(x, 16)
    got = oracle.fake_quantize_fp4_static(x, a, G, 16)
    p, s, g = oracle.quantize_nvfp4(x, mode="given", given=torch.tensor([2.0 ** j]))
    want = oracle.dequantize_nvfp4(p, s, g, torch.bfloat16)
    assert torch.equal(got, want)


@pytest.mark.parametrize("j", [-6, 0, 5])
def test_static_fp4_reduces_to_mxfp4_cache_when_every_block_peaks_at_the_global(j):
    """Blocks whose amax equals G = 6 * 2^j get the block scale 2^j exactly
    (448 is an e4m3 value), which is the mxfp4 cache scale pow2ceil(amax / 6)."""
    g = torch.Generator().manual_seed(65 + j)
    x = (torch.rand(16, 128, generator=g) * 12 - 6) * 2.0 ** j
    x[:, ::32] = 6.0 * 2.0 ** j
    x[1::2, 5::32] = -6.0 * 2.0 ** j
    x = x.to(torch.bfloat16)
    G = 6.0 * 2.0 ** j
    a = torch.full((16, 4), G)
    assert oracle.static_block_scale(G, G) == 2.0 ** j
    got = oracle.fake_quantize_fp4_static(x, a, G, 32)
    assert torch.equal(got, oracle.quantize_cache(x, "mxfp4", 32))


@pytest.mark.parametrize("j", [-20, 0, 9])
def test_static_fp4_floor_scale_closed_form(j):
    """A zero block amax takes the smallest block scale: (2^-9 / 448) * P
    scaled by 448 / P is 2^-9 up to roundings, whose e4m3 value is 2^-9; the
    dequantization scale is RN(2^-9 / (448 / P)) = RN(2^(j-9) / 448) for
    P = 2^j."""
    G = 6.0 * 2.0 ** j
    want = np.float32(2.0 ** (j - 9)) / np.float32(448.0)    # IEEE float32 division
    assert oracle.static_block_scale(0.0, G) == float(want)


def test_static_fp4_global_floor_and_saturation():
    # G so small that G / 6 <= 1e-8: P is the floor 1e-8
    P = np.float32(1e-8)
    t = np.float32(448.0) / P
    assert oracle.static_block_scale(0.0, 0.0) == oracle.static_block_scale(0.0, 1e-9)
    # a block amax beyond the global one saturates at the e4m3 maximum 448
    s = oracle.static_block_scale(1e-3, 1e-9)
    assert s == float(np.float32(448.0) / t)
    assert oracle.static_block_scale(100.0, 6.0) == 1.0      # 448 / 448
    # all-zero input under the floor stays zero
    y = oracle.fake_quantize_fp4_static(torch.zeros(2, 32, dtype=torch.bfloat16),
                                        torch.zeros(2, 2), 0.0, 16)
    assert float(y.float().abs().max()) == 0.0


def test_static_fp4_error_bound_and_grid():
    """Every output is an e2m1 value times its block's scale (after one
    rounding to float32), and |y - x| <= s' for |x| <= 6 s'."""
    x = synth.moe_nvfp4((1, 64, 512), seed=66).reshape(64, 512).float()
    G = float(x.abs().max())
    for B in (16, 32):
        a = _blocks_amax(x, B)
        y = oracle.fake_quantize_fp4_static(x, a, G, B).double()
        sp = torch.tensor([[oracle.static_block_scale(float(v), G) for v in row] for row in a],
                          dtype=torch.float64).repeat_interleave(B, -1)
        q = (y / sp).abs()
        grid = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float64)
        near = (q.unsqueeze(-1) - grid).abs().min(-1).values
        assert bool((near <= 6 * 2.0 ** -23).all())
        inside = x.double().abs() <= 6 * sp
        assert bool(((y - x.double()).abs() <= sp + 1e-30)[inside].all())
        # the block scale covers the block: a / 6 <= s' (1 + 2^-4)
        assert bool((a.double() / 6 <= sp[:, ::B] * (1 + 2.0 ** -4)).all())


# ------------------------------------------------------------------ paged KV cache

def _pages(nb, bt, H, D, seed):
    pages = []
    for b in range(nb):
        k = synth.kv_cache((bt, H, D), seed=seed + b).reshape(bt * H, D)
        p, s, g = oracle.quantize_nvfp4(k, mode="tensor")
        pages.append((p, s, float(k.float().abs().max()), g))
    return pages


def test_kv_pages_dequant_is_nvfp4_dequant_in_block_order():
    nb, bt, H, D = 5, 3, 4, 128
    pages = _pages(nb, bt, H, D, seed=70)
    order = [3, 0, 4, 1, 2]                         # the block list as the cache holds it
    vals = [pages[i][0] for i in order]
    scs = [pages[i][1] for i in order]
    am = [pages[i][2] for i in order]
    y = oracle.dequantize_kv_pages(vals, scs, am, bt, H, torch.bfloat16)
    assert y.shape == (1, nb * bt, H, D)
    for pos, i in enumerate(order):
        p, s, a, g = pages[i]
        # the page's global scale amax / (6 * 448) equals the tensor-mode row scale
        assert float(np.float32(a) / np.float32(2688.0)) == float(g[0])
        want = oracle.dequantize_nvfp4(p, s, g, torch.bfloat16).reshape(bt, H, D)
        assert torch.equal(y[0, pos * bt:(pos + 1) * bt], want)


# ------------------------------------------------------------------ k_smooth / quantize_kv

def test_k_smooth_pairwise_order_hand_case():
    """[1, 2^24, 1, -2^24, 0, ...]: pairwise, (1 + 2^24) + (1 - 2^24) = 2^24 +
    (-(2^24 - 1)) = 1, so the mean is 1/16; a left-to-right sum would lose
    both ones and give 0."""
    row = torch.zeros(1, 16, dtype=torch.float32)
    row[0, :4] = torch.tensor([1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)])
    ks = oracle.k_smooth(row)
    assert ks[0, 4].item() == -1.0 / 16
    assert ks[0, 0].item() == 1.0 - 1.0 / 16


def test_k_smooth_exact_on_small_integers():
    g = torch.Generator().manual_seed(71)
    h = torch.randint(-100, 100, (32, 64), generator=g).to(torch.float32)
    x = torch.cat([h, 6.0 - h], dim=1)         # pairs sum to 6: mean 3 exactly
    xb = x.to(torch.bfloat16)
    assert torch.equal(xb.float(), x)
    ks = oracle.k_smooth(xb)
    assert torch.equal(ks.float(), (x - 3.0).to(torch.bfloat16).float())
    c = torch.full((4, 64), 2.75).to(torch.bfloat16)
    assert float(oracle.k_smooth(c).float().abs().max()) == 0.0


def test_k_smooth_close_to_exact_mean_removal():
    x = synth.kv_cache((64, 4, 128), seed=72)
    ks = oracle.k_smooth(x).double()
    exact = x.double() - x.double().mean(-1, keepdim=True)
    # mean rounded to bf16 (rel 2^-9 of |mean|), then one bf16 rounding
    mean = x.double().mean(-1, keepdim=True).abs()
    bound = exact.abs() * 2.0 ** -8 + mean * 2.0 ** -8 + 1e-30
    assert bool(((ks - exact).abs() <= bound).all())


@pytest.mark.parametrize("smooth", [False, True])
def test_quantize_kv_is_per_head_tensor_nvfp4(smooth):
    S, H, D = 40, 3, 128
    k = synth.kv_cache((S, H, D), seed=73)
    p, s, g = oracle.quantize_kv_nvfp4(k, smooth=smooth)
    src = oracle.k_smooth(k) if smooth else k
    for h in range(H):
        ph, sh, gh = oracle.quantize_nvfp4(src[:, h, :].contiguous(), mode="tensor")
        assert torch.equal(p[:, h], ph) and torch.equal(s[:, h], sh)
        assert torch.equal(g[:, h], gh)
        assert float(gh[0]) == float(np.float32(src[:, h].float().abs().max()) / np.float32(2688.0))
