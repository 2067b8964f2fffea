"""The kernels' per-element arithmetic, built for the host, against the oracle.

The GPU kernels call the same functions (fp8_quantize_pack_amd/csrc/mxq_device.h)
for every number they produce; here they run on the CPU in the kernels' block
structure, over exhaustive and edge-case inputs.  The GPU parity tests then
cover lane mapping, memory layout and the GPU's own IEEE arithmetic.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import hostmath as hm


def _bf16_all_finite():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def _eq(a, b):
    if a.dtype in (torch.float32, torch.bfloat16, torch.float16):
        ia = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}[a.dtype]
        return torch.equal(a.view(ia), b.view(ia))
    return torch.equal(a, b)


# ------------------------------------------------------------------ MXFP4

def test_mxfp4_quant_exhaustive_bf16_every_scale():
    """Every bf16 value that can occur in a block, under every e8m0 scale:
    blocks are [anchor, 31 values] where the anchor 4 * 2^e fixes scale e and
    the values are all bf16 numbers below 8 * 2^e."""
    allv = _bf16_all_finite()
    expo = (allv.view(np.uint32) >> 23) & 0xFF
    rows = []
    for sb in range(0, 253):
        vals = allv[expo <= sb + 2]
        anchor = np.float32(2.0 ** (sb - 127 + 2)) if sb > 0 else np.float32(2.0 ** -125)
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 31)
        blk = np.concatenate([np.full((vals.shape[0], 1), anchor, np.float32), vals], 1)
        rows.append(blk)
    x = torch.from_numpy(np.concatenate(rows)).to(torch.bfloat16).reshape(-1, 32)
    po, so = oracle.quantize_mxfp4(x)
    ph, sh = hm.quantize_mxfp4(x)
    assert torch.equal(so, sh)
    assert torch.equal(po, ph)


def test_mxfp4_quant_all_f16_values():
    bits = np.arange(1 << 16, dtype=np.uint16)
    h = torch.from_numpy(bits.view(np.float16).copy())
    h = h[torch.isfinite(h)]
    g = torch.Generator().manual_seed(0)
    h = h[torch.randperm(h.numel(), generator=g)]
    h = torch.nn.functional.pad(h, (0, (-h.numel()) % 32)).reshape(-1, 32)
    assert _eq(oracle.quantize_mxfp4(h)[0], hm.quantize_mxfp4(h)[0])
    assert _eq(oracle.quantize_mxfp4(h)[1], hm.quantize_mxfp4(h)[1])


def test_mxfp4_quant_fp32_edges():
    rng = np.random.default_rng(1)
    base = rng.standard_normal((4096, 32)).astype(np.float32) * np.exp2(rng.integers(-140, 120, (4096, 1))).astype(np.float32)
    # plant exact midpoints and their neighbours (in units of the block scale)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    sc = np.exp2(rng.integers(-100, 100, 2048)).astype(np.float32)
    blk = np.zeros((2048, 32), np.float32)
    blk[:, 0] = 6.0 * sc
    for j in range(1, 32):
        m = mids[rng.integers(0, 7, 2048)]
        d = rng.integers(-1, 2, 2048)
        v = m.copy()
        v[d < 0] = np.nextafter(m[d < 0], np.float32(0))
        v[d > 0] = np.nextafter(m[d > 0], np.float32(9))
        blk[:, j] = v * sc * np.where(rng.random(2048) < 0.5, -1, 1)
    x = torch.from_numpy(np.concatenate([base, blk]))
    x[0] = 0
    x[1] = 1e-30 * x[2]
    po, so = oracle.quantize_mxfp4(x)
    ph, sh = hm.quantize_mxfp4(x)
    assert torch.equal(so, sh) and torch.equal(po, ph)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_mxfp4_dequant_all_codes_all_scales(dtype):
    codes = torch.arange(256, dtype=torch.uint8)             # every byte
    p = codes.repeat(256, 1).reshape(256, 256)               # row b: all bytes
    s = torch.arange(256, dtype=torch.uint8).reshape(256, 1).repeat(1, 16)
    yo = oracle.dequantize_mxfp4(p, s, dtype)
    yh = hm.dequantize_mxfp4(p, s, dtype)
    nan_o, nan_h = torch.isnan(yo.float()), torch.isnan(yh.float())
    assert torch.equal(nan_o, nan_h)
    assert _eq(yo[~nan_o], yh[~nan_h])


# ------------------------------------------------------------------ NVFP4

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_nvfp4_quant_row_mode_matches_oracle(dtype):
    x = synth.moe_nvfp4((2, 64, 512), seed=3).to(dtype)
    o = oracle.quantize_nvfp4(x)
    h = hm.quantize_nvfp4(x)
    for a, b in zip(o, h):
        assert _eq(a, b)


def test_nvfp4_quant_sweep_specials_match_oracle():
    x = synth.moe_sweep((2, 32, 1024), seed=7, special_frac=0.02)
    o = oracle.quantize_nvfp4(x)
    h = hm.quantize_nvfp4(x)
    for a, b in zip(o, h):
        assert _eq(a, b)


def test_nvfp4_quant_given_power_of_two_scales_exact_ties():
    # a power-of-two g makes x / (sigma * g) land exactly on midpoints often
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((256, 256)).astype(np.float32)).to(torch.bfloat16)
    g = torch.from_numpy(np.exp2(rng.integers(-12, -2, 256)).astype(np.float32))
    o = oracle.quantize_nvfp4(x, mode="given", given=g)
    h = hm.quantize_nvfp4(x, mode="given", given=g)
    for a, b in zip(o, h):
        assert _eq(a, b)


def test_nvfp4_quant_given_edge_scales():
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((8, 64)).astype(np.float32)).to(torch.bfloat16)
    x[3] = 0
    g = torch.tensor([0.0, 1e-42, 1e30, float("inf"), 2.0 ** -126, 3.0, 1e-20, 1e20])
    o = oracle.quantize_nvfp4(x, mode="given", given=g)
    h = hm.quantize_nvfp4(x, mode="given", given=g)
    for a, b in zip(o, h):
        assert _eq(a, b)


def test_nvfp4_quant_tensor_mode_and_zero_rows():
    x = synth.moe_nvfp4((1, 32, 128), seed=9)[0]
    x[5] = 0
    for mode in ("tensor", "row"):
        o = oracle.quantize_nvfp4(x, mode=mode)
        h = hm.quantize_nvfp4(x, mode=mode)
        for a, b in zip(o, h):
            assert _eq(a, b)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_nvfp4_dequant_all_codes_scales(dtype):
    rng = np.random.default_rng(8)
    R = 64
    p = torch.arange(256, dtype=torch.uint8).repeat(R, 8)              # K = 4096
    s = torch.arange(256, dtype=torch.uint8).repeat(R, 1)              # every byte
    g = torch.from_numpy(np.concatenate([
        np.exp2(rng.random(R - 6) * 60 - 40), [0.0, 1e-40, 3e38, 2.0 ** -126, 1.0, 6e4]]).astype(np.float32))
    yo = oracle.dequantize_nvfp4(p, s, g, dtype)
    yh = hm.dequantize_nvfp4(p, s, g, dtype)
    nan_o, nan_h = torch.isnan(yo.float()), torch.isnan(yh.float())
    assert torch.equal(nan_o, nan_h)
    assert _eq(yo[~nan_o], yh[~nan_h])


# ------------------------------------------------------------------ cache

@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("C,B", [(512, 32), (128, 32), (512, 16), (120, 32), (100, 16), (96, 7), (64, 64)])
def test_cache_qdq_matches_oracle(fmt, dtype, C, B):
    x = synth.kv_cache((3, 40, C), seed=C + B).to(dtype)
    x[0, 0] = 0
    x[0, 1, : min(C, 40)] = x[0, 1, : min(C, 40)] * 2.0 ** -125
    x[0, 2, :8] = -0.0
    yo = oracle.quantize_cache(x, fmt, B)
    yh = hm.quantize_cache(x, fmt, B)
    assert _eq(yo, yh)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_cache_qdq_all_bf16_values(fmt):
    v = torch.from_numpy(_bf16_all_finite()).to(torch.bfloat16)
    g = torch.Generator().manual_seed(3)
    v = v[torch.randperm(v.numel(), generator=g)]
    v = torch.nn.functional.pad(v, (0, (-v.numel()) % 32)).reshape(-1, 32)
    assert _eq(oracle.quantize_cache(v, fmt, 32), hm.quantize_cache(v, fmt, 32))
    assert _eq(oracle.quantize_cache(v, fmt, 16), hm.quantize_cache(v, fmt, 16))


# ------------------------------------------------------------------ element helpers

def test_e4m3_encoder_exhaustive_against_torch():
    """Every float32 in [2^-9, 448] (the clamped block-scale range)."""
    lo = np.float32(2.0 ** -9).view(np.uint32)
    hi = np.float32(448.0).view(np.uint32)
    step = 1 << 24
    for start in range(int(lo), int(hi) + 1, step):
        bits = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        u = torch.from_numpy(bits.view(np.float32))
        got = hm.apply("hm_e4m3_encode_pos", u, torch.uint8)
        want = u.to(torch.float8_e4m3fn).view(torch.uint8)
        assert torch.equal(got, want), start


def test_e4m3_round_value_exhaustive_against_torch():
    """Every float32 in [0, 448]: the fp8 cache's rounding to the e4m3 grid."""
    hi = int(np.float32(448.0).view(np.uint32))
    step = 1 << 25
    for start in range(0, hi + 1, step):
        bits = np.arange(start, min(start + step, hi + 1), dtype=np.uint32)
        r = torch.from_numpy(bits.view(np.float32))
        got = hm.apply("hm_e4m3_round_value", r, torch.float32)
        want = r.to(torch.float8_e4m3fn).float()
        assert torch.equal(got, want), start


def test_bf16_rounding_against_torch():
    rng = np.random.default_rng(2)
    bits = np.concatenate([rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32),
                           np.arange(0, 1 << 20, dtype=np.uint32)])
    f = torch.from_numpy(bits.view(np.float32))
    f = f[torch.isfinite(f)]
    got = hm.apply("hm_bf16_rne", f, torch.int16)
    assert torch.equal(got, f.to(torch.bfloat16).view(torch.int16))


def test_pow2_ceil_matches_oracle_on_all_exponents():
    rng = np.random.default_rng(4)
    v = np.concatenate([np.exp2(np.arange(-126, 127)),
                        np.exp2(rng.random(100000) * 250 - 125)]).astype(np.float32)
    v = np.concatenate([v, np.nextafter(v, np.float32(np.inf))])
    v = v[np.isfinite(v) & (v < 1.7e38)]
    got = hm.apply("hm_pow2_ceil", torch.from_numpy(v), torch.float32).numpy()
    want = np.array([oracle.pow2_ceil(float(t)) for t in v[:20000]], np.float32)
    assert np.array_equal(got[:20000], want)


def test_f16_rounding_against_torch():
    rng = np.random.default_rng(12)
    bits = np.concatenate([rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32),
                           # every float32 with an exponent in the float16 range and 12 low bits
                           ((np.arange(0x33000000 >> 12, 0x47800000 >> 12, dtype=np.uint32) << 12)
                            | rng.integers(0, 1 << 12, (0x47800000 >> 12) - (0x33000000 >> 12), dtype=np.uint32)),
                           np.array([0x80000000, 0, 0x33000000, 0x33000001, 0x477FEFFF, 0x477FF000], np.uint32)])
    f = torch.from_numpy(bits.view(np.float32))
    f = torch.cat([f, -f])
    f = f[~torch.isnan(f)]
    got = hm.apply("hm_f16_rne", f, torch.int16)
    assert torch.equal(got, f.to(torch.float16).view(torch.int16))


@pytest.mark.parametrize("wide", [0, 1])
def test_nvfp4_binary64_division_shortcut_stress(wide):
    """The kernels replace float32 divisions by binary64 products; on random
    and boundary-hugging pairs the decisions must match IEEE float32 division."""
    assert hm.lib().hm_nv_division_stress(3_000_000, 1234 + wide, wide) == 0


def test_cache_scale_binary64_quotients_exhaustive():
    """The cache scales take a / 6 and a / 448 as binary64 products rounded
    once to float32: over every non-negative finite float32 they equal IEEE
    float32 division (a / 448 wherever the quotient is at least 2^-126, and
    after the clamp to 2^-126 everywhere)."""
    assert hm.lib().hm_scale_division_check() == 0


def test_rounding_up_to_22_bits_keeps_every_e2m1_decision():
    """Exhaustive over all float32 magnitudes below 16 (about 1.1e9 values)."""
    assert hm.lib().hm_ceil22_check() == 0


def test_ties_to_even_model_on_grid_and_midpoints():
    """The host model of the fp4 converter (nearest, ties to the even code,
    saturating at 6) on every e2m1 value and midpoint."""
    assert hm.lib().hm_rne_model_check() == 0


def test_half_down_operand_step_keeps_every_e2m1_decision():
    """Exhaustive over all float32 magnitudes below 16, both signs (about
    2.2e9 values): ties-to-even rounding of half_down_for_rne(q) equals the
    round-half-down code of q, sign kept."""
    assert hm.lib().hm_half_down_check() == 0
