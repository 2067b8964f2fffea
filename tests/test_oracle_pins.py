"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: every expected value comes from
numbers printed on the pages (tests/golden), from closed forms evaluated in a
different way (exact float64 / Python integers), from library routines (torch's
CPU casts), from characterising properties, or from brute-force searches.
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import load_golden

G = load_golden("e2m1_tables.txt")
TABLE13 = [float(v) for v in G["e2m1_table"]]
MIDS = [float(v) for v in G["e2m1_midpoints"]]
MAGS = TABLE13[:8]


# ------------------------------------------------------------------ tables

def test_e2m1_table_matches_printed_values():
    for c, v in enumerate(TABLE13):
        got = oracle.e2m1_decode(c)
        assert got == v, (c, got, v)
        assert math.copysign(1.0, got) == math.copysign(1.0, v)
    # index 8 is printed as a plain 0.0: positive zero
    assert math.copysign(1.0, oracle.e2m1_decode(8)) == 1.0
    # entries 13..15 are cut off on the page: sign symmetry and E2M1_MAX = 6
    for c in range(1, 8):
        assert oracle.e2m1_decode(8 + c) == -oracle.e2m1_decode(c)
    assert max(oracle.e2m1_decode(c) for c in range(16)) == float(G["e2m1_max"][0])


def test_midpoints_are_the_printed_means_of_neighbours():
    # closed form: every printed midpoint is the mean of adjacent magnitudes
    for j, t in enumerate(MIDS):
        assert t == (MAGS[j] + MAGS[j + 1]) / 2


def test_round_mag_switches_exactly_at_printed_midpoints():
    # a value on a midpoint takes the lower bucket; one ulp above takes the upper
    for j, t in enumerate(MIDS):
        t32 = np.float32(t)
        above = np.nextafter(t32, np.float32(np.inf))
        below = np.nextafter(t32, np.float32(0))
        assert oracle.e2m1_round_mag(float(t32)) == j
        assert oracle.e2m1_round_mag(float(above)) == j + 1
        assert oracle.e2m1_round_mag(float(below)) == j
        assert oracle.e2m1_round_mag(-float(above)) == j + 1
    assert oracle.e2m1_round_mag(7.9) == 7
    assert oracle.e2m1_round_mag(1e30) == 7
    assert oracle.e2m1_round_mag(float("nan")) == 0


def _nearest_mag_bruteforce(q: np.ndarray) -> np.ndarray:
    """Nearest of the 8 printed magnitudes; on a tie the smaller magnitude
    (np.argmin returns the first of equal minima, magnitudes ascend)."""
    # clip: beyond 7 every magnitude is nearest to 6, and float64 cannot tell
    # huge values apart from huge - 6
    a = np.minimum(np.abs(q.astype(np.float64)), 1e6)[:, None]
    return np.argmin(np.abs(a - np.array(MAGS)[None, :]), axis=1)


def test_round_mag_bruteforce_all_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    # values far above the table saturate, so compare on the full range
    want = _nearest_mag_bruteforce(f)
    got = np.array([oracle.e2m1_round_mag(float(v)) for v in f])
    assert np.array_equal(got, want)


def test_round_mag_bruteforce_random_fp32():
    rng = np.random.default_rng(11)
    f = (rng.random(20000) * 8.0).astype(np.float32)
    # add exact midpoints and their float32 neighbours
    extra = []
    for t in MIDS:
        t32 = np.float32(t)
        extra += [t32, np.nextafter(t32, np.float32(9)), np.nextafter(t32, np.float32(0))]
    f = np.concatenate([f, np.array(extra, dtype=np.float32)])
    want = _nearest_mag_bruteforce(f)
    got = np.array([oracle.e2m1_round_mag(float(v)) for v in f])
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ e4m3 / e8m0 / bf16

def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64)
    for i in range(256):
        got = oracle.e4m3_decode(i)
        r = ref[i].item()
        if math.isnan(r):
            assert math.isnan(got)
        else:
            assert got == r and math.copysign(1, got) == math.copysign(1, r)


def _e4m3_candidates():
    vals = [float(oracle.e4m3_decode(b)) for b in range(0x7F)]
    out = set()
    for v in vals:
        v32 = np.float32(v)
        out.update([v32, np.nextafter(v32, np.float32(1e9)),
                    np.nextafter(v32, np.float32(0))])
    for a, b in zip(vals[:-1], vals[1:]):
        m = np.float32((a + b) / 2)  # exact: e4m3 midpoints fit in float32
        out.update([m, np.nextafter(m, np.float32(1e9)), np.nextafter(m, np.float32(0))])
    return np.array(sorted(out), dtype=np.float32)


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        _e4m3_candidates(),
        (rng.random(30000) * 448).astype(np.float32),
        np.exp2(rng.random(30000) * 18 - 12).astype(np.float32),
        ((np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)),
    ])
    v = v[np.isfinite(v) & (v >= 0) & (v <= 448)]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(x)) for x in v], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])
    # negative values keep the sign bit
    assert oracle.e4m3_encode(-1.0) == 0x80 | oracle.e4m3_encode(1.0)
    assert oracle.e4m3_encode(-0.0) == 0x80


def test_e4m3_encode_saturates_between_448_and_464():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(460.0) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E   # tie: 448 has the even mantissa
    assert oracle.e4m3_encode(float(np.nextafter(np.float32(448), np.float32(500)))) == 0x7E


def test_e8m0_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64)
    for i in range(255):
        assert oracle.e8m0_decode(i) == ref[i].item() == math.ldexp(1.0, i - 127)
    assert math.isnan(oracle.e8m0_decode(255)) and math.isnan(ref[255].item())


def test_round_binary_bf16_f16_match_torch():
    rng = np.random.default_rng(9)
    bits = np.concatenate([
        rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32),
        # exact bf16 ties and near-ties, subnormals included
        ((rng.integers(0, 1 << 16, 20000, dtype=np.uint32) << 16) | 0x8000),
        ((rng.integers(0, 1 << 16, 20000, dtype=np.uint32) << 16) | 0x7FFF),
        rng.integers(0, 1 << 23, 20000, dtype=np.uint32),
    ]).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.0e38)]
    t = torch.from_numpy(f.copy())
    ref_bf = t.to(torch.bfloat16).to(torch.float64).numpy()
    got_bf = np.array([oracle.round_binary(float(x), 8, -126) for x in f])
    assert np.array_equal(got_bf, ref_bf)
    small = f[np.abs(f) < 65504.0]
    ref_h = torch.from_numpy(small.copy()).to(torch.float16).to(torch.float64).numpy()
    got_h = np.array([oracle.round_binary(float(x), 11, -14) for x in small])
    assert np.array_equal(got_h, ref_h)


def test_store_rounds_like_torch_casts():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 5, 4000),
                           [0.0, -0.0, 1e-45, 3e-39, 65519.0, 65520.0, 7e4, -7e4,
                            6e-8, 2.9e-8, 3.0e-8, 3e38, 3.4e38]]).astype(np.float32)
    x = torch.from_numpy(vals)
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        got = oracle.store_values(x, dt)
        want = x.to(dt)
        assert torch.equal(got.view(torch.int16 if dt != torch.float32 else torch.int32),
                           want.view(torch.int16 if dt != torch.float32 else torch.int32)), dt


def test_floor_log2_exact_including_near_powers_and_subnormals():
    cases = [1.0, 2.0, 3.0, 2.0 ** 20 * (1 - 2.0 ** -24), 2.0 ** -126, 2.0 ** -149,
             2.0 ** -130 * 1.5, 3.4028234663852886e38, 0.3]
    for a in cases:
        a32 = float(np.float32(a))
        want = math.frexp(a32)[1] - 1  # exact in double
        assert oracle.floor_log2(a32) == want
        assert 2.0 ** want <= a32 < 2.0 ** (want + 1)


def test_pow2_ceil_characterisation():
    rng = np.random.default_rng(1)
    v = np.exp2(rng.random(50000) * 250 - 125).astype(np.float32)
    v = np.concatenate([v, np.exp2(np.arange(-126, 128)).astype(np.float32),
                        np.nextafter(np.exp2(np.arange(-126, 127)).astype(np.float32),
                                     np.float32(np.inf))])
    for x in v:
        p = oracle.pow2_ceil(float(x))
        m, _ = math.frexp(p)
        assert m == 0.5, (x, p)           # a power of two
        assert p >= x and p / 2 < x, (x, p)  # the smallest such power >= x


# ------------------------------------------------------------------ MXFP4

def _bf16_from_float(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)


def test_nibble_order_worked_case():
    g = load_golden("nibble_order.txt")
    vals = [float(v) for v in g["values"]]
    block = vals + [0.0] * (32 - len(vals))
    packed, scales = oracle.quantize_mxfp4(torch.tensor([block], dtype=torch.float32))
    want = [int(b, 16) for b in g["bytes"]]
    assert packed[0, :2].tolist() == want
    assert scales[0, 0].item() == 127     # max 6.0: floor(log2 6) - 2 = 0
    assert packed[0, 2:].tolist() == [0] * 14


def test_mxfp4_scale_characterisation_all_bf16_amax():
    # every positive finite bf16 value as the block amax
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (bits << 16).view(np.float32)
    x = torch.zeros(amax.size, 32, dtype=torch.float32)
    x[:, 5] = torch.from_numpy(amax)
    x[:, 17] = -torch.from_numpy(amax) / 3
    packed, scales = oracle.quantize_mxfp4(x.to(torch.bfloat16))
    b = scales[:, 0].numpy().astype(np.int64)
    e = b - 127
    a64 = amax.astype(np.float64)
    ratio = a64 / np.exp2(e.astype(np.float64))
    normal = b > 0
    # the scaled amax lands in [4, 8): the unique power of two with that property
    assert np.all((ratio[normal] >= 4) & (ratio[normal] < 8))
    # where no e8m0 exponent is small enough, the scale is the smallest one
    assert np.all(ratio[~normal] < 8)
    # the byte is torch's e8m0 encoding of the power-of-two scale
    ref = torch.from_numpy(np.exp2(e.astype(np.float32))).to(torch.float8_e8m0fnu)
    assert np.array_equal(ref.view(torch.uint8).numpy(), b.astype(np.uint8))
    # the max element rounds to 4 or 6 (codes 6/7) when the scale is exact
    hi = (packed[:, 2] & 0xF0) >> 4
    assert np.all(np.isin(hi.numpy()[normal], [6, 7]))


def test_mxfp4_scale_fp32_edge_amax():
    cases = [2.0 ** 20 * (1 - 2.0 ** -24), 2.0 ** 20, 1.0, 2.0 ** -125, 2.0 ** -126,
             2.0 ** -127, 2.0 ** -149, 1e-30, 3.4028234663852886e38, 0.0]
    x = torch.zeros(len(cases), 32, dtype=torch.float32)
    x[:, 0] = torch.tensor(cases, dtype=torch.float32)
    _, scales = oracle.quantize_mxfp4(x)
    for a, b in zip(cases, scales[:, 0].tolist()):
        a32 = float(np.float32(a))
        if a32 == 0.0:
            assert b == 0
            continue
        e = math.frexp(a32)[1] - 1 - 2
        assert b == max(e, -127) + 127, (a, b)


def _representable_blocks(rng, n, exp_lo=-120, exp_hi=120):
    codes = rng.integers(0, 16, size=(n, 32))
    s = rng.integers(exp_lo, exp_hi, size=(n, 1))
    vals = np.array(TABLE13 + [-3.0, -4.0, -6.0])[codes] * np.exp2(s.astype(np.float64))
    return vals


def test_mxfp4_roundtrip_claim_representable_values():
    """The mxfp4 page states that values which are already exactly
    representable come back value-exactly from quantize then dequantize."""
    rng = np.random.default_rng(7)
    vals = _representable_blocks(rng, 3000)
    x32 = torch.from_numpy(vals.astype(np.float32))
    for xin in (x32, x32.to(torch.bfloat16)):
        p, s = oracle.quantize_mxfp4(xin)
        for dt in (torch.float32, torch.bfloat16):
            y = oracle.dequantize_mxfp4(p, s, dt)
            assert torch.equal(y.float(), xin.float()), dt


def test_mxfp4_dequant_closed_form_all_codes_all_scales():
    codes = np.arange(16)
    packed = torch.tensor([[(c | (c << 4)) for c in codes] * 2], dtype=torch.uint8)  # K=64
    for b in range(256):
        scales = torch.tensor([[b, b]], dtype=torch.uint8)
        y32 = oracle.dequantize_mxfp4(packed, scales, torch.float32)[0].numpy()
        ybf = oracle.dequantize_mxfp4(packed, scales, torch.bfloat16)[0].float().numpy()
        full_table = TABLE13 + [-3.0, -4.0, -6.0]
        for k in range(64):
            c = codes[(k // 2) % 16]
            if b == 255:
                assert np.isnan(y32[k])
                continue
            want = full_table[c] * 2.0 ** (b - 127)   # exact in float64
            want32 = np.float32(want) if abs(want) < 3.5e38 else np.float32(np.inf) * np.sign(want)
            assert y32[k] == want32 or (np.isinf(want32) and np.isinf(y32[k]))
            assert np.signbit(y32[k]) == (want < 0)
            wbf = torch.tensor(float(want32)).to(torch.bfloat16).float().item()
            assert ybf[k] == wbf or (math.isinf(wbf) and math.isinf(ybf[k]))


def test_mxfp4_zero_blocks_and_negative_zero():
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    x[1] = -0.0
    p, s = oracle.quantize_mxfp4(x)
    assert s.eq(0).all()
    assert p[0].eq(0).all()
    assert p[1].eq(0x88).all()       # sign nibble kept for -0.0 (reading R2)
    y = oracle.dequantize_mxfp4(p, s, torch.float32)
    assert y.eq(0).all() and not torch.signbit(y).any()   # decode gives +0.0


def test_mxfp4_idempotent_on_dequantized_values():
    import synth
    x = synth.moe_mxfp4((2, 64, 256), seed=77)
    p, s = oracle.quantize_mxfp4(x)
    y = oracle.dequantize_mxfp4(p, s, torch.bfloat16)
    p2, s2 = oracle.quantize_mxfp4(y)
    y2 = oracle.dequantize_mxfp4(p2, s2, torch.bfloat16)
    assert torch.equal(y, y2)


def test_mxfp4_nearest_value_property():
    """Every dequantized value is the nearest of the 8 magnitudes (times the
    block scale) to the input, ties to the smaller magnitude."""
    import synth
    x = synth.moe_mxfp4((1, 32, 512), seed=5).float()
    p, s = oracle.quantize_mxfp4(x)
    y = oracle.dequantize_mxfp4(p, s, torch.float32)
    scale = torch.exp2(s.double() - 127).repeat_interleave(32, dim=-1)
    q = (x.double() / scale).abs().numpy().reshape(-1)
    want_mag = np.array(MAGS)[_nearest_mag_bruteforce(q)]
    got_mag = (y.double() / scale).abs().numpy().reshape(-1)
    assert np.array_equal(got_mag, want_mag)


# ------------------------------------------------------------------ NVFP4

def _nvfp4_bruteforce(x: torch.Tensor, g_given=None):
    """Independent re-derivation for tiny inputs: numpy float32 arithmetic in
    the order the nvfp4 page writes it, torch's e4m3 cast for the block scale,
    and a nearest-magnitude search for the codes."""
    xf = x.float().numpy().reshape(-1, x.shape[-1])
    R, K = xf.shape
    codes = np.zeros((R, K), np.int64)
    sbytes = np.zeros((R, K // 16), np.uint8)
    gs = np.zeros(R, np.float32)
    for r in range(R):
        if g_given is None:
            g = np.float32(np.abs(xf[r]).max()) / np.float32(2688.0)
        else:
            g = np.float32(g_given[r])
        gs[r] = g
        for b in range(K // 16):
            blk = xf[r, 16 * b:16 * b + 16]
            a = np.float32(np.abs(blk).max())
            with np.errstate(divide="ignore", invalid="ignore"):
                u = (a / np.float32(6.0)) / g
            u = np.float32(2.0 ** -9) if np.isnan(u) else np.float32(min(max(u, 2.0 ** -9), 448.0))
            sb = torch.tensor([u]).to(torch.float8_e4m3fn)
            sbytes[r, b] = sb.view(torch.uint8).item()
            sigma = np.float32(sb.float().item())
            den = np.float32(sigma * g)
            with np.errstate(divide="ignore", invalid="ignore"):
                q = blk / den
            q = np.where(np.isnan(q), 0, q)
            mag = _nearest_mag_bruteforce(np.minimum(np.abs(q), 1e30).astype(np.float32))
            codes[r, 16 * b:16 * b + 16] = mag | (np.signbit(blk).astype(np.int64) << 3)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbytes, gs


def test_nvfp4_bruteforce_tiny_rows():
    import synth
    x = synth.moe_nvfp4((2, 16, 64), seed=8)
    p, s, g = oracle.quantize_nvfp4(x)
    bp, bs, bg = _nvfp4_bruteforce(x)
    assert np.array_equal(g.numpy().reshape(-1), bg)
    assert np.array_equal(s.numpy().reshape(bs.shape), bs)
    assert np.array_equal(p.numpy().reshape(bp.shape), bp)


def test_nvfp4_bruteforce_given_scale_and_fp32_input():
    rng = np.random.default_rng(4)
    x = torch.from_numpy((rng.standard_normal((24, 48)) * np.exp2(rng.integers(-10, 10, (24, 1)))).astype(np.float32))
    gvals = torch.from_numpy(np.exp2(rng.random(24) * 10 - 12).astype(np.float32))
    p, s, g = oracle.quantize_nvfp4(x, mode="given", given=gvals)
    bp, bs, bg = _nvfp4_bruteforce(x, g_given=gvals.numpy())
    assert np.array_equal(g.numpy(), bg)
    assert np.array_equal(s.numpy(), bs)
    assert np.array_equal(p.numpy(), bp)


def test_nvfp4_row_max_block_gets_448_and_code_7():
    import synth
    x = synth.moe_nvfp4((4, 32, 256), seed=21)
    p, s, g = oracle.quantize_nvfp4(x)
    xf = x.float().reshape(-1, 256)
    codes = torch.stack([p.reshape(-1, 128) & 15, p.reshape(-1, 128) >> 4], -1).reshape(-1, 256)
    for r in range(xf.shape[0]):
        k = int(xf[r].abs().argmax())
        assert s.reshape(-1, 16)[r, k // 16].item() == 0x7E
        assert (codes[r, k] & 7).item() == 7


def test_nvfp4_power_of_two_covariance():
    import synth
    x = synth.moe_nvfp4((2, 16, 128), seed=12)
    p, s, g = oracle.quantize_nvfp4(x)
    for k in (-20, -3, 5, 30):
        xk = (x.float() * 2.0 ** k).to(torch.bfloat16)   # exact
        pk, sk, gk = oracle.quantize_nvfp4(xk)
        assert torch.equal(pk, p) and torch.equal(sk, s)
        assert torch.equal(gk, g * 2.0 ** k)


def test_nvfp4_rows_are_independent():
    import synth
    x = synth.moe_nvfp4((1, 64, 128), seed=13)[0]
    perm = torch.randperm(64, generator=torch.Generator().manual_seed(0))
    p, s, g = oracle.quantize_nvfp4(x)
    pp, sp, gp = oracle.quantize_nvfp4(x[perm])
    assert torch.equal(pp, p[perm]) and torch.equal(sp, s[perm]) and torch.equal(gp, g[perm])


def test_nvfp4_tensor_mode_equals_given_tensor_amax():
    import synth
    x = synth.moe_nvfp4((1, 32, 64), seed=14)[0]
    p, s, g = oracle.quantize_nvfp4(x, mode="tensor")
    gt = np.float32(x.float().abs().max().item()) / np.float32(2688.0)
    assert torch.all(g == torch.tensor(gt))
    p2, s2, g2 = oracle.quantize_nvfp4(x, mode="given", given=torch.tensor([gt]))
    assert torch.equal(p, p2) and torch.equal(s, s2)


def test_nvfp4_zero_row():
    x = torch.zeros(3, 32, dtype=torch.bfloat16)
    p, s, g = oracle.quantize_nvfp4(x)
    assert p.eq(0).all() and s.eq(1).all() and g.eq(0).all()
    y = oracle.dequantize_nvfp4(p, s, g, torch.bfloat16)
    assert y.eq(0).all() and not torch.signbit(y.float()).any()


def test_nvfp4_dequant_closed_form_and_order_sensitivity():
    rng = np.random.default_rng(2)
    codes = np.arange(16)
    full_table = np.array(TABLE13 + [-3.0, -4.0, -6.0])
    sbytes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    R = 400
    g = np.exp2(rng.random(R) * 40 - 30).astype(np.float32) * (1 + rng.random(R)).astype(np.float32)
    K = 16 * sbytes.size
    codes_rk = np.tile(np.repeat(codes, 1)[None, :], (R, K // 16))
    packed = torch.from_numpy((codes_rk[:, 0::2] | (codes_rk[:, 1::2] << 4)).astype(np.uint8))
    scales = torch.from_numpy(np.tile(sbytes[None, :], (R, 1)))
    y = oracle.dequantize_nvfp4(packed, scales, torch.from_numpy(g), torch.float32).numpy()
    sig = torch.from_numpy(sbytes).view(torch.float8_e4m3fn).double().numpy()
    D = full_table[codes_rk]
    S = np.repeat(sig, 16)[None, :]
    exact = D * S * g.astype(np.float64)[:, None]        # <= 30 significant bits: exact
    want = exact.astype(np.float32)                       # one rounding to float32
    assert np.array_equal(y, want)
    ybf = oracle.dequantize_nvfp4(packed, scales, torch.from_numpy(g), torch.bfloat16)
    assert torch.equal(ybf, torch.from_numpy(want).to(torch.bfloat16))
    # the stated order matters: D * (sigma * g) rounds differently somewhere
    alt = (D.astype(np.float32) * (S.astype(np.float32) * g[:, None])).astype(np.float32)
    assert not np.array_equal(alt, want)


def test_nvfp4_idempotent_on_blocks_with_max_code_7():
    """Re-quantizing dequantized values with the same row scale reproduces a
    block exactly when its largest magnitude code is 7 (that block's scale is
    recovered exactly, and every value is an exact grid point)."""
    import synth
    x = synth.moe_nvfp4((2, 32, 256), seed=31)
    p, s, g = oracle.quantize_nvfp4(x)
    y = oracle.dequantize_nvfp4(p, s, g, torch.bfloat16)
    p2, s2, g2 = oracle.quantize_nvfp4(y, mode="given", given=g.reshape(-1))
    y2 = oracle.dequantize_nvfp4(p2, s2, g2, torch.bfloat16)
    codes = torch.stack([p & 15, p >> 4], -1).reshape(y.shape)
    blk_max = (codes & 7).reshape(*y.shape[:-1], -1, 16).amax(-1)
    sel = (blk_max == 7)
    yb = y.reshape(*y.shape[:-1], -1, 16)[sel]
    y2b = y2.reshape(*y.shape[:-1], -1, 16)[sel]
    assert sel.sum() > 0.5 * sel.numel()
    assert torch.equal(yb, y2b)


def test_nvfp4_storage_density():
    g = load_golden("storage_density.txt")
    R, K = 48, 4096
    x = torch.randn(R, K).to(torch.bfloat16)
    p, s, rs = oracle.quantize_nvfp4(x)
    total = p.numel() * p.element_size() + s.numel() * s.element_size() + rs.numel() * 4
    assert total == float(g["nvfp4_bytes_per_param"][0]) * R * K + float(g["nvfp4_bytes_per_row"][0]) * R
    pm, sm = oracle.quantize_mxfp4(x)
    assert pm.numel() + sm.numel() == float(g["mxfp4_bytes_per_param"][0]) * R * K


# ------------------------------------------------------------------ cache QDQ

def _pow2ceil_torch(v: torch.Tensor) -> torch.Tensor:
    m, e = torch.frexp(v)               # v = m * 2^e, m in [0.5, 1)
    return torch.where(m == 0.5, v, torch.ldexp(torch.ones_like(v), e))


def _groups(x: torch.Tensor, B: int):
    C = x.shape[-1]
    pad = (-C) % B
    xp = torch.nn.functional.pad(x.float(), (0, pad))
    return xp.reshape(*x.shape[:-1], -1, B), C


def test_cache_fp8_matches_torch_cast_composition():
    import synth
    for C, B in ((512, 32), (120, 32), (96, 16)):
        x = synth.kv_cache((3, 17, C), seed=C + B)
        xg, _ = _groups(x, B)
        a = xg.abs().amax(-1, keepdim=True)
        v = torch.clamp_min(a / 448.0, torch.finfo(torch.float32).tiny)
        s = _pow2ceil_torch(v)
        want = ((xg / s).to(torch.float8_e4m3fn).float() * s).reshape(*x.shape[:-1], -1)[..., :C]
        got = oracle.quantize_cache(x, "fp8", B)
        assert got.dtype == x.dtype and got.shape == x.shape
        assert torch.equal(got, want.to(torch.bfloat16))


def _e2m1_qdq_bruteforce(q: torch.Tensor) -> torch.Tensor:
    mag = np.array(MAGS)[_nearest_mag_bruteforce(q.double().numpy().reshape(-1))]
    return torch.from_numpy(mag).reshape(q.shape)


def test_cache_mxfp4_matches_composition():
    import synth
    for C, B in ((128, 32), (120, 32), (64, 8)):
        x = synth.kv_cache((4, 9, C), seed=C * 3 + B)
        xg, _ = _groups(x, B)
        a = xg.abs().amax(-1, keepdim=True)
        s = _pow2ceil_torch(torch.clamp_min(a / 6.0, torch.finfo(torch.float32).tiny))
        mag = _e2m1_qdq_bruteforce(xg / s).float()
        val = torch.where(xg < 0, -mag, mag) * s
        want = val.reshape(*x.shape[:-1], -1)[..., :C].to(torch.bfloat16)
        got = oracle.quantize_cache(x, "mxfp4", B)
        assert torch.equal(got.float(), want.float())


def test_cache_nvfp4_matches_composition():
    import synth
    for C, B in ((512, 16), (120, 16), (96, 32)):
        x = synth.kv_cache((3, 11, C), seed=C * 5 + B)
        xg, _ = _groups(x, B)
        a = xg.abs().amax(-1, keepdim=True)
        u = torch.clamp(a / 6.0, 2.0 ** -9, 448.0)
        sigma = u.to(torch.float8_e4m3fn).float()
        mag = _e2m1_qdq_bruteforce(xg / sigma).float()
        val = torch.where(xg < 0, -mag, mag) * sigma
        want = val.reshape(*x.shape[:-1], -1)[..., :C].to(torch.bfloat16)
        got = oracle.quantize_cache(x, "nvfp4", B)
        assert torch.equal(got.float(), want.float())


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_cache_partial_group_equals_zero_padding(fmt):
    import synth
    B = 16 if fmt == "nvfp4" else 32
    x = synth.kv_cache((5, 7, 100), seed=99)
    xp = torch.nn.functional.pad(x, (0, (-100) % B))
    got = oracle.quantize_cache(x, fmt, B)
    want = oracle.quantize_cache(xp, fmt, B)[..., :100]
    assert torch.equal(got, want)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_cache_idempotent(fmt):
    import synth
    x = synth.kv_cache((4, 16, 256), seed=123)
    y = oracle.quantize_cache(x, fmt, 32)
    assert torch.equal(oracle.quantize_cache(y, fmt, 32), y)


def test_cache_zero_and_shape_dtype():
    for dt in (torch.float32, torch.bfloat16, torch.float16):
        x = torch.zeros(2, 3, 40, dtype=dt)
        for fmt, B in (("fp8", 32), ("mxfp4", 32), ("nvfp4", 16), ("mxfp4", 7)):
            y = oracle.quantize_cache(x, fmt, B)
            assert y.shape == x.shape and y.dtype == dt
            assert y.eq(0).all()


def test_cache_fp8_keeps_negative_zero_fp4_formats_do_not():
    x = torch.zeros(1, 32, dtype=torch.bfloat16)
    x[0, 0] = 1.0
    x[0, 1] = -1e-30     # underflows to zero in every format
    y8 = oracle.quantize_cache(x, "fp8", 32)
    y4 = oracle.quantize_cache(x, "mxfp4", 32)
    assert torch.signbit(y8[0, 1].float()) and y8[0, 1].item() == 0
    assert not torch.signbit(y4[0, 1].float()) and y4[0, 1].item() == 0


# ------------------------------------------------------------------ grouped GEMM
# [mxfp4 page] MXFP4GroupedMM.forward / backward and [nvfp4 page]
# NVFP4GroupedMM.forward / backward: expert e multiplies its contiguous token
# rows by W_e^T (forward) or W_e (backward); offs holds cumulative counts.

def _brute_grouped_mm(x, w, offs, trans):
    """Pure-Python loops over exact Fractions of the float values."""
    from fractions import Fraction
    T, din = x.shape
    E, N, K = w.shape
    dout = K if trans else N
    out = [[Fraction(0)] * dout for _ in range(T)]
    lo = 0
    for e in range(E):
        hi = int(offs[e])
        for r in range(lo, hi):
            for o in range(dout):
                acc = Fraction(0)
                for d in range(din):
                    wv = float(w[e, d, o]) if trans else float(w[e, o, d])
                    acc += Fraction(float(x[r, d])) * Fraction(wv)
                out[r][o] = acc
        lo = max(lo, hi)
    return out


@pytest.mark.parametrize("trans", [False, True])
def test_grouped_mm_bruteforce_tiny(trans):
    g = torch.Generator().manual_seed(5)
    E, N, K = 3, 5, 7
    offs = torch.tensor([3, 3, 6], dtype=torch.int32)      # expert 1 has no tokens
    T = 8                                                   # rows 6, 7 belong to no expert
    x = torch.randn(T, N if trans else K, generator=g).to(torch.bfloat16)
    w = torch.randn(E, N, K, generator=g).to(torch.bfloat16)
    out, absout = oracle.grouped_mm(x, w, offs, trans)
    ref = _brute_grouped_mm(x.float(), w.float(), offs, trans)
    for r in range(T):
        for o in range(out.shape[1]):
            assert out[r, o].item() == float(ref[r][o]), (r, o)
    assert torch.all(out[6:] == 0) and torch.all(absout[6:] == 0)
    assert torch.all(absout >= out.abs())


def test_grouped_mm_expert_isolation_and_scaling():
    g = torch.Generator().manual_seed(6)
    E, N, K, T = 4, 6, 10, 12
    offs = torch.tensor([2, 5, 9, 12], dtype=torch.int32)
    x = torch.randn(T, K, generator=g).to(torch.bfloat16)
    w = torch.randn(E, N, K, generator=g).to(torch.bfloat16)
    out, _ = oracle.grouped_mm(x, w, offs, False)
    w2 = w.clone()
    w2[2] = torch.randn(N, K, generator=g).to(torch.bfloat16)
    out2, _ = oracle.grouped_mm(x, w2, offs, False)
    assert torch.equal(out[:5], out2[:5]) and torch.equal(out[9:], out2[9:])
    assert not torch.equal(out[5:9], out2[5:9])
    out4, _ = oracle.grouped_mm((x.float() * 4).to(torch.bfloat16), w, offs, False)
    assert torch.equal(out4, out * 4)                       # power-of-two scaling is exact
    # the backward product with the transposed weights [E, K, N] is the forward one
    outb, _ = oracle.grouped_mm(x, w.transpose(1, 2).contiguous(), offs, True)
    assert torch.equal(outb, out)
