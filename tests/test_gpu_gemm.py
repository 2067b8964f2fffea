"""GPU parity of the grouped GEMM over packed fp4 expert weights
([mxfp4 page] MXFP4GroupedMM, [nvfp4 page] NVFP4GroupedMM: forward x @ W_e^T,
backward x @ W_e) against the oracle's binary64 sums, through the C ABI.

Tolerance, from the arithmetic: every product of two bfloat16 values is exact
in float32; a float32 sum of R products in any order is within
(R - 1) * 2^-24 * sum|x w| of the exact sum (the bound is doubled here for
accumulators that do not round each addition to nearest); one final rounding
to bfloat16 adds at most 2^-9 relative.  So |y - ref| <= 2^-8 |ref| +
R * 2^-22 * sum|x w|.  The weights are quantized by the oracle (never by the
GPU path) and dequantized by it to bfloat16, as the pages' dequantize-then-
grouped-matmul does; rows outside every expert's group must stay untouched."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def mxq():
    import fp8_quantize_pack_amd as m
    return m


def say(*a):
    print("[gemm]", *a, flush=True)


def _offs(counts):
    return torch.tensor(np.cumsum(counts), dtype=torch.int32)


def _weights(fmt, E, N, K, seed):
    w = synth.moe_mxfp4((E, N, K), seed=seed) if fmt == "mxfp4" else synth.moe_nvfp4((E, N, K), seed=seed)
    if fmt == "mxfp4":
        p, s = oracle.quantize_mxfp4(w)
        wd = oracle.dequantize_mxfp4(p, s, torch.bfloat16)
        return (p, s), wd
    p, s, g = oracle.quantize_nvfp4(w)
    wd = oracle.dequantize_nvfp4(p, s, g, torch.bfloat16)
    return (p, s, g), wd


def _run(fmt, q, x, offs, transpose, y):
    m = mxq()
    xd, od = x.to(DEV), offs.to(DEV)
    if fmt == "mxfp4":
        p, s = q
        m.mxq_grouped_mm_mxfp4(xd, p.to(DEV).view(torch.int8), s.to(DEV), od, y, transpose)
    else:
        p, s, g = q
        m.mxq_grouped_mm_nvfp4(xd, p.to(DEV), s.to(DEV), g.to(DEV), od, y, transpose)
    torch.cuda.synchronize()
    return y.cpu()


def _check(y, ref, absref, R, what):
    yd = y.double()
    tol = ref.abs() * 2.0 ** -8 + absref * R * 2.0 ** -22
    bad = (yd - ref).abs() > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs beyond the bound; worst "
                           f"{float(((yd - ref).abs() - tol).max())}")
    # the bound is not vacuous: most outputs are the correctly rounded sum
    exact = (y == ref.to(torch.bfloat16)).double().mean().item()
    assert exact > 0.9, f"{what}: only {exact:.3f} of the outputs are the rounded exact sum"


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("transpose", [False, True])
def test_grouped_mm_small_ragged(fmt, transpose):
    """Three experts with 100, 0 and 213 tokens, 11 trailing rows in no group."""
    E, N, K = 3, 256, 384
    counts = [100, 0, 213]
    T = sum(counts) + 11
    say(fmt, "transpose" if transpose else "forward", E, N, K, T)
    q, wd = _weights(fmt, E, N, K, seed=31)
    g = torch.Generator().manual_seed(32)
    x = torch.randn(T, N if transpose else K, generator=g).to(torch.bfloat16)
    offs = _offs(counts)
    sentinel = torch.full((T, K if transpose else N), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = _run(fmt, q, x, offs, transpose, sentinel)
    ref, absref = oracle.grouped_mm(x, wd, offs, transpose)
    T0 = sum(counts)
    _check(y[:T0], ref[:T0], absref[:T0], N if transpose else K, fmt)
    assert torch.isnan(y[T0:].float()).all(), "rows outside every group were written"


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_grouped_mm_tile_edges(fmt):
    """Groups that start and end inside 128-row tiles, single-token experts,
    and a leading empty expert."""
    E, N, K = 6, 128, 256
    counts = [0, 1, 127, 129, 1, 255]
    T = sum(counts)
    q, wd = _weights(fmt, E, N, K, seed=33)
    x = torch.randn(T, K, generator=torch.Generator().manual_seed(34)).to(torch.bfloat16)
    offs = _offs(counts)
    y = _run(fmt, q, x, offs, False, torch.empty(T, N, dtype=torch.bfloat16, device=DEV))
    ref, absref = oracle.grouped_mm(x, wd, offs, False)
    _check(y, ref, absref, K, fmt)


def test_grouped_mm_wrapper_shapes_and_errors():
    m = mxq()
    E, N, K = 2, 128, 128
    q, wd = _weights("mxfp4", E, N, K, seed=35)
    x = torch.randn(10, K).to(torch.bfloat16).to(DEV)
    offs = _offs([4, 6]).to(DEV)
    y = m.grouped_mm_mxfp4(x, q[0].to(DEV).view(torch.int8), q[1].to(DEV), offs)
    assert y.shape == (10, N) and y.dtype == torch.bfloat16
    with pytest.raises(ValueError):
        m.grouped_mm_mxfp4(x[:, :64], q[0].to(DEV).view(torch.int8), q[1].to(DEV), offs)
    with pytest.raises(TypeError):
        m.grouped_mm_mxfp4(x.float(), q[0].to(DEV).view(torch.int8), q[1].to(DEV), offs)


# ------------------------------------------------------------------ per-expert shapes of C2 / C3

@pytest.mark.parametrize("transpose", [False, True])
def test_grouped_mm_mxfp4_c2_expert_shape(transpose):
    """MXFP4 experts of the MoE config [*, 4096, 2048] (8 of the 32), ragged
    token groups, compared on sampled rows of every group."""
    E, N, K = 8, 4096, 2048
    counts = [700, 0, 1, 513, 1024, 300, 129, 2000]
    T = sum(counts)
    say("mxfp4 C2 experts", transpose, T)
    q, wd = _weights("mxfp4", E, N, K, seed=2)
    x = (torch.randn(T, N if transpose else K, generator=torch.Generator().manual_seed(36)) * 0.5).to(torch.bfloat16)
    offs = _offs(counts)
    y = _run("mxfp4", q, x, offs, transpose,
             torch.empty(T, K if transpose else N, dtype=torch.bfloat16, device=DEV))
    ends = offs.tolist()
    rows = sorted({r for a, b in zip([0] + ends[:-1], ends) if b > a for r in (a, b - 1, (a + b) // 2)})
    ref, absref = oracle.grouped_mm(x, wd, offs, transpose, rows=rows)
    _check(y[rows], ref, absref, N if transpose else K, "mxfp4 C2")


@pytest.mark.parametrize("transpose", [False, True])
def test_grouped_mm_nvfp4_c3_expert_shape(transpose):
    """NVFP4 experts of the fused gate/up config [*, 3072, 4096] (4 of the 64)."""
    E, N, K = 4, 3072, 4096
    counts = [1500, 37, 0, 900]
    T = sum(counts)
    say("nvfp4 C3 experts", transpose, T)
    q, wd = _weights("nvfp4", E, N, K, seed=3)
    x = (torch.randn(T, N if transpose else K, generator=torch.Generator().manual_seed(37)) * 0.5).to(torch.bfloat16)
    offs = _offs(counts)
    y = _run("nvfp4", q, x, offs, transpose,
             torch.empty(T, K if transpose else N, dtype=torch.bfloat16, device=DEV))
    ends = offs.tolist()
    rows = sorted({r for a, b in zip([0] + ends[:-1], ends) if b > a for r in (a, b - 1, (a + b) // 2)})
    ref, absref = oracle.grouped_mm(x, wd, offs, transpose, rows=rows)
    _check(y[rows], ref, absref, N if transpose else K, "nvfp4 C3")


# ------------------------------------------------------------------ the fused dequantization, bit for bit

def _byte_weights(fmt, E, N, K, seed):
    """Every code in every position under scale bytes spread over their range
    (finite, no overflow or bfloat16 subnormals, so that the one-hot products
    below are exact): random code bytes, MXFP4 e8m0 bytes in [27, 227], NVFP4
    e4m3 bytes of both signs and both zeros (no NaN bytes), row scales of a
    quantized tensor."""
    rng = np.random.default_rng(seed)
    p = torch.from_numpy(rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8))
    if fmt == "mxfp4":
        s = torch.from_numpy(rng.integers(27, 228, (E, N, K // 32), dtype=np.uint8))
        return (p, s), oracle.dequantize_mxfp4(p, s, torch.bfloat16)
    sb = rng.integers(0, 256, (E, N, K // 16), dtype=np.uint8)
    sb[(sb & 0x7F) == 0x7F] = 0x7E                     # no NaN scales
    sb.reshape(-1)[:4] = [0x00, 0x80, 0x01, 0x81]       # both zeros, smallest subnormals
    s = torch.from_numpy(sb)
    _, _, g = oracle.quantize_nvfp4(synth.moe_nvfp4((E, N, K), seed=seed))
    return (p, s, g), oracle.dequantize_nvfp4(p, s, g, torch.bfloat16)


@pytest.mark.parametrize("shape", [(2, 128, 256), (2, 256, 512)])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("transpose", [False, True])
def test_grouped_mm_one_hot_reproduces_dequantized_weights(fmt, transpose, shape):
    """With one-hot activation rows every output is one weight times 1.0 plus
    zeros, so the GEMM must return the dequantized weights exactly: W_e^T in
    the forward (rows over k), W_e in the backward (rows over n).  This pins
    the in-register dequantization to the dequantize definition bit for bit
    (zeros compared as values: their sign follows the accumulation).  The
    second shape spans two output tiles and several reduction steps in both
    directions."""
    E, N, K = shape
    q, wd = _byte_weights(fmt, E, N, K, seed=38)
    R = N if transpose else K
    x = torch.eye(R, dtype=torch.bfloat16).repeat(E, 1)
    offs = _offs([R] * E)
    y = _run(fmt, q, x, offs, transpose,
             torch.empty(E * R, K if transpose else N, dtype=torch.bfloat16, device=DEV))
    ref = torch.cat([wd[e] if transpose else wd[e].t() for e in range(E)]).contiguous()
    zero = ref.float() == 0
    assert torch.equal(y.float() == 0, zero), "zero pattern differs"
    yb, rb = y.view(torch.int16), ref.view(torch.int16)
    bad = (yb != rb) & ~zero
    assert not bad.any(), f"{fmt}: {int(bad.sum())} weights differ, first at {bad.nonzero()[:4].tolist()}"


# ------------------------------------------------------------------ 256-row tiles, whole outputs

@pytest.mark.parametrize("nk", [(256, 384), (128, 128)])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("transpose", [False, True])
def test_grouped_mm_tall_tiles_ragged(fmt, transpose, nk):
    """Enough tokens per expert for 256-row token tiles (T >= 256 E): groups
    that end inside a tile, an empty expert and trailing rows in no group,
    every output compared.  (128, 128) is the shortest reduction (two steps
    of 64), (256, 384) runs the reduction loop in both directions."""
    N, K = nk
    counts = [700, 0, 301]
    E = len(counts)
    T = sum(counts) + 11
    assert T >= 256 * E
    say("tall", fmt, "transpose" if transpose else "forward", E, N, K, T)
    q, wd = _weights(fmt, E, N, K, seed=39)
    x = torch.randn(T, N if transpose else K, generator=torch.Generator().manual_seed(40)).to(torch.bfloat16)
    offs = _offs(counts)
    sentinel = torch.full((T, K if transpose else N), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = _run(fmt, q, x, offs, transpose, sentinel)
    ref, absref = oracle.grouped_mm(x, wd, offs, transpose)
    T0 = sum(counts)
    _check(y[:T0], ref[:T0], absref[:T0], N if transpose else K, f"tall {fmt}")
    assert torch.isnan(y[T0:].float()).all(), "rows outside every group were written"


# ------------------------------------------------------------------ a reduction of 2^22

@pytest.mark.parametrize("transpose", [False, True])
def test_grouped_mm_mxfp4_long_reduction(transpose):
    """A reduction of 2^22 values (the forward's K, the backward's N): a
    token tile would need byte offsets of 2^31 or more from its first row, so
    the MXFP4 activations take the 64-bit pointer path instead of the buffer
    resource that every shorter MXFP4 shape here uses.  One expert, three
    tokens; random codes and scale bytes, dequantized by the oracle.  The
    backward reference is the oracle's forward sum over the transposed
    weights (the same products; the oracle reads its weights contiguously
    that way)."""
    R, C, T = 1 << 22, 128, 3
    N, K = (R, C) if transpose else (C, R)
    g = torch.Generator().manual_seed(41)
    p = torch.randint(0, 256, (1, N, K // 2), dtype=torch.uint8, generator=g)
    s = torch.randint(118, 126, (1, N, K // 32), dtype=torch.uint8, generator=g)
    wd = oracle.dequantize_mxfp4(p.view(torch.int8), s, torch.bfloat16)
    x = torch.randn(T, R, generator=g).to(torch.bfloat16)
    offs = _offs([T])
    say("mxfp4 long reduction", "transpose" if transpose else "forward", N, K, T)
    y = _run("mxfp4", (p.view(torch.int8), s), x, offs, transpose,
             torch.empty(T, C, dtype=torch.bfloat16, device=DEV))
    w_fwd = wd.transpose(1, 2).contiguous() if transpose else wd      # [1, C, R]
    del wd
    ref, absref = oracle.grouped_mm(x, w_fwd, offs, False)
    _check(y, ref, absref, R, "mxfp4 long reduction")


@pytest.mark.parametrize("counts", [[512, 300], [100, 50]])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("transpose", [False, True])
def test_grouped_mm_nan_scales(fmt, transpose, counts):
    """NaN scale bytes (e8m0 0xFF; e4m3 0x7F and 0xFF) make their block's
    weights NaN, and every output those weights reach is NaN: the GEMM's NaN
    outputs are exactly the oracle's, the others within the bound.  Both
    token-tile heights (256 rows for the first group mix, 128 for the
    second)."""
    E, N, K = 2, 256, 256
    say("nan scales", fmt, "transpose" if transpose else "forward", counts)
    q, _ = _weights(fmt, E, N, K, seed=41)
    s = q[1].clone()
    s[0, 3, 1] = 0xFF if fmt == "mxfp4" else 0x7F
    s[1, 200, 0] = 0xFF
    if fmt == "mxfp4":
        q = (q[0], s)
        wd = oracle.dequantize_mxfp4(q[0], s, torch.bfloat16)
    else:
        q = (q[0], s, q[2])
        wd = oracle.dequantize_nvfp4(q[0], s, q[2], torch.bfloat16)
    assert torch.isnan(wd.float()).any()
    T = sum(counts)
    x = torch.randn(T, N if transpose else K, generator=torch.Generator().manual_seed(42)).to(torch.bfloat16)
    offs = _offs(counts)
    y = _run(fmt, q, x, offs, transpose, torch.empty(T, K if transpose else N, dtype=torch.bfloat16, device=DEV))
    ref, absref = oracle.grouped_mm(x, wd, offs, transpose)
    nan_ref = torch.isnan(ref)
    assert nan_ref.any() and not nan_ref.all()
    assert torch.equal(torch.isnan(y.float()), nan_ref), "NaN outputs differ"
    keep = ~nan_ref
    _check(torch.where(keep, y, torch.zeros_like(y)), torch.where(keep, ref, torch.zeros_like(ref)),
           torch.where(keep, absref, torch.zeros_like(absref)), N if transpose else K, f"nan {fmt}")
