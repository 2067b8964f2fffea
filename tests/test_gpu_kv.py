"""GPU parity of the NVFP4 KV cache calls against the CPU oracle, bit for
bit, through the C ABI: paged dequantization into one contiguous tensor, and
per-head quantization with and without k_smooth.  The full-size workload
(a [32768, 12, 128] bfloat16 K tensor, 32 cache blocks of 1024 tokens) is
compared whole."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD = 4096


def say(*a):
    print("[gpu-kv]", *a, flush=True)
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


# ------------------------------------------------------------------ paged dequantization

def _pages_from_oracle(nb, bt, H, D, seed, zero_block=None):
    vals, scs, am = [], [], []
    for b in range(nb):
        k = synth.kv_cache((bt, H, D), seed=seed + b).reshape(bt * H, D)
        if b == zero_block:
            k.zero_()
        p, s, _ = oracle.quantize_nvfp4(k, mode="tensor")
        vals.append(p)
        scs.append(s)
        am.append(float(k.float().abs().max()))
    return vals, scs, am


def gpu_pages(vals, scs, am, bt, H, dtype):
    D = vals[0].shape[-1] * 2
    nb = len(vals)
    dv = [v.to(DEV) for v in vals]
    ds = [s.to(DEV) for s in scs]
    da = [torch.tensor([a], dtype=torch.float32, device=DEV) for a in am]
    tab = lambda ts: torch.tensor([t.data_ptr() for t in ts], dtype=torch.int64).to(DEV)
    ry, y = guarded((nb * bt, H, D), dtype)
    mxq().mxq_dequantize_kv_pages_nvfp4(tab(dv), tab(ds), tab(da), bt, y)
    check_guard(ry)
    return y


PAGE_CASES = [(5, 3, 4, 128), (1, 1, 1, 16), (7, 5, 3, 48), (4, 64, 12, 128), (3, 17, 2, 512)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("nb,bt,H,D", PAGE_CASES)
def test_kv_pages_dequant_small(nb, bt, H, D, dtype):
    say("kv pages", nb, bt, H, D, dtype)
    vals, scs, am = _pages_from_oracle(nb, bt, H, D, seed=100 + D, zero_block=nb // 2)
    order = list(np.random.default_rng(nb).permutation(nb))       # blocks as the list holds them
    vals, scs, am = [vals[i] for i in order], [scs[i] for i in order], [am[i] for i in order]
    y = gpu_pages(vals, scs, am, bt, H, dtype)
    assert_same(y, oracle.dequantize_kv_pages(vals, scs, am, bt, H, dtype)[0], "pages")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_kv_pages_every_code_every_scale_byte(dtype):
    """Random code and scale bytes (NaN scale bytes included) under amax
    values from zero to huge; NaNs compared by position."""
    say("kv pages random bytes", dtype)
    rng = np.random.default_rng(7)
    nb, bt, H, D = 6, 16, 4, 128
    vals = [torch.from_numpy(rng.integers(0, 256, (bt * H, D // 2), dtype=np.uint8)) for _ in range(nb)]
    scs = [torch.from_numpy(rng.integers(0, 256, (bt * H, D // 16), dtype=np.uint8)) for _ in range(nb)]
    am = [0.0, 1e-30, 1.0, 2688.0, 3.0e38, 37.25]
    y = gpu_pages(vals, scs, am, bt, H, dtype).cpu()
    yo = oracle.dequantize_kv_pages(vals, scs, am, bt, H, dtype)[0]
    nan = torch.isnan(yo.float())
    assert torch.equal(nan, torch.isnan(y.float()))
    assert_same(y[~nan], yo[~nan], "pages")


# ------------------------------------------------------------------ per-head quantization

def gpu_quantize_kv(k, smooth):
    S, H, D = k.shape
    rp, p = guarded((S, H, D // 2), torch.uint8)
    rs, s = guarded((S, H, D // 16), torch.uint8)
    rg, g = guarded((S, H), torch.float32)
    ha = torch.full((H * 32,), 123.0, dtype=torch.float32, device=DEV)   # stale scratch
    mxq().mxq_quantize_kv_nvfp4(k, ha, p, s, g, smooth)
    check_guard(rp); check_guard(rs); check_guard(rg)
    return p, s, g, ha[:H]


KV_SHAPES = [(40, 3, 128), (1000, 12, 128), (7, 5, 16), (33, 2, 512), (64, 4, 64), (17, 1, 32),
             (100, 3, 256), (300, 7, 128)]


@pytest.mark.parametrize("smooth", [True, False])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("shape", KV_SHAPES)
def test_quantize_kv_small(shape, dtype, smooth):
    say("quantize_kv", shape, dtype, smooth)
    k = synth.kv_cache(shape, seed=sum(shape)).to(dtype)
    po, so, go = oracle.quantize_kv_nvfp4(k, smooth=smooth)
    p, s, g, ha = gpu_quantize_kv(k.to(DEV), smooth)
    assert_same(g, go, "row scale")
    assert_same(s, so, "scales")
    assert_same(p, po, "packed")
    src = oracle.k_smooth(k) if smooth else k
    assert_same(ha, src.float().abs().amax(dim=(0, 2)), "head amax")


def test_quantize_kv_edge_rows():
    """Constant rows (smoothed to zero; one head entirely), a head of zeros,
    the pairwise-order row, signed zeros, and rows whose mean rounds."""
    say("quantize_kv edge rows")
    S, H, D = 64, 4, 128
    k = synth.kv_cache((S, H, D), seed=77).float()
    k[:, 0, :] = torch.linspace(-3, 3, S).reshape(S, 1)      # head 0: constant rows
    k[:, 1, :] = 0.0                                         # head 1: zeros
    k[5, 2, :4] = torch.tensor([1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)])
    k[5, 2, 4:] = 0.0
    k[6, 2, :] = -0.0
    k[7, 3, :] = k[7, 3, :] + 1000.0                         # large mean
    for dtype in (torch.float32, torch.bfloat16):
        kd = k.to(dtype)
        for smooth in (True, False):
            po, so, go = oracle.quantize_kv_nvfp4(kd, smooth=smooth)
            p, s, g, _ = gpu_quantize_kv(kd.to(DEV), smooth)
            assert_same(g, go, f"row scale {dtype} {smooth}")
            assert_same(s, so, f"scales {dtype} {smooth}")
            assert_same(p, po, f"packed {dtype} {smooth}")


def test_quantize_kv_then_dequantize_with_the_nvfp4_call():
    """The row scales make the output a plain NVFP4 tensor of S * H rows."""
    k = synth.kv_cache((50, 6, 128), seed=78).to(DEV)
    p, s, g = mxq().quantize_kv_nvfp4(k)
    y = mxq().dequantize_nvfp4(p, s, g, torch.bfloat16)
    po, so, go = oracle.quantize_kv_nvfp4(k.cpu())
    assert_same(y, oracle.dequantize_nvfp4(po, so, go, torch.bfloat16), "round trip")


# ------------------------------------------------------------------ full size

def test_full_kv_cache_workload():
    """K [32768, 12, 128] bf16: per-head quantization with k_smooth (compared
    whole), written as 32 cache blocks of 1024 tokens in the paged layout
    (each block re-quantized with its own amax by the oracle), then the paged
    dequantization of those blocks (compared whole)."""
    S, H, D, bt = 32768, 12, 128, 1024
    say("full kv", S, H, D, bt)
    k = synth.kv_cache((S, H, D), seed=5, device=DEV)
    p, s, g = mxq().quantize_kv_nvfp4(k, smooth=True)
    kc = k.cpu()
    po, so, go = oracle.quantize_kv_nvfp4(kc, smooth=True)
    assert_same(g, go, "row scale")
    assert_same(s.view(torch.uint8), so, "scales")
    assert_same(p, po, "packed")
    say("paged blocks")
    nb = S // bt
    blocks = kc.reshape(nb, bt * H, D)
    vals, scs, am = [], [], []
    for b in range(nb):
        pb, sb, _ = oracle.quantize_nvfp4(blocks[b], mode="tensor")
        vals.append(pb)
        scs.append(sb)
        am.append(float(blocks[b].float().abs().max()))
    y = gpu_pages(vals, scs, am, bt, H, torch.bfloat16)
    assert_same(y, oracle.dequantize_kv_pages(vals, scs, am, bt, H, torch.bfloat16)[0], "pages")
