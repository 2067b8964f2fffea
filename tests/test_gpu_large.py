"""One call over more than 2^31 elements and 2^32 bytes: the codec calls on a
bfloat16 [300000, 7168] tensor (2.15 G elements, 4.3 GB), compared with the
oracle on the rows that straddle the 2^31-element and 2^32-byte offsets, the
last rows and a random sample (every operation is row-local).  This is the
regime where 32-bit offsets would wrap; the sweep in the bench stays below it
(about 1 GiB per call)."""
import sys

import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
R, K = 300000, 7168


def say(*a):
    print("[gpu-large]", *a, flush=True)
    sys.stdout.flush()


def mxq():
    import fp8_quantize_pack_amd as m
    return m


def _rows():
    first_past = [(1 << 31) // K, (1 << 31) // K + 1, (1 << 32) // (2 * K), (1 << 32) // (2 * K) + 1]
    g = torch.Generator().manual_seed(300)
    sample = torch.randint(0, R, (160,), generator=g).tolist()
    rows = sorted(set([0, 1, R - 2, R - 1] + first_past + [r - 1 for r in first_past] + sample))
    assert all(0 <= r < R for r in rows)
    return torch.tensor(rows, dtype=torch.long)


def _same(gpu, ref, what):
    g = gpu.detach().cpu().contiguous()
    ref = ref.contiguous()
    if g.dtype in (torch.bfloat16, torch.float16):
        g, ref = g.view(torch.int16), ref.view(torch.int16)
    elif g.dtype == torch.float32:
        g, ref = g.view(torch.int32), ref.view(torch.int32)
    assert torch.equal(g, ref), f"{what}: {int((g != ref).sum())} mismatches"


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert R * K > (1 << 31) and R * K * 2 > (1 << 32)
    g = torch.Generator(device=DEV).manual_seed(301)
    x = torch.empty(R, K, dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, R, 50000):                 # seeded N(0, 0.02) rows, drawn in slabs
        r1 = min(R, r0 + 50000)
        x[r0:r1] = (torch.randn(r1 - r0, K, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    rows = _rows()
    xs = x[rows.to(DEV)].cpu()
    say("input ready", tuple(x.shape), "checked rows", rows.numel())
    yield x, rows, xs
    del x
    torch.cuda.empty_cache()


def test_large_mxfp4(big):
    x, rows, xs = big
    say("mxfp4")
    p, s = mxq().quantize_mxfp4(x)
    y = mxq().dequantize_mxfp4(p, s, torch.bfloat16)
    po, so = oracle.quantize_mxfp4(xs)
    ri = rows.to(DEV)
    _same(s.view(torch.uint8)[ri], so, "mxfp4 scales")
    _same(p.view(torch.uint8)[ri], po, "mxfp4 packed")
    _same(y[ri], oracle.dequantize_mxfp4(po, so, torch.bfloat16), "mxfp4 dequant")


def test_large_nvfp4(big):
    x, rows, xs = big
    say("nvfp4")
    p, s, g = mxq().quantize_nvfp4(x)
    y = mxq().dequantize_nvfp4(p, s, g, torch.bfloat16)
    po, so, go = oracle.quantize_nvfp4(xs)
    ri = rows.to(DEV)
    _same(g[ri], go, "nvfp4 row scale")
    _same(s.view(torch.uint8)[ri], so, "nvfp4 scales")
    _same(p[ri], po, "nvfp4 packed")
    _same(y[ri], oracle.dequantize_nvfp4(po, so, go, torch.bfloat16), "nvfp4 dequant")


def test_large_mxfp8_and_static_fp4(big):
    x, rows, xs = big
    say("mxfp8")
    c, s = mxq().quantize_mxfp8(x)
    ri = rows.to(DEV)
    co, so = oracle.quantize_mxfp8(xs)
    _same(s.view(torch.uint8)[ri], so, "mxfp8 scales")
    _same(c.view(torch.uint8)[ri], co, "mxfp8 codes")
    y = mxq().dequantize_mxfp8(c, s, torch.bfloat16)
    _same(y[ri], oracle.dequantize_mxfp8(co, so, torch.bfloat16), "mxfp8 dequant")
    del c, s, y
    say("static fp4")
    a = x.view(R, K // 16, 16).abs().amax(-1).float()
    G = x.abs().max().float().reshape(1)
    y = mxq().fake_quantize_fp4_static(x, a, G, 16)
    _same(y[ri], oracle.fake_quantize_fp4_static(xs, a[ri].cpu(), float(G), 16), "static fp4")


def test_large_cache_qdq(big):
    x, rows, xs = big
    say("cache fp8")
    y = mxq().quantize_cache(x, "fp8", 32)
    ri = rows.to(DEV)
    _same(y[ri], oracle.quantize_cache(xs, "fp8", 32), "cache fp8")
