"""mxq_quantize_kv_nvfp4_noalloc (no workspace argument; its per-head scratch
is the library's static device array) against mxq_quantize_kv_nvfp4 (caller
workspace), bit for bit, through the C ABI: two calls in a row, the second
with a smaller input, so the second must not see the first's scratch."""
import sys

import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)
    sys.stdout.flush()


def mxq():
    import fp8_quantize_pack_amd as m
    return m


def _outputs(k):
    S, H, D = k.shape
    return (torch.empty(S, H, D // 2, dtype=torch.uint8, device=DEV),
            torch.empty(S, H, D // 16, dtype=torch.uint8, device=DEV),
            torch.empty(S, H, dtype=torch.float32, device=DEV))


def _with_workspace(k, smooth):
    p, s, g = _outputs(k)
    ha = torch.empty(k.shape[1] * mxq().KV_AMAX_SLOTS, dtype=torch.float32, device=DEV)
    mxq().mxq_quantize_kv_nvfp4(k, ha, p, s, g, smooth)
    return p, s, g


def _no_alloc(k, smooth):
    p, s, g = _outputs(k)
    mxq().mxq_quantize_kv_nvfp4_noalloc(k, p, s, g, smooth)
    return p, s, g


def _same(a, b, what):
    torch.cuda.synchronize()
    for x, y, n in zip(a, b, ("packed", "scales", "row_scale")):
        xb = x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32)
        yb = y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32)
        assert torch.equal(xb.cpu(), yb.cpu()), f"{what}: {n} differs"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("smooth", [True, False])
def test_noalloc_matches_workspace_call_twice(smooth):
    # first call: 24 heads, large values (a large per-head amax stays in the
    # static array afterwards); second call: fewer heads and tokens, small values
    cases = [((8192, 24, 128), 31, 1.0), ((1000, 8, 64), 32, 2.0 ** -20)]
    for i, (shape, seed, gain) in enumerate(cases):
        k = (synth.kv_cache(shape, seed=seed, device=DEV).float() * gain).to(torch.bfloat16)
        say("call", i, shape, "smooth", smooth)
        ref = _with_workspace(k, smooth)
        got = _no_alloc(k, smooth)
        _same(got, ref, f"call {i}")
        po, so, go = oracle.quantize_kv_nvfp4(k.cpu(), smooth=smooth)
        _same(got, (po, so, go), f"call {i} vs oracle")


def test_noalloc_float32_and_max_heads():
    k = synth.kv_cache((64, 1024, 16), seed=33, device=DEV).float()
    say("float32, 1024 heads")
    _same(_no_alloc(k, True), _with_workspace(k, True), "1024 heads")


def test_noalloc_rejects_heads_beyond_its_scratch():
    k = torch.zeros(4, 1025, 16, dtype=torch.bfloat16, device=DEV)
    p, s, g = _outputs(k)
    with pytest.raises(Exception, match="MXQ_E_SCRATCH"):
        mxq().mxq_quantize_kv_nvfp4_noalloc(k, p, s, g, True)
