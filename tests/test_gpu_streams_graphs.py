"""The C-ABI calls under stream semantics and HIP graph capture (the codec
calls, MXFP8, the static FP4 round trip and both NVFP4 KV-cache calls).

Every call only enqueues on the stream it is given, allocates nothing and
clears its own scratch with a kernel (no memset nodes), so a captured
sequence must replay to the same bytes as the eager calls, replay after
replay, with unrelated eager work in between."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def mxq():
    import fp8_quantize_pack_amd as m
    return m


def _buffers():
    x = synth.moe_nvfp4((3, 256, 1024), seed=91).to(DEV)
    x7 = synth.moe_nvfp4((64, 7168), seed=96).to(DEV)    # 7 segments a row: the capped row kernel
    kv = synth.kv_cache((2, 64, 512), seed=92).to(DEV)
    R, K = 3 * 256, 1024
    out = {
        "mx_p": torch.empty(3, 256, K // 2, dtype=torch.int8, device=DEV),
        "mx_s": torch.empty(3, 256, K // 32, dtype=torch.uint8, device=DEV),
        "mx_y": torch.empty_like(x),
        "nv_p": torch.empty(3, 256, K // 2, dtype=torch.uint8, device=DEV),
        "nv_s": torch.empty(3, 256, K // 16, dtype=torch.uint8, device=DEV),
        "nv_g": torch.empty(R, dtype=torch.float32, device=DEV),
        "nt_p": torch.empty(3, 256, K // 2, dtype=torch.uint8, device=DEV),
        "nt_s": torch.empty(3, 256, K // 16, dtype=torch.uint8, device=DEV),
        "nt_g": torch.empty(R, dtype=torch.float32, device=DEV),
        "n7_p": torch.empty(64, 7168 // 2, dtype=torch.uint8, device=DEV),
        "n7_s": torch.empty(64, 7168 // 16, dtype=torch.uint8, device=DEV),
        "n7_g": torch.empty(64, dtype=torch.float32, device=DEV),
        "scratch": torch.zeros(4, dtype=torch.float32, device=DEV),
        "kv_y": torch.empty_like(kv),
        "m8_c": torch.empty(3, 256, K, dtype=torch.uint8, device=DEV),
        "m8_s": torch.empty(3, 256, K // 32, dtype=torch.uint8, device=DEV),
        "m8_y": torch.empty_like(x),
        "st_y": torch.empty_like(x),
        "kq_p": torch.empty(64, 8, 64, dtype=torch.uint8, device=DEV),
        "kq_s": torch.empty(64, 8, 8, dtype=torch.uint8, device=DEV),
        "kq_g": torch.empty(64, 8, dtype=torch.float32, device=DEV),
        "kq_amax": torch.zeros(8 * 32, dtype=torch.float32, device=DEV),
        "pg_y": torch.empty(64, 8, 128, dtype=torch.bfloat16, device=DEV),
    }
    return (x, x7), kv, out


def _static_inputs(x):
    a = x.float().abs().reshape(-1, 1024 // 16, 16).amax(-1).contiguous()
    g = x.float().abs().max().reshape(1).contiguous()
    return a, g


def _kv_inputs():
    k = synth.kv_cache((64, 8, 128), seed=93).to(DEV)
    blocks = [(synth.kv_cache((16 * 8, 64), seed=94 + b).to(DEV).view(torch.uint8)[:, :64].contiguous(),
               torch.randint(0x20, 0x50, (16 * 8, 8), dtype=torch.uint8,
                             generator=torch.Generator().manual_seed(95 + b)).to(DEV),
               torch.tensor([1.5 + b], dtype=torch.float32, device=DEV)) for b in range(4)]
    tab = lambda i: torch.tensor([blk[i].data_ptr() for blk in blocks], dtype=torch.int64).to(DEV)
    return k, blocks, (tab(0), tab(1), tab(2))


def _sequence(xs, kv, o, stream=None, extra=None):
    m = mxq()
    x, x7 = xs
    m.mxq_quantize_mxfp4(x, o["mx_p"], o["mx_s"], stream)
    m.mxq_dequantize_mxfp4(o["mx_p"], o["mx_s"], o["mx_y"], stream)
    m.mxq_quantize_nvfp4(x, o["nv_p"], o["nv_s"], o["nv_g"], stream=stream)
    m.mxq_quantize_nvfp4(x, o["nt_p"], o["nt_s"], o["nt_g"], mode="tensor", scratch=o["scratch"],
                         stream=stream)
    m.mxq_quantize_cache(kv, o["kv_y"], "nvfp4", 16, stream)
    m.mxq_quantize_nvfp4(x7, o["n7_p"], o["n7_s"], o["n7_g"], stream=stream)
    if extra is not None:
        (a, g), (k, _, (vt, st, at)) = extra
        m.mxq_quantize_mxfp8(x, o["m8_c"], o["m8_s"], stream)
        m.mxq_dequantize_mxfp8(o["m8_c"], o["m8_s"], o["m8_y"], stream)
        m.mxq_fake_quantize_fp4_static(x, a, g, o["st_y"], 16, stream)
        m.mxq_quantize_kv_nvfp4(k, o["kq_amax"], o["kq_p"], o["kq_s"], o["kq_g"], True, stream)
        m.mxq_dequantize_kv_pages_nvfp4(vt, st, at, 16, o["pg_y"], stream)


def _snapshot(o):
    return {k: v.clone() for k, v in o.items() if k not in ("scratch", "kq_amax")}


def _same(a, b):
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


def test_graph_capture_replays_match_eager():
    xs, kv, o = _buffers()
    extra = (_static_inputs(xs[0]), _kv_inputs())
    _sequence(xs, kv, o, extra=extra)
    torch.cuda.synchronize()
    eager = _snapshot(o)
    for v in o.values():
        v.zero_()
    s = torch.cuda.Stream()                       # default priority
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _sequence(xs, kv, o, s, extra=extra)
    for replay in range(3):
        for k, v in o.items():
            if k not in ("scratch", "kq_amax"):
                v.fill_(0x5A if v.dtype == torch.uint8 else 7)   # poison the outputs
        o["scratch"].fill_(123.0)                 # stale scratch: the graph must clear it
        o["kq_amax"].fill_(1e30)
        torch.randn(1 << 20, device=DEV).sum()    # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(eager, _snapshot(o))


def test_side_stream_orders_after_producer():
    """A call on a side stream that waits on the producer's event sees the
    producer's data; results equal the default-stream results."""
    xs, kv, o = _buffers()
    extra = (_static_inputs(xs[0]), _kv_inputs())
    _sequence(xs, kv, o, extra=extra)
    torch.cuda.synchronize()
    ref = _snapshot(o)
    s = torch.cuda.Stream()
    x2 = torch.empty_like(xs[0])
    x2.copy_(xs[0])                               # producer on the current stream
    ev = torch.cuda.Event()
    ev.record()
    s.wait_event(ev)
    with torch.cuda.stream(s):
        for v in o.values():
            v.zero_()
        _sequence((x2, xs[1]), kv, o, s, extra=extra)
    s.synchronize()
    _same(ref, _snapshot(o))
