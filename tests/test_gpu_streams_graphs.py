"""The C-ABI calls under stream semantics and HIP graph capture.

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
        "scratch": torch.zeros(4, dtype=torch.float32, device=DEV),
        "kv_y": torch.empty_like(kv),
    }
    return x, kv, out


def _sequence(x, kv, o, stream=None):
    m = mxq()
    m.mxq_quantize_mxfp4(x, o["mx_p"], o["mx_s"], stream)
    m.mxq_dequantize_mxfp4(o["mx_p"], o["mx_s"], o["mx_y"], stream)
    m.mxq_quantize_nvfp4(x, o["nv_p"], o["nv_s"], o["nv_g"], stream=stream)
    m.mxq_quantize_nvfp4(x, o["nt_p"], o["nt_s"], o["nt_g"], mode="tensor", scratch=o["scratch"],
                         stream=stream)
    m.mxq_quantize_cache(kv, o["kv_y"], "nvfp4", 16, stream)


def _snapshot(o):
    return {k: v.clone() for k, v in o.items() if k != "scratch"}


def _same(a, b):
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


def test_graph_capture_replays_match_eager():
    x, kv, o = _buffers()
    _sequence(x, kv, o)
    torch.cuda.synchronize()
    eager = _snapshot(o)
    for v in o.values():
        v.zero_()
    s = torch.cuda.Stream()                       # default priority
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _sequence(x, kv, o, s)
    for replay in range(3):
        for k, v in o.items():
            if k != "scratch":
                v.fill_(0x5A if v.dtype == torch.uint8 else 7)   # poison the outputs
        o["scratch"].fill_(123.0)                 # stale scratch: the graph must clear it
        torch.randn(1 << 20, device=DEV).sum()    # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(eager, _snapshot(o))


def test_side_stream_orders_after_producer():
    """A call on a side stream that waits on the producer's event sees the
    producer's data; results equal the default-stream results."""
    x, kv, o = _buffers()
    _sequence(x, kv, o)
    torch.cuda.synchronize()
    ref = _snapshot(o)
    s = torch.cuda.Stream()
    x2 = torch.empty_like(x)
    x2.copy_(x)                                   # producer on the current stream
    ev = torch.cuda.Event()
    ev.record()
    s.wait_event(ev)
    with torch.cuda.stream(s):
        for v in o.values():
            v.zero_()
        _sequence(x2, kv, o, s)
    s.synchronize()
    _same(ref, _snapshot(o))
