"""The measurement reference kernels of libmxq_roofline (the copy, read-only and
write-only streams the bench compares the codec with, and the shader clock
probe): they must move exactly the bytes they claim, so that the ceiling they
report is a ceiling of real work."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[roofline-ref]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rl():
    from fp8_quantize_pack_amd import roofline
    return roofline


# sizes: one 16-byte chunk, a ragged tail past the last full wave tile, and
# several grid-stride rounds' worth is left to the bench
@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16, 1 << 22])
@pytest.mark.parametrize("unroll", [1, 2, 4, 8])
def test_copy_moves_every_byte_once(rl, nbytes, unroll):
    say("copy", nbytes, unroll)
    g = torch.Generator(device=DEV).manual_seed(nbytes + unroll)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    rl.copy(src, dst[:nbytes], unroll=unroll)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())          # nothing past the end


@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16, 1 << 22])
@pytest.mark.parametrize("unroll", [1, 4])
def test_fill_writes_every_word_and_nothing_else(rl, nbytes, unroll):
    say("fill", nbytes, unroll)
    dst = torch.zeros(nbytes // 4 + 16, dtype=torch.int32, device=DEV)
    rl.fill(dst[:nbytes // 4], value=0x12345678, unroll=unroll)
    torch.cuda.synchronize()
    assert bool((dst[:nbytes // 4] == 0x12345678).all())
    assert bool((dst[nbytes // 4:] == 0).all())


@pytest.mark.parametrize("unroll", [1, 2, 4])
def test_read_visits_every_chunk(rl, unroll):
    # chunk c (16 bytes) holds the words (c + 1, 0, 0, 0); in step u of its
    # tile, lane l of tile t reads chunk t * 64 * unroll + 64 u + l and folds
    # it into an XOR, and writes that XOR to the sink only when it equals
    # `magic`.  Each lane's XOR is computed here; a magic that exactly one lane
    # holds (including lanes of the ragged last tile) must come back, and a
    # magic no lane holds must leave the sink alone.
    say("read", unroll)
    n = 777                                          # chunks: 12 full waves' worth + a tail
    words = torch.zeros(n, 4, dtype=torch.int32)
    words[:, 0] = torch.arange(1, n + 1, dtype=torch.int32)
    src = words.reshape(-1).to(DEV)
    per = 64 * unroll
    accs = []
    for t in range((n + per - 1) // per):
        for lane in range(64):
            a = 0
            for u in range(unroll):
                c = t * per + 64 * u + lane
                if c < n:
                    a ^= c + 1
            accs.append(a)
    unique = [a for a in set(accs) if accs.count(a) == 1 and a != 0]
    picks = sorted(unique)[:2] + sorted(unique)[-2:]
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for m in picks:
        sink.zero_()
        rl.read(src, sink, unroll=unroll, magic=m)
        torch.cuda.synchronize()
        assert int(sink.item()) == m, m
    absent = max(accs) + 1
    sink.zero_()
    rl.read(src, sink, unroll=unroll, magic=absent)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_clock_probe_reads_a_plausible_shader_clock(rl):
    say("clock")
    out = torch.zeros(2 * 64, dtype=torch.int64, device=DEV)
    rl.clock(out, iters=4096)
    torch.cuda.synchronize()
    v = out.view(-1, 2).cpu()
    assert bool((v > 0).all())
    mhz = rl.clock_mhz(out)
    say("clock MHz", round(mhz, 1))
    assert 100.0 < mhz < 5000.0
