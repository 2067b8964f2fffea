"""Host-side checks of bench.py that need no GPU: the refusal of other GPU
counts, the algorithmic bytes per element it divides by, and the use of the
committed HBM-traffic summary only while it matches the kernel sources."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_element(bench):
    # bf16 in, packed codes out, one scale byte per block (MXFP4: 32, NVFP4:
    # 16) and, for NVFP4, one float32 row scale
    n, rows = 36 * 2048 * 7168, 36 * 2048
    assert bench.bytes_mx(n) == n * 2.53125
    assert bench.bytes_nv(n, rows) == n * 2.5625 + 4 * rows
    assert bench.bytes_mx(n) == 1337720832 and bench.bytes_nv(n, rows) == 1354530816


def test_traffic_only_for_the_profiled_sources(bench):
    from fp8_quantize_pack_amd.profiling import kernel_source_hash
    h = kernel_source_hash()
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.txt")) as f:
        txt = f.read()
    if ("source_hash: " + h) not in txt:
        pytest.skip("the committed profile predates the current kernel sources")
    t = bench.measured_traffic("nvfp4_quant", h)
    assert t is not None and abs(t / 1204027392 - 1) < 0.01   # within 1% of the algorithmic bytes
    assert bench.measured_traffic("nvfp4_quant", "0" * 16) is None
    assert bench.measured_traffic("no_such_op", h) is None
