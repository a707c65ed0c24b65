"""Host checks of the measurement plumbing (no GPU): every committed traffic
summary under profiles/ parses, states the commands it came from and the copy
calibration, and bench.py's reader returns its bytes only while the kernel's
sources hash to the recorded value (else None, never an exception)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC = sorted(f for f in os.listdir(PROFILES) if f.startswith("traffic_") and f.endswith(".txt"))


def _fields(path):
    kv = {}
    with open(path) as fh:
        text = fh.read()
    for line in text.splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return text, kv


def test_there_are_traffic_summaries():
    assert TRAFFIC, "profiles/ holds no traffic summary"


@pytest.mark.parametrize("name", TRAFFIC)
def test_traffic_summary_is_complete_and_consistent(name):
    text, kv = _fields(os.path.join(PROFILES, name))
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    assert "--copy-calibration" in text
    for key in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "fetch_scale", "write_scale",
                "hbm_bytes_per_launch", "source_sha256_16"):
        assert key in kv, key
    fk, wk = float(kv["fetch_kib_per_dispatch"]), float(kv["write_kib_per_dispatch"])
    fs, ws = float(kv["fetch_scale"]), float(kv["write_scale"])
    total = float(kv["hbm_bytes_per_launch"])
    assert fk > 0 and wk > 0 and fs > 0 and ws > 0
    assert abs(total - (fk * fs + wk * ws) * 1024) <= 1e-4 * total   # fields are printed rounded
    kernel, workload = name[len("traffic_"):-len(".txt")].rsplit("_bf16_kernel_", 1)
    kernel += "_bf16_kernel"
    got = bench.measured_traffic(kernel, workload)
    if kv["source_sha256_16"] == bench.kernel_source_hash(kernel):
        assert got == total
    else:
        assert got is None


def test_reader_returns_none_without_a_summary():
    assert bench.measured_traffic("fwd_bf16_kernel", "no_such_workload") is None


def test_bench_refuses_more_than_one_gpu():
    """The library is one GPU's share: bench.py --gpus N>1 exits with a message
    (before touching a GPU)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr


def test_bench_layout_rows_match_the_oracle_sharded_order():
    """bench.py puts document ids into a layout's sharded order with its own
    small helper; it must agree with the oracle's definition."""
    from oracle import schedule as Z
    for S, P, pairs in ((64, 2, [(0, 3), (1, 2)]), (96, 3, [(0, 1), (2, 5), (3, 4)]),
                        (128, 4, [(0, 4), (1, 7), (3, 5), (2, 6)])):
        assert bench.layout_rows(S, P, pairs).tolist() == Z.sharded_order(S, P, pairs).tolist()


def test_bench_cpu_model_fields():
    m = bench.cpu_model()
    assert set(m) == {"name", "id", "logical"}
    assert m["logical"] >= 1
