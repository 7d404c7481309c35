"""Host-side checks of bench.py and of the committed rocprofv3 summaries it reads
(no GPU needed: nothing here launches a kernel)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

TRAFFIC_SUMMARIES = [
    "chunk_fwd_b8h16t2048d128_bf16_traffic.txt",
    "recurrent_step_n256h16d128_bf16_traffic.txt",
    "gdn_fwd_b8h16t2048d128_bf16.txt",
]


def _fields(path):
    kv = {}
    for line in open(path):
        line = line.strip()
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_bench_refuses_a_multi_rank_launch():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, cwd=ROOT, env=env)
    assert r.returncode == 2
    assert "WORLD_SIZE=2" in r.stderr


@pytest.mark.parametrize("name", TRAFFIC_SUMMARIES)
def test_traffic_summaries_are_well_formed(name):
    kv = _fields(os.path.join(bench.PROFILES, name))
    for key in ("kernel", "fetch_size_kib_per_dispatch", "write_size_kib_per_dispatch",
                "fetch_scale", "write_scale", "sources_sha256", "hbm_bytes_per_launch",
                "algorithmic_bytes_per_launch", "traffic_over_algorithmic"):
        assert key in kv, key
    fetch = float(kv["fetch_size_kib_per_dispatch"]) * float(kv["fetch_scale"])
    write = float(kv["write_size_kib_per_dispatch"]) * float(kv["write_scale"])
    hbm = float(kv["hbm_bytes_per_launch"])
    # the printed scale factors carry four decimals
    assert hbm == pytest.approx((fetch + write) * 1024, rel=1e-4)
    ratio = hbm / float(kv["algorithmic_bytes_per_launch"])
    assert ratio == pytest.approx(float(kv["traffic_over_algorithmic"]), abs=1e-3)
    # the counters can only read at least the bytes the kernel must move, and far
    # more would mean a mis-scaled calibration
    assert 0.99 < ratio < 1.5
    assert len(kv["sources_sha256"]) == 64


@pytest.mark.parametrize("changed", ["kernel.hip", "dispatch.h", "gla.h"])
def test_read_traffic_follows_every_source(tmp_path, changed):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    (csrc / "kernel.hip").write_text("// kernel v1\n")
    (csrc / "dispatch.h").write_text("// header v1\n")
    (tmp_path / "gla.h").write_text("// abi v1\n")
    old = (bench.PROFILES, bench.CSRC, bench.ROOT)
    try:
        bench.PROFILES, bench.CSRC, bench.ROOT = str(tmp_path), str(csrc), str(tmp_path)
        header = str(tmp_path / "gla.h")
        os.makedirs(tmp_path / "include", exist_ok=True)
        os.replace(header, tmp_path / "include" / "gla.h")
        digest = bench.sources_sha256()
        (tmp_path / "p.txt").write_text(
            "# header = ignored\nsources_sha256 = %s\nhbm_bytes_per_launch = 1234\n" % digest)
        assert bench.read_traffic("p.txt") == 1234.0
        path = tmp_path / "include" / "gla.h" if changed == "gla.h" else csrc / changed
        path.write_text(path.read_text() + "// changed\n")   # a source changed since the counters
        assert bench.read_traffic("p.txt") is None
        assert bench.read_traffic("missing.txt") is None
    finally:
        bench.PROFILES, bench.CSRC, bench.ROOT = old


def test_counter_summary_is_well_formed_and_read():
    kv = _fields(os.path.join(bench.PROFILES, "chunk_fwd_b8h16t2048d128_bf16_counters.txt"))
    for key in ("mfma_busy_frac", "executed_over_algorithmic", "wait_inst_any_over_wave_cycles",
                "lds_bank_conflict_over_active_lds", "sources_sha256"):
        assert key in kv, key
    assert 0.0 < float(kv["mfma_busy_frac"]) < 1.0
    # the executed MFMA work covers at least the algorithmic FLOPs
    assert float(kv["executed_over_algorithmic"]) >= 1.0
