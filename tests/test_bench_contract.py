"""The parts of bench.py's contract that need no GPU: it measures one GPU and
refuses more (exit status 2 with a message, before touching a device, also
when launched as one rank of several), and the K-scan traffic figure is only
reported while the kernel sources match the ones the counters were taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args, env", [
    (["--gpus", "2"], {}),
    (["--gpus", "8", "--steps", "3"], {}),
    ([], {"WORLD_SIZE": "4", "RANK": "0", "LOCAL_RANK": "0"}),
])
def test_bench_refuses_more_than_one_gpu(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                       text=True, env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_file_is_keyed_to_the_kernel_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    fake = tmp_path / "traffic.txt"
    fake.write_text("kernel_sources_sha256_16: %s\nhbm_bytes_per_launch: 123\n" % bench.kscan_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(fake))
    assert bench.stored_traffic() == 123
    fake.write_text("kernel_sources_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 123\n")
    assert bench.stored_traffic() is None
