"""Host logic of bench.py, no GPU: the counter summaries are read only while the
kernel sources match the profiled build, the MFMA and traffic figures follow
from the counters as stated, and more than one GPU is refused."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_traffic_and_mfma_follow_the_source_digest(tmp_path, monkeypatch):
    k = "chunk_intra64_kernel"
    dig = bench.source_digest(bench.KERNEL_SOURCES[k])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _write(tmp_path, "t.txt", (
        f"header line\ntraffic {k} fetch_bytes=1000 write_bytes=24 sha256={dig}\n"
        f"traffic {k} fetch_bytes=5 write_bytes=5 sha256={'0' * 64}\n")))
    assert bench.measured_traffic(k) == 1024
    # 8 XCDs x 1000 cycles each over 1024 SIMDs; 512 flops per MOPS unit
    monkeypatch.setattr(bench, "MFMA_FILE", _write(tmp_path, "m.txt", (
        f"mfma {k} mops_bf16=2000000 busy_cycles=512000 gui_active=8000 sha256={dig}\n")))
    m = bench.measured_mfma(k, 1e-3)
    assert m["flops_per_launch"] == 2000000 * 512
    assert abs(m["busy_pct"] - 50.0) < 1e-9
    assert abs(m["tflops"] - 1.024) < 0.05
    # a stale digest reads as unmeasured
    monkeypatch.setattr(bench, "MFMA_FILE", _write(tmp_path, "m2.txt", (
        f"mfma {k} mops_bf16=1 busy_cycles=1 gui_active=8 sha256={'f' * 64}\n")))
    assert bench.measured_mfma(k, 1e-3) is None
    assert bench.mfma_summary((k, "chunk_chain64_kernel"), 1e-3, 1e-3, 2e-3) is None


def test_committed_summaries_parse():
    """The committed profiles carry machine-readable lines for both prefill kernels
    (whatever their digests)."""
    for path, tag in ((bench.TRAFFIC_FILE, "traffic"), (bench.MFMA_FILE, "mfma")):
        with open(path) as f:
            kernels = {l.split()[1] for l in f if l.startswith(tag + " ")}
        assert {"chunk_intra64_kernel", "chunk_chain64_kernel"} <= kernels, (path, kernels)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
