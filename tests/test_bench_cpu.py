"""The benchmark's host-side contract, checked without a GPU: its byte accounting for the
roofline, the refusal of more than one GPU, and the traffic figure it takes from the committed
counter summary only while that summary matches the kernel sources."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes_of_the_fused_launch():
    """Each row read once and written once, gamma once: the OLMo-2-7B headline at T = 8192 moves
    8192 x (4096 + 4096) x 2 B x 2 + (4096 + 4096) x 2 B."""
    b = load_bench()
    assert b.fused_bytes(8192, 4096, 4096) == 268_451_840
    assert b.fused_bytes(4096, 4096, 4096) == 134_234_112
    assert b.fused_bytes(8192, 5120, 1024) == 201_338_880
    assert b.fused_bytes(64, 512, 512, es=4, gs=4) == 64 * 1024 * 8 + 1024 * 4


def test_recorded_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """The summary's traffic is used only when its source hash is that of the current row-kernel
    sources; a summary taken on other sources, or none, gives null."""
    b = load_bench()
    text = open(b.PMC_SUMMARY).read()
    if b.rows_source_hash() in text:
        assert isinstance(b.recorded_traffic(), int)
    stale = tmp_path / "summary.md"
    stale.write_text("traffic_bytes_per_launch: 123\nkernel source hash: `0123456789abcdef`\n")
    monkeypatch.setattr(b, "PMC_SUMMARY", str(stale))
    assert b.recorded_traffic() is None
    fresh = tmp_path / "fresh.md"
    fresh.write_text(f"traffic_bytes_per_launch: 123\nkernel source hash: `{b.rows_source_hash()}`\n")
    monkeypatch.setattr(b, "PMC_SUMMARY", str(fresh))
    assert b.recorded_traffic() == 123
    monkeypatch.setattr(b, "PMC_SUMMARY", str(tmp_path / "absent.md"))
    assert b.recorded_traffic() is None


def test_more_than_one_gpu_is_refused():
    """One GPU only: the benchmark exits with a message before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps",
                        "1", "--warmup", "0"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
