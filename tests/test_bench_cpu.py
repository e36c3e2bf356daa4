"""bench.py host logic: the one-GPU guard and the counter files' digest check
(no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_counters_follow_the_kernel_sources(tmp_path, monkeypatch):
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    srcs = [bench._STREAM, bench._TILED]           # a stage of two kernels' sources
    monkeypatch.setitem(bench.GEMM_SRC, "verify", srcs)
    good = ",".join(bench.src_digest(p) for p in srcs)
    f = tmp_path / "gate_up_verify_counters.txt"
    f.write_text(f"# comment: ignored\nsrc_sha: {good}\nfetch_bytes: 1000\nwrite_bytes: 24\n")
    assert bench.read_counters("verify") == 1024.0
    f.write_text(f"src_sha: {bench.src_digest(srcs[0])}\nfetch_bytes: 1000\nwrite_bytes: 24\n")
    assert bench.read_counters("verify") is None          # taken on other kernel code
    assert bench.read_counters("decode") is None          # no file
