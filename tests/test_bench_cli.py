"""bench.py's command-line contract that can be checked without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _parse(argv, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    return bench.parse()


def test_config_iters_and_no_oracle_flags(monkeypatch):
    a = _parse(["--config", "mxfp4_transform", "--iters", "7", "--no-oracle"], monkeypatch)
    assert a.extras == "mxfp4" and a.steps == 7 and a.no_cpu_baseline and not a.only_step
    a = _parse(["--config", "nvfp4_prefill"], monkeypatch)
    assert a.only_step and a.extras is None
    for name, extra in (("nvfp4_tiny", "tiny"), ("nvfp4_decode", "decode"), ("looped_sigma_delta", "sigma_delta")):
        assert _parse(["--config", name], monkeypatch).extras == extra
    a = _parse([], monkeypatch)
    assert a.steps == 100 and a.warmup == 10 and a.config is None and not a.no_cpu_baseline
