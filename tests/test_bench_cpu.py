"""Host-side pieces of bench.py: the one-GPU rule and the stored HBM-traffic lookup."""
import importlib.util
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    b = load_bench()
    csrc = tmp_path / "diffusion_dllm_block_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in b.COUNTED_SOURCES:
        shutil.copy(os.path.join(ROOT, "diffusion_dllm_block_amd", "csrc", f), csrc / f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    sha = b.source_sha()
    tab = {"wl:CLS": {"bytes_per_launch": 123.0, "source_sha": sha}}
    (tmp_path / "profiles" / "counters.json").write_text(json.dumps(tab))
    assert b.counters_for("CLS", "wl") == 123.0
    assert b.counters_for("OTHER", "wl") is None
    with open(csrc / b.COUNTED_SOURCES[0], "a") as fh:   # a kernel source changes
        fh.write("\n// changed\n")
    assert b.counters_for("CLS", "wl") is None
