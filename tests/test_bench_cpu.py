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


def test_generation_roofline_arithmetic():
    """The whole-generation roofline from the NFE: at the 8B DualCache shape a refresh is
    2 B S (layer params) L + 4 B S^2 Hq D L = 30.4 TFLOP (12.2 ms at 2.5 PFLOP/s) and a cached
    step streams the 15.0 GB of weights plus the 1.06 GB KV cache (2.0 ms at 8 TB/s)."""
    import synth
    b = load_bench()
    wl = synth.WORKLOADS["llada8b_dual_p1000_g1024"]
    r = b.generation_roofline(wl, 32, 918, 4.84)
    assert abs(r["refresh_tflop"] - 30.4) < 0.05
    assert abs(r["refresh_roof_ms"] - 12.16) < 0.01
    assert abs(r["step_gb"] - 16.056) < 0.001
    assert r["n_cached_steps"] == 886
    # 32 (refresh + fused-step tail) + 886 cached steps
    tail = (b.layer_params(wl.model) + wl.model.vocab * wl.model.d_model) * 2 / 8e12
    want = 32 * (12.16e-3 + tail) + 886 * 2.007e-3
    assert abs(r["t_roof_s"] - want) < 2e-3
    assert abs(r["frac"] - r["t_roof_s"] / 4.84) < 1e-3


def test_bench_accepts_a_workload_file(tmp_path):
    b = load_bench()
    import synth
    wl = synth.load_workload(os.path.join(synth.WORKLOAD_DIR, "llada8b_dual_p1000_g1024.json"))
    # the named 8B workloads take their oracle-calibrated scale, a custom one its own
    assert abs(b.logit_scale(wl) - 7.3032) < 1e-3
    from dataclasses import replace
    assert b.logit_scale(replace(wl, name="custom")) == wl.model.logit_scale
