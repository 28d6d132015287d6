"""Throughput of the Fast-dLLM block-cache decode path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A "step" of this benchmark is one whole generation (``dllm_generate``): prefill, every
cached denoising step with its confidence/unmask pass, and the refresh after each block,
for one batch of seeded synthetic prompts.  Weights, tokens, KV cache and workspace are
resident in HBM before the timed region.  The default workload is the LLaDA-8B-shaped
random-init model with DualCache: prompt 1000 tokens, 1024 generated in blocks of 32,
threshold 0.9, batch 1.

Prints one JSON line: generated tokens/s plus the roofline of the dominant kernel class
(timed live with HIP events on its stream) and the CPU oracle's throughput on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from dataclasses import replace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_VALU_TFLOPS = 157.3

# Dominant kernel class per workload (largest summed duration in the rocprofv3 kernel
# trace of this benchmark; see profiles/).
DOMINANT = {
    "llada8b_dual_p1000_g1024": "STEP_GATE_UP",
    "llada8b_prefix_p256_g256": "STEP_GATE_UP",
    "dream7b_dual_b8_p512_g512": "REF_GATE_UP",
    "tiny_dual": "STEP_GATE_UP",
}


METRIC = {
    "llada8b_dual_p1000_g1024":
        "generated tokens/sec @1 GPU (LLaDA-8B-shape, DualCache, \u03c4=0.9); attn GB/s",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def logit_scale(wl) -> float:
    """The oracle-calibrated logit scale of a named random-init 8B/7B workload
    (tests/golden/logit_scales.json), else the scale its config gives."""
    p = os.path.join(ROOT, "tests", "golden", "logit_scales.json")
    tab = json.load(open(p)) if os.path.exists(p) else {}
    if wl.name in tab:
        return float(tab[wl.name]["logit_scale"])
    return wl.model.logit_scale


def kernel_work(cls: str, wl, R_step: int):
    """Algorithmic (flops, bytes) of one launch of a kernel class."""
    m = wl.model
    B, S, d, F, V = wl.batch, wl.seq_len, m.d_model, m.d_ffn, m.vocab
    D, Hq, Hkv = m.head_dim, m.n_heads, m.n_kv_heads
    e = 2 if m.dtype == "bf16" else 4
    Nqkv = (Hq + 2 * Hkv) * D
    Mr, Ms = B * S, B * R_step

    def lin(M, N, K, out_bytes):
        return 2.0 * M * N * K, float(N * K * e + M * K * e + M * N * out_bytes)
    table = {
        "REF_QKV": lin(Mr, Nqkv, d, e), "REF_O": lin(Mr, d, Hq * D, 8),
        "REF_GATE_UP": lin(Mr, 2 * F, d, e / 2), "REF_DOWN": lin(Mr, d, F, 8),
        "STEP_QKV": lin(Ms, Nqkv, d, e), "STEP_O": lin(Ms, d, Hq * D, 8),
        "STEP_GATE_UP": lin(Ms, 2 * F, d, e / 2), "STEP_DOWN": lin(Ms, d, F, 8),
        "LM_HEAD": lin(B * wl.block_len, V, d, 4),
        "REF_ATTN": (4.0 * B * S * S * Hq * D, float(B * (2 * Hq + 2 * Hkv) * S * D * e)),
        "STEP_ATTN": (4.0 * Ms * S * Hq * D, float(B * 2 * Hkv * S * D * e + 2 * Ms * Hq * D * e)),
        "CONF_UNMASK": (5.0 * B * wl.block_len * V, float(B * wl.block_len * V * 4)),
    }
    return table[cls]


def layer_params(m) -> int:
    """Weights of one transformer layer (QKV, O, gate/up, down; norms are negligible)."""
    return ((m.n_heads + 2 * m.n_kv_heads) * m.head_dim * m.d_model
            + m.d_model * m.n_heads * m.head_dim + 3 * m.d_ffn * m.d_model)


def generation_roofline(wl, n_refresh: int, n_steps: int, seconds: float):
    """Roofline time of one whole generation from its measured NFE, against the measured
    wall time.  Algorithmic work only (what the method must move or compute):
      * a refresh is the full forward over all S rows, bound by the larger of its MFMA
        time, 2 B S (layer params) L + 4 B S^2 Hq D L flops at the bf16 peak, and its HBM
        time (layer weights once plus the K/V it writes);
      * a cached step reads every layer's weights, the LM head and the whole K/V cache
        once (HBM-bound at one block of rows);
      * each block's first step is fused with its refresh here: on top of the refresh it
        needs the last layer's weights and the LM head once more.
    T_roof = n_refresh (refresh + fused-step tail) + (n_steps - n_refresh) cached steps."""
    m = wl.model
    B, S, L, e = wl.batch, wl.seq_len, m.n_layers, 2 if m.dtype == "bf16" else 4
    P = layer_params(m)
    head = m.vocab * m.d_model
    kv = L * 2 * B * m.n_kv_heads * S * m.head_dim * e
    f_ref = 2.0 * B * S * P * L + 4.0 * B * S * S * m.n_heads * m.head_dim * L
    b_ref = P * L * e + kv
    t_ref = max(f_ref / (PEAK_BF16_TFLOPS * 1e12), b_ref / (PEAK_HBM_GBS * 1e9))
    b_step = (P * L + head) * e + kv
    t_step = b_step / (PEAK_HBM_GBS * 1e9)
    t_tail = (P + head) * e / (PEAK_HBM_GBS * 1e9)
    n_cached = n_steps - n_refresh
    t_roof = n_refresh * (t_ref + t_tail) + n_cached * t_step
    return {"t_roof_s": round(t_roof, 4), "t_s": round(seconds, 4),
            "frac": round(t_roof / seconds, 4),
            "refresh_roof_ms": round(t_ref * 1e3, 3), "refresh_tflop": round(f_ref / 1e12, 2),
            "step_roof_ms": round(t_step * 1e3, 3), "step_gb": round(b_step / 1e9, 3),
            "n_refresh": n_refresh, "n_cached_steps": n_cached}


def counters_for(cls: str, wl_name: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    tab = json.load(open(p))
    ent = tab.get(f"{wl_name}:{cls}")
    if not ent:
        return None
    if ent.get("source_sha") != source_sha():
        return None
    return ent.get("bytes_per_launch")


# The files the counted kernels (the GEMMs) are built from; a change to any of them
# invalidates the stored counter values.
COUNTED_SOURCES = ("k_gemm.hip", "kernels.h", "common.h")


def source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "diffusion_dllm_block_amd", "csrc")
    for f in COUNTED_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, nfe_steps: int, nfe_refreshes: int, budget_s: float = 12.0):
    """The oracle as it stands, in float32 with bf16 rounding at its storage points (its
    timed mode for bf16 models), on a bounded sample of the workload: one full layer over
    all S rows (a refresh layer) and one cached-step layer over the block rows against the
    cache, plus the LM head and the confidence/unmask rule, each run three times or more,
    until about ``budget_s`` seconds of work are spent (the fastest run of each kept).
    Scaled by the layer count and combined with the GPU run's NFE into generated tokens/s
    (extrapolated)."""
    from threadpoolctl import threadpool_info
    from oracle import decode
    from oracle import model as om
    m = wl.model
    dt = np.float32 if m.dtype == "bf16" else np.float64
    wl1 = replace(wl, model=replace(m, n_layers=1))
    M = om.OracleModel(wl1, dtype=dt)
    for n in ("embed", "final_norm", "lm_head"):
        M.w(n)
    for n in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate_up", "w_down"):
        M.w(n, 0)
    prompt = synth.make_prompt(wl1)
    B, P, S, K = wl.batch, wl.prompt_len, wl.seq_len, wl.block_len
    tokens = np.concatenate([prompt, np.full((B, wl.gen_len), m.mask_id, np.int64)], axis=1)

    # the four parts get shares of the budget: refresh layer 3/4, the rest 1/12 each
    def best(f, share):
        ts = []
        out = None
        while len(ts) < 3 or (sum(ts) < share * budget_s and len(ts) < 20):
            t0 = time.perf_counter()
            out = f()
            ts.append(time.perf_counter() - t0)
        return min(ts), sum(ts), out

    def ref_layer():
        x = om.embed(M, tokens)
        q, k, v = om.layer_qkv(M, 0, x, np.arange(S))
        om.layer_rest(M, 0, x, q, k, v)
        return k, v
    t_ref_layer, spent, (k, v) = best(ref_layer, 0.75)
    cache = om.KVCache(1, B, m.n_kv_heads, S, m.head_dim, dt)
    cache.K[0][...] = k
    cache.V[0][...] = v
    t_step_1, sp, logits = best(lambda: om.cached_step(M, tokens, cache, P, P + K, wl.cache_mode),
                                1 / 12)
    spent += sp

    def dec():
        conf, arg = decode.confidence_argmax(logits.reshape(B * K, -1), m.mask_id)
        decode.unmask(tokens[:, P:P + K], conf.reshape(B, K), arg.reshape(B, K), m.mask_id,
                      wl.threshold)
    t_dec, sp, _ = best(dec, 1 / 12)
    spent += sp
    # a 1-layer cached step = 1 layer + LM head; split the LM head off with a timed call
    t_head, sp, _ = best(lambda: om.lm_head(M, np.zeros((B, K, m.d_model), dt)), 1 / 12)
    spent += sp
    t_step_layer = max(t_step_1 - t_head, 0.0)
    L = m.n_layers
    t_refresh = L * t_ref_layer
    t_step = L * t_step_layer + t_head + t_dec
    total = nfe_refreshes * t_refresh + nfe_steps * t_step
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    prec = "float32 with bf16 rounding at the storage points" if dt == np.float32 else "float64"
    return {
        "value": round(B * wl.gen_len / total, 4), "unit": "tokens/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"oracle in {prec}, 1 of {L} layers timed (best of at least 3 runs, "
                   f"{spent:.1f} s of work): "
                   f"full-sequence layer {t_ref_layer:.2f} s, cached-step layer "
                   f"{t_step_layer:.3f} s, LM head {t_head:.3f} s, decode {t_dec:.3f} s; "
                   f"scaled x{L} and by the GPU run's NFE ({nfe_steps} steps, "
                   f"{nfe_refreshes} refreshes); extrapolated"),
        "sample_seconds": round(spent, 2),
        "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
        "blas_threads": threads,
        "openblas_num_threads_env": os.environ.get("OPENBLAS_NUM_THREADS"),
    }


def _graph_time(torch, launch_all, n_launch: int, rounds: int) -> float:
    """Average microseconds per launch of a sequence of launches captured once into a
    HIP graph and replayed back to back (no host launch cost inside the timed region)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch_all()                     # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch_all()
    g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(rounds):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (rounds * n_launch)


def _attn_rate(lib, torch, bd, S: int, nset: int, rounds: int, B=1, Hq=32, Hkv=32, R=32, D=128):
    """Block attention of R query rows per head against S cached keys, bf16, q/k/v
    N(0, 1) from the seeded device generator; nset buffer sets rotated per replay."""
    Sp = (S + 63) // 64 * 64
    sets = []
    st0 = bd.stream_handle()
    for i in range(nset):
        t = {}
        for name, n, tid in (("q", B * Hq * R * D, 0xA100), ("k", B * Hkv * Sp * D, 0xA101),
                             ("vt", B * Hkv * D * Sp, 0xA102)):
            t[name] = torch.empty(n, dtype=torch.int16, device="cuda")
            lib.call("dllm_synth_fill", bd.ptr(t[name]), n, 1, 42 + i, tid, 1.0, 0, st0)
        t["o"] = torch.empty(B * R * Hq * D, dtype=torch.int16, device="cuda")
        sets.append(t)
    wsb = lib.raw("dllm_kernel_workspace_bytes")(B, Hq, R, S, D, 0, 0)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def attn_all():
        st = bd.stream_handle()
        for t in sets:
            lib.call("dllm_kernel_block_attention", bd.ptr(t["q"]), bd.ptr(t["k"]),
                     bd.ptr(t["vt"]), bd.ptr(t["o"]), B, Hq, Hkv, R, S, Sp, D, 1, bd.ptr(ws),
                     wsb, st)
    us = _graph_time(torch, attn_all, nset, rounds)
    nbytes = (B * Hq * R * D * 2) * 2 + B * Hkv * S * D * 2 * 2
    return {"us": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
            "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4), "sets": nset,
            "shape": f"B{B} H{Hq}x{D} q{R} kv{S} bf16"}


def _conf_rate(lib, torch, bd, B: int, K: int, V: int, ldtype: str, nset: int, rounds: int,
               logits_of=None):
    """Confidence/unmask over B sequences of K block rows (all masked, tau 0.9); logits
    from logits_of(i) or N(0, 1) from the seeded device generator."""
    mask_id, tau = V - 1, 0.9
    dt = 1 if ldtype == "bf16" else 0
    tdt = torch.int16 if ldtype == "bf16" else torch.float32
    logits = []
    for i in range(nset):
        if logits_of is not None:
            logits.append(logits_of(i))
        else:
            z = torch.empty(B * K * V, dtype=tdt, device="cuda")
            lib.call("dllm_synth_fill", bd.ptr(z), z.numel(), dt, 43 + i, 0xB010, 1.0, 0,
                     bd.stream_handle())
            logits.append(z)
    toks = torch.full((nset, B * K), mask_id, dtype=torch.int32, device="cuda")
    conf = torch.empty(B * K, dtype=torch.float32, device="cuda")
    arg = torch.empty(B * K, dtype=torch.int32, device="cuda")
    nun = torch.empty(B, dtype=torch.int32, device="cuda")
    rem = torch.empty(B, dtype=torch.int32, device="cuda")
    uidx = torch.empty(B * K, dtype=torch.int32, device="cuda")
    wsb = lib.raw("dllm_kernel_workspace_bytes")(B, 0, 0, 0, 0, K, V)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def conf_all():
        st = bd.stream_handle()
        toks.fill_(mask_id)             # every launch sees fully masked blocks
        for i in range(nset):
            lib.call("dllm_kernel_confidence_unmask", bd.ptr(logits[i]), dt, B, K, V, mask_id,
                     tau, bd.ptr(toks[i]), K, bd.ptr(conf), bd.ptr(arg), bd.ptr(nun),
                     bd.ptr(rem), bd.ptr(uidx), bd.ptr(ws), wsb, st)
    us = _graph_time(torch, conf_all, nset, rounds)
    nbytes = B * K * V * (2 if ldtype == "bf16" else 4)
    return {"us": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
            "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4), "sets": nset,
            "shape": f"[{B * K}, {V}] {ldtype} logits, tau 0.9"}


def kernel_only(lib, torch, bd, rounds: int = 10):
    """Kernel-only rates.  The 8B step shape: block attention of 32 query rows per head
    (32 heads x 128) against 1024 cached keys, and the confidence/unmask pass over
    [32, 126464] bf16 logits (N(0,1) plus a U(0,12) boost at one id per row, tau 0.9, all
    32 positions masked).  Both are small enough to be bound by launch and DRAM latency,
    so the same kernels are also timed where bandwidth binds: attention against 16384
    cached keys (268 MB of K/V), and the confidence pass over the 7B shape's batch of 8
    blocks, [256, 152064] fp32 logits (156 MB).  Launches rotate through buffer sets
    totalling more than the 256 MB Infinity Cache and are replayed from a HIP graph; the
    time per launch is HIP events around the replays divided by the launches (so it
    includes the short gaps between kernels)."""
    out = {"attention": _attn_rate(lib, torch, bd, 1024, 20, rounds)}
    torch.cuda.empty_cache()
    out["attention_16k_keys"] = _attn_rate(lib, torch, bd, 16384, 3, rounds)
    torch.cuda.empty_cache()
    host = synth.boosted_logits(43, 32, 126464, 12.0, "bf16")
    one = torch.from_numpy(host.view(np.int16)).to("cuda")
    out["confidence"] = _conf_rate(lib, torch, bd, 1, 32, 126464, "bf16", 40, rounds,
                                   logits_of=lambda i: one.clone())
    torch.cuda.empty_cache()
    out["confidence_7b_batch8"] = _conf_rate(lib, torch, bd, 8, 32, 152064, "f32", 3, rounds)
    return out


def ablation(model, wl, torch, gen_lens=()):
    """The two halves of the method switched on one at a time, on the same model and
    prompts: no cache (every step a full forward) or the workload's cache, and one token
    per step (threshold 2 > 1: only the forced pick) or threshold decoding.  One timed
    generation each after a warm-up of the cached configuration, plus the other cache
    (prefix for a DualCache workload, and the reverse) with threshold decoding.  With
    gen_lens, the first four runs at each of those generation lengths (same prompt): the
    pages report the cache's speed-up growing with the generation length."""
    from diffusion_dllm_block_amd.engine import Session
    prompt = synth.make_prompt(wl)

    def four(G, other_cache=False):
        runs = [("no cache, one token per step", "none", 2.0),
                ("no cache, parallel decoding", "none", wl.threshold),
                (f"{wl.cache_mode} cache, one token per step", wl.cache_mode, 2.0),
                (f"{wl.cache_mode} cache, parallel decoding (Fast-dLLM)", wl.cache_mode,
                 wl.threshold)]
        if other_cache:  # the other cache of the pages, same decoding rule
            alt = "prefix" if wl.cache_mode == "dual" else "dual"
            runs.append((f"{alt} cache, parallel decoding", alt, wl.threshold))
        warm = Session(model, prompt, G, wl.block_len, wl.threshold, wl.cache_mode)
        warm.generate()
        del warm
        out = []
        for name, mode, tau in runs:
            sess = Session(model, prompt, G, wl.block_len, tau, mode)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            _, st = sess.generate()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            out.append({"config": name, "cache": mode, "threshold": tau,
                        "tokens_per_s": round(wl.batch * G / dt, 2),
                        "seconds": round(dt, 3), "steps": st["steps"],
                        "full_forwards": st["refreshes"],
                        "tokens_per_step": round(wl.batch * G / st["steps"], 3)})
            log(f"ablation G={G} {name}: {dt:.2f} s, {st['steps']} steps, "
                f"{st['refreshes']} full forwards")
            del sess
        base = out[0]["seconds"]
        for r in out:
            r["speedup_vs_no_cache_one_token"] = round(base / r["seconds"], 2)
        return out

    res = {"workload": wl.name, "gen_len": wl.gen_len, "runs": four(wl.gen_len, True)}
    trend = []
    for G in gen_lens:
        if G <= 0 or G % wl.block_len:
            raise SystemExit(f"--ablation-gen-lens: {G} is not a positive multiple of the "
                             f"block length {wl.block_len}")
        runs = res["runs"][:4] if G == wl.gen_len else four(G)
        trend.append({"gen_len": G, "runs": runs})
    if trend:
        res["gen_len_trend"] = trend
    return res


def staleness_trace(sess, wl, blocks: int):
    """Cache staleness across the steps of the first `blocks` blocks (dllm_cache_staleness
    before every cached step): per step, the cosine similarity of the cached and the
    exact K and V at the positions the step reads from the cache, averaged over layers,
    its worst layer mean and worst single vector, and the reuse ratio.  Random-init
    weights: a check that the instrumentation runs at the real shape, not a measurement of
    the pages' trained-model claim."""
    out = []
    sess.reset_tokens()
    for b in range(min(blocks, sess.n_blocks)):
        o = sess.refresh_step(b, logits=False)
        n = 1
        while int(o["remaining"].max().item()) > 0:
            st = sess.staleness(b)
            out.append({"block": b, "step": n,
                        "k_mean": round(float(st["k_mean"].mean()), 6),
                        "v_mean": round(float(st["v_mean"].mean()), 6),
                        "worst_layer_mean": round(float(min(st["k_mean"].min(),
                                                            st["v_mean"].min())), 6),
                        "worst_vector": round(float(min(st["k_min"].min(), st["v_min"].min())), 6),
                        "reuse": round(st["reuse"], 4)})
            o = sess.step(b, logits=False)
            n += 1
    return {"workload": wl.name, "steps": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llada8b_dual_p1000_g1024",
                    help=f"a named workload: {', '.join(sorted(synth.WORKLOADS))}")
    ap.add_argument("--config", default=None,
                    help="a workload JSON file (the format of synth/workloads/*.json) instead "
                         "of a named workload")
    ap.add_argument("--gen-len", type=int, default=0, help="override (for quick runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the kernel-only rates")
    ap.add_argument("--ablation", action="store_true",
                    help="cache on/off x parallel decoding on/off on the workload, one JSON line")
    ap.add_argument("--ablation-gen-lens", default="",
                    help="with --ablation: also run it at these generation lengths "
                         "(comma-separated multiples of the block length)")
    ap.add_argument("--staleness", type=int, default=0, metavar="BLOCKS",
                    help="cache staleness before every cached step of the first BLOCKS "
                         "blocks, one JSON line (no timing)")
    ap.add_argument("--graphs", action="store_true",
                    help="time generations with each block's cached steps replayed from a "
                         "HIP graph (no kernel-class timing), one JSON line")
    ap.add_argument("--kernels-only", action="store_true",
                    help="only the kernel-only rates (no generation; for profiling)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run plain device copies of this many MiB (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counter scale)")
    ap.add_argument("--stage", choices=["refresh", "step"], default=None,
                    help="time one stage at the workload's full shape instead of whole "
                         "generations: after a prefill, --repeat refreshes, or --repeat cached "
                         "steps of block 0 (for counter runs), one JSON line")
    ap.add_argument("--repeat", type=int, default=10)
    ap.add_argument("--roofline-kernel", default="auto")
    ap.add_argument("--profile-every", type=int, default=7,
                    help="time one launch in N of the roofline kernel class")
    ap.add_argument("--logit-scale", type=float, default=0.0,
                    help="override the calibrated scale (exploration only)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the multi-GPU "
              "layout is a design note, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from diffusion_dllm_block_amd import binding as bd
    from diffusion_dllm_block_amd.engine import Model, Session

    lib = bd.load()
    if a.copy_probe_mb:
        # one elementwise kernel per call that reads and writes exactly n bytes each
        n = a.copy_probe_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: 4 elementwise copies of {n} bytes")
        del src, dst
    if a.kernels_only:
        print(json.dumps({"kernels": kernel_only(lib, torch, bd)}), flush=True)
        return
    base = synth.load_workload(a.config) if a.config else synth.WORKLOADS[a.workload]
    wl = synth.with_scale(base, a.logit_scale if a.logit_scale else logit_scale(base))
    if a.gen_len:
        wl = replace(wl, gen_len=a.gen_len)
    log(f"workload {wl.name}: B={wl.batch} P={wl.prompt_len} G={wl.gen_len} K={wl.block_len} "
        f"mode={wl.cache_mode} scale={wl.model.logit_scale:.4f}")
    t = time.time()
    model = Model.synthetic(lib, wl) if wl.model.dtype == "bf16" else \
        Model.from_host(lib, wl.model, synth.make_weights(wl))
    sess = Session(model, synth.make_prompt(wl), wl.gen_len, wl.block_len, wl.threshold,
                   wl.cache_mode)
    torch.cuda.synchronize()
    log(f"weights + buffers ready in {time.time() - t:.1f} s")
    if a.ablation:
        del sess
        lens = [int(x) for x in a.ablation_gen_lens.split(",") if x.strip()]
        print(json.dumps({"ablation": ablation(model, wl, torch, lens)}), flush=True)
        return
    if a.stage:
        sess.prefill()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(a.repeat):
            if a.stage == "refresh":
                sess.refresh(0)
            else:
                sess.reset_tokens()
                sess.step(0, logits=False)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / a.repeat * 1e3
        log(f"{a.stage}: {ms:.3f} ms per call over {a.repeat}")
        print(json.dumps({"stage": a.stage, "workload": wl.name, "ms_per_call": round(ms, 3),
                          "repeat": a.repeat}), flush=True)
        return
    if a.staleness:
        print(json.dumps({"staleness": staleness_trace(sess, wl, a.staleness)}), flush=True)
        return
    if a.graphs:
        res = {}
        for graphs in (False, True, False, True):
            for _ in range(a.warmup):
                sess.reset_tokens()
                sess.generate(graphs=graphs)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(a.steps):
                sess.reset_tokens()
                _, st = sess.generate(graphs=graphs)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / a.steps
            key = "graphs" if graphs else "eager"
            res.setdefault(key, []).append(round(wl.batch * wl.gen_len / dt, 2))
            log(f"{key}: {dt * 1e3:.1f} ms per generation ({st['steps']} steps)")
        print(json.dumps({"graph_replay": {"workload": wl.name, "tokens_per_s": res}}),
              flush=True)
        return

    for i in range(a.warmup):
        sess.reset_tokens()
        _, st = sess.generate()
        log(f"warmup {i}: {st['ms_total']:.1f} ms, {st['steps']} steps")

    cls = DOMINANT.get(wl.name, "REF_GATE_UP") if a.roofline_kernel == "auto" else a.roofline_kernel
    cid = bd.KERNEL_CLASSES.index(cls)
    # time one launch in a.profile_every (7 is coprime with the layer counts, so the
    # sample rotates through every layer); each timed launch costs two event records
    lib.call("dllm_profile_select_every", cid, a.profile_every)
    stats = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        sess.reset_tokens()
        _, st = sess.generate()
        stats.append(st)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    import ctypes as C
    n_launch, tot_ms = C.c_int32(), C.c_double()
    lib.call("dllm_profile_read", C.byref(n_launch), C.byref(tot_ms))
    lib.call("dllm_profile_select", -1)
    for i, st in enumerate(stats):
        log(f"step {i}: {st['ms_total']:.1f} ms ({st['steps']} cached steps, {st['refreshes']} "
            f"refreshes, {st['speculative_steps']} speculative; refresh {st['ms_refresh']:.1f} ms, "
            f"steps {st['ms_step']:.1f} ms)")

    toks = wl.batch * wl.gen_len * a.steps
    value = toks / dt
    nfe_steps, nfe_ref = stats[-1]["steps"], stats[-1]["refreshes"]
    gen_roof = generation_roofline(wl, nfe_ref, nfe_steps, dt / a.steps) \
        if wl.cache_mode != "none" else None
    R_step = wl.block_len if wl.cache_mode == "dual" else wl.gen_len
    flops, bytes_ = kernel_work(cls, wl, R_step)
    avg_s = tot_ms.value / 1e3 / max(1, n_launch.value)
    mfma = cls.startswith("REF_") and cls != "REF_ATTN" or cls == "REF_ATTN"
    if mfma:
        roof = {"bound": "mfma", "achieved": round(flops / avg_s / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(bytes_ / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = counters_for(cls, wl.name)
    roof["kernel"] = cls
    roof["launches"] = n_launch.value
    roof["sampled_every"] = a.profile_every
    roof["avg_launch_us"] = round(avg_s * 1e6, 2)

    out = {
        "metric": METRIC.get(wl.name, f"generated tokens/sec @1 GPU ({wl.name})"),
        "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(dt / a.steps * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and prompts)",
        "config": {"workload": wl.name, "batch": wl.batch, "prompt_len": wl.prompt_len,
                   "gen_len": wl.gen_len, "block_len": wl.block_len, "cache": wl.cache_mode,
                   "threshold": wl.threshold, "logit_scale": round(wl.model.logit_scale, 4),
                   "nfe_steps": nfe_steps, "nfe_refreshes": nfe_ref,
                   "tokens_per_step": round(wl.batch * wl.gen_len / max(1, nfe_steps), 3),
                   "unmask_fraction_per_step": round(
                       wl.batch * wl.gen_len / max(1, stats[-1]["masked_at_step_start"]), 4)},
        "roofline": roof,
        "generation_roofline": gen_roof,
    }
    if not a.no_kernels:
        log("kernel-only rates (attention, confidence)")
        out["kernels"] = kernel_only(lib, torch, bd)
    if not a.no_cpu_baseline:
        del sess, model
        torch.cuda.empty_cache()
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl, nfe_steps, nfe_ref)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
