"""GPU parity of the whole decode path (prefill, refresh, cached steps, generate) against
the CPU oracle, through the C ABI."""
import numpy as np
import pytest
from dataclasses import replace

import synth
from gpu_util import (CONF_TOL_F32, grade_confidence_stage, grade_unmask_stage, rel_inf,
                      safe_sequences)
from oracle import decode
from oracle import model as om
from oracle.generate import Session as OSession

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from diffusion_dllm_block_amd import binding as bd  # noqa: E402
from diffusion_dllm_block_amd.engine import Model, Session  # noqa: E402


def gpu_model(lib, wl):
    return Model.from_host(lib, wl.model, synth.make_weights(wl))


def teacher_forced(lib, wl, logits_tol, conf_tol=None):
    """Step both sides from the oracle's token state; compare every step.

    Graded on every sequence of every step (per stage, as the decoding rule is pure
    compare-and-index work on what the GPU computed):
      * logits against the oracle's, to ``logits_tol`` relative;
      * the confidence pass against the oracle's definition on the GPU's own logits
        (argmax exact, confidence to fp32 rounding);
      * the unmask rule against the oracle's on the GPU's own confidences and argmaxes
        (tokens, counts, masks left: bit for bit).
    End to end (the GPU's decisions against the oracle's own) wherever no decision can
    flip under the measured logit error, counted.  With ``conf_tol`` the GPU's
    confidences must also lie within it of the oracle's."""
    m = wl.model
    M = om.OracleModel(wl)
    prompt = synth.make_prompt(wl)
    osess = OSession(M, prompt, wl.gen_len, wl.block_len, wl.threshold, wl.cache_mode)
    gsess = Session(gpu_model(lib, wl), prompt, wl.gen_len, wl.block_len, wl.threshold,
                    wl.cache_mode)
    st = {"worst": 0.0, "steps": 0, "seq_steps": 0, "checked": 0, "excluded": 0,
          "multi": 0, "max_dconf": 0.0}
    for b in range(osess.n_blocks):
        osess.refresh()
        if b == 0:
            gsess.prefill()
        else:
            gsess.refresh(b)
        while not osess.block_done(b):
            s0, s1 = osess.block_span(b)
            before = osess.tokens[:, s0:s1].copy()
            gsess.tokens.copy_(torch.from_numpy(osess.tokens.astype(np.int32)))
            g = gsess.step(b)
            o = osess.step(b)
            torch.cuda.synchronize()
            gl = g["logits"].cpu().numpy().reshape(o["logits"].shape).astype(np.float64)
            err = rel_inf(gl, o["logits"])
            st["worst"] = max(st["worst"], err)
            assert err < logits_tol, f"block {b}: logits rel err {err}"
            gconf = g["conf"].cpu().numpy().astype(np.float64)
            garg = g["argmax"].cpu().numpy()
            gtok = gsess.tokens.cpu().numpy()[:, s0:s1]
            gnun = g["n_unmasked"].cpu().numpy()
            grem = g["remaining"].cpu().numpy()
            grade_confidence_stage(gl.reshape(-1, m.vocab), gconf, garg, m.mask_id)
            grade_unmask_stage(before, gconf, garg, gtok, gnun, grem, m.mask_id, wl.threshold)
            st["steps"] += 1
            st["seq_steps"] += wl.batch
            st["multi"] += int(np.sum(gnun >= 2))
            masked = before == m.mask_id
            # per-row bound: |d log p_max| <= 2 max_v |d logit|, so a confidence c can move
            # by at most c (exp(2 dl) - 1), plus the fp32 rounding of the exp-sum
            dl = np.max(np.abs(gl - o["logits"]), axis=-1)            # [B, K]
            unc = o["conf"] * (np.expm1(2.0 * dl) + 2e-5)
            ok = safe_sequences(o["conf"], unc, wl.threshold, masked)
            for bb in range(wl.batch):
                for i in range(wl.block_len):
                    z = np.sort(o["logits"][bb, i][np.arange(m.vocab) != m.mask_id])
                    if z[-1] - z[-2] > 2.0 * dl[bb, i] + 1e-6:
                        assert garg[bb, i] == o["argmax"][bb, i], f"block {b} seq {bb} row {i}"
                if not ok[bb]:
                    st["excluded"] += 1
                    continue
                st["checked"] += 1
                assert np.array_equal(gtok[bb], osess.tokens[bb, s0:s1]), f"block {b} seq {bb}"
                assert gnun[bb] == o["n_unmasked"][bb]
                assert grem[bb] == o["remaining"][bb]
            dconf = float(np.max(np.abs(gconf - o["conf"])))
            st["max_dconf"] = max(st["max_dconf"], dconf)
            if conf_tol is not None:
                assert dconf <= conf_tol, f"block {b}: confidence differs by {dconf}"
    assert st["seq_steps"] > 0
    print(f"teacher-forced {wl.name} {wl.cache_mode} tau {wl.threshold}: {st}")
    return st


@pytest.mark.parametrize("mode,tau", [("dual", 0.9), ("prefix", 0.9), ("dual", 0.5),
                                      ("prefix", 0.7)])
def test_tiny_fp32_teacher_forced(lib, mode, tau):
    """The tiny fp32 model at 1e-4 (logits) in both cache modes.  At tau 0.9 it decodes
    one token per step; tau 0.5 and 0.7 take the multi-token path (several positions
    at or above the threshold decoded in one step), which must then be seen."""
    wl = replace(synth.WORKLOADS["tiny_dual"], cache_mode=mode, threshold=tau)
    st = teacher_forced(lib, wl, 1e-4, CONF_TOL_F32)
    assert st["checked"] >= 0.8 * (st["checked"] + st["excluded"])
    if tau < 0.9:
        assert st["multi"] >= 2, "no step decoded several tokens"


@pytest.mark.parametrize("mode,P", [("dual", 13), ("prefix", 13), ("dual", 18)])
def test_tiny_fp32_teacher_forced_ragged_prompt(lib, mode, P):
    """Prompt lengths that are not a multiple of 4: block positions and the sequence
    length S are then not in runs of 4, so the GEMM epilogues write the value cache and
    the RoPE'd rows element by element (the fallback of the 4-wide epilogue)."""
    wl = replace(synth.WORKLOADS["tiny_dual"], cache_mode=mode, prompt_len=P)
    st = teacher_forced(lib, wl, 1e-4, CONF_TOL_F32)
    assert st["steps"] >= wl.gen_len // wl.block_len


def free_running_compare(got, gspb, want, ospb, unsafe_blocks, K, n_blocks):
    """Blocks compared in order while every step of every earlier block (and the block
    itself) took decisions that cannot flip: identical tokens and steps per block.  The
    state entering such a block is identical on both sides, so its decisions must be.
    Returns the number of blocks compared."""
    n = 0
    for b in range(n_blocks):
        if b in unsafe_blocks:
            break
        assert np.array_equal(got[:, b * K:(b + 1) * K], want[:, b * K:(b + 1) * K]), f"block {b}"
        assert gspb[b] == ospb[b], f"block {b}: steps {gspb[b]} vs {ospb[b]}"
        n += 1
    return n


@pytest.mark.parametrize("tau", [0.9, 0.5])
def test_tiny_fp32_free_running_generate(lib, tau):
    """dllm_generate (each block's refresh fused with its first step, later steps
    queued ahead) against the oracle's generate, run independently.  Blocks are
    compared while no decision of the oracle's run lies within the fp32 confidence bound
    of a flip (CONF_TOL_F32, asserted by the teacher-forced tests); at least one must
    be."""
    wl = replace(synth.WORKLOADS["tiny_dual"], threshold=tau)
    M = om.OracleModel(wl)
    prompt = synth.make_prompt(wl)
    unsafe = set()
    osess = OSession(M, prompt, wl.gen_len, wl.block_len, wl.threshold, wl.cache_mode)

    def rec(b, n, out):
        s0, s1 = osess.block_span(b)
        masked = (osess.tokens[:, s0:s1] == wl.model.mask_id) | out["U"]
        if not safe_sequences(out["conf"], CONF_TOL_F32, wl.threshold, masked).all():
            unsafe.add(b)
    want, ost = osess.generate(on_step=rec)
    gs = Session(gpu_model(lib, wl), prompt, wl.gen_len, wl.block_len, wl.threshold,
                 wl.cache_mode)
    got, gst = gs.generate()
    assert gst["steps"] == sum(gst["steps_per_block"])
    assert gst["refreshes"] == wl.gen_len // wl.block_len
    n = free_running_compare(got, gst["steps_per_block"], want, ost["steps_per_block"], unsafe,
                             wl.block_len, osess.n_blocks)
    print(f"tau {tau}: blocks compared {n} of {osess.n_blocks}; steps per block "
          f"{ost['steps_per_block']}")
    assert n >= 1


def test_tiny_fp32_no_cache_generate(lib):
    """No-cache mode (every step a full forward) against the oracle's no-cache decoding,
    with and without parallel decoding (tau 0.9, and tau > 1: one token per step),
    compared block by block as in the free-running test."""
    for tau in (0.9, 1.5):
        wl = replace(synth.WORKLOADS["tiny_dual"], cache_mode="none", threshold=tau)
        m = wl.model
        M = om.OracleModel(wl)
        prompt = synth.make_prompt(wl)
        osess = OSession(M, prompt, wl.gen_len, wl.block_len, tau, "dual")
        unsafe, steps_per_block = set(), []
        for b in range(osess.n_blocks):
            n = 0
            while not osess.block_done(b):
                s0, s1 = osess.block_span(b)
                _, z = om.full_forward(M, osess.tokens, logit_rows=slice(s0, s1))
                B, K, V = z.shape
                conf, arg = decode.confidence_argmax(z.reshape(B * K, V), m.mask_id)
                conf, arg = conf.reshape(B, K), arg.reshape(B, K)
                masked = osess.tokens[:, s0:s1] == m.mask_id
                if not safe_sequences(conf, CONF_TOL_F32, tau, masked).all():
                    unsafe.add(b)
                new, *_ = decode.unmask(osess.tokens[:, s0:s1], conf, arg, m.mask_id, tau)
                osess.tokens[:, s0:s1] = new
                n += 1
            steps_per_block.append(n)
        gs = Session(gpu_model(lib, wl), prompt, wl.gen_len, wl.block_len, tau, "none")
        got, gst = gs.generate()
        assert gst["steps"] == sum(gst["steps_per_block"])
        assert gst["refreshes"] == gst["steps"]          # every step a full forward
        if tau > 1:
            assert gst["steps_per_block"] == [wl.block_len] * osess.n_blocks
        n = free_running_compare(got, gst["steps_per_block"], osess.tokens[:, wl.prompt_len:],
                                 steps_per_block, unsafe, wl.block_len, osess.n_blocks)
        print(f"no cache, tau {tau}: blocks compared {n} of {osess.n_blocks}")
        assert n >= 1


def small_bf16(Hq=2, Hkv=2, mode="dual", B=2, P=40, G=64, K=32, V=2048, gain=0.1, scale=12.0):
    m = synth.ModelShape(n_layers=2, d_model=256, n_heads=Hq, n_kv_heads=Hkv, head_dim=128,
                         d_ffn=512, vocab=V, logit_scale=scale, dtype="bf16")
    return synth.Workload("small_bf16", m, batch=B, prompt_len=P, gen_len=G, block_len=K,
                          cache_mode=mode, norm_gain_std=gain)


@pytest.mark.parametrize("Hq,Hkv,mode,B,K,P", [(2, 2, "dual", 2, 32, 40), (4, 1, "dual", 3, 16, 40),
                                             (2, 2, "prefix", 2, 32, 40), (2, 1, "prefix", 1, 8, 40),
                                             (2, 1, "dual", 2, 32, 400), (2, 1, "dual", 2, 32, 37),
                                             (2, 2, "prefix", 1, 16, 45),
                                             (2, 1, "dual", 2, 32, 401)])
def test_small_bf16_teacher_forced(lib, Hq, Hkv, mode, B, K, P):
    # P = 400: B * S = 928 rows, so the refresh runs the large-tile GEMM path; P = 37, 45
    # and 401 put the block positions and S off runs of 4 (element-by-element value-cache
    # and RoPE writes in the epilogues, on the mid, tiled and large-tile kernels)
    wl = small_bf16(Hq, Hkv, mode, B=B, K=K, P=P)
    st = teacher_forced(lib, wl, 2e-2)
    # bf16 logits differ by ~5e-3 relative, which moves confidences by up to
    # conf * (exp(2 dl) - 1): most end-to-end decisions are inside that band, so they
    # are counted where they cannot flip; every step's confidence pass and unmask rule
    # were graded per stage on the GPU's own outputs (inside teacher_forced)
    assert st["steps"] >= wl.gen_len // wl.block_len


def test_bf16_steps_are_deterministic(lib):
    wl = small_bf16()
    model = gpu_model(lib, wl)
    prompt = synth.make_prompt(wl)
    outs = []
    for _ in range(2):
        s = Session(model, prompt, wl.gen_len, wl.block_len, wl.threshold, wl.cache_mode)
        s.prefill()
        o = s.step(0)
        torch.cuda.synchronize()
        outs.append((o["logits"].cpu().numpy().copy(), s.tokens.cpu().numpy().copy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("entry", ["step", "refresh_step"])
def test_decisions_without_logits_match_with_logits(lib, entry):
    """Without a logits buffer the confidence pass sums the LM head's split partials
    itself (no fp32 logits in memory); with one it also stores them.  The logits are the
    same values either way, so confidence, argmax and the unmasked tokens must agree bit
    for bit (two sessions from the same state)."""
    wl = small_bf16(B=2, K=32)
    model = gpu_model(lib, wl)
    prompt = synth.make_prompt(wl)
    outs = []
    for want in (True, False):
        s = Session(model, prompt, wl.gen_len, wl.block_len, wl.threshold, wl.cache_mode)
        if entry == "step":
            s.prefill()
            o = s.step(0, logits=want)
        else:
            o = s.refresh_step(0, logits=want)
        torch.cuda.synchronize()
        assert (o["logits"] is not None) == want
        outs.append([o["conf"].cpu().numpy().copy(), o["argmax"].cpu().numpy().copy(),
                     s.tokens.cpu().numpy().copy(), o["n_unmasked"].cpu().numpy().copy()])
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)


def test_first_step_after_refresh_matches_full_forward_bf16(lib):
    """Property (a) on the GPU path: after a refresh, the first cached step's logits equal
    the oracle's no-cache full forward of the same tokens (both cache modes)."""
    for mode in ("dual", "prefix"):
        wl = small_bf16(mode=mode)
        M = om.OracleModel(wl)
        prompt = synth.make_prompt(wl)
        gs = Session(gpu_model(lib, wl), prompt, wl.gen_len, wl.block_len, wl.threshold, mode)
        gs.prefill()
        o = gs.step(0)
        torch.cuda.synchronize()
        toks = np.concatenate([prompt, np.full((wl.batch, wl.gen_len), wl.model.mask_id)], 1)
        s0 = wl.prompt_len
        _, ref = om.full_forward(M, toks, logit_rows=slice(s0, s0 + wl.block_len))
        got = o["logits"].cpu().numpy().reshape(ref.shape)
        assert rel_inf(got, ref) < 2e-2


@pytest.mark.parametrize("kind,mode", [("fp32", "dual"), ("fp32", "prefix"), ("bf16", "dual"),
                                       ("bf16", "prefix"), ("bf16_large_tiles", "dual")])
def test_refresh_step_matches_full_forward(lib, kind, mode):
    """dllm_refresh_step (a block's refresh fused with its first step) against the
    oracle's no-cache full forward of the same tokens, property (a), for block 0 (the
    prefill) and block 1; its unmask decisions wherever they cannot flip."""
    if kind == "fp32":
        wl, tol = replace(synth.WORKLOADS["tiny_dual"], cache_mode=mode), 1e-4
    else:
        wl, tol = small_bf16(mode=mode, P=400 if kind == "bf16_large_tiles" else 40), 2e-2
    m = wl.model
    M = om.OracleModel(wl)
    prompt = synth.make_prompt(wl)
    gs = Session(gpu_model(lib, wl), prompt, wl.gen_len, wl.block_len, wl.threshold, mode)
    r = np.random.default_rng(11)
    toks = np.concatenate([prompt, np.full((wl.batch, wl.gen_len), m.mask_id)], 1)
    K = wl.block_len
    for b in (0, 1):
        s0 = wl.prompt_len + b * K
        if b == 1:  # block 0 decoded (ids below mask_id = vocab - 1), some of block 1 too
            toks[:, s0 - K:s0] = r.integers(0, m.mask_id, (wl.batch, K))
            toks[:, s0:s0 + K // 4] = r.integers(0, m.mask_id, (wl.batch, K // 4))
        gs.tokens.copy_(torch.from_numpy(toks.astype(np.int32)))
        out = gs.refresh_step(b)
        torch.cuda.synchronize()
        _, ref = om.full_forward(M, toks, logit_rows=slice(s0, s0 + K))
        got = out["logits"].cpu().numpy().reshape(ref.shape).astype(np.float64)
        assert rel_inf(got, ref) < tol, f"block {b}"
        conf, arg = decode.confidence_argmax(ref.reshape(-1, m.vocab), m.mask_id)
        conf, arg = conf.reshape(wl.batch, K), arg.reshape(wl.batch, K)
        blk = toks[:, s0:s0 + K]
        # per stage, every sequence: confidence pass on the GPU's logits, unmask rule on
        # the GPU's confidences and argmaxes
        gconf = out["conf"].cpu().numpy()
        garg = out["argmax"].cpu().numpy()
        grade_confidence_stage(got.reshape(-1, m.vocab), gconf, garg, m.mask_id)
        grade_unmask_stage(blk, gconf, garg, gs.tokens.cpu().numpy()[:, s0:s0 + K],
                           out["n_unmasked"].cpu().numpy(), out["remaining"].cpu().numpy(),
                           m.mask_id, wl.threshold)
        if kind == "fp32":
            assert np.max(np.abs(gconf - conf)) <= CONF_TOL_F32
        want, U, wn, wr = decode.unmask(blk, conf, arg, m.mask_id, wl.threshold)
        dl = np.max(np.abs(got - ref), axis=-1)
        unc = conf * (np.expm1(2.0 * dl) + 2e-5)
        ok = safe_sequences(conf, unc, wl.threshold, blk == m.mask_id)
        gtok = gs.tokens.cpu().numpy()[:, s0:s0 + K]
        gchanged = gtok != blk
        for bb in np.nonzero(ok)[0]:
            assert np.array_equal(gchanged[bb], U[bb]), f"block {b} seq {bb}"
            assert out["n_unmasked"][bb].item() == wn[bb]
            assert out["remaining"][bb].item() == wr[bb]
            for i in np.nonzero(U[bb])[0]:
                z = np.sort(ref[bb, i][np.arange(m.vocab) != m.mask_id])
                if z[-1] - z[-2] > 2.0 * dl[bb, i] + 1e-6:
                    assert gtok[bb, i] == want[bb, i], f"block {b} seq {bb} row {i}"
        toks = gs.tokens.cpu().numpy().astype(np.int64)


def test_generate_properties_llada_shape_two_blocks(lib):
    """The 8B LLaDA shape (weights made on the device), DualCache, 2 blocks of 32:
    every step decodes >= 1 token, blocks finish in <= 32 steps, no mask token is
    emitted, and two runs give identical tokens."""
    wl = replace(synth.WORKLOADS["llada8b_dual_p1000_g1024"], gen_len=64)
    wl = synth.with_scale(wl, 20.0)
    model = Model.synthetic(lib, wl)
    prompt = synth.make_prompt(wl)
    res = []
    for _ in range(2):
        s = Session(model, prompt, wl.gen_len, wl.block_len, wl.threshold, wl.cache_mode)
        toks, st = s.generate()
        res.append(toks)
        assert all(1 <= n <= 32 for n in st["steps_per_block"])
        assert st["refreshes"] == 2
        assert not (toks == wl.model.mask_id).any()
        assert toks.min() >= 0 and toks.max() < wl.model.vocab - 1
    assert np.array_equal(res[0], res[1])
    del model
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode,tau", [("dual", 0.9), ("dual", 0.3), ("prefix", 0.5),
                                      ("none", 0.6)])
def test_generate_matches_the_step_by_step_loop(lib, mode, tau):
    """dllm_generate queues the next step before reading the previous step's outcome
    (and on speculation, one more when that outcome left two or more masks): tokens and
    steps per block must equal a host loop that reads every outcome before the next
    step.  Low thresholds decode several tokens per step, so speculative steps that
    find their block finished occur and must change nothing."""
    wl = small_bf16(Hq=2, Hkv=1, mode="dual" if mode == "none" else mode, B=2, K=16, P=40)
    model = gpu_model(lib, wl)
    prompt = synth.make_prompt(wl)
    s = Session(model, prompt, wl.gen_len, wl.block_len, tau, mode)
    spb = []
    for b in range(s.n_blocks):
        s.refresh_step(b, logits=False)
        n = 1
        while int(s.remaining.max().item()) > 0:
            if mode == "none":
                s.refresh_step(b, logits=False)
            else:
                s.step(b, logits=False)
            n += 1
            assert n <= wl.block_len
        spb.append(n)
    want = s.tokens.cpu().numpy()[:, s.P:].copy()
    g = Session(model, prompt, wl.gen_len, wl.block_len, tau, mode)
    got, st = g.generate()
    assert np.array_equal(got, want)
    assert st["steps_per_block"] == spb and st["steps"] == sum(spb)
    assert 0 <= st["speculative_steps"] <= s.n_blocks
    print(f"steps per block {spb}, speculative steps {st['speculative_steps']}")


@pytest.mark.parametrize("mode,tau", [("dual", 0.9), ("dual", 0.3), ("prefix", 0.9)])
def test_graph_replay_generate_matches_eager(lib, mode, tau):
    """dllm_generate_graphs replays each block's captured cached step; every replay is
    followed by the host's read of the step's outcome, and every step's decisions feed
    the next: tokens and steps per block must equal the eager loop's, bit for bit, over
    two runs (the second reuses nothing: graphs live for one call)."""
    wl = small_bf16(Hq=2, Hkv=1, mode=mode, B=2, K=16, P=40)
    model = gpu_model(lib, wl)
    prompt = synth.make_prompt(wl)
    e = Session(model, prompt, wl.gen_len, wl.block_len, tau, mode)
    want, st_e = e.generate()
    for _ in range(2):
        g = Session(model, prompt, wl.gen_len, wl.block_len, tau, mode)
        got, st_g = g.generate(graphs=True)
        assert np.array_equal(got, want)
        assert st_g["steps_per_block"] == st_e["steps_per_block"]
        assert st_g["steps"] == st_e["steps"]


def test_graph_replay_generate_matches_eager_llada_shape(lib):
    """The 8B LLaDA shape (weights made on the device), DualCache, two blocks."""
    wl = replace(synth.WORKLOADS["llada8b_dual_p1000_g1024"], gen_len=64)
    wl = synth.with_scale(wl, 20.0)
    model = Model.synthetic(lib, wl)
    prompt = synth.make_prompt(wl)
    out = []
    for graphs in (False, True):
        s = Session(model, prompt, wl.gen_len, wl.block_len, wl.threshold, wl.cache_mode)
        toks, st = s.generate(graphs=graphs)
        out.append((toks, st["steps_per_block"]))
    assert np.array_equal(out[0][0], out[1][0]) and out[0][1] == out[1][1]
    del model
    torch.cuda.empty_cache()


FULL_SIZE = ["llada8b_dual_p1000_g1024", "llada8b_prefix_p256_g256", "dream7b_dual_b8_p512_g512"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_first_step_full_size_matches_oracle_sample(lib, name):
    """The full 8B/7B shapes at their calibrated scale: after the prefill, the first
    cached step's logits at the oracle's sampled (row, id) pairs, its argmax and its
    confidence.  The sample was written by tests/golden/make_logit_scales.py from the
    oracle (float32 with bf16 storage rounding), so the bound is the bf16 one: logit
    errors within 2e-2 of the row's largest logit, argmax equal wherever the top-2 gap
    exceeds twice the observed error, confidence within conf * (exp(2 dl) - 1)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", f"first_step_{name}.json")
    if not os.path.exists(path):
        pytest.skip(f"no oracle sample for {name}")
    fx = json.load(open(path))
    wl = synth.with_scale(synth.WORKLOADS[name], fx["logit_scale"])
    model = Model.synthetic(lib, wl)
    s = Session(model, synth.make_prompt(wl), wl.gen_len, wl.block_len, wl.threshold,
                wl.cache_mode)
    s.prefill()
    o = s.step(0)
    torch.cuda.synchronize()
    V = wl.model.vocab
    lg = o["logits"].cpu().numpy().reshape(wl.batch, wl.block_len, V)[0].astype(np.float64)
    conf = o["conf"].cpu().numpy().reshape(wl.batch, wl.block_len)[0]
    arg = o["argmax"].cpu().numpy().reshape(wl.batch, wl.block_len)[0]
    scale = fx["logit_scale"]
    for row in fx["rows"]:
        r, ids = row["row"], np.array(row["ids"])
        ref = scale * np.array(row["z"])
        dl = np.max(np.abs(lg[r, ids] - ref))
        assert dl <= 2e-2 * np.abs(ref).max(), f"row {r}: logit error {dl}"
        if ref[0] - ref[1] > 2 * dl + 1e-6:
            assert arg[r] == row["argmax"], f"row {r}"
        assert abs(conf[r] - row["conf"]) <= row["conf"] * np.expm1(2 * dl) + 1e-6, f"row {r}"
    del model
    torch.cuda.empty_cache()


def staleness_tol(c, r):
    """Bound on how far a cosine moves when each of its two vectors carries a relative
    L2 error of at most r: to first order |dc| <= 2 r sqrt(1 - c^2) <= 2 r sqrt(2 (1 - c))
    (the gradient of the cosine in a is orthogonal to a, of length sqrt(1 - c^2) / |a|),
    plus r^2 for the second order.  The bound is concave in the cosine, so it also bounds
    the mean, by Jensen, and the minimum (c - bound(c) increases with c)."""
    return 2.0 * r * np.sqrt(2.0 * np.maximum(1.0 - c, 0.0)) + r * r + 1e-6


@pytest.mark.parametrize("kind,mode", [("f32", "dual"), ("f32", "prefix"), ("bf16", "dual"),
                                       ("bf16", "prefix")])
def test_cache_staleness_matches_oracle(lib, kind, mode):
    """dllm_cache_staleness against the oracle's measure on the same token state: 1 right
    after a refresh, layer 0 still 1 after block-only changes, and per layer the mean and
    minimum cosine of cached and exact K/V within the bound implied by the K/V error of
    the two sides (fp32: 1e-5 relative; bf16: 1e-2, a few bf16 ulps)."""
    if kind == "f32":
        wl = replace(synth.WORKLOADS["tiny_dual"], cache_mode=mode)
        r = 1e-5
    else:
        wl = small_bf16(Hq=2, Hkv=1, mode=mode, B=2, K=32, P=40)
        r = 1e-2
    M = om.OracleModel(wl)
    prompt = synth.make_prompt(wl)
    osess = OSession(M, prompt, wl.gen_len, wl.block_len, wl.threshold, mode)
    gsess = Session(gpu_model(lib, wl), prompt, wl.gen_len, wl.block_len, wl.threshold, mode)
    worst = 0.0
    for b in range(min(osess.n_blocks, 2)):
        osess.refresh()
        gsess.tokens.copy_(torch.from_numpy(osess.tokens.astype(np.int32)))
        if b == 0:
            gsess.prefill()
        else:
            gsess.refresh(b)
        g = gsess.staleness(b)
        for key in ("k_mean", "k_min", "v_mean", "v_min"):
            np.testing.assert_allclose(g[key], 1.0, atol=1e-6)
        for _ in range(2):
            if osess.block_done(b):
                break
            osess.step(b)
            gsess.tokens.copy_(torch.from_numpy(osess.tokens.astype(np.int32)))
            ost, oratio = osess.staleness(b)
            g = gsess.staleness(b)
            assert g["reuse"] == pytest.approx(oratio, abs=1e-12)
            for j, kv in enumerate("kv"):
                np.testing.assert_allclose(g[kv + "_mean"][0], 1.0, atol=1e-6)
                np.testing.assert_allclose(g[kv + "_min"][0], 1.0, atol=1e-6)
                for i, stat in enumerate(("_mean", "_min")):
                    got = g[kv + stat].astype(np.float64)
                    ref = ost[:, j, i]
                    err = np.abs(got - ref)
                    worst = max(worst, float(err.max()))
                    assert np.all(err <= staleness_tol(ref, r)), (b, kv + stat, got, ref)
        while not osess.block_done(b):
            osess.step(b)
    print(f"worst staleness difference {worst:.2e}")


@pytest.mark.parametrize("kind,mode", [("fp32", "dual"), ("bf16", "dual"), ("bf16", "prefix")])
def test_debug_mode_poisoned_buffers_and_guard_bands(lib, kind, mode):
    """Debug sessions start with a NaN-poisoned KV cache and workspace framed by canary
    guard bands.  A whole generation gives the same tokens as a normal session (no kernel
    reads a byte it has not written first), every guard band is intact afterwards, the
    cache padding past the last position is still the poison (never written), and a
    guard band that is overwritten is reported."""
    if kind == "fp32":
        wl = replace(synth.WORKLOADS["tiny_dual"], cache_mode=mode)
    else:
        wl = small_bf16(Hq=2, Hkv=1, mode=mode, B=2, K=16, P=40)
    model = gpu_model(lib, wl)
    prompt = synth.make_prompt(wl)
    want, st_w = Session(model, prompt, wl.gen_len, wl.block_len, wl.threshold, mode).generate()
    s = Session(model, prompt, wl.gen_len, wl.block_len, wl.threshold, mode, debug=True)
    got, st_g = s.generate()
    s.check_guards()
    assert np.array_equal(got, want) and st_g["steps_per_block"] == st_w["steps_per_block"]
    # layer 0 K of sequence 0, KV head 0: positions [S, Sp) were never written
    m = wl.model
    esz = 4 if m.dtype == "f32" else 2
    S, Sp = wl.seq_len, (wl.seq_len + 63) // 64 * 64
    k0 = s.cache[: Sp * m.head_dim * esz].cpu().numpy().view(np.uint8)
    pad = k0[S * m.head_dim * esz:]
    assert pad.size > 0 and np.all(pad == 0xFF)
    # a write into a guard band is caught
    full, g, n4 = s._guarded["workspace"]
    full[g + n4 + 5] = 0
    with pytest.raises(RuntimeError, match="workspace: guard band after"):
        s.check_guards()


def test_prefix_mode_empty_prompt_every_step_equals_full_forward(lib):
    """With an empty prompt, a prefix-mode step of block 0 recomputes every position, so
    each of its cached steps (not only the first after the prefill) must give the no-cache
    full forward's logits (ccyt168.com Fast-dLLM article, section 1.1: the prefix cache
    keeps only what precedes the block).  fp32 model at 1e-4, teacher-forced along the
    oracle's trajectory, one token per step (tau > 1) so the block takes 8 steps."""
    wl = replace(synth.WORKLOADS["tiny_dual"], prompt_len=0, gen_len=24, cache_mode="prefix",
                 threshold=1.5)
    m = wl.model
    M = om.OracleModel(wl)
    prompt = np.zeros((wl.batch, 0), dtype=np.int64)
    osess = OSession(M, prompt, wl.gen_len, wl.block_len, wl.threshold, "prefix")
    gsess = Session(gpu_model(lib, wl), prompt, wl.gen_len, wl.block_len, wl.threshold, "prefix")
    osess.refresh()
    gsess.prefill()
    n = 0
    while not osess.block_done(0):
        s0, s1 = osess.block_span(0)
        gsess.tokens.copy_(torch.from_numpy(osess.tokens.astype(np.int32)))
        _, ref = om.full_forward(M, osess.tokens, logit_rows=slice(s0, s1))
        g = gsess.step(0)
        torch.cuda.synchronize()
        got = g["logits"].cpu().numpy().reshape(ref.shape).astype(np.float64)
        assert rel_inf(got, ref) < 1e-4, f"step {n + 1}"
        grade_confidence_stage(got.reshape(-1, m.vocab), g["conf"].cpu().numpy(),
                               g["argmax"].cpu().numpy(), m.mask_id)
        osess.step(0)
        n += 1
    assert n == wl.block_len


@pytest.mark.parametrize("l_star,Hkv", [(0, 4), (1, 4), (1, 2)])
def test_dualcache_one_mixing_layer_every_step_equals_full_forward(lib, l_star, Hkv):
    """DualCache keeps every position outside the block at the K/V of the last refresh
    (ccyt168.com Fast-dLLM article, section 1.1; techwalker.com explainer, "Core
    innovation").  With the output projection of every layer but l* zeroed, layers 0..l*
    see each position's own token alone, so the cached K/V at l* equal fresh ones and the
    later layers never use theirs: every cached step of every block must give the no-cache
    full forward's logits.  fp32 at 1e-4 against the oracle's full forward (not its cached
    step), teacher-forced, one token per step (tau > 1)."""
    wl = replace(synth.WORKLOADS["tiny_dual"], threshold=1.5)
    wl = replace(wl, model=replace(wl.model, n_kv_heads=Hkv))
    m = wl.model
    W = synth.make_weights(wl)
    for l in range(m.n_layers):
        if l != l_star:
            W[f"w_o.{l}"] = np.zeros_like(W[f"w_o.{l}"])
    M = om.OracleModel(wl, weights=W)
    prompt = synth.make_prompt(wl)
    osess = OSession(M, prompt, wl.gen_len, wl.block_len, wl.threshold, "dual")
    gsess = Session(Model.from_host(lib, m, W), prompt, wl.gen_len, wl.block_len,
                    wl.threshold, "dual")
    n = 0
    for b in range(osess.n_blocks):
        osess.refresh()
        if b == 0:
            gsess.prefill()
        else:
            gsess.refresh(b)
        while not osess.block_done(b):
            s0, s1 = osess.block_span(b)
            gsess.tokens.copy_(torch.from_numpy(osess.tokens.astype(np.int32)))
            _, ref = om.full_forward(M, osess.tokens, logit_rows=slice(s0, s1))
            g = gsess.step(b)
            torch.cuda.synchronize()
            got = g["logits"].cpu().numpy().reshape(ref.shape).astype(np.float64)
            assert rel_inf(got, ref) < 1e-4, f"block {b} step {n}"
            osess.step(b)
            n += 1
    assert n == wl.gen_len


@pytest.mark.parametrize("kind", ["fp32", "bf16"])
def test_teacher_forced_largest_block(lib, kind):
    """Blocks of 64 positions, the largest the library takes (one wave ballot per block):
    teacher-forced parity with every step graded per stage."""
    if kind == "fp32":
        wl = replace(synth.WORKLOADS["tiny_dual"], gen_len=128, block_len=64, threshold=0.7)
        st = teacher_forced(lib, wl, 1e-4, CONF_TOL_F32)
    else:
        wl = small_bf16(Hq=2, Hkv=1, mode="dual", B=2, P=40, G=128, K=64)
        st = teacher_forced(lib, wl, 2e-2)
    assert st["steps"] >= 2
