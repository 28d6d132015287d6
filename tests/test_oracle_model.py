"""Pins for oracle/model.py: library routines, closed forms and the cache invariants."""
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import model as om
from oracle.generate import Session, generate_nocache

torch.set_default_dtype(torch.float64)


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ building blocks

def test_rmsnorm_matches_torch():
    x = rng(0).standard_normal((5, 7, 64))
    g = rng(1).standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(om.rmsnorm(x, g, 1e-5), ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2), (4, 1)])
def test_attention_matches_sdpa_noncausal(Hq, Hkv):
    r = rng(2)
    q = r.standard_normal((2, Hq, 5, 16))
    k = r.standard_normal((2, Hkv, 11, 16))
    v = r.standard_normal((2, Hkv, 11, 16))
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=False).numpy()
    np.testing.assert_allclose(om.attention(q, k, v), ref, rtol=1e-12, atol=1e-12)


def test_silu_matches_torch():
    x = rng(3).standard_normal(1000) * 10
    np.testing.assert_allclose(om.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14)


def test_rope_closed_forms():
    D, S = 16, 40
    x = rng(4).standard_normal((3, S, D))
    cos, sin = om.rope_cos_sin(np.arange(S), D, 10000.0)
    y = om.apply_rope(x, cos, sin)
    # position 0 is the identity
    np.testing.assert_allclose(y[:, 0], x[:, 0], rtol=0, atol=0)
    # each (i, i + D/2) pair is rotated: norms are preserved
    h = D // 2
    np.testing.assert_allclose(x[..., :h] ** 2 + x[..., h:] ** 2,
                               y[..., :h] ** 2 + y[..., h:] ** 2, rtol=1e-12)
    # complex form: (a + ib) * exp(i pos theta^(-2j/D))
    ang = np.arange(S)[:, None] * 10000.0 ** (-2.0 * np.arange(h) / D)
    c = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * ang)
    np.testing.assert_allclose(np.concatenate([c.real, c.imag], -1), y, rtol=1e-12, atol=1e-12)
    # relative position: <rope(q, m), rope(k, n)> depends only on m - n
    q, k = rng(5).standard_normal(D), rng(6).standard_normal(D)

    def dot(m, n):
        cm, sm = om.rope_cos_sin(np.array([m]), D, 10000.0)
        cn, sn = om.rope_cos_sin(np.array([n]), D, 10000.0)
        return float(om.apply_rope(q[None], cm, sm)[0] @ om.apply_rope(k[None], cn, sn)[0])
    assert abs(dot(7, 3) - dot(24, 20)) < 1e-12
    assert abs(dot(7, 3) - dot(3, 7)) > 1e-6


def test_round_bf16_matches_torch():
    x = rng(7).standard_normal(10000) * 100
    ref = torch.from_numpy(x).float().to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(om.round_bf16(x), ref)


# ------------------------------------------------------------------ full forward

def torch_full_forward(wl, W, tokens, bf16):
    """Independent float64 torch composition of the same architecture."""
    m = wl.model
    T = lambda a: torch.from_numpy(synth.as_float(a, m.dtype).astype(np.float64))
    rs = (lambda t: t.float().bfloat16().double()) if bf16 else (lambda t: t)
    rf = (lambda t: t.float().double()) if bf16 else (lambda t: t)
    tok = torch.from_numpy(np.asarray(tokens))
    B, S = tok.shape
    D, Hq, Hkv = m.head_dim, m.n_heads, m.n_kv_heads
    x = T(W["embed"])[tok]
    ang = torch.arange(S, dtype=torch.float64)[:, None] * \
        m.rope_theta ** (-2.0 * torch.arange(D // 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones_like(ang), ang)

    def rope(t):  # t [B,H,S,D]
        c = torch.complex(t[..., :D // 2], t[..., D // 2:]) * rot
        return torch.cat([c.real, c.imag], -1)
    ks, vs = [], []
    for l in range(m.n_layers):
        h = rs(F.rms_norm(x, (m.d_model,), T(W[f"attn_norm.{l}"]), eps=m.norm_eps))
        qkv = h @ T(W[f"w_qkv.{l}"]).T
        q, k, v = torch.split(qkv, [Hq * D, Hkv * D, Hkv * D], dim=-1)
        q = rs(rope(q.view(B, S, Hq, D).transpose(1, 2)))
        k = rs(rope(k.view(B, S, Hkv, D).transpose(1, 2)))
        v = rs(v.view(B, S, Hkv, D).transpose(1, 2))
        ks.append(k.numpy())
        vs.append(v.numpy())
        o = F.scaled_dot_product_attention(q, k.repeat_interleave(Hq // Hkv, 1),
                                           v.repeat_interleave(Hq // Hkv, 1))
        o = rs(o).transpose(1, 2).reshape(B, S, Hq * D)
        x = rf(x + o @ T(W[f"w_o.{l}"]).T)
        h = rs(F.rms_norm(x, (m.d_model,), T(W[f"ffn_norm.{l}"]), eps=m.norm_eps))
        g, u = torch.split(h @ T(W[f"w_gate_up.{l}"]).T, [m.d_ffn, m.d_ffn], dim=-1)
        x = rf(x + rs(F.silu(g) * u) @ T(W[f"w_down.{l}"]).T)
    h = rs(F.rms_norm(x, (m.d_model,), T(W["final_norm"]), eps=m.norm_eps))
    logits = rf(m.logit_scale * (h @ T(W["lm_head"]).T))
    return ks, vs, logits.numpy()


def small_workload(dtype="f32", Hq=4, Hkv=4, gain=0.1):
    m = synth.ModelShape(n_layers=2, d_model=32, n_heads=Hq, n_kv_heads=Hkv, head_dim=8,
                         d_ffn=48, vocab=40, logit_scale=4.0, dtype=dtype)
    return synth.Workload("small", m, batch=2, prompt_len=6, gen_len=8, block_len=4,
                          cache_mode="dual", norm_gain_std=gain)


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f32", 4, 4), ("f32", 4, 2), ("bf16", 4, 2)])
def test_full_forward_matches_torch_composition(dtype, Hq, Hkv):
    wl = small_workload(dtype, Hq, Hkv)
    W = synth.make_weights(wl)
    M = om.OracleModel(wl, weights=W)
    tokens = synth.uniform_ints(9, 9, 2 * 14, wl.model.vocab).reshape(2, 14)
    cache, logits = om.full_forward(M, tokens)
    ks, vs, ref = torch_full_forward(wl, W, tokens, dtype == "bf16")
    tol = 1e-12 if dtype == "f32" else 1e-6
    np.testing.assert_allclose(logits, ref, rtol=tol, atol=tol)
    for l in range(wl.model.n_layers):
        np.testing.assert_allclose(cache.K[l], ks[l], rtol=tol, atol=tol)
        np.testing.assert_allclose(cache.V[l], vs[l], rtol=tol, atol=tol)


def test_full_forward_without_logits_skips_only_the_tail():
    wl = small_workload()
    M = om.OracleModel(wl)
    tokens = synth.uniform_ints(3, 3, 28, wl.model.vocab).reshape(2, 14)
    c1, _ = om.full_forward(M, tokens)
    c2, lg = om.full_forward(M, tokens, logit_rows=None)
    assert lg is None
    for l in range(wl.model.n_layers):
        np.testing.assert_array_equal(c1.K[l], c2.K[l])
        np.testing.assert_array_equal(c1.V[l], c2.V[l])


# ------------------------------------------------------------------ cache invariants

@pytest.mark.parametrize("mode", ["dual", "prefix"])
def test_first_cached_step_equals_full_forward(mode):
    """Property (a): with a cache refreshed at the block boundary, the first step's
    block logits equal the no-cache bidirectional forward."""
    wl = replace(small_workload(), cache_mode=mode)
    M = om.OracleModel(wl)
    s = Session(M, synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, mode)
    for b in range(s.n_blocks):
        s.refresh()
        s0, s1 = s.block_span(b)
        _, ref = om.full_forward(M, s.tokens, logit_rows=slice(s0, s1))
        got = om.cached_step(M, s.tokens, s.cache, s0, s1, mode)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)
        while not s.block_done(b):
            s.step(b)


def test_prefix_and_dual_agree_on_first_step_of_every_block():
    wl = small_workload()
    M = om.OracleModel(wl)
    s = Session(M, synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, "dual")
    for b in range(s.n_blocks):
        s.refresh()
        s0, s1 = s.block_span(b)
        import copy
        c2 = copy.deepcopy(s.cache)
        a = om.cached_step(M, s.tokens, s.cache, s0, s1, "dual")
        p = om.cached_step(M, s.tokens, c2, s0, s1, "prefix")
        np.testing.assert_allclose(a, p, rtol=1e-11, atol=1e-11)
        while not s.block_done(b):
            s.step(b)


def test_layer0_kv_of_unchanged_tokens_equal_fresh_values():
    wl = small_workload()
    M = om.OracleModel(wl)
    s = Session(M, synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, "dual")
    s.refresh()
    s.step(0)
    before = s.tokens.copy()
    s.step(0)                     # writes block K/V computed from ``before``
    fresh, _ = om.full_forward(M, before, logit_rows=None)
    # layer 0 K/V depend only on the token and the position: every position (the stale
    # prefix/suffix included) equals a fresh forward of the tokens the step saw
    np.testing.assert_allclose(s.cache.K[0], fresh.K[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s.cache.V[0], fresh.V[0], rtol=1e-13, atol=1e-13)
    # later layers of the prefix/suffix are stale: they differ once the block changed
    assert not np.allclose(s.cache.K[1], fresh.K[1], rtol=1e-9, atol=1e-9)


def test_refresh_before_every_step_is_the_no_cache_algorithm():
    wl = small_workload()
    M = om.OracleModel(wl)
    prompt = synth.make_prompt(wl)
    ref, _ = generate_nocache(M, prompt, wl.gen_len, wl.block_len, 0.9)
    s = Session(M, prompt, wl.gen_len, wl.block_len, 0.9, "dual")
    for b in range(s.n_blocks):
        while not s.block_done(b):
            s.refresh()
            s.step(b)
    np.testing.assert_array_equal(s.tokens[:, s.P:], ref)


def test_prefix_mode_with_empty_prompt_is_the_full_forward_at_every_step():
    """Prefix-mode caching keeps only the positions before the block and recomputes the
    block together with everything after it on every step (ccyt168.com Fast-dLLM
    article, section 1.1: the prefix cache against DualCache, which also keeps the
    masked suffix; techwalker.com explainer, "Core innovation").  With an empty prompt
    and block 0, nothing comes from the cache at all, so every cached step of the block
    (not only the first) must equal the no-cache full forward of the current tokens.
    DualCache keeps the stale suffix K/V instead, so from the second step on its logits
    move away from the full forward.  A prefix step that recomputed only the block rows
    would behave like DualCache here and fail the first assertion."""
    wl = replace(small_workload(), prompt_len=0, gen_len=12, block_len=4, cache_mode="prefix")
    M = om.OracleModel(wl)
    prompt = np.zeros((wl.batch, 0), dtype=np.int64)
    # tau > 1: one token per step, so block 0 takes 4 steps
    s = Session(M, prompt, wl.gen_len, wl.block_len, 1.5, "prefix")
    d = Session(M, prompt, wl.gen_len, wl.block_len, 1.5, "dual")
    s.refresh()
    d.refresh()
    s0, s1 = s.block_span(0)
    assert (s0, s1) == (0, 4)
    n = 0
    while not s.block_done(0):
        n += 1
        d.tokens[...] = s.tokens           # both modes see the same token state
        _, ref = om.full_forward(M, s.tokens, logit_rows=slice(s0, s1))
        got_dual = om.cached_step(M, d.tokens, d.cache, s0, s1, "dual")
        out = s.step(0)
        np.testing.assert_allclose(out["logits"], ref, rtol=1e-11, atol=1e-11)
        dual_err = np.max(np.abs(got_dual - ref))
        if n == 1:
            assert dual_err < 1e-11           # property (a): both exact after a refresh
        else:
            assert dual_err > 1e-3, f"step {n}: DualCache should read a stale suffix"
    assert n == 4


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2)])
def test_dualcache_is_exact_when_only_one_layer_mixes_positions(Hq, Hkv):
    """DualCache keeps every position outside the block at the K/V of the last refresh
    and recomputes only the block rows (ccyt168.com Fast-dLLM article, section 1.1;
    techwalker.com explainer, "Core innovation").  The cached values go stale only
    because attention mixes positions: with the output projection of every layer but
    one (l*) set to zero, the inputs of layers 0..l* depend on each position's own token
    alone, so the K/V cached at layer l* equal fresh ones at every unchanged position,
    and the layers after l* (zero output projection) never use their cached K/V.  Every
    DualCache step of every block, later steps included, must then equal the no-cache
    full forward of the current tokens.  This pins the layer-l* cache read of the step
    for each l*: a step that skipped the masked suffix, kept the block's stale K/V, read
    another layer's cache or put the block at the wrong RoPE positions fails it.  With
    every projection kept, the steps after the first do differ (the stale cache)."""
    wl = replace(small_workload("f32", Hq, Hkv), prompt_len=5, gen_len=12, block_len=4)
    wl = replace(wl, model=replace(wl.model, n_layers=3))
    base = synth.make_weights(wl)
    prompt = synth.make_prompt(wl)
    L = wl.model.n_layers
    for l_star in list(range(L)) + [None]:
        W = dict(base)
        if l_star is not None:
            for l in range(L):
                if l != l_star:
                    W[f"w_o.{l}"] = np.zeros_like(base[f"w_o.{l}"])
        M = om.OracleModel(wl, weights=W)
        s = Session(M, prompt, wl.gen_len, wl.block_len, 1.5, "dual")  # one token per step
        worst_later = 0.0
        for b in range(wl.gen_len // wl.block_len):
            s.refresh()
            s0, s1 = s.block_span(b)
            n = 0
            while not s.block_done(b):
                n += 1
                _, ref = om.full_forward(M, s.tokens, logit_rows=slice(s0, s1))
                out = s.step(b)
                err = np.max(np.abs(out["logits"] - ref))
                if l_star is not None or n == 1:
                    assert err < 1e-11, f"l*={l_star} block {b} step {n}: {err}"
                else:
                    worst_later = max(worst_later, err)
            assert n == wl.block_len
        if l_star is None:
            assert worst_later > 1e-3, "the stale cache should show with every layer mixing"
