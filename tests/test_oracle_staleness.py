"""Pins for the oracle's cache-staleness measure (oracle/generate.py: cosine,
kv_cosine_stats, Session.reused_positions, Session.staleness): closed forms, a library
routine, hand-built caches and the invariants of the block cache."""
from dataclasses import replace

import numpy as np
import pytest
from scipy.spatial import distance

import synth
from oracle import model as om
from oracle.generate import Session, cosine, kv_cosine_stats


def small_workload(mode="dual"):
    m = synth.ModelShape(n_layers=2, d_model=32, n_heads=4, n_kv_heads=2, head_dim=8,
                         d_ffn=48, vocab=40, logit_scale=4.0, dtype="f32")
    return synth.Workload("small", m, batch=2, prompt_len=6, gen_len=8, block_len=4,
                          cache_mode=mode, norm_gain_std=0.1)


def test_cosine_closed_forms():
    th = np.linspace(0.0, np.pi, 7)
    a = np.stack([np.ones_like(th), np.zeros_like(th)], axis=-1)
    b = np.stack([np.cos(th), np.sin(th)], axis=-1) * 2.5       # length does not matter
    np.testing.assert_allclose(cosine(a, b), np.cos(th), atol=1e-15)
    v = np.array([0.3, -1.2, 4.0, 0.0])
    assert cosine(v, 7.0 * v) == pytest.approx(1.0, abs=1e-15)
    assert cosine(v, -v) == pytest.approx(-1.0, abs=1e-15)
    assert cosine(np.array([1.0, 0, 0]), np.array([0, 0, 3.0])) == 0.0
    z = np.zeros(4)
    assert cosine(z, z) == 1.0 and cosine(z, v) == 0.0 and cosine(v, z) == 0.0


def test_cosine_matches_scipy():
    r = np.random.default_rng(3)
    a, b = r.normal(size=(50, 16)), r.normal(size=(50, 16))
    ref = np.array([1.0 - distance.cosine(x, y) for x, y in zip(a, b)])
    np.testing.assert_allclose(cosine(a, b), ref, atol=1e-14)


def test_stats_on_a_hand_built_cache():
    """One vector of one layer's V turned by 60 degrees: the mean moves by (1 - 1/2)/N
    over the N compared vectors, the minimum is 1/2; K and the other layer stay at 1."""
    L, B, H, S, D = 2, 2, 3, 5, 4
    r = np.random.default_rng(1)
    fresh = om.KVCache(L, B, H, S, D, np.float64)
    for l in range(L):
        fresh.K[l][...] = r.normal(size=(B, H, S, D))
        fresh.V[l][...] = r.normal(size=(B, H, S, D))
    cached = om.KVCache(L, B, H, S, D, np.float64)
    for l in range(L):
        cached.K[l][...] = 2.0 * fresh.K[l]
        cached.V[l][...] = fresh.V[l]
    u = np.zeros(D)
    u[0] = 1.0
    w = np.zeros(D)
    w[1] = 1.0
    fresh.V[1][1, 2, 3] = u
    cached.V[1][1, 2, 3] = 0.5 * u + np.sqrt(3) / 2 * w
    keep = np.ones(S, dtype=bool)
    st = kv_cosine_stats(cached, fresh, keep)
    n = B * H * S
    np.testing.assert_allclose(st[0], 1.0, atol=1e-14)
    np.testing.assert_allclose(st[1, 0], 1.0, atol=1e-14)
    assert st[1, 1, 0] == pytest.approx(1.0 - 0.5 / n, abs=1e-14)
    assert st[1, 1, 1] == pytest.approx(0.5, abs=1e-14)
    keep[3] = False                                  # the turned position is not compared
    np.testing.assert_allclose(kv_cosine_stats(cached, fresh, keep), 1.0, atol=1e-14)
    np.testing.assert_array_equal(kv_cosine_stats(cached, fresh, np.zeros(S, bool)), 1.0)


@pytest.mark.parametrize("mode", ["dual", "prefix"])
def test_reused_positions_and_ratio(mode):
    wl = small_workload(mode)
    s = Session(om.OracleModel(wl), synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, mode)
    # S = 14, blocks [6, 10) and [10, 14)
    want0 = [1] * 6 + [0] * 4 + ([1] * 4 if mode == "dual" else [0] * 4)
    want1 = [1] * 10 + [0] * 4
    np.testing.assert_array_equal(s.reused_positions(0), np.array(want0, bool))
    np.testing.assert_array_equal(s.reused_positions(1), np.array(want1, bool))
    s.refresh()
    _, ratio = s.staleness(0)
    assert ratio == pytest.approx((10 if mode == "dual" else 6) / 14)


@pytest.mark.parametrize("mode", ["dual", "prefix"])
def test_fresh_after_refresh_stale_after_steps(mode):
    """Right after a refresh the cache is exact (every cosine 1).  Once steps change the
    block's tokens, layer 0 of the reused positions is still exact (its K/V depend only
    on the position's own token) while deeper layers have moved; block positions, whose
    layer-0 K/V do change, are not part of the comparison."""
    wl = small_workload(mode)
    M = om.OracleModel(wl)
    s = Session(M, synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, mode)
    for b in range(s.n_blocks):
        s.refresh()
        st, _ = s.staleness(b)
        np.testing.assert_allclose(st, 1.0, atol=1e-12)
        s.step(b)
        st, _ = s.staleness(b)
        np.testing.assert_allclose(st[0], 1.0, atol=1e-12)
        assert st[1, :, 1].max() < 1.0 - 1e-9 and st[1, :, 0].max() < 1.0 - 1e-10
        assert np.all(st[:, :, 1] <= st[:, :, 0] + 1e-15)
        while not s.block_done(b):
            s.step(b)


def test_staleness_leaves_the_session_untouched():
    wl = small_workload()
    s = Session(om.OracleModel(wl), synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, "dual")
    s.refresh()
    s.step(0)
    tok, k1 = s.tokens.copy(), s.cache.K[1].copy()
    s.staleness(0)
    np.testing.assert_array_equal(s.tokens, tok)
    np.testing.assert_array_equal(s.cache.K[1], k1)
