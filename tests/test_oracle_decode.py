"""Pins for oracle/decode.py, oracle/generate.py and oracle/theorem.py."""
import itertools

import numpy as np
import pytest
import torch

import synth
from oracle import decode, theorem
from oracle import model as om
from oracle.generate import Session, generate


# ------------------------------------------------------------------ confidence

def test_confidence_matches_torch_softmax_and_first_argmax():
    r = np.random.default_rng(0)
    z = r.standard_normal((50, 300)) * 3
    z[3, 17] = z[3, 40] = z[3].max() + 1.0          # a tie: lowest id wins
    mask = 299
    conf, arg = decode.confidence_argmax(z, mask)
    zt = torch.from_numpy(z.copy())
    zt[:, mask] = -float("inf")
    p = torch.softmax(zt, dim=1)
    np.testing.assert_allclose(conf, p.max(dim=1).values.numpy(), rtol=1e-13)
    zz = z.copy()
    zz[:, mask] = -np.inf
    np.testing.assert_array_equal(arg, np.argmax(zz, axis=1))
    assert arg[3] == 17


def test_confidence_uniform_rows_and_mask_exclusion():
    V = 64
    z = np.zeros((2, V))
    z[1, V - 1] = 100.0                              # the mask id has the largest logit
    conf, arg = decode.confidence_argmax(z, V - 1)
    np.testing.assert_allclose(conf, [1.0 / (V - 1)] * 2, rtol=1e-15)
    assert list(arg) == [0, 0]


def test_confidence_two_value_closed_form():
    # one logit a above V-2 others equal to 0 (mask excluded): conf = e^a / (e^a + V - 2)
    V, a = 10, 2.5
    z = np.zeros((1, V))
    z[0, 4] = a
    conf, arg = decode.confidence_argmax(z, V - 1)
    assert arg[0] == 4
    assert abs(conf[0] - np.exp(a) / (np.exp(a) + V - 2)) < 1e-15


# ------------------------------------------------------------------ unmask rule

def brute_force_unmask(tok, conf, tau, mask_id):
    """The decoded set by enumeration: the largest subset S of masked positions such
    that every member reaches tau, or -- if that set is empty -- the singleton of
    the most confident masked position (lowest on ties)."""
    K = len(tok)
    masked = [i for i in range(K) if tok[i] == mask_id]
    best = ()
    for r in range(K + 1):
        for S in itertools.combinations(range(K), r):
            if all(i in masked and conf[i] >= tau for i in S) and len(S) > len(best):
                best = S
    if not best and masked:
        top = max(conf[i] for i in masked)
        best = (min(i for i in masked if conf[i] == top),)
    return set(best)


@pytest.mark.parametrize("K", [1, 3, 8])
def test_unmask_matches_brute_force(K):
    r = np.random.default_rng(K)
    mask_id = 9
    for trial in range(300):
        tok = np.where(r.random(K) < 0.7, mask_id, r.integers(0, 9, K))
        conf = np.round(r.random(K), 1)             # coarse values -> ties happen
        tau = float(r.choice([0.0, 0.5, 0.9, 1.0, 1.5]))
        arg = r.integers(0, 9, K)
        new, U, n, rem = decode.unmask(tok[None], conf[None], arg[None], mask_id, tau)
        want = brute_force_unmask(tok, conf, tau, mask_id)
        assert set(np.nonzero(U[0])[0]) == want
        assert n[0] == len(want)
        assert rem[0] == int((tok == mask_id).sum()) - len(want)
        for i in range(K):
            assert new[0, i] == (arg[i] if i in want else tok[i])


def test_unmask_monotone_in_tau():
    r = np.random.default_rng(1)
    tok = np.full((4, 16), 7)
    conf = r.random((4, 16))
    arg = r.integers(0, 7, (4, 16))
    prev = None
    for tau in np.linspace(0, 1, 21):
        _, U, _, _ = decode.unmask(tok, conf, arg, 7, tau)
        if prev is not None:
            assert np.all(U <= prev) or U.sum(axis=1).min() == 1
        prev = U


def test_idle_sequence_gets_no_forced_unmask():
    tok = np.array([[5, 5, 5], [9, 9, 5]])
    conf = np.array([[0.1, 0.2, 0.3], [0.1, 0.2, 0.3]])
    new, U, n, rem = decode.unmask(tok, conf, np.array([[1, 1, 1], [2, 3, 4]]), 9, 0.9)
    assert list(n) == [0, 1] and list(rem) == [0, 1]
    assert list(new[1]) == [9, 3, 5]


# ------------------------------------------------------------------ generation loop

def tiny(tau_scale=None):
    return synth.WORKLOADS["tiny_dual"]


def test_tiny_config_confidence_spread():
    """The tiny config's x8 logit scale spreads confidences over about 0.2-1.0."""
    wl = tiny()
    M = om.OracleModel(wl)
    seen = []
    s = Session(M, synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, "dual")
    s.generate(on_step=lambda b, n, out: seen.append(out["conf"][0]))
    c = np.concatenate(seen)
    assert c.min() < 0.35 and c.max() > 0.95


@pytest.mark.parametrize("mode", ["dual", "prefix"])
def test_generation_progress_bounds(mode):
    """Property (c): each step decodes >= 1 token, so a block takes <= K steps."""
    wl = tiny()
    M = om.OracleModel(wl)
    seen = []
    s = Session(M, synth.make_prompt(wl), wl.gen_len, wl.block_len, 0.9, mode)
    toks, st = s.generate(on_step=lambda b, n, out: seen.append(int(out["n_unmasked"].min())))
    assert min(seen) >= 1
    assert all(1 <= n <= wl.block_len for n in st["steps_per_block"])
    assert wl.gen_len // wl.block_len <= st["steps"] <= wl.gen_len
    assert not (toks == wl.model.mask_id).any()
    assert toks.min() >= 0 and toks.max() < wl.model.vocab - 1


def test_tau_above_one_decodes_one_token_per_step_in_confidence_order():
    wl = tiny()
    M = om.OracleModel(wl)
    s = Session(M, synth.make_prompt(wl), wl.gen_len, wl.block_len, 1.5, "dual")

    def rec(b, n, out):
        s0, s1 = s.block_span(b)
        assert out["n_unmasked"][0] == 1
        U = out["U"][0]
        masked_before = (s.tokens[0, s0:s1] == wl.model.mask_id) | U
        i = int(np.nonzero(U)[0][0])
        c = np.where(masked_before, out["conf"][0], -np.inf)
        assert i == int(np.argmax(c))
    toks, st = s.generate(on_step=rec)
    assert st["steps"] == wl.gen_len


def test_tau_zero_decodes_a_block_per_step():
    wl = tiny()
    toks, st = generate(om.OracleModel(wl), synth.make_prompt(wl), wl.gen_len, wl.block_len,
                        0.0, "dual")
    assert st["steps"] == wl.gen_len // wl.block_len


def test_resume_from_block_boundary_is_identical():
    wl = tiny()
    M = om.OracleModel(wl)
    prompt = synth.make_prompt(wl)
    full, _ = generate(M, prompt, wl.gen_len, wl.block_len, 0.9, "dual")
    s = Session(M, prompt, wl.gen_len, wl.block_len, 0.9, "dual")
    for b in range(2):                               # run two blocks, then "crash"
        s.refresh()
        while not s.block_done(b):
            s.step(b)
    saved = s.tokens.copy()
    r = Session(M, prompt, wl.gen_len, wl.block_len, 0.9, "dual")
    r.tokens[...] = saved                            # resume state = tokens + block cursor
    for b in range(2, r.n_blocks):
        r.refresh()
        while not r.block_done(b):
            r.step(b)
    np.testing.assert_array_equal(r.tokens[:, r.P:], full)


# ------------------------------------------------------------------ theorem (b)

def peaked_joint(r, n, V):
    p = r.random((V,) * n) ** 3
    p /= p.sum()
    w = r.uniform(0.5, 1.0)
    star = tuple(r.integers(0, V, n))
    p *= (1 - w)
    p[star] += w
    return p


def test_theorem_parallel_equals_sequential_greedy():
    r = np.random.default_rng(42)
    held = 0
    for trial in range(20000):
        n = int(r.integers(1, 5))
        V = int(r.integers(2, 5))
        p = peaked_joint(r, n, V)
        ok, eps = theorem.condition_holds(p)
        if not ok:
            continue
        held += 1
        # the threshold rule at tau = 1 - eps selects all n positions and decodes their
        # marginal argmaxes
        mg = theorem.marginals(p)
        conf = np.array([[m.max() for m in mg]])
        arg = np.array([[int(np.argmax(m)) for m in mg]])
        tok, U, cnt, _ = decode.unmask(np.full((1, n), V), conf, arg, V, 1.0 - eps)
        assert cnt[0] == n
        par = tuple(int(t) for t in tok[0])
        assert par == theorem.parallel_greedy(p) == theorem.joint_mode(p)
        for order in theorem.all_orders(n):
            assert theorem.sequential_greedy(p, order) == par
    assert held > 2000


def test_theorem_bound_has_teeth():
    # p(A,A) = .25, p(A,B) = p(B,A) = .375: marginals are 0.625 (eps = .375,
    # (n+1) eps = 1.125 > 1); parallel decoding gives (A,A), sequential gives (A,B).
    p = np.array([[0.25, 0.375], [0.375, 0.0]])
    ok, eps = theorem.condition_holds(p)
    assert not ok
    assert theorem.parallel_greedy(p) == (0, 0)
    assert theorem.sequential_greedy(p) == (0, 1)
    assert theorem.joint_mode(p) in [(0, 1), (1, 0)]


# ------------------------------------------------------------------ calibration

def test_calibration_hits_the_requested_fraction():
    from oracle import calibrate
    r = np.random.default_rng(3)
    z = r.standard_normal((400, 500))
    mask = 499
    s = calibrate.calibrate_from_logits(z, mask, 0.9, 0.3)
    conf, _ = decode.confidence_argmax(z * s, mask)
    frac = (conf >= 0.9 - 1e-9).mean()
    assert abs(frac - 0.3) < 0.01
