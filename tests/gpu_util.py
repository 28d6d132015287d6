"""Helpers shared by the GPU tests: host <-> device conversion and the comparison
protocol for decisions taken from floating-point confidences."""
import numpy as np

import synth
from oracle import decode

# Bound on |GPU confidence - oracle confidence| for the fp32 (tiny) model, asserted by the
# fp32 teacher-forced and refresh-step tests and relied on by the free-running ones: the
# fp32 logits agree to about 1e-6 relative (|logit| < ~20), so a confidence c moves by at
# most c (exp(2 dl) - 1) ~ 4e-5 c, plus the fp32 rounding of the exp-sum.
CONF_TOL_F32 = 2e-5


def dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).view(torch.bfloat16).to(device)


def dev_f32(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 decoded exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_fp32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_inf(got, ref) -> float:
    """max |got - ref| / max |ref| (per whole array)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


MARGIN = 1e-3


def decision_margin_ok(conf, tau, masked, margin=MARGIN):
    """Per sequence: True where the threshold decisions are not within ``margin`` of a
    flip: every masked confidence is > margin away from tau, and if the forced-pick
    path is taken, the top masked confidence leads the runner-up by > margin."""
    conf = np.asarray(conf, np.float64)
    ok = np.ones(conf.shape[0], bool)
    for b in range(conf.shape[0]):
        c = conf[b][masked[b]]
        if c.size == 0:
            continue
        if np.any(np.abs(c - tau) <= margin):
            ok[b] = False
            continue
        if not np.any(c >= tau) and c.size > 1:
            s = np.sort(c)[::-1]
            if s[0] - s[1] <= margin:
                ok[b] = False
    return ok


def top2_gap(logits_row: np.ndarray, mask_id: int) -> float:
    """Probability gap between the top two tokens of a row (mask excluded)."""
    z = np.array(logits_row, np.float64)
    z[mask_id] = -np.inf
    p = np.exp(z - z.max())
    p /= p.sum()
    s = np.sort(p)[::-1]
    return float(s[0] - s[1])


def safe_sequences(conf_ref, conf_unc, tau, masked):
    """Per sequence: True where no threshold decision or forced pick can flip given an
    absolute confidence uncertainty ``conf_unc`` per position ([B, K] or scalar)."""
    conf = np.asarray(conf_ref, np.float64)
    unc = np.broadcast_to(np.asarray(conf_unc, np.float64), conf.shape)
    ok = np.ones(conf.shape[0], bool)
    for b in range(conf.shape[0]):
        m = masked[b]
        c, u = conf[b][m], unc[b][m]
        if c.size == 0:
            continue
        if np.any(np.abs(c - tau) <= u):
            ok[b] = False
            continue
        if not np.any(c >= tau) and c.size > 1:
            order = np.argsort(-c, kind="stable")
            if c[order[0]] - c[order[1]] <= u[order[0]] + u[order[1]]:
                ok[b] = False
    return ok


def grade_confidence_stage(logits_rows, gconf, garg, mask_id, rel=2e-5):
    """Per-stage grading of the confidence pass (max softmax probability, argmax with the
    mask id excluded): the oracle's definition applied to the very logits the GPU
    produced.  The maximum of identical fp32 values is exact, so the argmax (lowest id on
    ties) must match on every row; the confidence differs only by the fp32 rounding of
    the exp-sum.  Returns the largest relative confidence difference."""
    rc, ra = decode.confidence_argmax(np.asarray(logits_rows, np.float64), mask_id)
    garg = np.asarray(garg).reshape(-1)
    gconf = np.asarray(gconf, np.float64).reshape(-1)
    assert np.array_equal(garg, ra), f"argmax differs on rows {np.nonzero(garg != ra)[0][:8]}"
    d = float(np.max(np.abs(gconf - rc) / rc))
    assert d < rel, f"confidence rel diff {d}"
    return d


def grade_unmask_stage(before, gconf, garg, gtok, gnun, grem, mask_id, tau, gidx=None):
    """Per-stage grading of the threshold unmask: the oracle's rule applied to the GPU's
    own confidences and argmaxes must give the GPU's tokens, unmask counts and masks left
    bit for bit on every sequence (pure compare-and-index work; the threshold is compared
    in fp32 on both sides, as the kernel does).  Returns the unmask set U [B, K]."""
    before = np.asarray(before)
    B, K = before.shape
    tau32 = float(np.float32(tau))
    conf = np.asarray(gconf, np.float32).astype(np.float64).reshape(B, K)
    arg = np.asarray(garg).reshape(B, K)
    want, U, wn, wr = decode.unmask(before, conf, arg, mask_id, tau32)
    assert np.array_equal(np.asarray(gtok).reshape(B, K), want), "tokens differ"
    assert np.array_equal(np.asarray(gnun).reshape(B), wn), "n_unmasked differs"
    assert np.array_equal(np.asarray(grem).reshape(B), wr), "remaining differs"
    if gidx is not None:
        gidx = np.asarray(gidx).reshape(B, K)
        for b in range(B):
            sel = np.nonzero(U[b])[0]
            assert np.array_equal(gidx[b, :len(sel)], sel), f"unmasked_idx of sequence {b}"
            assert np.all(gidx[b, len(sel):] == -1)
    return U
