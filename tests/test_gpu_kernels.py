"""GPU parity of the single-stage kernels against the CPU oracle, through the C ABI.

Inputs are seeded and synthetic (``synth``); expected values come from the oracle only.
"""
import ctypes as C

import numpy as np
import pytest

import synth
from gpu_util import (dev_bf16, dev_f32, grade_confidence_stage, grade_unmask_stage, host,
                      rel_inf, safe_sequences)
from oracle import decode
from oracle import model as om

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from diffusion_dllm_block_amd import binding as bd  # noqa: E402


def stream():
    return bd.stream_handle()


# ------------------------------------------------------------------ synthetic fill

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode,std", [(0, 0.03125), (0, 1.0), (1, 0.1), (2, 1.0)])
def test_device_generator_is_bit_identical_to_host(lib, dtype, mode, std):
    n = 1_000_003
    dt = bd.F32 if dtype == "f32" else bd.BF16
    t = torch.empty(n, dtype=torch.float32 if dt == bd.F32 else torch.bfloat16, device="cuda")
    lib.call("dllm_synth_fill", bd.ptr(t), n, dt, 1234, 0x77, std, mode, stream())
    torch.cuda.synchronize()
    if mode == 0:
        ref = synth.normal_tensor(1234, 0x77, (n,), std, dtype)
    elif mode == 1:
        ref = synth.norm_gain(1234, 0x77, n, std, dtype)
    else:
        ref = synth.norm_gain(1234, 0x77, n, 0.0, dtype)
    got = t.cpu().numpy() if dt == bd.F32 else t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got.view(np.uint32 if dt == bd.F32 else np.uint16),
                          np.asarray(ref).view(np.uint32 if dt == bd.F32 else np.uint16))


# ------------------------------------------------------------------ confidence + unmask

def run_conf(lib, logits_dev, ldtype, B, K, V, mask_id, tau, tokens_np):
    toks = torch.from_numpy(tokens_np.astype(np.int32)).cuda()
    conf = torch.empty(B * K, dtype=torch.float32, device="cuda")
    arg = torch.empty(B * K, dtype=torch.int32, device="cuda")
    nun = torch.empty(B, dtype=torch.int32, device="cuda")
    rem = torch.empty(B, dtype=torch.int32, device="cuda")
    uidx = torch.empty(B * K, dtype=torch.int32, device="cuda")
    wsb = lib.raw("dllm_kernel_workspace_bytes")(B, 0, 0, 0, 0, K, V)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    lib.call("dllm_kernel_confidence_unmask", bd.ptr(logits_dev), ldtype, B, K, V, mask_id, tau,
             bd.ptr(toks), K, bd.ptr(conf), bd.ptr(arg), bd.ptr(nun), bd.ptr(rem), bd.ptr(uidx),
             bd.ptr(ws), wsb, stream())
    torch.cuda.synchronize()
    return (toks.cpu().numpy(), conf.cpu().numpy().reshape(B, K), arg.cpu().numpy().reshape(B, K),
            nun.cpu().numpy(), rem.cpu().numpy(), uidx.cpu().numpy().reshape(B, K))


CONF_CASES = [
    # name, B, K, V, boost, logits dtype, masked fraction
    ("llada_block_bf16", 1, 32, 126464, 12.0, "bf16", 1.0),
    ("llada_block_bf16_boost24", 1, 32, 126464, 24.0, "bf16", 1.0),
    ("llada_block_f32_partial", 1, 32, 126464, 24.0, "f32", 0.6),
    ("dream_batch_f32", 8, 32, 152064, 24.0, "f32", 0.8),
    ("ragged_vocab_scalar_path", 3, 7, 1001, 10.0, "f32", 0.7),
    ("k64_small_vocab", 2, 64, 4096, 9.0, "bf16", 0.9),
    ("k1", 4, 1, 640, 6.0, "f32", 1.0),
    # mask id inside a full slice (LLaDA's id), not in the ragged last one
    ("mask_mid_vocab_bf16", 2, 32, 126464, 12.0, "bf16", 1.0, 126336),
    # slices longer than one pass of the workgroup (vocabulary > 32 slices of 16384)
    ("huge_vocab_looped_slices", 1, 64, 600000, 12.0, "f32", 1.0),
]


@pytest.mark.parametrize("case", CONF_CASES, ids=[c[0] for c in CONF_CASES])
@pytest.mark.parametrize("tau", [0.9, 0.5, 1.5, 0.0])
def test_confidence_unmask_parity(lib, case, tau):
    name, B, K, V, boost, ldt, frac = case[:7]
    mask_id = case[7] if len(case) > 7 else V - 1
    z = synth.boosted_logits(43, B * K, V, boost, ldt)
    zf = synth.bf16_bits_to_fp32(z) if ldt == "bf16" else z
    dev = dev_bf16(z) if ldt == "bf16" else dev_f32(z)
    r = np.random.default_rng(B * 1000 + K)
    toks = np.where(r.random((B, K)) < frac, mask_id, r.integers(0, V - 1, (B, K)))
    if frac == 1.0:
        toks[:] = mask_id
    got_tok, conf, arg, nun, rem, uidx = run_conf(lib, dev, bd.F32 if ldt == "f32" else bd.BF16,
                                                   B, K, V, mask_id, tau, toks)
    rc, ra = decode.confidence_argmax(zf.astype(np.float64), mask_id)
    rc, ra = rc.reshape(B, K), ra.reshape(B, K)
    # argmax of identical inputs: exact (lowest id on ties); confidence: fp32 rounding
    grade_confidence_stage(zf, conf, arg, mask_id)
    # the unmask rule on the kernel's own confidences and argmaxes: bit for bit on every
    # sequence (tokens, counts, masks left, compacted indices)
    grade_unmask_stage(toks, conf, arg, got_tok, nun, rem, mask_id, tau, uidx)
    want_tok, U, wn, wr = decode.unmask(toks, rc, ra, mask_id, tau)
    # identical logits on both sides: confidences differ only by fp32 rounding (checked
    # above to 2e-5 relative), so every decision farther than that from a flip -- far
    # tighter than a 1e-3 margin -- must also match the oracle's own decisions
    ok = safe_sequences(rc, 2e-5 * rc, tau, toks == mask_id)
    for b in np.nonzero(ok)[0]:
        assert np.array_equal(got_tok[b], want_tok[b])
        assert nun[b] == wn[b] and rem[b] == wr[b]
        sel = np.nonzero(U[b])[0]
        assert np.array_equal(uidx[b, :len(sel)], sel)
        assert np.all(uidx[b, len(sel):] == -1)
    # whatever the margins: the rule's invariants hold
    masked = toks == mask_id
    assert np.all((nun >= 1) | (masked.sum(1) == 0))
    assert np.all(nun + rem == masked.sum(1))
    assert np.all(got_tok[~masked] == toks[~masked])


@pytest.mark.parametrize("ldt", ["bf16", "f32"])
def test_confidence_tied_maxima(lib, ldt):
    """Logits on a coarse grid: every row's maximum is reached at many ids, and the
    argmax must be the lowest of them (the mask id excluded even when it ties)."""
    B, K, V = 2, 32, 126464
    r = np.random.default_rng(7)
    zf = np.clip(np.round(r.standard_normal((B * K, V)) * 2) / 2, -4.0, 2.0).astype(np.float32)
    mask_id = 126336
    zf[:, mask_id] = 2.0
    if ldt == "bf16":
        z = (zf.view(np.uint32) >> 16).astype(np.uint16)   # exact: the grid values are bf16
        dev = dev_bf16(z)
    else:
        dev = dev_f32(zf)
    toks = np.full((B, K), mask_id)
    gtok, conf, arg, nun, rem, uidx = run_conf(lib, dev, bd.F32 if ldt == "f32" else bd.BF16,
                                               B, K, V, mask_id, 0.9, toks)
    grade_unmask_stage(toks, conf, arg, gtok, nun, rem, mask_id, 0.9, uidx)
    rc, ra = decode.confidence_argmax(zf.astype(np.float64), mask_id)
    assert np.array_equal(arg.reshape(-1), ra)
    assert np.max(np.abs(conf.reshape(-1) - rc) / rc) < 2e-5
    assert np.all(nun == 1) and np.all(rem == K - 1)


# ------------------------------------------------------------------ attention

def attn_inputs(seed, B, Hq, Hkv, R, S, dtype):
    D = 128 if dtype == "bf16" else 16
    q, k, v = synth.attention_inputs(seed, B, Hq, Hkv, R, S, D)
    if dtype == "f32":
        q, k, v = (synth.bf16_bits_to_fp32(a) for a in (q, k, v))
    return q, k, v, D


def run_attn(lib, q, k, v, B, Hq, Hkv, R, S, D, dtype):
    Sp = (S + 63) // 64 * 64
    dt = bd.BF16 if dtype == "bf16" else bd.F32
    to = dev_bf16 if dtype == "bf16" else dev_f32
    kp = np.zeros((B, Hkv, Sp, D), q.dtype)
    kp[:, :, :S] = k
    vp = np.zeros((B, Hkv, Sp, D), q.dtype)
    vp[:, :, :S] = v
    # poison the padding: keys >= S must never be read
    if dtype == "bf16":
        kp[:, :, S:] = 0x7FC0
        vp[:, :, S:] = 0x7FC0
    else:
        kp[:, :, S:] = np.nan
        vp[:, :, S:] = np.nan
    # values transposed in blocks of 32 keys: [B][Hkv][Sp/32][D][32]
    vt = np.ascontiguousarray(vp.reshape(B, Hkv, Sp // 32, 32, D).swapaxes(-1, -2))
    qd, kd, vd = to(q), to(kp), to(vt)
    o = torch.empty((B, R, Hq * D), dtype=qd.dtype, device="cuda")
    wsb = lib.raw("dllm_kernel_workspace_bytes")(B, Hq, R, S, D, 0, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    lib.call("dllm_kernel_block_attention", bd.ptr(qd), bd.ptr(kd), bd.ptr(vd), bd.ptr(o), B, Hq,
             Hkv, R, S, Sp, D, dt, bd.ptr(ws), wsb, stream())
    torch.cuda.synchronize()
    return host(o).reshape(B, R, Hq, D).transpose(0, 2, 1, 3)


ATTN_CASES = [
    # name, B, Hq, Hkv, R, S, dtype
    # (plan: four-wave chunks of 128 keys, 8 chunks)
    ("llada_block32_kv1024", 1, 32, 32, 32, 1024, "bf16"),
    # eight-wave chunks of 256 keys, ragged last chunk (the 8B step shape)
    ("llada_block32_kv2024", 1, 32, 32, 32, 2024, "bf16"),
    # eight-wave chunks whose last chunk has seven waves past the last key
    ("nw8_masked_waves", 1, 32, 32, 32, 1800, "bf16"),
    # six eight-wave chunks (192 workgroups, the fewest that take this form); the last
    # chunk holds 20 keys: one partial sub-tile and seven waves past the last key
    ("nw8_six_chunks_ragged", 1, 32, 32, 32, 1300, "bf16"),
    # grouped query heads (one workgroup per KV head and chunk, a wave per query head):
    # 32 chunks of one 32-key sub-tile, ragged last chunk
    ("gqa_7to1_b2", 2, 28, 4, 32, 1000, "bf16"),
    # the 7B batch-8 step shape: 8 chunks of 128 keys, 256 workgroups
    ("gqa_7to1_b8", 8, 28, 4, 32, 1024, "bf16"),
    # 10 chunks of 256 keys (the LDS limit), ragged last one
    ("gqa_7to1_b8_multi_subtile", 8, 28, 4, 32, 2500, "bf16"),
    # fewer rows than a tile, ragged keys, group of 4 (idle waves 4-7)
    ("gqa_4to1_rows20_ragged", 2, 8, 2, 20, 777, "bf16"),
    # a single chunk: the normalised output is written directly, no combine
    ("gqa_2to1_one_chunk", 1, 4, 2, 32, 30, "bf16"),
    # several sub-tiles per wave: 9 (odd) per wave over 4 chunks with a ragged last one
    ("multi_subtile_odd_ragged", 2, 32, 32, 32, 4400, "bf16"),
    # 17 eight-wave chunks: the merge walks its chunks in three rounds of loads
    ("many_chunks_ragged", 1, 32, 32, 32, 4100, "bf16"),
    ("ragged_rows_keys", 1, 4, 2, 20, 77, "bf16"),
    # one KV head per query head with 20 query rows: the head-dim-split kernel with 12
    # clamped rows, four-wave chunks of 128 keys, the last one 104 keys
    ("mha_rows20_ragged", 1, 8, 8, 20, 1000, "bf16"),
    ("two_row_tiles", 1, 2, 1, 64, 300, "bf16"),
    # 200 query rows: seven 32-row query tiles on the split-KV kernel (prefix-mode steps)
    ("split_kv_200_rows", 1, 2, 2, 200, 333, "bf16"),
    # the prefix workload's first step: 256 query rows (eight 32-row tiles) against 512
    # keys, eight-wave chunks of 256 keys with the P.V product split over the head dim
    ("prefix_256_rows_kv512", 1, 32, 32, 256, 512, "bf16"),
    # grouped query heads, chunks of four sub-tiles (walked unrolled) and a last chunk of
    # four keys (one sub-tile, walked by the loop)
    ("gqa_7to1_b8_ragged_last", 8, 28, 4, 32, 900, "bf16"),
    # past 256 rows the flash kernel: three 128-row tiles, the last ragged
    ("flash_300_rows", 1, 2, 2, 300, 333, "bf16"),
    ("flash_refresh_shape", 1, 4, 4, 2024, 2024, "bf16"),
    ("f32_small", 2, 4, 2, 8, 48, "f32"),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_parity(lib, case):
    name, B, Hq, Hkv, R, S, dtype = case
    q, k, v, D = attn_inputs(42, B, Hq, Hkv, R, S, dtype)
    got = run_attn(lib, q, k, v, B, Hq, Hkv, R, S, D, dtype)
    f = (lambda a: synth.bf16_bits_to_fp32(a).astype(np.float64)) if dtype == "bf16" else \
        (lambda a: a.astype(np.float64))
    ref = om.attention(f(q), f(k), f(v))
    assert np.all(np.isfinite(got))
    if dtype == "bf16":
        # bf16 output rounding (2^-9 relative) and bf16 probabilities in P.V: the bf16
        # bar, 2e-2 of the largest output, per (sequence, query head)
        err = np.max(np.abs(got - ref), axis=(2, 3)) / np.max(np.abs(ref), axis=(2, 3))
        print(f"{name}: worst per-head rel err {err.max():.2e}")
        assert err.max() <= 2e-2
        assert np.mean(np.abs(got - ref)) <= 2e-2 * np.mean(np.abs(ref))
    else:
        assert rel_inf(got, ref) < 1e-5


# ------------------------------------------------------------------ GEMM

def run_linear(lib, x, w, M, N, K, dtype, mode, scale=1.0, y0=None):
    to = dev_bf16 if dtype == "bf16" else dev_f32
    dt = bd.BF16 if dtype == "bf16" else bd.F32
    xd, wd = to(x), to(w)
    if mode == 0:
        y = torch.empty((M, N), dtype=xd.dtype, device="cuda")
    else:
        y = dev_f32(y0) if y0 is not None else torch.zeros((M, N), dtype=torch.float32, device="cuda")
    wsb = lib.raw("dllm_linear_workspace_bytes")(M, N, K, dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    lib.call("dllm_kernel_linear", bd.ptr(xd), bd.ptr(wd), bd.ptr(y), M, N, K, dt, mode, scale,
             bd.ptr(ws), wsb, stream())
    torch.cuda.synchronize()
    return host(y)


GEMM_CASES = [
    # name, M, N, K, dtype   (skinny: M <= 64; mid: 64 < M <= 256; tiled: 256 < M < 512;
    # big: M >= 512)
    ("skinny_m32_o_proj", 32, 4096, 4096, "bf16"),
    ("skinny_m7_ragged_n", 7, 1000, 512, "bf16"),
    ("skinny_m50_two_tiles", 50, 384, 1024, "bf16"),
    ("skinny_m32_down_k12288", 32, 512, 12288, "bf16"),
    # the 8B down projection (8 K ranges of 1536, 192-deep per wave, over 32 workgroups
    # each), 16 rows too
    ("skinny_m32_down_full", 32, 4096, 12288, "bf16"),
    ("skinny_m16_down_full", 16, 4096, 12288, "bf16"),
    # 33 rows: four 16-row MFMA tiles, 31 of the 64 staged rows clamped to the last; the
    # staged slice (64 rows of 1024 columns plus a pad chunk) ends in a partial load slot
    ("skinny_m33_clamped_rows", 33, 1024, 2048, "bf16"),
    ("tiled_m300_ragged", 300, 384, 512, "bf16"),
    # mid (64 < M <= 256): every tile split over K / whole tiles plus a split ragged
    # last round (2 rounds of 256 whole tiles, 9 tail tiles in 4 K pieces) / ragged N
    ("mid_m256_deep_splitk", 256, 256, 3584, "bf16"),
    ("mid_m96_ragged_n", 96, 1000, 512, "bf16"),
    ("mid_m200_whole_and_tail", 200, 33000, 256, "bf16"),
    ("mid_m130_rounds_and_tail", 130, 66624, 256, "bf16"),
    ("big_m600_ragged_splitk", 600, 640, 512, "bf16"),
    ("big_m1064_two_row_tiles", 1064, 768, 1024, "bf16"),
    # 72 x 4 large tiles: 256 whole tiles, then 8 column tiles x 4 row tiles in 8 K pieces
    ("big_m800_whole_and_split_tail", 800, 18400, 512, "bf16"),
    # 80 x 4 large tiles: 256 whole, then 16 x 4 column tiles in 4 K pieces
    ("big_m800_whole_and_split_tail_4", 800, 20400, 512, "bf16"),
    # 104 x 4 large tiles: 256 whole, then 40 x 4 (too many for two K pieces each in a
    # round) as 80 x 7 tiles of 128 x 128
    ("big_m800_whole_and_tiled_tail", 800, 26496, 512, "bf16"),
    ("f32_small", 20, 200, 64, "f32"),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_linear_parity(lib, case, mode):
    name, M, N, K, dtype = case
    x = synth.normal_tensor(7, 1, (M, K), 1.0, dtype)
    w = synth.normal_tensor(7, 2, (N, K), 1.0 / np.sqrt(K), dtype)
    y0 = synth.normal_tensor(7, 3, (M, N), 1.0, "f32") if mode == 2 else None
    got = run_linear(lib, x, w, M, N, K, dtype, mode, 0.75, y0)
    xf = synth.as_float(x, dtype).astype(np.float64)
    wf = synth.as_float(w, dtype).astype(np.float64)
    ref = om.linear(xf, wf)
    if mode == 1:
        ref = 0.75 * ref
    if mode == 2:
        ref = y0.astype(np.float64) + ref
    tol = 1e-2 if (mode == 0 and dtype == "bf16") else 1e-4
    assert rel_inf(got, ref) < tol


def test_lm_head_full_shape_sampled_columns(lib):
    """LLaDA-shape LM head (M=32, N=126464, K=4096), weights made on the device;
    sampled output columns checked against host-generated weight rows."""
    M, N, K = 32, 126464, 4096
    W = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    lib.call("dllm_synth_fill", bd.ptr(W), N * K, bd.BF16, 1234, synth.TID_LM_HEAD,
             1.0 / np.sqrt(K), 0, stream())
    x = synth.normal_tensor(9, 9, (M, K), 1.0, "bf16")
    xd = dev_bf16(x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsb = lib.raw("dllm_linear_workspace_bytes")(M, N, K, bd.BF16)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    lib.call("dllm_kernel_linear", bd.ptr(xd), bd.ptr(W), bd.ptr(y), M, N, K, bd.BF16, 1, 3.0,
             bd.ptr(ws), wsb, stream())
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([np.arange(0, 300), np.arange(N - 300, N),
                                     np.random.default_rng(0).integers(0, N, 400)]))
    idx = (cols[:, None] * K + np.arange(K)[None, :]).reshape(-1).astype(np.uint64)
    wrows = synth.fp32_to_bf16_bits(synth.normal_fp32(1234, synth.TID_LM_HEAD, idx, 1.0 / np.sqrt(K)))
    wf = synth.bf16_bits_to_fp32(wrows).reshape(len(cols), K).astype(np.float64)
    ref = 3.0 * om.linear(synth.bf16_bits_to_fp32(x).astype(np.float64), wf)
    got = y.cpu().numpy()[:, cols].astype(np.float64)
    assert rel_inf(got, ref) < 1e-4
