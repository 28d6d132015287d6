"""Seeded input generator: pinned to SplitMix64's published outputs and to torch's bf16."""
import numpy as np
import torch

import synth


def test_splitmix64_published_vectors():
    # SplitMix64 seeded with 0 (Vigna's splitmix64.c): the first three outputs are the
    # widely published test values below.  raw64 with x0 = 0 means seed such that the
    # stream state is 0 -- check the finaliser directly instead.
    z = np.array([0x9E3779B97F4A7C15 * k % (1 << 64) for k in (1, 2, 3)], dtype=np.uint64)
    got = [int(v) for v in synth._mix_np(z)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_indexing_matches_sequential_stream():
    x0 = synth.stream_state(1234, 7)
    M = (1 << 64) - 1
    seq = []
    x = x0
    for _ in range(5):
        x = (x + 0x9E3779B97F4A7C15) & M
        seq.append(synth._mix_int(x))
    assert [int(v) for v in synth.raw64(1234, 7, np.arange(5, dtype=np.uint64))] == seq
    # random access equals sequential access
    assert int(synth.raw64(1234, 7, np.array([3], np.uint64))[0]) == seq[3]


def test_streams_differ_by_seed_and_tensor():
    a = synth.raw64(1, 0, np.arange(8, dtype=np.uint64))
    b = synth.raw64(2, 0, np.arange(8, dtype=np.uint64))
    c = synth.raw64(1, 1, np.arange(8, dtype=np.uint64))
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_irwin_hall_moments_and_range():
    v = synth.normal_fp32(99, 3, np.arange(1 << 20, dtype=np.uint64)).astype(np.float64)
    assert abs(v.mean()) < 5e-3
    assert abs(v.std() - 1.0) < 5e-3
    assert v.max() <= 2 * np.sqrt(3) and v.min() >= -2 * np.sqrt(3)
    # Irwin-Hall(4) excess kurtosis is -6/(5*4) = -0.3
    k = ((v - v.mean()) ** 4).mean() / v.var() ** 2 - 3.0
    assert abs(k + 0.3) < 0.02


def test_bf16_rounding_matches_torch():
    x = synth.normal_fp32(5, 5, np.arange(100000, dtype=np.uint64), 3.0)
    x = np.concatenate([x, np.array([1.0, 1.00390625, 1.01171875, -2.5, 0.0, 65504.0,
                                     3.4e38, 1e-40], np.float32)])
    ours = synth.fp32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_fp32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_prompt_tokens_exclude_mask_and_are_per_sequence():
    wl = synth.WORKLOADS["dream7b_dual_b8_p512_g512"]
    p = synth.make_prompt(wl)
    assert p.shape == (8, 512)
    assert p.min() >= 0 and p.max() < wl.model.vocab - 1
    assert not np.array_equal(p[0], p[1])
    # sequence i uses seed prompt_seed + i
    assert np.array_equal(p[3], synth.uniform_ints(wl.prompt_seed + 3, synth.TID_PROMPT, 512,
                                                   wl.model.vocab - 1))


def test_weight_shapes_and_scale():
    wl = synth.WORKLOADS["tiny_dual"]
    W = synth.make_weights(wl)
    m = wl.model
    assert W["embed"].shape == (m.vocab, m.d_model)
    assert W["w_qkv.0"].shape == (3 * m.n_heads * m.head_dim, m.d_model)
    assert W["w_gate_up.1"].shape == (2 * m.d_ffn, m.d_model)
    assert W["w_down.1"].shape == (m.d_model, m.d_ffn)
    assert np.all(W["attn_norm.0"] == 1.0)
    s = W["w_down.0"].std() * np.sqrt(m.d_ffn)
    assert 0.9 < s < 1.1


def test_named_workloads_have_the_stated_shapes():
    """The workload files hold the shapes and settings the workloads are defined by: a tiny
    fp32 parity model, the LLaDA-8B shape in prefix and DualCache settings, and the
    Dream-7B shape with grouped-query attention and a batch of 8."""
    W = synth.WORKLOADS
    t = W["tiny_dual"]
    assert (t.model.n_layers, t.model.d_model, t.model.n_heads, t.model.head_dim, t.model.d_ffn,
            t.model.vocab, t.model.mask_id, t.model.logit_scale, t.model.dtype) == \
        (2, 64, 4, 16, 256, 256, 255, 8.0, "f32")
    assert (t.batch, t.prompt_len, t.gen_len, t.block_len, t.cache_mode, t.threshold) == \
        (1, 16, 32, 8, "dual", 0.9)
    for name, mode, P, G in (("llada8b_prefix_p256_g256", "prefix", 256, 256),
                             ("llada8b_dual_p1000_g1024", "dual", 1000, 1024)):
        w = W[name]
        assert (w.model.n_layers, w.model.d_model, w.model.n_heads, w.model.n_kv_heads,
                w.model.head_dim, w.model.d_ffn, w.model.vocab, w.model.dtype) == \
            (32, 4096, 32, 32, 128, 12288, 126464, "bf16")
        assert (w.batch, w.prompt_len, w.gen_len, w.block_len, w.cache_mode) == (1, P, G, 32, mode)
    d = W["dream7b_dual_b8_p512_g512"]
    assert (d.model.n_layers, d.model.d_model, d.model.n_heads, d.model.n_kv_heads,
            d.model.head_dim, d.model.d_ffn, d.model.vocab) == (28, 3584, 28, 4, 128, 18944, 152064)
    assert (d.batch, d.prompt_len, d.gen_len, d.block_len, d.cache_mode) == (8, 512, 512, 32, "dual")


def test_workload_files_round_trip_and_reject_unknown_keys(tmp_path):
    import json
    import pytest
    src = json.load(open(f"{synth.WORKLOAD_DIR}/tiny_dual.json"))
    p = tmp_path / "w.json"
    p.write_text(json.dumps(src))
    assert synth.load_workload(str(p)) == synth.WORKLOADS["tiny_dual"]
    bad = dict(src, treshold=0.5)
    p.write_text(json.dumps(bad))
    with pytest.raises(ValueError):
        synth.load_workload(str(p))
