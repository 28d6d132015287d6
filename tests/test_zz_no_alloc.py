"""dllm_kernel_confidence_unmask_noalloc (slice partials in the library's static device
array, no workspace) against dllm_kernel_confidence_unmask (caller workspace): identical
outputs, bit for bit, on two calls in a row, the second with a smaller input, and the
size limit rejected before anything is enqueued."""
import numpy as np
import pytest

import synth
from gpu_util import dev_bf16, dev_f32, grade_unmask_stage

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from diffusion_dllm_block_amd import binding as bd  # noqa: E402


def run(lib, noalloc, z, ldt, B, K, V, mask_id, tau, toks):
    dev = dev_bf16(z) if ldt == "bf16" else dev_f32(z)
    t = torch.from_numpy(toks.astype(np.int32)).cuda()
    conf = torch.full((B * K,), -7.0, dtype=torch.float32, device="cuda")
    arg = torch.full((B * K,), -7, dtype=torch.int32, device="cuda")
    nun = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    rem = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    uidx = torch.full((B * K,), -7, dtype=torch.int32, device="cuda")
    dt = bd.F32 if ldt == "f32" else bd.BF16
    st = bd.stream_handle()
    if noalloc:
        lib.call("dllm_kernel_confidence_unmask_noalloc", bd.ptr(dev), dt, B, K, V, mask_id, tau,
                 bd.ptr(t), K, bd.ptr(conf), bd.ptr(arg), bd.ptr(nun), bd.ptr(rem), bd.ptr(uidx),
                 st)
    else:
        wsb = lib.raw("dllm_kernel_workspace_bytes")(B, 0, 0, 0, 0, K, V)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        lib.call("dllm_kernel_confidence_unmask", bd.ptr(dev), dt, B, K, V, mask_id, tau,
                 bd.ptr(t), K, bd.ptr(conf), bd.ptr(arg), bd.ptr(nun), bd.ptr(rem), bd.ptr(uidx),
                 bd.ptr(ws), wsb, st)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (t, conf, arg, nun, rem, uidx)]


CASES = [
    # B, K, V, boost, logits dtype, masked fraction, tau: the larger call first
    (8, 32, 152064, 24.0, "f32", 0.8, 0.9),
    (1, 32, 126464, 12.0, "bf16", 1.0, 0.9),
]


def test_noalloc_matches_workspace_entry_two_calls(lib):
    for i, (B, K, V, boost, ldt, frac, tau) in enumerate(CASES):
        mask_id = V - 1
        z = synth.boosted_logits(43 + i, B * K, V, boost, ldt)
        r = np.random.default_rng(5 + i)
        toks = np.where(r.random((B, K)) < frac, mask_id, r.integers(0, V - 1, (B, K)))
        want = run(lib, False, z, ldt, B, K, V, mask_id, tau, toks)
        got = run(lib, True, z, ldt, B, K, V, mask_id, tau, toks)
        for a, b in zip(got, want):
            assert a.dtype == b.dtype
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b)
        gtok, conf, arg, nun, rem, uidx = got
        grade_unmask_stage(toks, conf.reshape(B, K), arg.reshape(B, K), gtok, nun, rem,
                           mask_id, tau, uidx)


def test_noalloc_rejects_oversized_calls(lib):
    # 40 sequences of 64 rows over a vocabulary that needs 32 slices per row:
    # 81920 > 65536 slice partials; rejected on the host, nothing enqueued
    B, K, V = 40, 64, 32 * 16384
    f = lib.raw("dllm_kernel_confidence_unmask_noalloc")
    fake = torch.empty(1, dtype=torch.float32, device="cuda")
    p = bd.ptr(fake)
    st = f(p, bd.F32, B, K, V, V - 1, 0.9, p, K, p, p, p, p, None, bd.stream_handle())
    assert st == -3
