"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before anything is enqueued."""
import ctypes as C
import math

import pytest

from diffusion_dllm_block_amd import binding as bd


@pytest.fixture(scope="module")
def lib():
    return bd.load()


def test_exports_every_declared_symbol(lib):
    names = bd.declared_functions()
    assert len(names) >= 16
    missing = [n for n in names if not hasattr(lib.cdll, n)]
    assert missing == []
    # and the binding knows the signature of each
    assert sorted(bd._SIGS) == names


def test_status_strings(lib):
    for code in bd.STATUS:
        assert lib.cdll.dllm_status_string(code)
    assert lib.cdll.dllm_status_string(-4) == b"buffer too small"


FAKE = 0x1000  # never dereferenced: every case below fails validation first


def model_desc(L=2, d=64, H=4, Hkv=4, D=16, F=256, V=256, dtype=bd.F32, **kw):
    arr = (C.c_void_p * L)(*([FAKE] * L))
    m = bd.ModelDesc(n_layers=L, d_model=d, n_heads=H, n_kv_heads=Hkv, head_dim=D, d_ffn=F,
                     vocab=V, mask_id=V - 1, rope_theta=10000.0, norm_eps=1e-5, logit_scale=8.0,
                     dtype=dtype, embed=FAKE, final_norm=FAKE, lm_head=FAKE,
                     attn_norm=C.cast(arr, C.POINTER(C.c_void_p)),
                     w_qkv=C.cast(arr, C.POINTER(C.c_void_p)), w_o=C.cast(arr, C.POINTER(C.c_void_p)),
                     ffn_norm=C.cast(arr, C.POINTER(C.c_void_p)),
                     w_gate_up=C.cast(arr, C.POINTER(C.c_void_p)),
                     w_down=C.cast(arr, C.POINTER(C.c_void_p)))
    for k, v in kw.items():
        setattr(m, k, v)
    m._keep = arr
    return m


def seq_desc(B=1, P=16, G=32, K=8, mode=bd.CACHE_DUAL, tau=0.9, **kw):
    s = bd.SeqDesc(batch=B, prompt_len=P, gen_len=G, block_len=K, cache_mode=mode, threshold=tau,
                   tokens=FAKE, kv_cache=FAKE, kv_cache_bytes=0, workspace=FAKE, workspace_bytes=0)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def sizes(lib, m, s):
    return (lib.cdll.dllm_kv_cache_bytes(C.byref(m), C.byref(s)),
            lib.cdll.dllm_workspace_bytes(C.byref(m), C.byref(s)))


def prefill(lib, m, s):
    return lib.cdll.dllm_prefill_cache(C.byref(m), C.byref(s), None)


def test_sizes_of_valid_descriptors(lib):
    m, s = model_desc(), seq_desc()
    cb, wb = sizes(lib, m, s)
    # cache: L * 2 * B * Hkv * Sp * D * 4 bytes with Sp = 48 rounded up to 64
    assert cb == 2 * 2 * 1 * 4 * 64 * 16 * 4
    assert wb > 0
    # the 8B shape, DualCache: cache 32*2*1*32*2048*128*2 bytes
    big = model_desc(L=32, d=4096, H=32, Hkv=32, D=128, F=12288, V=126464, dtype=bd.BF16)
    cb, wb = sizes(lib, big, seq_desc(P=1000, G=1024, K=32))
    assert cb == 32 * 2 * 32 * 2048 * 128 * 2
    assert 0 < wb < 2 << 30


@pytest.mark.parametrize("change,status", [
    (dict(seq=dict(G=30)), -2),
    (dict(seq=dict(K=128, G=128)), -3),
    (dict(seq=dict(tau=math.nan)), -7),
    (dict(seq=dict(mode=5)), -7),
    (dict(seq=dict(mode=-1)), -7),
    (dict(seq=dict(B=0)), -2),
    (dict(model=dict(n_kv_heads=3)), -2),
    (dict(model=dict(head_dim=24)), -3),
    (dict(model=dict(mask_id=256)), -7),
    (dict(model=dict(dtype=7)), -7),
    (dict(model=dict(embed=None)), -1),
    (dict(model=dict(dtype=bd.BF16)), -3),   # bf16 needs head_dim 128
])
def test_validation_rejects_before_enqueue(lib, change, status):
    mk = dict(change.get("model", {}))
    sk = dict(change.get("seq", {}))
    m = model_desc(**mk)
    s = seq_desc(**sk)
    assert sizes(lib, m, s) == (0, 0)
    assert prefill(lib, m, s) == status
    assert lib.cdll.dllm_last_error()


def test_small_buffers_and_bad_block_are_rejected(lib):
    m, s = model_desc(), seq_desc()
    cb, wb = sizes(lib, m, s)
    s.kv_cache_bytes, s.workspace_bytes = cb - 1, wb
    assert prefill(lib, m, s) == -4
    s.kv_cache_bytes, s.workspace_bytes = cb, wb - 1
    assert prefill(lib, m, s) == -4
    s.workspace_bytes = wb
    n = C.c_int32(0)
    for blk in (-1, 4):
        assert lib.cdll.dllm_refresh_cache(C.byref(m), C.byref(s), blk, None) == -6
        assert lib.cdll.dllm_block_step(C.byref(m), C.byref(s), blk, None, FAKE, FAKE, None,
                                        None, None) == -6
    s.tokens = None
    assert prefill(lib, m, s) == -1


def test_staleness_validation(lib):
    m, s = model_desc(), seq_desc()
    cb, wb = sizes(lib, m, s)
    s.kv_cache_bytes, s.workspace_bytes = cb, wb
    f = lib.cdll.dllm_cache_staleness
    for blk in (-1, 4):
        assert f(C.byref(m), C.byref(s), blk, FAKE, cb, FAKE, None, None) == -6
    assert f(C.byref(m), C.byref(s), 0, None, cb, FAKE, None, None) == -1
    assert f(C.byref(m), C.byref(s), 0, FAKE, cb, None, None, None) == -1
    assert f(C.byref(m), C.byref(s), 0, FAKE, cb - 1, FAKE, None, None) == -4
    s.cache_mode = bd.CACHE_NONE
    assert f(C.byref(m), C.byref(s), 0, FAKE, cb, FAKE, None, None) == -6


def test_null_descriptors(lib):
    assert lib.cdll.dllm_prefill_cache(None, None, None) == -1
    assert lib.cdll.dllm_workspace_bytes(None, None) == 0
    assert lib.cdll.dllm_generate(None, None, None, None) == -1


def test_kernel_entry_validation(lib):
    f = lib.cdll.dllm_kernel_block_attention
    # bf16 needs D == 128
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 4, 10, 32, 64, bd.BF16, None, 0, None) == -3
    # the value cache comes in 32-key blocks: Sp must be a multiple of 32
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 4, 10, 16, 128, bd.BF16, None, 0, None) == -3
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 3, 2, 4, 10, 16, 16, bd.F32, None, 0, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 4, 10, 8, 16, bd.F32, None, 0, None) == -2  # Sp < S
    g = lib.cdll.dllm_kernel_confidence_unmask
    assert g(FAKE, bd.BF16, 1, 65, 100, 99, 0.9, FAKE, 65, FAKE, FAKE, FAKE, FAKE, None, FAKE,
             1 << 20, None) == -3
    assert g(FAKE, bd.BF16, 1, 8, 100, 100, 0.9, FAKE, 8, FAKE, FAKE, FAKE, FAKE, None, FAKE,
             1 << 20, None) == -7
    assert g(FAKE, bd.BF16, 1, 8, 100, 5, 0.9, FAKE, 8, FAKE, FAKE, FAKE, FAKE, None, FAKE,
             0, None) == -4
    h = lib.cdll.dllm_kernel_linear
    assert h(FAKE, FAKE, FAKE, 4, 4, 100, bd.BF16, 0, 1.0, None, 0, None) == -3
    assert h(FAKE, FAKE, FAKE, 4, 4, 256, bd.BF16, 3, 1.0, None, 0, None) == -7
    assert h(FAKE, FAKE, FAKE, 4, 4, 384, bd.BF16, 0, 1.0, None, 0, None) == -3
    assert lib.cdll.dllm_profile_select(99) == -7
    assert lib.cdll.dllm_profile_select_every(99, 1) == -7
    assert lib.cdll.dllm_profile_select_every(0, 0) == -7
    assert lib.cdll.dllm_profile_select_every(-1, 7) == 0


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: without the built HIP library the binding raises instead of running
    anything else."""
    with pytest.raises(FileNotFoundError):
        bd.Lib(str(tmp_path / "libdllm.so"))
