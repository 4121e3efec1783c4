"""The C-ABI library loads, exports every symbol the header declares, and its
host-side checks return the documented status codes.  No device work."""
import ctypes
import os
import re

import numpy as np
import pytest

from protein_language_model_amd import esm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "esm_encoder.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(esm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = esm.load_library()
    names = declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding knows the signature of each
    assert set(names) == set(esm.SIGNATURES), set(names) ^ set(esm.SIGNATURES)
    src = open(HEADER).read()
    assert lib.esm_abi_version() == int(re.search(r"#define ESM_ABI_VERSION (\d+)", src).group(1))
    assert len(esm.KERNEL_CLASSES) == int(re.search(r"ESM_K_COUNT = (\d+)", src).group(1))
    assert esm.ATTN_TILE_ROWS == int(re.search(r"#define ESM_ATTN_TILE_ROWS (\d+)", src).group(1))


def test_head_weights_struct_has_eight_pointers():
    assert ctypes.sizeof(esm.EsmHeadWeights) == 64
    assert [f[0] for f in esm.EsmHeadWeights._fields_] == list(esm.HEAD_WEIGHT_NAMES)
    src = open(HEADER).read()
    body = src[src.index("const void* final_ln_gamma"):src.index("} esm_head_weights;")]
    assert re.findall(r"const void\* (\w+);", body) == list(esm.HEAD_WEIGHT_NAMES)


def test_fp8_state_struct_layout_matches_the_header():
    # two int32, four pointers, one uint32 (padded to the pointer alignment)
    assert ctypes.sizeof(esm.EsmFp8State) == 48
    assert esm.EsmFp8State.act_scale.offset == 8 and esm.EsmFp8State.nonfinite.offset == 40


def test_status_strings():
    lib = esm.load_library()
    for code, name in esm.STATUS_NAMES.items():
        assert lib.esm_status_str(code).decode() == name


def _status(fn, *args):
    lib = esm.load_library()
    return getattr(lib, fn)(*args), lib.esm_last_error().decode()


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


@pytest.mark.parametrize("cu,T,maxlen,code", [
    ([0, 3, 5], 5, 3, 0),
    ([0, 0, 0], 0, 0, 0),
    ([1, 3, 5], 5, 3, 3),       # cu[0] != 0
    ([0, 3, 2], 2, 3, 3),       # decreasing
    ([0, 3, 5], 6, 3, 3),       # cu[B] != T
    ([0, 3, 7], 7, 3, 3),       # a length above max_seqlen
    ([0, 3, 5], 5, 1027, 3),    # max_seqlen above max positions
    ([0, 1026], 1026, 1026, 0), # the longest allowed sequence
])
def test_check_cu_seqlens(cu, T, maxlen, code):
    a, p = _i32(cu)
    st, msg = _status("esm_check_cu_seqlens", p, a.size - 1, T, maxlen, 1026)
    assert st == code, msg
    if code:
        assert msg


@pytest.mark.parametrize("sl,S,code", [([3, 0, 8], 8, 0), ([3, 9], 8, 3), ([-1], 8, 3), ([4], 1027, 3)])
def test_check_seqlens(sl, S, code):
    a, p = _i32(sl)
    st, msg = _status("esm_check_seqlens", p, a.size, S, 1026)
    assert st == code, msg


def test_check_null_pointer():
    st, msg = _status("esm_check_cu_seqlens", None, 1, 1, 1, 1026)
    assert st == 1 and "NULL" in msg


def _cfg(**kw):
    c = esm.EsmConfig()
    esm.load_library().esm_config_default(ctypes.byref(c))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_config_default_is_esm2_650m():
    c = _cfg()
    assert (c.hidden_size, c.num_attention_heads, c.intermediate_size, c.num_hidden_layers) == (1280, 20, 5120, 33)
    assert (c.vocab_size, c.max_position_embeddings, c.amax_history_len) == (33, 1026, 16)
    assert abs(c.layer_norm_eps - 1e-5) < 1e-12 and c.rope_base == 10000.0


@pytest.mark.parametrize("kw,code", [
    (dict(hidden_size=1000), 2),
    (dict(num_attention_heads=7), 2),
    (dict(num_attention_heads=10), 4),    # head_dim 128 is not built
    (dict(intermediate_size=100), 2),
    (dict(vocab_size=0), 2),
    (dict(max_position_embeddings=0), 2),
    (dict(layer_norm_eps=0.0), 2),
    (dict(precision=7), 4),
    (dict(amax_history_len=0), 2),
    (dict(amax_history_len=1025), 2),
    (dict(precision=1, hidden_size=320, num_attention_heads=5, intermediate_size=1280), 4),  # FP8 K step 128
    (dict(precision=1, intermediate_size=5120 + 64), 4),
])
def test_create_rejects_bad_config_before_touching_a_device(kw, code):
    c = _cfg(**kw)
    h = ctypes.c_void_p()
    st, msg = _status("esm_encoder_create", ctypes.byref(c), 0, ctypes.byref(h))
    assert st == code, msg
    assert not h.value


def test_fp8_calls_fail_cleanly_without_a_handle():
    st, _ = _status("esm_fp8_reset", None, None)
    assert st == 1
    st, _ = _status("esm_fp8_prepare_layer", None, 0, None, None)
    assert st == 1
    st, _ = _status("esm_fp8_get_state", None, None, None)
    assert st == 1
    st, _ = _status("esm_fp8_quantize", None, None, 4, None, None, None, None)
    assert st == 1
    st, _ = _status("esm_layernorm_e4m3_fwd", None, None, None, None, None, None, None, 4, None)
    assert st == 1
    st, _ = _status("esm_set_layer_precision", None, None, 1, None)
    assert st == 1
    st, _ = _status("esm_linear_e4m3_fwd", None, None, None, None, None, None, None, None, None, None, 1, 64, 128,
                    0, None)
    assert st == 1


def test_null_handle_calls_fail_cleanly():
    lib = esm.load_library()
    assert lib.esm_encoder_destroy(None) == 0
    n = ctypes.c_size_t()
    st, _ = _status("esm_workspace_size", None, 10, 1, ctypes.byref(n))
    assert st == 1
    st, _ = _status("esm_layer_fwd", None, None, 0, None, None, None, None, 1, 1, 1, None, 0, None)
    assert st == 1
    st, _ = _status("esm_head_fwd", None, None, None, None, None, None, None, None, 1, 1, 1, None, 0, None)
    assert st == 1


def test_missing_library_fails_loudly(tmp_path):
    import importlib
    mod = importlib.reload(esm)
    try:
        mod._lib = None
        with pytest.raises(ImportError):
            mod.load_library(str(tmp_path / "nope.so"))
    finally:
        importlib.reload(esm)


def _size(fn, *args):
    n = ctypes.c_size_t()
    st, msg = _status(fn, *args, ctypes.byref(n))
    return st, msg, n.value


def test_linear_bwd_workspace_size():
    # W^T [K, N] bf16, db partials [ceil(M / 1024), N] fp32 and the dW GEMM's
    # S fp32 slices [S, N, K] (dy and x are read in place), each region
    # rounded up to 256 bytes.  fc1's shape at T = 32293: 100 tiles of
    # 256 x 256, so S = 5 (two rounds of 250 tiles per 1/5 of the contraction).
    M, N, K = 32293, 5120, 1280
    S = 5
    up = lambda b: (b + 255) // 256 * 256
    st, msg, n = _size("esm_linear_bwd_workspace_size", ctypes.c_int64(M), N, K)
    assert st == 0, msg
    assert n == up(K * N * 2) + up(-(-M // 1024) * N * 4) + up(S * N * K * 4)
    # below 2048 rows there is one slice
    st, msg, n = _size("esm_linear_bwd_workspace_size", ctypes.c_int64(1000), 64, 64)
    assert st == 0 and n == up(64 * 64 * 2) + up(64 * 4) + up(64 * 64 * 4)
    for bad in ((M, 100, K), (M, N, 0), (-1, N, K)):
        st, msg, _ = _size("esm_linear_bwd_workspace_size", ctypes.c_int64(bad[0]), bad[1], bad[2])
        assert st == 2 and msg


def test_layernorm_bwd_workspace_size():
    # per-row mean and rstd (fp32 pairs, 256-byte rounded), then [ceil(M / 1024), 2, H] fp32
    st, msg, n = _size("esm_layernorm_bwd_workspace_size", ctypes.c_int64(32293), 1280)
    assert st == 0, msg
    assert n == (32293 * 8 + 255) // 256 * 256 + 32 * 2 * 1280 * 4
    for H in (100, 4160, 0):
        st, msg, _ = _size("esm_layernorm_bwd_workspace_size", ctypes.c_int64(10), H)
        assert st == 2 and msg


def test_backward_calls_fail_cleanly_without_a_handle():
    p = ctypes.c_void_p(16)
    assert _status("esm_attention_fwd_lse", None, p, p, p, p, 1, ctypes.c_int64(1), p, ctypes.c_size_t(0), None)[0] == 1
    assert _status("esm_attention_bwd", None, p, p, p, p, p, p, p, 1, ctypes.c_int64(1), p, ctypes.c_size_t(0),
                   None)[0] == 1
    assert _status("esm_linear_bwd", None, p, p, p, p, p, p, ctypes.c_int64(1), 64, 64, p, ctypes.c_size_t(0),
                   None)[0] == 1
    assert _status("esm_layernorm_bwd", None, p, p, p, p, p, p, ctypes.c_int64(1), p, ctypes.c_size_t(0),
                   None)[0] == 1
    assert _status("esm_gelu_bwd", None, p, p, p, ctypes.c_int64(8), None)[0] == 1
    assert _status("esm_qkv_rope_bwd", None, p, p, p, 1, ctypes.c_int64(1), p, ctypes.c_size_t(0), None)[0] == 1


def test_training_layer_calls_fail_cleanly_without_a_handle():
    p = ctypes.c_void_p(16)
    n = ctypes.c_size_t()
    off = ctypes.c_size_t()
    assert _status("esm_layer_saved_size", None, ctypes.c_int64(10), ctypes.byref(n))[0] == 1
    assert _status("esm_layer_saved_region", None, ctypes.c_int64(10), 0, ctypes.byref(off), ctypes.byref(n))[0] == 1
    assert _status("esm_layer_bwd_workspace_size", None, ctypes.c_int64(10), 1, ctypes.byref(n))[0] == 1
    w = ctypes.byref(esm.EsmLayerWeights())
    g = ctypes.byref(esm.EsmLayerGrads())
    assert _status("esm_layer_fwd_train", None, w, 0, p, p, p, None, 1, ctypes.c_int64(1), 1, p, ctypes.c_size_t(0),
                   p, ctypes.c_size_t(0), None)[0] == 1
    assert _status("esm_layer_bwd", None, w, 0, p, p, ctypes.c_size_t(0), p, p, g, p, 1, ctypes.c_int64(1), p,
                   ctypes.c_size_t(0), None)[0] == 1
    assert _status("esm_stack_saved_size", None, ctypes.c_int64(10), ctypes.byref(n))[0] == 1
    assert _status("esm_stack_saved_layer", None, ctypes.c_int64(10), 0, ctypes.byref(off), ctypes.byref(n))[0] == 1
    assert _status("esm_stack_bwd_workspace_size", None, ctypes.c_int64(10), 1, ctypes.byref(n))[0] == 1
    assert _status("esm_stack_fwd_train", None, w, None, None, p, p, p, None, 1, ctypes.c_int64(1), 1, p,
                   ctypes.c_size_t(0), p, ctypes.c_size_t(0), None)[0] == 1
    assert _status("esm_stack_bwd", None, w, p, ctypes.c_size_t(0), p, p, g, None, None, p, 1, ctypes.c_int64(1), p,
                   ctypes.c_size_t(0), None)[0] == 1


def test_e5m2_wgrad_workspace_size():
    # dy^T [N, Mp] and x^T [K, Mp] bytes (Mp: M rounded up to 128 per K slice), then [S, N, K] fp32 slices
    st, msg, n = _size("esm_linear_e5m2_wgrad_workspace_size", ctypes.c_int64(1000), 1280, 320)
    assert st == 0, msg
    assert n == 1280 * 1024 + 320 * 1024            # one slice below 2048 rows
    st, msg, n = _size("esm_linear_e5m2_wgrad_workspace_size", ctypes.c_int64(32293), 5120, 1280)
    assert st == 0, msg
    up = lambda b: (b + 255) // 256 * 256             # noqa: E731
    S = 5                                             # 100 tiles: 5 slices fill 2 rounds of 256 CUs
    Mp = (32293 + 128 * S - 1) // (128 * S) * 128 * S
    assert n == up(5120 * Mp) + up(1280 * Mp) + up(S * 5120 * 1280 * 4)
    for bad in ((10, 100, 64), (10, 64, 0), (-1, 64, 64)):
        st, msg, _ = _size("esm_linear_e5m2_wgrad_workspace_size", ctypes.c_int64(bad[0]), bad[1], bad[2])
        assert st == 2 and msg
