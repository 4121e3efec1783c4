"""Python binding of the C ABI in include/esm_encoder.h (ctypes).

Argument marshalling only: torch tensors become device pointers and the
current torch stream becomes the hipStream_t.  Every step of the forward runs
in the library's HIP kernels; there is no other code path.  If libesmenc.so is
missing, loading raises instead of falling back to anything else."""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# ESM_LIBRARY may point at another build of the same library.
LIB_PATH = os.environ.get("ESM_LIBRARY") or os.path.join(_PKG, "libesmenc.so")

ESM_OK = 0
STATUS_NAMES = {0: "ESM_OK", 1: "ESM_ERR_NULL", 2: "ESM_ERR_SHAPE", 3: "ESM_ERR_SEQLENS", 4: "ESM_ERR_UNSUPPORTED",
                5: "ESM_ERR_WORKSPACE", 6: "ESM_ERR_ARCH", 7: "ESM_ERR_HIP", 8: "ESM_ERR_STATE"}
PRECISION = {"bf16": 0, "fp8": 1, "mxfp4": 2}
LAYOUT_THD, LAYOUT_BSHD = 0, 1
EPI_BIAS, EPI_BIAS_GELU, EPI_BIAS_RESIDUAL, EPI_BIAS_GELU_E4M3 = 0, 1, 2, 3
WS_REGIONS = {"ln1": 0, "qkv": 1, "ctx": 2, "x1": 3, "ln2": 4, "act": 5, "pos": 6, "tiles": 7, "ntiles": 8, "segs": 9,
              "stats": 10}
ATTN_TILE_ROWS = 256  # ESM_ATTN_TILE_ROWS: query rows per attention workgroup
KERNEL_CLASSES = ("segment", "embed", "layernorm", "gemm_qkv", "attention", "gemm_out", "gemm_fc1", "gemm_fc2",
                  "other", "fp8", "head", "biased_attention", "attention_bwd", "linear_bwd")
FP8_ACT_NAMES = ("ln1", "ctx", "ln2", "act")      # activation tensors tracked per layer, in state order
FP8_WEIGHT_NAMES = ("w_qkv", "w_out", "w_fc1", "w_fc2")
LAYER_WEIGHT_NAMES = ("ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_out", "b_out",
                      "ln2_gamma", "ln2_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2")

# Every function the header declares, with its ctypes signature.
_i32, _i64, _p, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


class EsmConfig(ctypes.Structure):
    _fields_ = [
        ("hidden_size", ctypes.c_int32), ("num_attention_heads", ctypes.c_int32),
        ("intermediate_size", ctypes.c_int32), ("num_hidden_layers", ctypes.c_int32),
        ("vocab_size", ctypes.c_int32), ("max_position_embeddings", ctypes.c_int32),
        ("layer_norm_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
        ("precision", ctypes.c_int32), ("amax_history_len", ctypes.c_int32),
    ]


class EsmLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHT_NAMES]


HEAD_WEIGHT_NAMES = ("final_ln_gamma", "final_ln_beta", "lm_dense_w", "lm_dense_b", "lm_ln_gamma", "lm_ln_beta",
                     "lm_decoder_w", "lm_decoder_b")


class EsmHeadWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in HEAD_WEIGHT_NAMES]


class EsmLayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHT_NAMES]


SAVED_REGIONS = {"h1": 0, "qkv": 1, "ctx": 2, "lse": 3, "x1": 4, "h2": 5, "z": 6, "a": 7}


class EsmFp8State(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("history_len", ctypes.c_int32),
        ("act_scale", ctypes.c_void_p), ("amax_history", ctypes.c_void_p), ("steps", ctypes.c_void_p),
        ("weight_scale", ctypes.c_void_p), ("nonfinite", ctypes.c_uint32),
    ]


SIGNATURES = {
    "esm_config_default": (None, [ctypes.POINTER(EsmConfig)]),
    "esm_encoder_create": (_i32, [ctypes.POINTER(EsmConfig), ctypes.c_int, ctypes.POINTER(_p)]),
    "esm_encoder_destroy": (_i32, [_p]),
    "esm_workspace_size": (_i32, [_p, _i64, _i32, ctypes.POINTER(_sz)]),
    "esm_stack_split": (_i32, [_i32, _i32, _p, _i32, _i64, ctypes.POINTER(_i32)]),
    "esm_workspace_region": (_i32, [_p, _i64, _i32, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "esm_layer_fwd": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _i32, _p, _p, _p, _p, _i32, _i64, _i32, _p, _sz,
                             _p]),
    "esm_layer_fwd_noalloc": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _i32, _p, _p, _p, _p, _i32, _i64, _i32,
                                     _p]),
    "esm_head_fwd": (_i32, [_p, ctypes.POINTER(EsmHeadWeights), _p, _p, _p, _p, _p, _p, _i32, _i64, _i32, _p, _sz,
                            _p]),
    "esm_stack_fwd": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _p, _p, _p, _p, _p, _p, _i32, _i64, _i32, _p, _sz,
                             _p]),
    "esm_layer_fwd_bshd": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _i32, _p, _p, _p, _p, _i32, _i32, _p, _sz,
                                  _p]),
    "esm_stack_fwd_bshd": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _p, _p, _p, _p, _p, _p, _i32, _i32, _p, _sz,
                                  _p]),
    "esm_segment_table": (_i32, [_p, _i32, _p, _i32, _i64, _i32, _p, _sz, _p]),
    "esm_attention_fwd": (_i32, [_p, _p, _p, _p, _i32, _i64, _p, _sz, _p]),
    "esm_attention_fwd_lse": (_i32, [_p, _p, _p, _p, _p, _i32, _i64, _p, _sz, _p]),
    "esm_linear_bwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _p, _sz, _p]),
    "esm_linear_bwd_workspace_size": (_i32, [_i64, _i32, _i32, _p]),
    "esm_layernorm_bwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _i64, _p, _sz, _p]),
    "esm_layernorm_bwd_workspace_size": (_i32, [_i64, _i32, _p]),
    "esm_gelu_bwd": (_i32, [_p, _p, _p, _p, _i64, _p]),
    "esm_e5m2_quantize": (_i32, [_p, _p, _i64, _p, _p, _p, _p]),
    "esm_linear_e5m2_dgrad": (_i32, [_p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _p]),
    "esm_linear_e5m2_wgrad": (_i32, [_p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _p, _sz, _p]),
    "esm_linear_e5m2_wgrad_workspace_size": (_i32, [_i64, _i32, _i32, _p]),
    "esm_qkv_rope_bwd": (_i32, [_p, _p, _p, _p, _i32, _i64, _p, _sz, _p]),
    "esm_attention_bwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i64, _p, _sz, _p]),
    "esm_biased_attention_fwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p]),
    "esm_mxfp4_quantize": (_i32, [_p, _p, _i64, _i32, _p, _p, _p]),
    "esm_linear_mxfp4_fwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _p]),
    "esm_linear_fwd": (_i32, [_p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _p]),
    "esm_layernorm_fwd": (_i32, [_p, _p, _p, _p, _p, _i64, _p]),
    "esm_layernorm_e4m3_fwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _i64, _p]),
    "esm_linear_e4m3_fwd": (_i32, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _p]),
    "esm_prepare_layer": (_i32, [_p, _i32, ctypes.POINTER(EsmLayerWeights), _p]),
    "esm_fp8_prepare_layer": (_i32, [_p, _i32, ctypes.POINTER(EsmLayerWeights), _p]),
    "esm_mxfp4_prepare_layer": (_i32, [_p, _i32, ctypes.POINTER(EsmLayerWeights), _p]),
    "esm_fp8_get_state": (_i32, [_p, ctypes.POINTER(EsmFp8State), _p]),
    "esm_fp8_set_state": (_i32, [_p, ctypes.POINTER(EsmFp8State), _p]),
    "esm_fp8_reset": (_i32, [_p, _p]),
    "esm_fp8_grad_quantize": (_i32, [_p, _i32, _i32, _p, _i64, _p, _p, _p]),
    "esm_fp8_grad_step": (_i32, [_p, _i32, _p]),
    "esm_fp8_grad_get_state": (_i32, [_p, _p, _p, _p, _p]),
    "esm_set_layer_precision": (_i32, [_p, _p, _i32, _p]),
    "esm_fp8_quantize": (_i32, [_p, _p, _i64, _p, _p, _p, _p]),
    "esm_mfma_peak": (_i32, [_p, _i32, _p, _sz, ctypes.POINTER(ctypes.c_double), _p]),
    "esm_layer_saved_size": (_i32, [_p, _i64, ctypes.POINTER(_sz)]),
    "esm_layer_saved_region": (_i32, [_p, _i64, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "esm_layer_fwd_train": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _i32, _p, _p, _p, _p, _i32, _i64, _i32, _p,
                                   _sz, _p, _sz, _p]),
    "esm_layer_bwd_workspace_size": (_i32, [_p, _i64, _i32, ctypes.POINTER(_sz)]),
    "esm_layer_bwd": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _i32, _p, _p, _sz, _p, _p,
                             ctypes.POINTER(EsmLayerGrads), _p, _i32, _i64, _p, _sz, _p]),
    "esm_stack_saved_size": (_i32, [_p, _i64, ctypes.POINTER(_sz)]),
    "esm_stack_saved_layer": (_i32, [_p, _i64, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "esm_stack_fwd_train": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _p, _p, _p, _p, _p, _p, _i32, _i64, _i32,
                                   _p, _sz, _p, _sz, _p]),
    "esm_stack_bwd_workspace_size": (_i32, [_p, _i64, _i32, ctypes.POINTER(_sz)]),
    "esm_stack_bwd": (_i32, [_p, ctypes.POINTER(EsmLayerWeights), _p, _sz, _p, _p, ctypes.POINTER(EsmLayerGrads),
                             _p, _p, _p, _i32, _i64, _p, _sz, _p]),
    "esm_profile_enable": (_i32, [_p, _i32]),
    "esm_profile_read": (_i32, [_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "esm_check_cu_seqlens": (_i32, [_p, _i32, _i64, _i32, _i32]),
    "esm_check_seqlens": (_i32, [_p, _i32, _i32, _i32]),
    "esm_last_error": (ctypes.c_char_p, []),
    "esm_status_str": (ctypes.c_char_p, [_i32]),
    "esm_abi_version": (_i32, []),
}

_lib: Optional[ctypes.CDLL] = None


class EsmError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status
        self.fn = fn


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m protein_language_model_amd.build` "
                          "(the encoder has no other implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _call(name: str, *args) -> None:
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != ESM_OK:
        raise EsmError(name, st, lib.esm_last_error().decode())


def check_cu_seqlens(cu, T: int, max_seqlen: int, max_positions: int = 1026) -> None:
    """Host-only validation of a cu_seqlens array (raises EsmError)."""
    a = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    _call("esm_check_cu_seqlens", a.ctypes.data_as(ctypes.c_void_p), int(a.size - 1), int(T), int(max_seqlen),
          int(max_positions))


def check_seqlens(seqlens, S: int, max_positions: int = 1026) -> None:
    a = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    _call("esm_check_seqlens", a.ctypes.data_as(ctypes.c_void_p), int(a.size), int(S), int(max_positions))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def stack_split(hidden_size: int, intermediate_size: int, cu_seqlens_host) -> int:
    """The sequence index where esm_stack_fwd splits this batch into its two
    groups (0: one group); host only."""
    cu = _host_i32(cu_seqlens_host)
    out = ctypes.c_int32()
    _call("esm_stack_split", int(hidden_size), int(intermediate_size), cu.ctypes.data_as(ctypes.c_void_p),
          int(cu.size - 1), int(cu[-1]), ctypes.byref(out))
    return int(out.value)


def _host_i32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    import torch
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def layer_weights_struct(w: Dict[str, "object"]) -> EsmLayerWeights:
    s = EsmLayerWeights()
    for n in LAYER_WEIGHT_NAMES:
        t = w.get(n)
        setattr(s, n, _ptr(t) if t is not None else None)
    return s


class Encoder:
    """Handle of the C library (esm_encoder_create / esm_encoder_destroy)."""

    def __init__(self, hidden_size: int = 1280, num_attention_heads: int = 20, intermediate_size: int = 5120,
                 num_hidden_layers: int = 33, vocab_size: int = 33, max_position_embeddings: int = 1026,
                 layer_norm_eps: float = 1e-5, rope_base: float = 10000.0, precision: str = "bf16",
                 amax_history_len: int = 16, device: int = 0):
        lib = load_library()
        cfg = EsmConfig()
        lib.esm_config_default(ctypes.byref(cfg))
        cfg.hidden_size, cfg.num_attention_heads = hidden_size, num_attention_heads
        cfg.intermediate_size, cfg.num_hidden_layers = intermediate_size, num_hidden_layers
        cfg.vocab_size, cfg.max_position_embeddings = vocab_size, max_position_embeddings
        cfg.layer_norm_eps, cfg.rope_base = layer_norm_eps, rope_base
        cfg.precision, cfg.amax_history_len = PRECISION[precision], amax_history_len
        self.cfg = cfg
        self.device = device
        h = ctypes.c_void_p()
        _call("esm_encoder_create", ctypes.byref(cfg), device, ctypes.byref(h))
        self._h = h

    # -- lifetime
    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            load_library().esm_encoder_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def hidden(self) -> int:
        return self.cfg.hidden_size

    # -- workspace
    def workspace_size(self, max_tokens: int, max_seqs: int) -> int:
        n = ctypes.c_size_t()
        _call("esm_workspace_size", self._h, int(max_tokens), int(max_seqs), ctypes.byref(n))
        return n.value

    def workspace(self, max_tokens: int, max_seqs: int):
        import torch
        n = self.workspace_size(max_tokens, max_seqs)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=f"cuda:{self.device}")
        assert ws.data_ptr() % 256 == 0
        return ws

    def workspace_region(self, ws, max_tokens: int, max_seqs: int, name: str):
        """A view of one named region of a workspace used by a call with (T, B)."""
        import torch
        off, nb = ctypes.c_size_t(), ctypes.c_size_t()
        _call("esm_workspace_region", self._h, int(max_tokens), int(max_seqs), WS_REGIONS[name], ctypes.byref(off),
              ctypes.byref(nb))
        raw = ws[off.value: off.value + nb.value]
        if name in ("pos", "tiles", "ntiles", "segs"):
            return raw.view(torch.int32)
        if name == "stats":
            return raw.view(torch.float32)
        if self.cfg.precision == PRECISION["fp8"] and name in ("ln1", "ctx", "ln2", "act"):
            return raw  # E4M3 codes, row-major with the bf16 row count
        return raw.view(torch.bfloat16)

    # -- forward
    def layer_fwd(self, weights, x_in, cu_seqlens, B: int, T: int, max_seqlen: int, *, x_out=None,
                  layer_idx: int = 0, cu_seqlens_host=None, workspace=None, stream=None):
        import torch
        if x_out is None:
            x_out = torch.empty_like(x_in)
        if workspace is None:
            workspace = self.workspace(T, B)
        w = layer_weights_struct(weights)
        cuh = _host_i32(cu_seqlens_host)
        _call("esm_layer_fwd", self._h, ctypes.byref(w), int(layer_idx), _ptr(x_in), _ptr(x_out), _ptr(cu_seqlens),
              cuh.ctypes.data_as(ctypes.c_void_p) if cuh is not None else None, int(B), int(T), int(max_seqlen),
              _ptr(workspace), workspace.numel(), _stream(stream))
        return x_out

    # -- training layer
    def saved_size(self, T: int) -> int:
        n = ctypes.c_size_t()
        _call("esm_layer_saved_size", self._h, int(T), ctypes.byref(n))
        return int(n.value)

    def saved_region(self, saved, T: int, name: str):
        """A view of one region of a layer's saved activations (esm_saved_region)."""
        import torch
        off, nb = ctypes.c_size_t(), ctypes.c_size_t()
        _call("esm_layer_saved_region", self._h, int(T), SAVED_REGIONS[name], ctypes.byref(off), ctypes.byref(nb))
        raw = saved[off.value: off.value + nb.value]
        return raw.view(torch.float32) if name == "lse" else raw.view(torch.bfloat16)

    def layer_fwd_train(self, weights, x_in, cu_seqlens, B: int, T: int, max_seqlen: int, *, x_out=None,
                        saved=None, layer_idx: int = 0, cu_seqlens_host=None, workspace=None, stream=None):
        """esm_layer_fwd_train: returns (x_out, saved), saved a uint8 device
        buffer holding the activations the layer's backward takes."""
        import torch
        if x_out is None:
            x_out = torch.empty_like(x_in)
        if saved is None:
            saved = torch.empty((max(self.saved_size(T), 256),), dtype=torch.uint8, device=x_in.device)
        if workspace is None:
            workspace = self.workspace(T, B)
        w = layer_weights_struct(weights)
        cuh = _host_i32(cu_seqlens_host)
        _call("esm_layer_fwd_train", self._h, ctypes.byref(w), int(layer_idx), _ptr(x_in), _ptr(x_out),
              _ptr(cu_seqlens), cuh.ctypes.data_as(ctypes.c_void_p) if cuh is not None else None, int(B), int(T),
              int(max_seqlen), _ptr(saved), saved.numel(), _ptr(workspace), workspace.numel(), _stream(stream))
        return x_out, saved

    def layer_bwd_workspace(self, T: int, B: int):
        import torch
        n = ctypes.c_size_t()
        _call("esm_layer_bwd_workspace_size", self._h, int(T), int(B), ctypes.byref(n))
        return torch.empty((max(int(n.value), 256),), dtype=torch.uint8, device=f"cuda:{self.device}")

    def layer_bwd(self, weights, x_in, saved, dy, cu_seqlens, B: int, T: int, *, dx=None, grads=None,
                  layer_idx: int = 0, workspace=None, stream=None):
        """esm_layer_bwd: returns (dx [T, H] bf16, grads), grads a dict of the 12
        parameter gradients (weights bf16, biases and LayerNorm vectors fp32)."""
        import torch
        H, F, dev = self.cfg.hidden_size, self.cfg.intermediate_size, dy.device
        if dx is None:
            dx = torch.empty_like(dy)
        if grads is None:
            grads = self._grad_tensors(dev)
        if workspace is None:
            workspace = self.layer_bwd_workspace(T, B)
        w = layer_weights_struct(weights)
        g = EsmLayerGrads()
        for n in LAYER_WEIGHT_NAMES:
            setattr(g, n, _ptr(grads[n]))
        _call("esm_layer_bwd", self._h, ctypes.byref(w), int(layer_idx), _ptr(x_in), _ptr(saved), saved.numel(),
              _ptr(dy), _ptr(dx), ctypes.byref(g), _ptr(cu_seqlens), int(B), int(T), _ptr(workspace),
              workspace.numel(), _stream(stream))
        return dx, grads

    def _grad_tensors(self, dev):
        import torch
        H, F = self.cfg.hidden_size, self.cfg.intermediate_size
        shapes = {"ln1_gamma": (H,), "ln1_beta": (H,), "w_qkv": (3 * H, H), "b_qkv": (3 * H,), "w_out": (H, H),
                  "b_out": (H,), "ln2_gamma": (H,), "ln2_beta": (H,), "w_fc1": (F, H), "b_fc1": (F,),
                  "w_fc2": (H, F), "b_fc2": (H,)}
        return {n: torch.empty(sh, dtype=torch.bfloat16 if n.startswith("w_") else torch.float32, device=dev)
                for n, sh in shapes.items()}

    def stack_saved_size(self, T: int) -> int:
        n = ctypes.c_size_t()
        _call("esm_stack_saved_size", self._h, int(T), ctypes.byref(n))
        return int(n.value)

    def stack_saved_layer(self, saved, T: int, l: int, name: str = None):
        """Layer l's input X_l (name None, bf16 [T, H]) or one of its saved
        regions (a name of SAVED_REGIONS, as saved_region returns it) inside
        esm_stack_fwd_train's buffer."""
        xo, so = ctypes.c_size_t(), ctypes.c_size_t()
        _call("esm_stack_saved_layer", self._h, int(T), int(l), ctypes.byref(xo), ctypes.byref(so))
        if name is None:
            n = int(T) * self.hidden * 2
            return saved[xo.value:xo.value + n].view(__import__("torch").bfloat16).view(int(T), self.hidden)
        return self.saved_region(saved[so.value:], T, name)

    def stack_fwd_train(self, weights: Sequence[Dict], cu_seqlens, B: int, T: int, max_seqlen: int, *,
                        token_ids=None, embedding=None, x_in=None, x_out=None, saved=None, cu_seqlens_host=None,
                        workspace=None, stream=None):
        """esm_stack_fwd_train: returns (x_out, saved)."""
        import torch
        if len(weights) != self.cfg.num_hidden_layers:
            raise ValueError(f"{len(weights)} layer weight sets for {self.cfg.num_hidden_layers} layers")
        dev = f"cuda:{self.device}"
        if x_out is None:
            x_out = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=dev)
        if saved is None:
            saved = torch.empty((max(self.stack_saved_size(T), 256),), dtype=torch.uint8, device=dev)
        if workspace is None:
            workspace = self.workspace(T, B)
        arr = (EsmLayerWeights * len(weights))(*[layer_weights_struct(w) for w in weights])
        cuh = _host_i32(cu_seqlens_host)
        _call("esm_stack_fwd_train", self._h, arr, _ptr(token_ids), _ptr(embedding), _ptr(x_in), _ptr(x_out),
              _ptr(cu_seqlens), cuh.ctypes.data_as(ctypes.c_void_p) if cuh is not None else None, int(B), int(T),
              int(max_seqlen), _ptr(saved), saved.numel(), _ptr(workspace), workspace.numel(), _stream(stream))
        return x_out, saved

    def stack_bwd_workspace(self, T: int, B: int):
        import torch
        n = ctypes.c_size_t()
        _call("esm_stack_bwd_workspace_size", self._h, int(T), int(B), ctypes.byref(n))
        return torch.empty((max(int(n.value), 256),), dtype=torch.uint8, device=f"cuda:{self.device}")

    def stack_bwd(self, weights: Sequence[Dict], saved, dy, cu_seqlens, B: int, T: int, *, dx=None, grads=None,
                  token_ids=None, d_embedding=None, workspace=None, stream=None):
        """esm_stack_bwd: returns (dx, [per-layer gradient dicts], d_embedding
        fp32 [vocab, H] or None); d_embedding is allocated when token_ids are
        given and it is not."""
        import torch
        L = self.cfg.num_hidden_layers
        if len(weights) != L:
            raise ValueError(f"{len(weights)} layer weight sets for {L} layers")
        if dx is None:
            dx = torch.empty_like(dy)
        if grads is None:
            grads = [self._grad_tensors(dy.device) for _ in range(L)]
        if token_ids is not None and d_embedding is None:
            d_embedding = torch.empty((self.cfg.vocab_size, self.hidden), dtype=torch.float32, device=dy.device)
        if workspace is None:
            workspace = self.stack_bwd_workspace(T, B)
        arr = (EsmLayerWeights * L)(*[layer_weights_struct(w) for w in weights])
        garr = (EsmLayerGrads * L)()
        for l in range(L):
            for n in LAYER_WEIGHT_NAMES:
                setattr(garr[l], n, _ptr(grads[l][n]))
        _call("esm_stack_bwd", self._h, arr, _ptr(saved), saved.numel(), _ptr(dy), _ptr(dx), garr, _ptr(token_ids),
              _ptr(d_embedding), _ptr(cu_seqlens), int(B), int(T), _ptr(workspace), workspace.numel(),
              _stream(stream))
        return dx, grads, d_embedding

    def layer_fwd_noalloc(self, weights, x_in, cu_seqlens, B: int, T: int, max_seqlen: int, *, x_out,
                          layer_idx: int = 0, cu_seqlens_host=None, stream=None):
        """esm_layer_fwd_noalloc: the caller passes the output; no workspace."""
        w = layer_weights_struct(weights)
        cuh = _host_i32(cu_seqlens_host)
        _call("esm_layer_fwd_noalloc", self._h, ctypes.byref(w), int(layer_idx), _ptr(x_in), _ptr(x_out),
              _ptr(cu_seqlens), cuh.ctypes.data_as(ctypes.c_void_p) if cuh is not None else None, int(B), int(T),
              int(max_seqlen), _stream(stream))
        return x_out

    def stack_fwd(self, weights: Sequence[Dict], cu_seqlens, B: int, T: int, max_seqlen: int, *, token_ids=None,
                  embedding=None, x_in=None, x_out=None, cu_seqlens_host=None, workspace=None, stream=None):
        import torch
        if len(weights) != self.cfg.num_hidden_layers:
            raise ValueError(f"{len(weights)} layer weight sets for {self.cfg.num_hidden_layers} layers")
        if x_out is None:
            x_out = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=f"cuda:{self.device}")
        if workspace is None:
            workspace = self.workspace(T, B)
        arr = (EsmLayerWeights * max(len(weights), 1))(*[layer_weights_struct(w) for w in weights])
        cuh = _host_i32(cu_seqlens_host)
        _call("esm_stack_fwd", self._h, arr, _ptr(token_ids), _ptr(embedding), _ptr(x_in), _ptr(x_out),
              _ptr(cu_seqlens), cuh.ctypes.data_as(ctypes.c_void_p) if cuh is not None else None, int(B), int(T),
              int(max_seqlen), _ptr(workspace), workspace.numel(), _stream(stream))
        return x_out

    def head_fwd(self, head_weights: Dict, x, cu_seqlens, B: int, T: int, max_seqlen: int, *, x_final=None,
                 logits=True, seq_emb=True, cu_seqlens_host=None, workspace=None, stream=None):
        """Final LayerNorm, masked-LM logits and per-sequence mean embeddings of
        the stack output x [T, H]; returns (x_final, logits or None, seq_emb or None).
        logits / seq_emb: True to allocate, a tensor to fill, or None / False to skip."""
        import torch
        dev = f"cuda:{self.device}"
        if x_final is None:
            x_final = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=dev)
        if logits is True:
            logits = torch.empty((T, self.cfg.vocab_size), dtype=torch.bfloat16, device=dev)
        if seq_emb is True:
            seq_emb = torch.empty((B, self.hidden), dtype=torch.float32, device=dev)
        logits = logits if logits is not False else None
        seq_emb = seq_emb if seq_emb is not False else None
        if workspace is None:
            workspace = self.workspace(T, B)
        hw = EsmHeadWeights()
        for n in HEAD_WEIGHT_NAMES:
            t = head_weights.get(n)
            setattr(hw, n, _ptr(t) if t is not None else None)
        cuh = _host_i32(cu_seqlens_host)
        _call("esm_head_fwd", self._h, ctypes.byref(hw), _ptr(x), _ptr(x_final), _ptr(logits), _ptr(seq_emb),
              _ptr(cu_seqlens), cuh.ctypes.data_as(ctypes.c_void_p) if cuh is not None else None, int(B), int(T),
              int(max_seqlen), _ptr(workspace), workspace.numel(), _stream(stream))
        return x_final, logits, seq_emb

    def layer_fwd_bshd(self, weights, x_in, seqlens, B: int, S: int, *, x_out=None, layer_idx: int = 0,
                       seqlens_host=None, workspace=None, stream=None):
        import torch
        if x_out is None:
            x_out = torch.empty_like(x_in)
        if workspace is None:
            workspace = self.workspace(B * S, B)
        w = layer_weights_struct(weights)
        slh = _host_i32(seqlens_host)
        _call("esm_layer_fwd_bshd", self._h, ctypes.byref(w), int(layer_idx), _ptr(x_in), _ptr(x_out), _ptr(seqlens),
              slh.ctypes.data_as(ctypes.c_void_p) if slh is not None else None, int(B), int(S), _ptr(workspace),
              workspace.numel(), _stream(stream))
        return x_out

    def stack_fwd_bshd(self, weights: Sequence[Dict], seqlens, B: int, S: int, *, token_ids=None, embedding=None,
                       x_in=None, x_out=None, seqlens_host=None, workspace=None, stream=None):
        import torch
        if len(weights) != self.cfg.num_hidden_layers:
            raise ValueError(f"{len(weights)} layer weight sets for {self.cfg.num_hidden_layers} layers")
        if x_out is None:
            x_out = torch.empty((B, S, self.hidden), dtype=torch.bfloat16, device=f"cuda:{self.device}")
        if workspace is None:
            workspace = self.workspace(B * S, B)
        arr = (EsmLayerWeights * max(len(weights), 1))(*[layer_weights_struct(w) for w in weights])
        slh = _host_i32(seqlens_host)
        _call("esm_stack_fwd_bshd", self._h, arr, _ptr(token_ids), _ptr(embedding), _ptr(x_in), _ptr(x_out),
              _ptr(seqlens), slh.ctypes.data_as(ctypes.c_void_p) if slh is not None else None, int(B), int(S),
              _ptr(workspace), workspace.numel(), _stream(stream))
        return x_out

    # -- kernel-level entries
    def segment_table(self, layout: int, lens, B: int, T: int, S: int = 0, *, workspace=None, stream=None):
        if workspace is None:
            workspace = self.workspace(T if layout == LAYOUT_THD else B * S, B)
        _call("esm_segment_table", self._h, int(layout), _ptr(lens), int(B), int(T), int(S), _ptr(workspace),
              workspace.numel(), _stream(stream))
        return workspace

    def attention_fwd(self, qkv, cu_seqlens, B: int, T: int, *, ctx=None, workspace=None, stream=None):
        import torch
        if ctx is None:
            ctx = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=qkv.device)
        if workspace is None:
            workspace = self.workspace(T, B)
        _call("esm_attention_fwd", self._h, _ptr(qkv), _ptr(ctx), _ptr(cu_seqlens), int(B), int(T), _ptr(workspace),
              workspace.numel(), _stream(stream))
        return ctx

    def attention_fwd_lse(self, qkv, cu_seqlens, B: int, T: int, *, ctx=None, lse=None, workspace=None,
                          stream=None):
        """(ctx [T, H] bf16, lse [heads, T] fp32): the attention and its softmax
        normaliser log sum_j exp(q.k_j / 8), for a backward pass."""
        import torch
        if ctx is None:
            ctx = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=qkv.device)
        if lse is None:
            lse = torch.empty((self.cfg.num_attention_heads, T), dtype=torch.float32, device=qkv.device)
        if workspace is None:
            workspace = self.workspace(T, B)
        _call("esm_attention_fwd_lse", self._h, _ptr(qkv), _ptr(ctx), _ptr(lse), _ptr(cu_seqlens), int(B), int(T),
              _ptr(workspace), workspace.numel(), _stream(stream))
        return ctx, lse

    def attention_bwd(self, qkv, ctx, dctx, lse, cu_seqlens, B: int, T: int, *, dqkv=None, delta=None,
                      workspace=None, stream=None):
        """dqkv [3, heads, T, 64] bf16: gradients of the attention with respect
        to q, k, v for the context gradient dctx [T, H]; ctx and lse are the
        forward's (attention_fwd_lse).  delta [heads, T] fp32 is scratch."""
        import torch
        if dqkv is None:
            dqkv = torch.empty_like(qkv)
        if delta is None:
            delta = torch.empty((self.cfg.num_attention_heads, T), dtype=torch.float32, device=qkv.device)
        if workspace is None:
            workspace = self.workspace(T, B)
        _call("esm_attention_bwd", self._h, _ptr(qkv), _ptr(ctx), _ptr(dctx), _ptr(lse), _ptr(delta), _ptr(dqkv),
              _ptr(cu_seqlens), int(B), int(T), _ptr(workspace), workspace.numel(), _stream(stream))
        return dqkv

    def layernorm_bwd(self, x, gamma, dy, *, dx=None, dgamma=None, dbeta=None, workspace=None, stream=None):
        """Backward of the LayerNorm (gamma, beta over hidden_size): returns
        (dx [M, H] bf16, dgamma [H] fp32, dbeta [H] fp32)."""
        import torch
        M, H = x.shape
        dev = x.device
        if dx is None:
            dx = torch.empty_like(x)
        if dgamma is None:
            dgamma = torch.empty((H,), dtype=torch.float32, device=dev)
        if dbeta is None:
            dbeta = torch.empty((H,), dtype=torch.float32, device=dev)
        if workspace is None:
            n = ctypes.c_size_t()
            _call("esm_layernorm_bwd_workspace_size", int(M), int(H), ctypes.byref(n))
            workspace = torch.empty((max(int(n.value), 1),), dtype=torch.uint8, device=dev)
        _call("esm_layernorm_bwd", self._h, _ptr(x), _ptr(gamma), _ptr(dy), _ptr(dx), _ptr(dgamma), _ptr(dbeta),
              int(M), _ptr(workspace), workspace.numel(), _stream(stream))
        return dx, dgamma, dbeta

    def e5m2_quantize(self, x, scale, *, y8=None, amax=None, stream=None):
        """(y8 uint8 codes of cast_e5m2(x * scale[0]), amax fp32-bits int32 [1]) for bf16 x."""
        import torch
        if y8 is None:
            y8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if amax is None:
            amax = torch.zeros((1,), dtype=torch.int32, device=x.device)
        _call("esm_e5m2_quantize", self._h, _ptr(x), int(x.numel()), _ptr(scale), _ptr(y8), _ptr(amax),
              _stream(stream))
        return y8, amax

    def linear_e5m2_dgrad(self, dy8, dy_scale, wt8, w_scale, *, dx=None, stream=None):
        """dx [M, K] bf16 = (dy8 / dy_scale) (wt8 / w_scale)^T with dy8 E5M2 [M, N], wt8 E4M3 [K, N]."""
        import torch
        M, N = dy8.shape
        K = wt8.shape[0]
        if dx is None:
            dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy8.device)
        _call("esm_linear_e5m2_dgrad", self._h, _ptr(dy8), _ptr(dy_scale), _ptr(wt8), _ptr(w_scale), _ptr(dx),
              int(M), int(N), int(K), _stream(stream))
        return dx

    def linear_e5m2_wgrad(self, dy8, dy_scale, x8, x_scale, *, dw=None, workspace=None, stream=None):
        """dW [N, K] bf16 = (dy8 / dy_scale)^T (x8 / x_scale) with dy8 E5M2 [M, N], x8 E4M3 [M, K]."""
        import torch
        M, N = dy8.shape
        K = x8.shape[1]
        if dw is None:
            dw = torch.empty((N, K), dtype=torch.bfloat16, device=dy8.device)
        if workspace is None:
            n = ctypes.c_size_t()
            _call("esm_linear_e5m2_wgrad_workspace_size", int(M), int(N), int(K), ctypes.byref(n))
            workspace = torch.empty((max(int(n.value), 256),), dtype=torch.uint8, device=dy8.device)
        _call("esm_linear_e5m2_wgrad", self._h, _ptr(dy8), _ptr(dy_scale), _ptr(x8), _ptr(x_scale), _ptr(dw),
              int(M), int(N), int(K), _ptr(workspace), workspace.numel(), _stream(stream))
        return dw

    def gelu_bwd(self, z, dy, *, dz=None, stream=None):
        """dz = dy * GELU'(z) (bf16, same shape; the element count a multiple of 8)."""
        import torch
        if dz is None:
            dz = torch.empty_like(dy)
        _call("esm_gelu_bwd", self._h, _ptr(z), _ptr(dy), _ptr(dz), int(z.numel()), _stream(stream))
        return dz

    def qkv_rope_bwd(self, dqkv, cu_seqlens, B: int, T: int, *, dy=None, workspace=None, stream=None):
        """dy [T, 3H] (the fused QKV linear's output gradient, interleaved
        columns) from the planar dqkv [3, heads, T, 64] of esm_attention_bwd."""
        import torch
        if dy is None:
            dy = torch.empty((T, 3 * self.hidden), dtype=torch.bfloat16, device=dqkv.device)
        if workspace is None:
            workspace = self.workspace(T, B)
        _call("esm_qkv_rope_bwd", self._h, _ptr(dqkv), _ptr(dy), _ptr(cu_seqlens), int(B), int(T), _ptr(workspace),
              workspace.numel(), _stream(stream))
        return dy

    @staticmethod
    def linear_bwd_workspace_size(M: int, N: int, K: int) -> int:
        n = ctypes.c_size_t()
        _call("esm_linear_bwd_workspace_size", int(M), int(N), int(K), ctypes.byref(n))
        return int(n.value)

    def linear_bwd(self, x, w, dy, *, dx=True, dw=True, db=True, workspace=None, stream=None):
        """Backward of y = x W^T + b: returns (dx [M, K] bf16, dW [N, K] bf16,
        db [N] fp32); pass dx/dw/db=False to skip one, or a tensor to write into."""
        import torch
        M, N = dy.shape
        K = w.shape[1] if w is not None else x.shape[1]
        dev = dy.device
        if dx is True:
            dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        if dw is True:
            dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        if db is True:
            db = torch.empty((N,), dtype=torch.float32, device=dev)
        dx, dw, db = (t if t is not False else None for t in (dx, dw, db))
        if workspace is None:
            workspace = torch.empty((self.linear_bwd_workspace_size(M, N, K),), dtype=torch.uint8, device=dev)
        _call("esm_linear_bwd", self._h, _ptr(x), _ptr(w), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(db), int(M), int(N),
              int(K), _ptr(workspace), workspace.numel(), _stream(stream))
        return dx, dw, db

    def biased_attention_fwd(self, q, k, v, mask_bias=None, pair_bias=None, *, out=None, stream=None):
        """out = softmax(q k^T / 8 + mask_bias + pair_bias) v per (b, n, h) on
        q, k, v [B, N, L, heads, 64]; mask_bias [B, N, 1, 1, L] (or [B, N, L]),
        pair_bias [B, 1, heads, L, L] (or [B, heads, L, L]), both optional."""
        import torch
        if q.dim() != 5 or q.shape[-1] != 64 or k.shape != q.shape or v.shape != q.shape:
            raise ValueError("q, k, v must be [B, N, L, heads, 64] of one shape")
        B, N, L, heads, _ = q.shape
        if mask_bias is not None and mask_bias.numel() != B * N * L:
            raise ValueError("mask_bias must be [B, N, 1, 1, L]")
        if pair_bias is not None and pair_bias.numel() != B * heads * L * L:
            raise ValueError("pair_bias must be [B, 1, heads, L, L]")
        for t in (q, k, v, mask_bias, pair_bias):
            if t is not None and t.dtype != torch.bfloat16:
                raise TypeError("biased attention takes bf16 tensors")
        if out is None:
            out = torch.empty_like(q)
        _call("esm_biased_attention_fwd", self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(mask_bias), _ptr(pair_bias),
              _ptr(out), int(B), int(N), int(L), int(heads), _stream(stream))
        return out

    def mxfp4_quantize(self, x, *, codes=None, scales=None, stream=None):
        """x bf16 [M, K] -> (codes uint8 [M, K/2], scales uint8 [K/256, M2, 8]), the
        MXFP4 layout of esm_mxfp4_quantize (M2 = M rounded up to even)."""
        import torch
        M, K = x.shape
        M2 = M + (M & 1)
        if codes is None:
            codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        if scales is None:
            scales = torch.empty((K // 256, M2, 8), dtype=torch.uint8, device=x.device)
        _call("esm_mxfp4_quantize", self._h, _ptr(x), int(M), int(K), _ptr(codes), _ptr(scales), _stream(stream))
        return codes, scales

    def linear_mxfp4_fwd(self, xq, wq, b=None, *, residual=None, epilogue: int = EPI_BIAS, y=None, stream=None):
        """MXFP4 GEMM: xq = (codes [M, K/2], scales) and wq likewise, as returned
        by mxfp4_quantize; y bf16 [M, N]."""
        import torch
        (xc, xs), (wc, ws) = xq, wq
        M, K = xc.shape[0], 2 * xc.shape[1]
        N = wc.shape[0]
        if y is None:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=xc.device)
        _call("esm_linear_mxfp4_fwd", self._h, _ptr(xc), _ptr(xs), _ptr(wc), _ptr(ws), _ptr(b), _ptr(residual),
              _ptr(y), int(M), int(N), int(K), int(epilogue), _stream(stream))
        return y

    def linear_fwd(self, x, w, b=None, *, residual=None, epilogue: int = EPI_BIAS, y=None, stream=None):
        import torch
        M, K = x.shape
        N = w.shape[0]
        if y is None:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        _call("esm_linear_fwd", self._h, _ptr(x), _ptr(w), _ptr(b), _ptr(residual), _ptr(y), int(M), int(N), int(K),
              int(epilogue), _stream(stream))
        return y

    def layernorm_fwd(self, x, gamma, beta, *, y=None, stream=None):
        import torch
        if y is None:
            y = torch.empty_like(x)
        _call("esm_layernorm_fwd", self._h, _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), int(x.shape[0]),
              _stream(stream))
        return y

    def layernorm_e4m3_fwd(self, x, gamma, beta, scale, *, y8=None, amax=None, stream=None):
        """LayerNorm of bf16 x [M, H] cast to E4M3 codes with scale[0]; returns (codes, amax tensor)."""
        import torch
        if y8 is None:
            y8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if amax is None:
            amax = torch.zeros(1, dtype=torch.int32, device=x.device)
        _call("esm_layernorm_e4m3_fwd", self._h, _ptr(x), _ptr(gamma), _ptr(beta), _ptr(scale), _ptr(y8),
              _ptr(amax), int(x.shape[0]), _stream(stream))
        return y8, amax

    def linear_e4m3_fwd(self, x8, x_scale, w8, w_scale, b=None, *, residual=None, epilogue: int = EPI_BIAS, y=None,
                        y_scale=None, y_amax=None, stream=None):
        """E4M3 GEMM: x8 [M, K] and w8 [N, K] uint8 codes, scales as device float32[1] tensors."""
        import torch
        M, K = x8.shape
        N = w8.shape[0]
        if y is None:
            dt = torch.uint8 if epilogue == EPI_BIAS_GELU_E4M3 else torch.bfloat16
            y = torch.empty((M, N), dtype=dt, device=x8.device)
        _call("esm_linear_e4m3_fwd", self._h, _ptr(x8), _ptr(x_scale), _ptr(w8), _ptr(w_scale), _ptr(b),
              _ptr(residual), _ptr(y), _ptr(y_scale), _ptr(y_amax), int(M), int(N), int(K), int(epilogue),
              _stream(stream))
        return y

    # -- FP8 delayed scaling
    def prepare_layer(self, layer_idx: int, weights, stream=None) -> None:
        w = layer_weights_struct(weights)
        _call("esm_prepare_layer", self._h, int(layer_idx), ctypes.byref(w), _stream(stream))

    def prepare(self, weights: Sequence[Dict], stream=None) -> None:
        for l, w in enumerate(weights):
            self.prepare_layer(l, w, stream)

    def fp8_prepare_layer(self, layer_idx: int, weights, stream=None) -> None:
        w = layer_weights_struct(weights)
        _call("esm_fp8_prepare_layer", self._h, int(layer_idx), ctypes.byref(w), _stream(stream))

    def fp8_prepare(self, weights: Sequence[Dict], stream=None) -> None:
        for l, w in enumerate(weights):
            self.fp8_prepare_layer(l, w, stream)

    # -- MXFP4 (the FP4 recipe)
    def mxfp4_prepare_layer(self, layer_idx: int, weights, stream=None) -> None:
        w = layer_weights_struct(weights)
        _call("esm_mxfp4_prepare_layer", self._h, int(layer_idx), ctypes.byref(w), _stream(stream))

    def mxfp4_prepare(self, weights: Sequence[Dict], stream=None) -> None:
        for l, w in enumerate(weights):
            self.mxfp4_prepare_layer(l, w, stream)

    def fp8_get_state(self, stream=None) -> Dict[str, np.ndarray]:
        L, HL = self.cfg.num_hidden_layers, self.cfg.amax_history_len
        out = {"act_scale": np.zeros((L, 4), np.float32), "amax_history": np.zeros((L, 4, HL), np.float32),
               "steps": np.zeros(L, np.int64), "weight_scale": np.zeros((L, 4), np.float32)}
        st = EsmFp8State(num_layers=L, history_len=HL)
        for k, a in out.items():
            setattr(st, k, a.ctypes.data_as(ctypes.c_void_p))
        _call("esm_fp8_get_state", self._h, ctypes.byref(st), _stream(stream))
        out["nonfinite"] = bool(st.nonfinite)
        return out

    def fp8_set_state(self, state: Dict, stream=None) -> None:
        L, HL = self.cfg.num_hidden_layers, self.cfg.amax_history_len
        arrs = {"act_scale": np.ascontiguousarray(state["act_scale"], np.float32).reshape(L, 4),
                "amax_history": np.ascontiguousarray(state["amax_history"], np.float32).reshape(L, 4, HL),
                "steps": np.ascontiguousarray(state["steps"], np.int64).reshape(L),
                "weight_scale": np.zeros((L, 4), np.float32)}
        st = EsmFp8State(num_layers=L, history_len=HL, nonfinite=1 if state.get("nonfinite") else 0)
        for k, a in arrs.items():
            setattr(st, k, a.ctypes.data_as(ctypes.c_void_p))
        _call("esm_fp8_set_state", self._h, ctypes.byref(st), _stream(stream))

    def fp8_reset(self, stream=None) -> None:
        _call("esm_fp8_reset", self._h, _stream(stream))

    def fp8_grad_quantize(self, layer_idx: int, slot: int, g, *, y8=None, scale_out=None, stream=None):
        """E5M2 codes of a gradient (bf16 g) with the slot's delayed scale;
        returns (y8 uint8, scale_out fp32 [1] on the device: the scale used)."""
        import torch
        if y8 is None:
            y8 = torch.empty(g.shape, dtype=torch.uint8, device=g.device)
        if scale_out is None:
            scale_out = torch.empty((1,), dtype=torch.float32, device=g.device)
        _call("esm_fp8_grad_quantize", self._h, int(layer_idx), int(slot), _ptr(g), g.numel(), _ptr(y8),
              _ptr(scale_out), _stream(stream))
        return y8, scale_out

    def fp8_grad_step(self, layer_idx: int, stream=None) -> None:
        _call("esm_fp8_grad_step", self._h, int(layer_idx), _stream(stream))

    def fp8_grad_get_state(self, stream=None) -> Dict[str, np.ndarray]:
        L, HL = self.cfg.num_hidden_layers, self.cfg.amax_history_len
        scale = np.zeros((L, 4), np.float32)
        hist = np.zeros((L, 4, HL), np.float32)
        steps = np.zeros((L,), np.int64)
        _call("esm_fp8_grad_get_state", self._h, scale.ctypes.data_as(ctypes.c_void_p),
              hist.ctypes.data_as(ctypes.c_void_p), steps.ctypes.data_as(ctypes.c_void_p), _stream(stream))
        return {"scale": scale, "history": hist, "steps": steps}

    def set_layer_precision(self, precisions: Sequence[str], stream=None) -> None:
        """Per-layer precision of an FP8 or MXFP4 encoder: "fp8", "mxfp4" or "bf16"
        for every layer, in any mix."""
        arr = np.ascontiguousarray(np.array([PRECISION[p] for p in precisions], np.int32))
        _call("esm_set_layer_precision", self._h, arr.ctypes.data_as(ctypes.c_void_p), len(arr), _stream(stream))

    def fp8_quantize(self, x, scale, *, y=None, amax=None, stream=None):
        """E4M3 codes of x * scale[0] (x float32 on the device); returns (codes, amax tensor)."""
        import torch
        if y is None:
            y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if amax is None:
            amax = torch.zeros(1, dtype=torch.int32, device=x.device)
        _call("esm_fp8_quantize", self._h, _ptr(x), int(x.numel()), _ptr(scale), _ptr(y), _ptr(amax),
              _stream(stream))
        return y, amax

    # -- timing
    def mfma_peak(self, iters: int, sink, stream=None) -> float:
        """Launch the matrix-core rate probe; returns its flop count."""
        fl = ctypes.c_double(0.0)
        _call("esm_mfma_peak", self._h, int(iters), _ptr(sink), sink.numel() * sink.element_size(),
              ctypes.byref(fl), _stream(stream))
        return fl.value

    def profile_enable(self, on: bool = True) -> None:
        _call("esm_profile_enable", self._h, 1 if on else 0)

    def profile_read(self) -> Dict[str, tuple]:
        n = len(KERNEL_CLASSES)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _call("esm_profile_read", self._h, ms, cnt)
        return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}
