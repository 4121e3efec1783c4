"""Seeded synthetic inputs for the ESM-2 encoder forward.

This module is shared by the HIP path (bench, tests) and the CPU oracle
(tests).  It holds none of the encoder's arithmetic: it draws random numbers,
rounds them to bfloat16 and arranges them in the layouts the boundary takes.

Workload shapes follow the ESM-2 model card of the BioNeMo framework (section
"模型概述": 650M = 33 layers, 20 heads, hidden 1280; 3B = 36 layers, 40 heads,
hidden 2560) and the TransformerEngine ESM-2 article (config.json: vocabulary
33, 1026 positions).  No protein dataset is available here, so lognormal
sequence lengths stand in for the length mix of UniProt/UniRef sequences and
uniform token ids over the 33-token vocabulary stand in for residues.

Recipe (seed s, stream k):  numpy Generator over SeedSequence([s, k]).
  stream 0      sequence lengths, one scalar draw at a time:
                L = int(clip(rint(lognormal(ln(median), 0.6)), 17, 1024));
                with a residue budget N, drawing stops at the first length that
                would push the total above N (that draw is discarded)
  stream 1      token ids, integers(0, vocab, T, int32)
  stream 2      hidden states N(0, 1)  [T, H]
  stream 3      embedding table N(0, 0.02)  [vocab, H]
  stream 4      permutation of sequences (for permutation tests)
  streams 20-24 biased attention ([B, N, L, heads, 64] tensors): q, k, v
                N(0, 1) (streams 20, 21, 22); mask bias (stream 23): per
                (b, n) a valid length drawn integers(ceil(3L/4), L + 1), keys
                at or past it get the mask value (default -1e9), the rest 0;
                pair bias N(0, 1) [B, heads, L, L] (stream 24)
  stream 1000+l weights of layer l in the order W_qkv, b_qkv, W_o, b_o, W_1,
                b_1, W_2, b_2, each N(0, 0.02); LayerNorm gamma = 1, beta = 0
All float draws are float64 -> float32 -> bfloat16 (round to nearest even).

Deep stacks (33 or 36 layers, 0.65 or 2.8 billion weights) use a second,
faster weight recipe that draws on the device with torch's generator:
  layer l: torch.Generator(device).manual_seed(seed * 1_000_003 + 1000 + l),
  then randn(float32) * 0.02 -> bfloat16 (round to nearest even), in the same
  tensor order as above.  Weights for the oracle are copied back to the host.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "rng", "to_bf16_bits", "bf16_bits_to_f64",
    "draw_lengths", "make_batch", "make_layer_weights", "make_embedding",
    "make_hidden", "LAYER_WEIGHT_NAMES", "BiasedAttnShape", "BIASED_ATTN_WORKLOADS",
    "make_biased_attention_inputs",
]

# Order of the per-layer tensors (names follow nn.Linear's [out, in] layout).
LAYER_WEIGHT_NAMES = (
    "ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_out", "b_out",
    "ln2_gamma", "ln2_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2",
)


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def to_bf16_bits(x) -> np.ndarray:
    """float -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are first rounded to float32; NaN maps to a quiet NaN."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class ModelShape:
    hidden: int
    heads: int
    ffn: int
    layers: int
    vocab: int = 33
    max_positions: int = 1026

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    lengths_fixed: Optional[tuple] = None   # explicit lengths, in packing order
    median: float = 300.0
    count: Optional[int] = None             # fixed number of draws
    budget: Optional[int] = None            # residue budget
    input: str = "ids"                      # "ids" (embedding) or "hidden"
    precision: str = "bf16"


ESM2_TINY = ModelShape(hidden=320, heads=5, ffn=1280, layers=1)
ESM2_650M = ModelShape(hidden=1280, heads=20, ffn=5120, layers=33)
ESM2_3B = ModelShape(hidden=2560, heads=40, ffn=10240, layers=36)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", ESM2_TINY, lengths_fixed=(17, 64, 100, 200), input="ids"),
    "650m_layer": Workload("650m_layer", dataclasses.replace(ESM2_650M, layers=1),
                           median=300, count=46, input="hidden"),
    "650m": Workload("650m", ESM2_650M, median=300, budget=32768, input="ids"),
    "3b": Workload("3b", ESM2_3B, median=400, budget=16384, input="ids"),
    "650m_fp8": Workload("650m_fp8", ESM2_650M, median=300, budget=32768, input="ids",
                         precision="fp8"),
}


def draw_lengths(seed: int, median: float, count: Optional[int] = None,
                 budget: Optional[int] = None, sigma: float = 0.6,
                 lo: int = 17, hi: int = 1024) -> List[int]:
    if (count is None) == (budget is None):
        raise ValueError("give exactly one of count, budget")
    r = rng(seed, 0)
    out: List[int] = []
    total = 0
    while True:
        L = int(np.clip(np.rint(r.lognormal(np.log(median), sigma)), lo, hi))
        if count is not None:
            out.append(L)
            if len(out) == count:
                return out
        else:
            if total + L > budget:
                return out
            out.append(L)
            total += L


@dataclasses.dataclass
class Batch:
    lengths: np.ndarray        # int32 [B]
    cu_seqlens: np.ndarray     # int32 [B+1]
    ids: Optional[np.ndarray]  # int32 [T] or None
    hidden: Optional[np.ndarray]  # uint16 bf16 bits [T, H] or None

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def B(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def max_seqlen(self) -> int:
        return int(self.lengths.max()) if self.lengths.size else 0


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.size + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu.astype(np.int32)


def make_hidden(T: int, H: int, seed: int = 0, stream: int = 2) -> np.ndarray:
    return to_bf16_bits(rng(seed, stream).standard_normal((T, H)).astype(np.float32))


def make_batch(w: Workload, seed: int = 0, lengths=None) -> Batch:
    if lengths is None:
        if w.lengths_fixed is not None:
            lengths = list(w.lengths_fixed)
        else:
            lengths = draw_lengths(seed, w.median, count=w.count, budget=w.budget)
    lengths = np.asarray(lengths, dtype=np.int32)
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    ids = hidden = None
    if w.input == "ids":
        ids = rng(seed, 1).integers(0, w.model.vocab, T, dtype=np.int32)
    else:
        hidden = make_hidden(T, w.model.hidden, seed)
    return Batch(lengths=lengths, cu_seqlens=cu, ids=ids, hidden=hidden)


def make_embedding(vocab: int, H: int, seed: int = 0) -> np.ndarray:
    r = rng(seed, 3)
    return to_bf16_bits((r.standard_normal((vocab, H)) * 0.02).astype(np.float32))


def make_layer_weights(H: int, F: int, layer: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """bf16 bit patterns of one layer's tensors, nn.Linear layout [out, in].

    w_qkv rows are grouped per head: row 192*n + 64*c + j holds component c
    (0 = query, 1 = key, 2 = value) of head n, dimension j."""
    r = rng(seed, 1000 + layer)

    def draw(shape):
        return to_bf16_bits((r.standard_normal(shape) * 0.02).astype(np.float32))

    out: Dict[str, np.ndarray] = {}
    out["w_qkv"] = draw((3 * H, H))
    out["b_qkv"] = draw((3 * H,))
    out["w_out"] = draw((H, H))
    out["b_out"] = draw((H,))
    out["w_fc1"] = draw((F, H))
    out["b_fc1"] = draw((F,))
    out["w_fc2"] = draw((H, F))
    out["b_fc2"] = draw((H,))
    one = to_bf16_bits(np.ones(H, np.float32))
    zero = to_bf16_bits(np.zeros(H, np.float32))
    out["ln1_gamma"], out["ln1_beta"] = one.copy(), zero.copy()
    out["ln2_gamma"], out["ln2_beta"] = one.copy(), zero.copy()
    return out


def make_head_weights(H: int, embedding_bits: np.ndarray, seed: int = 0, random_ln: bool = False) -> Dict[str, np.ndarray]:
    """bf16 bit patterns of the final LayerNorm and the masked-LM head (stream
    2000): dense [H, H] and biases N(0, 0.02); the decoder is the embedding
    table itself (tied); LayerNorms gamma = 1, beta = 0 unless random_ln."""
    r = rng(seed, 2000)

    def draw(shape, scale=0.02):
        return to_bf16_bits((r.standard_normal(shape) * scale).astype(np.float32))

    out: Dict[str, np.ndarray] = {"lm_dense_w": draw((H, H)), "lm_dense_b": draw((H,)),
                                  "lm_decoder_w": np.ascontiguousarray(embedding_bits),
                                  "lm_decoder_b": draw((embedding_bits.shape[0],))}
    for n in ("final_ln", "lm_ln"):
        if random_ln:
            out[n + "_gamma"] = to_bf16_bits((1 + 0.1 * r.standard_normal(H)).astype(np.float32))
            out[n + "_beta"] = draw((H,), 0.1)
        else:
            out[n + "_gamma"] = to_bf16_bits(np.ones(H, np.float32))
            out[n + "_beta"] = to_bf16_bits(np.zeros(H, np.float32))
    return out


def make_layer_weights_device(H: int, F: int, layer: int, seed: int = 0, device: str = "cuda:0"):
    """Same tensors as make_layer_weights, drawn on the device (torch generator).

    Returns torch bfloat16 tensors; gamma = 1 and beta = 0."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + 1000 + layer)

    def draw(shape):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * 0.02).to(torch.bfloat16)

    out = {}
    out["w_qkv"] = draw((3 * H, H))
    out["b_qkv"] = draw((3 * H,))
    out["w_out"] = draw((H, H))
    out["b_out"] = draw((H,))
    out["w_fc1"] = draw((F, H))
    out["b_fc1"] = draw((F,))
    out["w_fc2"] = draw((H, F))
    out["b_fc2"] = draw((H,))
    out["ln1_gamma"] = torch.ones(H, dtype=torch.bfloat16, device=device)
    out["ln1_beta"] = torch.zeros(H, dtype=torch.bfloat16, device=device)
    out["ln2_gamma"] = torch.ones(H, dtype=torch.bfloat16, device=device)
    out["ln2_beta"] = torch.zeros(H, dtype=torch.bfloat16, device=device)
    return out


def tensor_bits(t) -> np.ndarray:
    """torch bfloat16 tensor (any device) -> uint16 bit patterns on the host."""
    return t.detach().contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def random_layernorm_params(H: int, seed: int, stream: int = 5) -> Dict[str, np.ndarray]:
    """Non-trivial LayerNorm gamma/beta for unit tests (gamma ~ 1 + N(0, 0.1), beta ~ N(0, 0.1))."""
    r = rng(seed, stream)
    return {
        "ln1_gamma": to_bf16_bits((1 + 0.1 * r.standard_normal(H)).astype(np.float32)),
        "ln1_beta": to_bf16_bits((0.1 * r.standard_normal(H)).astype(np.float32)),
        "ln2_gamma": to_bf16_bits((1 + 0.1 * r.standard_normal(H)).astype(np.float32)),
        "ln2_beta": to_bf16_bits((0.1 * r.standard_normal(H)).astype(np.float32)),
    }


def permutation(B: int, seed: int = 0) -> np.ndarray:
    return rng(seed, 4).permutation(B)


@dataclasses.dataclass(frozen=True)
class BiasedAttnShape:
    """Shape of one biased-attention call: q, k, v are [B, N, L, heads, 64]."""
    name: str
    B: int
    N: int
    L: int
    heads: int


# The Evoformer MSA row attention layout of the DeepSpeed4Science page
# (section 5.3: Q, K, V [Batch, N_seq, N_res, Head, Dim], a residue mask bias
# and a pair bias); the page gives no sizes, so these are synthetic: 128 MSA
# rows of 512 residues, 8 heads of 64.
BIASED_ATTN_WORKLOADS: Dict[str, BiasedAttnShape] = {
    "tiny": BiasedAttnShape("tiny", 2, 3, 77, 2),
    "msa_row_512": BiasedAttnShape("msa_row_512", 1, 128, 512, 8),
}


def make_biased_attention_inputs(B: int, N: int, L: int, heads: int, seed: int = 0,
                                 mask_value: float = -1e9) -> Dict[str, np.ndarray]:
    """bf16 bit patterns: q, k, v [B, N, L, heads, 64]; mask [B, N, 1, 1, L];
    pair [B, 1, heads, L, L] (see the module recipe, streams 20-24)."""
    shape = (B, N, L, heads, 64)
    out = {}
    for name, stream in (("q", 20), ("k", 21), ("v", 22)):
        out[name] = to_bf16_bits(rng(seed, stream).standard_normal(shape).astype(np.float32))
    valid = rng(seed, 23).integers(-(-3 * L // 4), L + 1, size=(B, N))
    mask = np.where(np.arange(L)[None, None, :] >= valid[:, :, None], mask_value, 0.0)
    out["mask"] = to_bf16_bits(mask.reshape(B, N, 1, 1, L).astype(np.float32))
    out["pair"] = to_bf16_bits(rng(seed, 24).standard_normal((B, 1, heads, L, L)).astype(np.float32))
    return out
