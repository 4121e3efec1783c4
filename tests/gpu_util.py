"""Helpers for the GPU tests: moving bf16 bit patterns to and from torch
device tensors, and building weight sets for the library and the oracle from
the same seeded draws."""
import numpy as np
import torch

from oracle import esm_oracle as O
from protein_language_model_amd import datagen as D

DEV = "cuda:0"


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> float64 numpy (exact)."""
    torch.cuda.synchronize()
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return D.bf16_bits_to_f64(bits)


def bits_of(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def layer_weights(H, F, layer=0, seed=0, random_ln=False):
    bits = D.make_layer_weights(H, F, layer, seed)
    if random_ln:
        bits.update(D.random_layernorm_params(H, seed + 100 + layer))
    dev = {k: to_dev_bf16(v) for k, v in bits.items()}
    ref = O.weights_to_f64(bits)
    return dev, ref, bits


def rel_err(got, ref) -> float:
    return O.rel_max_err(got, ref)
