"""Small numpy/scipy helpers the oracle pins use as independent checks.

These are library-routine formulations (dense matmuls, scipy's expit and the
normal CDF, stable sorts) of special cases the oracle must reduce to; they are
not a second copy of the oracle's loops.
"""
import numpy as np
import torch
from scipy.special import expit
from scipy.stats import norm


def to_np(t):
    """torch tensor -> numpy (bf16 as raw uint16 bits)."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decode(a):
    """numpy array (uint16 bf16 bits or float32) -> float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ffn_dense(x, w1, w3, w2, act):
    """Rows x [n, din] through one expert with [out, in] weights, float64."""
    a = x @ decode(w1).T
    if act == "gelu":
        hdn = a * norm.cdf(a)
    else:
        hdn = a * expit(a) * (x @ decode(w3).T)
    return hdn @ decode(w2).T


def softmax(z, axis=-1):
    z = z - z.max(axis=axis, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=axis, keepdims=True)


def inputs_np(inp):
    return {k: to_np(v) for k, v in inp.items()}
