"""fp64 reference of one ViT encoder block on packed token rows.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``): only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; it
shares no code with the HIP library.

"Dispatch-Aware Ragged Attention for Pruned Vision Transformers" (abstract)
reports end-to-end throughput of pruned DeiT models whose blocks run on the
packed tokens; the pages fix the attention step and the packing only.  The
rest of the block is DeiT's standard pre-norm encoder block, written out here
in the order it is defined:

    h   = LayerNorm1(x)                       (biased variance, eps inside the root)
    qkv = h Wqkv + bqkv                       (columns q | k | v, each head-major)
    a   = attention per image and head        (bidirectional, softmax(scale q k^T) v)
    x1  = x + a Wproj + bproj
    m   = GELU(LayerNorm2(x1) W1 + b1)
    y   = x1 + m W2 + b2

Everything is fp64; bf16 inputs (bit patterns as uint16) are decoded exactly.
numpy's matmul serves as the matrix product.  GELU is DeiT's: the exact form
x * Phi(x) with Phi the standard normal CDF ("erf"); the tanh approximation of
the same ("tanh") is kept only as a named alternative that the pins tell
apart from it.

The composition (pre-norm order, which tensor each residual adds to, the
q | k | v column blocks and their head split) is pinned against torch's own
fp64 nn.TransformerEncoderLayer(norm_first=True, activation="gelu") in the
tests, an implementation this module shares nothing with.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact values of bfloat16 bit patterns (uint16): the upper half of fp32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def layernorm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    mean = x.mean(axis=1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def gelu(x: np.ndarray, form: str) -> np.ndarray:
    if form == "erf":
        return 0.5 * x * (1.0 + np.vectorize(math.erf)(x / math.sqrt(2.0)))
    if form == "tanh":
        return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))
    raise ValueError("GELU form is 'erf' or 'tanh'")


def attention(qkv: np.ndarray, cu_seqlens: np.ndarray, H: int, d: int, scale: float) -> np.ndarray:
    """Per image b (rows cu[b] .. cu[b+1]-1) and head h: softmax(scale Q K^T) V."""
    C = H * d
    out = np.zeros((qkv.shape[0], C), dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(cu.shape[0] - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e == s:
            continue
        for h in range(H):
            q = qkv[s:e, h * d:(h + 1) * d]
            k = qkv[s:e, C + h * d:C + (h + 1) * d]
            v = qkv[s:e, 2 * C + h * d:2 * C + (h + 1) * d]
            sc = scale * (q @ k.T)
            sc = sc - sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p = p / p.sum(axis=1, keepdims=True)
            out[s:e, h * d:(h + 1) * d] = p @ v
    return out


def block(x_bits: np.ndarray, params: dict, cu_seqlens: np.ndarray, H: int, scale: float,
          eps: float = 1e-6, gelu_form: str = "erf", d: int = 64) -> np.ndarray:
    """y = block(x) over packed rows.  x_bits: uint16 bf16 patterns [T, C];
    params: w_* as uint16 bf16 patterns [in, out], b_* / ln*_gamma / ln*_beta
    as float32.  Returns fp64 [T, C]."""
    x = bf16_bits_to_f64(x_bits)
    W = {k: bf16_bits_to_f64(params[k]) for k in ("w_qkv", "w_proj", "w_fc1", "w_fc2")}
    P = {k: np.asarray(params[k], dtype=np.float64)
         for k in ("ln1_gamma", "ln1_beta", "ln2_gamma", "ln2_beta", "b_qkv", "b_proj", "b_fc1",
                   "b_fc2")}
    h = layernorm(x, P["ln1_gamma"], P["ln1_beta"], eps)
    qkv = h @ W["w_qkv"] + P["b_qkv"]
    a = attention(qkv, cu_seqlens, H, d, scale)
    x1 = x + a @ W["w_proj"] + P["b_proj"]
    h2 = layernorm(x1, P["ln2_gamma"], P["ln2_beta"], eps)
    m = gelu(h2 @ W["w_fc1"] + P["b_fc1"], gelu_form)
    return x1 + m @ W["w_fc2"] + P["b_fc2"]
