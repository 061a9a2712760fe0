"""Seeded synthetic inputs shaped like the pages' DeiT workloads.

This module only draws inputs: keep masks and Q/K/V values.  It holds none of
the method's arithmetic (no packing, no offsets, no attention), so both the HIP
path and the CPU oracle can be fed from it without sharing any logic.

Shapes follow "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
(abstract: DeiT models, at most 197 tokens after pruning at 224x224, and
384x384 inputs; the v1 abstract lists DeiT-T/S/B): N = 197 = 14*14 + 1 (one
CLS token plus 196 patches) or N = 577 = 24*24 + 1, head dimension 64, heads
3 / 6 / 12.  The pruning decision itself is taken as given by the method; a
top-k of random token scores (CLS always kept) stands in for a trained pruner.

Generator: numpy PCG64 (``numpy.random.default_rng(seed)``).  Draw order:
per-image kept lengths (if random), then the keep choice (scores or uniform
picks), then one fp32 N(0,1) tensor of shape [B, N, 3, H, d] (Q, K, V
interleaved per token, i.e. a fused qkv row of 3*H*d values).  bf16 workloads
round those fp32 draws to bfloat16 (round to nearest even, via torch's own
conversion) and carry the raw 16-bit patterns as uint16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    N: int
    H: int
    d: int
    dtype: str  # "f32" or "bf16"
    scale: float
    seed: int
    keep: np.ndarray  # uint8 [B, N], nonzero = keep
    qkv: np.ndarray  # [B, N, 3, H, d]: float32, or uint16 bf16 bit patterns
    lengths: np.ndarray  # int64 [B], kept tokens per image (count of nonzero keep)
    recipe: str

    @property
    def C(self) -> int:
        return self.H * self.d

    @property
    def T(self) -> int:
        return int(self.lengths.sum())

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def row_bytes(self) -> int:
        """Bytes of one fused qkv token row."""
        return 3 * self.C * self.elem_bytes


def kept_length(N: int, prune_permille: int) -> int:
    """Kept tokens (CLS included) at a prune rate given in thousandths:
    ceil((1 - p) * N), computed in integers."""
    keep_pm = 1000 - prune_permille
    return max(1, (keep_pm * N + 999) // 1000)


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch  # local: plumbing for the rounding only

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _keep_topk(rng: np.random.Generator, B: int, N: int, lengths: np.ndarray) -> np.ndarray:
    """CLS (position 0) plus the top-(L_b - 1) of N(0,1) scores over the patches.
    Ties (measure zero) go to the lower index."""
    scores = rng.standard_normal((B, N - 1))
    keep = np.zeros((B, N), dtype=np.uint8)
    for b in range(B):
        L = int(lengths[b])
        if L <= 0:
            continue
        keep[b, 0] = 1
        order = np.argsort(-scores[b], kind="stable")
        keep[b, 1 + order[: L - 1]] = 1
    return keep


def _keep_uniform(rng: np.random.Generator, B: int, N: int, lengths: np.ndarray) -> np.ndarray:
    """CLS plus L_b - 1 patches drawn uniformly without replacement."""
    keep = np.zeros((B, N), dtype=np.uint8)
    for b in range(B):
        L = int(lengths[b])
        if L <= 0:
            continue
        keep[b, 0] = 1
        keep[b, 1 + rng.choice(N - 1, size=L - 1, replace=False)] = 1
    return keep


def _finish(name, rng, B, N, H, d, dtype, keep, seed, recipe) -> Workload:
    x = rng.standard_normal((B, N, 3, H, d), dtype=np.float32)
    qkv = x if dtype == "f32" else _to_bf16_bits(x)
    lengths = (keep != 0).sum(axis=1).astype(np.int64)
    return Workload(name=name, B=B, N=N, H=H, d=d, dtype=dtype, scale=1.0 / math.sqrt(d),
                    seed=seed, keep=keep, qkv=qkv, lengths=lengths, recipe=recipe)


def tiny(seed: int = 0) -> Workload:
    """B=2, N=197, H=3, d=64 (DeiT-T heads), kept lengths {99, 40}, CLS kept, other
    kept positions uniform without replacement, fp32 Q/K/V."""
    B, N, H, d = 2, 197, 3, 64
    rng = np.random.default_rng(seed)
    lengths = np.array([99, 40])
    keep = _keep_uniform(rng, B, N, lengths)
    return _finish("tiny_b2_n197_h3_f32", rng, B, N, H, d, "f32", keep, seed,
                   "lengths {99,40}; CLS + uniform w/o replacement; fp32 N(0,1)")


def deits(B: int = 4, prune_permille: int = 800, seed: int = 0) -> Workload:
    """DeiT-S layer shape: N=197, H=6, d=64, bf16; every image keeps
    ceil((1-p)*197) tokens (CLS + top-k of random scores)."""
    N, H, d = 197, 6, 64
    rng = np.random.default_rng(seed)
    lengths = np.full(B, kept_length(N, prune_permille))
    keep = _keep_topk(rng, B, N, lengths)
    return _finish("deits_b%d_n197_h6_p%03d" % (B, prune_permille), rng, B, N, H, d, "bf16",
                   keep, seed, "L=ceil((1-p)N) each; CLS + top-k of N(0,1) scores; bf16 N(0,1)")


def deitb_ragged(B: int = 64, seed: int = 0) -> Workload:
    """DeiT-B throughput batch: N=197, H=12, d=64, bf16; L_b uniform in [20, 197]."""
    N, H, d = 197, 12, 64
    rng = np.random.default_rng(seed)
    lengths = rng.integers(20, 198, size=B)
    keep = _keep_topk(rng, B, N, lengths)
    return _finish("deitb_b%d_n197_h12_ragged" % B, rng, B, N, H, d, "bf16", keep, seed,
                   "L_b ~ U{20..197}; CLS + top-k of N(0,1) scores; bf16 N(0,1)")


def deitb384(B: int = 32, seed: int = 0) -> Workload:
    """384x384 input: N=577, H=12, d=64, bf16; keep ratio 0.5 +- U(-0.1, 0.1) per image."""
    N, H, d = 577, 12, 64
    rng = np.random.default_rng(seed)
    ratio = 0.5 + rng.uniform(-0.1, 0.1, size=B)
    lengths = np.minimum(N, np.ceil(ratio * N).astype(np.int64))
    keep = _keep_topk(rng, B, N, lengths)
    return _finish("deitb384_b%d_n577_h12" % B, rng, B, N, H, d, "bf16", keep, seed,
                   "L_b = ceil((0.5+U(-0.1,0.1))*577); CLS + top-k; bf16 N(0,1)")


def custom(B: int, N: int, H: int, lengths, d: int = 64, dtype: str = "bf16", seed: int = 0,
           keep_kind: str = "topk", name: Optional[str] = None) -> Workload:
    """Any shape with explicit per-image kept lengths (0 allowed: an empty image)."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64).reshape(B)
    if (lengths < 0).any() or (lengths > N).any():
        raise ValueError("kept lengths must lie in [0, N]")
    if keep_kind == "topk":
        keep = _keep_topk(rng, B, N, lengths)
    elif keep_kind == "uniform":
        keep = _keep_uniform(rng, B, N, lengths)
    elif keep_kind == "prefix":
        keep = (np.arange(N)[None, :] < lengths[:, None]).astype(np.uint8)
    else:
        raise ValueError(keep_kind)
    return _finish(name or "custom_b%d_n%d_h%d" % (B, N, H), rng, B, N, H, d, dtype, keep, seed,
                   "explicit lengths; keep=%s" % keep_kind)


#: The pruning sweep on the DeiT-S shape: batch sizes and prune rates (thousandths).
SWEEP_BATCHES: List[int] = [1, 2, 4, 256]
SWEEP_PRUNE_PERMILLE: List[int] = [0, 500, 800, 900]


def named() -> Dict[str, "callable"]:
    """Every named workload: the four fixed shapes plus the 16 sweep points."""
    out = {
        "tiny": tiny,
        "deits_b4_p800": lambda seed=0: deits(4, 800, seed),
        "deitb_ragged_b64": lambda seed=0: deitb_ragged(64, seed),
        "deitb384_b32": lambda seed=0: deitb384(32, seed),
    }
    for B in SWEEP_BATCHES:
        for p in SWEEP_PRUNE_PERMILLE:
            out["deits_b%d_p%03d" % (B, p)] = (lambda B=B, p=p: lambda seed=0: deits(B, p, seed))()
    return out


def rows(w: Workload) -> np.ndarray:
    """The fused qkv tensor viewed as [B*N, 3*C] token rows."""
    return w.qkv.reshape(w.B * w.N, 3 * w.C)


def split_qkv(rows_2d: np.ndarray, C: int):
    """Views of Q, K, V ([rows, C] each, row stride 3C) inside fused rows."""
    return rows_2d[:, 0:C], rows_2d[:, C:2 * C], rows_2d[:, 2 * C:3 * C]


def second_stage_keep(w: Workload, kept: int, seed: int) -> np.ndarray:
    """Keep bytes for a later pruning stage over w's packed rows (image by image
    in order, each image's rows in ascending original position): every image
    keeps its first packed row (CLS) and min(kept, L_b) - 1 of its other rows,
    drawn uniformly without replacement (numpy PCG64, ``seed``).  uint8 [T]."""
    rng = np.random.default_rng(seed)
    k2 = np.zeros(w.T, dtype=np.uint8)
    start = 0
    for L in w.lengths.tolist():
        if L > 0:
            k2[start] = 1
            m = min(kept, L) - 1
            if m > 0:
                k2[start + 1 + rng.choice(L - 1, size=m, replace=False)] = 1
        start += L
    return k2


def vit_block_params(C: int, mlp_ratio: int, seed: int) -> Dict[str, np.ndarray]:
    """Random weights for one pre-norm ViT encoder block (numpy PCG64, ``seed``;
    draw order as listed): matrices N(0, 0.02^2) rounded to bf16 (uint16 bit
    patterns, row-major [in, out]); biases N(0, 0.02^2), LayerNorm gamma
    1 + N(0, 0.1^2) and beta N(0, 0.1^2) as float32.  The scale follows ViT's
    initialisation; gamma, beta and the biases are perturbed so that every
    parameter shows in the output."""
    rng = np.random.default_rng(seed)
    hid = C * mlp_ratio
    out: Dict[str, np.ndarray] = {}
    for name, shape in (("w_qkv", (C, 3 * C)), ("w_proj", (C, C)), ("w_fc1", (C, hid)),
                        ("w_fc2", (hid, C))):
        out[name] = _to_bf16_bits((0.02 * rng.standard_normal(shape)).astype(np.float32))
    for name, n in (("b_qkv", 3 * C), ("b_proj", C), ("b_fc1", hid), ("b_fc2", C)):
        out[name] = (0.02 * rng.standard_normal(n)).astype(np.float32)
    for ln in ("ln1", "ln2"):
        out[ln + "_gamma"] = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
        out[ln + "_beta"] = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return out


def hidden_rows(B: int, N: int, C: int, seed: int) -> np.ndarray:
    """Token hidden states [B*N, C]: N(0, 1) draws rounded to bf16 (uint16)."""
    rng = np.random.default_rng(seed)
    return _to_bf16_bits(rng.standard_normal((B * N, C)).astype(np.float32))
