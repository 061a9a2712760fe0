"""Helpers for the GPU parity tests: move a workload to the GPU, call the HIP
path through the C ABI (binding), and bring results back as numpy arrays.
No arithmetic of the method happens here."""
import numpy as np
import torch

from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

SENTINEL_BYTE = 0xA5


def to_gpu_rows(w: wl.Workload) -> torch.Tensor:
    rows = wl.rows(w)
    if w.dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(rows))
    else:
        t = torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def torch_dtype(w: wl.Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def sentinel_like(shape, dtype) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(SENTINEL_BYTE)
    return t


def as_numpy_rows(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> numpy with the same bit patterns (bf16 as uint16)."""
    c = t.detach().cpu().contiguous()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def gpu_pack(w: wl.Workload, want_max=True):
    B, N = w.B, w.N
    keep = torch.from_numpy(w.keep).cuda()
    src = to_gpu_rows(w)
    packed = sentinel_like((B * N, 3 * w.C), torch_dtype(w))
    cu = sentinel_like((B + 1,), torch.int32)
    gather = sentinel_like((B * N,), torch.int32)
    mx = sentinel_like((1,), torch.int32) if want_max else None
    binding.rag_pack(keep, src, packed, cu, gather, mx)
    torch.cuda.synchronize()
    return dict(keep=keep, src=src, packed=packed, cu=cu, gather=gather, max=mx)


def gpu_attn(packed: torch.Tensor, cu: torch.Tensor, w: wl.Workload, out_dtype, max_seqlen=None,
             tiled=False):
    C = w.C
    q, k, v = packed[:, 0:C], packed[:, C:2 * C], packed[:, 2 * C:3 * C]
    o = sentinel_like((packed.shape[0], C), out_dtype)
    binding.rag_attn(q, k, v, cu, max_seqlen or w.N, o, H=w.H, scale=w.scale, tiled=tiled)
    torch.cuda.synchronize()
    return o


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
