"""GPU parity at the largest sizes the boundary accepts: N = RAG_MAX_N (8192
tokens per image) and B = RAG_MAX_B (65535 images).

Pack and unpack are compared bit for bit with the oracle.  Attention at N = 8192
is compared on sampled query rows (oracle.attn_rows: the same per-row
definition as oracle.attn), within the 2e-3 bar; at B = 65535 every image is
tiny and the whole output is compared.  The other layouts (gathered, padded) run
at the same sizes and are checked against the ragged result (gathered: bit for
bit at the kept rows) or the oracle (padded: kept rows).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (SENTINEL_BYTE, as_numpy_rows, gpu_attn, gpu_pack, sentinel_like,
                         to_gpu_rows)
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3
RAG_MAX_N = 8192
RAG_MAX_B = 65535


def _check_pack_unpack(w, g):
    packed_ref, cu_ref, gather_ref = oracle.pack(w.keep, wl.rows(w))
    T = int(cu_ref[-1])
    assert (g["cu"].cpu().numpy() == cu_ref).all()
    gather = g["gather"].cpu().numpy()
    assert (gather[:T] == gather_ref).all()
    packed = as_numpy_rows(g["packed"])
    assert (packed[:T].view(np.uint8) == packed_ref.view(np.uint8)).all()
    assert (packed[T:].view(np.uint8) == SENTINEL_BYTE).all()
    # unpack the packed rows back into a sentinel batch
    dst = sentinel_like(g["src"].shape, g["src"].dtype)
    binding.rag_unpack(g["packed"], g["cu"], g["gather"], dst, N=w.N)
    torch.cuda.synchronize()
    want = oracle.unpack(packed_ref, cu_ref, gather_ref,
                         np.full(as_numpy_rows(dst).shape, 0, dtype=packed_ref.dtype))
    got = as_numpy_rows(dst)
    assert (got[gather_ref].view(np.uint8) == want[gather_ref].view(np.uint8)).all()
    dropped = np.setdiff1d(np.arange(w.B * w.N), gather_ref)
    assert (got[dropped].view(np.uint8) == SENTINEL_BYTE).all()
    return packed_ref, cu_ref, gather_ref


def _gathered(w, out_dtype):
    src = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    C = w.C
    o = sentinel_like((w.B * w.N, C), out_dtype)
    binding.rag_attn_gathered(keep, src[:, :C], src[:, C:2 * C], src[:, 2 * C:], o, H=w.H,
                              scale=w.scale)
    torch.cuda.synchronize()
    return o


def _padded(w, out_dtype):
    src = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    C = w.C
    o = sentinel_like((w.B * w.N, C), out_dtype)
    binding.rag_attn_padded(src[:, :C], src[:, C:2 * C], src[:, 2 * C:], keep, o, H=w.H,
                            scale=w.scale)
    torch.cuda.synchronize()
    return o


def test_longest_images():
    """N = 8192: one image keeping every token, one keeping 3001."""
    w = wl.custom(B=2, N=RAG_MAX_N, H=1, lengths=[RAG_MAX_N, 3001], seed=31)
    print("N", w.N, "T", w.T, flush=True)
    g = gpu_pack(w)
    packed_ref, cu_ref, gather_ref = _check_pack_unpack(w, g)
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=RAG_MAX_N)
    o16 = gpu_attn(g["packed"], g["cu"], w, torch.bfloat16, max_seqlen=RAG_MAX_N)
    T = w.T
    rne = o32.cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (as_numpy_rows(o16)[:T] == rne[:T]).all()
    rng = np.random.default_rng(31)
    rows = sorted(set([0, 1, RAG_MAX_N - 1, RAG_MAX_N, T - 1] + rng.integers(0, T, 11).tolist()))
    q, k, v = wl.split_qkv(packed_ref, w.C)
    want = oracle.attn_rows(q, k, v, cu_ref, w.H, w.d, w.scale, rows)
    got = o32.cpu().numpy().astype(np.float64)[rows]
    err = np.abs(got - want).max()
    print("sampled rows", len(rows), "max abs err", err, flush=True)
    assert err <= ATOL
    # the gathered layout gives the same bits at the kept rows
    gz = as_numpy_rows(_gathered(w, torch.float32))
    assert (gz[gather_ref].view(np.uint8) == as_numpy_rows(o32)[:T].view(np.uint8)).all()
    # padded: the kept rows of the sampled set agree with the oracle
    pz = _padded(w, torch.float32).cpu().numpy().astype(np.float64)
    err_p = np.abs(pz[gather_ref[rows]] - want).max()
    print("padded max abs err", err_p, flush=True)
    assert err_p <= ATOL


def test_most_images():
    """B = 65535 images of N = 2 tokens, 0, 1 or 2 kept each."""
    rng = np.random.default_rng(32)
    w = wl.custom(B=RAG_MAX_B, N=2, H=1, lengths=rng.integers(0, 3, size=RAG_MAX_B), seed=32)
    print("B", w.B, "T", w.T, flush=True)
    g = gpu_pack(w)
    packed_ref, cu_ref, gather_ref = _check_pack_unpack(w, g)
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=2)
    q, k, v = wl.split_qkv(packed_ref, w.C)
    want = oracle.attn(q, k, v, cu_ref, w.H, w.d, w.scale)
    T = w.T
    err = np.abs(o32.cpu().numpy()[:T].astype(np.float64) - want).max()
    print("max abs err", err, flush=True)
    assert err <= ATOL
    gz = as_numpy_rows(_gathered(w, torch.float32))
    assert (gz[gather_ref].view(np.uint8) == as_numpy_rows(o32)[:T].view(np.uint8)).all()
    pz = _padded(w, torch.float32).cpu().numpy().astype(np.float64)
    assert np.abs(pz[gather_ref] - want).max() <= ATOL


def test_tile_kernel_grid_over_several_rows():
    """fp32 input takes the 64-key tile kernel, whose slots ((image, head) pair,
    q-tile) form a grid of (32 * q-tiles, blocks of 32 pairs): B = 65535 images
    of H = 17 heads give 1 114 095 pairs in 34 816 blocks.  Every row of the
    output matches the oracle; the gathered and padded layouts (the same
    kernel) agree."""
    rng = np.random.default_rng(33)
    w = wl.custom(B=RAG_MAX_B, N=2, H=17, lengths=rng.integers(0, 3, size=RAG_MAX_B), dtype="f32",
                  seed=33)
    print("B", w.B, "H", w.H, "T", w.T, flush=True)
    assert w.B * w.H > (1 << 20)
    g = gpu_pack(w)
    packed_ref, cu_ref, gather_ref = oracle.pack(w.keep, wl.rows(w))
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=2)
    q, k, v = wl.split_qkv(packed_ref, w.C)
    want = oracle.attn(q, k, v, cu_ref, w.H, w.d, w.scale)
    T = w.T
    out = o32.cpu().numpy()
    err = np.abs(out[:T].astype(np.float64) - want).max()
    print("max abs err", err, flush=True)
    assert err <= ATOL
    assert (out[T:].view(np.uint32) == np.uint32(SENTINEL_BYTE * 0x01010101)).all()
    gz = as_numpy_rows(_gathered(w, torch.float32))
    assert (gz[gather_ref].view(np.uint8) == as_numpy_rows(o32)[:T].view(np.uint8)).all()
    pz = _padded(w, torch.float32).cpu().numpy().astype(np.float64)
    assert np.abs(pz[gather_ref] - want).max() <= ATOL


def test_tile_kernel_pair_blocks_folded_into_z():
    """bf16 input with max_seqlen = 257 takes the 64-key tile kernel (5 q-tiles
    per pair).  B = 65535 images of H = 33 heads give 2 162 655 pairs, 67 584
    blocks of 32: more than the 65 535 grid rows, so the blocks continue in a
    second z layer, and the images at the end of the batch are served from it.
    Every row of the output matches the oracle; rows past the packed ones are
    untouched."""
    rng = np.random.default_rng(34)
    w = wl.custom(B=RAG_MAX_B, N=2, H=33, lengths=rng.integers(0, 3, size=RAG_MAX_B), seed=34)
    print("B", w.B, "H", w.H, "T", w.T, flush=True)
    assert (w.B * w.H + 31) // 32 > 65535
    g = gpu_pack(w)
    packed_ref, cu_ref, gather_ref = oracle.pack(w.keep, wl.rows(w))
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=257)
    q, k, v = wl.split_qkv(packed_ref, w.C)
    want = oracle.attn(q, k, v, cu_ref, w.H, w.d, w.scale)
    T = w.T
    out = o32.cpu().numpy()
    err = np.abs(out[:T].astype(np.float64) - want).max()
    print("max abs err", err, flush=True)
    assert err <= ATOL
    assert (out[T:].view(np.uint32) == np.uint32(SENTINEL_BYTE * 0x01010101)).all()
