"""Randomised GPU parity: seeded random shapes through every entry point.

Each case draws B, N, H, the kept lengths (empty and full images included),
the input and output dtypes and a max_seqlen bound, then checks on the GPU:
  * rag_pack against the oracle bit for bit (cu_seqlens, gather index, rows);
  * rag_attn (and rag_attn_tiled where its limits allow) against the oracle
    within 2e-3 on every image, bf16 output as the RNE of fp32 output, the
    tiled launch bit for bit equal to the grid launch;
  * rag_unpack bit for bit (and the zero-dropped flag);
  * rag_attn_gathered bit for bit equal to the packed result at the kept rows;
  * rag_attn_padded within 2e-3 of the oracle on the kept rows;
  * rag_repack with a random second-stage keep mask against oracle.repack.
A second draw takes more (image, head) pairs (B up to 96, H up to 12) at lengths
around the LDS-resident limit, so both sides of the attention's few/many-pairs
switch are exercised.
max_seqlen is either the longest image (every row attended) or a bound below
it (images truncated to their first max_seqlen rows, which the oracle is given
the same way: its input is the truncated batch).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import SENTINEL_BYTE, as_numpy_rows, gpu_pack, sentinel_like, to_gpu_rows
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3
CASES = 24
MANY_CASES = 8


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.choice([1, 7, 64, 65, 130, 197, 300, 577]))
    B = int(rng.integers(1, 17))
    H = int(rng.integers(1, 5))
    kind = rng.integers(0, 3)
    if kind == 0:
        lengths = rng.integers(0, N + 1, size=B)
    elif kind == 1:
        lengths = np.full(B, max(1, N // 5))
    else:
        lengths = rng.choice([0, 1, N], size=B)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    out_dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    w = wl.custom(B=B, N=N, H=H, lengths=lengths, dtype=dtype, seed=2000 + seed)
    mx = int(w.lengths.max()) if w.T else 1
    bound = mx if rng.random() < 0.7 else max(1, int(rng.integers(1, mx + 1)))
    return w, out_dtype, bound


def _draw_many(seed):
    """More (image, head) pairs: B 8-96, H 1-12, lengths near the LDS-resident limit of
    256 rows and the 64-row tile, so that both sides of the few/many-pairs switch (256
    pairs) and of the per-wave output slots' LDS limit are drawn."""
    rng = np.random.default_rng(5000 + seed)
    N = int(rng.choice([16, 63, 64, 127, 128, 129, 192, 197, 255, 256, 257, 320]))
    B = int(rng.integers(8, 97))
    H = int(rng.integers(1, 13))
    kind = rng.integers(0, 3)
    if kind == 0:
        lengths = rng.integers(0, N + 1, size=B)
    elif kind == 1:
        lengths = np.full(B, N)
    else:
        lengths = np.clip(rng.normal(0.5 * N, 0.1 * N, size=B).astype(int), 0, N)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    out_dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    w = wl.custom(B=B, N=N, H=H, lengths=lengths, dtype=dtype, seed=6000 + seed)
    mx = int(w.lengths.max()) if w.T else 1
    bound = mx if rng.random() < 0.8 else max(1, int(rng.integers(1, mx + 1)))
    return w, out_dtype, bound


def _attn(packed, cu, w, out_dtype, bound, tiled=False):
    C = w.C
    o = sentinel_like((packed.shape[0], C), out_dtype)
    binding.rag_attn(packed[:, :C], packed[:, C:2 * C], packed[:, 2 * C:], cu, bound, o, H=w.H,
                     scale=w.scale, tiled=tiled)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("seed", range(CASES))
def test_random_case(seed):
    w, out_dtype, bound = _draw(seed)
    _check_case(w, out_dtype, bound, seed)


@pytest.mark.parametrize("seed", range(MANY_CASES))
def test_random_case_many_pairs(seed):
    w, out_dtype, bound = _draw_many(seed)
    _check_case(w, out_dtype, bound, 10000 + seed)


def test_every_image_empty():
    """T = 0: nothing is packed, attended or written, through every entry point."""
    w = wl.custom(B=5, N=65, H=2, lengths=[0] * 5, seed=77)
    _check_case(w, torch.bfloat16, 1, 77)


def _check_case(w, out_dtype, bound, seed):
    print("seed", seed, "B", w.B, "N", w.N, "H", w.H, "T", w.T, w.dtype, out_dtype, "bound", bound,
          flush=True)
    rows = wl.rows(w)
    packed_ref, cu_ref, gather_ref = oracle.pack(w.keep, rows)
    T = int(cu_ref[-1])
    g = gpu_pack(w, want_max=False)
    assert (g["cu"].cpu().numpy() == cu_ref).all()
    assert (g["gather"].cpu().numpy()[:T] == gather_ref).all()
    pk = as_numpy_rows(g["packed"])
    assert (pk[:T].view(np.uint8) == packed_ref.view(np.uint8)).all()

    # attention: the oracle sees each image truncated to its first `bound` rows
    o32 = _attn(g["packed"], g["cu"], w, torch.float32, bound)
    oo = _attn(g["packed"], g["cu"], w, out_dtype, bound)
    written = np.zeros(T, dtype=bool)  # the first `bound` rows of every image
    for b in range(w.B):
        s = int(cu_ref[b])
        written[s:s + min(int(cu_ref[b + 1]) - s, bound)] = True
    if out_dtype == torch.bfloat16:
        rne = o32.cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (as_numpy_rows(oo)[:T][written] == rne[:T][written]).all()
    assert (as_numpy_rows(oo)[:T][~written].view(np.uint8) == SENTINEL_BYTE).all()
    if w.B <= 1024 and bound <= 960 and w.H <= 64:
        ot = _attn(g["packed"], g["cu"], w, torch.float32, bound, tiled=True)
        assert (as_numpy_rows(ot)[:T].view(np.uint8) == as_numpy_rows(o32)[:T].view(np.uint8)).all()
    got = o32.cpu().numpy().astype(np.float64)
    q, k, v = wl.split_qkv(packed_ref, w.C)
    for b in range(w.B):
        s, e = int(cu_ref[b]), int(cu_ref[b + 1])
        L = min(e - s, bound)
        if L == 0:
            continue
        want = oracle.attn(q[s:s + L], k[s:s + L], v[s:s + L], np.array([0, L], np.int32), w.H, w.d,
                           w.scale)
        assert np.abs(got[s:s + L] - want).max() <= ATOL, b
        # rows past the bound are neither attended nor written
        assert (as_numpy_rows(o32)[s + L:e].view(np.uint8) == SENTINEL_BYTE).all()

    # unpack of the fp32 attention output, both flag settings
    for flags in (0, binding.RAG_UNPACK_ZERO_DROPPED):
        dst = sentinel_like((w.B * w.N, w.C), torch.float32)
        binding.rag_unpack(o32, g["cu"], g["gather"], dst, N=w.N, flags=flags)
        torch.cuda.synchronize()
        want = oracle.unpack(as_numpy_rows(o32)[:max(T, 1)], cu_ref, gather_ref,
                             as_numpy_rows(sentinel_like((w.B * w.N, w.C), torch.float32)))
        if flags:
            dropped = np.setdiff1d(np.arange(w.B * w.N), gather_ref)
            want[dropped] = 0
        assert (as_numpy_rows(dst).view(np.uint8) == want.view(np.uint8)).all(), flags

    # the gathered pass: the packed result's bits at the kept rows
    src = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    C = w.C
    gz = sentinel_like((w.B * w.N, C), torch.float32)
    binding.rag_attn_gathered(keep, src[:, :C], src[:, C:2 * C], src[:, 2 * C:], gz, H=w.H,
                              scale=w.scale, max_seqlen=min(bound, w.N))
    torch.cuda.synchronize()
    gzn = as_numpy_rows(gz)
    for b in range(w.B):
        s, e = int(cu_ref[b]), int(cu_ref[b + 1])
        L = min(e - s, bound)
        if L:
            assert (gzn[gather_ref[s:s + L]].view(np.uint8) ==
                    as_numpy_rows(o32)[s:s + L].view(np.uint8)).all(), b

    # padded comparator on the kept rows (no bound: every kept key)
    pz = sentinel_like((w.B * w.N, C), torch.float32)
    binding.rag_attn_padded(src[:, :C], src[:, C:2 * C], src[:, 2 * C:], keep, pz, H=w.H,
                            scale=w.scale)
    torch.cuda.synchronize()
    if T:
        want_all = oracle.attn(q, k, v, cu_ref, w.H, w.d, w.scale)
        assert np.abs(pz.cpu().numpy()[gather_ref].astype(np.float64) - want_all).max() <= ATOL

    # a second pruning stage on the packed rows
    rng = np.random.default_rng(3000 + seed)
    k2 = (rng.random(w.B * w.N) < 0.6).astype(np.uint8)
    want_p, want_cu, want_g = oracle.repack(k2[:T], cu_ref, gather_ref, packed_ref)
    dst = sentinel_like(g["packed"].shape, g["packed"].dtype)
    cu2 = sentinel_like((w.B + 1,), torch.int32)
    g2 = sentinel_like((w.B * w.N,), torch.int32)
    binding.rag_repack(torch.from_numpy(k2).cuda(), g["cu"], g["gather"], w.N, g["packed"], dst, cu2,
                       g2)
    torch.cuda.synchronize()
    T2 = int(want_cu[-1])
    assert (cu2.cpu().numpy() == want_cu).all()
    assert (g2.cpu().numpy()[:T2] == want_g).all()
    assert (as_numpy_rows(dst)[:T2].view(np.uint8) == want_p.view(np.uint8)).all()
