"""GPU parity of rag_attn_tiled: ragged attention launched over the tile list.

Its 1-D grid covers (image, head, query-block range) items that every
workgroup derives from cu_seqlens (longest images first, pairs dealt to the
XCDs).  The same arithmetic runs in the same order as in rag_attn's
per-(head, image) grids, so:
  * against rag_attn the output is equal bit for bit, for both kernels (the
    LDS-resident one up to 256 keys, the 64-key tile kernel beyond and for
    fp32 input);
  * against the gathered layout the packed output is equal bit for bit at the
    kept rows;
  * every output row is written (outputs start as a sentinel), and the values
    are within the 2e-3 bar of the fp64 oracle.
The cases cover several 64-image chunks of the decode (B not a multiple of 64),
empty images, every key-tile class up to the limit (nkt = 15), classes with
fewer pairs than XCDs, both item shapes (a whole (image, head) pair on two-block
waves with many pairs, 4 blocks with few), fp32 input, max_seqlen bounds that
truncate, and the largest batch the tile list takes.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import SENTINEL_BYTE, as_numpy_rows, gpu_attn, gpu_pack, sentinel_like, to_gpu_rows
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3
EDGE_LENGTHS = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 191, 192, 193, 196, 197]


def _lengths(B, N, seed, edges):
    rng = np.random.default_rng(seed)
    e = [x for x in edges if x <= N]
    L = np.array([e[i] if i < len(e) else int(rng.integers(0, N + 1)) for i in range(B)])
    return rng.permutation(L)


CASES = {
    # many (image, head) pairs: one item per pair; three 64-image chunks
    "b130_n197_h2": lambda: wl.custom(B=130, N=197, H=2, lengths=_lengths(130, 197, 1, EDGE_LENGTHS),
                                      seed=21),
    # few pairs: items of up to 4 query blocks
    "b7_n197_h3": lambda: wl.custom(B=7, N=197, H=3, lengths=[197, 0, 150, 3, 64, 65, 100], seed=22),
    # one long image: a class with fewer pairs than XCDs
    "b3_n197_h1": lambda: wl.custom(B=3, N=197, H=1, lengths=[0, 197, 20], seed=23),
    # 64-key tile kernel (longer than the LDS-resident kernel holds): classes 1..10
    "b70_n577_h2": lambda: wl.custom(B=70, N=577, H=2,
                                     lengths=_lengths(70, 577, 2, [0, 1, 64, 65, 257, 320, 321, 576,
                                                                   577]), seed=24),
    # the tile list's longest images (15 key tiles)
    "b3_n960_h1": lambda: wl.custom(B=3, N=960, H=1, lengths=[960, 959, 1], seed=25),
    # fp32 input (always the tile kernel)
    "f32_b5_n300_h2": lambda: wl.custom(B=5, N=300, H=2, lengths=[300, 0, 65, 64, 129], dtype="f32",
                                        seed=26),
}


def _gathered(w, out_dtype):
    src = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    C = w.C
    o = sentinel_like((w.B * w.N, C), out_dtype)
    binding.rag_attn_gathered(keep, src[:, :C], src[:, C:2 * C], src[:, 2 * C:], o, H=w.H,
                              scale=w.scale)
    torch.cuda.synchronize()
    return o


def _check_oracle(w, ref, o32, images):
    packed_ref, cu_ref, _ = ref
    got = o32.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in images:
        s, e = int(cu_ref[b]), int(cu_ref[b + 1])
        if e == s:
            continue
        q, k, v = wl.split_qkv(packed_ref[s:e], w.C)
        want = oracle.attn(q, k, v, np.array([0, e - s], np.int32), w.H, w.d, w.scale)
        err = np.abs(got[s:e] - want).max()
        worst = max(worst, err)
        assert err <= ATOL, "image %d: max abs err %.3g" % (b, err)
    return worst


@pytest.mark.parametrize("name", sorted(CASES))
def test_tile_list_bit_for_bit_and_oracle(name):
    w = CASES[name]()
    mx = int(w.lengths.max())
    print("case", name, "B", w.B, "N", w.N, "H", w.H, "T", w.T, "max", mx, flush=True)
    ref = oracle.pack(w.keep, wl.rows(w))
    g = gpu_pack(w)
    T = w.T
    for out_dtype in (torch.float32, torch.bfloat16):
        tz = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=mx, tiled=True))
        assert (tz[T:].view(np.uint8) == SENTINEL_BYTE).all(), "rows past T written"
        grid = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=mx))
        assert (tz[:T].view(np.uint8) == grid[:T].view(np.uint8)).all(), "tile list != grid"
        if w.dtype == "bf16" and mx <= 256:
            gz = as_numpy_rows(_gathered(w, out_dtype))
            assert (gz[ref[2]].view(np.uint8) == tz[:T].view(np.uint8)).all(), "tile list != gathered"
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=mx, tiled=True)
    print("max abs err", _check_oracle(w, ref, o32, range(w.B)), flush=True)


@pytest.mark.parametrize("max_seqlen", [40, 100, 197])
def test_tile_list_short_and_truncating_bounds(max_seqlen):
    """The launch shapes max_seqlen selects (many pairs, B = 256: whole pairs on
    one-block waves up to 128 rows, on two-block waves beyond; few pairs, B = 2:
    whole pairs up to 64 rows, 64-row query tiles beyond), including bounds
    below the longest image (rows past max_seqlen are neither attended nor
    written)."""
    for B in (256, 2):
        rng = np.random.default_rng(28 + B)
        w = wl.custom(B=B, N=197, H=6, lengths=rng.integers(0, 198, size=B), seed=28 + B)
        g = gpu_pack(w)
        for out_dtype in (torch.float32, torch.bfloat16):
            a = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=max_seqlen,
                                       tiled=True))
            b = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=max_seqlen))
            assert (a.view(np.uint8) == b.view(np.uint8)).all(), (B, out_dtype)


def test_tile_list_largest_batch():
    """B = 1024 (the largest batch the tile list takes; 16 chunks of 64 images)
    against the gathered layout bit for bit, and sampled images against the
    oracle."""
    rng = np.random.default_rng(27)
    w = wl.custom(B=1024, N=197, H=1, lengths=rng.integers(0, 198, size=1024), seed=27)
    ref = oracle.pack(w.keep, wl.rows(w))
    g = gpu_pack(w)
    mx = int(w.lengths.max())
    o16 = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, torch.bfloat16, max_seqlen=mx, tiled=True))
    gz = as_numpy_rows(_gathered(w, torch.bfloat16))
    assert (gz[ref[2]].view(np.uint8) == o16[:w.T].view(np.uint8)).all()
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=mx, tiled=True)
    images = sorted(set(rng.choice(1024, size=12, replace=False).tolist())
                    | {0, 1023, int(np.argmax(w.lengths))})
    print("max abs err", _check_oracle(w, ref, o32, images), flush=True)


@pytest.mark.parametrize("seed", range(16))
def test_tile_list_random_shapes(seed):
    """Seeded random shapes inside the tile list's limits (B <= 1024, N <= 960,
    H <= 12, B N <= 40000): the tiled launch equals the grid launch bit for bit,
    rows past T and past the max_seqlen bound stay unwritten, and sampled images
    (fp32 output) are within the bar of the oracle."""
    rng = np.random.default_rng(50000 + seed)
    N = int(rng.integers(1, 961))
    B = int(rng.integers(1, min(1024, max(1, 40000 // N)) + 1))
    H = int(rng.integers(1, 13))
    kind = rng.integers(0, 4)
    if kind == 0:
        lengths = rng.integers(0, N + 1, size=B)
    elif kind == 1:
        lengths = np.full(B, int(rng.integers(0, N + 1)))
    elif kind == 2:
        lengths = rng.choice([0, 1, N], size=B)
    else:
        lengths = np.minimum(N, rng.geometric(0.02, size=B))
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    w = wl.custom(B=B, N=N, H=H, lengths=lengths, dtype=dtype, seed=60000 + seed)
    mx = int(w.lengths.max()) if w.T else 1
    bound = mx if rng.random() < 0.8 else int(rng.integers(1, mx + 1))
    od = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    print("seed", seed, "B", B, "N", N, "H", H, "T", w.T, dtype, od, "bound", bound, flush=True)
    g = gpu_pack(w, want_max=False)
    T = w.T
    a = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, od, max_seqlen=bound))
    b = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, od, max_seqlen=bound, tiled=True))
    assert (a.view(np.uint8) == b.view(np.uint8)).all(), "tile list != grid"
    assert (a[T:].view(np.uint8) == SENTINEL_BYTE).all(), "rows past T written"
    if T == 0:
        return
    o32 = a if od == torch.float32 else as_numpy_rows(
        gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=bound, tiled=True))
    packed_ref, cu_ref, _ = oracle.pack(w.keep, wl.rows(w))
    for im in rng.choice(B, size=min(B, 4), replace=False):
        s, e = int(cu_ref[im]), int(cu_ref[im + 1])
        L = min(e - s, bound)
        if L == 0:
            continue
        q, k, v = wl.split_qkv(packed_ref[s:s + L], w.C)
        want = oracle.attn(q, k, v, np.array([0, L], np.int32), w.H, w.d, w.scale)
        assert np.abs(o32[s:s + L].astype(np.float64) - want).max() <= ATOL, int(im)
        assert (a[s + L:e].view(np.uint8) == SENTINEL_BYTE).all(), "rows past the bound written"
