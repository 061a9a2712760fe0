"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: hand-derived worked
examples (tests/golden), a library routine that computes the same quantity
(numpy.flatnonzero, torch's bf16 conversion, torch's fp64 SDPA), closed forms,
invariants, and brute force written a different way (pure Python, math.fsum,
no max subtraction).  Chosen so that a dropped term, a wrong sign or index, a
transposed operand, a missing scale or a cross-image leak fails at least one.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from ragged_attention_token_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    data = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            data.setdefault(key, []).append(vals)
    return data


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- bf16 decode
def test_bf16_decode_exhaustive_matches_torch():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    # sign bit and exponent bias spot checks
    assert oracle.bf16_to_f64(0x3F80) == 1.0
    assert oracle.bf16_to_f64(0xBF80) == -1.0
    assert oracle.bf16_to_f64(0x4040) == 3.0
    assert oracle.bf16_to_f64(0x0001) == 2.0 ** -133


# ---------------------------------------------------------------------- pack
def test_pack_golden():
    g = _read_golden("pack_worked_example.txt")
    B, N = int(g["B"][0][0]), int(g["N"][0][0])
    keep = np.array([[int(x) for x in row] for row in g["keep"]], dtype=np.uint8)
    assert keep.shape == (B, N)
    src = np.arange(B * N * 4, dtype=np.int32).reshape(B * N, 4)
    packed, cu, gather = oracle.pack(keep, src)
    assert cu.tolist() == [int(x) for x in g["cu_seqlens"][0]]
    assert gather.tolist() == [int(x) for x in g["gather_idx"][0]]
    assert (packed == src[gather]).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("density", [0.0, 0.05, 0.5, 1.0])
def test_pack_matches_flatnonzero(seed, density):
    rng = np.random.default_rng(seed)
    B, N = 7, 37
    keep = (rng.random((B, N)) < density).astype(np.uint8) * rng.integers(1, 256, (B, N)).astype(np.uint8)
    src = rng.integers(0, 2 ** 16, size=(B * N, 24), dtype=np.uint16)
    packed, cu, gather = oracle.pack(keep, src)
    ref_gather = np.flatnonzero(keep.reshape(-1))
    assert (gather == ref_gather).all()
    ref_cu = np.concatenate([[0], np.cumsum(np.count_nonzero(keep, axis=1))])
    assert (cu == ref_cu).all()
    assert (packed == src[ref_gather]).all()


@pytest.mark.parametrize("make", [wl.tiny, lambda: wl.deits(4, 800), lambda: wl.deitb_ragged(64)])
def test_pack_invariants_on_workloads(make):
    w = make()
    rows = wl.rows(w)
    packed, cu, gather = oracle.pack(w.keep, rows)
    assert cu[0] == 0 and (np.diff(cu) >= 0).all()
    assert cu[-1] == np.count_nonzero(w.keep) == w.T
    assert (np.diff(cu) == w.lengths).all()
    for b in range(w.B):
        seg = gather[cu[b]:cu[b + 1]]
        assert (np.diff(seg) > 0).all()
        assert (seg // w.N == b).all()
        assert seg[0] == b * w.N  # CLS is always kept
    assert (packed == rows[gather]).all()


def test_unpack_roundtrip_and_sentinel():
    w = wl.deits(4, 800)
    rows = wl.rows(w)
    packed, cu, gather = oracle.pack(w.keep, rows)
    sentinel = np.full_like(rows, 0xA5A5)
    out = oracle.unpack(packed, cu, gather, sentinel)
    kept = w.keep.reshape(-1) != 0
    assert (out[kept] == rows[kept]).all()
    assert (out[~kept] == 0xA5A5).all()
    # golden indices
    g = _read_golden("pack_worked_example.txt")
    B, N = int(g["B"][0][0]), int(g["N"][0][0])
    keep = np.array([[int(x) for x in row] for row in g["keep"]], dtype=np.uint8)
    src = np.arange(B * N * 2, dtype=np.float32).reshape(B * N, 2)
    pk, cu2, ga = oracle.pack(keep, src)
    out2 = oracle.unpack(pk, cu2, ga, np.full_like(src, -1.0))
    mask = keep.reshape(-1) != 0
    assert (out2[mask] == src[mask]).all() and (out2[~mask] == -1.0).all()


# ----------------------------------------------------------------- attention
def test_attn_golden_worked_example():
    g = _read_golden("attn_worked_example.txt")
    d = int(g["d"][0][0])
    cu = np.array([int(x) for x in g["cu_seqlens"][0]], dtype=np.int32)
    q = _f32([[float(x) for x in r] for r in g["q"]])
    k = _f32([[float(x) for x in r] for r in g["k"]])
    v = _f32([[float(x) for x in r] for r in g["v"]])
    want = np.array([[float(x) for x in r] for r in g["o"]])
    got = oracle.attn(q, k, v, cu, H=1, d=d, scale=math.log(3.0))
    assert np.abs(got - want).max() < 1e-12


def _rand_case(rng, lengths, H, d, dtype="f32"):
    T = int(sum(lengths))
    x = rng.standard_normal((T, 3, H * d)).astype(np.float32)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return x, cu


def _decode(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    return a.astype(np.float64)


def test_attn_length_one_returns_v_row():
    rng = np.random.default_rng(3)
    x, cu = _rand_case(rng, [1, 1, 1], H=2, d=8)
    o = oracle.attn(x[:, 0], x[:, 1], x[:, 2], cu, H=2, d=8, scale=0.35)
    assert (o == x[:, 2].astype(np.float64)).all()


def test_attn_zero_query_or_zero_scale_gives_mean_of_v():
    rng = np.random.default_rng(4)
    x, cu = _rand_case(rng, [5, 3], H=2, d=8)
    for scale, q in ((0.7, np.zeros_like(x[:, 0])), (0.0, x[:, 0])):
        o = oracle.attn(np.ascontiguousarray(q), x[:, 1], x[:, 2], cu, H=2, d=8, scale=scale)
        for b in range(2):
            seg = slice(cu[b], cu[b + 1])
            mean = x[seg, 2].astype(np.float64).mean(axis=0)
            assert np.abs(o[seg] - mean).max() < 1e-12


def test_attn_constant_v_and_identical_keys():
    rng = np.random.default_rng(5)
    x, cu = _rand_case(rng, [6], H=1, d=8)
    vconst = np.tile(x[:1, 2], (6, 1))
    o = oracle.attn(x[:, 0], x[:, 1], vconst, cu, H=1, d=8, scale=0.5)
    assert np.abs(o - vconst[0].astype(np.float64)).max() < 1e-12
    ksame = np.tile(x[:1, 1], (6, 1))
    o2 = oracle.attn(x[:, 0], ksame, x[:, 2], cu, H=1, d=8, scale=0.5)
    assert np.abs(o2 - x[:, 2].astype(np.float64).mean(axis=0)).max() < 1e-12


def test_attn_probability_rows_sum_to_one():
    """With V the identity (one-hot rows, d >= L) the output row is the row of
    attention weights itself: non-negative, summing to 1, zero past column L."""
    rng = np.random.default_rng(11)
    L, d = 6, 8
    x, cu = _rand_case(rng, [L], H=1, d=d)
    v = np.zeros((L, d), dtype=np.float32)
    v[np.arange(L), np.arange(L)] = 1.0
    p = oracle.attn(x[:, 0], x[:, 1], v, cu, H=1, d=d, scale=0.9)
    assert (p >= 0).all()
    assert np.abs(p[:, :L].sum(axis=1) - 1.0).max() < 1e-12
    assert (p[:, L:] == 0).all()
    # the largest weight of each row sits on its largest score
    q, k = _decode(x[:, 0]), _decode(x[:, 1])
    assert (p[:, :L].argmax(axis=1) == (q @ k.T).argmax(axis=1)).all()


def test_attn_permutation_equivariant_within_image():
    rng = np.random.default_rng(6)
    x, cu = _rand_case(rng, [7, 5], H=2, d=8)
    o = oracle.attn(x[:, 0], x[:, 1], x[:, 2], cu, H=2, d=8, scale=0.3)
    perm = np.concatenate([rng.permutation(7), 7 + rng.permutation(5)])
    xp = x[perm]
    op = oracle.attn(xp[:, 0], xp[:, 1], xp[:, 2], cu, H=2, d=8, scale=0.3)
    assert np.abs(op - o[perm]).max() < 1e-13


def test_attn_bounded_by_v_and_no_leakage():
    rng = np.random.default_rng(7)
    x, cu = _rand_case(rng, [4, 9, 3], H=2, d=8)
    o = oracle.attn(x[:, 0], x[:, 1], x[:, 2], cu, H=2, d=8, scale=1.3)
    for b in range(3):
        seg = slice(cu[b], cu[b + 1])
        v = x[seg, 2].astype(np.float64)
        assert (o[seg] <= v.max(axis=0) + 1e-12).all() and (o[seg] >= v.min(axis=0) - 1e-12).all()
    y = x.copy()
    y[cu[1]:cu[2]] = rng.standard_normal(y[cu[1]:cu[2]].shape).astype(np.float32)
    o2 = oracle.attn(y[:, 0], y[:, 1], y[:, 2], cu, H=2, d=8, scale=1.3)
    assert (o2[cu[0]:cu[1]] == o[cu[0]:cu[1]]).all()
    assert (o2[cu[2]:cu[3]] == o[cu[2]:cu[3]]).all()
    assert not (o2[cu[1]:cu[2]] == o[cu[1]:cu[2]]).all()


def _brute_force(q, k, v, cu, H, d, scale):
    """Pure-Python loops, exp without max subtraction, math.fsum sums."""
    T = int(cu[-1])
    out = [[0.0] * (H * d) for _ in range(T)]
    for b in range(len(cu) - 1):
        rows = range(int(cu[b]), int(cu[b + 1]))
        for h in range(H):
            cols = range(h * d, h * d + d)
            for i in rows:
                w = {j: math.exp(scale * math.fsum(float(q[i][c]) * float(k[j][c]) for c in cols))
                     for j in rows}
                z = math.fsum(w.values())
                for c in cols:
                    out[i][c] = math.fsum(w[j] * float(v[j][c]) for j in rows) / z
    return np.array(out)


@pytest.mark.parametrize("lengths,H,d", [([1, 2, 3], 1, 4), ([5, 2], 2, 3), ([4, 1, 5], 2, 8)])
def test_attn_brute_force_tiny(lengths, H, d):
    rng = np.random.default_rng(sum(lengths) * 10 + H)
    x, cu = _rand_case(rng, lengths, H=H, d=d)
    q, k, v = (x[:, i].astype(np.float64).tolist() for i in range(3))
    want = _brute_force(q, k, v, cu, H, d, 0.4)
    got = oracle.attn(x[:, 0], x[:, 1], x[:, 2], cu, H=H, d=d, scale=0.4)
    assert np.abs(got - want).max() < 1e-12


def _sdpa_ref(q, k, v, cu, H, d, scale):
    """torch's fp64 SDPA on the CPU, one image at a time ([1, H, L, d])."""
    T = int(cu[-1])
    Q, K, V = (torch.from_numpy(_decode(a).reshape(-1, H * d)[:T]) for a in (q, k, v))
    out = torch.zeros(T, H * d, dtype=torch.float64)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e == s:
            continue
        qh, kh, vh = (X[s:e].reshape(e - s, H, d).transpose(0, 1).unsqueeze(0) for X in (Q, K, V))
        o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, scale=scale)
        out[s:e] = o[0].transpose(0, 1).reshape(e - s, H * d)
    return out.numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attn_matches_torch_sdpa_fp64(dtype):
    rng = np.random.default_rng(11)
    lengths = [33, 1, 70, 0, 12]
    x, cu = _rand_case(rng, lengths, H=3, d=64, dtype=dtype)
    got = oracle.attn(x[:, 0], x[:, 1], x[:, 2], cu, H=3, d=64, scale=0.125)
    want = _sdpa_ref(x[:, 0], x[:, 1], x[:, 2], cu, 3, 64, 0.125)
    assert np.abs(got - want).max() < 1e-12


def test_attn_rows_match_torch_sdpa_on_sampled_rows():
    """attn_rows (the sampled-row form used at sizes too large to compute whole)
    against torch's fp64 SDPA on the rows it is asked for: first and last rows
    of images, rows of images that follow empty ones, and random rows, in any
    order and with repeats."""
    rng = np.random.default_rng(19)
    lengths = [5, 0, 0, 40, 1, 0, 17]
    x, cu = _rand_case(rng, lengths, H=2, d=64, dtype="bf16")
    want = _sdpa_ref(x[:, 0], x[:, 1], x[:, 2], cu, 2, 64, 0.3)
    T = int(cu[-1])
    rows = [0, 4, 5, 44, 45, 46, 62, T - 1] + rng.integers(0, T, size=12).tolist() + [5, 0]
    got = oracle.attn_rows(x[:, 0], x[:, 1], x[:, 2], cu, H=2, d=64, scale=0.3, rows=rows)
    assert got.shape == (len(rows), 128)
    assert np.abs(got - want[rows]).max() < 1e-12


def test_attn_rows_rejects_rows_outside_the_batch():
    rng = np.random.default_rng(20)
    x, cu = _rand_case(rng, [3, 2], H=1, d=64, dtype="f32")
    for bad in ([5], [-1]):
        with pytest.raises(ValueError):
            oracle.attn_rows(x[:, 0], x[:, 1], x[:, 2], cu, H=1, d=64, scale=0.1, rows=bad)


def test_attn_on_tiny_workload_matches_sdpa():
    w = wl.tiny()
    rows = wl.rows(w)
    packed, cu, _ = oracle.pack(w.keep, rows)
    q, k, v = wl.split_qkv(packed, w.C)
    got = oracle.attn(q, k, v, cu, w.H, w.d, w.scale)
    want = _sdpa_ref(q, k, v, cu, w.H, w.d, w.scale)
    assert np.abs(got - want).max() < 1e-12


def test_keep_all_equals_dense_attention():
    w = wl.custom(B=2, N=23, H=2, lengths=[23, 23], dtype="bf16", seed=9)
    rows = wl.rows(w)
    packed, cu, gather = oracle.pack(w.keep, rows)
    assert (gather == np.arange(2 * 23)).all()
    q, k, v = wl.split_qkv(packed, w.C)
    got = oracle.attn(q, k, v, cu, w.H, w.d, w.scale)
    Q, K, V = (torch.from_numpy(_decode(np.ascontiguousarray(a))) for a in wl.split_qkv(rows, w.C))
    for b in range(2):
        for h in range(2):
            sl = slice(b * 23, (b + 1) * 23)
            cs = slice(h * 64, (h + 1) * 64)
            s = w.scale * Q[sl, cs] @ K[sl, cs].T
            ref = torch.softmax(s, dim=-1) @ V[sl, cs]
            assert (got[sl, cs] - ref.numpy()).__abs__().max() < 1e-12


# ------------------------------------------------------------ padded form
def test_padded_kept_rows_equal_ragged_and_dropped_rows_match_masked_sdpa():
    w = wl.custom(B=3, N=19, H=2, lengths=[5, 19, 1], dtype="bf16", seed=12)
    rows = wl.rows(w)
    q, k, v = wl.split_qkv(rows, w.C)
    pad = oracle.attn_padded(q, k, v, w.keep, w.H, w.d, w.scale)
    packed, cu, gather = oracle.pack(w.keep, rows)
    pq, pk, pv = wl.split_qkv(packed, w.C)
    rag = oracle.attn(pq, pk, pv, cu, w.H, w.d, w.scale)
    assert np.abs(pad[gather] - rag).max() < 1e-13
    # every query row (kept or dropped) against torch SDPA with a boolean key mask
    Q, K, V = (torch.from_numpy(_decode(np.ascontiguousarray(a))) for a in (q, k, v))
    for b in range(w.B):
        sl = slice(b * w.N, (b + 1) * w.N)
        mask = torch.from_numpy(w.keep[b] != 0)[None, None, None, :]
        qh, kh, vh = (X[sl].reshape(w.N, w.H, w.d).transpose(0, 1).unsqueeze(0) for X in (Q, K, V))
        o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=w.scale)
        ref = o[0].transpose(0, 1).reshape(w.N, w.C).numpy()
        assert np.abs(pad[sl] - ref).max() < 1e-12


def test_padded_empty_image_is_zero():
    w = wl.custom(B=2, N=8, H=1, lengths=[0, 3], d=16, dtype="f32", seed=13)
    rows = wl.rows(w)
    q, k, v = wl.split_qkv(rows, w.C)
    pad = oracle.attn_padded(q, k, v, w.keep, w.H, w.d, w.scale)
    assert (pad[:8] == 0).all()
    assert np.isfinite(pad).all()


# -------------------------------------------------------------- workloads
def test_workload_shapes_and_lengths():
    t = wl.tiny()
    assert (t.B, t.N, t.H, t.d, t.dtype) == (2, 197, 3, 64, "f32")
    assert sorted(t.lengths.tolist()) == [40, 99] and (t.keep[:, 0] == 1).all()
    s = wl.deits(4, 800)
    assert (s.lengths == 40).all() and s.C == 384 and s.dtype == "bf16"
    r = wl.deitb_ragged(64)
    assert r.lengths.min() >= 20 and r.lengths.max() <= 197 and r.C == 768
    b384 = wl.deitb384(32)
    assert b384.N == 577 and b384.lengths.min() >= 231 and b384.lengths.max() <= 347
    assert [wl.kept_length(197, p) for p in (0, 500, 800, 900)] == [197, 99, 40, 20]
    # bf16 rounding of the draws is round-to-nearest-even of the fp32 draw
    x = np.random.default_rng(0).standard_normal(1000, dtype=np.float32)
    bits = wl._to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert (np.abs(back - x) <= np.abs(x) * 2.0 ** -8).all()


def _random_keep(rng, shape, density):
    keep = (rng.random(shape) < density).astype(np.uint8)
    return keep * rng.integers(1, 256, shape).astype(np.uint8)  # any nonzero byte keeps


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("d1,d2", [(0.5, 0.5), (0.9, 0.2), (1.0, 1.0), (0.3, 0.0)])
def test_repack_equals_pack_of_the_composed_mask(seed, d1, d2):
    """Two pruning stages: pack with k1, then re-pack the packed rows with k2.
    The result is pack with the composed mask (kept by both), gather indices
    included: a second formulation of the same compaction."""
    rng = np.random.default_rng(seed)
    B, N = 6, 41
    k1 = _random_keep(rng, (B, N), d1)
    src = rng.integers(0, 2 ** 16, size=(B * N, 12), dtype=np.uint16)
    p1, cu1, g1 = oracle.pack(k1, src)
    k2 = _random_keep(rng, (p1.shape[0],), d2)
    p2, cu2, g2 = oracle.repack(k2, cu1, g1, p1)
    k12 = np.zeros(B * N, dtype=np.uint8)
    k12[g1[k2 != 0]] = 1
    ref_p, ref_cu, ref_g = oracle.pack(k12.reshape(B, N), src)
    assert (cu2 == ref_cu).all()
    assert (g2 == ref_g).all()
    assert (p2 == ref_p).all()


def test_repack_keep_all_is_identity_and_keep_none_is_empty():
    w = wl.deitb_ragged(64)
    rows = wl.rows(w)
    p1, cu1, g1 = oracle.pack(w.keep, rows)
    p2, cu2, g2 = oracle.repack(np.full(p1.shape[0], 7, np.uint8), cu1, g1, p1)
    assert (cu2 == cu1).all() and (g2 == g1).all() and (p2 == p1).all()
    p3, cu3, g3 = oracle.repack(np.zeros(p1.shape[0], np.uint8), cu1, g1, p1)
    assert p3.shape[0] == 0 and (cu3 == 0).all() and g3.shape[0] == 0
    # an empty packed batch (every image dropped) re-packs to an empty batch
    p4, cu4, g4 = oracle.repack(np.zeros(0, np.uint8), cu3, g3, p3)
    assert p4.shape == (0, p1.shape[1]) and (cu4 == 0).all() and g4.shape[0] == 0


def test_repack_brute_force_per_image():
    """Image by image with numpy: the surviving rows of image b, in order."""
    rng = np.random.default_rng(5)
    cu_in = np.array([0, 3, 3, 10, 11, 20], dtype=np.int32)
    T = int(cu_in[-1])
    gather_in = np.sort(rng.choice(1000, size=T, replace=False)).astype(np.int32)
    rows = rng.integers(0, 2 ** 31, size=(T, 4), dtype=np.int32)
    keep = _random_keep(rng, (T,), 0.6)
    out, cu_out, g_out = oracle.repack(keep, cu_in, gather_in, rows)
    t = 0
    for b in range(cu_in.shape[0] - 1):
        sel = [r for r in range(cu_in[b], cu_in[b + 1]) if keep[r] != 0]
        assert cu_out[b] == t and cu_out[b + 1] == t + len(sel)
        for i, r in enumerate(sel):
            assert g_out[t + i] == gather_in[r]
            assert (out[t + i] == rows[r]).all()
        t += len(sel)


# ---- the ViT block reference (end-to-end timing row) -----------------------
from oracle import vit_block as vb  # noqa: E402


def test_layernorm_golden():
    g = _read_golden("layernorm_worked_example.txt")
    x = np.array([[float(v) for v in g["x"][0]]])
    want = np.array([float(v) for v in g["y"][0]])
    got = vb.layernorm(x, np.ones(4), np.zeros(4), 0.0)[0]
    assert np.abs(got - want).max() < 1e-15


def test_gelu_forms_against_the_normal_cdf_table():
    """erf form: x * Phi(x), with Phi from a printed normal table (Phi(1) =
    0.8413447, Phi(2) = 0.9772499, Phi(-1) = 0.1586553); the tanh form stays
    within 5e-4 of it everywhere and is not the same function (it falls short
    of Phi by ~24% relative at x = -3.5)."""
    table = {1.0: 0.8413447, 2.0: 0.9772499, -1.0: 0.1586553}
    for xv, phi in table.items():
        assert abs(vb.gelu(np.array([xv]), "erf")[0] - xv * phi) < 2e-7
    xs = np.linspace(-8, 8, 4001)
    e, t = vb.gelu(xs, "erf"), vb.gelu(xs, "tanh")
    assert np.abs(e - t).max() < 5e-4
    assert vb.gelu(np.array([0.0]), "tanh")[0] == 0.0
    assert abs(vb.gelu(np.array([-3.5]), "tanh")[0] / vb.gelu(np.array([-3.5]), "erf")[0] - 0.757) < 0.01


def test_block_attention_step_matches_the_c_oracle():
    """The block's numpy attention against oracle.attn (C) on bf16-exact q|k|v
    rows: two independent implementations of the same definition."""
    w = wl.deits(3, 800)
    rows = wl.rows(w)
    packed, cu, _ = oracle.pack(w.keep, rows)
    q, k, v = wl.split_qkv(packed, w.C)
    want = oracle.attn(q, k, v, cu, w.H, w.d, w.scale)
    got = vb.attention(vb.bf16_bits_to_f64(packed), cu, w.H, w.d, w.scale)
    assert np.abs(got - want).max() < 1e-12


def test_block_with_zero_weights_is_the_identity():
    C = 128
    P = wl.vit_block_params(C, 4, 0)
    for k in P:
        if k.startswith(("w_", "b_")):
            P[k] = np.zeros_like(P[k])
    x = wl.hidden_rows(2, 7, C, 1)
    y = vb.block(x, P, np.array([0, 5, 14]), 2, 0.125)
    assert (y == vb.bf16_bits_to_f64(x)).all()


def _block_brute_force(x, P, cu, H, d, scale, eps, form):
    """Pure-Python loops, tiny sizes: the block written element by element."""
    T, C = len(x), len(x[0])

    def ln(rows, g, b):
        out = []
        for r in rows:
            mu = math.fsum(r) / C
            var = math.fsum((v - mu) ** 2 for v in r) / C
            out.append([(r[c] - mu) / math.sqrt(var + eps) * g[c] + b[c] for c in range(C)])
        return out

    def mm(A, Wt, bias):
        return [[math.fsum(A[i][k] * Wt[k][j] for k in range(len(Wt))) + bias[j]
                 for j in range(len(Wt[0]))] for i in range(len(A))]

    def act(v):
        if form == "erf":
            return 0.5 * v * (1 + math.erf(v / math.sqrt(2)))
        return 0.5 * v * (1 + math.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3)))

    xs = [list(r) for r in x]
    h = ln(xs, P["ln1_gamma"], P["ln1_beta"])
    qkv = mm(h, P["w_qkv"], P["b_qkv"])
    a = [[0.0] * C for _ in range(T)]
    for b in range(len(cu) - 1):
        for hh in range(H):
            for i in range(cu[b], cu[b + 1]):
                s = [scale * math.fsum(qkv[i][hh * d + c] * qkv[j][C + hh * d + c] for c in range(d))
                     for j in range(cu[b], cu[b + 1])]
                mx = max(s)
                e = [math.exp(v - mx) for v in s]
                z = math.fsum(e)
                for c in range(d):
                    a[i][hh * d + c] = math.fsum(
                        e[jj] / z * qkv[cu[b] + jj][2 * C + hh * d + c] for jj in range(len(e)))
    pa = mm(a, P["w_proj"], P["b_proj"])
    x1 = [[xs[i][c] + pa[i][c] for c in range(C)] for i in range(T)]
    f1 = mm(ln(x1, P["ln2_gamma"], P["ln2_beta"]), P["w_fc1"], P["b_fc1"])
    m = [[act(v) for v in r] for r in f1]
    f2 = mm(m, P["w_fc2"], P["b_fc2"])
    return np.array([[x1[i][c] + f2[i][c] for c in range(C)] for i in range(T)])


@pytest.mark.parametrize("form", ["erf", "tanh"])
def test_block_brute_force_tiny(form):
    """C = 4 (two heads of width 2), images of 3, 1 and 2 rows; weights that are
    not symmetric, so a transposed operand or a swapped q/k/v block shows."""
    rng = np.random.default_rng(7)
    C, H, d, hid = 4, 2, 2, 8
    P = {"w_qkv": rng.standard_normal((C, 3 * C)), "w_proj": rng.standard_normal((C, C)),
         "w_fc1": rng.standard_normal((C, hid)), "w_fc2": rng.standard_normal((hid, C)),
         "b_qkv": rng.standard_normal(3 * C), "b_proj": rng.standard_normal(C),
         "b_fc1": rng.standard_normal(hid), "b_fc2": rng.standard_normal(C),
         "ln1_gamma": 1 + rng.standard_normal(C), "ln1_beta": rng.standard_normal(C),
         "ln2_gamma": 1 + rng.standard_normal(C), "ln2_beta": rng.standard_normal(C)}
    x = rng.standard_normal((6, C))
    cu = [0, 3, 4, 6]
    bits = lambda a: np.asarray(a, np.float32)  # noqa: E731
    # the oracle takes bf16 bit patterns for x and matrices: round the draws
    # to bf16 first so both sides see the same exact values
    Pb = dict(P)
    for k in ("w_qkv", "w_proj", "w_fc1", "w_fc2"):
        Pb[k] = wl._to_bf16_bits(bits(P[k]))
        P[k] = vb.bf16_bits_to_f64(Pb[k])
    xb = wl._to_bf16_bits(bits(x))
    xv = vb.bf16_bits_to_f64(xb)
    for k in P:
        if not k.startswith("w_"):
            Pb[k] = bits(P[k])
            P[k] = Pb[k].astype(np.float64)
    got = vb.block(xb, Pb, np.array(cu), H, 0.7, eps=1e-5, gelu_form=form, d=d)
    want = _block_brute_force(xv.tolist(), {k: (v.tolist() if hasattr(v, "tolist") else v)
                                            for k, v in P.items()}, cu, H, d, 0.7, 1e-5, form)
    assert np.abs(got - want).max() < 1e-11


def test_block_matches_torch_transformer_encoder_layer_fp64():
    """The block's composition against an implementation that shares nothing
    with it: torch's nn.TransformerEncoderLayer in float64 on the CPU, built as
    DeiT's pre-norm block (norm_first, exact GELU, LayerNorm eps 1e-6, MLP 4C,
    no dropout) and given the same weights (torch's Linear stores [out, in]:
    the transposes of the [in, out] matrices here; the attention's in-projection
    rows are q | k | v, each split into heads of 64 columns).  Each image of the
    packed batch is run through torch on its own, which is what the block's
    attention over cu_seqlens means."""
    import torch
    H, d = 2, 64
    C = H * d
    P = wl.vit_block_params(C, 4, 21)
    lengths = [5, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x = wl.hidden_rows(1, int(cu[-1]), C, 22)
    got = vb.block(x, P, cu, H, 1.0 / math.sqrt(d))

    layer = torch.nn.TransformerEncoderLayer(
        d_model=C, nhead=H, dim_feedforward=4 * C, dropout=0.0, activation="gelu",
        layer_norm_eps=1e-6, batch_first=True, norm_first=True, dtype=torch.float64)
    f64 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731
    W = {k: vb.bf16_bits_to_f64(P[k]) for k in ("w_qkv", "w_proj", "w_fc1", "w_fc2")}
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(f64(W["w_qkv"].T))
        layer.self_attn.in_proj_bias.copy_(f64(P["b_qkv"]))
        layer.self_attn.out_proj.weight.copy_(f64(W["w_proj"].T))
        layer.self_attn.out_proj.bias.copy_(f64(P["b_proj"]))
        layer.linear1.weight.copy_(f64(W["w_fc1"].T))
        layer.linear1.bias.copy_(f64(P["b_fc1"]))
        layer.linear2.weight.copy_(f64(W["w_fc2"].T))
        layer.linear2.bias.copy_(f64(P["b_fc2"]))
        layer.norm1.weight.copy_(f64(P["ln1_gamma"]))
        layer.norm1.bias.copy_(f64(P["ln1_beta"]))
        layer.norm2.weight.copy_(f64(P["ln2_gamma"]))
        layer.norm2.bias.copy_(f64(P["ln2_beta"]))
        layer.eval()
        xv = vb.bf16_bits_to_f64(x)
        want = np.concatenate([layer(f64(xv[cu[b]:cu[b + 1]])[None])[0].numpy()
                               for b in range(len(lengths))])
    assert np.abs(got - want).max() < 1e-10, np.abs(got - want).max()
    # the exact GELU is the one that matches: the tanh form lands visibly apart
    other = vb.block(x, P, cu, H, 1.0 / math.sqrt(d), gelu_form="tanh")
    assert np.abs(other - want).max() > 1e-6


def test_block_images_are_independent():
    """Rows of one image do not move when another image's rows change."""
    C = 128
    P = wl.vit_block_params(C, 2, 3)
    x = wl.hidden_rows(1, 9, C, 4)
    cu = np.array([0, 4, 9])
    y1 = vb.block(x, P, cu, 2, 0.125)
    x2 = x.copy()
    x2[4:] = wl.hidden_rows(1, 5, C, 5)
    y2 = vb.block(x2, P, cu, 2, 0.125)
    assert (y1[:4] == y2[:4]).all() and not (y1[4:] == y2[4:]).all()
