"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: pack / unpack bit-exact (indices and bytes, capacity tails untouched);
attention within 2e-3 max abs error of fp64 attention for fp32 output; bf16
output is the round-to-nearest-even of the fp32 output, bit for bit, and so lies
within 2e-3 + 2^-8 |o| of the oracle.  The oracle always computes from the
workload's own inputs (its own packing), never from a GPU result.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (SENTINEL_BYTE, as_numpy_rows, bf16_bits_to_f64, gpu_attn, gpu_pack,
                         sentinel_like, to_gpu_rows, torch_dtype)
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3

FULL = {  # workloads the oracle finishes in seconds: compared on every output
    "tiny": wl.tiny,
    "deits_b4_p800": lambda: wl.deits(4, 800),
    "deitb_ragged_b64": lambda: wl.deitb_ragged(64),
    "deits_b1_p000": lambda: wl.deits(1, 0),
    "deits_b2_p500": lambda: wl.deits(2, 500),
    "deits_b4_p900": lambda: wl.deits(4, 900),
    "deits_b1_p800": lambda: wl.deits(1, 800),
    "empty_and_full": lambda: wl.custom(B=5, N=197, H=6, lengths=[0, 197, 1, 0, 64], seed=3),
    "n5_golden_like": lambda: wl.custom(B=3, N=5, H=2, lengths=[3, 0, 3], keep_kind="uniform",
                                        seed=4),
    "n1": lambda: wl.custom(B=5, N=1, H=1, lengths=[1, 0, 1, 1, 0], seed=5),
    "tile_edges": lambda: wl.custom(B=6, N=129, H=3, lengths=[63, 64, 65, 128, 129, 16], seed=6),
    "n577_two": lambda: wl.custom(B=2, N=577, H=2, lengths=[577, 2], seed=7),
    "f32_odd": lambda: wl.custom(B=3, N=70, H=2, lengths=[70, 33, 5], dtype="f32", seed=8),
}
SAMPLED = {  # full-size workloads: pack/unpack compared whole, attention on sampled images
    "deitb384_b32": (lambda: wl.deitb384(32), 6),
    "deits_b256_p000": (lambda: wl.deits(256, 0), 4),
    "deits_b256_p500": (lambda: wl.deits(256, 500), 6),
    "deits_b256_p800": (lambda: wl.deits(256, 800), 8),
    "deits_b256_p900": (lambda: wl.deits(256, 900), 8),
}


def _oracle_pack(w):
    return oracle.pack(w.keep, wl.rows(w))


def _check_pack(w, g, ref):
    packed_ref, cu_ref, gather_ref = ref
    T = int(cu_ref[-1])
    cu = g["cu"].cpu().numpy()
    assert (cu == cu_ref).all(), "cu_seqlens differ"
    gather = g["gather"].cpu().numpy()
    assert (gather[:T] == gather_ref).all(), "gather_idx differs"
    assert (gather[T:].view(np.uint32) == np.uint32(0xA5A5A5A5)).all(), "gather tail written"
    packed = as_numpy_rows(g["packed"])
    assert (packed[:T].view(np.uint8) == packed_ref.view(np.uint8)).all(), "packed bytes differ"
    assert (packed[T:].view(np.uint8) == SENTINEL_BYTE).all(), "packed tail written"
    assert int(g["max"].item()) == int(w.lengths.max())


def _oracle_attn_images(w, ref, images):
    """Oracle attention for the listed images only, from the oracle's own packing."""
    packed_ref, cu_ref, _ = ref
    out = {}
    for b in images:
        s, e = int(cu_ref[b]), int(cu_ref[b + 1])
        if e == s:
            continue
        q, k, v = wl.split_qkv(packed_ref[s:e], w.C)
        out[b] = oracle.attn(q, k, v, np.array([0, e - s], np.int32), w.H, w.d, w.scale)
    return out


def _check_attn(w, ref, o_f32, o_bf16, images):
    cu_ref = ref[1]
    o32 = o_f32.cpu().numpy().astype(np.float64)
    o16 = as_numpy_rows(o_bf16)
    # bf16 output is RNE of the fp32 output (same kernel, epilogue rounding only)
    rne = o_f32.cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    T = int(cu_ref[-1])
    assert (o16[:T] == rne[:T]).all(), "bf16 output is not RNE(fp32 output)"
    worst = 0.0
    for b, want in _oracle_attn_images(w, ref, images).items():
        s, e = int(cu_ref[b]), int(cu_ref[b + 1])
        err = np.abs(o32[s:e] - want).max()
        worst = max(worst, err)
        assert err <= ATOL, "image %d: max abs err %.3g" % (b, err)
        err16 = np.abs(bf16_bits_to_f64(o16[s:e]) - want) - (ATOL + np.abs(want) * 2.0 ** -8)
        assert (err16 <= 0).all(), "image %d: bf16 output outside its bound" % b
    return worst


@pytest.mark.parametrize("name", sorted(FULL))
def test_pack_and_attention_full(name):
    w = FULL[name]()
    print("case", name, "B", w.B, "N", w.N, "H", w.H, "T", w.T, flush=True)
    ref = _oracle_pack(w)
    g = gpu_pack(w)
    _check_pack(w, g, ref)
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32)
    o16 = gpu_attn(g["packed"], g["cu"], w, torch.bfloat16)
    worst = _check_attn(w, ref, o32, o16, range(w.B))
    print("max abs err", worst, flush=True)
    # rows past T are never written
    T = w.T
    assert (as_numpy_rows(o32)[T:].view(np.uint8) == SENTINEL_BYTE).all()


@pytest.mark.parametrize("name", sorted(SAMPLED))
def test_pack_and_attention_full_size_sampled(name):
    make, nsample = SAMPLED[name]
    w = make()
    print("case", name, "B", w.B, "N", w.N, "H", w.H, "T", w.T, flush=True)
    ref = _oracle_pack(w)
    g = gpu_pack(w)
    _check_pack(w, g, ref)
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32)
    o16 = gpu_attn(g["packed"], g["cu"], w, torch.bfloat16)
    rng = np.random.default_rng(0)
    images = sorted(set(rng.choice(w.B, size=min(nsample, w.B), replace=False).tolist())
                    | {0, w.B - 1})
    worst = _check_attn(w, ref, o32, o16, images)
    print("max abs err over", images, worst, flush=True)
    o = o32.cpu().numpy()
    assert np.isfinite(o[:w.T]).all()


def test_keep_bytes_other_than_one_count_as_kept():
    w = wl.custom(B=4, N=197, H=6, lengths=[40, 100, 1, 197], seed=10)
    rng = np.random.default_rng(1)
    w.keep = (w.keep * rng.integers(1, 256, w.keep.shape)).astype(np.uint8)
    ref = _oracle_pack(w)
    _check_pack(w, gpu_pack(w), ref)


def test_length_one_returns_v_row():
    """A one-token image attends only to itself, so O is its V row.  The
    kernel's exponent is fma(s, c, -m) with m the rounded c*s_max, so the single
    weight is 2^r (r = that rounding residual, |r| <= 2^-24 |m|) carried as
    bf16 hi + lo: O matches V to about 2^-16 relative, not bit for bit."""
    w = wl.custom(B=7, N=33, H=6, lengths=[1] * 7, seed=11)
    g = gpu_pack(w)
    o = gpu_attn(g["packed"], g["cu"], w, torch.float32).cpu().numpy()
    packed_ref, cu_ref, _ = _oracle_pack(w)
    v = bf16_bits_to_f64(packed_ref[:, 2 * w.C:3 * w.C])
    assert (np.abs(o[:w.T].astype(np.float64) - v) <= np.abs(v) * 2.0 ** -14 + 1e-30).all()


def test_attention_is_deterministic():
    w = wl.deitb_ragged(64)
    g = gpu_pack(w)
    a = gpu_attn(g["packed"], g["cu"], w, torch.float32)
    b = gpu_attn(g["packed"], g["cu"], w, torch.float32)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_max_seqlen_larger_than_needed_changes_nothing():
    w = wl.deits(4, 800)
    g = gpu_pack(w)
    a = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=40)
    b = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=197)
    assert torch.equal(a[:w.T].view(torch.int32), b[:w.T].view(torch.int32))


@pytest.mark.parametrize("flags", [0, binding.RAG_UNPACK_ZERO_DROPPED])
def test_unpack_bit_exact(flags):
    w = wl.deitb_ragged(64)
    _, cu_ref, gather_ref = _oracle_pack(w)
    T = int(cu_ref[-1])
    rng = np.random.default_rng(12)
    packed = rng.integers(0, 2 ** 16, size=(w.B * w.N, w.C), dtype=np.uint16)
    dst0 = np.full((w.B * w.N, w.C), 0xA5A5, dtype=np.uint16)
    want = oracle.unpack(packed[:T], cu_ref, gather_ref, dst0)
    if flags:
        want[w.keep.reshape(-1) == 0] = 0
    gather_full = np.zeros(w.B * w.N, np.int32)
    gather_full[:T] = gather_ref
    dev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    dst = dev(dst0.copy())
    binding.rag_unpack(dev(packed), dev(cu_ref), dev(gather_full), dst, N=w.N, flags=flags)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16)
    assert (got == want).all()


def test_padded_comparator():
    for w in (wl.deits(4, 800), wl.custom(B=3, N=70, H=2, lengths=[70, 0, 9], dtype="f32", seed=13),
              wl.deitb384(2)):
        print("padded case", w.name, flush=True)
        src = to_gpu_rows(w)
        keep = torch.from_numpy(w.keep).cuda()
        C = w.C
        o = sentinel_like((w.B * w.N, C), torch.float32)
        binding.rag_attn_padded(src[:, :C], src[:, C:2 * C], src[:, 2 * C:], keep, o, H=w.H,
                                scale=w.scale)
        torch.cuda.synchronize()
        rows = wl.rows(w)
        q, k, v = wl.split_qkv(rows, C)
        want = oracle.attn_padded(q, k, v, w.keep, w.H, w.d, w.scale)
        got = o.cpu().numpy().astype(np.float64)
        err = np.abs(got - want).max()
        print("padded max abs err", err, flush=True)
        assert err <= ATOL


def _pipeline_buffers(w, out_dtype):
    B, N, C = w.B, w.N, w.C
    bufs = dict(
        keep=torch.from_numpy(w.keep).cuda(), src=to_gpu_rows(w),
        packed=sentinel_like((B * N, 3 * C), torch_dtype(w)),
        cu=sentinel_like((B + 1,), torch.int32), gather=sentinel_like((B * N,), torch.int32),
        o_packed=sentinel_like((B * N, C), out_dtype), dst=sentinel_like((B * N, C), out_dtype),
        mx=sentinel_like((1,), torch.int32))
    return bufs


def _make_pipeline(w, bufs, flags=0):
    return binding.Pipeline(bufs["keep"], bufs["src"], bufs["packed"], bufs["cu"], bufs["gather"],
                            bufs["o_packed"], bufs["dst"], H=w.H, scale=w.scale,
                            max_seqlen_dev=bufs["mx"], unpack_flags=flags)


@pytest.mark.parametrize("name,out_dtype", [("deits_b256_p800", torch.bfloat16),
                                            ("tiny", torch.float32),
                                            ("deitb_ragged_b64", torch.float32)])
def test_pipeline_graph_replays_match_eager_and_oracle(name, out_dtype):
    w = {"deits_b256_p800": lambda: wl.deits(256, 800), "tiny": wl.tiny,
         "deitb_ragged_b64": lambda: wl.deitb_ragged(64)}[name]()
    print("pipeline case", name, flush=True)
    bufs = _pipeline_buffers(w, out_dtype)
    pipe = _make_pipeline(w, bufs)
    pipe.launch_eager()
    torch.cuda.synchronize()
    eager = {k: bufs[k].clone() for k in ("packed", "cu", "gather", "o_packed", "dst", "mx")}
    for rep in range(3):
        for k in ("packed", "cu", "gather", "o_packed", "dst"):
            bufs[k].view(torch.uint8).fill_(SENTINEL_BYTE)
        torch.cuda.synchronize()
        pipe.launch()
        torch.cuda.synchronize()
        for k, t in eager.items():
            assert torch.equal(bufs[k].view(torch.uint8), t.view(torch.uint8)), (rep, k)
        scratch = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del scratch
    # against the oracle
    ref = _oracle_pack(w)
    g = dict(cu=bufs["cu"], gather=bufs["gather"], packed=bufs["packed"], max=bufs["mx"])
    _check_pack(w, g, ref)
    images = range(w.B) if w.B <= 64 else [0, 1, 77, 128, 255]
    want = _oracle_attn_images(w, ref, images)
    dst = as_numpy_rows(bufs["dst"])
    o_packed = as_numpy_rows(bufs["o_packed"])
    _, cu_ref, gather_ref = ref
    T = int(cu_ref[-1])
    # unpack is a byte copy of the attention output to the kept rows
    assert (dst[gather_ref].view(np.uint8) == o_packed[:T].view(np.uint8)).all()
    dropped = np.setdiff1d(np.arange(w.B * w.N), gather_ref)
    assert (dst[dropped].view(np.uint8) == SENTINEL_BYTE).all()
    for b, ref_o in want.items():
        s, e = int(cu_ref[b]), int(cu_ref[b + 1])
        got = dst[gather_ref[s:e]]
        got = bf16_bits_to_f64(got) if out_dtype == torch.bfloat16 else got.astype(np.float64)
        tol = ATOL + (np.abs(ref_o) * 2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0)
        assert (np.abs(got - ref_o) <= tol).all(), b
    pipe.close()


def test_pipeline_zero_dropped_flag():
    w = wl.deits(4, 800)
    bufs = _pipeline_buffers(w, torch.float32)
    pipe = _make_pipeline(w, bufs, flags=binding.RAG_UNPACK_ZERO_DROPPED)
    pipe.launch()
    torch.cuda.synchronize()
    dst = bufs["dst"].cpu().numpy()
    assert (dst[w.keep.reshape(-1) == 0] == 0).all()
    assert np.isfinite(dst).all()
    pipe.close()


def test_dispatch_measurement_runs():
    w = wl.deits(1, 800)
    bufs = _pipeline_buffers(w, torch.bfloat16)
    pipe = _make_pipeline(w, bufs)
    res = pipe.measure_dispatch(warmup=5, iters=20)
    for k, v in res.items():
        assert 0 < v["p10"] <= v["p50"] <= v["p90"] < 1e6, (k, v)
    pipe.close()


def test_stage_measurement_runs():
    w = wl.deits(4, 800)
    bufs = _pipeline_buffers(w, torch.bfloat16)
    pipe = _make_pipeline(w, bufs)
    res = pipe.measure_stages(iters=20)
    assert set(res) == {"pack", "attn", "unpack", "padded", "eager_pass", "graph_pass", "fused_pass"}
    for k, v in res.items():
        assert 0 < v < 1e5, (k, v)
    pipe.close()


def _gathered(w, out_dtype, flags=0):
    src = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    C = w.C
    o = sentinel_like((w.B * w.N, C), out_dtype)
    binding.rag_attn_gathered(keep, src[:, :C], src[:, C:2 * C], src[:, 2 * C:], o, H=w.H,
                              scale=w.scale, flags=flags)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("name", ["tiny", "deits_b4_p800", "deitb_ragged_b64", "empty_and_full", "deits_b1_p000",
                                  "n1", "tile_edges", "n577_two", "f32_odd", "n5_golden_like"])
def test_gathered_equals_three_stage_pipeline_and_oracle(name):
    w = FULL[name]()
    print("gathered case", name, flush=True)
    ref = _oracle_pack(w)
    packed_ref, cu_ref, gather_ref = ref
    g = gpu_pack(w)
    for out_dtype in (torch.float32, torch.bfloat16):
        staged = gpu_attn(g["packed"], g["cu"], w, out_dtype)
        fused = _gathered(w, out_dtype)
        fz = as_numpy_rows(fused)
        sz = as_numpy_rows(staged)
        T = w.T
        # bit for bit the packed result, at the kept rows; dropped rows untouched
        assert (fz[gather_ref].view(np.uint8) == sz[:T].view(np.uint8)).all()
        dropped = np.setdiff1d(np.arange(w.B * w.N), gather_ref)
        assert (fz[dropped].view(np.uint8) == SENTINEL_BYTE).all()
    got = as_numpy_rows(_gathered(w, torch.float32)).astype(np.float64)
    for b, want in _oracle_attn_images(w, ref, range(w.B)).items():
        s_, e_ = int(cu_ref[b]), int(cu_ref[b + 1])
        assert np.abs(got[gather_ref[s_:e_]] - want).max() <= ATOL, b


def test_gathered_unpruned_images_and_single_dropped_rows():
    """Few (image, head) pairs with max_seqlen = N: the one-launch pass requests
    K, V and Q in natural order beside the keep bytes and keeps them only when
    every row of the image is kept.  Images with all rows kept, or one dropped
    row at a position read by lane 0 of a wave (64, 128), by other lanes (1,
    100) or at the end (196), or a kept prefix, must all equal the three-stage
    result bit for bit and leave the dropped rows untouched."""
    N, H = 197, 2
    masks = [np.ones(N, np.uint8)]
    for drop in (1, 64, 100, 128, 196):
        m = np.ones(N, np.uint8)
        m[drop] = 0
        masks.append(m)
    prefix = np.zeros(N, np.uint8)
    prefix[:150] = 1
    masks += [prefix, np.ones(N, np.uint8)]
    B = len(masks)
    w = wl.custom(B=B, N=N, H=H, lengths=[int(m.sum()) for m in masks], keep_kind="prefix", seed=24)
    w.keep = np.stack(masks).astype(np.uint8)
    print("case natural-order gathered B", B, "N", N, "H", H, flush=True)
    ref = _oracle_pack(w)
    _, cu_ref, gather_ref = ref
    g = gpu_pack(w)
    for out_dtype in (torch.float32, torch.bfloat16):
        staged = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, out_dtype))
        fused = as_numpy_rows(_gathered(w, out_dtype))
        assert (fused[gather_ref].view(np.uint8) == staged[:w.T].view(np.uint8)).all()
        dropped = np.setdiff1d(np.arange(w.B * w.N), gather_ref)
        assert (fused[dropped].view(np.uint8) == SENTINEL_BYTE).all()
    got = as_numpy_rows(_gathered(w, torch.float32)).astype(np.float64)
    for b, want in _oracle_attn_images(w, ref, range(w.B)).items():
        s_, e_ = int(cu_ref[b]), int(cu_ref[b + 1])
        assert np.abs(got[gather_ref[s_:e_]] - want).max() <= ATOL, b


@pytest.mark.parametrize("name", ["deits_b256_p800", "deitb384_b32", "deits_b256_p000"])
def test_gathered_full_size_sampled(name):
    make, nsample = SAMPLED[name]
    w = make()
    print("gathered full-size case", name, flush=True)
    ref = _oracle_pack(w)
    _, cu_ref, gather_ref = ref
    got = as_numpy_rows(_gathered(w, torch.float32)).astype(np.float64)
    rng = np.random.default_rng(1)
    images = sorted(set(rng.choice(w.B, size=min(nsample, w.B), replace=False).tolist()) | {w.B - 1})
    for b, want in _oracle_attn_images(w, ref, images).items():
        s_, e_ = int(cu_ref[b]), int(cu_ref[b + 1])
        assert np.abs(got[gather_ref[s_:e_]] - want).max() <= ATOL, b
    dropped = np.setdiff1d(np.arange(w.B * w.N), gather_ref)
    assert (as_numpy_rows(_gathered(w, torch.bfloat16))[dropped].view(np.uint8) == SENTINEL_BYTE).all()


def test_gathered_zero_dropped_and_fused_pipeline():
    w = wl.custom(B=5, N=197, H=6, lengths=[0, 197, 1, 40, 64], seed=14)
    o = _gathered(w, torch.float32, flags=binding.RAG_UNPACK_ZERO_DROPPED).cpu().numpy()
    assert (o[w.keep.reshape(-1) == 0] == 0).all()
    bufs = _pipeline_buffers(w, torch.float32)
    pipe = _make_pipeline(w, bufs)
    pipe.launch_eager()
    torch.cuda.synchronize()
    staged = bufs["dst"].clone()
    bufs["dst"].view(torch.uint8).fill_(SENTINEL_BYTE)
    pipe.launch_fused()
    torch.cuda.synchronize()
    assert torch.equal(bufs["dst"].view(torch.uint8), staged.view(torch.uint8))
    res = pipe.measure_dispatch(warmup=3, iters=10)
    assert res["fused_roundtrip"]["p50"] > 0
    st = pipe.measure_stages(iters=10)
    assert st["fused_pass"] > 0
    pipe.close()


@pytest.mark.parametrize("flags", [0, binding.RAG_UNPACK_ZERO_DROPPED])
def test_fused_graph_pipeline_replays_the_one_launch_pass(flags):
    """A pipeline created with RAG_PIPELINE_FUSED captures the one-launch pass:
    every replay writes dst exactly as the three-stage pass does (the same
    kernel arithmetic), with unrelated eager work between the replays, and
    leaves the packed buffers, offsets and gather index untouched."""
    w = wl.custom(B=6, N=197, H=6, lengths=[0, 197, 1, 40, 64, 40], seed=19)
    bufs = _pipeline_buffers(w, torch.bfloat16)
    staged_pipe = _make_pipeline(w, bufs, flags=flags)
    staged_pipe.launch_eager()
    torch.cuda.synchronize()
    staged = bufs["dst"].clone()
    staged_pipe.close()
    bufs = _pipeline_buffers(w, torch.bfloat16)
    pipe = binding.Pipeline(bufs["keep"], bufs["src"], bufs["packed"], bufs["cu"], bufs["gather"],
                            bufs["o_packed"], bufs["dst"], H=w.H, scale=w.scale, unpack_flags=flags,
                            fused_graph=True)
    for rep in range(3):
        bufs["dst"].view(torch.uint8).fill_(SENTINEL_BYTE)
        torch.cuda.synchronize()
        pipe.launch()
        torch.cuda.synchronize()
        assert torch.equal(bufs["dst"].view(torch.uint8), staged.view(torch.uint8)), rep
        for k in ("packed", "cu", "gather", "o_packed"):
            assert (bufs[k].view(torch.uint8) == SENTINEL_BYTE).all(), (rep, k)
        scratch = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del scratch
    res = pipe.measure_dispatch(warmup=3, iters=10)
    assert res["graph1_launch"]["p50"] > 0 and res["graph1_roundtrip"]["p50"] > 0
    pipe.close()


@pytest.mark.parametrize("fused", [False, True])
def test_direct_pipeline_launch_is_the_pass(fused):
    """With RAG_PIPELINE_DIRECT no graph is captured and rag_pipeline_launch
    enqueues the pass's direct launches: the three stages, or with
    RAG_PIPELINE_FUSED the one gathered launch (which leaves the packed
    buffers, offsets and gather index untouched).  Every launch writes dst as
    the eager three-stage pass does, bit for bit."""
    w = wl.custom(B=6, N=197, H=6, lengths=[0, 197, 1, 40, 64, 40], seed=23)
    bufs = _pipeline_buffers(w, torch.bfloat16)
    staged_pipe = _make_pipeline(w, bufs)
    staged_pipe.launch_eager()
    torch.cuda.synchronize()
    staged = bufs["dst"].clone()
    staged_pipe.close()
    bufs = _pipeline_buffers(w, torch.bfloat16)
    pipe = binding.Pipeline(bufs["keep"], bufs["src"], bufs["packed"], bufs["cu"], bufs["gather"],
                            bufs["o_packed"], bufs["dst"], H=w.H, scale=w.scale,
                            fused_graph=fused, direct=True)
    for rep in range(3):
        bufs["dst"].view(torch.uint8).fill_(SENTINEL_BYTE)
        torch.cuda.synchronize()
        pipe.launch()
        torch.cuda.synchronize()
        assert torch.equal(bufs["dst"].view(torch.uint8), staged.view(torch.uint8)), rep
        if fused:
            for k in ("packed", "cu", "gather", "o_packed"):
                assert (bufs[k].view(torch.uint8) == SENTINEL_BYTE).all(), (rep, k)
    res = pipe.measure_dispatch(warmup=3, iters=10)
    assert res["graph_roundtrip"]["p50"] > 0
    pipe.close()


def test_attn_plan_equals_the_call():
    """binding.AttnPlan prepares a rag_attn call once; calling it gives the
    call's output bit for bit (on torch's current stream and on another)."""
    w = wl.deits(3, 500)
    g = gpu_pack(w)
    C = w.C
    ref = gpu_attn(g["packed"], g["cu"], w, torch.float32)
    o = sentinel_like((w.B * w.N, C), torch.float32)
    p = g["packed"]
    plan = binding.AttnPlan(p[:, :C], p[:, C:2 * C], p[:, 2 * C:], g["cu"], w.N, o, H=w.H, scale=w.scale)
    plan()
    torch.cuda.synchronize()
    assert torch.equal(o[:w.T].view(torch.uint8), ref[:w.T].view(torch.uint8))
    o.view(torch.uint8).fill_(SENTINEL_BYTE)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan()
    side.synchronize()
    assert torch.equal(o[:w.T].view(torch.uint8), ref[:w.T].view(torch.uint8))


def test_lds_resident_and_tile_kernels_agree_bit_for_bit():
    """bf16 input takes the LDS-resident kernel when max_seqlen is small enough
    for the image's K and V to sit in LDS, and the 64-key tile kernel otherwise.
    Both do the same arithmetic in the same order, so the outputs are equal bit
    for bit; the oracle checks the values."""
    w = wl.custom(B=4, N=577, H=2, lengths=[200, 5, 77, 0], seed=15)
    ref = _oracle_pack(w)
    g = gpu_pack(w)
    for out_dtype in (torch.float32, torch.bfloat16):
        tile = gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=577)
        lds = gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=200)
        assert torch.equal(tile[:w.T].view(torch.uint8), lds[:w.T].view(torch.uint8)), out_dtype
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=200)
    o16 = gpu_attn(g["packed"], g["cu"], w, torch.bfloat16, max_seqlen=200)
    _check_attn(w, ref, o32, o16, range(w.B))


def test_few_pairs_at_the_longest_lds_resident_length():
    """Few (image, head) pairs at 256 keys, the LDS-resident kernel's longest
    sequences, where its output leaves through per-wave LDS slots beside 64 KiB
    of K and V: 72 KiB in all with bf16 output, exactly the 80 KiB limit with
    fp32 output (ragged layout); past it for the padded layout's fp32 output,
    which keeps the direct stores.  Every form equals the 64-key tile kernel or
    the three-stage result bit for bit, and the oracle."""
    w = wl.custom(B=3, N=256, H=2, lengths=[256, 255, 1], seed=41)
    ref = _oracle_pack(w)
    gather_ref = ref[2]
    g = gpu_pack(w)
    for out_dtype in (torch.float32, torch.bfloat16):
        lds = gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=256)
        tile = gpu_attn(g["packed"], g["cu"], w, out_dtype, max_seqlen=257)
        assert torch.equal(lds[:w.T].view(torch.uint8), tile[:w.T].view(torch.uint8)), out_dtype
        fused = as_numpy_rows(_gathered(w, out_dtype))
        assert (fused[gather_ref].view(np.uint8) == as_numpy_rows(lds)[:w.T].view(np.uint8)).all(), out_dtype
    o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=256)
    o16 = gpu_attn(g["packed"], g["cu"], w, torch.bfloat16, max_seqlen=256)
    _check_attn(w, ref, o32, o16, range(w.B))
    C = w.C
    q, k, v = wl.split_qkv(wl.rows(w), C)
    want = oracle.attn_padded(q, k, v, w.keep, w.H, w.d, w.scale)
    src = g["src"]
    for out_dtype in (torch.float32, torch.bfloat16):
        o = sentinel_like((w.B * w.N, C), out_dtype)
        binding.rag_attn_padded(src[:, :C], src[:, C:2 * C], src[:, 2 * C:], g["keep"], o, H=w.H,
                                scale=w.scale)
        torch.cuda.synchronize()
        got = o.float().cpu().numpy().astype(np.float64)
        bound = ATOL + (np.abs(want) * 2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0)
        assert (np.abs(got - want) <= bound).all(), out_dtype


def _truncate_keep(keep: np.ndarray, m: int) -> np.ndarray:
    """The first m kept positions of every image (what a max_seqlen of m keeps)."""
    out = np.zeros_like(keep)
    for b in range(keep.shape[0]):
        pos = np.flatnonzero(keep[b])[:m]
        out[b, pos] = keep[b, pos]
    return out


def test_gathered_max_seqlen_bound_and_truncation():
    w = wl.custom(B=6, N=197, H=6, lengths=[40, 40, 12, 0, 40, 33], seed=16)
    src = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    C = w.C

    def run(m):
        o = sentinel_like((w.B * w.N, C), torch.float32)
        binding.rag_attn_gathered(keep, src[:, :C], src[:, C:2 * C], src[:, 2 * C:], o, H=w.H,
                                  scale=w.scale, max_seqlen=m)
        torch.cuda.synchronize()
        return o

    full = run(0)
    tight = run(40)  # the exact bound: same result, smaller launch
    assert torch.equal(full.view(torch.int32), tight.view(torch.int32))
    # a bound below some images' kept count: those images are their first 25
    # kept rows; the later kept rows are not written
    got = run(25).cpu().numpy().astype(np.float64)
    kt = _truncate_keep(w.keep, 25)
    packed_t, cu_t, gather_t = oracle.pack(kt, wl.rows(w))
    for b in range(w.B):
        s, e = int(cu_t[b]), int(cu_t[b + 1])
        if e > s:
            q, k, v = wl.split_qkv(packed_t[s:e], C)
            want = oracle.attn(q, k, v, np.array([0, e - s], np.int32), w.H, w.d, w.scale)
            assert np.abs(got[gather_t[s:e]] - want).max() <= ATOL, b
    unwritten = np.setdiff1d(np.arange(w.B * w.N), gather_t)
    assert (as_numpy_rows(run(25))[unwritten].view(np.uint8) == SENTINEL_BYTE).all()


@pytest.mark.parametrize("scale", [0.0, -0.3, 1e-6, 2.5])
def test_attention_any_scale(scale):
    """The kernels fold the scale's sign into Q (a zero scale becomes a tiny
    positive one); the oracle takes the scale as given.  Both kernels (LDS
    resident: max_seqlen 130; 64-key tiles: fp32 input) are covered.  A zero
    scale gives every image the mean of its V rows."""
    for w in (wl.custom(B=3, N=130, H=2, lengths=[130, 7, 64], seed=17),
              wl.custom(B=2, N=70, H=2, lengths=[70, 3], dtype="f32", seed=18)):
        w.scale = scale
        ref = _oracle_pack(w)
        g = gpu_pack(w)
        o32 = gpu_attn(g["packed"], g["cu"], w, torch.float32)
        o16 = gpu_attn(g["packed"], g["cu"], w, torch.bfloat16)
        worst = _check_attn(w, ref, o32, o16, range(w.B))
        print("scale", scale, w.dtype, "max abs err", worst, flush=True)


def _second_stage_keep(w, seed, density):
    """A keep byte per packed row (a later pruning stage), CLS rows kept: the
    input generator's draw at a kept count of about density * N."""
    k = wl.second_stage_keep(w, max(1, int(round(density * w.N))), seed)
    rng = np.random.default_rng(seed + 100)  # any nonzero byte keeps
    return (k * rng.integers(1, 256, k.shape)).astype(np.uint8)


def _gpu_repack(g, k2_np, w, max_rows_in):
    rows = w.B * w.N
    k2 = torch.zeros(rows, dtype=torch.uint8, device="cuda")
    k2[:k2_np.shape[0]] = torch.from_numpy(k2_np).cuda()
    dst = sentinel_like((rows, 3 * w.C), g["packed"].dtype)
    cu_out = sentinel_like((w.B + 1,), torch.int32)
    g_out = sentinel_like((rows,), torch.int32)
    binding.rag_repack(k2, g["cu"], g["gather"], max_rows_in, g["packed"], dst, cu_out, g_out)
    torch.cuda.synchronize()
    return dst, cu_out, g_out


@pytest.mark.parametrize("name,density", [("deits_b4_p800", 0.5), ("deitb_ragged_b64", 0.3),
                                          ("empty_and_full", 0.7), ("f32_odd", 0.5),
                                          ("n577_two", 0.4), ("tile_edges", 1.0)])
def test_repack_bit_exact(name, density):
    """A second pruning stage on the packed buffer: cu, composed gather index and
    rows bit for bit the oracle's; rows and entries past T' untouched."""
    w = FULL[name]()
    print("repack case", name, flush=True)
    packed_ref, cu_ref, gather_ref = _oracle_pack(w)
    g = gpu_pack(w)
    k2 = _second_stage_keep(w, 19, density)
    want_rows, want_cu, want_g = oracle.repack(k2, cu_ref, gather_ref, packed_ref)
    dst, cu_out, g_out = _gpu_repack(g, k2, w, int(w.lengths.max()) if w.T else 1)
    T2 = int(want_cu[-1])
    assert (cu_out.cpu().numpy() == want_cu).all()
    assert (g_out.cpu().numpy()[:T2] == want_g).all()
    assert (g_out.cpu().numpy()[T2:].view(np.uint32) == np.uint32(0xA5A5A5A5)).all()
    d = as_numpy_rows(dst)
    assert (d[:T2].view(np.uint8) == want_rows.view(np.uint8)).all()
    assert (d[T2:].view(np.uint8) == SENTINEL_BYTE).all()


def test_repack_equals_pack_of_composed_mask_full_size():
    """deits at B = 256 without pruning, then a 60% second stage: the same bits
    as packing the batch with the composed mask in one go."""
    w = wl.deits(256, 0)
    g = gpu_pack(w)
    k2 = _second_stage_keep(w, 20, 0.6)
    dst, cu_out, g_out = _gpu_repack(g, k2, w, w.N)
    _, cu_ref, gather_ref = _oracle_pack(w)
    k12 = np.zeros(w.B * w.N, dtype=np.uint8)
    k12[gather_ref[k2 != 0]] = 1
    w2 = wl.custom(B=w.B, N=w.N, H=w.H, lengths=np.count_nonzero(k12.reshape(w.B, w.N), axis=1),
                   seed=0)
    w2.keep = k12.reshape(w.B, w.N)
    w2.qkv = w.qkv
    g2 = gpu_pack(w2)
    T2 = int(np.count_nonzero(k12))
    assert torch.equal(cu_out, g2["cu"])
    assert torch.equal(g_out[:T2], g2["gather"][:T2])
    assert torch.equal(dst[:T2].view(torch.uint8), g2["packed"][:T2].view(torch.uint8))


def test_repack_then_attention_and_unpack():
    """The second stage feeds attention and unpack directly (gather_out holds
    batch rows): the result equals the oracle on the composed mask."""
    w = wl.deits(4, 500)
    g = gpu_pack(w)
    k2 = _second_stage_keep(w, 21, 0.5)
    dst, cu_out, g_out = _gpu_repack(g, k2, w, int(w.lengths.max()))
    o = gpu_attn(dst, cu_out, w, torch.float32, max_seqlen=int(w.lengths.max()))
    packed_ref, cu_ref, gather_ref = _oracle_pack(w)
    rows2, cu2, g2 = oracle.repack(k2, cu_ref, gather_ref, packed_ref)
    q, k, v = wl.split_qkv(rows2, w.C)
    want = oracle.attn(q, k, v, cu2, w.H, w.d, w.scale)
    T2 = int(cu2[-1])
    assert np.abs(o.cpu().numpy()[:T2].astype(np.float64) - want).max() <= ATOL
    out = sentinel_like((w.B * w.N, w.C), torch.float32)
    binding.rag_unpack(o, cu_out, g_out, out, N=w.N)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[g2].view(np.uint8) == o.cpu().numpy()[:T2].view(np.uint8)).all()


@pytest.mark.parametrize("max_seqlen,dtype", [(100, "bf16"), (300, "bf16"), (100, "f32")])
def test_attention_on_separate_strided_buffers(max_seqlen, dtype):
    """q, k, v and o as four separate allocations, each with its own padded row
    stride (rows wider than H*64, o's row stride different again): the same
    result as the fused packed view, bit for bit, and the oracle's values.
    max_seqlen 100 takes the LDS-resident kernel for bf16, 300 the 64-key
    tile kernel (fp32 input always does)."""
    N = max_seqlen
    w = wl.custom(B=3, N=N, H=2, lengths=[N, N // 3, 0], dtype=dtype, seed=41)
    ref = _oracle_pack(w)
    g = gpu_pack(w)
    T, C = w.T, w.C
    fused = gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=max_seqlen)
    pk = g["packed"][:T]
    pads = {"q": 64, "k": 128, "v": 8}
    bufs = {}
    for i, name in enumerate(("q", "k", "v")):
        wide = torch.zeros(T, C + pads[name], dtype=pk.dtype, device="cuda")
        wide[:, :C] = pk[:, i * C:(i + 1) * C]
        bufs[name] = wide[:, :C]
    o_wide = sentinel_like((T, C + 24), torch.float32)
    binding.rag_attn(bufs["q"], bufs["k"], bufs["v"], g["cu"], max_seqlen, o_wide[:, :C], H=w.H,
                     scale=w.scale)
    torch.cuda.synchronize()
    got = o_wide[:, :C].cpu().numpy()
    assert (got.view(np.uint32) == fused[:T].cpu().numpy().view(np.uint32)).all()
    assert (as_numpy_rows(o_wide)[:, C:].view(np.uint8) == SENTINEL_BYTE).all(), "pad columns written"
    for b, want in _oracle_attn_images(w, ref, range(w.B)).items():
        s, e = int(ref[1][b]), int(ref[1][b + 1])
        assert np.abs(got[s:e].astype(np.float64) - want).max() <= ATOL
