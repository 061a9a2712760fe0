"""The entry points run on the stream the caller gives them, and can be captured
in a graph.

On a side stream, a long matrix product is queued first and the input rows are
written after it; pack, attention and unpack (and the pipeline's three-launch
pass) are then enqueued on the same stream with no synchronisation in between.
Work that ran on another stream would start before the rows exist and read
uninitialised memory; on the caller's stream it waits for them, and the results
match the oracle (pack bit for bit, attention within 2e-3)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import as_numpy_rows, sentinel_like, to_gpu_rows
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def _delay(n=4096):
    """About a millisecond of GPU work on the current stream."""
    a = torch.ones(n, n, device="cuda", dtype=torch.float32)
    for _ in range(4):
        a = a @ a * (1.0 / n)
    return a


def _expected(w):
    packed_ref, cu_ref, gather_ref = oracle.pack(w.keep, wl.rows(w))
    q, k, v = wl.split_qkv(packed_ref, w.C)
    return packed_ref, cu_ref, gather_ref, oracle.attn(q, k, v, cu_ref, w.H, w.d, w.scale)


def test_entry_points_follow_the_callers_stream():
    w = wl.custom(B=6, N=197, H=3, lengths=[40, 197, 0, 1, 77, 130], seed=61)
    packed_ref, cu_ref, gather_ref, o_ref = _expected(w)
    T, C = w.T, w.C
    src_host = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        src = torch.empty_like(src_host)
        packed = sentinel_like((w.B * w.N, 3 * C), src.dtype)
        cu = sentinel_like((w.B + 1,), torch.int32)
        gather = sentinel_like((w.B * w.N,), torch.int32)
        o = sentinel_like((w.B * w.N, C), torch.float32)
        dst = torch.zeros(w.B * w.N, C, dtype=torch.float32, device="cuda")
        _delay()
        src.copy_(src_host)  # the rows exist only after the delay, on stream s
        binding.rag_pack(keep, src, packed, cu, gather)
        binding.rag_attn(packed[:, :C], packed[:, C:2 * C], packed[:, 2 * C:], cu, w.N, o, H=w.H,
                         scale=w.scale)
        binding.rag_unpack(o, cu, gather, dst, N=w.N)
    s.synchronize()
    assert (cu.cpu().numpy() == cu_ref).all()
    assert (gather.cpu().numpy()[:T] == gather_ref).all()
    assert (as_numpy_rows(packed)[:T].view(np.uint8) == packed_ref.view(np.uint8)).all()
    got = dst.cpu().numpy().astype(np.float64)[gather_ref]
    assert np.abs(got - o_ref).max() <= ATOL


def test_pipeline_pass_follows_the_given_stream():
    w = wl.deits(4, 800)
    packed_ref, cu_ref, gather_ref, o_ref = _expected(w)
    C = w.C
    src_host = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    src = torch.empty_like(src_host)
    packed = torch.empty(w.B * w.N, 3 * C, dtype=src.dtype, device="cuda")
    cu = torch.zeros(w.B + 1, dtype=torch.int32, device="cuda")
    gather = torch.zeros(w.B * w.N, dtype=torch.int32, device="cuda")
    o = torch.empty(w.B * w.N, C, dtype=torch.float32, device="cuda")
    dst = torch.zeros(w.B * w.N, C, dtype=torch.float32, device="cuda")
    pipe = binding.Pipeline(keep, src, packed, cu, gather, o, dst, H=w.H, scale=w.scale,
                            max_seqlen=int(w.lengths.max()))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        _delay()
        src.copy_(src_host)
    pipe.launch_eager(stream=s)
    s.synchronize()
    assert (cu.cpu().numpy() == cu_ref).all()
    got = dst.cpu().numpy().astype(np.float64)[gather_ref]
    assert np.abs(got - o_ref).max() <= ATOL
    pipe.close()


def test_entry_points_captured_in_a_graph_replay_correctly():
    """rag_pack, rag_attn and rag_unpack captured in one CUDA graph (as a caller
    would, with torch.cuda.graph), replayed three times with new input rows and
    a new keep mask copied in between, eager work and synchronisations between
    the replays; every replay matches the oracle for its own inputs."""
    B, N, H = 5, 197, 2
    cases = [wl.custom(B=B, N=N, H=H, lengths=lens, seed=70 + i)
             for i, lens in enumerate(([40, 0, 197, 3, 90], [197, 197, 1, 0, 64], [0, 0, 0, 5, 40]))]
    C = cases[0].C
    src = torch.empty_like(to_gpu_rows(cases[0]))
    keep = torch.zeros(B, N, dtype=torch.uint8, device="cuda")
    packed = torch.empty(B * N, 3 * C, dtype=src.dtype, device="cuda")
    cu = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    gather = torch.zeros(B * N, dtype=torch.int32, device="cuda")
    o = torch.empty(B * N, C, dtype=torch.float32, device="cuda")
    dst = torch.zeros(B * N, C, dtype=torch.float32, device="cuda")

    def run():
        binding.rag_pack(keep, src, packed, cu, gather)
        binding.rag_attn(packed[:, :C], packed[:, C:2 * C], packed[:, 2 * C:], cu, N, o, H=H,
                         scale=cases[0].scale)
        binding.rag_unpack(o, cu, gather, dst, N=N)

    src.copy_(to_gpu_rows(cases[0]))
    keep.copy_(torch.from_numpy(cases[0].keep))
    run()  # eager once before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for w in cases:
        src.copy_(to_gpu_rows(w))
        keep.copy_(torch.from_numpy(w.keep))
        dst.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        packed_ref, cu_ref, gather_ref, o_ref = _expected(w)
        assert (cu.cpu().numpy() == cu_ref).all()
        T = w.T
        assert (gather.cpu().numpy()[:T] == gather_ref).all()
        if T:
            got = dst.cpu().numpy().astype(np.float64)[gather_ref]
            assert np.abs(got - o_ref).max() <= ATOL
        dropped = np.setdiff1d(np.arange(B * N), gather_ref)
        assert (dst.cpu().numpy()[dropped] == 0).all()


def test_two_streams_at_once_share_nothing():
    """Two different batches through pack, attention and unpack on two streams
    with no ordering between them: each matches the oracle for its own batch
    (the library keeps no state between calls)."""
    ws = [wl.custom(B=7, N=197, H=3, lengths=[40, 197, 0, 1, 77, 130, 12], seed=81),
          wl.custom(B=3, N=577, H=2, lengths=[577, 300, 2], seed=82)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for w in ws:
        C = w.C
        outs.append(dict(src=to_gpu_rows(w), keep=torch.from_numpy(w.keep).cuda(),
                         packed=torch.empty(w.B * w.N, 3 * C, dtype=torch.bfloat16, device="cuda"),
                         cu=torch.zeros(w.B + 1, dtype=torch.int32, device="cuda"),
                         gather=torch.zeros(w.B * w.N, dtype=torch.int32, device="cuda"),
                         o=torch.empty(w.B * w.N, C, dtype=torch.float32, device="cuda"),
                         dst=torch.zeros(w.B * w.N, C, dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    for rep in range(3):
        for w, b, s in zip(ws, outs, streams):
            C = w.C
            with torch.cuda.stream(s):
                binding.rag_pack(b["keep"], b["src"], b["packed"], b["cu"], b["gather"])
                binding.rag_attn(b["packed"][:, :C], b["packed"][:, C:2 * C], b["packed"][:, 2 * C:],
                                 b["cu"], w.N, b["o"], H=w.H, scale=w.scale)
                binding.rag_unpack(b["o"], b["cu"], b["gather"], b["dst"], N=w.N)
    torch.cuda.synchronize()
    for w, b in zip(ws, outs):
        packed_ref, cu_ref, gather_ref, o_ref = _expected(w)
        assert (b["cu"].cpu().numpy() == cu_ref).all()
        got = b["dst"].cpu().numpy().astype(np.float64)[gather_ref]
        assert np.abs(got - o_ref).max() <= ATOL
