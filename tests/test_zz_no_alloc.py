"""The allocation-free encoder-block forward, rag_block_forward_static (its
intermediates in the library's static device array), against the
buffer-taking rag_block_forward, both through the C ABI on the same inputs:
two calls in a row, the second with fewer rows (the array keeps the first
call's contents).  Same kernels, same launch shapes, no atomics: the outputs
must be identical bit for bit, and both within the block's bar of the fp64
oracle (2^-6 (|y| + 1) per element, mean error below 4e-3)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import vit_block as vb
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bf16_gpu(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _params_gpu(P):
    return {k: (_bf16_gpu(np.ascontiguousarray(v.T)) if k.startswith("w_") else torch.from_numpy(v).cuda())
            for k, v in P.items()}


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_static_forward_equals_the_scratch_forward_on_two_calls():
    C, H = 384, 6
    P = wl.vit_block_params(C, 4, 31)
    blk = binding.Block(_params_gpu(P), H=H, scale=1.0 / 8.0)
    for w, seed in ((wl.deits(24, 500), 32), (wl.deits(5, 800), 33)):  # 2376 rows, then 200
        print("static block case", w.name, "rows", w.T, flush=True)
        xb = wl.hidden_rows(w.B, w.N, C, seed)
        packed, cu, _ = oracle.pack(w.keep, xb)
        x = _bf16_gpu(packed)
        cu_d = torch.from_numpy(cu).cuda()
        L = int(w.lengths.max())
        y_ref = torch.full_like(x, 3.0)
        y_st = torch.full_like(x, -5.0)
        blk.forward(x, y_ref, w.T, cu_d, L)
        blk.forward_static(x, y_st, w.T, cu_d, L)
        torch.cuda.synchronize()
        assert torch.equal(y_ref.view(torch.int16), y_st.view(torch.int16))
        want = vb.block(packed, P, cu, H, 1.0 / 8.0)
        got = vb.bf16_bits_to_f64(_bits(y_st))
        err = np.abs(got - want)
        assert (err <= 2.0 ** -6 * (np.abs(want) + 1.0)).all() and err.mean() < 4e-3, err.max()
    blk.close()


def test_static_forward_refuses_more_rows_than_its_array():
    C, H = 384, 6
    blk = binding.Block(_params_gpu(wl.vit_block_params(C, 4, 1)), H=H, scale=0.125)
    per_row = (6 * C + 4 * C) * 2
    too_many = (128 << 20) // per_row + 1
    x = torch.zeros(16, C, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 16], dtype=torch.int32, device="cuda")
    # (through the C ABI directly: the binding would refuse rows beyond x's own)
    with pytest.raises(binding.RagError, match="static scratch holds"):
        binding._check(binding.load().rag_block_forward_static(blk._h, x.data_ptr(), x.data_ptr(), too_many,
                                                               cu.data_ptr(), 1, 16, None))
    blk.close()
