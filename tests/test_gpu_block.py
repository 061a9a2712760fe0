"""GPU parity of the ViT encoder block (the end-to-end timing row): the block
through the C ABI (this library's LayerNorm, GEMMs and attention) against the
fp64 block oracle on the same seeded inputs.

Bar: every intermediate of the GPU block is stored as bf16 (7 roundings of at
most 2^-9 relative each, through stages of about unit gain), so the output is
compared element-wise within 2^-6 * (|y| + 1) of the fp64 oracle, and the mean
absolute error must stay below 4e-3.  A CPU emulation of exactly those roundings
lands at 0.0052 * (|y| + 1) at most and 1.6e-3 on average (deits B = 4, 80%
prune), so the bound has a 3x margin.

The weights are drawn in the [in, out] layout the oracle multiplies with
(y = x W) and uploaded transposed, in the [out, in] layout of a linear layer's
weight that the C ABI takes.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import vit_block as vb
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

GELU_FORM = "erf"  # DeiT's MLP activation, x * Phi(x); the oracle's default


def _bf16_gpu(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _params_gpu(P):
    """Block parameters on the GPU; matrices transposed to [out, in]."""
    return {k: (_bf16_gpu(np.ascontiguousarray(v.T)) if k.startswith("w_") else torch.from_numpy(v).cuda())
            for k, v in P.items()}


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _to_bf16_f64(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _check(got_bits, want):
    got = vb.bf16_bits_to_f64(got_bits)
    err = np.abs(got - want)
    bound = 2.0 ** -6 * (np.abs(want) + 1.0)
    assert np.isfinite(got).all()
    assert (err <= bound).all(), "max err %.3g, worst ratio %.3g" % (err.max(), (err / bound).max())
    assert err.mean() < 4e-3, err.mean()
    return err.max()


def test_block_gelu_is_the_exact_form():
    """Weights chosen so that y = bf16(GELU(b1)) exactly: x = 0, every matrix
    zero except W2 = [I; 0] (column j of y takes m[:, j]), LayerNorm2's gamma 0.
    The exact GELU and its tanh approximation differ by up to ~24% relative at
    x = -3.5, far more than a bf16 step, so the output tells them apart: it
    must be the exact form the oracle uses."""
    H, C, ratio = 2, 128, 4
    hid = C * ratio
    P = wl.vit_block_params(C, ratio, 0)
    for k in P:
        if k.startswith(("w_", "b_")):
            P[k] = np.zeros_like(P[k])
    P["ln2_gamma"] = np.zeros(C, np.float32)
    probes = np.linspace(-4.0, 4.0, C).astype(np.float32)
    P["b_fc1"] = np.concatenate([probes, np.zeros(hid - C, np.float32)])
    w2 = np.zeros((hid, C), np.float32)
    w2[np.arange(C), np.arange(C)] = 1.0
    P["w_fc2"] = wl._to_bf16_bits(w2)
    blk = binding.Block(_params_gpu(P), H=H, scale=0.125, mlp_ratio=ratio)
    rows = 16
    x = torch.zeros(rows, C, dtype=torch.bfloat16, device="cuda")
    y = torch.full((rows, C), 7.0, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, rows], dtype=torch.int32, device="cuda")
    blk.forward(x, y, rows, cu, rows)
    torch.cuda.synchronize()
    got = vb.bf16_bits_to_f64(_bits(y))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 1e-30))) - 7)
    for form in ("tanh", "erf"):
        want = _to_bf16_f64(vb.gelu(probes.astype(np.float64), form))
        ok = (np.abs(got - want[None, :]) <= ulp).all()
        print("GELU form", form, "matches:", ok, flush=True)
        assert ok == (form == GELU_FORM)
    blk.close()


def _block_case(w, C, H, seed):
    P = wl.vit_block_params(C, 4, seed)
    xb = wl.hidden_rows(w.B, w.N, C, seed + 1)
    packed, cu, gather = oracle.pack(w.keep, xb)
    want = vb.block(packed, P, cu, H, 1.0 / 8.0, gelu_form=GELU_FORM)
    return P, xb, packed, cu, gather, want


@pytest.mark.parametrize("name", ["deits_b4_p800", "deitb_ragged_b64", "empty_images", "deitt_b8_ragged"])
def test_block_on_packed_rows_matches_oracle(name):
    """Row counts that leave a partial 128-row GEMM tile; DeiT-T's C = 192
    also leaves a partial 128-column tile in three of the four products."""
    w, C, H = {"deits_b4_p800": (wl.deits(4, 800), 384, 6),
               "deitb_ragged_b64": (wl.deitb_ragged(64), 768, 12),
               "empty_images": (wl.custom(B=4, N=197, H=6, lengths=[0, 40, 0, 197], seed=9),
                                384, 6),
               "deitt_b8_ragged": (wl.custom(B=8, N=197, H=3, lengths=[197, 20, 77, 1, 130, 64, 65, 9],
                                             seed=4), 192, 3)}[name]
    print("block case", name, "T", w.T, flush=True)
    P, xb, packed, cu, gather, want = _block_case(w, C, H, 11)
    blk = binding.Block(_params_gpu(P), H=H, scale=1.0 / 8.0)
    T = w.T
    x = _bf16_gpu(packed)
    y = torch.empty_like(x)
    blk.forward(x, y, T, torch.from_numpy(cu).cuda(), int(w.lengths.max()))
    torch.cuda.synchronize()
    print("max abs err", _check(_bits(y), want), flush=True)
    blk.close()


def test_block_on_padded_rows_kept_rows_match_oracle():
    """The comparator: the same block on all B*N rows with masked keys; its
    kept rows are the packed block's result (within the same bar)."""
    w = wl.deits(4, 800)
    C, H = 384, 6
    P, xb, packed, cu, gather, want = _block_case(w, C, H, 13)
    blk = binding.Block(_params_gpu(P), H=H, scale=1.0 / 8.0)
    x = _bf16_gpu(xb)
    y = torch.empty_like(x)
    blk.forward_padded(x, y, torch.from_numpy(w.keep).cuda())
    torch.cuda.synchronize()
    got = _bits(y)
    print("max abs err", _check(got[gather], want), flush=True)
    assert np.isfinite(vb.bf16_bits_to_f64(got)).all()
    blk.close()
