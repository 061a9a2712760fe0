"""GPU checks of properties that pin attention without the oracle.

* No leakage: changing one image's Q/K/V rows leaves every other image's output
  equal bit for bit (packed, gathered and padded layouts; the LDS-resident
  kernel and the 64-key tile kernel).
* Closed forms, in fp32 output within the 2e-3 bar: an image whose V rows are
  all equal returns that row; an image whose K rows are all equal returns the
  mean of its V rows; a zero query row returns the mean of V.
* Permutation: reordering an image's rows reorders its output rows (within the
  bar, since the key order changes the order of summation).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import as_numpy_rows, bf16_bits_to_f64, gpu_attn, gpu_pack, sentinel_like, to_gpu_rows
from ragged_attention_token_amd import binding
from ragged_attention_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def _bf16_rows(rng, n, width):
    x = torch.from_numpy(rng.standard_normal((n, width)).astype(np.float32))
    return x.to(torch.bfloat16).cuda()


def _attn_packed(q, k, v, cu, max_seqlen, H, scale=0.125):
    o = sentinel_like((q.shape[0], q.shape[1]), torch.float32)
    binding.rag_attn(q, k, v, cu, max_seqlen, o, H=H, scale=scale)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("N,lengths,max_seqlen", [
    (197, [40, 197, 0, 100], 197),   # LDS-resident kernel
    (577, [300, 5, 577, 64], 577),   # 64-key tile kernel
])
def test_no_leakage_between_images(N, lengths, max_seqlen):
    w = wl.custom(B=len(lengths), N=N, H=2, lengths=lengths, seed=51)
    g = gpu_pack(w)
    cu = g["cu"].cpu().numpy()
    o1 = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=max_seqlen))
    s, e = int(cu[1]), int(cu[2])
    g["packed"][s:e] = _bf16_rows(np.random.default_rng(52), e - s, 3 * w.C)
    o2 = as_numpy_rows(gpu_attn(g["packed"], g["cu"], w, torch.float32, max_seqlen=max_seqlen))
    T = w.T
    others = np.r_[0:s, e:T]
    assert (o2[others].view(np.uint32) == o1[others].view(np.uint32)).all()
    assert not (o2[s:e] == o1[s:e]).all()

    # the same in the batch layouts: change image 1's source rows
    src = to_gpu_rows(w)
    keep = torch.from_numpy(w.keep).cuda()
    C = w.C

    def run(src_rows):
        gz = sentinel_like((w.B * N, C), torch.float32)
        binding.rag_attn_gathered(keep, src_rows[:, :C], src_rows[:, C:2 * C], src_rows[:, 2 * C:], gz,
                                  H=w.H, scale=w.scale)
        pz = sentinel_like((w.B * N, C), torch.float32)
        binding.rag_attn_padded(src_rows[:, :C], src_rows[:, C:2 * C], src_rows[:, 2 * C:], keep, pz,
                                H=w.H, scale=w.scale)
        torch.cuda.synchronize()
        return as_numpy_rows(gz), as_numpy_rows(pz)

    g1, p1 = run(src)
    src2 = src.clone()
    src2[N:2 * N] = _bf16_rows(np.random.default_rng(53), N, 3 * C)
    g2, p2 = run(src2)
    rest = np.r_[0:N, 2 * N:w.B * N]
    assert (g2[rest].view(np.uint32) == g1[rest].view(np.uint32)).all()
    assert (p2[rest].view(np.uint32) == p1[rest].view(np.uint32)).all()


def _decode(t):
    return bf16_bits_to_f64(as_numpy_rows(t))


@pytest.mark.parametrize("max_seqlen", [197, 300])  # LDS-resident, then the 64-key tile kernel
def test_closed_forms(max_seqlen):
    """Image 0: all V rows equal -> O = that row.  Image 1: all K rows equal
    (per head) -> O = mean of V.  Image 2: Q = 0 -> O = mean of V."""
    H, d = 2, 64
    C = H * d
    lengths = [50, 197, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(54)
    q = _bf16_rows(rng, T, C)
    k = _bf16_rows(rng, T, C)
    v = _bf16_rows(rng, T, C)
    v[cu[0]:cu[1]] = v[cu[0]]
    k[cu[1]:cu[2]] = k[cu[1]]
    q[cu[2]:cu[3]] = 0
    o = _attn_packed(q, k, v, torch.from_numpy(cu).cuda(), max_seqlen, H).cpu().numpy().astype(np.float64)
    vd = _decode(v)
    assert np.abs(o[cu[0]:cu[1]] - vd[cu[0]]).max() <= ATOL
    for b in (1, 2):
        mean = vd[cu[b]:cu[b + 1]].mean(axis=0)
        assert np.abs(o[cu[b]:cu[b + 1]] - mean).max() <= ATOL, b


@pytest.mark.parametrize("max_seqlen", [197, 300])
def test_permutation_within_an_image(max_seqlen):
    H, C = 2, 128
    lengths = [60, 197]
    cu = np.array([0, 60, 257], dtype=np.int32)
    rng = np.random.default_rng(55)
    qkv = _bf16_rows(rng, 257, 3 * C)
    perm = np.concatenate([rng.permutation(60), 60 + rng.permutation(197)])
    cu_t = torch.from_numpy(cu).cuda()

    def run(x):
        return _attn_packed(x[:, :C], x[:, C:2 * C], x[:, 2 * C:], cu_t, max_seqlen, H).cpu().numpy()

    o = run(qkv)
    op = run(qkv[torch.from_numpy(perm).cuda()].contiguous())
    assert np.abs(op.astype(np.float64) - o[perm]).max() <= ATOL
    assert sum(lengths) == 257
