"""The C ABI on a machine without a GPU: the library loads, exports every symbol
include/rag.h declares, and rejects every kind of bad argument on the host with
the documented status before anything is enqueued (no call here reaches HIP).
"""
import ctypes
import os
import re

import pytest

from ragged_attention_token_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rag.h")

OK, INVALID, UNSUPPORTED, ALIGN = 0, 1, 2, 3
F32, BF16 = 0, 1
A = 0x100000  # a 16-byte aligned fake device address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from ragged_attention_token_amd import build
        build.build()
    return binding.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"RAG_API\s+[\w\s\*]+?\b(rag_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("rag_pack", "rag_attn", "rag_unpack", "rag_attn_padded", "rag_pipeline_create",
                 "rag_pipeline_launch", "rag_pipeline_destroy", "rag_last_error"):
        assert name in syms
    assert sorted(binding.EXPORTS) == syms


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    for name in ("RAG_STAGES_N", "RAG_FLOOR_N", "RAG_MAX_N", "RAG_MAX_B", "RAG_HEAD_DIM",
                 "RAG_UNPACK_ZERO_DROPPED"):
        m = re.search(r"#define\s+%s\s+(\S+)" % name, text)
        assert m, name
        if hasattr(binding, name):
            assert int(m.group(1).rstrip("uU"), 0) == getattr(binding, name), name


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.rag_version() >= 100
    assert lib.rag_status_string(3) == b"RAG_ERR_ALIGNMENT"
    for code, name in binding.STATUS.items():
        assert lib.rag_status_string(code) == name.encode()


def pack(lib, keep=A, B=2, N=197, src=A, ss=2304, rb=2304, packed=A, ps=2304, cu=A, g=A, m=None):
    return lib.rag_pack(keep, B, N, src, ss, rb, packed, ps, cu, g, m, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(B=0), INVALID, "B=0"),
    (dict(N=0), INVALID, "N=0"),
    (dict(B=70000), UNSUPPORTED, "limits"),
    (dict(N=9000), UNSUPPORTED, "limits"),
    (dict(keep=None), INVALID, "keep"),
    (dict(keep=A + 3), ALIGN, "keep"),
    (dict(rb=8), INVALID, "row_bytes"),
    (dict(rb=2308), ALIGN, "row_bytes"),
    (dict(src=None), INVALID, "src"),
    (dict(src=A + 8), ALIGN, "src"),
    (dict(ss=2000), INVALID, "src row stride"),
    (dict(ps=2320 + 8), ALIGN, "packed"),
    (dict(cu=None), INVALID, "cu_seqlens"),
    (dict(g=None), INVALID, "gather_idx"),
])
def test_pack_rejects(lib, kwargs, status, needle):
    assert pack(lib, **kwargs) == status
    assert needle in binding.last_error()


def repack(lib, keep=A, cu_in=A, g_in=A, B=2, maxr=40, total=80, src=A, ss=2304, rb=2304,
           dst=A + 0x1000000, ds=2304, cu_out=A, g_out=A):
    return lib.rag_repack(keep, cu_in, g_in, B, maxr, total, src, ss, rb, dst, ds, cu_out, g_out,
                          None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(B=0), INVALID, "B=0"),
    (dict(maxr=0), INVALID, "N=0"),
    (dict(maxr=9000), UNSUPPORTED, "limits"),
    (dict(total=-1), INVALID, "total_rows"),
    (dict(keep=None), INVALID, "keep_packed"),
    (dict(keep=A + 3), ALIGN, "keep_packed"),
    (dict(cu_in=None), INVALID, "cu_in"),
    (dict(g_in=None), INVALID, "gather_in"),
    (dict(cu_out=None), INVALID, "cu_out"),
    (dict(g_out=None), INVALID, "gather_out"),
    (dict(rb=8), INVALID, "row_bytes"),
    (dict(rb=2308), ALIGN, "row_bytes"),
    (dict(src=None), INVALID, "src"),
    (dict(ds=2300), INVALID, "dst row stride"),
    (dict(dst=A + 8), ALIGN, "dst"),
    (dict(dst=A), INVALID, "overlap"),
    (dict(maxr=8192, ss=1 << 20), UNSUPPORTED, "2^31"),
])
def test_repack_rejects(lib, kwargs, status, needle):
    assert repack(lib, **kwargs) == status
    assert needle in binding.last_error()


def attn(lib, q=A, k=A, v=A, qs=1152, ks=1152, vs=1152, dt=BF16, cu=A, B=4, maxlen=197, tr=788,
         H=6, hd=64, scale=0.125, o=A, os_=384, odt=F32, fn="rag_attn"):
    return getattr(lib, fn)(q, k, v, qs, ks, vs, dt, cu, B, maxlen, tr, H, hd, scale, o, os_, odt,
                            None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(hd=32), UNSUPPORTED, "head_dim"),
    (dict(dt=7), UNSUPPORTED, "dtype"),
    (dict(odt=2), UNSUPPORTED, "dtype"),
    (dict(H=0), INVALID, "H=0"),
    (dict(B=0), INVALID, "B=0"),
    (dict(maxlen=0), INVALID, "max_seqlen"),
    (dict(tr=-1), INVALID, "total_rows"),
    (dict(cu=None), INVALID, "cu_seqlens"),
    (dict(q=None), INVALID, "q is NULL"),
    (dict(v=A + 2), ALIGN, "v base"),
    (dict(qs=100), INVALID, "q row stride"),
    (dict(ks=388), ALIGN, "k base"),          # 388 bf16 = 776 B, not a multiple of 16
    (dict(os_=386), ALIGN, "o base"),         # 386 fp32 = 1544 B, not a multiple of 16
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(maxlen=65535 * 64 + 1), UNSUPPORTED, "max_seqlen"),
    (dict(maxlen=8192, qs=192000, ks=192000, vs=192000, os_=192000), UNSUPPORTED, "2^31"),
])
def test_attn_rejects(lib, kwargs, status, needle):
    for fn in ("rag_attn", "rag_attn_tiled"):
        assert attn(lib, fn=fn, **kwargs) == status
        assert needle in binding.last_error()


def test_attn_rejects_more_pairs_than_32_bit_ids(lib):
    """The kernels number (head, image) pairs with 32-bit integers: B*H above
    2^31 - 1 is refused before any launch."""
    H = 32769  # 65535 * 32769 = 2^31 + 32768
    w = H * 64
    kw = dict(B=65535, H=H, maxlen=1, tr=65535, qs=3 * w, ks=3 * w, vs=3 * w, os_=w)
    assert attn(lib, **kw) == UNSUPPORTED
    assert "B*H" in binding.last_error()
    # one head fewer is below the limit: the check after it (the scale) decides
    assert attn(lib, **dict(kw, H=H - 1, qs=3 * (w - 64), ks=3 * (w - 64), vs=3 * (w - 64),
                            os_=w - 64, scale=float("inf"))) == INVALID
    assert "scale" in binding.last_error()
    assert lib.rag_attn_padded(A, A, A, 3 * w, 3 * w, 3 * w, BF16, A, 65535, 1, H, 64, 0.125, A,
                               w, F32, None) == UNSUPPORTED
    assert "B*H" in binding.last_error()


@pytest.mark.parametrize("kwargs,needle", [(dict(B=1025, tr=1025 * 197), "B=1025"),
                                           (dict(H=65, os_=65 * 64, qs=3 * 65 * 64, ks=3 * 65 * 64,
                                                 vs=3 * 65 * 64), "H=65"),
                                           (dict(maxlen=961), "max_seqlen=961")])
def test_attn_tiled_limits(lib, kwargs, needle):
    """The tile list's own limits; rag_attn takes the same calls (no GPU work
    happens here: the checks fail first, or the call is not made)."""
    assert attn(lib, fn="rag_attn_tiled", **kwargs) == UNSUPPORTED
    assert needle in binding.last_error()


def test_unpack_and_padded_reject(lib):
    assert lib.rag_unpack(A, 768, 768, A, A, 4, 197, A, 768, 2, None) == UNSUPPORTED
    assert "flags" in binding.last_error()
    assert lib.rag_unpack(A, 768, 768, None, A, 4, 197, A, 768, 0, None) == INVALID
    assert lib.rag_unpack(A, 768, 768, A, A, 4, 197, A + 4, 768, 0, None) == ALIGN
    assert lib.rag_unpack(A, 768, 768, A, A, 0, 197, A, 768, 0, None) == INVALID
    assert lib.rag_attn_padded(A, A, A, 1152, 1152, 1152, BF16, None, 4, 197, 6, 64, 0.125, A, 384,
                               F32, None) == INVALID
    assert lib.rag_attn_padded(A, A, A, 1152, 1152, 1152, BF16, A, 4, 197, 6, 48, 0.125, A, 384,
                               F32, None) == UNSUPPORTED
    assert lib.rag_attn_padded(A, A, A, 1152, 1152, 1152, BF16, A, 4, 0, 6, 64, 0.125, A, 384,
                               F32, None) == INVALID


def test_pipeline_rejects(lib):
    h = ctypes.c_void_p()
    assert lib.rag_pipeline_create(None, ctypes.byref(h)) == INVALID
    d = binding.PipelineDesc()
    d.keep, d.B, d.N, d.H, d.head_dim = A, 4, 197, 6, 64
    d.in_dtype, d.out_dtype, d.scale = BF16, BF16, 0.125
    d.src, d.src_row_stride = A, 2304
    d.packed, d.packed_row_stride = A, 2304
    d.cu_seqlens, d.gather_idx = A, A
    d.o_packed, d.o_packed_row_stride = A, 768
    d.dst, d.dst_row_stride = A, 768
    for field, value, status in (("head_dim", 80, UNSUPPORTED), ("max_seqlen", 500, INVALID),
                                 ("src_row_stride", 2000, INVALID), ("dst", A + 8, ALIGN),
                                 ("unpack_flags", 4, UNSUPPORTED), ("in_dtype", 5, UNSUPPORTED),
                                 ("flags", 4, UNSUPPORTED)):
        saved = getattr(d, field)
        setattr(d, field, value)
        assert lib.rag_pipeline_create(ctypes.byref(d), ctypes.byref(h)) == status, field
        assert h.value is None
        setattr(d, field, saved)
    # the direct forms capture nothing, so creating them runs no HIP call
    for flags in (binding.RAG_PIPELINE_DIRECT, binding.RAG_PIPELINE_DIRECT | binding.RAG_PIPELINE_FUSED):
        d.flags = flags
        assert lib.rag_pipeline_create(ctypes.byref(d), ctypes.byref(h)) == OK, flags
        assert h.value is not None
        lib.rag_pipeline_destroy(h)
        h = ctypes.c_void_p()
    d.flags = 0
    assert lib.rag_pipeline_launch(None, None) == INVALID
    assert lib.rag_pipeline_launch_eager(None, None) == INVALID
    lib.rag_pipeline_destroy(None)  # a no-op
    out = (ctypes.c_double * binding.RAG_FLOOR_N)()
    assert lib.rag_measure_dispatch(None, 1, 1, out, None) == INVALID


def test_binding_refuses_cpu_tensors():
    import torch
    keep = torch.zeros(2, 4, dtype=torch.uint8)
    with pytest.raises(TypeError):
        binding.rag_pack(keep, keep, keep, keep, keep)


def test_binding_rejects_rows_narrower_than_the_kernels_touch():
    """The C ABI sees a pointer and a row stride only, so a view narrower than
    the bytes a kernel reads or writes per row (e.g. the last columns of a
    wider buffer) must be refused by the binding, before anything is launched.
    CPU tensors suffice: the width is checked before the device is."""
    import torch
    H, C = 6, 384
    bf = torch.bfloat16
    wide = torch.zeros(8, 3 * C, dtype=bf)
    q, k, v = wide[:, :C], wide[:, C:2 * C], wide[:, 2 * C:]
    narrow = wide[:, 2 * C + 64:]            # C - 64 columns: 64 short of a head set
    o = torch.zeros(8, C, dtype=torch.float32)
    o_narrow = torch.zeros(8, 2 * C, dtype=torch.float32)[:, C + 8:]
    cu = torch.zeros(3, dtype=torch.int32)
    keep = torch.ones(2, 4, dtype=torch.uint8)
    for call in (lambda: binding.rag_attn(q, k, v, cu, 4, o_narrow, H=H, scale=0.125),
                 lambda: binding.rag_attn(narrow, k, v, cu, 4, o, H=H, scale=0.125),
                 lambda: binding.rag_attn(q, narrow, v, cu, 4, o, H=H, scale=0.125, tiled=True),
                 lambda: binding.rag_attn(q, k, narrow, cu, 4, o, H=H, scale=0.125),
                 lambda: binding.rag_attn_padded(q, k, narrow, keep, o, H=H, scale=0.125),
                 lambda: binding.rag_attn_gathered(keep, q, k, v, o_narrow, H=H, scale=0.125)):
        with pytest.raises(ValueError, match="rows hold"):
            call()
    # pack / re-pack / unpack: the destination must hold the source's row bytes,
    # and an explicit row_bytes must fit both
    src = torch.zeros(8, 3 * C, dtype=bf)
    g = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError, match="packed rows hold"):
        binding.rag_pack(keep, src, src[:, 8:], cu, g)
    with pytest.raises(ValueError, match="src rows hold"):
        binding.rag_pack(keep, src, src.clone(), cu, g, row_bytes=3 * C * 2 + 16)
    with pytest.raises(ValueError, match="dst rows hold"):
        binding.rag_repack(keep.view(-1), cu, g, 4, src, src[:, 8:], cu, g)
    with pytest.raises(ValueError, match="packed rows hold"):
        binding.rag_unpack(o_narrow, cu, g, o, N=4)
    # the pipeline: fused q|k|v rows for src and packed, H*64 for o_packed and dst
    for args in ((src[:, 8:], src, o, o), (src, src, o, o_narrow), (src, src, o_narrow, o)):
        with pytest.raises(ValueError, match="rows hold"):
            binding.Pipeline(keep, args[0], args[1], cu, g, args[2], args[3], H=H, scale=0.125)
    # full-width CPU tensors get past the width checks and are refused as not on the GPU
    with pytest.raises(TypeError, match="on the GPU"):
        binding.rag_attn(q, k, v, cu, 4, o, H=H, scale=0.125)


def test_attn_gathered_rejects(lib):
    def call(keep=A, B=4, N=197, q=A, qs=1152, dt=BF16, H=6, hd=64, scale=0.125, o=A, os_=384,
             odt=F32, flags=0, max_seqlen=0):
        return lib.rag_attn_gathered(keep, B, N, max_seqlen, q, q, q, qs, qs, qs, dt, H, hd, scale,
                                     o, os_, odt, flags, None)
    assert call(flags=2) == UNSUPPORTED and "flags" in binding.last_error()
    assert call(keep=None) == INVALID
    assert call(N=0) == INVALID
    assert call(max_seqlen=-1) == INVALID and "max_seqlen" in binding.last_error()
    assert call(max_seqlen=198) == INVALID
    assert call(hd=128) == UNSUPPORTED
    assert call(q=A + 4) == ALIGN
    assert call(scale=float("nan")) == INVALID
    assert lib.rag_pipeline_launch_fused(None, None) == INVALID


def _block_desc(**kw):
    d = binding.BlockDesc()
    d.H, d.mlp_ratio, d.eps, d.scale = 6, 4, 1e-6, 0.125
    for i, name in enumerate(binding.Block.NAMES):
        setattr(d, name, A + 0x1000 * i)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(H=0), UNSUPPORTED, "H=0"),
    (dict(H=33), UNSUPPORTED, "H=33"),
    (dict(mlp_ratio=9), UNSUPPORTED, "mlp_ratio"),
    (dict(eps=0.0), INVALID, "eps"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(w_qkv=None), INVALID, "w_qkv"),
    (dict(b_fc2=A + 4), ALIGN, "b_fc2"),
    (dict(w_fc1=A + 8), ALIGN, "w_fc1"),
])
def test_block_create_rejects(lib, kwargs, status, needle):
    h = ctypes.c_void_p()
    d = _block_desc(**kwargs)
    assert lib.rag_block_create(ctypes.byref(d), ctypes.byref(h)) == status
    assert needle in binding.last_error()
    assert not h.value


def test_block_calls_reject_without_a_block(lib):
    assert lib.rag_block_create(None, None) == INVALID
    assert lib.rag_block_forward(None, A, A, 10, A, 1, 10, A, 1 << 20, None) == INVALID
    assert lib.rag_block_forward_padded(None, A, A, A, 1, 10, A, 1 << 20, None) == INVALID
    assert lib.rag_block_forward_static(None, A, A, 10, A, 1, 10, None) == INVALID
    lib.rag_block_destroy(None)  # a no-op
    assert lib.rag_block_scratch_bytes(-1, 6, 4) == 0
    assert lib.rag_block_scratch_bytes(10, 6, 4) == 10 * (6 * 384 + 4 * 384) * 2
