"""Thin ctypes binding of librag.so (argument marshalling only).

Every function here takes torch tensors that live on the GPU, turns them into
pointers, strides and sizes, and calls the C entry point of the same name on
torch's current stream.  No arithmetic of the path happens in Python, and there
is no fallback: if librag.so is missing or a tensor is not on the GPU the call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librag.so")

RAG_OK = 0
STATUS = {0: "RAG_OK", 1: "RAG_ERR_INVALID_ARG", 2: "RAG_ERR_UNSUPPORTED", 3: "RAG_ERR_ALIGNMENT",
          4: "RAG_ERR_HIP", 5: "RAG_ERR_NO_MEMORY"}
RAG_DTYPE_F32 = 0
RAG_DTYPE_BF16 = 1
RAG_UNPACK_ZERO_DROPPED = 1
RAG_HEAD_DIM = 64
RAG_PIPELINE_FUSED = 1
RAG_PIPELINE_DIRECT = 2
RAG_FLOOR_N = 36
RAG_STAGES_N = 7

#: Every symbol include/rag.h declares.
EXPORTS = ("rag_pack", "rag_repack", "rag_attn", "rag_attn_tiled", "rag_unpack", "rag_attn_padded", "rag_attn_gathered",
           "rag_pipeline_create", "rag_pipeline_launch", "rag_pipeline_launch_eager",
           "rag_pipeline_launch_fused", "rag_pipeline_destroy",
           "rag_measure_dispatch", "rag_measure_stages", "rag_last_error", "rag_status_string",
           "rag_version", "rag_block_scratch_bytes", "rag_block_create", "rag_block_forward",
           "rag_block_forward_padded", "rag_block_forward_static", "rag_block_destroy")

_lib = None


class RagError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class PipelineDesc(ctypes.Structure):
    _fields_ = [
        ("keep", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("H", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("max_seqlen", ctypes.c_int32),
        ("src", ctypes.c_void_p), ("src_row_stride", ctypes.c_int64),
        ("packed", ctypes.c_void_p), ("packed_row_stride", ctypes.c_int64),
        ("cu_seqlens", ctypes.c_void_p), ("gather_idx", ctypes.c_void_p),
        ("max_seqlen_dev", ctypes.c_void_p),
        ("o_packed", ctypes.c_void_p), ("o_packed_row_stride", ctypes.c_int64),
        ("dst", ctypes.c_void_p), ("dst_row_stride", ctypes.c_int64),
        ("unpack_flags", ctypes.c_uint32), ("flags", ctypes.c_uint32),
    ]


class BlockDesc(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int32), ("mlp_ratio", ctypes.c_int32),
        ("eps", ctypes.c_float), ("scale", ctypes.c_float),
        ("ln1_gamma", ctypes.c_void_p), ("ln1_beta", ctypes.c_void_p),
        ("w_qkv", ctypes.c_void_p), ("b_qkv", ctypes.c_void_p),
        ("w_proj", ctypes.c_void_p), ("b_proj", ctypes.c_void_p),
        ("ln2_gamma", ctypes.c_void_p), ("ln2_beta", ctypes.c_void_p),
        ("w_fc1", ctypes.c_void_p), ("b_fc1", ctypes.c_void_p),
        ("w_fc2", ctypes.c_void_p), ("b_fc2", ctypes.c_void_p),
    ]


def load(path: str = LIB_PATH):
    """Open librag.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("librag.so is not built (%s); run "
                           "`python -m ragged_attention_token_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, i64, u32, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                              ctypes.c_float)
    lib.rag_pack.argtypes = [vp, i32, i32, vp, i64, i32, vp, i64, vp, vp, vp, vp]
    lib.rag_attn.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, i32, i32, i32, i32, i32, f32, vp,
                             i64, i32, vp]
    lib.rag_attn_tiled.argtypes = lib.rag_attn.argtypes
    lib.rag_unpack.argtypes = [vp, i64, i32, vp, vp, i32, i32, vp, i64, u32, vp]
    lib.rag_repack.argtypes = [vp, vp, vp, i32, i32, i32, vp, i64, i32, vp, i64, vp, vp, vp]
    lib.rag_attn_padded.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, i32, i32, i32, i32, f32,
                                    vp, i64, i32, vp]
    lib.rag_attn_gathered.argtypes = [vp, i32, i32, i32, vp, vp, vp, i64, i64, i64, i32, i32, i32, f32,
                                      vp, i64, i32, u32, vp]
    lib.rag_pipeline_create.argtypes = [ctypes.POINTER(PipelineDesc), ctypes.POINTER(vp)]
    lib.rag_pipeline_launch_fused.argtypes = [vp, vp]
    lib.rag_pipeline_launch.argtypes = [vp, vp]
    lib.rag_pipeline_launch_eager.argtypes = [vp, vp]
    lib.rag_pipeline_destroy.argtypes = [vp]
    lib.rag_pipeline_destroy.restype = None
    lib.rag_measure_dispatch.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_double), vp]
    lib.rag_measure_stages.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double), vp]
    lib.rag_block_scratch_bytes.argtypes = [i32, i32, i32]
    lib.rag_block_scratch_bytes.restype = ctypes.c_size_t
    lib.rag_block_create.argtypes = [ctypes.POINTER(BlockDesc), ctypes.POINTER(vp)]
    lib.rag_block_forward.argtypes = [vp, vp, vp, i32, vp, i32, i32, vp, ctypes.c_size_t, vp]
    lib.rag_block_forward_padded.argtypes = [vp, vp, vp, vp, i32, i32, vp, ctypes.c_size_t, vp]
    lib.rag_block_forward_static.argtypes = [vp, vp, vp, i32, vp, i32, i32, vp]
    lib.rag_block_destroy.argtypes = [vp]
    lib.rag_block_destroy.restype = None
    lib.rag_last_error.restype = ctypes.c_char_p
    lib.rag_status_string.argtypes = [i32]
    lib.rag_status_string.restype = ctypes.c_char_p
    lib.rag_version.restype = i32
    for name in ("rag_pack", "rag_repack", "rag_attn", "rag_attn_tiled", "rag_unpack", "rag_attn_padded", "rag_attn_gathered",
                 "rag_pipeline_create", "rag_pipeline_launch", "rag_pipeline_launch_eager",
                 "rag_pipeline_launch_fused", "rag_measure_dispatch", "rag_measure_stages",
                 "rag_block_create", "rag_block_forward", "rag_block_forward_padded",
                 "rag_block_forward_static"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def last_error() -> str:
    return load().rag_last_error().decode()


def _check(status: int):
    if status != RAG_OK:
        raise RagError(status, last_error())


try:  # the current stream's handle without building a Stream object
    _raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover
    _raw_stream = None


def _stream(stream, device: Optional[int] = None) -> int:
    """hipStream_t of `stream` (a torch stream or a raw handle), or of torch's
    current stream on `device` (default: the current device)."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device() if device is None else device)
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _gpu(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a torch tensor on the GPU" % name)
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RAG_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return RAG_DTYPE_BF16
    raise TypeError("dtype must be float32 or bfloat16, got %s" % t.dtype)


def _row_bytes(t: torch.Tensor) -> int:
    """Bytes of one row: the elements of every axis after the first."""
    n = 1
    for s in t.shape[1:]:
        n *= s
    return n * t.element_size()


def _inner_contiguous(t: torch.Tensor) -> bool:
    """Whether the axes after the first are laid out contiguously (read from the
    strides, without building a view)."""
    shape, strides = t.shape, t.stride()
    if len(shape) == 2:  # the common case, without the general loop
        return strides[1] == 1 or shape[1] == 1
    expect = 1
    for size, stride in zip(reversed(shape[1:]), reversed(strides[1:])):
        if size != 1 and stride != expect:
            return False
        expect *= size
    return True


def _check_rows(t: torch.Tensor, name: str, min_row_bytes: int = 0) -> None:
    """A tensor whose first axis is rows and whose remaining axes are contiguous,
    each row holding at least `min_row_bytes` bytes.  The kernels read or write
    that many bytes from the start of every row, and the C ABI sees only a
    pointer and a stride, so the width is checked here: a narrower view (e.g.
    the last columns of a wider buffer) would let the kernels touch the
    neighbouring columns or run past the end of the allocation.  (Shape and
    strides are read once: this runs on every call.)"""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor on the GPU" % name)
    shape = t.shape
    if len(shape) == 2:
        if t.stride(1) != 1 and shape[1] != 1:
            raise ValueError("%s: elements within a row must be contiguous" % name)
        row_bytes = shape[1] * t.element_size()
    else:
        if len(shape) < 2:
            raise ValueError("%s must have a row axis and a column axis" % name)
        if not _inner_contiguous(t):
            raise ValueError("%s: elements within a row must be contiguous" % name)
        row_bytes = _row_bytes(t)
    if row_bytes < min_row_bytes:
        raise ValueError("%s rows hold %d bytes; the call reads or writes %d bytes of each row"
                         % (name, row_bytes, min_row_bytes))


def _rows(t: torch.Tensor, name: str, min_row_bytes: int = 0, checked: bool = False):
    """(pointer, row stride in elements) of a row tensor on the GPU (checked as
    in _check_rows, unless the caller has just done so)."""
    if not checked:
        _check_rows(t, name, min_row_bytes)
    _gpu(t, name)
    return t.data_ptr(), t.stride(0)


def _qkvo(q, k, v, o, H, head_dim):
    """Pointers and row strides of attention's q, k, v, o: each row must hold
    the H * head_dim elements the kernels read (q, k, v) or write (o)."""
    named = ((q, "q"), (k, "k"), (v, "v"), (o, "o"))
    for t, name in named:  # every width before any device check
        _check_rows(t, name, int(H) * int(head_dim) * getattr(t, "element_size", lambda: 0)())
    out = []
    for t, name in named:
        out.extend(_rows(t, name, checked=True))
    return out


def rag_pack(keep: torch.Tensor, src: torch.Tensor, packed: torch.Tensor, cu_seqlens: torch.Tensor,
             gather_idx: torch.Tensor, max_seqlen_dev: Optional[torch.Tensor] = None,
             row_bytes: Optional[int] = None, stream=None) -> None:
    """keep [B,N] uint8; src rows [B*N, ...]; packed rows [>= B*N, ...];
    cu_seqlens int32 [B+1]; gather_idx int32 [>= B*N]; max_seqlen_dev int32 [1]."""
    if not isinstance(keep, torch.Tensor) or keep.dtype != torch.uint8 or keep.dim() != 2 \
            or not keep.is_contiguous():
        raise ValueError("keep must be a contiguous uint8 [B, N] tensor")
    B, N = keep.shape
    rb = _row_bytes(src) if row_bytes is None else int(row_bytes)
    _check_rows(src, "src", rb)
    _check_rows(packed, "packed", rb)
    sp, ss = _rows(src, "src", checked=True)
    pp, ps = _rows(packed, "packed", checked=True)
    _gpu(keep, "keep")
    for t, name in ((cu_seqlens, "cu_seqlens"), (gather_idx, "gather_idx")):
        _gpu(t, name)
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % name)
    if src.shape[0] < B * N or packed.shape[0] < B * N or gather_idx.numel() < B * N \
            or cu_seqlens.numel() < B + 1:
        raise ValueError("buffers smaller than the B*N capacity")
    mp = None
    if max_seqlen_dev is not None:
        _gpu(max_seqlen_dev, "max_seqlen_dev")
        mp = max_seqlen_dev.data_ptr()
    _check(load().rag_pack(keep.data_ptr(), B, N, sp, ss * src.element_size(), rb, pp,
                           ps * packed.element_size(), cu_seqlens.data_ptr(),
                           gather_idx.data_ptr(), mp, _stream(stream)))


def rag_repack(keep_packed: torch.Tensor, cu_in: torch.Tensor, gather_in: torch.Tensor,
               max_rows_in: int, src: torch.Tensor, dst: torch.Tensor, cu_out: torch.Tensor,
               gather_out: torch.Tensor, row_bytes: Optional[int] = None, stream=None) -> None:
    """A later pruning stage on packed rows: keep_packed uint8 [>= rows] (one
    byte per input row); cu_in int32 [B+1]; gather_in int32 [>= rows]; src /
    dst rows [rows, ...]; cu_out int32 [B+1]; gather_out int32 [>= rows]."""
    if not isinstance(keep_packed, torch.Tensor) or keep_packed.dtype != torch.uint8 \
            or not keep_packed.is_contiguous():
        raise ValueError("keep_packed must be a contiguous uint8 tensor")
    rb = _row_bytes(src) if row_bytes is None else int(row_bytes)
    _check_rows(src, "src", rb)
    _check_rows(dst, "dst", rb)
    sp, ss = _rows(src, "src", checked=True)
    dp, ds = _rows(dst, "dst", checked=True)
    _gpu(keep_packed, "keep_packed")
    for t, name in ((cu_in, "cu_in"), (gather_in, "gather_in"), (cu_out, "cu_out"),
                    (gather_out, "gather_out")):
        _gpu(t, name)
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % name)
    B = cu_in.numel() - 1
    rows = src.shape[0]
    if keep_packed.numel() < rows or gather_in.numel() < rows or dst.shape[0] < rows \
            or gather_out.numel() < rows or cu_out.numel() < B + 1:
        raise ValueError("buffers smaller than src's rows")
    _check(load().rag_repack(keep_packed.data_ptr(), cu_in.data_ptr(), gather_in.data_ptr(), B,
                             int(max_rows_in), rows, sp, ss * src.element_size(), rb, dp,
                             ds * dst.element_size(), cu_out.data_ptr(), gather_out.data_ptr(),
                             _stream(stream)))


def rag_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
             max_seqlen: int, o: torch.Tensor, H: int, scale: float, head_dim: int = RAG_HEAD_DIM,
             total_rows: Optional[int] = None, stream=None, tiled: bool = False) -> None:
    """q, k, v, o: [rows, >= H*head_dim] (row stride free, rows contiguous inside);
    cu_seqlens int32 [B+1] on the GPU; max_seqlen a host upper bound.  tiled:
    call rag_attn_tiled (the same result over the device-built tile list)."""
    qp, qs, kp, ks, vp, vs, op, os_ = _qkvo(q, k, v, o, H, head_dim)
    _gpu(cu_seqlens, "cu_seqlens")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    rows = min(q.shape[0], k.shape[0], v.shape[0], o.shape[0])
    tr = rows if total_rows is None else int(total_rows)
    if tr > rows:
        raise ValueError("total_rows larger than the buffers")
    B = cu_seqlens.numel() - 1
    fn = load().rag_attn_tiled if tiled else load().rag_attn
    _check(fn(qp, kp, vp, qs, ks, vs, _dtype_code(q), cu_seqlens.data_ptr(), B, int(max_seqlen), tr,
              int(H), int(head_dim), float(scale), op, os_, _dtype_code(o), _stream(stream)))


def rag_attn_tiled(q, k, v, cu_seqlens, max_seqlen, o, H, scale, head_dim=RAG_HEAD_DIM,
                   total_rows=None, stream=None) -> None:
    """rag_attn over the device-built tile list (B <= 1024, max_seqlen <= 960)."""
    rag_attn(q, k, v, cu_seqlens, max_seqlen, o, H, scale, head_dim, total_rows, stream, tiled=True)


class AttnPlan:
    """A prepared rag_attn call on fixed tensors: the arguments are checked and
    turned into C values once, so that each call only looks up the current
    stream and enters the C ABI (the per-call cost of a Python caller stays
    near the C++ dispatch floor).  Arguments as rag_attn; the tensors are kept
    alive here and must keep their storage."""

    def __init__(self, q, k, v, cu_seqlens, max_seqlen, o, H, scale, head_dim=RAG_HEAD_DIM,
                 total_rows=None, tiled=False):
        qp, qs, kp, ks, vp, vs, op, os_ = _qkvo(q, k, v, o, H, head_dim)
        _gpu(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        if not (q.dtype == k.dtype == v.dtype):
            raise TypeError("q, k, v must share a dtype")
        rows = min(q.shape[0], k.shape[0], v.shape[0], o.shape[0])
        tr = rows if total_rows is None else int(total_rows)
        if tr > rows:
            raise ValueError("total_rows larger than the buffers")
        lib = load()
        self._fn = lib.rag_attn_tiled if tiled else lib.rag_attn
        c = ctypes
        self._args = (c.c_void_p(qp), c.c_void_p(kp), c.c_void_p(vp), c.c_int64(qs), c.c_int64(ks),
                      c.c_int64(vs), c.c_int32(_dtype_code(q)), c.c_void_p(cu_seqlens.data_ptr()),
                      c.c_int32(cu_seqlens.numel() - 1), c.c_int32(int(max_seqlen)), c.c_int32(tr),
                      c.c_int32(int(H)), c.c_int32(int(head_dim)), c.c_float(float(scale)),
                      c.c_void_p(op), c.c_int64(os_), c.c_int32(_dtype_code(o)))
        self._dev = q.device.index
        self._keep_alive = (q, k, v, cu_seqlens, o)

    def __call__(self, stream=None) -> None:
        status = self._fn(*self._args, _stream(stream, self._dev))
        if status != RAG_OK:
            raise RagError(status, last_error())


def rag_unpack(packed: torch.Tensor, cu_seqlens: torch.Tensor, gather_idx: torch.Tensor,
               dst: torch.Tensor, N: int, flags: int = 0, row_bytes: Optional[int] = None,
               stream=None) -> None:
    """packed rows [>= B*N, ...] -> dst rows [B*N, ...]."""
    rb = _row_bytes(dst) if row_bytes is None else int(row_bytes)
    _check_rows(packed, "packed", rb)
    _check_rows(dst, "dst", rb)
    pp, ps = _rows(packed, "packed", checked=True)
    dp, ds = _rows(dst, "dst", checked=True)
    for t, name in ((cu_seqlens, "cu_seqlens"), (gather_idx, "gather_idx")):
        _gpu(t, name)
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % name)
    B = cu_seqlens.numel() - 1
    if dst.shape[0] < B * N or packed.shape[0] < B * N or gather_idx.numel() < B * N:
        raise ValueError("buffers smaller than the B*N capacity")
    _check(load().rag_unpack(pp, ps * packed.element_size(), rb, cu_seqlens.data_ptr(),
                             gather_idx.data_ptr(), B, int(N), dp, ds * dst.element_size(),
                             int(flags), _stream(stream)))


def rag_attn_padded(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: torch.Tensor,
                    o: torch.Tensor, H: int, scale: float, head_dim: int = RAG_HEAD_DIM,
                    stream=None) -> None:
    """Padded comparator: q/k/v/o rows b*N + n of the [B, N] layout."""
    qp, qs, kp, ks, vp, vs, op, os_ = _qkvo(q, k, v, o, H, head_dim)
    _gpu(keep, "keep")
    if keep.dtype != torch.uint8 or keep.dim() != 2 or not keep.is_contiguous():
        raise ValueError("keep must be a contiguous uint8 [B, N] tensor")
    B, N = keep.shape
    if min(q.shape[0], k.shape[0], v.shape[0], o.shape[0]) < B * N:
        raise ValueError("q/k/v/o need B*N rows")
    _check(load().rag_attn_padded(qp, kp, vp, qs, ks, vs, _dtype_code(q), keep.data_ptr(), B, N,
                                  int(H), int(head_dim), float(scale), op, os_, _dtype_code(o),
                                  _stream(stream)))


def rag_attn_gathered(keep: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      o: torch.Tensor, H: int, scale: float, flags: int = 0,
                      head_dim: int = RAG_HEAD_DIM, max_seqlen: int = 0, stream=None) -> None:
    """Pack + attend + unpack in one launch: q/k/v/o rows b*N + n of the [B, N]
    layout; attention over each image's kept rows, written to those rows of o.
    max_seqlen: host bound of the kept count per image (0 = N)."""
    qp, qs, kp, ks, vp, vs, op, os_ = _qkvo(q, k, v, o, H, head_dim)
    _gpu(keep, "keep")
    if keep.dtype != torch.uint8 or keep.dim() != 2 or not keep.is_contiguous():
        raise ValueError("keep must be a contiguous uint8 [B, N] tensor")
    B, N = keep.shape
    if min(q.shape[0], k.shape[0], v.shape[0], o.shape[0]) < B * N:
        raise ValueError("q/k/v/o need B*N rows")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    _check(load().rag_attn_gathered(keep.data_ptr(), B, N, int(max_seqlen), qp, kp, vp, qs, ks, vs, _dtype_code(q),
                                    int(H), int(head_dim), float(scale), op, os_, _dtype_code(o),
                                    int(flags), _stream(stream)))


class Pipeline:
    """pack -> attend -> unpack captured once into a HIP graph.

    src: fused rows [B*N, 3*H*64] (q | k | v); all buffers are kept alive here
    and fixed for the pipeline's lifetime."""

    def __init__(self, keep, src, packed, cu_seqlens, gather_idx, o_packed, dst, H, scale,
                 max_seqlen: int = 0, max_seqlen_dev=None, unpack_flags: int = 0,
                 fused_graph: bool = False, direct: bool = False):
        B, N = keep.shape
        C = int(H) * RAG_HEAD_DIM
        # row widths the three kernels touch: fused q|k|v rows of src / packed,
        # output rows of o_packed / dst
        for t, name, elems in ((src, "src", 3 * C), (packed, "packed", 3 * C),
                               (o_packed, "o_packed", C), (dst, "dst", C)):
            _check_rows(t, name, elems * getattr(t, "element_size", lambda: 0)())
        for t, name in ((keep, "keep"), (cu_seqlens, "cu_seqlens"), (gather_idx, "gather_idx")):
            _gpu(t, name)
        if src.dtype != packed.dtype or o_packed.dtype != dst.dtype:
            raise TypeError("src/packed and o_packed/dst must share dtypes")
        if min(src.shape[0], packed.shape[0], o_packed.shape[0], dst.shape[0],
               gather_idx.numel()) < B * N or cu_seqlens.numel() < B + 1:
            raise ValueError("buffers smaller than the B*N capacity")
        self._keep_alive = (keep, src, packed, cu_seqlens, gather_idx, o_packed, dst,
                            max_seqlen_dev)
        d = PipelineDesc()
        d.keep = keep.data_ptr()
        d.B, d.N, d.H, d.head_dim = B, N, int(H), RAG_HEAD_DIM
        d.in_dtype, d.out_dtype = _dtype_code(src), _dtype_code(dst)
        d.scale = float(scale)
        d.max_seqlen = int(max_seqlen)
        d.src, d.src_row_stride = src.data_ptr(), src.stride(0) * src.element_size()
        d.packed, d.packed_row_stride = packed.data_ptr(), packed.stride(0) * packed.element_size()
        d.cu_seqlens, d.gather_idx = cu_seqlens.data_ptr(), gather_idx.data_ptr()
        d.max_seqlen_dev = max_seqlen_dev.data_ptr() if max_seqlen_dev is not None else None
        d.o_packed = o_packed.data_ptr()
        d.o_packed_row_stride = o_packed.stride(0) * o_packed.element_size()
        d.dst, d.dst_row_stride = dst.data_ptr(), dst.stride(0) * dst.element_size()
        d.unpack_flags = int(unpack_flags)
        d.flags = (RAG_PIPELINE_FUSED if fused_graph else 0) | (RAG_PIPELINE_DIRECT if direct else 0)
        self.desc = d
        self._dev = keep.device.index
        handle = ctypes.c_void_p()
        _check(load().rag_pipeline_create(ctypes.byref(d), ctypes.byref(handle)))
        self._h = handle

    def launch(self, stream=None) -> None:
        _check(load().rag_pipeline_launch(self._h, _stream(stream, self._dev)))

    def launch_eager(self, stream=None) -> None:
        _check(load().rag_pipeline_launch_eager(self._h, _stream(stream, self._dev)))

    def launch_fused(self, stream=None) -> None:
        _check(load().rag_pipeline_launch_fused(self._h, _stream(stream, self._dev)))

    def measure_dispatch(self, warmup: int = 100, iters: int = 1000, stream=None) -> dict:
        out = (ctypes.c_double * RAG_FLOOR_N)()
        _check(load().rag_measure_dispatch(self._h, int(warmup), int(iters), out, _stream(stream)))
        keys = ["empty_roundtrip", "empty_enqueue", "attn_roundtrip", "attn_enqueue",
                "eager3_roundtrip", "graph_roundtrip", "padded_roundtrip", "fused_roundtrip",
                "fused_enqueue", "empty_arg_enqueue", "graph1_roundtrip", "graph1_launch"]
        res = {}
        for i, k in enumerate(keys):
            res[k] = {"p10": out[3 * i], "p50": out[3 * i + 1], "p90": out[3 * i + 2]}
        return res

    def measure_stages(self, iters: int = 500, stream=None) -> dict:
        """Device microseconds per launch of each stage (see rag_measure_stages)."""
        out = (ctypes.c_double * RAG_STAGES_N)()
        _check(load().rag_measure_stages(self._h, int(iters), out, _stream(stream)))
        return dict(zip(("pack", "attn", "unpack", "padded", "eager_pass", "graph_pass",
                         "fused_pass"), list(out)))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            load().rag_pipeline_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Block:
    """One DeiT encoder block on packed (or padded) bf16 token rows; see
    rag_block_desc in include/rag.h.  `params` maps names to GPU tensors:
    ln1_gamma, ln1_beta, ln2_gamma, ln2_beta, b_qkv, b_proj, b_fc1, b_fc2
    (fp32) and w_qkv [3C, C], w_proj [C, C], w_fc1 [hidden, C], w_fc2
    [C, hidden] (bf16, the [out, in] layout of a linear layer's weight).  The
    tensors are kept alive here; their shapes are checked against H and
    mlp_ratio, since the C ABI sees only pointers."""

    NAMES = ("ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_proj", "b_proj", "ln2_gamma",
             "ln2_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2")

    def __init__(self, params: dict, H: int, scale: float, mlp_ratio: int = 4, eps: float = 1e-6):
        self.H, self.mlp_ratio = int(H), int(mlp_ratio)
        self.C = self.H * RAG_HEAD_DIM
        C, hid = self.C, self.C * self.mlp_ratio
        shapes = {"ln1_gamma": (C,), "ln1_beta": (C,), "ln2_gamma": (C,), "ln2_beta": (C,),
                  "w_qkv": (3 * C, C), "b_qkv": (3 * C,), "w_proj": (C, C), "b_proj": (C,),
                  "w_fc1": (hid, C), "b_fc1": (hid,), "w_fc2": (C, hid), "b_fc2": (C,)}
        for k in self.NAMES:
            t = params[k]
            want = torch.bfloat16 if k.startswith("w_") else torch.float32
            if not isinstance(t, torch.Tensor) or tuple(t.shape) != shapes[k] or t.dtype != want:
                raise ValueError("%s must be a %s tensor of shape %s" % (k, want, shapes[k]))
        self.params = {k: _gpu(params[k], k).contiguous() for k in self.NAMES}
        d = BlockDesc()
        d.H, d.mlp_ratio, d.eps, d.scale = self.H, self.mlp_ratio, float(eps), float(scale)
        for k in self.NAMES:
            setattr(d, k, self.params[k].data_ptr())
        self._desc = d
        handle = ctypes.c_void_p()
        _check(load().rag_block_create(ctypes.byref(d), ctypes.byref(handle)))
        self._h = handle
        self._scratch = None

    def _scratch_for(self, rows: int) -> torch.Tensor:
        need = load().rag_block_scratch_bytes(int(rows), self.H, self.mlp_ratio)
        if self._scratch is None or self._scratch.numel() < need:
            self._scratch = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        return self._scratch

    def _rows(self, x, y, rows):
        for t, name in ((x, "x"), (y, "y")):
            _gpu(t, name)
            if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 2 \
                    or t.shape[1] != self.C or t.shape[0] < rows:
                raise ValueError("%s must be a contiguous bf16 [>= rows, C] tensor" % name)

    def forward(self, x: torch.Tensor, y: torch.Tensor, rows: int, cu_seqlens: torch.Tensor,
                max_seqlen: int, stream=None) -> None:
        """y[:rows] = block(x[:rows]) with ragged attention over cu_seqlens."""
        self._rows(x, y, rows)
        _gpu(cu_seqlens, "cu_seqlens")
        sc = self._scratch_for(rows)
        _check(load().rag_block_forward(self._h, x.data_ptr(), y.data_ptr(), int(rows),
                                        cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                        int(max_seqlen), sc.data_ptr(), sc.numel(),
                                        _stream(stream)))

    def forward_static(self, x: torch.Tensor, y: torch.Tensor, rows: int, cu_seqlens: torch.Tensor,
                       max_seqlen: int, stream=None) -> None:
        """forward() with the intermediates in the library's static device
        array: the call allocates nothing (see rag_block_forward_static)."""
        self._rows(x, y, rows)
        _gpu(cu_seqlens, "cu_seqlens")
        _check(load().rag_block_forward_static(self._h, x.data_ptr(), y.data_ptr(), int(rows),
                                               cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                               int(max_seqlen), _stream(stream)))

    def forward_padded(self, x: torch.Tensor, y: torch.Tensor, keep: torch.Tensor,
                       stream=None) -> None:
        """y = block(x) on all B*N rows, padded attention with masked keys."""
        _gpu(keep, "keep")
        B, N = keep.shape
        self._rows(x, y, B * N)
        sc = self._scratch_for(B * N)
        _check(load().rag_block_forward_padded(self._h, x.data_ptr(), y.data_ptr(),
                                               keep.data_ptr(), B, N, sc.data_ptr(), sc.numel(),
                                               _stream(stream)))

    def close(self) -> None:
        if self._h:
            load().rag_block_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
