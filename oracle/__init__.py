"""Plain fp64 CPU oracle for ragged pack -> attend -> unpack.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and imports nothing from it; the HIP library never calls it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, single thread); this module
only marshals numpy arrays into it.  Sources for each routine are cited in
``oracle.c``:

* pack / unpack: agents-report.net, "Triton Ragged Attention 與
  pack-attend-unpack", section 方法概覽 (method overview), the token-packing and
  write-back steps;
* ragged attention: "Dispatch-Aware Ragged Attention for Pruned Vision
  Transformers", abstract (bidirectional attention over each image's surviving
  tokens) and the same blog section (the ragged attention kernel);
* padded attention: the blog's section 問題 (problem): pad to one length, mask;
* re-pack (a later pruning stage on packed tokens): the paper's earlier
  abstract (fugumt.com summary page) lists the pruning methods, which drop
  tokens at more than one depth; the compaction is the pack step above.

Pins (see ``tests/test_oracle.py``): exhaustive bf16 decode against torch's own
conversion; pack against ``numpy.flatnonzero``; hand-derived worked examples under
``tests/golden/``; closed forms; invariants; brute force with ``math.fsum``;
torch's fp64 ``scaled_dot_product_attention`` on the CPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = dbl
    lib.oracle_pack.argtypes = [vp, i32, i32, vp, i64, i32, vp, i64, vp, vp]
    lib.oracle_pack.restype = i64
    lib.oracle_unpack.argtypes = [vp, i64, i32, vp, vp, i32, vp, i64]
    lib.oracle_unpack.restype = None
    lib.oracle_repack.argtypes = [vp, vp, vp, i32, vp, i64, i32, vp, i64, vp, vp]
    lib.oracle_repack.restype = i64
    lib.oracle_attn.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, i32, i32, i32, dbl, vp,
                                i64, vp, vp]
    lib.oracle_attn.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, i32, i32, i32, dbl, vp,
                                     i32, vp, i64, vp, vp]
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_padded.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, i32, i32, i32,
                                       i32, dbl, vp, i64, vp, vp]
    lib.oracle_attn_padded.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(_LIB_PATH)
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DTYPE_F32
    if a.dtype == np.uint16:  # raw bfloat16 bit patterns
        return DTYPE_BF16
    raise TypeError("oracle inputs are float32 or uint16 (bfloat16 bits), got %s" % a.dtype)


def bf16_to_f64(bits: int) -> float:
    """Exact value of one bfloat16 bit pattern."""
    return _load().oracle_bf16_to_f64(int(bits) & 0xFFFF)


def pack(keep: np.ndarray, src_rows: np.ndarray):
    """Pack the kept rows of ``src_rows`` ([B*N, row] of any dtype, C-contiguous).

    Returns (packed [T, row], cu_seqlens int32 [B+1], gather_idx int32 [T]).
    """
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    B, N = keep.shape
    src = np.ascontiguousarray(src_rows).reshape(B * N, -1)
    row_bytes = src.shape[1] * src.itemsize
    packed = np.zeros_like(src)
    cu = np.zeros(B + 1, dtype=np.int32)
    gather = np.zeros(B * N, dtype=np.int32)
    T = _load().oracle_pack(_ptr(keep), B, N, _ptr(src), row_bytes, row_bytes, _ptr(packed),
                            row_bytes, _ptr(cu), _ptr(gather))
    return packed[:T].copy(), cu, gather[:T].copy()


def repack(keep_packed: np.ndarray, cu_in: np.ndarray, gather_in: np.ndarray,
           packed_rows: np.ndarray):
    """Re-prune packed rows: keep_packed[t] != 0 keeps packed row t of the image
    cu_in says it belongs to.  Returns (rows [T', row], cu_out int32 [B+1],
    gather_out int32 [T']) with gather_out composed through gather_in."""
    cu = np.ascontiguousarray(cu_in, dtype=np.int32)
    B = cu.shape[0] - 1
    T = int(cu[B])
    if cu[0] != 0 or (np.diff(cu) < 0).any():
        raise ValueError("cu_in must start at 0 and not decrease")
    keep = np.ascontiguousarray(keep_packed, dtype=np.uint8)
    g = np.ascontiguousarray(gather_in, dtype=np.int32)
    src = np.ascontiguousarray(packed_rows)
    # (an explicit row width: reshape cannot infer it from zero rows)
    src = src.reshape(src.shape[0], int(np.prod(src.shape[1:], dtype=np.int64)))
    if keep.shape[0] < T or g.shape[0] < T or src.shape[0] < T:
        raise ValueError("keep / gather / rows shorter than cu_in[B]")
    row_bytes = src.shape[1] * src.itemsize
    out = np.zeros((max(T, 1), src.shape[1]), dtype=src.dtype)
    cu_out = np.zeros(B + 1, dtype=np.int32)
    g_out = np.zeros(max(T, 1), dtype=np.int32)
    T2 = _load().oracle_repack(_ptr(keep), _ptr(cu), _ptr(g), B, _ptr(src), row_bytes, row_bytes,
                               _ptr(out), row_bytes, _ptr(cu_out), _ptr(g_out))
    return out[:T2].copy(), cu_out, g_out[:T2].copy()


def unpack(packed: np.ndarray, cu_seqlens: np.ndarray, gather_idx: np.ndarray,
           dst: np.ndarray) -> np.ndarray:
    """Scatter packed rows into a copy of ``dst`` ([B*N, row]); returns the copy."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    B = cu.shape[0] - 1
    T = int(cu[B])
    out = np.ascontiguousarray(dst).copy()
    rows = out.reshape(out.shape[0], -1)
    pk = np.ascontiguousarray(packed).reshape(-1, rows.shape[1])
    if pk.dtype != rows.dtype:
        raise TypeError("packed and dst dtypes differ")
    g = np.ascontiguousarray(gather_idx, dtype=np.int32)
    if g.shape[0] < T or pk.shape[0] < T:
        raise ValueError("gather_idx / packed shorter than cu_seqlens[B]")
    if T and (g[:T].min() < 0 or g[:T].max() >= rows.shape[0]):
        raise ValueError("gather index out of range")
    row_bytes = rows.shape[1] * rows.itemsize
    _load().oracle_unpack(_ptr(pk), row_bytes, row_bytes, _ptr(cu), _ptr(g), B, _ptr(rows),
                          row_bytes)
    return out


def attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: np.ndarray, H: int, d: int,
         scale: float) -> np.ndarray:
    """Ragged attention on packed rows.

    q, k, v: [T, >= H*d] float32 or uint16 (bf16 bits), any row stride (rows are
    the first axis; head h is columns h*d .. h*d+d-1).  Returns fp64 [T, H*d].
    """
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    B = cu.shape[0] - 1
    T = int(cu[B])
    code = _dtype_code(q)
    arrs = []
    for a in (q, k, v):
        if _dtype_code(a) != code:
            raise TypeError("q, k, v dtypes differ")
        a2 = a.reshape(a.shape[0], -1)
        if a2.strides[1] != a2.itemsize:
            a2 = np.ascontiguousarray(a2)
        if a2.shape[0] < T or a2.shape[1] < H * d:
            raise ValueError("q/k/v too small for cu_seqlens / H*d")
        arrs.append(a2)
    lens = np.diff(cu)
    if (lens < 0).any() or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    Lmax = int(lens.max()) if B else 0
    o = np.zeros((T, H * d), dtype=np.float64)
    s_buf = np.zeros(max(Lmax, 1), dtype=np.float64)
    r_buf = np.zeros(max(Lmax, 1), dtype=np.int64)
    qs, ks, vs = (a.strides[0] // a.itemsize for a in arrs)
    rc = _load().oracle_attn(_ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]), qs, ks, vs, code,
                             _ptr(cu), B, H, d, float(scale), _ptr(o), H * d, _ptr(s_buf),
                             _ptr(r_buf))
    if rc != 0:
        raise ValueError("oracle_attn rejected its arguments")
    return o


def attn_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: np.ndarray, H: int, d: int,
              scale: float, rows) -> np.ndarray:
    """attn() for the listed packed query rows only: fp64 [len(rows), H*d], row r
    of the result being attn(...)[rows[r]] (the same arithmetic)."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    B = cu.shape[0] - 1
    code = _dtype_code(q)
    arrs = []
    for a in (q, k, v):
        if _dtype_code(a) != code:
            raise TypeError("q, k, v dtypes differ")
        a2 = a.reshape(a.shape[0], -1)
        if a2.strides[1] != a2.itemsize:
            a2 = np.ascontiguousarray(a2)
        arrs.append(a2)
    lens = np.diff(cu)
    if (lens < 0).any() or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    r = np.ascontiguousarray(rows, dtype=np.int64)
    Lmax = int(lens.max()) if B else 0
    o = np.zeros((r.shape[0], H * d), dtype=np.float64)
    s_buf = np.zeros(max(Lmax, 1), dtype=np.float64)
    r_buf = np.zeros(max(Lmax, 1), dtype=np.int64)
    qs, ks, vs = (a.strides[0] // a.itemsize for a in arrs)
    rc = _load().oracle_attn_rows(_ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]), qs, ks, vs, code,
                                  _ptr(cu), B, H, d, float(scale), _ptr(r), int(r.shape[0]), _ptr(o),
                                  H * d, _ptr(s_buf), _ptr(r_buf))
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return o


def attn_padded(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray, H: int, d: int,
                scale: float) -> np.ndarray:
    """Padded, key-masked attention over [B*N] rows; returns fp64 [B*N, H*d]."""
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    B, N = keep.shape
    code = _dtype_code(q)
    arrs = []
    for a in (q, k, v):
        a2 = a.reshape(B * N, -1)
        if a2.strides[1] != a2.itemsize:
            a2 = np.ascontiguousarray(a2)
        if _dtype_code(a2) != code or a2.shape[1] < H * d:
            raise ValueError("bad q/k/v for padded attention")
        arrs.append(a2)
    o = np.zeros((B * N, H * d), dtype=np.float64)
    s_buf = np.zeros(max(N, 1), dtype=np.float64)
    r_buf = np.zeros(max(N, 1), dtype=np.int64)
    qs, ks, vs = (a.strides[0] // a.itemsize for a in arrs)
    rc = _load().oracle_attn_padded(_ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]), qs, ks, vs, code,
                                    _ptr(keep), B, N, H, d, float(scale), _ptr(o), H * d,
                                    _ptr(s_buf), _ptr(r_buf))
    if rc != 0:
        raise ValueError("oracle_attn_padded rejected its arguments")
    return o
