"""FP64 CPU oracle for dense noncausal attention and prefix-cached attention.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library and its
Python binding never import it, and it imports nothing from them.

Two independent evaluations of the same definition are provided:

* :func:`attention_rows` / :func:`attention` / :func:`prefix_attention` call the
  plain C loops in ``attn_oracle.c`` (FP64, one query row at a time).
* :mod:`oracle.attn_np` writes the same formula with numpy FP64 matrix products and
  a numpy softmax, for small shapes.

The definition (page "Audit SGLang interfaces and refresh validated kernel
solutions", definitions/dense_attention/noncausal_dense_attention_h32_d{64,128}.json
"reference", and definitions/block_causal_attention/
prefix_cached_block_causal_h32_d128.json "reference"):

    O[b,i,h,:] = sum_j softmax_j( D**-0.5 * <Q[b,i,h,:], K[b,j,h,:]> ) * V[b,j,h,:]

with K, V the concatenation (K_prefix, K_current), (V_prefix, V_current) for the
prefix-cached operator. The block-causal operator without prefix (same page,
definitions/block_causal_attention/prefix_cached_block_causal_h32_d128_prefix0.json
"reference") restricts row i's softmax to the keys j with j <= i or with the same
nonnegative image id (image_ids [N], text = -1); see :func:`block_causal_rows`. Inputs are BF16 bit patterns held in ``numpy.uint16``
arrays of layout [B, N, H, D]; outputs are unrounded FP64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        # ORACLE_LIB lets the mutation test point the pins at a deliberately broken
        # build of attn_oracle.c; normal runs use the library built next to it.
        path = os.environ.get("ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.oracle_attn_rows.restype = ctypes.c_int
        p = ctypes.c_void_p
        L = ctypes.c_long
        lib.oracle_attn_rows.argtypes = [p, p, p, L, p, p, L, L, L, L, L, p, L, p, p, p,
                                         ctypes.c_double]
        lib.oracle_block_causal_rows.restype = ctypes.c_int
        lib.oracle_block_causal_rows.argtypes = [p, p, p, p, L, L, L, L, p, L, p, p, p]
        lib.oracle_na3d_rows.restype = ctypes.c_int
        lib.oracle_na3d_rows.argtypes = [p, p, p] + [L] * 9 + [p, L, p]
        lib.oracle_num_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def num_threads() -> int:
    """OpenMP threads the C oracle uses."""
    return int(_lib().oracle_num_threads())


def _bits(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.ndim != 4:
        raise TypeError(f"{name}: expected uint16 BF16 bits of rank 4, got {a.dtype} {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def attention_rows(q, k0, v0, k1=None, v1=None, rows=None, scale=None,
                   want_lse=False, want_psum=False):
    """FP64 attention output for selected query rows.

    q: [B, Nq, H, D] bits; (k0, v0): [B, n0, H, D] first key segment; (k1, v1):
    optional [B, n1, H, D] second segment appended after the first.
    rows: flat indices (b*Nq + i)*H + h, or None for all rows in [B, Nq, H] order.
    Returns out [len(rows), D] (and lse, psum if requested).
    """
    q = _bits(q, "q")
    B, Nq, H, D = q.shape
    k0 = _bits(k0, "k0")
    v0 = _bits(v0, "v0")
    n0 = k0.shape[1]
    if k1 is not None:
        k1 = _bits(k1, "k1")
        v1 = _bits(v1, "v1")
        n1 = k1.shape[1]
    else:
        n1 = 0
    for t, n in ((k0, n0), (v0, n0)) + (((k1, n1), (v1, n1)) if n1 else ()):
        if t.shape != (B, n, H, D):
            raise ValueError(f"key/value shape {t.shape} does not match q {q.shape}")
    if rows is None:
        nrows = B * Nq * H
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.empty((nrows, D), dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64) if want_lse else None
    psum = np.empty(nrows, dtype=np.float64) if want_psum else None
    rc = _lib().oracle_attn_rows(
        _ptr(q), _ptr(k0), _ptr(v0), n0, _ptr(k1), _ptr(v1), n1, B, Nq, H, D,
        _ptr(rows_arr), nrows, _ptr(out), _ptr(lse), _ptr(psum),
        float(scale) if scale is not None else 0.0)
    if rc != 0:
        raise RuntimeError(f"oracle_attn_rows failed with code {rc}")
    res = [out]
    if want_lse:
        res.append(lse)
    if want_psum:
        res.append(psum)
    return res[0] if len(res) == 1 else tuple(res)


def attention(q, k, v, scale=None):
    """Dense attention, full output [B, Nq, H, D] in FP64."""
    B, Nq, H, D = q.shape
    return attention_rows(q, k, v, scale=scale).reshape(B, Nq, H, D)


def prefix_attention(q, kp, vp, kc, vc, scale=None):
    """Prefix-cached attention: keys (kp then kc), values (vp then vc). [B, Nq, H, D]."""
    B, Nq, H, D = q.shape
    if kp.shape[1] == 0:
        return attention(q, kc, vc, scale=scale)
    return attention_rows(q, kp, vp, kc, vc, scale=scale).reshape(B, Nq, H, D)



def _ids(image_ids, n):
    ids = np.ascontiguousarray(np.asarray(image_ids), dtype=np.int32)
    if ids.shape != (n,):
        raise ValueError(f"image_ids: expected shape ({n},), got {ids.shape}")
    return ids


def block_causal_rows(q, k, v, image_ids, rows=None, want_lse=False, want_psum=False):
    """FP64 block-causal attention (no prefix) for selected query rows.

    q, k, v: [B, N, H, D] bits; image_ids: [N] int32 (text = -1). Row i sees key j
    when j <= i, or when image_ids[i] >= 0 and image_ids[j] == image_ids[i].
    rows: flat indices (b*N + i)*H + h, or None for every row. Returns out [rows, D].
    """
    q, k, v = _bits(q, "q"), _bits(k, "k"), _bits(v, "v")
    B, N, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"k {k.shape} / v {v.shape} must match q {q.shape}")
    ids = _ids(image_ids, N)
    if rows is None:
        nrows = B * N * H
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.empty((nrows, D), dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64) if want_lse else None
    psum = np.empty(nrows, dtype=np.float64) if want_psum else None
    rc = _lib().oracle_block_causal_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(ids), B, N, H, D,
                                         _ptr(rows_arr), nrows, _ptr(out), _ptr(lse),
                                         _ptr(psum))
    if rc != 0:
        raise RuntimeError(f"oracle_block_causal_rows failed with code {rc}")
    res = [out]
    if want_lse:
        res.append(lse)
    if want_psum:
        res.append(psum)
    return res[0] if len(res) == 1 else tuple(res)


def block_causal_attention(q, k, v, image_ids):
    """Block-causal attention (no prefix), full output [B, N, H, D] in FP64."""
    B, N, H, D = q.shape
    return block_causal_rows(q, k, v, image_ids).reshape(B, N, H, D)


def _bits6(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.ndim != 6:
        raise TypeError(f"{name}: expected uint16 BF16 bits of rank 6, got {a.dtype} {a.shape}")
    return a


def na3d_rows(q, k, v, kernel, rows=None):
    """FP64 3-D neighborhood attention for selected query rows.

    q, k, v: [B, T, Y, X, H, D] bits; kernel = (kt, ky, kx), odd, each at most its
    axis. rows: flat indices ((((b*T + t)*Y + y)*X + x)*H + h), or None for every row.
    Returns out [rows, D].
    """
    q, k, v = _bits6(q, "q"), _bits6(k, "k"), _bits6(v, "v")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"k {k.shape} / v {v.shape} must match q {q.shape}")
    B, T, Y, X, H, D = q.shape
    kt, ky, kx = (int(x) for x in kernel)
    if rows is None:
        nrows = B * T * Y * X * H
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.empty((nrows, D), dtype=np.float64)
    rc = _lib().oracle_na3d_rows(_ptr(q), _ptr(k), _ptr(v), B, T, Y, X, H, D, kt, ky, kx,
                                 _ptr(rows_arr), nrows, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_na3d_rows failed with code {rc}")
    return out


def na3d_attention(q, k, v, kernel):
    """3-D neighborhood attention, full output [B, T, Y, X, H, D] in FP64."""
    return na3d_rows(q, k, v, kernel).reshape(q.shape)
