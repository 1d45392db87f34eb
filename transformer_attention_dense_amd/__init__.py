"""Python binding of the MI355X dense attention library (libattn_dense.so).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in include/attn_dense.h. There is no CPU fallback; if the
library is missing or fails to load, importing the low-level functions raises.

Low-level functions (same names and arguments as the C ABI; tensors passed as raw
device addresses, ``stream`` as an integer hipStream_t):
    attn_dense, attn_prefix, attn_cross, attn_block_causal, attn_na3d, attn_fwd_ex,
    attn_fwd_ex_noalloc,
    attn_plan, attn_na3d_plan, attn_reserve_workspace, attn_set_workspace, attn_strerror,
    attn_abi_version

Tensor-level helpers (torch is used for device memory and the current stream):
    dense(q, k, v, out=None), prefix(q, kp, vp, kc, vc, out=None),
    cross(q, k, v, out=None), fwd_ex(...), set_workspace(buffer_or_None)
Operations follow page "Audit SGLang interfaces and refresh validated kernel
solutions": definitions/dense_attention/noncausal_dense_attention_h32_d{64,128}.json
and definitions/block_causal_attention/prefix_cached_block_causal_h32_d128.json.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_dense.so")

ATTN_OK = 0
ERRORS = {
    -1: "ATTN_ERR_NULL",
    -2: "ATTN_ERR_SHAPE",
    -3: "ATTN_ERR_UNSUPPORTED",
    -4: "ATTN_ERR_ALIGN",
    -5: "ATTN_ERR_ALIAS",
    -6: "ATTN_ERR_OVERFLOW",
    -7: "ATTN_ERR_WORKSPACE",
    -8: "ATTN_ERR_HIP",
}

# Exported symbols, in header order.
SYMBOLS = ("attn_dense", "attn_prefix", "attn_cross", "attn_block_causal", "attn_na3d",
           "attn_fwd_ex", "attn_fwd_ex_noalloc",
           "attn_plan", "attn_na3d_plan", "attn_reserve_workspace", "attn_set_workspace",
           "attn_strerror", "attn_abi_version")


class AttnError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({strerror(code)})")


_lib = None


def library() -> ctypes.CDLL:
    """Loads libattn_dense.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    p, i, ll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.attn_dense.argtypes = [p, p, p, p, i, i, i, i, p]
    lib.attn_prefix.argtypes = [p, p, p, p, p, p, i, i, i, i, i, p]
    lib.attn_cross.argtypes = [p, p, p, p, i, i, i, i, i, p]
    lib.attn_block_causal.argtypes = [p, p, p, p, p, i, i, i, i, p]
    lib.attn_na3d.argtypes = [p, p, p, p] + [i] * 9 + [p]
    lib.attn_fwd_ex.argtypes = [p, p, p, i, p, p, i, p, i, i, i, i, i, i, p]
    lib.attn_fwd_ex_noalloc.argtypes = [p, p, p, i, p, p, i, p, i, i, i, i, i, i, p]
    lib.attn_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i),
                              ctypes.POINTER(ll), ctypes.POINTER(ll)]
    lib.attn_na3d_plan.argtypes = [i] * 9 + [ctypes.POINTER(i), ctypes.POINTER(ll)]
    lib.attn_reserve_workspace.argtypes = [ll]
    lib.attn_set_workspace.argtypes = [p, ll]
    lib.attn_strerror.argtypes = [i]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    for name in SYMBOLS:
        if name != "attn_strerror":
            getattr(lib, name).restype = i
    _lib = lib
    return lib


# ---------------------------------------------------------------- C ABI, same names

def attn_dense(q, k, v, out, B, N, H, D, stream=0) -> int:
    return library().attn_dense(q, k, v, out, B, N, H, D, stream)


def attn_prefix(q, kp, vp, kc, vc, out, B, Nq, Np, H, D, stream=0) -> int:
    return library().attn_prefix(q, kp, vp, kc, vc, out, B, Nq, Np, H, D, stream)


def attn_cross(q, k, v, out, B, Nq, Nk, H, D, stream=0) -> int:
    return library().attn_cross(q, k, v, out, B, Nq, Nk, H, D, stream)


def attn_block_causal(q, k, v, image_ids, out, B, N, H, D, stream=0) -> int:
    return library().attn_block_causal(q, k, v, image_ids, out, B, N, H, D, stream)


def attn_na3d(q, k, v, out, B, T, Y, X, H, D, kt, ky, kx, stream=0) -> int:
    return library().attn_na3d(q, k, v, out, B, T, Y, X, H, D, kt, ky, kx, stream)


def attn_fwd_ex(q, k0, v0, n0, k1, v1, n1, out, B, Nq, H, D, num_splits=0, waves=0,
                stream=0) -> int:
    return library().attn_fwd_ex(q, k0, v0, n0, k1, v1, n1, out, B, Nq, H, D, num_splits,
                                 waves, stream)


def attn_fwd_ex_noalloc(q, k0, v0, n0, k1, v1, n1, out, B, Nq, H, D, num_splits=0, waves=0,
                        stream=0) -> int:
    return library().attn_fwd_ex_noalloc(q, k0, v0, n0, k1, v1, n1, out, B, Nq, H, D,
                                         num_splits, waves, stream)


def attn_na3d_plan(B, T, Y, X, H, D, kt, ky, kx):
    """Host-only launch plan of attn_na3d: dict(query_cols, workgroups)."""
    qc, wg = ctypes.c_int(), ctypes.c_longlong()
    rc = library().attn_na3d_plan(B, T, Y, X, H, D, kt, ky, kx, ctypes.byref(qc),
                                  ctypes.byref(wg))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_na3d_plan")
    return {"query_cols": qc.value, "workgroups": wg.value}


def attn_plan(B, Nq, Nk, H, D, num_splits=0, waves=0):
    """Host-only launch plan: dict(splits, waves, workgroups, workspace_bytes)."""
    s, w = ctypes.c_int(), ctypes.c_int()
    wg, ws = ctypes.c_longlong(), ctypes.c_longlong()
    rc = library().attn_plan(B, Nq, Nk, H, D, num_splits, waves, ctypes.byref(s),
                             ctypes.byref(w), ctypes.byref(wg), ctypes.byref(ws))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_plan")
    return {"splits": s.value, "waves": w.value, "workgroups": wg.value,
            "workspace_bytes": ws.value}


def attn_reserve_workspace(nbytes) -> int:
    return library().attn_reserve_workspace(nbytes)


def attn_set_workspace(ptr, nbytes) -> int:
    return library().attn_set_workspace(ptr, nbytes)


def attn_strerror(code) -> str:
    return library().attn_strerror(code).decode()


def attn_abi_version() -> int:
    return library().attn_abi_version()


def strerror(code) -> str:
    try:
        return attn_strerror(code)
    except OSError:
        return "library not loaded"


# ---------------------------------------------------------------- tensor helpers

_torch = None


def _t():
    """torch, imported on first use (the low-level functions above do not need it)."""
    global _torch
    if _torch is None:
        import torch
        _torch = torch
    return _torch


def _check(t, name, shape=None):
    torch = _t()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, N, H, D] tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(t):
    """The current stream of t's device as a raw hipStream_t. torch's raw accessor
    returns the handle without building a Stream object (a few microseconds per call,
    which is most of the host cost of a small call); the public path is the fallback."""
    torch = _t()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _out(q, out):
    torch = _t()
    if out is None:
        return torch.empty_like(q)
    _check(out, "out", q.shape)
    return out


def dense(q, k, v, out=None):
    """O = softmax(Q K^T D^-0.5) V for q, k, v of shape [B, N, H, D] (bf16, GPU)."""
    _check(q, "q")
    B, N, H, D = q.shape
    _check(k, "k", q.shape)
    _check(v, "v", q.shape)
    out = _out(q, out)
    rc = attn_dense(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, N, H, D,
                    _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_dense")
    return out


def cross(q, k, v, out=None):
    """Cross attention: q [B, Nq, H, D], k/v [B, Nk, H, D]."""
    _check(q, "q")
    B, Nq, H, D = q.shape
    _check(k, "k")
    Nk = k.shape[1]
    _check(k, "k", (B, Nk, H, D))
    _check(v, "v", (B, Nk, H, D))
    out = _out(q, out)
    rc = attn_cross(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Nq, Nk, H, D,
                    _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_cross")
    return out


def prefix(q, kp, vp, kc, vc, out=None):
    """Prefix-cached attention in the pages' operand order (Q, K_prefix, V_prefix,
    K_current, V_current); keys are the prefix rows followed by the current rows."""
    _check(q, "q")
    B, Nq, H, D = q.shape
    _check(kp, "k_prefix")
    Np = kp.shape[1]
    _check(kp, "k_prefix", (B, Np, H, D))
    _check(vp, "v_prefix", (B, Np, H, D))
    _check(kc, "k_current", q.shape)
    _check(vc, "v_current", q.shape)
    out = _out(q, out)
    kpp = kp.data_ptr() if Np else None
    vpp = vp.data_ptr() if Np else None
    rc = attn_prefix(q.data_ptr(), kpp, vpp, kc.data_ptr(), vc.data_ptr(), out.data_ptr(), B,
                     Nq, Np, H, D, _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_prefix")
    return out


def block_causal(q, k, v, image_ids, out=None):
    """Block-causal attention without prefix in the pages' operand order (Q, K_current,
    V_current, image_ids): row i sees key j when j <= i or when both carry the same
    nonnegative image id. image_ids: int32 [N] on the same GPU (text = -1)."""
    torch = _t()
    _check(q, "q")
    B, N, H, D = q.shape
    _check(k, "k_current", q.shape)
    _check(v, "v_current", q.shape)
    if not isinstance(image_ids, torch.Tensor) or image_ids.dtype != torch.int32:
        raise TypeError("image_ids must be an int32 torch.Tensor")
    if image_ids.device != q.device or tuple(image_ids.shape) != (N,) or \
            not image_ids.is_contiguous():
        raise ValueError(f"image_ids must be a contiguous [{N}] tensor on {q.device}")
    out = _out(q, out)
    rc = attn_block_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), image_ids.data_ptr(),
                           out.data_ptr(), B, N, H, D, _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_block_causal")
    return out


def na3d(q, k, v, kernel, out=None):
    """3-D neighborhood attention: q, k, v [B, T, Y, X, H, D] bf16 on the GPU, D = 64,
    kernel = (kt, ky, kx) odd window sizes; scores are plain dot products (the model's
    scale is in q)."""
    torch = _t()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 torch.Tensor")
        if t.device.type != "cuda" or t.dim() != 6 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, T, Y, X, H, D] tensor on a GPU")
        if tuple(t.shape) != tuple(q.shape) or t.device != q.device:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(q.shape)}")
    B, T, Y, X, H, D = q.shape
    kt, ky, kx = (int(x) for x in kernel)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    rc = attn_na3d(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, T, Y, X, H, D,
                   kt, ky, kx, _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_na3d")
    return out


def fwd_ex(q, k0, v0, k1=None, v1=None, out=None, num_splits=0, waves=0):
    """General form: keys k0 then k1 (optional), explicit split count and waves."""
    _check(q, "q")
    B, Nq, H, D = q.shape
    _check(k0, "k0")
    n0 = k0.shape[1]
    _check(v0, "v0", (B, n0, H, D))
    n1 = 0
    if k1 is not None:
        n1 = k1.shape[1]
        _check(k1, "k1", (B, n1, H, D))
        _check(v1, "v1", (B, n1, H, D))
    out = _out(q, out)
    rc = attn_fwd_ex(q.data_ptr(), k0.data_ptr() if n0 else None, v0.data_ptr() if n0 else None,
                     n0, k1.data_ptr() if n1 else None, v1.data_ptr() if n1 else None, n1,
                     out.data_ptr(), B, Nq, H, D, num_splits, waves, _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_ex")
    return out


def set_workspace(buf):
    """Hands the library a caller-owned work space for buf's device (a contiguous GPU
    tensor of any dtype, e.g. torch.empty(nbytes, dtype=torch.uint8, device=...)), or
    reverts the current device to the library's own buffer with None. The caller keeps
    buf alive while calls that use it may still run."""
    torch = _t()
    if buf is None:
        rc = attn_set_workspace(None, 0)
    else:
        if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or \
                not buf.is_contiguous():
            raise ValueError("the work space must be a contiguous GPU tensor")
        if buf.device.index != torch.cuda.current_device():
            raise ValueError("the work space must be on the current device")
        rc = attn_set_workspace(buf.data_ptr(), buf.numel() * buf.element_size())
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_set_workspace")
