"""numpy FP64 form of the attention definition, for small shapes.

TEST INFRASTRUCTURE ONLY (see the package docstring). This is a second, independent
evaluation of the definition: library matrix products and a library-style softmax,
where ``attn_oracle.c`` uses explicit loops. It follows the reference of page "Audit
SGLang interfaces and refresh validated kernel solutions",
definitions/dense_attention/noncausal_dense_attention_h32_d{64,128}.json: scores from
the bqhd,bkhd->bhqk contraction, times head_dim ** -0.5, softmax over keys, then the
bhqk,bkhd->bqhd contraction with V. The prefix-cached operator
(definitions/block_causal_attention/prefix_cached_block_causal_h32_d128.json) first
concatenates prefix and current keys and values along the sequence axis. The
block-causal operator without prefix
(definitions/block_causal_attention/prefix_cached_block_causal_h32_d128_prefix0.json)
builds a boolean visibility matrix from positions and image ids, fills the hidden
scores with -inf and takes the same softmax.
"""
import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns (uint16) to float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def softmax_last(x: np.ndarray) -> np.ndarray:
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, scale=None, allowed=None):
    """q [B,Nq,H,D], k/v [B,Nk,H,D] as BF16 bits or float arrays -> FP64 [B,Nq,H,D].
    allowed: optional [Nq, Nk] boolean visibility (False -> score -inf)."""
    qf = bf16_bits_to_f64(q) if q.dtype == np.uint16 else np.asarray(q, np.float64)
    kf = bf16_bits_to_f64(k) if k.dtype == np.uint16 else np.asarray(k, np.float64)
    vf = bf16_bits_to_f64(v) if v.dtype == np.uint16 else np.asarray(v, np.float64)
    D = qf.shape[-1]
    s = D ** -0.5 if scale is None else scale
    # [B,H,Nq,D] @ [B,H,D,Nk] -> [B,H,Nq,Nk]
    scores = np.matmul(qf.transpose(0, 2, 1, 3), kf.transpose(0, 2, 3, 1)) * s
    if allowed is not None:
        scores = np.where(allowed[None, None], scores, -np.inf)
    p = softmax_last(scores)
    # [B,H,Nq,Nk] @ [B,H,Nk,D] -> [B,H,Nq,D] -> [B,Nq,H,D]
    return np.matmul(p, vf.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)


def prefix_attention(q, kp, vp, kc, vc, scale=None):
    """Keys cat(kp, kc) and values cat(vp, vc) along the sequence axis."""
    return attention(q, np.concatenate([kp, kc], axis=1), np.concatenate([vp, vc], axis=1),
                     scale=scale)


def block_causal_visibility(image_ids) -> np.ndarray:
    """[N, N] boolean: query i sees key j iff j <= i or both share an id >= 0."""
    ids = np.asarray(image_ids, dtype=np.int64)
    pos = np.arange(ids.size)
    same_image = (ids[:, None] == ids[None, :]) & (ids[:, None] >= 0)
    return (pos[None, :] <= pos[:, None]) | same_image


def block_causal_attention(q, k, v, image_ids):
    return attention(q, k, v, allowed=block_causal_visibility(image_ids))


def na_window_search(L: int, k: int) -> np.ndarray:
    """[L, L] boolean: position i sees j on an axis of length L with an odd window k.
    Among all windows of k consecutive positions inside [0, L) that contain i, the one
    whose centre is nearest to i (a search over the windows, independent of the start
    formula of the C oracle)."""
    vis = np.zeros((L, L), dtype=bool)
    for i in range(L):
        best = None
        for s in range(0, L - k + 1):
            if s <= i < s + k:
                dist = abs(s + k // 2 - i)
                if best is None or dist < best[0]:
                    best = (dist, s)
        vis[i, best[1]:best[1] + k] = True
    return vis


def na3d_visibility(T: int, Y: int, X: int, kernel) -> np.ndarray:
    """[T*Y*X, T*Y*X] boolean visibility of 3-D neighborhood attention: the product of
    the per-axis windows, positions flattened as (t*Y + y)*X + x."""
    kt, ky, kx = kernel
    vt, vy, vx = na_window_search(T, kt), na_window_search(Y, ky), na_window_search(X, kx)
    return (vt[:, None, None, :, None, None] & vy[None, :, None, None, :, None] &
            vx[None, None, :, None, None, :]).reshape(T * Y * X, T * Y * X)


def na3d_attention(q, k, v, kernel):
    """[B, T, Y, X, H, D] -> FP64 [B, T, Y, X, H, D]; scores are plain dot products."""
    B, T, Y, X, H, D = q.shape
    flat = lambda a: a.reshape(B, T * Y * X, H, D)
    o = attention(flat(q), flat(k), flat(v), scale=1.0, allowed=na3d_visibility(T, Y, X, kernel))
    return o.reshape(B, T, Y, X, H, D)
