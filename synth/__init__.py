"""Seeded synthetic inputs for the attention workloads.

This module holds input generation and workload bookkeeping only (shapes, seeds,
FLOP and byte counts). It contains none of the attention arithmetic, so both the
FP64 oracle and the HIP library can be fed from it without sharing any code.

The pages measure on captured serving activations (page "Audit SGLang interfaces
and refresh validated kernel solutions", README "Task acceptance configs" and the
dataset description) that are not available here; these seeded inputs stand in for
them, keeping the operators' shapes (H = 32, D in {64, 128}, layout [B, N, H, D],
prefix operand order Q, K_prefix, V_prefix, K_current, V_current) and the BF16 type.

Generator: numpy ``Generator(PCG64(seed))``, ``standard_normal(dtype=float32)``
times sigma, rounded to BF16 with round-to-nearest-even on the FP32 bit pattern.
Seeds are ``1000 * (k + 1) + t`` for workload index k and tensor index t in call
order (dense: Q=0, K=1, V=2; prefix: Q=0, K_prefix=1, V_prefix=2, K_current=3,
V_current=4; block-causal: Q=0, K_current=1, V_current=2), so every tensor is
reproducible on its own.

Block-causal image ids follow the serving engine's segment list as the pages
describe it (same page, the capture script's block-attention hook): text tokens
-1, image segments numbered 0, 1, ... in order of appearance, each a contiguous
block. A workload states its segments as (kind, length) pairs.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

H_PAGES = 32  # the pages fix H = 32 for every attention definition


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 values to BF16 (round to nearest, ties to even); returns uint16 bits.

    NaN inputs are not expected from the generator and are not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bits to FP32 (for inspection and input statistics)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """BF16 bits of iid N(0, sigma^2) draws from PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def outlier_channels(seed: int, H: int, D: int, count: int = 4) -> np.ndarray:
    """[H, count] distinct channel indices per head, drawn from PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return np.stack([np.sort(g.choice(D, size=count, replace=False)) for _ in range(H)])


def normal_bf16_outliers(shape, seed: int, sigma: float, channels: np.ndarray,
                         factor: float) -> np.ndarray:
    """N(0, sigma^2) draws with the given per-head channels multiplied by ``factor``
    before rounding to BF16. shape is [B, N, H, D]; channels is [H, count]."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(sigma)
    H = shape[2]
    for h in range(H):
        x[:, :, h, channels[h]] *= np.float32(factor)
    return f32_to_bf16_bits(x)


@dataclass
class Workload:
    """One synthetic attention workload.

    kind "dense": Q [B,Nq,H,D], K/V [B,Nk,H,D] (Nk == Nq for self attention).
    kind "prefix": Q [B,Nq,H,D], K/V_prefix [B,Np,H,D], K/V_current [B,Nq,H,D].
    kind "block_causal": Q, K_current, V_current [B,Nq,H,D] and image_ids [Nq] from
    ``segments`` (a list of ("text" | "image", length) pairs summing to Nq).
    kind "na3d": Q, K, V [B,T,Y,X,H,D] (``grid`` = (T, Y, X)), 3-D neighborhood attention
    with window ``kernel``; every query sees kt*ky*kx keys.
    """
    name: str
    kind: str
    B: int
    Nq: int
    H: int
    D: int
    index: int            # workload index k used in the seeds
    Nk: int = 0           # dense: key count (defaults to Nq)
    Np: int = 0           # prefix: prefix length
    sigma_qk: float = 1.0
    outliers: int = 0     # channels per head scaled by outlier_factor in Q and K
    outlier_factor: float = 8.0
    segments: Tuple[Tuple[str, int], ...] = ()
    grid: Tuple[int, int, int] = ()     # na3d: (T, Y, X); Nq = T*Y*X positions
    kernel: Tuple[int, int, int] = ()   # na3d: (kt, ky, kx) window sizes
    description: str = ""
    extra: Dict = field(default_factory=dict)

    def __post_init__(self):
        if self.kind == "na3d":
            T, Y, X = self.grid
            self.Nq = T * Y * X
            if any(k % 2 == 0 or k > L for k, L in zip(self.kernel, self.grid)):
                raise ValueError(f"{self.name}: windows must be odd and fit their axes")
        if self.kind in ("dense", "block_causal") and self.Nk == 0:
            self.Nk = self.Nq
        if self.kind == "block_causal":
            if sum(n for _, n in self.segments) != self.Nq:
                raise ValueError(f"{self.name}: segments do not add up to Nq={self.Nq}")

    def image_ids(self) -> np.ndarray:
        """int32 [Nq]: -1 for text, 0, 1, ... for the image segments in order."""
        ids = np.empty(self.Nq, dtype=np.int32)
        pos, nxt = 0, 0
        for kind, n in self.segments:
            if kind == "text":
                ids[pos:pos + n] = -1
            elif kind == "image":
                ids[pos:pos + n] = nxt
                nxt += 1
            else:
                raise ValueError(f"unknown segment kind {kind}")
            pos += n
        return ids

    def visible_per_row(self) -> np.ndarray:
        """int64 [Nq]: keys a block-causal query row sees (contiguous image blocks)."""
        out = np.empty(self.Nq, dtype=np.int64)
        pos = 0
        for kind, n in self.segments:
            out[pos:pos + n] = np.arange(pos + 1, pos + n + 1) if kind == "text" else pos + n
            pos += n
        return out

    @property
    def visible_pairs(self) -> int:
        """Query-key pairs a block-causal call computes: a text row i sees i + 1 keys,
        a row of an image block ending at e sees e keys (contiguous blocks)."""
        total, pos = 0, 0
        for kind, n in self.segments:
            if kind == "text":
                total += n * pos + n * (n + 1) // 2
            else:
                total += n * (pos + n)
            pos += n
        return total

    @property
    def keys(self) -> int:
        """Keys per query row."""
        if self.kind == "na3d":
            kt, ky, kx = self.kernel
            return kt * ky * kx
        return self.Np + self.Nq if self.kind == "prefix" else self.Nk

    @property
    def flop(self) -> int:
        """4*B*H*Nq*Nk*D: the two contractions (QK^T and PV), 2 FLOP per multiply-add.
        Block-causal: 4*B*H*D per visible query-key pair."""
        if self.kind == "block_causal":
            return 4 * self.B * self.H * self.D * self.visible_pairs
        return 4 * self.B * self.H * self.Nq * self.keys * self.D

    @property
    def exps(self) -> int:
        if self.kind == "block_causal":
            return self.B * self.H * self.visible_pairs
        return self.B * self.H * self.Nq * self.keys

    @property
    def algorithmic_bytes(self) -> int:
        """Every input read once and the output written once, 2 bytes per element."""
        q = self.B * self.Nq * self.H * self.D
        if self.kind == "na3d":  # Q, K, V and O all cover the whole volume
            return 2 * 4 * q
        kv = 2 * self.B * self.keys * self.H * self.D
        ids = 4 * self.Nq if self.kind == "block_causal" else 0  # int32 image ids
        return 2 * (q + kv + q) + ids

    def seed(self, t: int) -> int:
        return 1000 * (self.index + 1) + t

    def tensors(self) -> Tuple[np.ndarray, ...]:
        """Arrays in call order: BF16 bits (Q, K, V) or (Q, Kp, Vp, Kc, Vc); block-causal
        (Q, K_current, V_current, image_ids)."""
        B, Nq, H, D = self.B, self.Nq, self.H, self.D
        if self.kind == "na3d":  # Q carries the model's scale: sigma_qk
            shape = (B,) + tuple(self.grid) + (H, D)
            return (normal_bf16(shape, self.seed(0), self.sigma_qk),
                    normal_bf16(shape, self.seed(1), 1.0), normal_bf16(shape, self.seed(2), 1.0))
        if self.kind == "block_causal":
            return tuple(normal_bf16((B, Nq, H, D), self.seed(t), self.sigma_qk if t < 2 else 1.0)
                         for t in range(3)) + (self.image_ids(),)
        if self.kind == "dense":
            shapes = [(B, Nq, H, D), (B, self.Nk, H, D), (B, self.Nk, H, D)]
            qk = {0, 1}
        else:
            shapes = [(B, Nq, H, D), (B, self.Np, H, D), (B, self.Np, H, D),
                      (B, Nq, H, D), (B, Nq, H, D)]
            qk = {0, 1, 3}
        chans = None
        if self.outliers:
            chans = outlier_channels(1000 * (self.index + 1) + 99, H, D, self.outliers)
        out = []
        for t, shp in enumerate(shapes):
            if t in qk and chans is not None:
                out.append(normal_bf16_outliers(shp, self.seed(t), self.sigma_qk, chans,
                                                self.outlier_factor))
            elif t in qk:
                out.append(normal_bf16(shp, self.seed(t), self.sigma_qk))
            else:
                out.append(normal_bf16(shp, self.seed(t), 1.0))
        return tuple(out)


# The six workloads. Index k feeds the seeds; k = 0..5.
WORKLOADS: List[Workload] = [
    Workload("dense_b1_n256_h32_d64", "dense", 1, 256, 32, 64, 0,
             description="Dense noncausal MHA, B=1 N=256 H=32 D=64, N(0,1), scale 1/8"),
    Workload("dense_b1_n4096_h32_d128", "dense", 1, 4096, 32, 128, 1,
             description="Dense noncausal MHA, B=1 N=4096 H=32 D=128, N(0,1), "
                         "scale 1/sqrt(128)"),
    Workload("dense_b2_n16384_h32_d64", "dense", 2, 16384, 32, 64, 2,
             description="Dense noncausal MHA long sequence, B=2 N=16384 H=32 D=64, "
                         "N(0,1), scale 1/8"),
    Workload("prefix_b1_nq4096_np1024_h32_d128", "prefix", 1, 4096, 32, 128, 3, Np=1024,
             description="Prefix-cached attention, Q [1,4096,32,128], K/V prefix "
                         "[1,1024,32,128], K/V current [1,4096,32,128], 5120 keys, "
                         "scale 1/sqrt(128)"),
    Workload("dense_b1024_n64_h32_d64", "dense", 1024, 64, 32, 64, 4,
             description="Many short sequences, B=1024 N=64 H=32 D=64, N(0,1)"),
    Workload("dense_b8_n1999_h32_d128_outliers", "dense", 8, 1999, 32, 128, 5,
             sigma_qk=3.0, outliers=4, outlier_factor=8.0,
             description="Ragged stress, B=8 N=1999 H=32 D=128, Q,K ~ N(0,3^2) with 4 "
                         "outlier channels per head (same in Q and K) scaled x8, V ~ N(0,1)"),
]

# Block-causal attention without prefix (the pages' "_prefix0" definition, 12 captured
# workloads whose shapes the pages do not print): a text prompt, two images and text
# around them; index 6 in the seeds.
WORKLOADS.append(
    Workload("block_causal_b1_n4096_h32_d128", "block_causal", 1, 4096, 32, 128, 6,
             segments=(("text", 128), ("image", 1920), ("text", 64), ("image", 1920),
                       ("text", 64)),
             description="Block-causal attention without prefix, B=1 N=4096 H=32 D=128: "
                         "text 128, image 1920, text 64, image 1920, text 64; N(0,1), "
                         "scale 1/sqrt(128)"))

# 3-D neighborhood attention (the pages' four na3d definitions, D = 64, scale 1 with the
# model's scale folded into Q; the pages print window sizes and head counts but no volume
# shapes): decoder-like volumes, Q ~ N(0, 1/64), K, V ~ N(0, 1); indices 7..10.
for _i, (_g, _h, _k) in enumerate((((8, 64, 64), 16, (3, 7, 7)), ((8, 32, 32), 32, (3, 7, 7)),
                                   ((16, 32, 32), 4, (11, 11, 11)), ((8, 64, 64), 8, (3, 5, 5)))):
    WORKLOADS.append(Workload(
        f"na3d_b1_t{_g[0]}_y{_g[1]}_x{_g[2]}_h{_h}_d64_k{_k[0]}x{_k[1]}x{_k[2]}", "na3d", 1, 0,
        _h, 64, 7 + _i, grid=_g, kernel=_k, sigma_qk=0.125,
        description=f"3-D neighborhood attention, B=1 T={_g[0]} Y={_g[1]} X={_g[2]} H={_h} "
                    f"D=64, window {_k[0]}x{_k[1]}x{_k[2]}, Q ~ N(0,1/64) (pre-scaled), "
                    f"K, V ~ N(0,1), scale 1"))

BY_NAME = {w.name: w for w in WORKLOADS}


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    return BY_NAME[name_or_index]


def small(kind: str, B: int, Nq: int, H: int, D: int, seed_base: int, Nk: Optional[int] = None,
          Np: int = 0, sigma_qk: float = 1.0, segments=()) -> Workload:
    """An ad-hoc seeded workload (tests); seed_base plays the role of the index k."""
    return Workload(f"{kind}_b{B}_nq{Nq}_h{H}_d{D}_s{seed_base}", kind, B, Nq, H, D,
                    seed_base, Nk=Nk or 0, Np=Np, sigma_qk=sigma_qk, segments=tuple(segments))
