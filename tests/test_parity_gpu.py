"""GPU parity: the HIP library through its C ABI against the FP64 oracle.

Small shapes compare every element. The workloads at full size compare every element
too, except the one whose oracle would take minutes (B=2 N=16384 H=32 D=64, 4.4e12
multiply-adds): there every wave of 32 query rows of every head contributes one
randomly chosen row (plus edge rows), so a mis-mapped workgroup or wave cannot go
unseen. Properties that hold at any size are checked on the whole output as well.
Every input is seeded (synth), identical bits feed both sides.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
import transformer_attention_dense_amd as attn
from acceptance import assert_accepted, bf16_bits_to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_ex(q, k0, v0, k1=None, v1=None, splits=0, waves=0):
    tq, tk0, tv0 = dev(q), dev(k0), dev(v0)
    tk1 = dev(k1) if k1 is not None else None
    tv1 = dev(v1) if v1 is not None else None
    out = attn.fwd_ex(tq, tk0, tv0, tk1, tv1, num_splits=splits, waves=waves)
    return host(out)


# ---------------------------------------------------------------- small, every element

DENSE_CASES = [
    # B, Nq, Nk, H, D
    (1, 1, 1, 1, 64), (1, 1, 1, 1, 128), (1, 2, 2, 1, 64), (1, 15, 15, 2, 128),
    (1, 63, 63, 2, 64), (1, 64, 64, 2, 128), (1, 65, 65, 2, 64), (3, 127, 127, 2, 128),
    (1, 129, 129, 3, 64), (2, 200, 200, 2, 128), (1, 257, 257, 1, 64), (1, 300, 577, 2, 128),
    (1, 96, 33, 4, 64), (2, 1, 700, 2, 128), (1, 700, 1, 2, 64),
]


@pytest.mark.parametrize("B,Nq,Nk,H,D", DENSE_CASES)
@pytest.mark.parametrize("splits,waves", [(0, 0), (1, 4), (1, 2), (3, 4), (7, 2), (1, 8), (3, 8)])
def test_dense_small_all_elements(B, Nq, Nk, H, D, splits, waves):
    say(f"dense B{B} Nq{Nq} Nk{Nk} H{H} D{D} splits{splits} waves{waves}")
    w = synth.small("dense", B, Nq, H, D, 300 + Nq + 3 * Nk, Nk=Nk, sigma_qk=2.0)
    q, k, v = w.tensors()
    got = run_ex(q, k, v, splits=splits, waves=waves)
    ref = oracle.attention(q, k, v)
    assert_accepted(got, ref, f"dense {w.name} s{splits} w{waves}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Np", [0, 1, 17, 64, 100])
@pytest.mark.parametrize("splits,waves", [(0, 0), (1, 0), (4, 0), (1, 8), (2, 8)])
def test_prefix_small_all_elements(Np, splits, waves, D):
    """Every element; with 8 waves at D = 64 the first 128-key tile holds both segments."""
    B, Nq, H = 2, 77, 3
    say(f"prefix Np{Np} D{D} splits{splits} waves{waves}")
    w = synth.small("prefix", B, Nq, H, D, 400 + Np, Np=Np, sigma_qk=2.0)
    q, kp, vp, kc, vc = w.tensors()
    ref = oracle.prefix_attention(q, kp, vp, kc, vc)
    if splits == 0 and waves == 0:
        out = attn.prefix(dev(q), dev(kp) if Np else torch.empty(B, 0, H, D, dtype=torch.bfloat16,
                                                                  device="cuda"),
                          dev(vp) if Np else torch.empty(B, 0, H, D, dtype=torch.bfloat16,
                                                         device="cuda"),
                          dev(kc), dev(vc))
        got = host(out)
    else:
        got = (run_ex(q, kp, vp, kc, vc, splits=splits, waves=waves) if Np
               else run_ex(q, kc, vc, splits=splits, waves=waves))
    assert_accepted(got, ref, f"prefix Np{Np} D{D}")


def test_cross_attention_unequal_lengths():
    B, Nq, Nk, H, D = 2, 100, 333, 4, 64
    w = synth.small("dense", B, Nq, H, D, 500, Nk=Nk, sigma_qk=2.0)
    q, k, v = w.tensors()
    got = host(attn.cross(dev(q), dev(k), dev(v)))
    assert_accepted(got, oracle.attention(q, k, v), "cross")


def test_outlier_logits_small():
    """Logit spread of hundreds (Q, K ~ N(0, 9) with aligned x8 channels): the running
    maximum jumps between tiles."""
    w = synth.Workload("t", "dense", 2, 333, 4, 128, 600, sigma_qk=3.0, outliers=4)
    q, k, v = w.tensors()
    ref = oracle.attention(q, k, v)
    for splits, waves in ((1, 0), (5, 0), (1, 8), (3, 8)):
        assert_accepted(run_ex(q, k, v, splits=splits, waves=waves), ref,
                        f"outliers s{splits} w{waves}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits,waves", [(1, 8), (1, 4), (2, 8)])
def test_logits_growing_along_the_keys(D, splits, waves):
    """Later keys carry logits far above the first tile's (the last 100 keys x6, then
    x12 on the last 20): the running reference of the first tile is no longer close
    enough, so the tiles are redone against their own maximum, and the rows that needed
    it stay on that path."""
    B, N, H = 1, 700, 3
    w = synth.small("dense", B, N, H, D, 650 + D, sigma_qk=1.0)
    q, k, v = w.tensors()
    kf = synth.bf16_bits_to_f32(k).copy()
    kf[:, -100:] *= 6.0
    kf[:, -20:] *= 2.0
    k = synth.f32_to_bf16_bits(kf)
    say(f"growing logits D{D} splits{splits} waves{waves}")
    assert_accepted(run_ex(q, k, v, splits=splits, waves=waves), oracle.attention(q, k, v),
                    f"growing logits D{D} s{splits} w{waves}")


# ---------------------------------------------------------------- short sequences

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,Nq,Nk,H", [(100, 50, 37, 32), (97, 64, 64, 32), (3, 1, 5, 7),
                                       (130, 33, 64, 24), (2, 64, 1, 3)])
def test_short_sequences_every_element(B, Nq, Nk, H, D):
    """At most 64 query rows and keys per (batch, head), many (batch, head) pairs: one
    key tile per two-wave workgroup (the one-tile kernel); ragged row and key counts,
    one wave idle when Nq <= 32."""
    plan = attn.attn_plan(B, Nq, Nk, H, D)
    assert plan["splits"] == 1 and plan["waves"] == 2
    say(f"short B{B} Nq{Nq} Nk{Nk} H{H}: {plan}")
    w = synth.small("dense", B, Nq, H, D, 1800 + Nq + Nk, Nk=Nk, sigma_qk=2.0)
    q, k, v = w.tensors()
    got = host(attn.cross(dev(q), dev(k), dev(v)) if Nq != Nk else attn.dense(dev(q), dev(k), dev(v)))
    assert_accepted(got, oracle.attention(q, k, v), f"short B{B} Nq{Nq} Nk{Nk} H{H}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nk,splits,waves", [(200, 64, 1, 4), (96, 50, 1, 4),
                                                (70, 256, 4, 2), (130, 250, 4, 4)])
def test_one_tile_key_ranges(Nq, Nk, splits, waves, D):
    """Calls whose key ranges are one 64-key tile each: short keys under four-wave
    workgroups, and keys split into 64-key ranges (partials merged by the combine
    kernel), the last range ragged."""
    B, H = 3, 5
    plan = attn.attn_plan(B, Nq, Nk, H, D, splits, waves)
    assert plan["waves"] == waves and plan["splits"] == splits
    assert -(-Nk // 64) <= splits  # one 64-key tile per key range
    w = synth.small("dense", B, Nq, H, D, 1870 + Nq + Nk, Nk=Nk, sigma_qk=2.0)
    q, k, v = w.tensors()
    say(f"one-tile ranges D{D} Nq{Nq} Nk{Nk} splits{splits} waves{waves}")
    assert_accepted(run_ex(q, k, v, splits=splits, waves=waves), oracle.attention(q, k, v),
                    f"one-tile D{D} Nq{Nq} Nk{Nk} s{splits} w{waves}")


def test_short_prefix_keys_from_both_segments():
    """Prefix-cached call whose prefix and current keys together fit in one short tile."""
    B, Nq, Np, H, D = 100, 40, 20, 32, 64
    w = synth.small("prefix", B, Nq, H, D, 1850, Np=Np, sigma_qk=2.0)
    q, kp, vp, kc, vc = w.tensors()
    got = host(attn.prefix(dev(q), dev(kp), dev(vp), dev(kc), dev(vc)))
    assert_accepted(got, oracle.prefix_attention(q, kp, vp, kc, vc), "short prefix")


# ---------------------------------------------------------------- block-causal, every element

def ids_from(segments):
    return synth.small("block_causal", 1, sum(n for _, n in segments), 1, 64, 0,
                       segments=segments).image_ids()


BC_CASES = [
    # B, N, H, D, image ids (name, array)
    (2, 100, 2, 128, "text_image_text_image",
     ids_from([("text", 10), ("image", 40), ("text", 5), ("image", 45)])),
    (1, 200, 3, 64, "all_text_causal", np.full(200, -1, np.int32)),
    (2, 130, 2, 128, "one_image_dense", np.zeros(130, np.int32)),
    (1, 1, 2, 128, "single_token", np.full(1, -1, np.int32)),
    (3, 33, 2, 64, "short_ragged", ids_from([("image", 20), ("text", 13)])),
    (1, 700, 2, 128, "image_across_workgroups",
     ids_from([("text", 50), ("image", 600), ("text", 50)])),
    (1, 600, 2, 128, "images_back_to_back",
     ids_from([("image", 200), ("image", 150), ("text", 3), ("image", 247)])),
    (1, 300, 2, 64, "large_and_negative_ids",
     np.array([-5] * 40 + [10 ** 6] * 100 + [-1] * 60 + [7] * 100, np.int32)),
    # more than 64 key tiles: the last row blocks classify their tiles in two chunks, the
    # second image crossing the chunk boundary at key 4096
    (1, 4700, 2, 128, "more_than_64_tiles",
     ids_from([("text", 100), ("image", 2100), ("text", 60), ("image", 2380), ("text", 60)])),
    (1, 4700, 1, 64, "more_than_64_tiles_d64",
     ids_from([("image", 3000), ("text", 40), ("image", 1600), ("text", 60)])),
]


@pytest.mark.parametrize("B,N,H,D,name,ids", BC_CASES, ids=[c[4] for c in BC_CASES])
def test_block_causal_small_all_elements(B, N, H, D, name, ids):
    say(f"block-causal {name} B{B} N{N} H{H} D{D}")
    w = synth.small("dense", B, N, H, D, 1100 + N, sigma_qk=2.0)
    q, k, v = w.tensors()
    ref = oracle.block_causal_attention(q, k, v, ids)
    got = host(attn.block_causal(dev(q), dev(k), dev(v), torch.from_numpy(ids).cuda()))
    assert_accepted(got, ref, f"block-causal {name}")


@pytest.mark.parametrize("seed", [0, 1])
def test_block_causal_arbitrary_ids(seed):
    """Ids that are not contiguous blocks (the same id in separate runs): the kernel
    evaluates the definition exactly, not a per-row key bound."""
    rng = np.random.default_rng(seed)
    B, N, H, D = 1, 333, 2, 128
    ids = rng.integers(-1, 5, size=N).astype(np.int32)
    w = synth.small("dense", B, N, H, D, 1200 + seed, sigma_qk=2.0)
    q, k, v = w.tensors()
    ref = oracle.block_causal_attention(q, k, v, ids)
    got = host(attn.block_causal(dev(q), dev(k), dev(v), torch.from_numpy(ids).cuda()))
    assert_accepted(got, ref, f"block-causal arbitrary ids {seed}")


def test_block_causal_extremes_match_other_calls():
    """All one image equals dense attention; the same GPU inputs through both calls."""
    B, N, H, D = 1, 512, 2, 128
    w = synth.small("dense", B, N, H, D, 1300, sigma_qk=2.0)
    tq, tk, tv = (dev(t) for t in w.tensors())
    a = host(attn.block_causal(tq, tk, tv, torch.zeros(N, dtype=torch.int32, device="cuda")))
    b = host(attn.dense(tq, tk, tv))
    # two GPU paths (different kernels and tile sizes) under the acceptance rule
    assert_accepted(a, bf16_bits_to_f64(b), "block-causal one image vs dense")


# ---------------------------------------------------------------- closed forms on the GPU

def test_identical_keys_give_mean_of_values():
    D = 128
    q = synth.normal_bf16((1, 130, 2, D), 701, 3.0)
    k = np.repeat(synth.normal_bf16((1, 1, 2, D), 702), 190, axis=1)
    v = synth.normal_bf16((1, 190, 2, D), 703)
    got = bf16_bits_to_f64(run_ex(q, k, v))
    mean = bf16_bits_to_f64(v).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(got, np.broadcast_to(mean, got.shape), atol=2e-3, rtol=1e-2)


def test_single_key_returns_its_value_row():
    q = synth.normal_bf16((2, 70, 3, 64), 711, 3.0)
    k = synth.normal_bf16((2, 1, 3, 64), 712)
    v = synth.normal_bf16((2, 1, 3, 64), 713)
    got = run_ex(q, k, v)
    assert np.array_equal(got, np.broadcast_to(v, got.shape))


def test_prefix_equals_dense_on_concatenation():
    B, Nq, Np, H, D = 1, 200, 70, 2, 128
    w = synth.small("prefix", B, Nq, H, D, 720, Np=Np)
    q, kp, vp, kc, vc = w.tensors()
    a = run_ex(q, kp, vp, kc, vc, splits=1)
    b = run_ex(q, np.concatenate([kp, kc], 1), np.concatenate([vp, vc], 1), splits=1)
    # same keys in the same order and tiles aligned differently: equal up to rounding
    np.testing.assert_allclose(bf16_bits_to_f64(a), bf16_bits_to_f64(b), atol=4e-3, rtol=1e-2)


def test_deterministic_and_inputs_untouched_and_no_out_of_bounds_writes():
    B, N, H, D = 1, 333, 3, 128
    w = synth.small("dense", B, N, H, D, 730, sigma_qk=2.0)
    q, k, v = w.tensors()
    tq, tk, tv = dev(q), dev(k), dev(v)
    numel = B * N * H * D
    guard = 4096
    buf = torch.full((numel + 2 * guard,), -7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[guard:guard + numel].view(B, N, H, D)
    attn.fwd_ex(tq, tk, tv, out=out, num_splits=3)
    first = host(out).copy()
    attn.fwd_ex(tq, tk, tv, out=out, num_splits=3)
    assert np.array_equal(first, host(out))
    canary = host(buf)
    assert np.all(bf16_bits_to_f64(canary[:guard]) == -7.0)
    assert np.all(bf16_bits_to_f64(canary[guard + numel:]) == -7.0)
    assert np.array_equal(host(tq), q) and np.array_equal(host(tk), k) and np.array_equal(
        host(tv), v)


def test_invalid_call_leaves_output_untouched():
    x = dev(synth.normal_bf16((1, 8, 1, 64), 740))
    out = torch.full_like(x, 3.0)
    with pytest.raises(attn.AttnError):
        attn.fwd_ex(x, x, x, out=out, waves=3)
    assert torch.all(out == 3.0)


# ---------------------------------------------------------------- the workloads, full size

# Oracle work (multiply-adds x 2) up to which a full-size workload is compared on every
# element: the FP64 oracle runs ~3.5e10 of them per second on 16 host cores, so the
# largest such workload (B=8 N=1999 H=32 D=128, 5.2e11) takes ~15 s.
FULL_CHECK_FLOP = 1.2e12


def rows_per_wave(w, seed):
    """One random query row from every block of 32 consecutive rows of every (b, h) (a
    wave's rows in every kernel), plus the first, middle and last rows of each batch for
    every head."""
    rng = np.random.default_rng(seed)
    blocks = -(-w.Nq // 32)
    rows = set()
    for b in range(w.B):
        for h in range(w.H):
            i = np.minimum(np.arange(blocks) * 32 + rng.integers(0, 32, size=blocks), w.Nq - 1)
            rows.update(((b * w.Nq + i) * w.H + h).tolist())
            for e in (0, w.Nq // 2, w.Nq - 1):
                rows.add((b * w.Nq + e) * w.H + h)
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("idx", range(len(synth.WORKLOADS)))
def test_workload_full_size(idx):
    w = synth.WORKLOADS[idx]
    say(f"workload {w.name}: generating inputs")
    ts = w.tensors()
    say(f"workload {w.name}: GPU call")
    if w.kind == "na3d":
        check_na3d_full_size(w, ts, idx)
        return
    if w.kind == "block_causal":
        dts = [dev(t) for t in ts[:3]] + [torch.from_numpy(ts[3]).cuda()]
        out = attn.block_causal(*dts)
    else:
        dts = [dev(t) for t in ts]
    if w.kind == "dense":
        out = attn.dense(*dts) if w.Nk == w.Nq else attn.cross(*dts)
    elif w.kind == "prefix":
        out = attn.prefix(*dts)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    # convex combination: every output lies within the per-(b, h, d) range of V
    vs = [dts[2]] if w.kind != "prefix" else [dts[2], dts[4]]
    vmin = torch.stack([x.float().amin(dim=1) for x in vs]).amin(0)
    vmax = torch.stack([x.float().amax(dim=1) for x in vs]).amax(0)
    o = out.float()
    assert bool((o >= vmin[:, None] - 1e-2).all()) and bool((o <= vmax[:, None] + 1e-2).all())
    got = host(out).reshape(-1, w.D)
    rows = None if w.flop <= FULL_CHECK_FLOP else rows_per_wave(w, 800 + idx)
    say(f"workload {w.name}: oracle, "
        f"{'every row' if rows is None else f'{rows.size} rows (one per wave)'}")
    if w.kind == "block_causal":
        ref = oracle.block_causal_rows(ts[0], ts[1], ts[2], ts[3], rows=rows)
    else:
        ref = oracle.attention_rows(ts[0], ts[1], ts[2], *ts[3:5], rows=rows)
    sel = got if rows is None else got[rows]
    res = assert_accepted(sel, ref, w.name)
    say(f"workload {w.name}: {res}")


def check_na3d_full_size(w, ts, idx):
    dts = [dev(t) for t in ts]
    out = attn.na3d(*dts, w.kernel)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    # convex combination of values: within the per-(b, h, d) range of V over the volume
    vf = dts[2].float().flatten(1, 3)
    vmin, vmax = vf.amin(dim=1), vf.amax(dim=1)
    o = out.float().flatten(1, 3)
    assert bool((o >= vmin[:, None] - 1e-2).all()) and bool((o <= vmax[:, None] + 1e-2).all())
    got = host(out).reshape(-1, w.D)
    assert w.flop <= FULL_CHECK_FLOP
    say(f"workload {w.name}: oracle, every row")
    ref = oracle.na3d_rows(ts[0], ts[1], ts[2], w.kernel)
    res = assert_accepted(got, ref, w.name)
    say(f"workload {w.name}: {res}")


# ---------------------------------------------------------------- 3-D neighborhood attention

NA_CASES = [
    # (B, T, Y, X, H, (kt, ky, kx)); the wave tile the library picks (rows y x positions
    # on X) and the workgroup's arrangement (frames x row tiles) in brackets
    (1, 3, 5, 7, 4, (3, 3, 5)),      # [4x8 4x1] one strip; windows moved inside at every border
    (2, 4, 6, 40, 3, (3, 5, 7)),     # [4x8 1x4] five strips; two idle waves
    (1, 7, 19, 24, 2, (3, 7, 5)),    # [4x8 2x2] the last frame pair's second frame past T
    (1, 6, 33, 21, 2, (3, 9, 9)),    # [4x8 2x2] a row tile of one row; a one-query strip
    (1, 5, 9, 33, 5, (5, 7, 11)),    # [8x4 4x1] a one-query strip; a block past the Y axis
    (1, 2, 3, 64, 8, (1, 3, 1)),     # [4x8 1x4] windows of one position on T and X
    (1, 1, 2, 35, 2, (1, 1, 17)),    # [2x16 4x1] the widest X window; three frames past T
    (1, 3, 11, 19, 3, (3, 9, 17)),   # [2x16 4x1] widest X window, wave rows split by Y windows
    (1, 2, 21, 24, 2, (1, 5, 13)),   # [2x16 4x1] eleven row tiles, most of them interior
    (1, 3, 37, 30, 2, (3, 9, 11)),   # [8x4 4x1] ragged row tiles and strips
    (1, 2, 9, 20, 3, (1, 3, 5)),     # [4x8 1x4] the last key block's second row past the Y axis
    (1, 3, 3, 3, 4, (3, 3, 3)),      # [4x8 4x1] the window covers the volume
    (1, 2, 4, 97, 4, (1, 3, 9)),     # [4x8 1x4] 13 strips, the last one query wide
    # 8x4 query tiles over key blocks of four rows of 8 positions (kx <= 5); the last
    # block of a frame reaches rows past the Y axis
    (1, 3, 13, 22, 2, (3, 5, 5)),    # [8x4] ragged rows and strips
    (2, 2, 19, 9, 3, (1, 7, 3)),     # [8x4] two batches, a one-query strip
    (1, 4, 10, 30, 2, (3, 9, 5)),    # [8x4] the Y window nearly the axis
    (1, 5, 7, 5, 2, (5, 5, 5)),      # [8x4] the X window covers the axis
]


@pytest.mark.parametrize("case", NA_CASES, ids=[f"{c[:5]}-{c[5]}" for c in NA_CASES])
def test_na3d_small_all_elements(case):
    B, T, Y, X, H, kernel = case
    shape = (B, T, Y, X, H, 64)
    say(f"na3d {case}")
    seed = 1500 + 7 * sum(shape) + sum(kernel)
    q = synth.normal_bf16(shape, seed, 0.5)
    k = synth.normal_bf16(shape, seed + 1, 1.0)
    v = synth.normal_bf16(shape, seed + 2, 1.0)
    out = attn.na3d(dev(q), dev(k), dev(v), kernel)
    ref = oracle.na3d_attention(q, k, v, kernel)
    assert_accepted(host(out).reshape(-1, 64), ref.reshape(-1, 64), f"na3d {case}")


def test_na3d_large_logits_rescale_across_blocks():
    """Logits with a spread of hundreds (Q scaled by 6, K by 2: score sd about 96) raise
    the running maximum many times over a query's blocks; two batches, the 2x2 workgroup
    arrangement."""
    shape = (2, 4, 13, 22, 2, 64)
    kernel = (3, 7, 5)
    say(f"na3d large logits {shape} {kernel}")
    q = synth.normal_bf16(shape, 1700, 6.0)
    k = synth.normal_bf16(shape, 1701, 2.0)
    v = synth.normal_bf16(shape, 1702, 1.0)
    out = attn.na3d(dev(q), dev(k), dev(v), kernel)
    ref = oracle.na3d_attention(q, k, v, kernel)
    assert_accepted(host(out).reshape(-1, 64), ref.reshape(-1, 64), "na3d large logits")


def test_na3d_writes_only_its_output():
    shape = (1, 2, 3, 40, 4, 64)
    q, k, v = (dev(synth.normal_bf16(shape, 1600 + i, 1.0)) for i in range(3))
    big = torch.full((3 * q.numel(),), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[q.numel():2 * q.numel()].view(shape)
    attn.na3d(q, k, v, (1, 3, 5), out=out)
    torch.cuda.synchronize()
    assert bool((big[:q.numel()] == 7.0).all()) and bool((big[2 * q.numel():] == 7.0).all())


# ---------------------------------------------------------------- tensors of 2^31 elements

def need_free_gib(gib):
    free = torch.cuda.mem_get_info()[0]
    if free < gib * 2**30:
        pytest.skip(f"needs {gib} GiB of free device memory, {free / 2**30:.1f} GiB free")


def batched_copies(one_shape, B, seeds_first, seeds_last, sigmas):
    """Three device tensors of B batches: batch 0 and batch B - 1 from seeded inputs of
    their own, the batches between copies of batch 0. Also returns the host bits of the
    first and the last batch."""
    first = [synth.normal_bf16(one_shape, s, sg) for s, sg in zip(seeds_first, sigmas)]
    last = [synth.normal_bf16(one_shape, s, sg) for s, sg in zip(seeds_last, sigmas)]
    full = (B,) + tuple(one_shape[1:])
    ts = []
    for f, l in zip(first, last):
        t = torch.empty(full, dtype=torch.bfloat16, device="cuda")
        t[:-1].copy_(dev(f).expand((B - 1,) + tuple(one_shape[1:])))
        t[-1:].copy_(dev(l))
        ts.append(t)
    return ts, first, last


def middle_batches_match_first(out):
    bits = out.view(torch.int16)
    return bool((bits[1:-1] == bits[:1]).all())


def test_dense_tensors_of_2_pow_31_elements():
    """B=128 N=4096 H=32 D=128: 2^31 elements (4 GiB) per tensor, so offsets past one
    batch need 64 bits. Sampled rows of the first and the last batch (inputs of their
    own) against the oracle; the batches between (copies of the first) bit-identical to
    it."""
    B, N, H, D = 128, 4096, 32, 128
    need_free_gib(24)
    say(f"dense B{B} N{N} H{H} D{D}: 2^31 elements per tensor")
    (q, k, v), first, last = batched_copies((1, N, H, D), B, (1800, 1801, 1802),
                                            (1810, 1811, 1812), (1.0, 1.0, 1.0))
    out = attn.dense(q, k, v)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1820).choice(N * H, 512, replace=False))
    for b, src in ((0, first), (B - 1, last)):
        got = host(out[b]).reshape(-1, D)[rows]
        ref = oracle.attention_rows(*src, rows=rows)
        say(f"dense 2^31 batch {b}: {assert_accepted(got, ref, f'dense 2^31 batch {b}')}")
    assert middle_batches_match_first(out)


def test_prefix_tensors_of_2_pow_31_elements():
    """Prefix attention, B=128 Nq=4096 Np=1024 H=32 D=128: Q, the current keys and values
    and the output hold 2^31 elements each, the cached ones 2^29; checked as the dense
    case above."""
    B, Nq, Np, H, D = 128, 4096, 1024, 32, 128
    need_free_gib(28)
    say(f"prefix B{B} Nq{Nq} Np{Np} H{H} D{D}: 2^31 elements per current tensor")
    (q, kc, vc), first, last = batched_copies((1, Nq, H, D), B, (1860, 1861, 1862),
                                              (1870, 1871, 1872), (1.0, 1.0, 1.0))
    (kp, vp), pfirst, plast = batched_copies((1, Np, H, D), B, (1863, 1864), (1873, 1874),
                                             (1.0, 1.0))
    out = attn.prefix(q, kp, vp, kc, vc)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1880).choice(Nq * H, 512, replace=False))
    for b, cur, pre in ((0, first, pfirst), (B - 1, last, plast)):
        got = host(out[b]).reshape(-1, D)[rows]
        ref = oracle.attention_rows(cur[0], pre[0], pre[1], cur[1], cur[2], rows=rows)
        say(f"prefix 2^31 batch {b}: {assert_accepted(got, ref, f'prefix 2^31 batch {b}')}")
    assert middle_batches_match_first(out)


def test_block_causal_tensors_of_2_pow_31_elements():
    """Block-causal attention, B=128 N=4096 H=32 D=128 with the image ids of the
    block-causal workload (shared by the batch): 2^31 elements per tensor; checked as
    the dense case above."""
    B, N, H, D = 128, 4096, 32, 128
    need_free_gib(24)
    say(f"block-causal B{B} N{N} H{H} D{D}: 2^31 elements per tensor")
    ids = synth.workload("block_causal_b1_n4096_h32_d128").image_ids()
    (q, k, v), first, last = batched_copies((1, N, H, D), B, (1890, 1891, 1892),
                                            (1895, 1896, 1897), (1.0, 1.0, 1.0))
    out = attn.block_causal(q, k, v, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1899).choice(N * H, 512, replace=False))
    for b, src in ((0, first), (B - 1, last)):
        got = host(out[b]).reshape(-1, D)[rows]
        ref = oracle.block_causal_rows(*src, ids, rows=rows)
        say(f"block-causal 2^31 batch {b}: "
            f"{assert_accepted(got, ref, f'block-causal 2^31 batch {b}')}")
    assert middle_batches_match_first(out)


def test_na3d_tensors_of_2_pow_31_elements():
    """B=64 T=8 Y=64 X=64 H=16 D=64, window 3x7x7: 2^31 elements per tensor, checked as
    the dense case above."""
    B, T, Y, X, H, D = 64, 8, 64, 64, 16, 64
    kernel = (3, 7, 7)
    need_free_gib(24)
    say(f"na3d B{B} T{T} Y{Y} X{X} H{H} D{D} {kernel}: 2^31 elements per tensor")
    (q, k, v), first, last = batched_copies((1, T, Y, X, H, D), B, (1830, 1831, 1832),
                                            (1840, 1841, 1842), (0.125, 1.0, 1.0))
    out = attn.na3d(q, k, v, kernel)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1850).choice(T * Y * X * H, 512, replace=False))
    for b, src in ((0, first), (B - 1, last)):
        got = host(out[b]).reshape(-1, D)[rows]
        ref = oracle.na3d_rows(*src, kernel, rows=rows)
        say(f"na3d 2^31 batch {b}: {assert_accepted(got, ref, f'na3d 2^31 batch {b}')}")
    assert middle_batches_match_first(out)


# ---------------------------------------------------------------- streams

def test_calls_run_on_the_current_stream():
    """The tensor helpers enqueue on the caller's current stream (here a side stream of
    default priority): the handle they pass is that stream's, and the result equals the
    same call on the default stream bit for bit."""
    say("current-stream case: dense B=1 N=130 H=2 D=64 on a side stream")
    w = synth.small("dense", 1, 130, 2, 64, 905)
    q, k, v = (dev(t) for t in w.tensors())
    ref = host(attn.dense(q, k, v))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert attn._stream(q) == side.cuda_stream
        out = attn.dense(q, k, v)
    side.synchronize()
    assert np.array_equal(host(out), ref)


# ---------------------------------------------------------------- HIP graph capture

def test_graph_capture_replays_match_eager():
    """Calls captured in a HIP graph (through torch's capture of the current stream)
    replay to the eager bits, for a one-split call, a split-KV call (work space reserved
    by an earlier uncaptured call) and a block-causal call. Eager work on the same
    stream runs between replays."""
    B, N, H, D = 1, 640, 4, 128
    w = synth.small("dense", B, N, H, D, 1400, sigma_qk=2.0)
    tq, tk, tv = (dev(t) for t in w.tensors())
    ids = torch.from_numpy(ids_from([("text", 40), ("image", 500), ("text", 100)])).cuda()
    calls = {
        "dense": lambda out: attn.fwd_ex(tq, tk, tv, out=out, num_splits=1),
        "split_kv": lambda out: attn.fwd_ex(tq, tk, tv, out=out, num_splits=4),
        "block_causal": lambda out: attn.block_causal(tq, tk, tv, ids, out=out),
    }
    scratch = torch.ones(1 << 20, device="cuda")
    for name, call in calls.items():
        say(f"graph capture {name}")
        eager = torch.empty_like(tq)
        call(eager)  # also reserves any work space outside the capture
        ref = host(eager).copy()
        static_out = torch.zeros_like(tq)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(static_out)
        for r in range(3):
            static_out.zero_()
            g.replay()
            scratch.mul_(1.0001)  # unrelated eager work between replays
            assert np.array_equal(host(static_out), ref), f"{name}: replay {r} differs"


# ---------------------------------------------------------------- work space

def test_work_space_allocation_failure_leaves_output_untouched(monkeypatch):
    """With allocation failing (fault injection), a split-KV call that needs a larger
    work space than any call before it returns ATTN_ERR_WORKSPACE and writes nothing."""
    attn.set_workspace(None)
    B, Nq, Nk, H, D, splits = 1, 1024, 16384, 4, 128, 256
    need = attn.attn_plan(B, Nq, Nk, H, D, num_splits=splits)["workspace_bytes"]
    assert need > 512 << 20  # more than any other call of this suite reserves
    say(f"work-space failure case: B{B} Nq{Nq} Nk{Nk} H{H} D{D} splits{splits}, {need} bytes")
    q = dev(synth.normal_bf16((B, Nq, H, D), 760))
    kv = dev(synth.normal_bf16((B, Nk, H, D), 761))
    out = torch.full_like(q, 5.0)
    monkeypatch.setenv("ATTN_TEST_FAIL_ALLOC", "1")
    with pytest.raises(attn.AttnError) as e:
        attn.fwd_ex(q, kv, kv, out=out, num_splits=splits)
    assert e.value.code == -7
    assert attn.attn_reserve_workspace(need) == -7
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
    monkeypatch.delenv("ATTN_TEST_FAIL_ALLOC")


def test_caller_work_space_used_and_checked():
    """attn_set_workspace: a split-KV call runs in the caller's buffer (same bits as in
    the library's), a too small buffer gives ATTN_ERR_WORKSPACE, one overlapping the
    call's tensors ATTN_ERR_ALIAS, and None reverts to the library's buffer."""
    B, N, H, D = 1, 300, 2, 128
    w = synth.small("dense", B, N, H, D, 770, sigma_qk=2.0)
    tq, tk, tv = (dev(t) for t in w.tensors())
    need = attn.attn_plan(B, N, N, H, D, num_splits=3)["workspace_bytes"]
    ref = host(attn.fwd_ex(tq, tk, tv, num_splits=3)).copy()
    buf = torch.empty(need, dtype=torch.uint8, device="cuda")
    try:
        attn.set_workspace(buf)
        assert np.array_equal(host(attn.fwd_ex(tq, tk, tv, num_splits=3)), ref)
        attn.set_workspace(buf[:need - 256])
        with pytest.raises(attn.AttnError) as e:
            attn.fwd_ex(tq, tk, tv, num_splits=3)
        assert e.value.code == -7
        # an output that starts 256 bytes before the end of the work space the call uses
        big = torch.empty(need + tq.numel() * 2 + 4096, dtype=torch.uint8, device="cuda")
        off = (need // 256) * 256 - 256
        outv = big[off:off + tq.numel() * 2].view(torch.bfloat16).view(tq.shape)
        attn.set_workspace(big)
        with pytest.raises(attn.AttnError) as e:
            attn.fwd_ex(tq, tk, tv, out=outv, num_splits=3)
        assert e.value.code == -5
        with pytest.raises(attn.AttnError) as e:
            attn.set_workspace(buf[1:])
        assert e.value.code == -4
    finally:
        attn.set_workspace(None)
    assert np.array_equal(host(attn.fwd_ex(tq, tk, tv, num_splits=3)), ref)


def test_graph_capture_with_caller_work_space():
    """A split-KV call captured in a HIP graph with a caller-supplied work space (no
    allocation inside the capture) replays to the eager bits, with eager work between
    the replays; block-causal summaries in the caller's buffer likewise."""
    B, N, H, D = 1, 520, 3, 64
    w = synth.small("dense", B, N, H, D, 780, sigma_qk=2.0)
    tq, tk, tv = (dev(t) for t in w.tensors())
    ids = torch.from_numpy(ids_from([("text", 20), ("image", 400), ("text", 100)])).cuda()
    need = attn.attn_plan(B, N, N, H, D, num_splits=5)["workspace_bytes"]
    buf = torch.empty(need, dtype=torch.uint8, device="cuda")
    calls = {"split_kv": lambda out: attn.fwd_ex(tq, tk, tv, out=out, num_splits=5),
             "block_causal": lambda out: attn.block_causal(tq, tk, tv, ids, out=out)}
    other = torch.ones(1 << 20, device="cuda")
    try:
        attn.set_workspace(buf)
        for name, call in calls.items():
            say(f"graph capture with caller work space: {name}")
            eager = torch.empty_like(tq)
            call(eager)
            ref = host(eager).copy()
            static_out = torch.zeros_like(tq)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call(static_out)
            for r in range(3):
                static_out.zero_()
                g.replay()
                other.mul_(1.0001)
                assert np.array_equal(host(static_out), ref), f"{name}: replay {r} differs"
    finally:
        attn.set_workspace(None)


# ---------------------------------------------------------------- launch plans at the GPU's size

@pytest.mark.parametrize("B,N,H,D", [(1, 2048, 32, 128), (2, 1024, 32, 64)])
def test_grids_of_one_workgroup_per_cu_do_not_split(B, N, H, D):
    """256 blocks of 256 query rows fill the GPU's 256 CUs with the 8-wave kernel (one
    workgroup per CU): one key range, no combine step, and every element correct."""
    plan = attn.attn_plan(B, N, N, H, D)
    assert plan == {"splits": 1, "waves": 8, "workgroups": 256, "workspace_bytes": 0}
    say(f"256-workgroup plan: B{B} N{N} H{H} D{D}")
    w = synth.small("dense", B, N, H, D, 790 + D)
    q, k, v = w.tensors()
    got = host(attn.dense(dev(q), dev(k), dev(v)))
    assert_accepted(got, oracle.attention(q, k, v), f"256 workgroups B{B} N{N} D{D}")


# ---------------------------------------------------------------- nonfinite inputs

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits,waves", [(1, 0), (3, 4), (1, 8)])
def test_nonfinite_inputs_propagate_like_the_definition(D, splits, waves):
    """NaN and infinity are not special-cased: the nonfinite outputs are exactly the
    elements the definition (the FP64 oracle) makes nonfinite, and every other element
    passes the acceptance rule. A NaN in a key row poisons every row of its head; +inf
    in one key dimension makes the rows whose query has a positive entry there NaN
    (the score is +inf, and inf - inf appears in the softmax), while rows with a
    negative entry give that key weight 0; a NaN in a query row poisons that row only;
    an inf in a value row makes that dimension infinite for every row of its head."""
    B, N, H = 1, 150, 4
    w = synth.small("dense", B, N, H, D, 795 + D, sigma_qk=1.0)
    q, k, v = (t.copy() for t in w.tensors())
    nan, pinf = np.uint16(0x7FC0), np.uint16(0x7F80)
    k[0, 37, 0, 5] = nan          # head 0: every row NaN
    k[0, 91, 1, 3] = pinf         # head 1: rows with q[., 3] > 0 NaN, < 0 unaffected
    q[0, 10, 2, :] = 0
    q[0, 10, 2, 7] = nan          # head 2: row 10 only
    v[0, 120, 3, 9] = pinf        # head 3: dimension 9 infinite in every row
    say(f"nonfinite case D{D} splits{splits} waves{waves}")
    ref = oracle.attention(q, k, v)
    got = bf16_bits_to_f64(run_ex(q, k, v, splits=splits, waves=waves))
    bad_ref, bad_got = ~np.isfinite(ref), ~np.isfinite(got)
    assert bad_ref[0, :, 0].all() and not bad_ref[0, :, 2][np.arange(N) != 10].any()
    assert bad_ref[0, :, 3, 9].all() and 0 < bad_ref[0, :, 1].all(axis=-1).sum() < N
    assert np.array_equal(bad_got, bad_ref), (
        f"{int((bad_got != bad_ref).sum())} elements differ in finiteness")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~bad_ref
    assert_accepted(got[fin], ref[fin], f"nonfinite case D{D}, finite elements")
