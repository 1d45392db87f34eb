"""Pins for the FP64 oracle, run on the CPU.

Each check ties the oracle to something other than itself: the pages' printed
contract constants (tests/golden/contracts.json), closed forms of softmax
attention, invariants of the definition, brute force with explicit index formulas,
and an independent numpy evaluation. Together they are chosen so that a plausible
slip in the oracle (wrong or missing scale, wrong sign in the exponent, a
transposed operand or wrong stride, a missing normalisation, prefix and current
segments mixed up) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import attn_np
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "contracts.json")


def bits(x):
    """BF16 bits of values that are exactly representable (small integers, halves...)."""
    x = np.asarray(x, dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert np.array_equal(synth.bf16_bits_to_f32(b), x), "test value not exact in BF16"
    return b


def rand_bits(shape, seed, sigma=1.0):
    return synth.normal_bf16(shape, seed, sigma)


# ---------------------------------------------------------------- contract constants

def test_scale_matches_pages_printed_constants():
    """The pages print 128 ** -0.5 and 64 ** -0.5 as the fixed scales. A two-key
    problem with logits 0 and c*scale has the closed form sigmoid(c*scale)."""
    g = json.load(open(GOLDEN))
    for name in ("noncausal_dense_attention_h32_d128", "noncausal_dense_attention_h32_d64"):
        op = g["operators"][name]
        D = op["D"]
        assert op["scale"] == D ** -0.5
        q = np.zeros((1, 1, 1, D), np.float32)
        q[0, 0, 0, 0] = 16.0
        k = np.zeros((1, 2, 1, D), np.float32)
        k[0, 1, 0, 0] = 1.0
        v = np.zeros((1, 2, 1, D), np.float32)
        v[0, 0, 0, 0] = 1.0
        v[0, 1, 0, 1] = 1.0
        out = oracle.attention(bits(q), bits(k), bits(v))[0, 0, 0]
        s1 = 16.0 * op["scale"]
        p1 = 1.0 / (1.0 + math.exp(-s1))
        assert out[0] == pytest.approx(1.0 - p1, rel=1e-14)
        assert out[1] == pytest.approx(p1, rel=1e-14)
        assert np.all(out[2:] == 0.0)


def test_prefix_operand_order_matches_pages():
    """Keys are (K_prefix then K_current) and values (V_prefix then V_current): a query
    that matches only the prefix key must return the prefix value."""
    g = json.load(open(GOLDEN))
    op = g["operators"]["prefix_cached_block_causal_h32_d128"]
    assert op["inputs"] == ["Q", "K_prefix", "V_prefix", "K_current", "V_current"]
    D = op["D"]
    q = np.zeros((1, 1, 1, D), np.float32)
    q[0, 0, 0, 0] = 64.0
    kp = np.zeros((1, 1, 1, D), np.float32)
    kp[0, 0, 0, 0] = 64.0          # logit 64*64/sqrt(128) ~ 362 -> dominant
    kc = np.zeros((1, 1, 1, D), np.float32)
    vp = np.full((1, 1, 1, D), 3.0, np.float32)
    vc = np.full((1, 1, 1, D), -5.0, np.float32)
    out = oracle.prefix_attention(bits(q), bits(kp), bits(vp), bits(kc), bits(vc))
    assert np.all(out == 3.0)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("D", [64, 128])
def test_identical_keys_give_mean_of_values(D):
    rng = np.random.default_rng(1)
    q = rand_bits((1, 5, 2, D), 11)
    krow = rand_bits((1, 1, 2, D), 12)
    k = np.repeat(krow, 7, axis=1)
    v = rand_bits((1, 7, 2, D), 13)
    out = oracle.attention(q, k, v)
    mean_v = attn_np.bf16_bits_to_f64(v).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(mean_v, out.shape), rtol=1e-13, atol=1e-15)
    del rng


def test_zero_query_gives_mean_of_values():
    q = np.zeros((2, 3, 2, 64), np.uint16)
    k = rand_bits((2, 9, 2, 64), 21, 3.0)
    v = rand_bits((2, 9, 2, 64), 22)
    out = oracle.attention(q, k, v)
    mean_v = attn_np.bf16_bits_to_f64(v).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(mean_v, out.shape), rtol=1e-13, atol=1e-15)


def test_single_key_returns_its_value_exactly():
    q = rand_bits((2, 4, 3, 128), 31, 5.0)
    k = rand_bits((2, 1, 3, 128), 32, 5.0)
    v = rand_bits((2, 1, 3, 128), 33)
    out = oracle.attention(q, k, v)
    np.testing.assert_array_equal(out, np.broadcast_to(attn_np.bf16_bits_to_f64(v), out.shape))


def test_dominant_logit_returns_that_value():
    """One key aligned with the query with a scaled-logit gap >= 40 over the rest:
    the output is that key's value row within N * e^-40."""
    D, N = 64, 50
    rng = np.random.default_rng(4)
    q = np.zeros((1, 1, 1, D), np.float32)
    q[0, 0, 0, :4] = 8.0
    k = rng.integers(-1, 2, size=(1, N, 1, D)).astype(np.float32)
    k[0, :, 0, :4] = 0.0
    star = 17
    k[0, star, 0, :4] = 16.0     # logit 4*8*16/8 = 64; others 0
    v = rng.integers(-4, 5, size=(1, N, 1, D)).astype(np.float32)
    out = oracle.attention(bits(q), bits(k), bits(v))[0, 0, 0]
    assert np.max(np.abs(out - v[0, star, 0])) <= N * math.exp(-40) * 8


def test_constant_values_give_that_constant():
    q = rand_bits((1, 6, 2, 128), 41, 4.0)
    k = rand_bits((1, 11, 2, 128), 42, 4.0)
    v = np.full((1, 11, 2, 128), synth.f32_to_bf16_bits(np.float32(-2.5)), np.uint16)
    out = oracle.attention(q, k, v)
    np.testing.assert_allclose(out, -2.5, rtol=1e-13)


def test_probabilities_sum_to_one_and_lse_is_logsumexp():
    w = synth.small("dense", 1, 7, 3, 64, 50, Nk=13, sigma_qk=3.0)
    q, k, v = w.tensors()
    out, lse, psum = oracle.attention_rows(q, k, v, want_lse=True, want_psum=True)
    np.testing.assert_allclose(psum, 1.0, rtol=0, atol=1e-13)
    qf, kf = attn_np.bf16_bits_to_f64(q), attn_np.bf16_bits_to_f64(k)
    s = np.einsum("bqhd,bkhd->bqhk", qf, kf) * 0.125
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1).reshape(-1), rtol=1e-13)


# ---------------------------------------------------------------- brute force

def _brute_force(q, k, v):
    """Explicit loops with the [B, N, H, D] index formula written out, for tiny inputs."""
    qf, kf, vf = (attn_np.bf16_bits_to_f64(x).reshape(-1) for x in (q, k, v))
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    scale = D ** -0.5
    out = np.zeros(q.shape)
    for b in range(B):
        for i in range(Nq):
            for h in range(H):
                logits = []
                for j in range(Nk):
                    acc = 0.0
                    for d in range(D):
                        acc += qf[((b * Nq + i) * H + h) * D + d] * kf[((b * Nk + j) * H + h) * D + d]
                    logits.append(acc * scale)
                m = max(logits)
                e = [math.exp(x - m) for x in logits]
                tot = sum(e)
                for d in range(D):
                    out[b, i, h, d] = sum(e[j] / tot * vf[((b * Nk + j) * H + h) * D + d]
                                          for j in range(Nk))
    return out


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 64), (2, 3, 2, 4, 64), (1, 2, 3, 5, 128)])
def test_brute_force_tiny(shape):
    B, Nq, H, Nk, D = shape
    w = synth.small("dense", B, Nq, H, D, 60 + Nk, Nk=Nk, sigma_qk=2.0)
    q, k, v = w.tensors()
    np.testing.assert_allclose(oracle.attention(q, k, v), _brute_force(q, k, v), rtol=1e-12,
                               atol=1e-14)


# ---------------------------------------------------------------- independent numpy form

@pytest.mark.parametrize("B,Nq,Nk,H,D", [(1, 1, 1, 1, 64), (2, 7, 3, 2, 64), (1, 65, 130, 3, 128),
                                          (2, 64, 64, 32, 64), (1, 33, 17, 2, 128)])
def test_c_oracle_matches_numpy_form(B, Nq, Nk, H, D):
    w = synth.small("dense", B, Nq, H, D, 70 + Nq, Nk=Nk, sigma_qk=2.0)
    q, k, v = w.tensors()
    np.testing.assert_allclose(oracle.attention(q, k, v), attn_np.attention(q, k, v),
                               rtol=1e-12, atol=1e-14)


def test_c_oracle_matches_numpy_form_large_logits():
    """Logit spread of hundreds: a wrong max subtraction overflows or loses the answer."""
    w = synth.Workload("t", "dense", 1, 9, 2, 128, 80, Nk=21, sigma_qk=3.0, outliers=4)
    q, k, v = w.tensors()
    ref = attn_np.attention(q, k, v)
    out = oracle.attention(q, k, v)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("Np", [1, 5, 17])
def test_prefix_matches_numpy_concatenation(Np):
    w = synth.small("prefix", 2, 9, 2, 128, 90 + Np, Np=Np, sigma_qk=2.0)
    q, kp, vp, kc, vc = w.tensors()
    np.testing.assert_allclose(oracle.prefix_attention(q, kp, vp, kc, vc),
                               attn_np.prefix_attention(q, kp, vp, kc, vc), rtol=1e-12,
                               atol=1e-14)


# ---------------------------------------------------------------- invariants

def test_joint_key_value_permutation_and_query_permutation():
    w = synth.small("dense", 1, 12, 2, 64, 100, Nk=19, sigma_qk=2.0)
    q, k, v = w.tensors()
    base = oracle.attention(q, k, v)
    rng = np.random.default_rng(5)
    pk = rng.permutation(19)
    np.testing.assert_allclose(oracle.attention(q, k[:, pk], v[:, pk]), base, rtol=1e-12)
    pq = rng.permutation(12)
    np.testing.assert_allclose(oracle.attention(q[:, pq], k, v), base[:, pq], rtol=1e-12)


def test_linear_in_values_and_shift_invariant_in_keys():
    rng = np.random.default_rng(6)
    D = 64
    q = rng.integers(-3, 4, size=(1, 4, 2, D)).astype(np.float32) * 0.25
    k = rng.integers(-3, 4, size=(1, 6, 2, D)).astype(np.float32) * 0.25
    v1 = rng.integers(-8, 9, size=(1, 6, 2, D)).astype(np.float32)
    v2 = rng.integers(-8, 9, size=(1, 6, 2, D)).astype(np.float32)
    a = oracle.attention(bits(q), bits(k), bits(v1))
    b = oracle.attention(bits(q), bits(k), bits(v2))
    c = oracle.attention(bits(q), bits(k), bits(v1 + v2))
    np.testing.assert_allclose(c, a + b, rtol=1e-12, atol=1e-12)
    u = rng.integers(-2, 3, size=(1, 1, 2, D)).astype(np.float32)
    shifted = oracle.attention(bits(q), bits(k + u), bits(v1))
    np.testing.assert_allclose(shifted, a, rtol=1e-11, atol=1e-11)


def test_output_is_convex_combination_of_values():
    w = synth.small("dense", 2, 8, 2, 128, 110, Nk=33, sigma_qk=3.0)
    q, k, v = w.tensors()
    out = oracle.attention(q, k, v)
    vf = attn_np.bf16_bits_to_f64(v)
    lo = vf.min(axis=1, keepdims=True)
    hi = vf.max(axis=1, keepdims=True)
    assert np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)


def test_each_head_slice_equals_single_head_call():
    """Pins the [B, N, H, D] strides: head h of batch b alone gives the same rows."""
    w = synth.small("dense", 2, 5, 3, 64, 120, Nk=7)
    q, k, v = w.tensors()
    full = oracle.attention(q, k, v)
    for b in range(2):
        for h in range(3):
            one = oracle.attention(q[b:b + 1, :, h:h + 1].copy(), k[b:b + 1, :, h:h + 1].copy(),
                                   v[b:b + 1, :, h:h + 1].copy())
            np.testing.assert_array_equal(one[0, :, 0], full[b, :, h])


@pytest.mark.parametrize("split", [1, 4, 8])
def test_prefix_equals_dense_on_concatenation_for_every_split(split):
    w = synth.small("dense", 1, 6, 2, 128, 130, Nk=9, sigma_qk=2.0)
    q, k, v = w.tensors()
    dense = oracle.attention(q, k, v)
    pre = oracle.prefix_attention(q, k[:, :split].copy(), v[:, :split].copy(),
                                  k[:, split:].copy(), v[:, split:].copy()) if split < 9 else None
    if pre is not None:
        np.testing.assert_array_equal(pre, dense)


def test_log_sum_exp_merge_of_key_halves_equals_whole():
    """Splitting the keys into two parts and merging the two partial results with their
    log-sum-exp weights reproduces the whole (the identity a split-KV path relies on)."""
    w = synth.small("dense", 1, 5, 2, 64, 140, Nk=23, sigma_qk=3.0)
    q, k, v = w.tensors()
    whole = oracle.attention_rows(q, k, v)
    o1, l1 = oracle.attention_rows(q, k[:, :10].copy(), v[:, :10].copy(), want_lse=True)
    o2, l2 = oracle.attention_rows(q, k[:, 10:].copy(), v[:, 10:].copy(), want_lse=True)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (o1 * w1[:, None] + o2 * w2[:, None]) / (w1 + w2)[:, None]
    np.testing.assert_allclose(merged, whole, rtol=1e-12, atol=1e-14)


def test_selected_rows_match_full_output():
    w = synth.small("dense", 2, 9, 3, 64, 150, Nk=11)
    q, k, v = w.tensors()
    full = oracle.attention_rows(q, k, v)
    rows = np.array([0, 5, 17, 53, 2 * 9 * 3 - 1])
    np.testing.assert_array_equal(oracle.attention_rows(q, k, v, rows=rows), full[rows])


def test_bad_rows_and_shapes_raise():
    w = synth.small("dense", 1, 3, 1, 64, 160)
    q, k, v = w.tensors()
    with pytest.raises(RuntimeError):
        oracle.attention_rows(q, k, v, rows=[3])
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v[:, :2].copy())


# ---------------------------------------------------------------- input generator

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38, 1e-40],
                 np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0
    assert back[0] == 1.0 and back[1] == 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert back[2] == 1.0 + 2 ** -6
    assert back[3] == -1.0
    assert np.isfinite(back[4])


def test_generator_is_seeded_and_shaped():
    w = synth.workload(0)
    a = w.tensors()
    b = w.tensors()
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert a[0].shape == (1, 256, 32, 64) and a[0].dtype == np.uint16
    assert not np.array_equal(a[0], a[1])
    f = synth.bf16_bits_to_f32(a[0])
    assert abs(float(f.mean())) < 0.01 and abs(float(f.std()) - 1.0) < 0.01


def test_outlier_workload_statistics():
    w = synth.Workload("t", "dense", 1, 256, 32, 128, 5, sigma_qk=3.0, outliers=4)
    q, k, v = w.tensors()
    ch = synth.outlier_channels(6099, 32, 128)
    qf = synth.bf16_bits_to_f32(q)
    kf = synth.bf16_bits_to_f32(k)
    for h in (0, 31):
        assert abs(float(qf[0, :, h, ch[h]].std()) - 24.0) < 2.0
        assert abs(float(kf[0, :, h, ch[h]].std()) - 24.0) < 2.0
        others = np.setdiff1d(np.arange(128), ch[h])
        assert abs(float(qf[0, :, h, others].std()) - 3.0) < 0.2
    assert abs(float(synth.bf16_bits_to_f32(v).std()) - 1.0) < 0.05
