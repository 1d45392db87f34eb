"""Pins for the FP64 oracle of block-causal attention without prefix, on the CPU.

The operator (page "Audit SGLang interfaces and refresh validated kernel solutions",
definitions/block_causal_attention/prefix_cached_block_causal_h32_d128_prefix0.json):
row i of Q attends to the keys j with j <= i, or with image_ids[i] >= 0 and
image_ids[j] == image_ids[i]; image_ids is [N] int32, text = -1, shared by the batch.

Each pin ties the oracle to something other than its own mask: the full-visibility
oracle (a separate function) evaluated on the key slices a row is known to see for a
layout built by hand, closed forms at the two extremes of the mask, and invariants.
"""
import numpy as np
import pytest

import oracle
from oracle import attn_np
import synth


def tensors(B, N, H, D, seed, sigma=2.0):
    q = synth.normal_bf16((B, N, H, D), seed, sigma)
    k = synth.normal_bf16((B, N, H, D), seed + 1, sigma)
    v = synth.normal_bf16((B, N, H, D), seed + 2)
    return q, k, v


def dense_row(q, k, v, b, i, keys):
    """Full-visibility oracle for query (b, i) over the listed key positions, all heads."""
    keys = np.asarray(keys)
    return oracle.attention(q[b:b + 1, i:i + 1], np.ascontiguousarray(k[b:b + 1, keys]),
                            np.ascontiguousarray(v[b:b + 1, keys]))[0, 0]


# ---------------------------------------------------------------- closed forms

def test_all_text_is_causal_attention():
    """No image ids: row i sees exactly keys 0..i."""
    B, N, H, D = 2, 37, 2, 64
    q, k, v = tensors(B, N, H, D, 900)
    out = oracle.block_causal_attention(q, k, v, np.full(N, -1, np.int32))
    for b in range(B):
        for i in range(N):
            np.testing.assert_allclose(out[b, i], dense_row(q, k, v, b, i, range(i + 1)),
                                       rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("image_id", [0, 7])
def test_one_image_everywhere_is_dense_attention(image_id):
    B, N, H, D = 1, 45, 3, 128
    q, k, v = tensors(B, N, H, D, 910)
    out = oracle.block_causal_attention(q, k, v, np.full(N, image_id, np.int32))
    np.testing.assert_allclose(out, oracle.attention(q, k, v), rtol=1e-12, atol=1e-14)


def test_first_text_row_returns_first_value():
    B, N, H, D = 2, 20, 2, 64
    q, k, v = tensors(B, N, H, D, 920)
    ids = np.full(N, -1, np.int32)
    ids[5:12] = 0
    out = oracle.block_causal_attention(q, k, v, ids)
    assert np.array_equal(out[:, 0], attn_np.bf16_bits_to_f64(v[:, 0]))


# ---------------------------------------------------------------- hand-built layouts

def test_text_image_text_image_layout():
    """Text [0,6), image 0 [6,20), text [20,25), image 1 [25,40): an image row sees
    every key up to the end of its block; a text row sees keys 0..i."""
    B, N, H, D = 2, 40, 2, 64
    q, k, v = tensors(B, N, H, D, 930)
    ids = np.full(N, -1, np.int32)
    ids[6:20] = 0
    ids[25:40] = 1
    out = oracle.block_causal_attention(q, k, v, ids)
    for b in range(B):
        for i in range(N):
            end = 20 if 6 <= i < 20 else 40 if i >= 25 else i + 1
            np.testing.assert_allclose(out[b, i], dense_row(q, k, v, b, i, range(end)),
                                       rtol=1e-12, atol=1e-14)


def test_same_id_in_two_separate_runs():
    """Id 4 at [3,6) and again at [15,18), text elsewhere: rows 3..5 also see the
    later run; rows of the later run see keys 0..17 (their causal past contains the
    earlier run anyway)."""
    B, N, H, D = 1, 24, 2, 64
    q, k, v = tensors(B, N, H, D, 940)
    ids = np.full(N, -1, np.int32)
    ids[3:6] = 4
    ids[15:18] = 4
    out = oracle.block_causal_attention(q, k, v, ids)
    for i in range(N):
        if 3 <= i < 6:
            keys = list(range(6)) + list(range(15, 18))
        elif 15 <= i < 18:
            keys = list(range(18))
        else:
            keys = list(range(i + 1))
        np.testing.assert_allclose(out[0, i], dense_row(q, k, v, 0, i, keys), rtol=1e-12,
                                   atol=1e-14)


# ---------------------------------------------------------------- invariants

def test_relabelling_image_ids_changes_nothing():
    B, N, H, D = 1, 50, 2, 128
    q, k, v = tensors(B, N, H, D, 950)
    ids = np.full(N, -1, np.int32)
    ids[4:19] = 0
    ids[22:30] = 1
    ids[30:47] = 2
    relab = ids.copy()
    for old, new in ((0, 12), (1, 3), (2, 1000000)):
        relab[ids == old] = new
    assert np.array_equal(oracle.block_causal_attention(q, k, v, ids),
                          oracle.block_causal_attention(q, k, v, relab))


def test_keys_a_row_cannot_see_do_not_matter_and_visible_ones_do():
    B, N, H, D = 1, 30, 2, 64
    q, k, v = tensors(B, N, H, D, 960)
    ids = np.full(N, -1, np.int32)
    ids[10:20] = 0
    base = oracle.block_causal_attention(q, k, v, ids)
    k2, v2 = k.copy(), v.copy()
    k2[:, 25:] = synth.normal_bf16((B, 5, H, D), 961, 2.0)
    v2[:, 25:] = synth.normal_bf16((B, 5, H, D), 962)
    moved = oracle.block_causal_attention(q, k2, v2, ids)
    assert np.array_equal(moved[:, :25], base[:, :25])   # nobody before 25 sees keys >= 25
    assert not np.allclose(moved[:, 25:], base[:, 25:])
    k3 = k.copy()
    k3[:, 18] = synth.normal_bf16((B, 1, H, D), 963, 2.0)[:, 0]
    moved = oracle.block_causal_attention(q, k3, v, ids)
    assert np.array_equal(moved[:, :10], base[:, :10])   # text before the image
    assert not np.allclose(moved[:, 10:18], base[:, 10:18])  # image rows see key 18


def test_probabilities_sum_to_one():
    B, N, H, D = 2, 33, 2, 64
    q, k, v = tensors(B, N, H, D, 970)
    ids = np.full(N, -1, np.int32)
    ids[8:30] = 5
    _, psum = oracle.block_causal_rows(q, k, v, ids, want_psum=True)
    np.testing.assert_allclose(psum, 1.0, atol=1e-12)


# ---------------------------------------------------------------- independent numpy form

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_c_oracle_matches_numpy_form_random_ids(seed):
    rng = np.random.default_rng(seed)
    B, N, H, D = 2, 41, 2, 64 if seed % 2 else 128
    q, k, v = tensors(B, N, H, D, 980 + seed)
    ids = rng.integers(-1, 4, size=N).astype(np.int32)   # arbitrary, not contiguous
    np.testing.assert_allclose(oracle.block_causal_attention(q, k, v, ids),
                               attn_np.block_causal_attention(q, k, v, ids), rtol=1e-12,
                               atol=1e-14)


def test_selected_rows_and_bad_arguments():
    B, N, H, D = 1, 20, 2, 64
    q, k, v = tensors(B, N, H, D, 990)
    ids = np.full(N, -1, np.int32)
    ids[2:9] = 0
    full = oracle.block_causal_rows(q, k, v, ids)
    rows = np.array([0, 7, 17, 39])
    assert np.array_equal(oracle.block_causal_rows(q, k, v, ids, rows=rows), full[rows])
    with pytest.raises(ValueError):
        oracle.block_causal_rows(q, k, v, ids[:-1])
    with pytest.raises(RuntimeError):
        oracle.block_causal_rows(q, k, v, ids, rows=[B * N * H])
