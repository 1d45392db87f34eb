"""Pins for the FP64 oracle of 3-D neighborhood attention, on the CPU.

The operator (page "Audit SGLang interfaces and refresh validated kernel solutions",
definitions/neighborhood_attention/neighborhood_attention_3d_*: natten.functional.na3d
with kernel_size (kt, ky, kx) and scale 1; Q already carries the model's scale; layout
[B, T, Y, X, H, D]). The pages leave the neighborhood itself to NATTEN; the reading is
NATTEN's published one: on each axis the window of odd size k is centred on the query
and moved inside the axis at its ends, so every query has exactly kt*ky*kx keys.

Each pin ties the C oracle to something other than its own window code: the dense
attention oracle (a full window is all keys), values returned unchanged (a 1x1x1
window), key sets written out literally for 1-D cases, and a numpy form whose windows
come from a search over all windows rather than the start formula.
"""
import numpy as np
import pytest

import oracle
from oracle import attn_np
import synth


def tensors(shape, seed, sigma=1.0):
    q = synth.normal_bf16(shape, seed, sigma)
    k = synth.normal_bf16(shape, seed + 1, sigma)
    v = synth.normal_bf16(shape, seed + 2)
    return q, k, v


def flat(a):
    B, T, Y, X, H, D = a.shape
    return np.ascontiguousarray(a.reshape(B, T * Y * X, H, D))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("shape", [(1, 3, 5, 5, 2, 64), (2, 1, 3, 7, 1, 64), (1, 5, 1, 3, 3, 32)])
def test_window_covering_the_volume_is_dense_attention(shape):
    B, T, Y, X, H, D = shape
    q, k, v = tensors(shape, 100)
    out = oracle.na3d_attention(q, k, v, (T, Y, X))
    dense = oracle.attention(flat(q), flat(k), flat(v), scale=1.0)
    np.testing.assert_allclose(out.reshape(dense.shape), dense, rtol=1e-12, atol=1e-14)


def test_unit_window_returns_the_values():
    shape = (2, 3, 4, 5, 2, 64)
    q, k, v = tensors(shape, 110)
    out = oracle.na3d_attention(q, k, v, (1, 1, 1))
    assert np.array_equal(out, attn_np.bf16_bits_to_f64(v))


# ---------------------------------------------------------------- literal 1-D windows

# Axis of length 7, window 3: the query's own position in the middle, except at the
# ends, where the window stays inside the axis.
WINDOWS_L7_K3 = {0: [0, 1, 2], 1: [0, 1, 2], 2: [1, 2, 3], 3: [2, 3, 4], 4: [3, 4, 5],
                 5: [4, 5, 6], 6: [4, 5, 6]}
# Axis of length 6, window 5.
WINDOWS_L6_K5 = {0: [0, 1, 2, 3, 4], 1: [0, 1, 2, 3, 4], 2: [0, 1, 2, 3, 4],
                 3: [1, 2, 3, 4, 5], 4: [1, 2, 3, 4, 5], 5: [1, 2, 3, 4, 5]}


@pytest.mark.parametrize("axis", [0, 1, 2])
@pytest.mark.parametrize("L,kk,windows", [(7, 3, WINDOWS_L7_K3), (6, 5, WINDOWS_L6_K5)])
def test_one_axis_windows_match_literal_key_sets(axis, L, kk, windows):
    dims = [1, 1, 1]
    dims[axis] = L
    kernel = [1, 1, 1]
    kernel[axis] = kk
    shape = (2, dims[0], dims[1], dims[2], 2, 64)
    q, k, v = tensors(shape, 120 + axis)
    out = oracle.na3d_attention(q, k, v, tuple(kernel))
    qf, kf, vf = flat(q), flat(k), flat(v)
    of = out.reshape(qf.shape)
    for b in range(2):
        for i in range(L):
            keys = np.asarray(windows[i])
            ref = oracle.attention(qf[b:b + 1, i:i + 1], np.ascontiguousarray(kf[b:b + 1, keys]),
                                   np.ascontiguousarray(vf[b:b + 1, keys]), scale=1.0)[0, 0]
            np.testing.assert_allclose(of[b, i], ref, rtol=1e-12, atol=1e-14)


def test_window_search_agrees_with_the_literal_sets():
    for L, kk, windows in ((7, 3, WINDOWS_L7_K3), (6, 5, WINDOWS_L6_K5)):
        vis = attn_np.na_window_search(L, kk)
        for i, keys in windows.items():
            assert list(np.flatnonzero(vis[i])) == keys


# ---------------------------------------------------------------- independent numpy form

@pytest.mark.parametrize("shape,kernel", [((2, 3, 6, 7, 2, 64), (3, 3, 5)),
                                          ((1, 5, 4, 9, 3, 64), (3, 3, 7)),
                                          ((1, 4, 8, 8, 1, 32), (3, 5, 5)),
                                          ((1, 2, 5, 11, 2, 64), (1, 5, 11))])
def test_c_oracle_matches_numpy_window_search(shape, kernel):
    q, k, v = tensors(shape, 130, sigma=2.0)
    np.testing.assert_allclose(oracle.na3d_attention(q, k, v, kernel),
                               attn_np.na3d_attention(q, k, v, kernel), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- invariants

def test_keys_outside_the_window_do_not_matter():
    shape = (1, 3, 7, 9, 2, 64)
    q, k, v = tensors(shape, 140)
    base = oracle.na3d_attention(q, k, v, (3, 3, 3))
    k2, v2 = k.copy(), v.copy()
    # corner (t=2, y=6, x=8) is outside the window of query (0, 0, 0) on the y and x axes
    k2[0, 2, 6, 8] = synth.normal_bf16((2, 64), 141)
    v2[0, 2, 6, 8] = synth.normal_bf16((2, 64), 142)
    moved = oracle.na3d_attention(q, k2, v2, (3, 3, 3))
    assert np.array_equal(moved[0, 0, 0, 0], base[0, 0, 0, 0])
    assert not np.allclose(moved[0, 2, 6, 8], base[0, 2, 6, 8])   # its own window
    assert not np.allclose(moved[0, 1, 5, 7], base[0, 1, 5, 7])   # a neighbour's


def test_selected_rows_and_bad_arguments():
    shape = (1, 3, 5, 5, 2, 64)
    q, k, v = tensors(shape, 150)
    full = oracle.na3d_rows(q, k, v, (3, 3, 3))
    rows = np.array([0, 7, 31, 149])
    assert np.array_equal(oracle.na3d_rows(q, k, v, (3, 3, 3), rows=rows), full[rows])
    for kernel in ((2, 3, 3), (3, 3, 4), (5, 3, 3), (3, 7, 3)):   # even, or longer than the axis
        with pytest.raises(RuntimeError):
            oracle.na3d_rows(q, k, v, kernel)
    with pytest.raises(RuntimeError):
        oracle.na3d_rows(q, k, v, (3, 3, 3), rows=[150])
