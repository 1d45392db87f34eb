"""C ABI checks that need no GPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments before any HIP call (pointer values here are
never dereferenced)."""
import os
import re

import pytest

import transformer_attention_dense_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_dense.h")

A = 0x7F0000000000  # fake, 16-byte aligned device addresses; never dereferenced
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_abi_and_library_exports_it():
    names = declared_functions()
    assert set(names) == set(attn.SYMBOLS), names
    lib = attn.library()
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"


def test_probe_library_exports_its_header_and_checks_arguments():
    """The benchmark's clock probe: a library of its own (not the attention ABI) that
    exports what include/attn_probe.h declares and rejects bad arguments before any
    HIP call."""
    import ctypes
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "attn_probe.h")).read(),
                  flags=re.S)
    names = re.findall(r"^\s*\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)
    assert set(names) == {"attn_probe_clock", "attn_probe_realtime_mhz"}
    lib = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_dense_amd", "libattn_probe.so"))
    for n in names:
        assert hasattr(lib, n)
    lib.attn_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    assert lib.attn_probe_clock(None, 256, 2000, None) == -1
    assert lib.attn_probe_clock(A, 0, 2000, None) == -2
    assert lib.attn_probe_clock(A, 256, 0, None) == -2


def test_error_codes_match_header():
    text = open(HEADER).read()
    codes = dict((int(v), k) for k, v in re.findall(r"#define (ATTN_ERR_\w+) \((-\d+)\)", text))
    assert codes == attn.ERRORS
    for c in list(codes) + [0, -99]:
        assert isinstance(attn.attn_strerror(c), str) and attn.attn_strerror(c)


def test_abi_version():
    assert attn.attn_abi_version() == 1


def dense_call(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, B=1, N=256, H=32, D=64):
    return attn.attn_dense(q, k, v, out, B, N, H, D, None)


def test_null_pointers_rejected():
    assert dense_call(q=None) == -1
    assert dense_call(k=None) == -1
    assert dense_call(v=None) == -1
    assert dense_call(out=None) == -1
    assert attn.attn_prefix(A, None, None, None, A + MB, A + 2 * MB, 1, 4, 0, 1, 64, None) == -1
    assert attn.attn_prefix(A, None, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, 1, 4, 2, 1, 64,
                            None) == -1


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(H=0), dict(B=-1), dict(N=-5)])
def test_bad_shapes_rejected(kw):
    assert dense_call(**kw) == -2


def test_prefix_negative_prefix_rejected():
    assert attn.attn_prefix(A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB,
                            1, 4, -1, 1, 64, None) == -2


@pytest.mark.parametrize("D", [0, 32, 96, 256, 65])
def test_unsupported_head_dim_rejected(D):
    assert dense_call(D=D) == -3


def test_bad_launch_options_rejected():
    assert attn.attn_fwd_ex(A, A + MB, A + 2 * MB, 4, None, None, 0, A + 3 * MB, 1, 4, 1, 64,
                            -1, 0, None) == -3
    for w in (1, 3, 6, 16):
        assert attn.attn_fwd_ex(A, A + MB, A + 2 * MB, 4, None, None, 0, A + 3 * MB, 1, 4, 1,
                                64, 0, w, None) == -3


def test_misaligned_pointers_rejected():
    assert dense_call(q=A + 2) == -4
    assert dense_call(k=A + 64 * MB + 8) == -4
    assert dense_call(out=A + 192 * MB + 1) == -4


def test_output_overlapping_an_input_rejected():
    # q, k, v each 1*256*32*64*2 = 1 MiB
    assert dense_call(out=A) == -5
    assert dense_call(out=A + 64 * MB - 512 * 1024) == -5
    assert dense_call(out=A + 128 * MB + 16) == -5
    # adjacent but not overlapping is fine as far as validation goes
    assert attn.attn_plan(1, 256, 256, 32, 64)["splits"] >= 1


def test_sizes_beyond_index_range_rejected():
    assert dense_call(N=1 << 20, H=32, D=128) == -6
    with pytest.raises(attn.AttnError):
        attn.attn_plan(1, 1 << 20, 16, 32, 128)


def test_plan_for_the_workloads():
    # enough query blocks to fill 256 CUs with 8-wave (256-row) workgroups
    p1 = attn.attn_plan(1, 4096, 4096, 32, 128)
    assert p1["splits"] == 1 and p1["waves"] == 8 and p1["workgroups"] == 16 * 32
    assert p1["workspace_bytes"] == 0
    p3 = attn.attn_plan(1, 4096, 5120, 32, 128)
    assert p3["splits"] == 1 and p3["waves"] == 8 and p3["workgroups"] == 512
    # D = 64 as well when the 256-row blocks fill the GPU
    p2 = attn.attn_plan(2, 16384, 16384, 32, 64)
    assert p2["waves"] == 8 and p2["workgroups"] == 64 * 64 and p2["splits"] == 1
    # too few 256-row blocks, and fewer than 256 128-row blocks: 2-wave workgroups
    # (64 rows each); short sequences: 2 waves
    p0 = attn.attn_plan(1, 256, 256, 32, 64)
    assert p0["waves"] == 2 and p0["workgroups"] == 4 * 32 and p0["splits"] == 1
    # 256 blocks of 256 rows: ping-pong; 256 blocks of 128 rows: 4 waves; fewer: 2 waves
    assert attn.attn_plan(1, 1024, 1024, 64, 64)["waves"] == 8
    assert attn.attn_plan(1, 512, 512, 64, 64)["waves"] == 4
    assert attn.attn_plan(1, 512, 512, 32, 64)["waves"] == 2
    # exactly 256 blocks of 256 rows: one 8-wave workgroup per CU, no key split
    for B, N, H, D in [(1, 2048, 32, 64), (1, 2048, 32, 128), (2, 1024, 32, 128),
                       (1, 4096, 16, 128)]:
        assert attn.attn_plan(B, N, N, H, D) == {"splits": 1, "waves": 8, "workgroups": 256,
                                                 "workspace_bytes": 0}, (B, N, H, D)
    # an explicit 8-wave launch on a small grid splits the keys up to 256 workgroups
    p8 = attn.attn_plan(1, 512, 8192, 32, 128, waves=8)
    assert p8["waves"] == 8 and p8["workgroups"] == 256 and p8["splits"] == 4


def test_set_workspace_checks_before_any_device_work():
    assert attn.attn_set_workspace(A + 16, 1 << 20) == -4   # not 256-byte aligned
    assert attn.attn_set_workspace(A, -1) == -2
    # without a GPU the current device cannot be found; with one this sets a buffer
    # that the test immediately withdraws again
    rc = attn.attn_set_workspace(A, 1 << 20)
    assert rc in (0, -8)
    if rc == 0:
        assert attn.attn_set_workspace(None, 0) == 0
    assert attn.attn_plan(1024, 64, 64, 32, 64)["waves"] == 2
    # the 2- and 4-wave kernels split only while the shorter key loops outweigh the merge:
    # 256 four-wave workgroups of 16 key tiles stay whole; 32 two-wave ones with 64 key
    # tiles become 256 (one per CU), 128 with 64 tiles 512 (16 tiles per split)
    assert attn.attn_plan(1, 1024, 1024, 32, 128) == {"splits": 1, "waves": 4, "workgroups": 256,
                                                      "workspace_bytes": 0}
    assert attn.attn_plan(1, 64, 4096, 32, 128)["splits"] == 8
    assert attn.attn_plan(1, 256, 1024, 32, 128)["splits"] == 2
    # small grids take 4 waves (with their splits) over 32 key tiles or more, else 2
    p = attn.attn_plan(1, 256, 4096, 32, 128)
    assert p["waves"] == 4 and p["splits"] == 4 and p["workgroups"] == 256
    assert attn.attn_plan(1, 512, 512, 32, 128)["waves"] == 2
    assert attn.attn_plan(1, 64, 16384, 32, 64)["waves"] == 2
    # few query blocks and long keys -> the keys are split and a work space is needed
    ps = attn.attn_plan(1, 64, 8192, 2, 128)
    assert ps["splits"] > 1 and ps["workspace_bytes"] > 0
    # explicit split counts are clamped to the number of key tiles, with no empty split
    pe = attn.attn_plan(1, 100, 130, 1, 64, num_splits=16)
    assert pe["splits"] == 3
    pe = attn.attn_plan(1, 100, 1999, 1, 64, num_splits=7)
    tiles = -(-1999 // 64)
    per = -(-tiles // 7)
    assert pe["splits"] == -(-tiles // per)


def test_python_helpers_validate_before_the_library():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.dense(x, x, x)  # CPU tensors are rejected
    with pytest.raises(TypeError):
        attn.dense(x.float(), x, x)


def bc_call(q=A, k=A + 64 * MB, v=A + 128 * MB, ids=A + 192 * MB, out=A + 256 * MB, B=1, N=256,
            H=32, D=128):
    return attn.attn_block_causal(q, k, v, ids, out, B, N, H, D, None)


def test_block_causal_rejects_bad_arguments():
    assert bc_call(ids=None) == -1
    assert bc_call(q=None) == -1 and bc_call(out=None) == -1
    assert bc_call(N=0) == -2 and bc_call(B=0) == -2 and bc_call(H=-1) == -2
    assert bc_call(D=96) == -3
    assert bc_call(ids=A + 192 * MB + 4) == -4
    assert bc_call(k=A + 64 * MB + 2) == -4
    assert bc_call(out=A) == -5                     # output over q
    assert bc_call(out=A + 192 * MB - 1024) == -5   # output over the image ids
    assert bc_call(N=1 << 20, H=32) == -6


def test_python_block_causal_validates_before_the_library():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        attn.block_causal(x, x, x, torch.zeros(4, dtype=torch.int32))


def na_call(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, B=1, T=4, Y=8, X=40, H=4,
            D=64, kt=3, ky=5, kx=7):
    return attn.attn_na3d(q, k, v, out, B, T, Y, X, H, D, kt, ky, kx, None)


def test_na3d_rejects_bad_arguments():
    assert na_call(q=None) == -1 and na_call(v=None) == -1 and na_call(out=None) == -1
    assert na_call(B=0) == -2 and na_call(T=0) == -2 and na_call(X=-1) == -2 and na_call(H=0) == -2
    assert na_call(kt=2) == -2 and na_call(ky=0) == -2 and na_call(kx=8) == -2  # even / empty
    assert na_call(kt=5) == -2 and na_call(ky=9) == -2 and na_call(X=5) == -2   # longer than axis
    assert na_call(D=128) == -3
    assert na_call(X=64, kx=19) == -3            # window wider than a tile allows
    assert na_call(k=A + 64 * MB + 2) == -4
    assert na_call(out=A + 1024) == -5            # output over q
    assert na_call(X=1 << 16, H=1 << 10, kx=3) == -6


def test_python_na3d_validates_before_the_library():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 2, 2, 1, 64, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        attn.na3d(x, x, x, (1, 1, 1))  # CPU tensors are rejected
    with pytest.raises((ValueError, TypeError)):
        attn.na3d(x[0], x[0], x[0], (1, 1, 1))


@pytest.mark.parametrize("window,cols,width", [
    ((3, 7, 7), 8, 16), ((3, 5, 5), 4, 8), ((11, 11, 11), 4, 16), ((1, 1, 17), 16, 32),
    ((1, 3, 13), 16, 32), ((1, 7, 13), 4, 16), ((1, 1, 15), 16, 32), ((1, 9, 9), 8, 16),
    ((1, 5, 3), 4, 8), ((1, 3, 5), 8, 16)])
def test_na3d_plan_picks_a_tile_that_holds_the_window(window, cols, width):
    """A wave's query tile is 32 / c rows by c positions; its key blocks hold 32 keys: 32
    positions of one row (c = 16), 16 positions of two rows (c = 8, 4) or 8 positions of four
    rows (c = 4), so the X windows of the c positions, c - 1 + kx positions wide, must fit
    the block width; among those the fewest blocks per query and t' (32 / c + ky - 1 rows
    in blocks of 32 / width rows) wins, ties to the tile listed first (1x3x5: 4x8 queries
    over 16-position blocks and 8x4 queries over 8-position blocks both take three blocks)."""
    kt, ky, kx = window
    B, T, Y, X, H = 2, 11, 37, 45, 3
    plan = attn.attn_na3d_plan(B, T, Y, X, H, 64, kt, ky, kx)
    c = plan["query_cols"]
    assert c == cols
    assert c - 1 + kx <= width
    assert plan["workgroups"] == na3d_grid(B, T, Y, X, H, window, c, width)


def na3d_grid(B, T, Y, X, H, window, c, width):
    """Four waves per workgroup, arranged as wt frames t by 4 / wt tiles of 32 / c rows,
    wt in (1, 2, 4) walking the fewest key blocks: the union of the waves' windows, kt + wt - 1
    frames times blocks of 32 / width rows over the union of their Y windows (ties to the
    larger wt)."""
    kt, ky, _ = window
    rows = 32 // c
    rpb = 32 // width
    best = None
    for wt in (1, 2, 4):
        steps = min(T, kt + wt - 1) * -(-min(Y, 4 // wt * rows + ky - 1) // rpb)
        if best is None or steps <= best[0]:
            best = (steps, wt)
    wt = best[1]
    return B * -(-T // wt) * -(-Y // (4 // wt * rows)) * -(-X // c) * H


def test_na3d_plan_arranges_waves_where_windows_overlap_most():
    """The pages' four neighborhood volumes: 3x7x7 on 64x64 or 32x32 walks 28 blocks with
    two frames by two row tiles (30 with four frames, 33 with four row tiles); 11x11x11 on
    32x32 126 with four frames (156, 176); 3x5x5 on 64x64, 8x4 query tiles over blocks of
    four rows, 18 with four frames (20, 27)."""
    for (T, Y, X, H, win, wt, width) in [(8, 64, 64, 16, (3, 7, 7), 2, 16),
                                         (8, 32, 32, 32, (3, 7, 7), 2, 16),
                                         (16, 32, 32, 4, (11, 11, 11), 4, 16),
                                         (8, 64, 64, 8, (3, 5, 5), 4, 8)]:
        plan = attn.attn_na3d_plan(1, T, Y, X, H, 64, *win)
        c = plan["query_cols"]
        rows = 32 // c
        assert plan["workgroups"] == -(-T // wt) * -(-Y // (4 // wt * rows)) * -(-X // c) * H
        assert plan["workgroups"] == na3d_grid(1, T, Y, X, H, win, c, width)


def test_na3d_plan_errors_match_the_call():
    assert attn.attn_na3d_plan(1, 4, 8, 40, 4, 64, 3, 5, 7)["workgroups"] > 0
    for args, code in [((1, 4, 8, 40, 4, 64, 2, 5, 7), -2), ((1, 4, 8, 40, 4, 128, 3, 5, 7), -3),
                       ((1, 4, 8, 64, 4, 64, 3, 5, 19), -3), ((1, 4, 8, 1 << 16, 1 << 10, 64, 3, 5, 3), -6)]:
        with pytest.raises(attn.AttnError) as e:
            attn.attn_na3d_plan(*args)
        assert e.value.code == code
