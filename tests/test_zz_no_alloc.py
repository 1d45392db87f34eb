"""attn_fwd_ex_noalloc (the entry point that allocates nothing) through the C ABI,
against attn_fwd_ex on the same inputs and launch options, and against the FP64 oracle
under the acceptance rule: two calls in a row, the second with a smaller input, then a
plan beyond the static scratch array's size."""
import sys

import numpy as np
import pytest

import oracle
import synth
import transformer_attention_dense_amd as attn
from acceptance import assert_accepted

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20  # the size include/attn_dense.h states for the static array


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def call(fn, q, k0, v0, k1, v1, out, splits, waves):
    B, Nq, H, D = q.shape
    n0 = k0.shape[1]
    n1 = k1.shape[1] if k1 is not None else 0
    rc = fn(q.data_ptr(), k0.data_ptr(), v0.data_ptr(), n0,
            k1.data_ptr() if n1 else None, v1.data_ptr() if n1 else None, n1,
            out.data_ptr(), B, Nq, H, D, splits, waves,
            torch.cuda.current_stream().cuda_stream)
    return rc


CASES = [
    # kind, B, Nq, H, D, keys (dense) or Np (prefix), splits, waves
    ("dense", 2, 500, 4, 128, 900, 4, 4),
    ("prefix", 1, 130, 2, 64, 170, 3, 2),   # smaller than the first: stale scratch contents
]


def test_two_calls_match_the_allocating_entry_point():
    for kind, B, Nq, H, D, nk, splits, waves in CASES:
        say(f"no-alloc {kind} B{B} Nq{Nq} H{H} D{D} keys{nk} splits{splits} waves{waves}")
        if kind == "dense":
            w = synth.small("dense", B, Nq, H, D, 1700 + Nq, Nk=nk, sigma_qk=2.0)
            q, k0, v0 = w.tensors()
            k1 = v1 = None
            ref = oracle.attention(q, k0, v0)
        else:
            w = synth.small("prefix", B, Nq, H, D, 1700 + Nq, Np=nk, sigma_qk=2.0)
            q, k0, v0, k1, v1 = w.tensors()
            ref = oracle.prefix_attention(q, k0, v0, k1, v1)
        plan = attn.attn_plan(B, Nq, k0.shape[1] + (Nq if k1 is not None else 0), H, D,
                              num_splits=splits, waves=waves)
        assert plan["splits"] > 1 and 0 < plan["workspace_bytes"] <= SCRATCH_BYTES
        t = [dev(x) if x is not None else None for x in (q, k0, v0, k1, v1)]
        out_a = torch.full_like(t[0], 9.0)
        out_b = torch.full_like(t[0], -9.0)
        assert call(attn.library().attn_fwd_ex, *t, out_a, splits, waves) == 0
        assert call(attn.library().attn_fwd_ex_noalloc, *t, out_b, splits, waves) == 0
        a, b = host(out_a), host(out_b)
        assert np.array_equal(a, b), f"{kind}: no-alloc output differs from attn_fwd_ex"
        assert_accepted(b, ref, f"no-alloc {kind}")


def test_plan_beyond_the_scratch_array_is_rejected_untouched():
    B, Nq, Nk, H, D, splits = 1, 1024, 16384, 4, 128, 64
    plan = attn.attn_plan(B, Nq, Nk, H, D, num_splits=splits)
    assert plan["workspace_bytes"] > SCRATCH_BYTES
    say(f"no-alloc oversize plan: {plan['workspace_bytes']} bytes")
    q = dev(synth.normal_bf16((B, Nq, H, D), 1750))
    kv = dev(synth.normal_bf16((B, Nk, H, D), 1751))
    out = torch.full_like(q, 4.0)
    assert call(attn.library().attn_fwd_ex_noalloc, q, kv, kv, None, None, out, splits,
                0) == -7
    torch.cuda.synchronize()
    assert bool((out == 4.0).all())


def test_one_range_plan_needs_no_scratch():
    w = synth.small("dense", 1, 300, 2, 64, 1760)
    q, k, v = w.tensors()
    t = [dev(x) for x in (q, k, v)]
    out = torch.empty_like(t[0])
    assert call(attn.library().attn_fwd_ex_noalloc, t[0], t[1], t[2], None, None, out, 1,
                0) == 0
    assert_accepted(host(out), oracle.attention(q, k, v), "no-alloc one range")
