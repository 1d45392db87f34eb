"""Mutation check of the oracle's pins, on the CPU.

Each case plants one plausible mistake in a copy of oracle/attn_oracle.c, builds it
into a temporary library and runs the pin suites (tests/test_oracle.py and
tests/test_oracle_block_causal.py) against it in a subprocess. Every mutant must make at least one pin fail; the unmodified source
must pass. This shows the pins constrain the oracle rather than restate it.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

MUTANTS = {
    "scale_dropped": ("s[j] = dot * scale;", "s[j] = dot;"),
    "scale_inverse_d": ("pow((double)D, -0.5)", "(1.0 / (double)D)"),
    "exponent_sign": ("s[j] = exp(s[j] - mx);", "s[j] = exp(mx - s[j]);"),
    "max_not_subtracted": ("s[j] = exp(s[j] - mx);", "s[j] = exp(s[j]);"),
    "not_normalised": ("const double p = s[j] / l;", "const double p = s[j];"),
    "key_layout_bhnd": ("if (j < n0) return s0 + ((b * n0 + j) * H + h) * D;",
                        "if (j < n0) return s0 + ((b * H + h) * n0 + j) * D;"),
    "query_head_index_swapped": ("const long h = r % H;\n                const long bi = r / H;\n"
                                 "                const long i = bi % Nq;\n"
                                 "                const long b = bi / Nq;",
                                 "const long i = r % Nq;\n                const long bi = r / Nq;\n"
                                 "                const long h = bi % H;\n"
                                 "                const long b = bi / H;"),
    "segments_swapped": ("if (j < n0) return s0 + ((b * n0 + j) * H + h) * D;\n"
                         "    return s1 + ((b * n1 + (j - n0)) * H + h) * D;",
                         "if (j < n1) return s1 + ((b * n1 + j) * H + h) * D;\n"
                         "    return s0 + ((b * n0 + (j - n1)) * H + h) * D;"),
    "values_read_from_keys": ("seq_row(v0, n0, v1, n1, b, j, H, D, h)",
                              "seq_row(k0, n0, k1, n1, b, j, H, D, h)"),
    "last_key_dropped": ("for (long j = 0; j < nk; ++j) {\n                    const uint16_t* kr",
                         "for (long j = 0; j < nk - 1; ++j) {\n                    const uint16_t* kr"),
    # block-causal operator (no prefix)
    "bc_strictly_causal": ("allowed[j] = (unsigned char)(j <= i || same_image);",
                           "allowed[j] = (unsigned char)(j < i || same_image);"),
    "bc_no_causal_part": ("allowed[j] = (unsigned char)(j <= i || same_image);",
                          "allowed[j] = (unsigned char)(j == i || same_image);"),
    "bc_text_sees_future_text": ("const int same_image = ids[i] >= 0 && ids[i] == ids[j];",
                                 "const int same_image = ids[i] == ids[j];"),
    "bc_image_sees_everything": ("const int same_image = ids[i] >= 0 && ids[i] == ids[j];",
                                 "const int same_image = ids[i] >= 0;"),
    "na_window_not_moved_inside": ("    if (s > L - k) s = L - k;\n    if (s < 0) s = 0;\n    *lo = s;\n    *hi = s + k;",
                                   "    *lo = s < 0 ? 0 : s;\n    *hi = (i + k / 2 + 1 < L) ? i + k / 2 + 1 : L;"),
    "na_window_off_centre": ("    long s = i - k / 2;", "    long s = i - k / 2 + 1;"),
    "na_axes_y_x_swapped": ("                na_window(y, ky, Y, &y0, &y1);\n                na_window(x, kx, X, &x0, &x1);",
                            "                na_window(y, kx, X, &y0, &y1);\n                na_window(x, ky, Y, &x0, &x1);"),
    "na_scaled_by_head_dim": ("                            s[n] = dot;", "                            s[n] = dot * pow((double)D, -0.5);"),
    "na_values_of_first_key": ("                    const uint16_t* vr = v + (kidx[j] * H + h) * D;",
                               "                    const uint16_t* vr = v + (kidx[0] * H + h) * D;"),
    "bc_key_id_index": ("const int same_image = ids[i] >= 0 && ids[i] == ids[j];",
                        "const int same_image = ids[i] >= 0 && ids[i] == ids[j > 0 ? j - 1 : 0];"),
}


def _build_variant(tmp_path, name, src_text):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    str(c), "-lm"], check=True)
    return str(so)


def _run_pins(lib):
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle.py"),
                           os.path.join(ROOT, "tests", "test_oracle_block_causal.py"),
                           os.path.join(ROOT, "tests", "test_oracle_na3d.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_unmodified_oracle_passes_pins(tmp_path):
    lib = _build_variant(tmp_path, "clean", open(SRC).read())
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_some_pin(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    # a slip in an idiom both operator functions share is planted in both
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    lib = _build_variant(tmp_path, name, src.replace(old, new))
    r = _run_pins(lib)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
