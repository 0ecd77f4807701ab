"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a flipped sign, a wrong index or denominator, an
off-by-one window, a dropped scale or rotation, a wrong position) in a copy of
the oracle's C source, builds that copy into a temporary library on the CPU,
and runs the pin suite against it in a fresh process. The pin suite must fail
for every case. The real oracle library is never touched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

# name: (text in the oracle, replacement)
MUTATIONS = {
    "rotation_sign": ("y[2 * p] = x0 * c - x1 * s;", "y[2 * p] = x0 * c + x1 * s;"),
    "freq_denominator_R": ("pow(theta, -2.0 * (double)p / (double)D)",
                           "pow(theta, -2.0 * (double)p / (double)rotary_dims)"),
    "rotate_every_pair": ("for (int p = 0; p < rotary_dims / 2; ++p) {",
                          "for (int p = 0; p < D / 2; ++p) {"),
    "gqa_interleaved": ("int g = h / G;\n      memcpy(k_rep", "int g = h % Hkv;\n      memcpy(k_rep"),
    "window_off_by_one": ("if (W > 0 && i - j >= W) return 0;", "if (W > 0 && i - j > W) return 0;"),
    "causal_excludes_self": ("if (j > i) return 0;", "if (j >= i && i > 0) return 0;"),
    "k_not_rotated": ("if (rope_mask & 2)\n        rope_vec(src, dst, Dk, rotary_dims, theta, pos0 + t);",
                      "if (0)\n        rope_vec(src, dst, Dk, rotary_dims, theta, pos0 + t);"),
    "k_position_ignores_pos0": ("rope_vec(src, dst, Dk, rotary_dims, theta, pos0 + t);",
                                "rope_vec(src, dst, Dk, rotary_dims, theta, t);"),
    "decode_query_position": ("rope_vec(q + (size_t)h * Dk, qr, Dk, rotary_dims, theta, L);",
                              "rope_vec(q + (size_t)h * Dk, qr, Dk, rotary_dims, theta, kv_len);"),
    "scale_dropped": ("s *= scale;\n    scores[t] = s;", "scores[t] = s;"),
    "decode_gqa_interleaved": ("const int g = h / G;", "const int g = h % Hkv;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in the oracle"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(mut),
                    "-lm"], check=True)
    env = dict(os.environ, ATTN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    assert r.returncode != 0, f"pins missed the planted mistake {name}:\n{r.stdout[-2000:]}"


PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
# Mistakes planted in the oracle's Python layer (K = V, verify, int8, 2-D RoPE).
PY_MUTATIONS = {
    "kv_shared_unrotated_values": ("return prefill(q, kr, kr,", "return prefill(q, kr, k,"),
    "verify_not_causal_in_draft": ("m = n - n_q + j + 1", "m = n"),
    "int8_round_half_away": ("code = np.rint(x32 / safe[..., None]).astype(np.float32)",
                             "code = np.trunc(x32 / safe[..., None] + np.copysign(np.float32(0.5), x32)).astype(np.float32)"),
    "int8_scale_128": ("s = (amax / np.float32(127.0)).astype(np.float32)",
                       "s = (amax / np.float32(128.0)).astype(np.float32)"),
    "rope_2d_coordinates_swapped": ("first = rope(np.ascontiguousarray(x[:, :, :h]), pxy[:, 0],",
                                    "first = rope(np.ascontiguousarray(x[:, :, :h]), pxy[:, 1],"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_pins_catch_planted_python_mistake(name, tmp_path):
    old, new = PY_MUTATIONS[name]
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found in the oracle"
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(src.replace(old, new))
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    env = dict(os.environ, ATTN_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    # import the mutated copy first, so the pins (and conftest's path setup)
    # find it already loaded
    code = ("import sys; sys.path.insert(0, sys.argv[1]); import oracle; "
            "assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__; "
            "import pytest; sys.exit(pytest.main(sys.argv[2:]))")
    r = subprocess.run([sys.executable, "-c", code, str(tmp_path), "-x", "-q", "-p",
                        "no:cacheprovider", "-k", "kv_shared or verify or int8 or rope_2d",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    assert "AssertionError: /" not in r.stderr, r.stderr[-2000:]
    assert r.returncode == 1, f"pins missed the planted mistake {name}:\n{r.stdout[-2000:]}"
