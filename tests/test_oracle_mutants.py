"""Pin strength (CPU only): plausible mistakes planted in copies of the
oracle must each fail a pin.

Each case below rewrites one spot of orc.c -- the kind of slip a reader of
the pages could make (a reciprocal scale, a tie rule, a swapped stochastic
rounding comparison or plane, the NVFP4 scale association, the delayed
window slot, the MX exponent offset, a Philox constant, the Hadamard stage
order, the random-bit layout, saturation) -- builds the copy with the
oracle's own flags, and runs the pins that target that spot against it in a
child process (the ORC_LIB variable points the oracle package at the copy).
The pins must fail for every mutant and pass for the unchanged oracle."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "oracle"))
import build as orc_build  # noqa: E402

T = "tests/"
MUTANTS = [
    ("alpha as the reciprocal of s", "float al = fmax / a;", "float al = 1.0f / (a / fmax);",
     [T + "test_oracle_recipes.py::test_worked_example_current_scaling"]),
    ("ties to the odd code", "k = (lo & 1u) ? hi : lo;", "k = (lo & 1u) ? lo : hi;",
     [T + "test_oracle_codecs.py::test_encode_brute_force_at_ties_and_neighbours"]),
    ("saturation to NaN", "    if (a >= v[top]) {\n        k = top;", "    if (a >= v[top]) {\n        k = top + 1;",
     [T + "test_oracle_codecs.py::test_saturation_and_signed_zero"]),
    ("FP8 stochastic rounding by comparison", "g * 65536.0 >= (double)(65536u - (u & 0xFFFFu)) ? hi : lo",
     "(double)(u & 0xFFFFu) < g * 65536.0 ? hi : lo",
     [T + "test_oracle_sr8.py::test_fp8_sr_neighbours_exact_up_count_and_unbiased"]),
    ("E2M1 stochastic rounding by comparison", "if (g * 65536.0f >= (float)(65536u - u))",
     "if ((float)u < g * 65536.0f)", [T + "test_oracle_sr.py::test_e2m1_sr_neighbours_and_exact_up_count"]),
    ("per-tensor SR planes swapped", "sr_ctx sr_row = {1, seed, offset, 0}, sr_col = {1, seed, offset, 1};",
     "sr_ctx sr_row = {1, seed, offset, 1}, sr_col = {1, seed, offset, 0};",
     [T + "test_oracle_sr8.py::test_per_tensor_sr_recomputed"]),
    ("NVFP4 elements x / d", "float y = load_x(x, dt, i * ld + j) * r;", "float y = load_x(x, dt, i * ld + j) / d;",
     [T + "test_oracle_nvfp4_pins.py"]),
    ("NVFP4 tensor scale 2688 / A", "orc_tensor_scales(b_amax, 448.0f, &t.alpha_s, &t.S);",
     "orc_tensor_scales(A, 2688.0f, &t.alpha_s, &t.S);", [T + "test_oracle_nvfp4_pins.py"]),
    ("delayed window slot off by one", "hist[step % H] = a;", "hist[(step + 1) % H] = a;",
     [T + "test_oracle_recipes.py::test_delayed_window_expiry",
      T + "test_oracle_recipes.py::test_delayed_ring_matches_window_max"]),
    ("MX exponent one too high", "e = (ex - 1) - fmt_emax(fmt);", "e = ex - fmt_emax(fmt);",
     [T + "test_oracle_recipes.py::test_mx_code_closed_form_all_bf16"]),
    ("Philox multiplier typo", "0xD2511F53u", "0xD2511F55u",
     [T + "test_oracle_sr.py::test_philox_matches_torch_engine"]),
    ("Hadamard stages in reverse order", "for (h = 1; h < 16; h *= 2)", "for (h = 8; h >= 1; h /= 2)",
     [T + "test_oracle_rht.py::test_rht_fp32_stage_order"]),
    ("random bits from the wrong word", "return (out[j / 2] >> (16 * (j % 2))) & 0xFFFFu;",
     "return (out[j % 4] >> (16 * (j / 4))) & 0xFFFFu;",
     [T + "test_oracle_sr.py::test_sr_bits_follow_one_torch_stream"]),
    ("FP4 nibbles in the other order", "p[r * (C / 2) + k] = (uint8_t)(nib[r * C + 2 * k] | (nib[r * C + 2 * k + 1] << 4));",
     "p[r * (C / 2) + k] = (uint8_t)(nib[r * C + 2 * k + 1] | (nib[r * C + 2 * k] << 4));",
     [T + "test_oracle_recipes.py::test_nvfp4_nibble_order"]),
    ("tile amax over half the tile", "float a = amax_rect(x, dt, C, tr * br, br, tc * bc, bc);",
     "float a = amax_rect(x, dt, C, tr * br, br, tc * bc, bc / 2);",
     [T + "test_oracle_recipes.py::test_block_brute_force_tiny", T + "test_oracle_recipes.py::test_block_invariants"]),
    ("delayed scale from an all-zero window", "    if (m > 0.0f)", "    if (m >= 0.0f)",
     [T + "test_oracle_recipes.py::test_delayed_zero_window_keeps_scale"]),
    ("SR bits of the next element", "q[i] = (uint8_t)encode_plane(fmt, y, sr, i);",
     "q[i] = (uint8_t)encode_plane(fmt, y, sr, i + 1);", [T + "test_oracle_sr8.py::test_per_tensor_sr_recomputed"]),
]


def run_pins(lib, targets):
    env = dict(os.environ, ORC_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *targets],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode, r.stdout[-2000:]


def build_copy(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *orc_build.CFLAGS, c, "-o", path, "-lm"], check=True, capture_output=True)
    return path


@pytest.fixture(scope="module")
def orc_source():
    with open(os.path.join(ROOT, "oracle", "orc.c")) as f:
        return f.read()


def test_pins_pass_on_the_unchanged_oracle(orc_source, tmp_path):
    lib = build_copy(orc_source, str(tmp_path / "liborc_same.so"))
    targets = sorted({t for m in MUTANTS for t in m[3]})
    rc, out = run_pins(lib, targets)
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new,targets", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_the_mutant(orc_source, tmp_path, name, old, new, targets):
    assert orc_source.count(old) == 1, f"{name}: the spot to mutate must occur once"
    lib = build_copy(orc_source.replace(old, new), str(tmp_path / "liborc_mutant.so"))
    rc, out = run_pins(lib, targets)
    assert rc != 0, f"{name}: no pin failed\n{out}"
