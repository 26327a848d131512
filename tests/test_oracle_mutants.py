"""The pins must catch plausible mistakes in the oracle (CPU).

Each case plants one mistake in a copy of ``oracle/trace_oracle.c`` (a
textual substitution that must apply exactly as often as stated), builds the
copy with the oracle's own gcc flags, and runs the pins of
``test_oracle_pins.py`` against it in a child process (``TRACE_ORACLE_LIB``
points the oracle module at the copy).  The case passes when the pins fail.
An unmodified copy taken through the same route must pass them.

Mutants that cannot change any result are left out on purpose: e.g. dropping
the saturation shortcut of the E4M3 encoder or of RTN (the literal nearest
search saturates by itself), storing the whole nibble for k < 4 (its low k
bits are those of the magnitude index), or moving the MX clamp at the top of
E8M0's range (the largest finite float gives code 252, so it is never hit).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "trace_oracle.c")

# name -> (original text, planted text, occurrences), or a list of such
# substitutions planted together
MUTANTS = {
    # global scale: amax / 448 instead of amax / (6 * 448)
    "global_scale_drops_6": ("g_out[gi] = A / 2688.0f;", "g_out[gi] = A / 448.0f;", 1),
    # block scale: t = a_b / g instead of a_b / (6 g)
    "block_scale_drops_6": ("float six_g = 6.0f * g;", "float six_g = g;", 1),
    # combined scale without the global scale
    "combined_scale_drops_g": ("float c = (float)oracle_e4m3_value(s) * g;",
                               "float c = (float)oracle_e4m3_value(s);", 1),
    # E4M3 ties to the odd code
    "e4m3_ties_to_odd": ("(w == 0 && (c & 1) == 0)", "(w == 0 && (c & 1) == 1)", 1),
    # E4M3 decode with bias 8
    "e4m3_wrong_bias": ("return ldexp(8.0 + m, e - 10);", "return ldexp(8.0 + m, e - 11);", 1),
    # E2M1 normal magnitudes one binade low
    "e2m1_wrong_bias": ("return ldexp(1.0 + 0.5 * m, e - 1);", "return ldexp(1.0 + 0.5 * m, e - 2);", 1),
    # RTN ties to the odd index
    "rtn_ties_to_odd": ("(w == 0 && (j & 1) == 0)", "(w == 0 && (j & 1) == 1)", 1),
    # RTN loses the sign
    "rtn_drops_sign": ("return (signbit(v) ? 8 : 0) | oracle_rtn_index(v);", "return oracle_rtn_index(v);", 1),
    # normalise by dividing by the reciprocal
    "normalise_divides": ("float v = oracle_bf16_to_f32(y[e]) * inv;", "float v = oracle_bf16_to_f32(y[e]) / inv;", 1),
    # block amax of signed values
    "block_amax_signed": ("float a = fabsf(oracle_bf16_to_f32(y[16 * b + i]));",
                          "float a = oracle_bf16_to_f32(y[16 * b + i]);", 1),
    # global amax of signed values
    "global_amax_signed": ("float a = fabsf(f);", "float a = f;", 1),
    # the nearer end reversed
    "nearer_end_reversed": ("if (w < 0) return lo;\n    if (w > 0) return hi;",
                            "if (w < 0) return hi;\n    if (w > 0) return lo;", 1),
    # guidance compared with the high k bits of the index instead of the low
    "guidance_high_bits": ("if (((nib & 7) & mask) != gb) continue;",
                           "if (((nib & 7) >> (3 - k)) != gb) continue;", 2),
    # the tie fallback to RTN removed
    "no_rtn_fallback_on_tie": ("if (distinct > 1)\n", "if (0)\n", 1),
    # an on-grid value no longer its own lower bracket end
    "bracket_excludes_grid": ("if (val <= x && val > L) L = val;", "if (val < x && val > L) L = val;", 1),
    # element 2m in the high nibble
    "nibble_order_swapped": ("int sh = (i & 1) ? 4 : 0;", "int sh = (i & 1) ? 0 : 4;", 1),
    # bit plane filled most significant bit first
    "bitplane_msb_first": ("uint8_t m = (uint8_t)(1u << (p % 8));", "uint8_t m = (uint8_t)(1u << (7 - p % 8));", 1),
    # dequantise without the global scale
    "dequant_drops_g": ("float y = p * g;", "float y = p;", 1),
    # bf16 ties to the odd mantissa
    "bf16_ties_to_odd": ("pick = ((lo >> 16) & 1) ? hi : lo;", "pick = ((lo >> 16) & 1) ? lo : hi;", 1),
    # MX shared exponent with emax 1 instead of 2
    "mx_wrong_emax": ("int shared = (e - 1) - 2;", "int shared = (e - 1) - 1;", 1),
    # MX dequantisation drops the sign
    "mx_dequant_drops_sign": ("return (nib & 8) ? -(float)y : (float)y;", "return (float)y;", 1),
    # no clamp of the MX shared exponent at the bottom of E8M0's range (block maxima below 2^-125)
    "mx_no_low_clamp": ("if (code < 0) code = 0;", "", 1),
    # an all-zero MX block gets scale 1 (code 127) instead of code 0
    "mx_zero_block_code": ("    if (!(amax > 0.0f))\n        return 0;", "    if (!(amax > 0.0f))\n        return 127;", 1),
    # the full-code rule compares with the rollout value's magnitude, ignoring its sign
    "fullcode_ignores_sign": ("pick_nearer(lo, hi, oracle_e2m1_value(r), v)",
                              "pick_nearer(lo, hi, fabs(oracle_e2m1_value(r)), v)", 1),
    # E4M3 subnormal scales flushed to zero
    "e4m3_subnormals_flushed": ("return ldexp((double)m, -9);", "return 0.0 * m;", 1),
    # dequantised values lose the code's sign
    "dequant_drops_sign": ("return (nib & 8) ? -y : y;", "return y;", 1),
    # the chosen code's sign taken from the chosen value (loses -0) instead of v
    "guided_sign_from_chosen": ("return (signbit(v) ? 8 : 0) | magnitude_index_of(chosen);",
                                "return (signbit(chosen) ? 8 : 0) | magnitude_index_of(chosen);", 2),
    # the global amax misses each group's last element
    "amax_skips_group_end": ("i < (gi + 1) * per; ++i", "i < (gi + 1) * per - 1; ++i", 1),
    # no zero pad between the guidance scale plane and the bit plane
    "no_guidance_pad": ("    int64_t sp = n / 16;\n    return (sp + 255) / 256 * 256;",
                        "    int64_t sp = n / 16;\n    return sp;", 1),
    # +0 and -0 counted as two distinct candidates, so a nearest zero code reads as a tie (RTN fallback)
    "zero_signs_distinct": ("if (val != best && nearer(best, val, (double)v) == 0) distinct = 2;",
                            "if ((val != best || signbit(val) != signbit(best)) && nearer(best, val, (double)v) == 0)"
                            " distinct = 2;", 1),
    # an on-grid value no longer its own upper bracket end
    "bracket_hi_excludes_grid": ("if (val >= x && val < H) H = val;", "if (val > x && val < H) H = val;", 1),
    # a k-bit field written and read most significant bit first (a consistent layout mistake)
    "kbit_fields_reversed": [("if ((value >> j) & 1)", "if ((value >> (k - 1 - j)) & 1)", 1),
                             ("value |= ((plane[p / 8] >> (p % 8)) & 1) << j;",
                              "value |= ((plane[p / 8] >> (p % 8)) & 1) << (k - 1 - j);", 1)],
    # the gradient mask: the saturation edge itself excluded (|v| < 6 instead of <= 6)
    "ste_strict_edge": ("mask[e] = fabs((double)v) <= 6.0 ? 1 : 0;", "mask[e] = fabs((double)v) < 6.0 ? 1 : 0;", 1),
    # the gradient mask compares the raw input with 6, forgetting the scales
    "ste_ignores_scales": ("mask[e] = fabs((double)v) <= 6.0 ? 1 : 0;",
                           "mask[e] = fabs((double)oracle_bf16_to_f32(x[e])) <= 6.0 ? 1 : 0;", 1),
    # the gradient mask inverted (passes only where the forward saturated)
    "ste_mask_inverted": ("mask[e] = fabs((double)v) <= 6.0 ? 1 : 0;", "mask[e] = fabs((double)v) <= 6.0 ? 0 : 1;", 1),
    # each block takes the first group's global scale
    "ste_first_group_only": ("float inv = inv_from_scale(scales[b], g[b / bpg]);",
                             "float inv = inv_from_scale(scales[b], g[0]);", 1),
}


CONTROL = "unmodified"


def _build(name, tmp):
    src = open(SRC).read()
    if name != CONTROL:
        subs = MUTANTS[name] if isinstance(MUTANTS[name], list) else [MUTANTS[name]]
        for orig, planted, count in subs:
            assert src.count(orig) == count, f"{name}: expected {count} occurrence(s) of {orig!r}"
            src = src.replace(orig, planted)
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    sys.path.insert(0, ROOT)
    import oracle

    lib = os.path.join(tmp, f"lib_{name}.so")
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, "-w", path, "-o", lib, "-lm"])
    return lib


def _run_pins(lib):
    env = dict(os.environ, TRACE_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x", "-q",
           "-p", "no:cacheprovider", "--hypothesis-seed=0", "-m", "not gpu"]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED") or "passed" in ln or "failed" in ln]
    return r.returncode, lines


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("oracle_mutants"))
    libs = {name: _build(name, tmp) for name in [CONTROL, *MUTANTS]}
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run_pins, lib) for name, lib in libs.items()}
        return {name: f.result() for name, f in futs.items()}


def test_control_copy_passes_the_pins(outcomes):
    """The same build-and-load route with nothing planted passes, so a failure
    below comes from the planted mistake and not from the route."""
    rc, lines = outcomes[CONTROL]
    assert rc == 0, f"unmodified copy failed the pins (exit {rc}): {lines[-3:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(outcomes, name):
    rc, lines = outcomes[name]
    assert rc == 1, f"mutant {name} survived the pins (exit {rc}): {lines[-3:]}"
