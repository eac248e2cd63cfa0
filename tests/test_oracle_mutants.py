"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutant is one textual change to oracle/mla_oracle.c: a dropped term, a
wrong sign, a wrong index, an off-by-one in the causal mask, a transposed
operand.  The mutated copy is compiled into a temporary directory and
swapped in for the real library while a set of pins runs; at least one pin
must fail for every mutant.
"""
import ctypes
import os
import subprocess

import pytest

from oracle import oracle as orc
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(orc.__file__), "mla_oracle.c")

MUTANTS = {
    "drop_scale": ("s[t] = scale64 * dot;", "s[t] = dot;"),
    "causal_off_by_one": ("n - s_q + 1 + i : n;", "n - s_q + i : n;"),
    "causal_reversed": ("n - s_q + 1 + i : n;", "n - i : n;"),
    "lse_drops_max": ("lse[r] = m + log(l);", "lse[r] = log(l);"),
    "softmax_sign": ("const double w = exp(s[t] - m);", "const double w = exp(m - s[t]);"),
    "value_from_rope": ("orow[e] += w * bf16_bits_to_double(krow[t][e]);",
                        "orow[e] += w * bf16_bits_to_double(krow[t][e + (d_qk - d_v)]);"),
    "block_index": ("block_table[(int64_t)b * bt_stride + j / page]",
                    "block_table[(int64_t)b * bt_stride + j % page]"),
    "row_in_page": ("(phys * page + j % page) * d_qk", "(phys * page + (j / page) % page) * d_qk"),
    "no_normalize": ("for (int e = 0; e < d_v; ++e) orow[e] /= l;", ""),
    "combine_weight_uses_max": ("const double w = exp(lp - L);", "const double w = exp(lp - M);"),
    "combine_lse_drops_max": ("const double L = M + log(total);", "const double L = log(total);"),
    "bmm_transposed_weight": ("wh[(int64_t)k * N + n]", "wh[(int64_t)(n % K) * N + (k % N)]"),
    "query_of_wrong_head": ("const double *qrow = q + r * d_qk;",
                            "const double *qrow = q + (r - r % h_q) * d_qk;"),
    "mask_ignored_with_range": ("if (hi > L) hi = L;", "if (hi > n) hi = n;"),
    "e4m3_bias_8": ("else v = ldexp(1.0 + m / 8.0, e - 7);", "else v = ldexp(1.0 + m / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("if (e == 0) v = ldexp((double)m, -9);",
                             "if (e == 0) v = ldexp((double)m, -10);"),
    "e4m3_mantissa_bits": ("else v = ldexp(1.0 + m / 8.0, e - 7);",
                           "else v = ldexp(1.0 + m / 16.0, e - 7);"),
    "bf16_truncates": ("r = ldexp(nearbyint(ldexp(a, 8 - e)), e - 8);",
                       "r = ldexp(floor(ldexp(a, 8 - e)), e - 8);"),
    "bf16_seven_bits": ("r = ldexp(nearbyint(ldexp(a, 8 - e)), e - 8);",
                        "r = ldexp(nearbyint(ldexp(a, 7 - e)), e - 7);"),
    "fp8_block_index_swapped": ("scale[((int64_t)h * kb + k / blk) * nb + n / blk]",
                                "scale[((int64_t)h * kb + (n / blk) % kb) * nb + (k / blk) % nb]"),
    "fp8_block_of_wrong_head": ("scale[((int64_t)h * kb + k / blk) * nb + n / blk]",
                                "scale[(k / blk) * nb + n / blk]"),
}

PINS = [
    lambda: pins.test_golden_fixture(),
    lambda: pins.test_bruteforce_random_small(1, [1, 5, 9], 1, False),
    lambda: pins.test_bruteforce_random_small(3, [6, 11, 2, 1], 3, True),
    lambda: pins.test_bruteforce_random_small(5, [8, 16], 2, False),
    lambda: pins.test_single_key_closed_form(),
    lambda: pins.test_split_combine_equals_unsplit(21),
    lambda: pins.test_causal_row_equals_shorter_decode(),
    lambda: pins.test_absorb_bmm_bruteforce(),
    lambda: pins.test_empty_rows(),
    lambda: pins.test_e4m3_known_codes(),
    lambda: pins.test_e4m3_code_structure(),
    lambda: pins.test_bf16_rounding_of_exact_products(),
    lambda: pins.test_dequant_block_scales_land_on_their_blocks(),
]


def _caught(lib):
    saved = orc._lib
    orc._lib = lib
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                return True
        return False
    finally:
        orc._lib = saved


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "lib_clean.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", SRC,
                           "-o", str(so), "-lm"])
    assert not _caught(orc.bind(ctypes.CDLL(str(so))))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not found once: " + old
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / ("lib_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(src),
                           "-o", str(so), "-lm"])
    assert _caught(orc.bind(ctypes.CDLL(str(so)))), "no pin caught mutant " + name
