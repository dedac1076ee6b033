"""Planted mistakes in copies of the oracle's C source: the pin battery must
catch each one (CPU only; the oracle file itself is never modified)."""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sparse_attn_ref.c")

MUTANTS = {
    "sink_left_out_of_denominator": ("const double wz = sink ? exp(z - m) : 0.0;",
                                     "const double wz = 0.0;"),
    "exponent_sign_flipped": ("s[k] = exp(s[k] - m);", "s[k] = exp(m - s[k]);"),
    "scale_dropped": ("s[k] = sc * dot;", "s[k] = dot;"),
    "wrong_query_head": ("const uint16_t *qh = q + (qi * H + h) * D;",
                         "const uint16_t *qh = q + (qi * H + (H - 1 - h)) * D;"),
    "no_normalisation": ("oh[d] = acc[d] / L;", "oh[d] = acc[d];"),
    "rows_of_sequence_zero": ("const uint16_t *kvb = kv + b * N * D;",
                              "const uint16_t *kvb = kv;"),
    "dot_product_short_by_one": ("for (int64_t d = 0; d < D; ++d)\n                    dot +=",
                                 "for (int64_t d = 0; d + 1 < D; ++d)\n                    dot +="),
    "sink_weight_doubled": ("double L = wz;", "double L = 2.0 * wz;"),
    "dedup_flag_ignored": ("if (use[k] && (flags & ORACLE_DEDUP))", "if (use[k] && 0)"),
    "dedup_always_applied": ("if (use[k] && (flags & ORACLE_DEDUP))", "if (use[k])"),
    "sink_scale_flag_ignored": ("const double z = (flags & ORACLE_SINK_SCALED) ? sc * zraw : zraw;",
                                "const double z = zraw;"),
    "sink_scale_flag_always": ("const double z = (flags & ORACLE_SINK_SCALED) ? sc * zraw : zraw;",
                               "const double z = sc * zraw;"),
}


def test_unmodified_source_passes(ref):
    assert pins.run_battery(ref) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_battery_catches_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                           "-o", str(lib), str(src), "-lm"])
    fails = pins.run_battery(oracle.ref_from_library(str(lib)))
    assert fails, f"no pin caught the planted mistake {name}"
