"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/ep_oracle.cpp, plants one plausible mistake by a text
substitution (a wrong tie rule, a wrong constant, an unfused or reordered
sum, a lost sign, an unstable order, an inclusive scan, a dropped term ...),
compiles the copy with the oracle's own flags into a temporary library, swaps
it in for the oracle, and runs the fast pins.  At least one pin must fail.
All of this runs on the CPU; the real oracle is untouched.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import oracle.build as obuild
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(obuild.__file__), "ep_oracle.cpp")

MUTANTS = {
    "e4m3_tie_to_odd": ("else c = (lo % 2 == 0) ? lo : hi;", "else c = (lo % 2 == 0) ? hi : lo;"),
    "e4m3_no_saturation_tie": ("if (a >= kE4m3.v[126]) return sign | 0x7e;",
                               "if (a > kE4m3.v[126]) return sign | 0x7e;\n    if (a == kE4m3.v[126]) return sign | 0x7d;"),
    "e4m3_drop_negative_zero": ("uint8_t sign = std::signbit(f) ? 0x80 : 0x00;",
                                "uint8_t sign = (f < 0.0f) ? 0x80 : 0x00;"),
    "bf16_tie_to_odd": ("else pick = (lo % 2 == 0) ? lo : hi;", "else pick = (lo % 2 == 0) ? hi : lo;"),
    "scale_constant": ("scale = amax / 448.0f;", "scale = amax / 440.0f;"),
    "ue8m0_strict_bound": ("while (448.0 * std::ldexp(1.0, s) < static_cast<double>(amax)) ++s;",
                           "while (448.0 * std::ldexp(1.0, s) <= static_cast<double>(amax)) ++s;"),
    "ue8m0_bias": ("exps[b] = static_cast<uint8_t>(s + 127);", "exps[b] = static_cast<uint8_t>(s + 128);"),
    "ue8m0_no_clamp_at_2_pow_minus_127": ("int s = -127;", "int s = -126;"),
    "scale_reciprocal_multiply": ("e4m3_encode(v / scale)", "e4m3_encode(v * (1.0f / scale))"),
    "scale_block_shift": ("float v = bf16_bits_to_float(xt[b * 128 + c]);\n                    assert",
                          "float v = bf16_bits_to_float(xt[(b * 128 + c + 1) % H]);\n                    assert"),
    "combine_unfused": ("acc = std::fmaf(topk_weights[e], v, acc);", "acc = topk_weights[e] * v + acc;"),
    "combine_reverse_order": ("int64_t e = static_cast<int64_t>(t) * k + j;",
                              "int64_t e = static_cast<int64_t>(t) * k + (k - 1 - j);"),
    "combine_drop_last_term": ("for (int32_t j = 0; j < k; ++j) {\n                int64_t e",
                               "for (int32_t j = 0; j < k - (k > 1); ++j) {\n                int64_t e"),
    "combine_swapped_weight_index": ("acc = std::fmaf(topk_weights[e], v, acc);",
                                     "acc = std::fmaf(topk_weights[static_cast<int64_t>(t) * k + (j + 1) % k], v, acc);"),
    "layout_unstable_order": ("int32_t r = cursor[e]++;", "int32_t r = count[e] - 1 - cursor[e]++;"),
    "layout_inclusive_scan_slot": ("slot = static_cast<int64_t>(offset[e]) + r;",
                                   "slot = static_cast<int64_t>(offset[e + 1]) - 1 - r;"),
    "layout_invalid_counted": ("if (e >= 0 && e < E) ++count[e]; else ++num_invalid;",
                               "if (e >= 0 && e < E) ++count[e]; else { ++num_invalid; if (e == E && E > 1) ++count[E - 1]; }"),
    "layout_capacity_off_by_one": ("} else if (r < cap) {", "} else if (r < cap - 1) {"),
}


def _fast_pins():
    return [
        lambda: pins.test_layout_exhaustive_tiny(2, 2, 2),
        lambda: pins.test_layout_exhaustive_tiny(3, 1, 2),
        pins.test_layout_capacity_overflow_drops_later_tokens,
        pins.test_layout_fuzz_vs_stable_sort,
        pins.test_e4m3_decode_named_and_structure,
        pins.test_e4m3_named_ties_and_saturation,
        pins.test_bf16_named,
        pins.test_dispatch_fp8_exact_when_scale_is_power_of_two,
        pins.test_dispatch_fp8_near_ties_vs_exact_rational,
        pins.test_dispatch_ue8m0_vs_exact_exponent_and_torch,
        pins.test_combine_single_term_is_gather,
        pins.test_combine_fma_chain_vs_exact_rational,
        pins.test_combine_skips_unplaced_entries,
        pins.test_combine_vs_exact_sum,
    ]


def test_fast_pins_pass_on_the_real_oracle():
    for pin in _fast_pins():
        pin()


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="ep_oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, tmpdir_mod, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in the oracle"
    path = os.path.join(tmpdir_mod, f"{name}.cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmpdir_mod, f"lib_{name}.so")
    subprocess.run(["g++", *obuild.CXXFLAGS, "-w", path, "-o", lib], check=True)
    saved = oracle._lib
    oracle._lib = None
    monkeypatch.setattr(oracle, "_LIB_PATH", lib)
    try:
        caught = []
        for pin in _fast_pins():
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(getattr(pin, "__name__", "lambda"))
        assert caught, f"no pin caught the planted mistake {name!r}"
    finally:
        oracle._lib = saved
