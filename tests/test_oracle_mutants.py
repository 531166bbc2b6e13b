"""Mutation check of the oracle's pins (CPU only).

Each mutant is the oracle's C source with one plausible mistake planted in a copy (the
pitfalls listed by "Scaled dot-product attention (forward and backward)", section 5, plus
index/sign slips), compiled with gcc into a temporary directory.  Every mutant must fail
at least one pin in ``oracle_checks``; otherwise the pins would not notice that mistake.
"""

import shutil
from pathlib import Path

import pytest

from oracle import Oracle, build_oracle
from oracle_checks import ALL_CHECKS

SRC = Path(__file__).resolve().parent.parent / "oracle" / "sdpa_oracle.c"

# name -> list of (exact source fragment, replacement); each fragment occurs exactly once
MUTANTS = {
    # pitfall 1: scale by 1/d instead of 1/sqrt(d)
    "s01_scale_1_over_d": [("1.0 / sqrt((double)p->Dk)", "1.0 / (double)p->Dk")],
    # pitfall 3: blocked keys still counted in the normaliser (masking after the softmax)
    "s03_mask_after_softmax": [("    l += P[j];\n", "    l += (s[j] == -INFINITY) ? exp(-m) : P[j];\n")],
    # pitfall 4: softmax VJP without the -D term
    "s04_no_minus_D": [("const double dS = P[j] * (dP[j] - D);", "const double dS = P[j] * dP[j];")],
    # pitfall 5: dK accumulated on the query index (the missing transpose)
    "s05_dk_no_transpose": [("double* dkj = dkg + (int64_t)j * p->Dk;",
                             "double* dkj = dkg + (int64_t)(i % p->Lk) * p->Dk;")],
    # pitfall 6: scale forgotten in dQ
    "s06_dq_no_scale": [("dqi[t] += alpha * dS * kj[t];", "dqi[t] += dS * kj[t];")],
    # pitfall 9: -inf replaced by a large finite negative number
    "s10_mask_minus_1e9": [("      sj += mv;\n", "      sj += isinf(mv) ? -1e9 : mv;\n"),
                           ("      s[j] = -INFINITY;\n      continue;", "      s[j] = -1e9;\n      continue;")],
    # slips: sign of dS, LSE without the max, GQA head map, causal diagonal, dV weight,
    # length bound off by one
    "dS_sign": [("const double dS = P[j] * (dP[j] - D);", "const double dS = P[j] * (D - dP[j]);")],
    "lse_without_max": [("*lse = m + log(l);", "*lse = log(l);")],
    "gqa_modulo_map": [("  const int g = h / G;\n", "  const int g = h % p->Hkv;\n"),
                       ("row_output(p, v, P, b, h / G, o + r * p->Dv);",
                        "row_output(p, v, P, b, h % p->Hkv, o + r * p->Dv);")],
    "causal_strict": [("(!p->is_causal || j <= i + off)", "(!p->is_causal || j < i + off)")],
    # bottom-right alignment: offset with the wrong sign, or from the padded shapes
    # instead of the batch's actual lengths
    "bottom_right_sign": [("? kv_len - q_len : 0;", "? q_len - kv_len : 0;")],
    "bottom_right_padded_shapes": [("? kv_len - q_len : 0;", "? p->Lk - p->Lq : 0;")],
    "dv_uses_dS": [("for (int t = 0; t < p->Dv; ++t) dvj[t] += P[j] * dOi[t];",
                    "for (int t = 0; t < p->Dv; ++t) dvj[t] += dS * dOi[t];")],
    "len_kv_inclusive": [("j < kv_len &&", "j <= kv_len &&")],
    # the window's left edge off by one (a row would see W + 1 keys), or ignoring the
    # bottom-right offset
    "window_inclusive_edge": [("j > i + off - p->window", "j >= i + off - p->window")],
    "window_top_left_only": [("j > i + off - p->window", "j > i - p->window")],
    "dq_missing_row_max": [("P[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);",
                            "P[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j]);")],
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    d = tmp_path_factory.mktemp("oracle_mutants")
    shutil.copy(SRC.parent / "sdpa_oracle.h", d / "sdpa_oracle.h")
    return d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = SRC.read_text()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutant {name}: fragment not found exactly once: {old!r}"
        src = src.replace(old, new)
    csrc = mutant_dir / f"{name}.c"
    csrc.write_text(src)
    lib = build_oracle(out=mutant_dir / f"lib{name}.so", src=csrc, extra_flags=[f"-I{mutant_dir}"])
    orc = Oracle(lib)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
