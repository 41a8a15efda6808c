"""The fp64 oracle against hand-derived examples, closed forms, invariants, brute force and
library routines (CPU only)."""

import os
import shutil
import subprocess

import pytest

import pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "oracle.c")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_mod, pin):
    pin(oracle_mod)


# Planted mistakes: each (original, replacement) is applied to a copy of the oracle's source,
# compiled separately, and must make at least one pin fail.
MUTANTS = {
    "eps-outside-root": ("double r = 1.0 / sqrt(s / (double)d + eps);",
                         "double r = 1.0 / (sqrt(s / (double)d) + eps);"),
    "gamma-dropped": ("double g = gamma ? oracle_elem(gdt, gamma, i) : 1.0;\n"
                      "            y[t * ldy + i] = oracle_elem(xdt, x, t * ldx + i) * g * r;",
                      "double g = 1.0; (void)gdt;\n"
                      "            y[t * ldy + i] = oracle_elem(xdt, x, t * ldx + i) * g * r;"),
    "local-divisor": ("S / (double)d_full", "S / (double)d_local"),
    "ext-dropped": ("S += oracle_elem(edt, s_ext, e * ld_ext + t);",
                    "S += 0.0 * oracle_elem(edt, s_ext, e * ld_ext + t);"),
    "ext-wrong-index": ("S += oracle_elem(edt, s_ext, e * ld_ext + t);",
                        "S += oracle_elem(edt, s_ext, e + t * n_ext);"),
    "abs-square": ("s += v * v;", "s += fabs(v);"),
    "sign-lost": ("y[t * ldy + i] = oracle_elem(xdt, x, t * ldx + i) * g * r;\n        }\n    }\n}",
                  "y[t * ldy + i] = fabs(oracle_elem(xdt, x, t * ldx + i)) * g * r;\n        }\n    }\n}"),
    "transposed-weight": ("acc += oracle_elem(xdt, x, t * ldx + k) * oracle_elem(wdt, wf, k * ldw + n);",
                          "acc += oracle_elem(xdt, x, t * ldx + k) * oracle_elem(wdt, wf, n * ldw + k);"),
    "fold-no-gamma": ("wf[k * ldwf + n] = g * oracle_elem", "wf[k * ldwf + n] = (g - g + 1.0) * oracle_elem"),
    "rne-ties-away": ("double q = nearbyint(", "double q = round("),
    "bf16-low-half": ("<< 16;\n    float f;", "<< 15;\n    float f;"),
    "unfused-no-r": ("double xn = oracle_elem(xdt, x, t * ldx + k) * g * r;",
                     "double xn = oracle_elem(xdt, x, t * ldx + k) * g;"),
    "elim-eps-no-pre": ("(row_sumsq(xdt, x, t * ldx, K) / (double)K + eps_pre)",
                        "(row_sumsq(xdt, x, t * ldx, K) / (double)K + 0.0 * eps_pre)"),
    "elim-eps-inverted": ("eps = eps_qk * (row_sumsq", "eps = eps_qk / (row_sumsq"),
    "chain-no-prenorm": ("h[i] = oracle_elem(xdt, x, t * ldx + i) * g * r1;",
                         "h[i] = oracle_elem(xdt, x, t * ldx + i) * g + 0.0 * r1;"),
    "qk-partial-width": ("for (int64_t i = 0; i < d; ++i) s += v[i] * v[i];",
                         "for (int64_t i = 0; i < d / 2 + 1; ++i) s += v[i] * v[i];"),
    "ln-no-mean": ("double c = oracle_elem(dtype, x, off + i) - m;",
                   "double c = oracle_elem(dtype, x, off + i) - 0.0 * m;"),
    "ln-sample-variance": ("*var = v / (double)d;", "*var = v / (double)(d - 1);"),
    "ln-beta-dropped": ("double b = beta ? oracle_elem(bdt, beta, i) : 0.0;\n            y[t * ldy + i]",
                        "double b = 0.0; (void)bdt;\n            y[t * ldy + i]"),
    "deferred-no-mean-term": ("r * (acc - mu * oracle_elem(cdt, colsum, n)) + b",
                              "r * (acc - 0.0 * mu * oracle_elem(cdt, colsum, n)) + b"),
    "deferred-bias-scaled": ("r * (acc - mu * oracle_elem(cdt, colsum, n)) + b",
                             "r * (acc - mu * oracle_elem(cdt, colsum, n) + b)"),
    "colsum-transposed": ("s += oracle_elem(wdt, w, k * ldw + n);",
                          "s += oracle_elem(wdt, w, (n * K + k) % (K * N));"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    import oracle

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(ORACLE_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    (tmp_path / "oracle.c").write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-w",
                           str(tmp_path / "oracle.c"), "-o", str(so), "-lm"])
    monkeypatch.setattr(oracle, "_LIB", str(so))
    monkeypatch.setattr(oracle, "_lib", None)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(oracle)
        except AssertionError:
            failed.append(pin.__name__)
    monkeypatch.setattr(oracle, "_lib", None)
    assert failed, f"planted mistake {name} passed every pin"
