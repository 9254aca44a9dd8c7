"""The oracle's pins are strong enough to catch plausible mistakes.

Each mutant below is a copy of oracle/nsa_oracle.c with one planted bug (a
dropped term, a wrong sign, an off-by-one, a transposed operand, a wrong head
map).  It is compiled on the CPU, swapped in for the real oracle, and the pin
checks of test_oracle_pins.py are run against it: at least one must fail.
"""
import contextlib
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_sink as sink_pins
import test_oracle_subsets as subset_pins
import test_oracle_window as window_pins
import test_oracle_bottom_right as br_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "nsa_oracle.c")

MUTANTS = {
    "dq drops scale": ("dq_out[d] += sh->scale * dS * kj[d];", "dq_out[d] += dS * kj[d];"),
    "dS sign": ("double dS = P[a] * (dP[a] - delta);", "double dS = P[a] * (dP[a] + delta);"),
    "causal strict": ("j < sh->Tk && j <= tp;", "j < sh->Tk && j < tp;"),
    "block start off by one": ("for (int j = u * sh->bs; j <", "for (int j = u * sh->bs + 1; j <"),
    "dk uses dO": ("dk_out[d] += sh->scale * dS * q_r[d];", "dk_out[d] += sh->scale * dS * do_r[d];"),
    "dv uses dS": ("dv_out[d] += Pj * do_r[d];", "dv_out[d] += dS * do_r[d];"),
    "dkdv skips diagonal": ("for (int t = t0 < 0 ? 0 : t0; t < sh->T; ++t)",
                            "for (int t = (t0 < 0 ? 0 : t0) + 1; t < sh->T; ++t)"),
    "delta drops P": ("delta += P[a] * dP[a];", "delta += dP[a];"),
    "head map transposed": ("int G = sh->Hq / sh->Hkv, hkv = h / G, D = sh->D;\n    const double* K",
                            "int G = sh->Hq / sh->Hkv, hkv = h % sh->Hkv, D = sh->D;\n    const double* K"),
    "lse drops log": ("double lse = m + log(sum);", "double lse = m + sum;"),
    "no scale in scores": ("P[a] = sh->scale * dot(q_r,", "P[a] = dot(q_r,"),
    "o uses k": ("const double* V = krow(sh, v, b, hkv, 0);\n    int n = selected_keys",
                 "const double* V = krow(sh, k, b, hkv, 0);\n    int n = selected_keys"),
    "sink left out of the sum": ("double sum = sh->sink ? exp(sk - m) : 0.0;", "double sum = 0.0;"),
    "sink ignored on empty rows": ("if (n == 0) return sk;", "if (n == 0) return -INFINITY;"),
    "window off by one": ("j > tp - sh->window) keys[n++] = j;", "j >= tp - sh->window) keys[n++] = j;"),
    "dkdv ignores the window": ("if (sh->window > 0 && kpos(sh, t) >= j + sh->window) break;", ";"),
    # the subset calls: a listed row / key computed as if the list were absent
    "row list ignored": ("int64_t r = rows ? rows[i] : i;", "int64_t r = i;"),
    "key list ignored": ("int64_t r = keys ? keys[i] : i;", "int64_t r = i;"),
    "bottom-right offset dropped": ("static int kpos(const shape_t* sh, int t) { return t + (sh->Tk - sh->T); }",
                                    "static int kpos(const shape_t* sh, int t) { return t; }"),
    "dkdv rows start at the key": ("int t0 = j - (sh->Tk - sh->T);", "int t0 = j;"),
    "keys capped at the query count": ("j < sh->Tk && j <= tp;", "j < sh->T && j <= tp;"),
}


@contextlib.contextmanager
def _swapped(lib_path):
    saved = oracle._lib
    oracle._lib = None
    real = oracle._LIB_PATH
    real_src = oracle._SRC
    try:
        oracle._LIB_PATH = lib_path
        oracle._SRC = lib_path  # mtime check passes: the library is its own source
        yield
    finally:
        oracle._LIB_PATH = real
        oracle._SRC = real_src
        oracle._lib = saved


CHECKS = [
    lambda: pins.test_finite_differences(pins.TINY[0]),
    lambda: pins.test_finite_differences(pins.TINY[1]),
    lambda: pins.test_dense_masked_autograd(11, 2, 4, 2, 40, 8, 4, 5),
    lambda: pins.test_full_selection_is_causal_sdpa(2, 4, 1, 48, 16, 8),
    lambda: pins.test_gqa_equals_sum_over_heads(),
    lambda: pins.test_closed_forms(),
    lambda: pins.test_rows_sum_to_one_and_invariants(),
    lambda: sink_pins.test_sink_finite_differences(pins.TINY[0]),
    lambda: sink_pins.test_sink_dense_autograd(21, 2, 4, 2, 40, 8, 4, 5),
    lambda: sink_pins.test_sink_closed_forms_and_empty_rows(),
    lambda: window_pins.test_window_finite_differences(window_pins.WTINY[0]),
    lambda: window_pins.test_window_dense_autograd(41, 2, 4, 2, 40, 8, 4, 5, 7),
    lambda: subset_pins.test_row_and_key_subsets_equal_full_call(),
    lambda: subset_pins.test_packed_batch_equals_block_diagonal_autograd(subset_pins.PACKED[0]),
    lambda: br_pins.test_bottom_right_dense_autograd(*br_pins.BR_CASES[0]),
    lambda: br_pins.test_bottom_right_finite_differences(),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {name}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", lib,
                    str(path), "-lm"], check=True)
    caught = []
    with _swapped(lib):
        for i, check in enumerate(CHECKS):
            try:
                check()
            except AssertionError:
                caught.append(i)
    assert caught, f"no pin caught mutant {name!r}"


def test_unmutated_oracle_passes_all_checks():
    for check in CHECKS:
        check()
