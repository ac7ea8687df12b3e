"""CPU tests: the fp64 oracle against what the pages and the mathematics fix.

Besides running every pin on the oracle, each planted mistake (a patched
copy of oracle.c compiled to a scratch library on the CPU) must fail at
least one pin, which shows the pins would catch that class of error.
"""
import ctypes
import json
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import oracle_checks as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def oracle_attn(q, k, v, scale, causal):
    return oracle.attention(q, k, v, scale, causal)


@pytest.mark.parametrize("pin", oc.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_passes_pin(pin):
    pin(oracle_attn)


# ---------------------------------------------------------------- mutations

_SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "scale_dropped": [("S[j - key_lo] = scale * dot;", "S[j - key_lo] = dot;")],
    "feature_index_reversed": [("dot += qi[c] * kj[c];", "dot += qi[c] * kj[d - 1 - c];")],
    "dot_term_dropped": [("for (int64_t c = 0; c < d; c++)\n                    dot",
                          "for (int64_t c = 0; c < d - 1; c++)\n                    dot")],
    "exp_sign_flipped": [("l += exp(S[j - key_lo] - m);", "l += exp(m - S[j - key_lo]);"),
                         ("S[j - key_lo] = exp(S[j - key_lo] - m) / l;",
                          "S[j - key_lo] = exp(m - S[j - key_lo]) / l;")],
    "not_normalised": [("S[j - key_lo] = exp(S[j - key_lo] - m) / l;",
                        "S[j - key_lo] = exp(S[j - key_lo] - m);")],
    "value_row_reversed": [("const double *vj = v + j * d;",
                            "const double *vj = v + (j_end - 1 - j + key_lo) * d;")],
    "value_column_shifted": [("oi[c] += p * vj[c];", "oi[c] += p * vj[(c + 1) % d];")],
    "causal_sees_next_key": [("const int64_t j_end = causal ? (j_vis < key_hi ? j_vis : key_hi) : key_hi;",
                              "const int64_t j_end = causal ? (j_vis + 1 < key_hi ? j_vis + 1 : key_hi) : key_hi;")],
    "lse_in_log2": [("lse_rows[r] = m + log(l);", "lse_rows[r] = m + log2(l);")],
    "lse_without_max": [("lse_rows[r] = m + log(l);", "lse_rows[r] = log(l);")],
}


def _build_mutant(name, tmp_path):
    src = open(_SRC).read()
    for old, new in MUTATIONS[name]:
        assert src.count(old) == 1, "mutation %s no longer applies to oracle.c (%r)" % (name, old)
        src = src.replace(old, new)
    cpath = tmp_path / ("oracle_%s.c" % name)
    cpath.write_text(src)
    so = tmp_path / ("liboracle_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                           str(cpath), "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int]

    def attn(q, k, v, scale, causal):
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        n, d = q.shape
        rows = np.arange(n, dtype=np.int64)
        o = np.empty((n, d))
        lse = np.empty(n)
        with np.errstate(all="ignore"):
            rc = lib.oracle_attention_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, k.shape[0], d,
                                           rows.ctypes.data, n, float(scale), int(causal),
                                           o.ctypes.data, lse.ctypes.data, 1)
        assert rc == 0
        return o, lse
    return attn


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_some_pin(name, tmp_path):
    attn = _build_mutant(name, tmp_path)
    caught = []
    for pin in oc.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %s passed every pin" % name


@pytest.mark.parametrize("mutation", ["no_rescale", "flipped_exponent", "block_softmax"])
def test_broken_merge_disagrees_with_oracle(mutation):
    """The blocked recomputation is a sensitive check: dropping the exp(m_old - m_new)
    rescale when block statistics are combined, flipping its exponent, or
    normalising each key block separately (lesson 13 lists "softmax each block and
    concatenate" as a disqualifying misconception) must all break agreement with
    the oracle."""
    rng = np.random.default_rng(21)
    n, d = 96, 16
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    sc = 1.0 / math.sqrt(d)
    o, lse = oracle_attn(q, k, v, sc, False)
    ok, _ = oc.blocked_tree(q, k, v, sc, False, 32, 32)
    assert np.abs(ok - o).max() < 1e-12
    ob, _ = oc.blocked_tree(q, k, v, sc, False, 32, 32, mutation=mutation)
    assert np.abs(ob - o).max() > 1e-3


# ------------------------------------------------------------ worked example

def test_lesson13_seeded_example():
    """Lesson 13's seeded comparison: materialised vs blocked attention agree to
    about 1e-15 (the page prints ~1e-15 and asserts allclose at 1e-6)."""
    g = json.load(open(os.path.join(GOLDEN, "p3_blocked_vs_standard.json")))["what_the_page_fixes"]
    rng = np.random.default_rng(0)
    n, d = g["n"], g["d"]
    q = rng.standard_normal((n, d)) * g["q_multiplier"]
    k = rng.standard_normal((n, d)) * g["k_multiplier"]
    v = rng.standard_normal((n, d)) * g["v_multiplier"]
    o, lse = oracle_attn(q, k, v, g["scale"], False)
    ob, lb = oc.blocked_tree(q, k, v, g["scale"], False, g["block_size"], g["block_size"])
    err = np.abs(o - ob).max()
    assert err < 1e-13, err
    assert err <= g["asserted_atol"]
    assert np.abs(lse - lb).max() < 1e-13
    assert n * n == g["printed_score_elements"]


# ------------------------------------------------------------ widening / rows

def test_widening_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    want = np.array([1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -0.0])
    got = oracle.widen(bits, "bf16")
    assert np.array_equal(got, want) and np.signbit(got[-1])
    h = np.array([1.0, 2.0 ** -24, 65504.0, -0.5], dtype=np.float16)
    assert np.array_equal(oracle.widen(h, "f16"), np.array([1.0, 2.0 ** -24, 65504.0, -0.5]))
    assert oracle.gpu_scale(1 / math.sqrt(128)) == float(np.float32(1 / math.sqrt(128)))


def test_row_subset_matches_full():
    rng = np.random.default_rng(22)
    n, d = 50, 8
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    for causal in (False, True):
        o, lse = oracle_attn(q, k, v, 0.35, causal)
        rows = np.array([0, 3, 17, 49], dtype=np.int64)
        os_, ls_ = oracle.attention_rows(q[rows], k, v, rows, 0.35, causal, n_threads=2)
        assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, lse[rows])


def test_oracle_rejects_bad_arguments():
    q = np.zeros((2, 4))
    with pytest.raises(ValueError):
        oracle.attention_rows(q, np.zeros((3, 4)), np.zeros((3, 4)), np.array([0, 5]), 1.0, False)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, np.zeros((3, 4)), np.zeros((3, 4)), np.array([0, 1]), float("nan"), False)
