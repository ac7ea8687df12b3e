"""CPU tests: the oracle's key-split partials and its lse merge, pinned.

A key split restricts every query row to the keys of one range [lo, hi);
the partial result is the plain definition over that set (an empty set
gives lse = -inf, O = 0).  The merge recombines partials of disjoint key
sets with the online-softmax merge step (KingOfEgg's FlashAttention v1
post, section 4.3: running maximum, exp(m_old - m_new) rescale of the old
sum and output, new block added).  The pins below fix both to facts that do
not come from the oracle itself: 40-digit decimal brute force, closed forms
(a single key, an empty range, equal parts, a hand-worked two-part merge)
and the union identity (merging the partials of a partition of the keys
gives the full result, itself pinned in test_oracle_pins.py).  Each planted
mistake must fail at least one pin.
"""
import ctypes
import decimal
import inspect
import math
import os
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def decimal_partial(q, k, v, scale, causal, lo, hi, prec=40):
    """Brute force over keys lo <= j < hi (and j <= i when causal) in 40-digit
    decimal arithmetic; an empty key set gives (0, -inf)."""
    ctx = decimal.Context(prec=prec)
    D = decimal.Decimal
    n, d = q.shape
    o = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    sc = D(float(scale))
    for i in range(n):
        js = [j for j in range(lo, hi) if not causal or j <= i]
        if not js:
            continue
        s = {j: ctx.multiply(sc, sum((ctx.multiply(D(float(q[i, c])), D(float(k[j, c])))
                                      for c in range(d)), D(0))) for j in js}
        m = max(s.values())
        e = {j: ctx.exp(ctx.subtract(s[j], m)) for j in js}
        tot = sum(e.values(), D(0))
        for c in range(d):
            o[i, c] = float(sum((ctx.multiply(ctx.divide(e[j], tot), D(float(v[j, c]))) for j in js), D(0)))
        lse[i] = float(ctx.add(m, ctx.ln(tot)))
    return o, lse


# --------------------------------------------------------------------------
# pins of the partial (key-range) result: part(q, k, v, scale, causal, lo, hi)
# --------------------------------------------------------------------------

def pin_partial_decimal(part):
    rng = np.random.default_rng(31)
    for (n, d, lo, hi) in ((6, 3, 2, 5), (7, 2, 0, 3), (5, 4, 4, 5), (6, 3, 1, 6)):
        q, k, v = _rand(rng, n, d, s=1.5), _rand(rng, n, d, s=1.5), _rand(rng, n, d)
        for causal in (False, True):
            o, lse = part(q, k, v, 0.8, causal, lo, hi)
            od, ld = decimal_partial(q, k, v, 0.8, causal, lo, hi)
            assert np.array_equal(np.isinf(lse), np.isinf(ld))
            fin = np.isfinite(ld)
            np.testing.assert_allclose(lse[fin], ld[fin], rtol=0, atol=1e-14)
            np.testing.assert_allclose(o, od, rtol=0, atol=1e-14)


def pin_partial_single_key(part):
    """Range [j, j+1): a visible row's weights are all on key j, so O_i = v_j and
    lse_i = scale * q_i . k_j; rows that cannot see key j (causal, i < j) are empty."""
    rng = np.random.default_rng(32)
    n, d = 9, 5
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    for j in (0, 4, 8):
        for causal in (False, True):
            o, lse = part(q, k, v, 0.6, causal, j, j + 1)
            for i in range(n):
                if causal and i < j:
                    assert lse[i] == -np.inf and np.all(o[i] == 0.0)
                else:
                    np.testing.assert_allclose(o[i], v[j], rtol=0, atol=1e-15)
                    want = 0.6 * math.fsum(q[i, c] * k[j, c] for c in range(d))
                    assert abs(lse[i] - want) < 1e-14


def pin_partial_empty(part):
    rng = np.random.default_rng(33)
    n, d = 6, 3
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    for causal in (False, True):
        o, lse = part(q, k, v, 1.0, causal, 3, 3)
        assert np.all(lse == -np.inf) and np.all(o == 0.0)


def pin_partial_union(part):
    """Merging the partials of a partition of the keys gives the full result."""
    rng = np.random.default_rng(34)
    n, d = 40, 6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = oracle.attention(q, k, v, 0.4, False)
    oc, lc = oracle.attention(q, k, v, 0.4, True)
    for cuts in ((0, 40), (0, 16, 40), (0, 1, 17, 17, 39, 40), (0, 13, 26, 39, 40)):
        for causal, (ow, lw) in ((False, (o, lse)), (True, (oc, lc))):
            parts = [part(q, k, v, 0.4, causal, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
            mo, ml = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            np.testing.assert_allclose(mo, ow, rtol=0, atol=1e-12)
            np.testing.assert_allclose(ml, lw, rtol=0, atol=1e-12)


PARTIAL_PINS = (pin_partial_decimal, pin_partial_single_key, pin_partial_empty, pin_partial_union)


def oracle_partial(q, k, v, scale, causal, lo, hi):
    return oracle.attention(q, k, v, scale, causal, key_range=(lo, hi))


@pytest.mark.parametrize("pin", PARTIAL_PINS, ids=lambda f: f.__name__)
def test_oracle_partial_passes_pin(pin):
    pin(oracle_partial)


# --------------------------------------------------------------------------
# pins of the merge: merge(part_o [P, ..., D], part_lse [P, ...]) -> (O, lse)
# --------------------------------------------------------------------------

def pin_merge_hand_example(merge):
    """lse = (0, ln 3): the weights are e^0 : e^(ln 3) = 1 : 3, so O = O_0/4 + 3 O_1/4
    and lse = ln(1 + 3) = ln 4."""
    po = np.array([[[1.0, -2.0, 4.0]], [[5.0, 2.0, 0.0]]])
    pl = np.array([[0.0], [math.log(3.0)]])
    o, lse = merge(po, pl)
    np.testing.assert_allclose(o, [[0.25 * 1 + 0.75 * 5, 0.25 * -2 + 0.75 * 2, 0.25 * 4]], rtol=0, atol=1e-15)
    assert abs(lse[0] - math.log(4.0)) < 1e-15


def pin_merge_equal_parts(merge):
    """P parts with the same lse and the same O: O unchanged, lse + ln P."""
    rng = np.random.default_rng(35)
    for P in (1, 2, 5):
        o1, l1 = rng.standard_normal((3, 4)), rng.standard_normal(3) * 3
        o, lse = merge(np.stack([o1] * P), np.stack([l1] * P))
        np.testing.assert_allclose(o, o1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, l1 + math.log(P), rtol=0, atol=1e-14)


def pin_merge_empty_parts(merge):
    """A part with lse = -inf has no key: it adds nothing, and its O is not read
    (NaN there must not leak).  A row whose parts are all empty stays empty."""
    o1 = np.array([[1.0, 2.0], [3.0, 4.0]])
    po = np.stack([o1, np.full((2, 2), np.nan)])
    pl = np.array([[0.5, -np.inf], [-np.inf, -np.inf]])
    with np.errstate(invalid="ignore"):
        o, lse = merge(po, pl)
    np.testing.assert_array_equal(o[0], o1[0])
    assert lse[0] == 0.5
    assert lse[1] == -np.inf and np.all(o[1] == 0.0)


def pin_merge_far_apart(merge):
    """Parts whose lse differ by far more than fp64 exp can span: the larger one
    takes all the weight (and the smaller one underflows to nothing)."""
    po = np.array([[[2.0, -1.0]], [[7.0, 7.0]]])
    pl = np.array([[900.0], [-900.0]])
    o, lse = merge(po, pl)
    np.testing.assert_array_equal(o, [[2.0, -1.0]])
    assert lse[0] == 900.0


def pin_merge_permutation(merge):
    rng = np.random.default_rng(36)
    po, pl = rng.standard_normal((4, 5, 3)), rng.standard_normal((4, 5)) * 4
    o, lse = merge(po, pl)
    perm = [2, 0, 3, 1]
    o2, l2 = merge(po[perm], pl[perm])
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-14)


def pin_merge_union(merge):
    """Partials of a partition of the keys, merged, give the full result."""
    rng = np.random.default_rng(37)
    q, k, v = _rand(rng, 2, 33, 8), _rand(rng, 2, 33, 8), _rand(rng, 2, 33, 8)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.5, causal)
        cuts = (0, 7, 8, 20, 33)
        parts = [oracle.attention(q, k, v, 0.5, causal, key_range=(a, b)) for a, b in zip(cuts[:-1], cuts[1:])]
        with np.errstate(invalid="ignore"):
            mo, ml = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        np.testing.assert_allclose(mo, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)


MERGE_PINS = (pin_merge_hand_example, pin_merge_equal_parts, pin_merge_empty_parts,
              pin_merge_far_apart, pin_merge_permutation, pin_merge_union)


@pytest.mark.parametrize("pin", MERGE_PINS, ids=lambda f: f.__name__)
def test_oracle_merge_passes_pin(pin):
    pin(oracle.lse_merge)


def test_merge_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        oracle.lse_merge(np.zeros((2, 3, 4)), np.zeros((2, 4)))


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

PARTIAL_MUTATIONS = {
    "value_index_relative_to_range": [("const double *vj = v + j * d;",
                                       "const double *vj = v + (j - key_lo) * d;")],
    "key_index_relative_to_range": [("const double *kj = k + j * d;",
                                     "const double *kj = k + (j - key_lo) * d;")],
    "causal_range_drops_diagonal": [("const int64_t j_end = causal ? (j_vis < key_hi ? j_vis : key_hi) : key_hi;",
                                     "const int64_t j_end = causal ? (j_vis - 1 < key_hi ? j_vis - 1 : key_hi) : key_hi;")],
    "range_ignores_upper_end": [("const int64_t j_end = causal ? (j_vis < key_hi ? j_vis : key_hi) : key_hi;",
                                 "const int64_t j_end = causal ? j_vis : n_keys;")],
}


def _build_partial_mutant(name, tmp_path):
    src = open(_SRC).read()
    for old, new in PARTIAL_MUTATIONS[name]:
        assert src.count(old) == 1, "mutation %s no longer applies to oracle.c (%r)" % (name, old)
        src = src.replace(old, new)
    cpath = tmp_path / ("oracle_%s.c" % name)
    cpath.write_text(src)
    so = tmp_path / ("liboracle_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                           str(cpath), "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    fn = lib.oracle_attention_rows_range
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]

    def part(q, k, v, scale, causal, lo, hi):
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        n, d = q.shape
        rows = np.arange(n, dtype=np.int64)
        o = np.empty((n, d))
        lse = np.empty(n)
        with np.errstate(all="ignore"):
            rc = fn(q.ctypes.data, k.ctypes.data, v.ctypes.data, k.shape[0], d, rows.ctypes.data, n,
                    lo, hi, float(scale), int(causal), o.ctypes.data, lse.ctypes.data, 1)
        assert rc == 0
        return o, lse
    return part


def _caught(pins, fn):
    caught = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    return caught


@pytest.mark.parametrize("name", sorted(PARTIAL_MUTATIONS))
def test_planted_partial_mistake_fails_some_pin(name, tmp_path):
    part = _build_partial_mutant(name, tmp_path)
    assert _caught(PARTIAL_PINS, part), "planted mistake %s passed every pin" % name


MERGE_MUTATIONS = {
    "weight_sign_flipped": [("np.exp(part_lse - m_safe)", "np.exp(m_safe - part_lse)")],
    "not_divided_by_l": [("contrib.sum(axis=0) / np.where(empty, 1.0, l)[..., None]", "contrib.sum(axis=0)")],
    "lse_without_max": [("m_safe + np.log(np.where(empty, 1.0, l))", "np.log(np.where(empty, 1.0, l))")],
    "plain_average": [("w[..., None] * np.nan_to_num(part_o)", "np.nan_to_num(part_o) / part_o.shape[0]")],
    "no_max_shift": [("m = part_lse.max(axis=0)", "m = np.zeros(part_lse.shape[1:])")],
    "lse_in_log2": [("m_safe + np.log(np.where(empty, 1.0, l))", "m_safe + np.log2(np.where(empty, 1.0, l))")],
}


@pytest.mark.parametrize("name", sorted(MERGE_MUTATIONS))
def test_planted_merge_mistake_fails_some_pin(name):
    src = inspect.getsource(oracle.lse_merge)
    for old, new in MERGE_MUTATIONS[name]:
        assert src.count(old) == 1, "mutation %s no longer applies to lse_merge (%r)" % (name, old)
        src = src.replace(old, new)
    ns = {"np": np}
    exec(compile(src, "<mutant %s>" % name, "exec"), ns)
    assert _caught(MERGE_PINS, ns["lse_merge"]), "planted mistake %s passed every pin" % name
