"""CPU tests: the oracle for packed variable-length sequences, pinned.

A packed batch concatenates sequences without padding; cu_seqlens[b] is the
first row of sequence b (the interface the "08 · FlashAttention" page, part
4, recommends over padding masks).  Each sequence is an independent slice
with n_q queries and n_k keys; causal masking is aligned at the bottom right
(query i sees keys j <= i + n_k - n_q), which is the square top-left mask when
n_q = n_k.  Pins: 40-digit decimal brute force with explicit key sets, the
one-key and empty closed forms, the packing identity against the (pinned)
square oracle, and the bottom-right alignment facts (the last query sees
every key; with n_q > n_k the first n_q - n_k queries see none).  Planted
mistakes in the C routine and in the packing wrapper must each fail a pin.
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


def decimal_cross(q, k, v, scale, causal, prec=40):
    """Brute force for n_q queries against n_k keys, causal bottom-right, 40 digits;
    a row with no visible key gives (0, -inf)."""
    ctx = decimal.Context(prec=prec)
    D = decimal.Decimal
    nq, d = q.shape
    nk = k.shape[0]
    o = np.zeros((nq, d))
    lse = np.full(nq, -np.inf)
    sc = D(float(scale))
    for i in range(nq):
        js = [j for j in range(nk) if not causal or j <= i + nk - nq]
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
# pins of one slice with n_q != n_k: cross(q [nq, d], k [nk, d], v, scale, causal)
# --------------------------------------------------------------------------

def pin_cross_decimal(cross):
    rng = np.random.default_rng(71)
    for (nq, nk, d) in ((3, 7, 3), (7, 3, 2), (5, 5, 4), (1, 6, 3), (6, 1, 2)):
        q, k, v = _rand(rng, nq, d, s=1.5), _rand(rng, nk, d, s=1.5), _rand(rng, nk, d)
        for causal in (False, True):
            o, lse = cross(q, k, v, 0.7, causal)
            od, ld = decimal_cross(q, k, v, 0.7, causal)
            assert np.array_equal(lse == -np.inf, ld == -np.inf)
            fin = np.isfinite(ld)
            np.testing.assert_allclose(lse[fin], ld[fin], rtol=0, atol=1e-14)
            np.testing.assert_allclose(o, od, rtol=0, atol=1e-14)


def pin_cross_one_key(cross):
    """n_k = 1: without the mask every row is v_0 with lse = scale q_i.k_0; with the
    bottom-right mask only the last query (i = n_q - 1) sees key 0."""
    rng = np.random.default_rng(72)
    nq, d = 6, 4
    q, k, v = _rand(rng, nq, d), _rand(rng, 1, d), _rand(rng, 1, d)
    for causal in (False, True):
        o, lse = cross(q, k, v, 0.9, causal)
        for i in range(nq):
            if causal and i < nq - 1:
                assert lse[i] == -np.inf and np.all(o[i] == 0.0)
            else:
                np.testing.assert_allclose(o[i], v[0], rtol=0, atol=1e-15)
                assert abs(lse[i] - 0.9 * math.fsum(q[i, c] * k[0, c] for c in range(d))) < 1e-14


def pin_cross_alignment(cross):
    """Bottom-right alignment: with n_k >= n_q the last query sees every key (causal
    equals non-causal there) and query i sees i + n_k - n_q + 1 keys; with n_q > n_k
    the first n_q - n_k queries see none."""
    rng = np.random.default_rng(73)
    d = 3
    q, k, v = _rand(rng, 4, d), _rand(rng, 9, d), _rand(rng, 9, d)
    oc, lc = cross(q, k, v, 0.5, True)
    on, ln = cross(q, k, v, 0.5, False)
    np.testing.assert_allclose(oc[-1], on[-1], rtol=0, atol=1e-14)
    assert abs(lc[-1] - ln[-1]) < 1e-14
    # V = e_j picks out the weight of key j: keys past i + 5 get exactly 0
    q9, k9 = _rand(rng, 4, 9), _rand(rng, 9, 9)
    oe, _ = cross(q9, k9, np.eye(9), 0.5, True)
    for i in range(4):
        assert np.all(oe[i, i + 6:] == 0.0) and np.all(oe[i, :i + 6] > 0.0)
    q2, k2, v2 = _rand(rng, 8, d), _rand(rng, 3, d), _rand(rng, 3, d)
    o2, l2 = cross(q2, k2, v2, 0.5, True)
    assert np.all(l2[:5] == -np.inf) and np.all(o2[:5] == 0.0) and np.all(np.isfinite(l2[5:]))


def pin_cross_square_is_topleft(cross):
    """n_q = n_k: the bottom-right mask is the square top-left mask (pinned dense oracle)."""
    rng = np.random.default_rng(74)
    q, k, v = _rand(rng, 12, 4), _rand(rng, 12, 4), _rand(rng, 12, 4)
    for causal in (False, True):
        o, lse = cross(q, k, v, 0.6, causal)
        od, ld = oracle.attention(q, k, v, 0.6, causal)
        np.testing.assert_allclose(o, od, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-14)


CROSS_PINS = (pin_cross_decimal, pin_cross_one_key, pin_cross_alignment, pin_cross_square_is_topleft)


def oracle_cross(q, k, v, scale, causal):
    rows = np.arange(q.shape[0], dtype=np.int64)
    return oracle.attention_rows(q, k, v, rows, scale, causal, causal_offset=k.shape[0] - q.shape[0])


@pytest.mark.parametrize("pin", CROSS_PINS, ids=lambda f: f.__name__)
def test_oracle_cross_passes_pin(pin):
    pin(oracle_cross)


# --------------------------------------------------------------------------
# pins of the packing: varlen(q [H, Tq, D], k, v [H, Tk, D], cu_q, cu_k, scale, causal)
# --------------------------------------------------------------------------

def _packed(rng, H, lens_q, lens_k, d):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    q = _rand(rng, H, int(cu_q[-1]), d)
    k = _rand(rng, H, int(cu_k[-1]), d)
    v = _rand(rng, H, int(cu_k[-1]), d)
    return q, k, v, cu_q, cu_k


def pin_varlen_is_per_sequence(varlen):
    """Each packed sequence equals the decimal brute force on its own rows."""
    rng = np.random.default_rng(75)
    lens_q, lens_k = [3, 0, 5, 2], [4, 2, 5, 1]
    q, k, v, cu_q, cu_k = _packed(rng, 2, lens_q, lens_k, 3)
    for causal in (False, True):
        res = varlen(q, k, v, cu_q, cu_k, 0.8, causal)
        assert [r[0] for r in res] == [0, 1, 2, 3]
        for b, rows, o, lse in res:
            assert rows.size == lens_q[b]
            for h in range(2):
                qs = q[h, cu_q[b]:cu_q[b + 1]]
                ks, vs = k[h, cu_k[b]:cu_k[b + 1]], v[h, cu_k[b]:cu_k[b + 1]]
                od, ld = decimal_cross(qs, ks, vs, 0.8, causal)
                assert np.array_equal(lse[h] == -np.inf, ld == -np.inf)
                np.testing.assert_allclose(o[h], od, rtol=0, atol=1e-14)
                fin = np.isfinite(ld)
                np.testing.assert_allclose(lse[h][fin], ld[fin], rtol=0, atol=1e-14)


def pin_varlen_square_batch(varlen):
    """Equal-length square sequences packed head-major equal the dense [B, H, N, D]
    oracle on the same data."""
    rng = np.random.default_rng(76)
    B, H, N, d = 3, 2, 7, 4
    qd, kd, vd = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    pack = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(H, B * N, d))
    cu = np.arange(0, B * N + 1, N)
    for causal in (False, True):
        od, ld = oracle.attention(qd, kd, vd, 0.5, causal)
        for b, rows, o, lse in varlen(pack(qd), pack(kd), pack(vd), cu, cu, 0.5, causal):
            np.testing.assert_allclose(o, od[b], rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse, ld[b], rtol=0, atol=1e-14)


def pin_varlen_row_subset(varlen):
    rng = np.random.default_rng(77)
    q, k, v, cu_q, cu_k = _packed(rng, 2, [6, 9], [8, 4], 3)
    full = varlen(q, k, v, cu_q, cu_k, 0.4, True)
    part = varlen(q, k, v, cu_q, cu_k, 0.4, True, seqs=[1], rows_of=lambda b: [0, 4, 8])
    assert len(part) == 1 and part[0][0] == 1
    np.testing.assert_array_equal(part[0][2], full[1][2][:, [0, 4, 8]])


VARLEN_PINS = (pin_varlen_is_per_sequence, pin_varlen_square_batch, pin_varlen_row_subset)


@pytest.mark.parametrize("pin", VARLEN_PINS, ids=lambda f: f.__name__)
def test_oracle_varlen_passes_pin(pin):
    pin(oracle.attention_varlen)


def test_general_rejects_negative_row():
    with pytest.raises(ValueError):
        oracle.attention_rows(np.zeros((1, 2)), np.zeros((3, 2)), np.zeros((3, 2)), np.array([-1]), 1.0, True,
                              causal_offset=2)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

C_MUTATIONS = {
    "offset_ignored": [("const int64_t j_vis = i + causal_offset + 1;", "const int64_t j_vis = i + 1;")],
    "offset_sign_flipped": [("const int64_t j_vis = i + causal_offset + 1;",
                             "const int64_t j_vis = i - causal_offset + 1;")],
    "mask_excludes_diagonal": [("const int64_t j_vis = i + causal_offset + 1;",
                                "const int64_t j_vis = i + causal_offset;")],
}


def _build_c_mutant(name, tmp_path):
    src = open(_SRC).read()
    for old, new in C_MUTATIONS[name]:
        assert src.count(old) == 1, "mutation %s no longer applies to oracle.c (%r)" % (name, old)
        src = src.replace(old, new)
    cpath = tmp_path / ("oracle_%s.c" % name)
    cpath.write_text(src)
    so = tmp_path / ("liboracle_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                           str(cpath), "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    fn = lib.oracle_attention_rows_general
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                   ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]

    def cross(q, k, v, scale, causal):
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        nq, d = q.shape
        nk = k.shape[0]
        rows = np.arange(nq, dtype=np.int64)
        o = np.empty((nq, d))
        lse = np.empty(nq)
        with np.errstate(all="ignore"):
            rc = fn(q.ctypes.data, k.ctypes.data, v.ctypes.data, nk, d, rows.ctypes.data, nq, 0, nk,
                    float(scale), int(causal), nk - nq, o.ctypes.data, lse.ctypes.data, 1)
        assert rc == 0
        return o, lse
    return cross


def _caught(pins, fn):
    caught = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    return caught


@pytest.mark.parametrize("name", sorted(C_MUTATIONS))
def test_planted_cross_mistake_fails_some_pin(name, tmp_path):
    assert _caught(CROSS_PINS, _build_c_mutant(name, tmp_path)), "planted mistake %s passed every pin" % name


PY_MUTATIONS = {
    "keys_sliced_with_query_offsets": [("k[h, k0:k1], v[h, k0:k1]", "k[h, q0:q1], v[h, q0:q1]")],
    "offset_reversed": [("causal_offset=(k1 - k0) - (q1 - q0)", "causal_offset=(q1 - q0) - (k1 - k0)")],
    "offset_dropped": [("causal_offset=(k1 - k0) - (q1 - q0)", "causal_offset=0")],
    "queries_of_first_sequence": [("q[h, q0 + rows]", "q[h, rows]")],
}


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_planted_packing_mistake_fails_some_pin(name):
    src = inspect.getsource(oracle.attention_varlen)
    for old, new in PY_MUTATIONS[name]:
        assert src.count(old) == 1, "mutation %s no longer applies (%r)" % (name, old)
        src = src.replace(old, new)
    ns = {"np": np, "attention_rows": oracle.attention_rows}
    exec(compile(src, "<mutant %s>" % name, "exec"), ns)
    assert _caught(VARLEN_PINS, ns["attention_varlen"]), "planted mistake %s passed every pin" % name
