"""CPU tests: the oracle's backward pass (dQ, dK, dV), pinned.

The gradient is the derivative of the forward definition, so its strongest
pin is the forward oracle itself (pinned in test_oracle_pins.py): central
finite differences of L = sum(dO * O(Q, K, V)) in fp64 for every input
element on tiny slices.  Closed forms add exact checks (identical V rows,
N = 1, scale = 0, the column sums of dV and dK), and an independent
vectorised numpy form builds each row's softmax Jacobian diag(p) - p p^T
explicitly.  Planted mistakes in the C routine must each fail a pin.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def loss(q, k, v, dout, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(dout * o))


def pin_finite_differences(bwd):
    rng = np.random.default_rng(81)
    h = 1e-5
    for (n, d, causal) in ((5, 3, False), (6, 2, True), (4, 4, True)):
        q, k, v, do = (_rand(rng, n, d) for _ in range(4))
        dq, dk, dv = bwd(q, k, v, do, 0.7, causal)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = {"q": q, "k": k, "v": v}
                args_p[name], args_m[name] = xp, xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"], do, 0.7, causal)
                            - loss(args_m["q"], args_m["k"], args_m["v"], do, 0.7, causal)) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=0, atol=1e-8, err_msg="d%s" % name)


def pin_identical_values(bwd):
    """All V rows equal: O is that row whatever the weights, so dQ = dK = 0 and
    dV_j = sum_i P_ij dO_i still sums to sum_i dO_i."""
    rng = np.random.default_rng(82)
    n, d = 7, 3
    q, k, do = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    v = np.tile(_rand(rng, 1, d), (n, 1))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.9, causal)
        assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-13)


def pin_column_sums(bwd):
    """Rows of P sum to 1, so sum_j dV_j = sum_i dO_i; rows of dS sum to 0, so
    sum_j dK_j = 0."""
    rng = np.random.default_rng(83)
    n, d = 9, 4
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-13)


def pin_trivial(bwd):
    """N = 1: O = v_0, so dV = dO and dQ = dK = 0.  scale = 0: uniform weights over
    the visible keys, dQ = dK = 0 and dV_j = sum over rows i that see j of dO_i / |J(i)|."""
    rng = np.random.default_rng(84)
    q, k, v, do = (_rand(rng, 1, 3) for _ in range(4))
    dq, dk, dv = bwd(q, k, v, do, 1.3, False)
    assert np.all(dq == 0) and np.all(dk == 0) and np.array_equal(dv, do)
    n, d = 5, 2
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.0, causal)
        assert np.all(dq == 0) and np.all(dk == 0)
        want = np.zeros((n, d))
        for i in range(n):
            vis = range(i + 1) if causal else range(n)
            for j in vis:
                want[j] += do[i] / len(vis)
        np.testing.assert_allclose(dv, want, rtol=0, atol=1e-15)


def pin_jacobian_form(bwd):
    """Vectorised numpy: P from a masked softmax, dS_i = J_i dP_i with the explicit
    Jacobian J_i = diag(p_i) - p_i p_i^T."""
    rng = np.random.default_rng(85)
    n, d = 11, 5
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    for causal in (False, True):
        s = 0.6 * (q @ k.T)
        if causal:
            s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = do @ v.T
        ds = np.stack([(np.diag(p[i]) - np.outer(p[i], p[i])) @ dp[i] for i in range(n)])
        dq, dk, dv = bwd(q, k, v, do, 0.6, causal)
        np.testing.assert_allclose(dv, p.T @ do, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dq, 0.6 * ds @ k, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, 0.6 * ds.T @ q, rtol=0, atol=1e-13)


BWD_PINS = (pin_finite_differences, pin_identical_values, pin_column_sums, pin_trivial, pin_jacobian_form)


def oracle_bwd(q, k, v, do, scale, causal):
    return oracle.attention_bwd(q, k, v, do, scale, causal)


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda f: f.__name__)
def test_oracle_bwd_passes_pin(pin):
    pin(oracle_bwd)


def test_bwd_batched_shapes():
    rng = np.random.default_rng(86)
    q, k, v, do = (_rand(rng, 2, 3, 6, 4) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.4, True)
    for b in range(2):
        for h in range(3):
            one = oracle.attention_bwd(q[b, h], k[b, h], v[b, h], do[b, h], 0.4, True)
            for x, y in zip((dq, dk, dv), one):
                np.testing.assert_array_equal(x[b, h], y)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, k, v[..., :3], do, 0.4, True)


MUTATIONS = {
    "no_delta": [("dSi[j] = Pi[j] * (dSi[j] - delta);", "dSi[j] = Pi[j] * dSi[j];")],
    "delta_sign": [("dSi[j] = Pi[j] * (dSi[j] - delta);", "dSi[j] = Pi[j] * (dSi[j] + delta);")],
    "dk_untransposed": [("ak += dS[i * n + j] * q[i * d + c];", "ak += dS[j * n + i] * q[i * d + c];")],
    "dq_without_scale": [("dq[i * d + c] = scale * acc;", "dq[i * d + c] = acc;")],
    "dv_from_ds": [("av += P[i * n + j] * dout[i * d + c];", "av += dS[i * n + j] * dout[i * d + c];")],
    "dq_uses_values": [("acc += dSi[j] * k[j * d + c];", "acc += dSi[j] * v[j * d + c];")],
    "backward_ignores_mask": [("const int64_t n_vis = causal ? i + 1 : n;\n        for (int64_t j = 0; j < n; j++) {\n            if (j >= n_vis) {",
                               "const int64_t n_vis = n;\n        for (int64_t j = 0; j < n; j++) {\n            if (j >= n_vis) {")],
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
    fn = lib.oracle_attention_bwd
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int] + \
                  [ctypes.c_void_p] * 3 + [ctypes.c_int]

    def bwd(q, k, v, do, scale, causal):
        arrs = [np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, do)]
        n, d = arrs[0].shape
        outs = [np.empty((n, d)) for _ in range(3)]
        with np.errstate(all="ignore"):
            rc = fn(*(a.ctypes.data for a in arrs), n, d, float(scale), int(causal),
                    *(o.ctypes.data for o in outs), 1)
        assert rc == 0
        return tuple(outs)
    return bwd


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_bwd_mistake_fails_some_pin(name, tmp_path):
    bwd = _build_mutant(name, tmp_path)
    caught = []
    for pin in BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %s passed every pin" % name
