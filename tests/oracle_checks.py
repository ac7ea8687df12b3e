"""Independent checks that pin the fp64 oracle to something other than itself.

Each ``pin_*`` function takes an ``attn(q, k, v, scale, causal) -> (O, lse)``
callable on one float64 [N, D] slice and raises AssertionError when the
callable violates a fact fixed by the pages or by the mathematics of
softmax attention.  The test suite runs them on the oracle (must pass) and
on deliberately broken variants of it (each must fail at least one pin).

Facts used (cited by page title and section):
  * every row of P is a probability distribution -- KingOfEgg's
    FlashAttention v1 post, section 1.1;
  * subtracting the row maximum does not change softmax, and a tiled
    computation that keeps per-block statistics (maximum m, exp-sum l,
    unnormalised output) and rescales them by exp(m_old - m_new) when they
    are combined, dividing by l once at the end, reaches the same result as
    the materialising computation -- "08 · FlashAttention" parts 2-3;
    lesson 13 core concept 4; pwwt.cn essay section 2.2;
  * the per-step normalised merge of the original Algorithm 1 (O kept
    normalised after every key block) -- KingOfEgg's post, sections 2 and
    4.3;
  * closed forms that follow from the definition (uniform weights, one
    dominant score, a single key, linearity in V, permutation symmetry).
"""
from __future__ import annotations

import decimal
import math

import numpy as np


# --------------------------------------------------------------------------
# Independent recomputations (not the oracle's three-pass structure)
# --------------------------------------------------------------------------

def block_stats(s, vb):
    """Statistics of one block of scores s [rows, keys] over value rows vb:
    the block's row maximum m, its exp-sum l = sum_j e^(s_j - m) and the
    unnormalised output A = sum_j e^(s_j - m) v_j.  A row with no visible key
    (every score -inf) is the empty block (m, l, A) = (-inf, 0, 0)."""
    m = s.max(axis=1)
    has = np.isfinite(m)
    w = np.exp(s - np.where(has, m, 0.0)[:, None])
    w = np.where(has[:, None], w, 0.0)
    return m, w.sum(axis=1), w @ vb


def merge_stats(x, y, mutation=None):
    """Combine the statistics of two disjoint key sets.  The softmax sums over
    their union are exact sums of the two parts once both are referred to the
    common maximum m = max(m_x, m_y): l = l_x e^(m_x - m) + l_y e^(m_y - m),
    and the same factors scale A.  The operation is associative, so the key
    blocks can be combined in any grouping.  (`mutation` plants a mistake for
    the tests that must catch it.)"""
    (mx, lx, ax), (my, ly, ay) = x, y
    m = np.maximum(mx, my)
    safe = np.where(np.isfinite(m), m, 0.0)

    def factor(mp):
        if mutation == "no_rescale":
            return np.where(np.isfinite(mp), 1.0, 0.0)
        e = (safe - mp) if mutation == "flipped_exponent" else (mp - safe)
        return np.where(np.isfinite(mp), np.exp(e), 0.0)

    fx, fy = factor(mx), factor(my)
    return m, lx * fx + ly * fy, ax * fx[:, None] + ay * fy[:, None]


def blocked_tree(q, k, v, scale, causal, br, bc, mutation=None):
    """Tiled forward from per-block statistics: every (query block of br rows,
    key block of bc keys) pair is reduced to (m, l, A) on its own, the key
    blocks of a query block are combined pairwise in a balanced tree with
    merge_stats, and only then O = A / l and lse = m + ln l.  Nothing here
    runs left to right over the keys, so it checks the exactness of tiling
    without repeating the running-state recurrence.  mutation="block_softmax"
    normalises each key block on its own and averages them (lesson 13 lists
    "softmax each block and concatenate" as a disqualifying misconception)."""
    n, d = q.shape
    nk = k.shape[0]
    o = np.zeros((n, d))
    lse = np.zeros(n)
    for r0 in range(0, n, br):
        rows = np.arange(r0, min(n, r0 + br))
        parts = []
        for c0 in range(0, nk, bc):
            cols = np.arange(c0, min(nk, c0 + bc))
            s = scale * (q[rows] @ k[cols].T)
            if causal:
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            parts.append(block_stats(s, v[cols]))
        if mutation == "block_softmax":
            outs = [a / np.where(l > 0, l, 1.0)[:, None] for (_, l, a) in parts]
            o[rows] = sum(outs) / len(outs)
            lse[rows] = np.nan
            continue
        while len(parts) > 1:
            nxt = [merge_stats(parts[i], parts[i + 1], mutation) for i in range(0, len(parts) - 1, 2)]
            if len(parts) % 2:
                nxt.append(parts[-1])
            parts = nxt
        m, l, a = parts[0]
        o[rows] = a / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


def blocked_normalised(q, k, v, scale, causal, bc):
    """KV-block merge that keeps O normalised after every block (Algorithm 1 form):
    with block statistics (m~, l~) and unnormalised block output P~V,
    m_new = max(m, m~), l_new = e^(m-m_new) l + e^(m~-m_new) l~,
    O = (e^(m-m_new) l O + e^(m~-m_new) P~V) / l_new."""
    n, d = q.shape
    nk = k.shape[0]
    o = np.zeros((n, d))
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    rows = np.arange(n)
    for c0 in range(0, nk, bc):
        cols = np.arange(c0, min(nk, c0 + bc))
        s = scale * (q @ k[cols].T)
        if causal:
            s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
        mt = s.max(axis=1)
        has = np.isfinite(mt)
        mt_safe = np.where(has, mt, 0.0)
        pt = np.exp(s - mt_safe[:, None])
        lt = pt.sum(axis=1)
        m_new = np.maximum(m, mt)
        a_old = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        a_blk = np.where(has, np.exp(mt_safe - m_new), 0.0)
        l_new = a_old * l + a_blk * lt
        upd = l_new > 0
        o_new = (a_old[:, None] * l[:, None] * o + a_blk[:, None] * (pt @ v[cols]))
        o = np.where(upd[:, None], o_new / np.where(upd, l_new, 1.0)[:, None], o)
        m, l = np.where(upd, m_new, m), l_new
    return o, m + np.log(l)


def decimal_attention(q, k, v, scale, causal, prec=40):
    """Brute force in 40-digit decimal arithmetic (exact inputs, correctly
    rounded exp/ln at that precision).  Only for tiny inputs."""
    ctx = decimal.Context(prec=prec)
    D = decimal.Decimal
    n, d = q.shape
    nk = k.shape[0]
    qd = [[D(float(x)) for x in row] for row in q]
    kd = [[D(float(x)) for x in row] for row in k]
    vd = [[D(float(x)) for x in row] for row in v]
    sc = D(float(scale))
    o = np.zeros((n, d))
    lse = np.zeros(n)
    for i in range(n):
        js = range(i + 1) if causal else range(nk)
        s = {j: ctx.multiply(sc, sum((ctx.multiply(qd[i][c], kd[j][c]) for c in range(d)), D(0)))
             for j in js}
        m = max(s.values())
        e = {j: ctx.exp(ctx.subtract(s[j], m)) for j in js}
        tot = sum(e.values(), D(0))
        for c in range(d):
            o[i, c] = float(sum((ctx.multiply(ctx.divide(e[j], tot), vd[j][c]) for j in js), D(0)))
        lse[i] = float(ctx.add(m, ctx.ln(tot)))
    return o, lse


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _vis(i, n, causal):
    return np.arange(i + 1) if causal else np.arange(n)


def pin_uniform(attn):
    """scale = 0 (or identical keys): equal weights over the visible keys."""
    rng = np.random.default_rng(11)
    for causal in (False, True):
        n, d = 9, 5
        q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
        o, lse = attn(q, k, v, 0.0, causal)
        for i in range(n):
            J = _vis(i, n, causal)
            np.testing.assert_allclose(o[i], v[J].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[i] - math.log(J.size)) < 1e-13
        # identical keys: every score of row i is the same value s_i
        kk = np.repeat(_rand(rng, 1, d), n, axis=0)
        sc = 0.7
        o, lse = attn(q, kk, v, sc, causal)
        for i in range(n):
            J = _vis(i, n, causal)
            np.testing.assert_allclose(o[i], v[J].mean(axis=0), rtol=0, atol=1e-13)
            s_i = sc * float(q[i] @ kk[0])
            assert abs(lse[i] - (s_i + math.log(J.size))) < 1e-12


def pin_probabilities(attn):
    """With V = I (N = D) the output is P itself: rows are distributions, causal
    rows vanish above the diagonal, and log(P_ij / P_ij') equals the score
    difference scale * q_i . (k_j - k_j')."""
    rng = np.random.default_rng(12)
    n = d = 12
    for causal in (False, True):
        q, k = _rand(rng, n, d), _rand(rng, n, d)
        sc = 0.45
        o, _ = attn(q, k, np.eye(n), sc, causal)
        assert np.all(o >= 0.0)
        np.testing.assert_allclose(o.sum(axis=1), np.ones(n), rtol=0, atol=1e-13)
        for i in range(n):
            J = _vis(i, n, causal)
            if causal:
                assert np.all(o[i, i + 1:] == 0.0)
            for j in J:
                want = sc * float(q[i] @ (k[j] - k[J[0]]))
                got = math.log(o[i, j]) - math.log(o[i, J[0]])
                assert abs(got - want) < 1e-11, (i, j, got, want)


def pin_shift(attn):
    """Adding c to every score of row i leaves O unchanged and shifts lse by c.
    Realised through the inputs: K[:, D-1] = 1 and Q[i, D-1] += c / scale."""
    rng = np.random.default_rng(13)
    n, d, sc = 10, 6, 0.3
    for causal in (False, True):
        q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
        k[:, d - 1] = 1.0
        o0, l0 = attn(q, k, v, sc, causal)
        shift = np.linspace(-30.0, 45.0, n)
        q2 = q.copy()
        q2[:, d - 1] += shift / sc
        o1, l1 = attn(q2, k, v, sc, causal)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l1 - l0, shift, rtol=0, atol=1e-11)


def pin_one_hot(attn):
    """One score exceeding every other score of its row by >= 40 selects that value row."""
    rng = np.random.default_rng(14)
    n, d, sc = 16, 4, 0.5
    for causal in (False, True):
        q = np.zeros((n, d))
        q[:, 0] = 1.0
        k = _rand(rng, n, d, s=0.1)
        v = _rand(rng, n, d)
        i, jstar = n - 1, 5
        k[jstar, 0] = 100.0 / sc
        o, lse = attn(q, k, v, sc, causal)
        np.testing.assert_allclose(o[i], v[jstar], rtol=0, atol=1e-12)
        s_star = sc * float(q[i] @ k[jstar])
        assert abs(lse[i] - s_star) < 1e-12


def pin_single_key(attn):
    """N = 1: O = V_0 and lse = scale * q_0 . k_0; causal row 0 likewise; the last
    causal row sees every key, so it equals the non-causal last row."""
    rng = np.random.default_rng(15)
    d, sc = 7, 0.8
    q, k, v = _rand(rng, 1, d), _rand(rng, 1, d), _rand(rng, 1, d)
    for causal in (False, True):
        o, lse = attn(q, k, v, sc, causal)
        assert np.array_equal(o[0], v[0])
        assert abs(lse[0] - sc * float(q[0] @ k[0])) < 1e-14
    n = 11
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    oc, lc = attn(q, k, v, sc, True)
    on, ln = attn(q, k, v, sc, False)
    assert np.array_equal(oc[0], v[0])
    assert abs(lc[0] - sc * float(q[0] @ k[0])) < 1e-14
    np.testing.assert_allclose(oc[n - 1], on[n - 1], rtol=0, atol=1e-14)
    assert abs(lc[n - 1] - ln[n - 1]) < 1e-14


def pin_symmetry(attn):
    """Joint permutation of key/value rows (non-causal) changes nothing; a
    permutation of query rows permutes the outputs; O is linear in V; V = 1 gives 1."""
    rng = np.random.default_rng(16)
    n, d, sc = 13, 5, 0.6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attn(q, k, v, sc, False)
    perm = rng.permutation(n)
    o2, l2 = attn(q, k[perm], v[perm], sc, False)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-13)
    o3, l3 = attn(q[perm], k, v, sc, False)
    np.testing.assert_allclose(o3, o[perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l3, lse[perm], rtol=0, atol=1e-14)
    for causal in (False, True):
        v1, v2 = _rand(rng, n, d), _rand(rng, n, d)
        a, b = 1.75, -0.5
        oa, _ = attn(q, k, v1, sc, causal)
        ob, _ = attn(q, k, v2, sc, causal)
        oab, _ = attn(q, k, a * v1 + b * v2, sc, causal)
        np.testing.assert_allclose(oab, a * oa + b * ob, rtol=0, atol=1e-13)
        ones, _ = attn(q, k, np.ones((n, d)), sc, causal)
        np.testing.assert_allclose(ones, np.ones((n, d)), rtol=0, atol=1e-14)


def pin_blocked(attn):
    """The tiled forward assembled from per-block statistics (tree merge,
    deferred 1/l) and the per-step normalised merge reach the same result for
    several tile shapes, including tiles that do not divide N."""
    rng = np.random.default_rng(17)
    for (n, d) in ((100, 8), (64, 16)):
        for causal in (False, True):
            q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
            sc = 1.0 / math.sqrt(d)
            o, lse = attn(q, k, v, sc, causal)
            for (br, bc) in ((1, 1), (16, 32), (32, 16), (n, n), (7, 13)):
                ob, lb = blocked_tree(q, k, v, sc, causal, br, bc)
                np.testing.assert_allclose(ob, o, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lb, lse, rtol=0, atol=1e-12)
            for bc in (1, 32, 13):
                on, ln = blocked_normalised(q, k, v, sc, causal, bc)
                np.testing.assert_allclose(on, o, rtol=0, atol=1e-12)
                np.testing.assert_allclose(ln, lse, rtol=0, atol=1e-12)


def pin_decimal(attn):
    """Tiny inputs against 40-digit decimal brute force."""
    rng = np.random.default_rng(18)
    for (n, d) in ((1, 3), (5, 2), (7, 4)):
        for causal in (False, True):
            q, k, v = _rand(rng, n, d, s=2.0), _rand(rng, n, d, s=2.0), _rand(rng, n, d)
            sc = 0.9
            o, lse = attn(q, k, v, sc, causal)
            od, ld = decimal_attention(q, k, v, sc, causal)
            np.testing.assert_allclose(o, od, rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-14)


ALL_PINS = (pin_uniform, pin_probabilities, pin_shift, pin_one_hot, pin_single_key,
            pin_symmetry, pin_blocked, pin_decimal)
