"""Pins of the fp64 oracle: each check raises AssertionError when the oracle
disagrees with exact arithmetic, a closed form or an invariant.

They are plain functions so that ``test_oracle_pins.py`` runs them against the
oracle and ``test_oracle_mutations.py`` runs them against deliberately broken
copies of it (a mutation must make at least one pin fail).
"""
from __future__ import annotations

import math
from decimal import Decimal
from fractions import Fraction

import numpy as np

import exact as X


def _bf16_values(rng, shape, scale=1.0):
    """Random bf16-representable float64 values (8 significant bits)."""
    z = rng.standard_normal(shape) * scale
    m, e = np.frexp(z)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def _close_dec(got, want, rtol=1e-13, atol=1e-15):
    got = float(got)
    want = float(want)
    assert abs(got - want) <= atol + rtol * abs(want), (got, want)


# --------------------------------------------------------------------------- storage

def pin_round_bf16(o):
    one = 1.0
    # ties go to the even neighbour
    assert o.round_bf16(np.array([one + 2.0 ** -8]))[0] == one
    assert o.round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6
    assert o.round_bf16(np.array([-(one + 2.0 ** -8)]))[0] == -one
    # just above a tie rounds up
    assert o.round_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 2.0 ** -7
    # random values over a wide exponent range, against exact rational rounding
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(300),
        rng.standard_normal(100) * 1e-3,
        rng.standard_normal(100) * 1e30,
        rng.standard_normal(50) * 2.0 ** -128,      # bf16 subnormal range
        np.array([0.0, 2.0 ** -126, 2.0 ** -133, 1.5 * 2.0 ** -133, 3.0e38]),
    ])
    got = o.round_bf16(vals)
    for v, g in zip(vals, got):
        want = X.round_bf16_exact(Fraction(float(v)))
        assert Fraction(float(g)) == want, (v, g, float(want))


def pin_widen_bf16(o):
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, (2.0 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133]
    got = o.widen_bf16(bits)
    assert list(got) == want, (got, want)


# --------------------------------------------------------------------------- GEMM and stage 1

def pin_matmul_exact(o):
    rng = np.random.default_rng(1)
    for (m, k, n) in [(4, 4, 4), (3, 5, 2), (1, 7, 1), (5, 1, 3), (2, 3, 6)]:
        A = _bf16_values(rng, (m, k))
        B = _bf16_values(rng, (k, n))
        P = o.matmul(A, B)
        assert P.shape == (m, n)
        E = X.mm(X.mat(A), X.mat(B))
        for i in range(m):
            for j in range(n):
                mag = sum((abs(X.F(A[i, p]) * X.F(B[p, j])) for p in range(k)), Fraction(0))
                bound = k * 2.0 ** -52 * float(mag)
                assert abs(Fraction(float(P[i, j])) - E[i][j]) <= Fraction(bound), (m, k, n, i, j)
    # K = 1: the outer product, exactly
    a = _bf16_values(rng, (6, 1))
    b = _bf16_values(rng, (1, 5))
    assert np.array_equal(o.matmul(a, b), a[:, 0][:, None] * b[0][None, :])


def pin_stage1_exact(o):
    rng = np.random.default_rng(2)
    m, k, n = 3, 4, 5
    A = _bf16_values(rng, (m, k))
    B = _bf16_values(rng, (k, n))
    bias = _bf16_values(rng, (n,))
    R = _bf16_values(rng, (m, n))
    alpha = 0.375
    P = o.matmul(A, B)
    for act in ("none", "relu"):
        Y = o.elementwise_stage(P, alpha, bias, R, act)
        E = X.mm(X.mat(A), X.mat(B))
        for i in range(m):
            for j in range(n):
                v = Fraction(alpha) * E[i][j] + X.F(bias[j]) + X.F(R[i, j])
                if act == "relu" and v < 0:
                    v = Fraction(0)
                assert abs(Fraction(float(Y[i, j])) - v) <= Fraction(1, 2 ** 48), (act, i, j)


# --------------------------------------------------------------------------- row operations

def pin_softmax(o):
    rng = np.random.default_rng(3)
    Xm = rng.standard_normal((6, 9)) * 3
    Y = o.row_softmax(Xm)
    assert np.all(np.abs(Y.sum(-1) - 1) <= 9 * 1e-15)
    # invariant to a per-row shift
    assert np.allclose(o.row_softmax(Xm + rng.standard_normal((6, 1)) * 50), Y, rtol=1e-12, atol=0)
    # constant row -> 1/N
    assert np.allclose(o.row_softmax(np.full((2, 7), 3.25)), 1.0 / 7, rtol=1e-15, atol=0)
    # two columns -> logistic of the difference
    a, b = 1.3, -0.4
    y = o.row_softmax(np.array([[a, b]]))[0]
    assert math.isclose(y[0], 1 / (1 + math.exp(b - a)), rel_tol=1e-15)
    assert math.isclose(y[1], 1 / (1 + math.exp(a - b)), rel_tol=1e-15)
    # large logits must not overflow (max subtraction)
    big = np.array([[1000.0, 999.0, 990.0]])
    yb = o.row_softmax(big)
    want = X.softmax_row([Fraction(v) for v in big[0]])
    for g, w in zip(yb[0], want):
        _close_dec(g, w)
    # 40-digit brute force on a 4x5 block
    Z = rng.standard_normal((4, 5)) * 2
    YZ = o.row_softmax(Z)
    for i in range(4):
        for g, w in zip(YZ[i], X.softmax_row([X.F(v) for v in Z[i]])):
            _close_dec(g, w)


def pin_layernorm(o):
    rng = np.random.default_rng(4)
    Xm = rng.standard_normal((5, 8)) * 2 + 3
    for eps in (1e-5, 0.5):
        Y = o.layer_norm(Xm, None, None, eps)
        assert np.all(np.abs(Y.mean(-1)) <= 1e-14)
        for i in range(5):
            xs = [X.F(v) for v in Xm[i]]
            mu = sum(xs, Fraction(0)) / len(xs)
            var = sum(((x - mu) ** 2 for x in xs), Fraction(0)) / len(xs)
            want = float(var / (var + X.F(eps)))        # variance after normalising
            got = float(np.mean(Y[i] ** 2))
            assert math.isclose(got, want, rel_tol=1e-13), (eps, got, want)
    gamma = rng.standard_normal(8)
    beta = rng.standard_normal(8)
    # constant row -> beta
    Yc = o.layer_norm(np.full((2, 8), -4.5), gamma, beta, 1e-5)
    assert np.allclose(Yc, beta[None, :], rtol=0, atol=1e-15)
    # [a, -a] -> [-1, 1] * a / sqrt(a^2 + eps) * gamma + beta
    a, eps = 0.75, 0.01
    y2 = o.layer_norm(np.array([[-a, a]]), gamma[:2], beta[:2], eps)[0]
    s = a / math.sqrt(a * a + eps)
    assert math.isclose(y2[0], -s * gamma[0] + beta[0], rel_tol=1e-14)
    assert math.isclose(y2[1], s * gamma[1] + beta[1], rel_tol=1e-14)
    # 40-digit brute force with the affine step
    Z = rng.standard_normal((3, 6))
    g6, b6 = gamma[:6], beta[:6]
    YZ = o.layer_norm(Z, g6, b6, 1e-5)
    for i in range(3):
        for g, w in zip(YZ[i], X.layernorm_row([X.F(v) for v in Z[i]], 1e-5, g6, b6)):
            _close_dec(g, w, rtol=1e-12, atol=1e-14)


def pin_rmsnorm(o):
    rng = np.random.default_rng(5)
    Xm = rng.standard_normal((5, 8)) * 1.7
    for eps in (1e-6, 0.25):
        Y = o.rms_norm(Xm, None, eps)
        for i in range(5):
            xs = [X.F(v) for v in Xm[i]]
            ms = sum((x * x for x in xs), Fraction(0)) / len(xs)
            want = float(ms / (ms + X.F(eps)))
            assert math.isclose(float(np.mean(Y[i] ** 2)), want, rel_tol=1e-13)
    w = rng.standard_normal(8)
    c, eps = -1.25, 1e-3
    Yc = o.rms_norm(np.full((1, 8), c), w, eps)[0]
    assert np.allclose(Yc, c / math.sqrt(c * c + eps) * w, rtol=1e-14, atol=0)
    Z = rng.standard_normal((3, 7))
    YZ = o.rms_norm(Z, w[:7], 1e-6)
    for i in range(3):
        for g, ww in zip(YZ[i], X.rmsnorm_row([X.F(v) for v in Z[i]], 1e-6, w[:7])):
            _close_dec(g, ww, rtol=1e-12, atol=1e-14)


def pin_gemm_epilogue_composition(o):
    """Every row operation composed with bias + residual + ReLU, against brute force."""
    rng = np.random.default_rng(6)
    m, k, n = 3, 4, 6
    A = _bf16_values(rng, (m, k))
    B = _bf16_values(rng, (k, n))
    bias = _bf16_values(rng, (n,))
    R = _bf16_values(rng, (m, n))
    g = 1 + 0.1 * _bf16_values(rng, (n,))
    be = 0.1 * _bf16_values(rng, (n,))
    alpha = 1.5
    E = X.mm(X.mat(A), X.mat(B))
    Xf = [[max(Fraction(alpha) * E[i][j] + X.F(bias[j]) + X.F(R[i, j]), Fraction(0))
           for j in range(n)] for i in range(m)]
    for row_op in ("none", "softmax", "layernorm", "rmsnorm"):
        Y = o.gemm_epilogue(A, B, alpha=alpha, bias=bias, residual=R, act="relu",
                            row_op=row_op, gamma=g, beta=be, eps=1e-5)
        for i in range(m):
            if row_op == "none":
                want = [X.D(v) for v in Xf[i]]
            elif row_op == "softmax":
                want = X.softmax_row(Xf[i])
            elif row_op == "layernorm":
                want = X.layernorm_row(Xf[i], 1e-5, g, be)
            else:
                want = X.rmsnorm_row(Xf[i], 1e-5, g)
            for gv, wv in zip(Y[i], want):
                _close_dec(gv, wv, rtol=1e-12, atol=1e-13)


def pin_two_outputs(o):
    """(Y, X) of the two-sink epilogue against brute force: X is the elementwise
    stage (exact rationals), Y the row operation of that X (40-digit decimals)."""
    rng = np.random.default_rng(11)
    m, k, n = 3, 5, 4
    A = _bf16_values(rng, (m, k))
    B = _bf16_values(rng, (k, n))
    bias = _bf16_values(rng, (n,))
    R = _bf16_values(rng, (m, n))
    g = 1 + 0.1 * _bf16_values(rng, (n,))
    be = 0.1 * _bf16_values(rng, (n,))
    alpha = 0.75
    E = X.mm(X.mat(A), X.mat(B))
    for act in ("none", "relu"):
        Xf = [[Fraction(alpha) * E[i][j] + X.F(bias[j]) + X.F(R[i, j]) for j in range(n)] for i in range(m)]
        if act == "relu":
            Xf = [[max(v, Fraction(0)) for v in row] for row in Xf]
        for row_op in ("none", "softmax", "layernorm", "rmsnorm"):
            Y, Xo = o.gemm_epilogue_with_x(A, B, alpha=alpha, bias=bias, residual=R, act=act,
                                           row_op=row_op, gamma=g, beta=be, eps=1e-5)
            for i in range(m):
                for j in range(n):
                    assert abs(Fraction(float(Xo[i, j])) - Xf[i][j]) <= Fraction(1, 2 ** 48), (act, row_op, i, j)
                if row_op == "none":
                    want = [X.D(v) for v in Xf[i]]
                elif row_op == "softmax":
                    want = X.softmax_row(Xf[i])
                elif row_op == "layernorm":
                    want = X.layernorm_row(Xf[i], 1e-5, g, be)
                else:
                    want = X.rmsnorm_row(Xf[i], 1e-5, g)
                for gv, wv in zip(Y[i], want):
                    _close_dec(gv, wv, rtol=1e-12, atol=1e-13)


def pin_two_stage(o):
    """Two row operations in sequence against brute force (stage 1 and stage 2
    in 40-digit decimals, stage 2 on stage 1's decimal output) for all nine
    (softmax, LayerNorm, RMSNorm) pairs, each with its own affine vectors and
    eps; then closed forms of the compositions on random rows."""
    rng = np.random.default_rng(29)
    m, k, n = 3, 4, 5
    A = _bf16_values(rng, (m, k))
    B = _bf16_values(rng, (k, n))
    bias = _bf16_values(rng, (n,))
    g1, b1 = 1 + 0.1 * _bf16_values(rng, (n,)), 0.1 * _bf16_values(rng, (n,))
    g2, b2 = 1 + 0.2 * _bf16_values(rng, (n,)), 0.2 * _bf16_values(rng, (n,))
    E = X.mm(X.mat(A), X.mat(B))
    Xf = [[Fraction(0.5) * E[i][j] + X.F(bias[j]) for j in range(n)] for i in range(m)]

    def stage(xs_frac, op, g, b, eps):
        if op == "softmax":
            return X.softmax_row(xs_frac)
        if op == "layernorm":
            return X.layernorm_row(xs_frac, eps, g, b)
        return X.rmsnorm_row(xs_frac, eps, g)

    ops = ("softmax", "layernorm", "rmsnorm")
    for op1 in ops:
        for op2 in ops:
            Z = o.gemm_epilogue_two_stage(A, B, alpha=0.5, bias=bias, row_op=op1, gamma=g1, beta=b1, eps=1e-3,
                                          row_op2=op2, gamma2=g2, beta2=b2, eps2=1e-2)
            for i in range(m):
                y = [X.dec_to_frac(v) for v in stage(Xf[i], op1, g1, b1, 1e-3)]
                want = stage(y, op2, g2, b2, 1e-2)
                for gv, wv in zip(Z[i], want):
                    _close_dec(gv, wv, rtol=1e-11, atol=1e-12)
    # closed forms (unit affine): LayerNorm of a LayerNorm output, whose mean is
    # 0 and variance s2/(s2 + e1), is y / sqrt(s2/(s2 + e1) + e2); RMSNorm of an
    # RMSNorm output, whose mean square is ms/(ms + e1), is y / sqrt(ms/(ms + e1) + e2);
    # the softmax of a two-column softmax is the logistic function of 2 p - 1,
    # p = logistic(x0 - x1)
    Xr = rng.normal(0.3, 2.0, (6, 7))
    e1, e2 = 0.5, 0.25
    Z = o.row_stage(o.row_stage(Xr, "layernorm", eps=e1), "layernorm", eps=e2)
    mu, s2 = Xr.mean(axis=1, keepdims=True), Xr.var(axis=1, keepdims=True)
    y = (Xr - mu) / np.sqrt(s2 + e1)
    assert np.allclose(Z, y / np.sqrt(s2 / (s2 + e1) + e2), rtol=1e-12, atol=1e-13)
    Z = o.row_stage(o.row_stage(Xr, "rmsnorm", eps=e1), "rmsnorm", eps=e2)
    ms = (Xr ** 2).mean(axis=1, keepdims=True)
    y = Xr / np.sqrt(ms + e1)
    assert np.allclose(Z, y / np.sqrt(ms / (ms + e1) + e2), rtol=1e-12, atol=1e-13)
    d = rng.normal(0.0, 3.0, 9)
    Z = o.row_stage(o.row_stage(np.stack([d, np.zeros_like(d)], axis=1), "softmax"), "softmax")
    p = 1.0 / (1.0 + np.exp(-d))
    assert np.allclose(Z[:, 0], 1.0 / (1.0 + np.exp(-(2.0 * p - 1.0))), rtol=1e-12, atol=1e-14)
    # the second stage of "none" is the identity: the single-stage epilogue
    Z = o.gemm_epilogue_two_stage(A, B, alpha=0.5, bias=bias, row_op="layernorm", gamma=g1, beta=b1, eps=1e-3)
    for i in range(m):
        for gv, wv in zip(Z[i], X.layernorm_row(Xf[i], 1e-3, g1, b1)):
            _close_dec(gv, wv, rtol=1e-12, atol=1e-13)


def pin_row_topk(o):
    """Top-k against brute force: exact rational x on tiny shapes, every row's
    candidates compared pairwise (value, then column); duplicated columns of B
    make exact ties, which must keep column order; k = 1 agrees with argmax."""
    rng = np.random.default_rng(37)
    m, kk, n = 4, 3, 9
    A = _bf16_values(rng, (m, kk))
    B = _bf16_values(rng, (kk, n))
    B[:, 6] = B[:, 2]            # columns 2 and 6 equal in every row
    B[:, 8] = B[:, 2]
    bias = _bf16_values(rng, (n,))
    bias[6] = bias[2]
    bias[8] = bias[2]
    E = X.mm(X.mat(A), X.mat(B))
    Xf = [[Fraction(0.75) * E[i][j] + X.F(bias[j]) for j in range(n)] for i in range(m)]
    for k in (1, 3, 5, 9):
        idx, val = o.gemm_epilogue_topk(A, B, k, alpha=0.75, bias=bias)
        assert idx.shape == (m, k) and val.shape == (m, k)
        for i in range(m):
            order = sorted(range(n), key=lambda j: (-Xf[i][j], j))[:k]
            assert [int(v) for v in idx[i]] == order, (k, i, list(idx[i]), order)
            for j, c in enumerate(order):
                assert abs(Fraction(float(val[i, j])) - Xf[i][c]) <= Fraction(1, 2 ** 48)
    ai, av = o.row_argmax(np.array([[1.0, 3.0, 3.0, -2.0]]))
    ti, tv = o.row_topk(np.array([[1.0, 3.0, 3.0, -2.0]]), 1)
    assert int(ti[0, 0]) == int(ai[0]) == 1 and tv[0, 0] == av[0] == 3.0
    ti, tv = o.row_topk(np.array([[np.nan, 2.0, 5.0, 2.0]]), 3)
    assert [int(v) for v in ti[0]] == [2, 1, 3]
    # NaN ranks as -inf at its own column: behind every number, level with -inf
    ti, tv = o.row_topk(np.array([[-np.inf, np.nan, 1.0, -np.inf, np.inf]]), 5)
    assert [int(v) for v in ti[0]] == [4, 2, 0, 1, 3]


# --------------------------------------------------------------------------- back-to-back GEMM

def pin_b2b_relu(o):
    rng = np.random.default_rng(7)
    m, k, l, n = 4, 3, 5, 4
    A = _bf16_values(rng, (m, k))
    B0 = _bf16_values(rng, (k, l))
    B1 = _bf16_values(rng, (l, n))
    bias = _bf16_values(rng, (l,))
    alpha = 0.5
    O = o.b2bgemm(A, B0, B1, alpha=alpha, bias=bias, act="relu")
    S = X.mm(X.mat(A), X.mat(B0))
    Pm = [[X.round_bf16_exact(max(Fraction(alpha) * S[i][j] + X.F(bias[j]), Fraction(0)))
           for j in range(l)] for i in range(m)]
    E = X.mm(Pm, X.mat(B1))
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(float(O[i, j])) - E[i][j]) <= Fraction(1, 2 ** 45), (i, j)
    # unrounded operand: exact relu(S) . B1
    Ou = o.b2bgemm(A, B0, B1, alpha=alpha, bias=bias, act="relu", round_operand=False)
    Pu = [[max(Fraction(alpha) * S[i][j] + X.F(bias[j]), Fraction(0)) for j in range(l)]
          for i in range(m)]
    Eu = X.mm(Pu, X.mat(B1))
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(float(Ou[i, j])) - Eu[i][j]) <= Fraction(1, 2 ** 45)
    # B1 = identity: the output is the rounded intermediate itself
    Oi = o.b2bgemm(A, B0, np.eye(l), alpha=alpha, bias=bias, act="relu")
    for i in range(m):
        for j in range(l):
            assert Fraction(float(Oi[i, j])) == Pm[i][j]
    # [L, K] storage of B0 gives the same result
    assert np.array_equal(o.b2bgemm(A, B0.T.copy(), B1, alpha=alpha, bias=bias, act="relu",
                                    b0_layout="lk"), O)


def _softmax_operand_bruteforce(srow):
    """Decimal brute force of the bf16-operand softmax for one row of S (Fractions)."""
    log2e = X.CTX.divide(Decimal(1), X.LN2)
    ts = [X.CTX.multiply(X.D(s), log2e) for s in srow]
    c = max(ts).to_integral_value(rounding="ROUND_CEILING")
    pts = [X.dexp(X.CTX.multiply(X.CTX.subtract(t, c), X.LN2)) for t in ts]
    num = [X.round_bf16_exact(X.dec_to_frac(p)) for p in pts]
    den = sum(pts, Decimal(0))
    return num, den


def pin_b2b_softmax(o):
    rng = np.random.default_rng(8)
    m, k, l, n = 4, 6, 7, 5
    A = _bf16_values(rng, (m, k), 2.0)
    B0 = _bf16_values(rng, (l, k), 2.0)        # keys stored [L, K]
    B1 = _bf16_values(rng, (l, n))
    alpha = 0.125
    O = o.b2bgemm(A, B0, B1, alpha=alpha, row_op="softmax", b0_layout="lk")
    S = X.mm(X.mat(A), [list(r) for r in zip(*X.mat(B0))])
    for i in range(m):
        num, den = _softmax_operand_bruteforce([Fraction(alpha) * s for s in S[i]])
        for j in range(n):
            acc = sum((num[p] * X.F(B1[p, j]) for p in range(l)), Fraction(0))
            _close_dec(O[i, j], X.CTX.divide(X.D(acc), den), rtol=1e-12, atol=1e-14)
    # unrounded operand: softmax(S) . B1
    Ou = o.b2bgemm(A, B0, B1, alpha=alpha, row_op="softmax", b0_layout="lk", round_operand=False)
    for i in range(m):
        p = X.softmax_row([Fraction(alpha) * s for s in S[i]])
        for j in range(n):
            want = sum((X.CTX.multiply(p[q], X.D(X.F(B1[q, j]))) for q in range(l)), Decimal(0))
            _close_dec(Ou[i, j], want, rtol=1e-12, atol=1e-14)
    # B1 = identity: the rows are round_bf16(p~) / l, within 2**-8 of softmax(S)
    Oi = o.b2bgemm(A, B0, np.eye(l), alpha=alpha, row_op="softmax", b0_layout="lk")
    Ps = o.row_softmax(alpha * o.matmul(A, B0.T))
    assert np.all(np.abs(Oi - Ps) <= 2.0 ** -8 * Ps + 1e-300)
    assert np.all(np.abs(Oi.sum(-1) - 1) <= 2.0 ** -8)
    # integer stabiliser: the largest numerator of each row lies in (1/2, 1] and
    # every numerator is a bf16 value
    num, den = o.softmax_bf16_operand(alpha * o.matmul(A, B0.T))
    mx = num.max(-1)
    assert np.all((mx > 0.5) & (mx <= 1.0))
    assert np.array_equal(o.round_bf16(num), num)
    # batched input equals per-batch evaluation
    Ab = np.stack([A, A[::-1]])
    B0b = np.stack([B0, B0 * 0.5])
    B1b = np.stack([B1, -B1])
    Ob = o.b2bgemm(Ab, B0b, B1b, alpha=alpha, row_op="softmax", b0_layout="lk")
    assert np.array_equal(Ob[1], o.b2bgemm(A[::-1], B0 * 0.5, -B1, alpha=alpha,
                                           row_op="softmax", b0_layout="lk"))


def pin_b2b_causal(o):
    """Causal softmax B2BGEMM: each row against the brute force of the un-masked
    computation on the visible prefix of keys only (slicing, not masking), for
    M < L (queries at the end), M == L and M > L (rows that see nothing give 0)."""
    rng = np.random.default_rng(12)
    k, n, alpha = 5, 3, 0.25
    for m, l in ((3, 6), (5, 5), (6, 4)):
        A = _bf16_values(rng, (m, k), 2.0)
        B0 = _bf16_values(rng, (l, k), 2.0)
        B1 = _bf16_values(rng, (l, n))
        O = o.b2bgemm(A, B0, B1, alpha=alpha, row_op="softmax", b0_layout="lk", causal=True)
        Ou = o.b2bgemm(A, B0, B1, alpha=alpha, row_op="softmax", b0_layout="lk", causal=True,
                       round_operand=False)
        S = X.mm(X.mat(A), [list(r) for r in zip(*X.mat(B0))])
        for i in range(m):
            vis = i + (l - m) + 1              # keys 0 .. i + L - M
            if vis <= 0:
                assert np.all(O[i] == 0.0) and np.all(Ou[i] == 0.0), (m, l, i)
                continue
            num, den = _softmax_operand_bruteforce([Fraction(alpha) * s for s in S[i][:vis]])
            p = X.softmax_row([Fraction(alpha) * s for s in S[i][:vis]])
            for j in range(n):
                acc = sum((num[q] * X.F(B1[q, j]) for q in range(vis)), Fraction(0))
                _close_dec(O[i, j], X.CTX.divide(X.D(acc), den), rtol=1e-12, atol=1e-14)
                want = sum((X.CTX.multiply(p[q], X.D(X.F(B1[q, j]))) for q in range(vis)), Decimal(0))
                _close_dec(Ou[i, j], want, rtol=1e-12, atol=1e-14)
        # the first query of a square problem sees only key 0: O[0] = B1[0] exactly (unrounded operand)
        if m == l:
            assert np.array_equal(Ou[0], B1[0])
    # a single query at the end of the sequence sees every key: the unmasked result
    A = _bf16_values(rng, (1, k))
    B0 = _bf16_values(rng, (7, k))
    B1 = _bf16_values(rng, (7, n))
    assert np.array_equal(o.b2bgemm(A, B0, B1, alpha=alpha, row_op="softmax", b0_layout="lk", causal=True),
                          o.b2bgemm(A, B0, B1, alpha=alpha, row_op="softmax", b0_layout="lk"))


def pin_row_statistics(o):
    """Log-sum-exp, LayerNorm (mean, 1/sigma) and RMSNorm 1/rms of each row against
    40-digit decimals and closed forms."""
    rng = np.random.default_rng(13)
    Xr = _bf16_values(rng, (3, 7), 3.0)
    eps = 1e-5
    for row_op in ("softmax", "layernorm", "rmsnorm"):
        st = o.row_statistics(Xr, row_op, eps)
        for i in range(3):
            xs = [X.D(X.F(v)) for v in Xr[i]]
            n = X.D(len(xs))
            if row_op == "softmax":
                want = [X.CTX.ln(sum((X.dexp(v) for v in xs), Decimal(0)))]
                got = [st[i]]
            elif row_op == "layernorm":
                mu = X.CTX.divide(sum(xs, Decimal(0)), n)
                var = X.CTX.divide(sum(((v - mu) * (v - mu) for v in xs), Decimal(0)), n)
                want = [mu, X.CTX.divide(Decimal(1), X.dsqrt(var + X.D(eps)))]
                got = list(st[i])
            else:
                ms = X.CTX.divide(sum((v * v for v in xs), Decimal(0)), n)
                want = [X.CTX.divide(Decimal(1), X.dsqrt(ms + X.D(eps)))]
                got = [st[i]]
            for gv, wv in zip(got, want):
                _close_dec(gv, wv, rtol=1e-13, atol=1e-14)
    # closed forms: a constant row c of n values has log-sum-exp c + ln n, mean c and
    # 1/sigma = 1/sqrt(eps); rmsnorm of c gives 1/sqrt(c^2 + eps)
    c = np.full((1, 8), 1.25)
    assert abs(o.row_statistics(c, "softmax")[0] - (1.25 + math.log(8))) < 1e-14
    ln = o.row_statistics(c, "layernorm", eps)[0]
    assert ln[0] == 1.25 and abs(ln[1] - 1 / math.sqrt(eps)) < 1e-9
    assert abs(o.row_statistics(c, "rmsnorm", eps)[0] - 1 / math.sqrt(1.25 ** 2 + eps)) < 1e-14
    # log-sum-exp is shift-covariant: lse(x + t) = lse(x) + t
    assert abs(o.row_statistics(Xr + 5.0, "softmax") - o.row_statistics(Xr, "softmax") - 5.0).max() < 1e-13
    # through the GEMM: the statistics of the elementwise stage's result
    A = _bf16_values(rng, (3, 4))
    B = _bf16_values(rng, (4, 6))
    R = _bf16_values(rng, (3, 6))
    st = o.gemm_epilogue_row_stats(A, B, alpha=0.5, residual=R, row_op="rmsnorm", eps=eps)
    E = X.mm(X.mat(A), X.mat(B))
    for i in range(3):
        xs = [X.D(Fraction(1, 2) * E[i][j] + X.F(R[i, j])) for j in range(6)]
        ms = X.CTX.divide(sum((v * v for v in xs), Decimal(0)), X.D(6))
        _close_dec(st[i], X.CTX.divide(Decimal(1), X.dsqrt(ms + X.D(eps))), rtol=1e-13, atol=1e-14)


def pin_b2b_logsumexp(o):
    """Attention log-sum-exp against brute force on the visible prefix of keys; a
    causal row that sees no key gives -inf."""
    rng = np.random.default_rng(14)
    k, alpha = 5, 0.25
    for m, l, causal in ((3, 6, True), (4, 4, False), (5, 3, True)):
        A = _bf16_values(rng, (m, k), 2.0)
        B0 = _bf16_values(rng, (l, k), 2.0)
        got = o.b2b_logsumexp(A, B0, alpha=alpha, b0_layout="lk", causal=causal)
        S = X.mm(X.mat(A), [list(r) for r in zip(*X.mat(B0))])
        for i in range(m):
            vis = min(l, i + (l - m) + 1) if causal else l
            if vis <= 0:
                assert got[i] == -np.inf
                continue
            want = X.CTX.ln(sum((X.dexp(X.D(Fraction(alpha) * S[i][j])) for j in range(vis)), Decimal(0)))
            _close_dec(got[i], want, rtol=1e-13, atol=1e-14)


def pin_row_argmax(o):
    """Row argmax against an exact brute force (first column attaining the
    maximum of exact rationals), with exact ties built from duplicated columns."""
    rng = np.random.default_rng(15)
    m, k, n = 4, 5, 9
    A = _bf16_values(rng, (m, k))
    B = _bf16_values(rng, (k, n))
    B[:, 6] = B[:, 2]               # column 6 ties column 2 exactly in every row
    B[:, 8] = B[:, 0]
    bias = _bf16_values(rng, (n,))
    bias[6] = bias[2]
    bias[8] = bias[0]
    R = np.zeros((m, n))
    R[1] = 5.0                      # row 1: every column shifted alike
    E = X.mm(X.mat(A), X.mat(B))
    for act in ("none", "relu"):
        idx, val = o.gemm_epilogue_argmax(A, B, alpha=0.5, bias=bias, residual=R, act=act)
        for i in range(m):
            xs = [Fraction(1, 2) * E[i][j] + X.F(bias[j]) + X.F(R[i, j]) for j in range(n)]
            if act == "relu":
                xs = [max(v, Fraction(0)) for v in xs]
            best = max(xs)
            first = xs.index(best)
            assert int(idx[i]) == first, (act, i, int(idx[i]), first)
            assert Fraction(float(val[i])) == best
    # a constant row: column 0; a strictly increasing row: the last column
    i0, v0 = o.row_argmax(np.full((1, 5), 2.5))
    i1, v1 = o.row_argmax(np.arange(6.0)[None, :])
    assert int(i0[0]) == 0 and v0[0] == 2.5 and int(i1[0]) == 5 and v1[0] == 5.0
    # NaN ranks as -inf: it never beats a number, and rows of NaN and -inf
    # alone give their first column
    ni, _ = o.row_argmax(np.array([[np.nan, 2.0, 5.0, 5.0], [np.nan, np.nan, np.nan, np.nan],
                                   [-np.inf, np.nan, -np.inf, -np.inf], [1.0, np.nan, np.inf, np.nan]]))
    assert [int(v) for v in ni] == [2, 0, 0, 2], list(ni)


def pin_column_ops(o):
    """Column reductions against brute force on each column (the exact row
    routines applied to the column's values), closed forms and invariants."""
    rng = np.random.default_rng(21)
    Xm = rng.standard_normal((7, 5)) * 2 + 1
    eps = 1e-5
    gamma = rng.standard_normal(5)
    beta = rng.standard_normal(5)
    # softmax over m: every column sums to 1, a per-column shift changes nothing
    Ys = o.column_stage(Xm, "softmax")
    assert np.all(np.abs(Ys.sum(0) - 1) <= 7 * 1e-15)
    assert np.allclose(o.column_stage(Xm + rng.standard_normal((1, 5)) * 40, "softmax"), Ys, rtol=1e-12, atol=0)
    # large logits in a column must not overflow (the column maximum is subtracted)
    big = np.array([[1000.0, 0.5], [999.0, 0.25], [990.0, -1.0]])
    yb = o.column_stage(big, "softmax")
    for j in range(2):
        for g, w in zip(yb[:, j], X.softmax_row([Fraction(v) for v in big[:, j]])):
            _close_dec(g, w)
    # LayerNorm over m: zero column mean, variance var / (var + eps) before the affine step
    Yl = o.column_stage(Xm, "layernorm", None, None, eps)
    assert np.all(np.abs(Yl.mean(0)) <= 1e-14)
    for j in range(5):
        xs = [X.F(v) for v in Xm[:, j]]
        mu = sum(xs, Fraction(0)) / len(xs)
        var = sum(((x - mu) ** 2 for x in xs), Fraction(0)) / len(xs)
        assert math.isclose(float(np.mean(Yl[:, j] ** 2)), float(var / (var + X.F(eps))), rel_tol=1e-13)
    # a constant column -> beta of that column
    Xc = Xm.copy()
    Xc[:, 2] = 3.5
    assert np.allclose(o.column_stage(Xc, "layernorm", gamma, beta, eps)[:, 2], beta[2], rtol=0, atol=1e-15)
    # 40-digit brute force, column by column, with the per-column affine vectors
    Z = rng.standard_normal((4, 3)) * 2
    for op in ("softmax", "layernorm", "rmsnorm"):
        g3 = None if op == "softmax" else gamma[:3]
        b3 = beta[:3] if op == "layernorm" else None
        Y = o.column_stage(Z, op, g3, b3, eps)
        for j in range(3):
            col = [X.F(v) for v in Z[:, j]]
            if op == "softmax":
                want = X.softmax_row(col)
            elif op == "layernorm":
                want = X.layernorm_row(col, eps, [gamma[j]] * 4, [beta[j]] * 4)
            else:
                want = X.rmsnorm_row(col, eps, [gamma[j]] * 4)
            for i in range(4):
                _close_dec(Y[i, j], want[i], rtol=1e-12, atol=1e-14)
    # statistics: log-sum-exp, (mean, 1/sigma) and 1/rms of each column
    for op in ("softmax", "layernorm", "rmsnorm"):
        st = o.column_statistics(Z, op, eps)
        for j in range(3):
            xs = [X.D(X.F(v)) for v in Z[:, j]]
            n = X.D(len(xs))
            if op == "softmax":
                want, got = [X.CTX.ln(sum((X.dexp(v) for v in xs), Decimal(0)))], [st[j]]
            elif op == "layernorm":
                mu = X.CTX.divide(sum(xs, Decimal(0)), n)
                var = X.CTX.divide(sum(((v - mu) * (v - mu) for v in xs), Decimal(0)), n)
                want, got = [mu, X.CTX.divide(Decimal(1), X.dsqrt(var + X.D(eps)))], list(st[j])
            else:
                ms = X.CTX.divide(sum((v * v for v in xs), Decimal(0)), n)
                want, got = [X.CTX.divide(Decimal(1), X.dsqrt(ms + X.D(eps)))], [st[j]]
            for gv, wv in zip(got, want):
                _close_dec(gv, wv, rtol=1e-13, atol=1e-14)
    # through the GEMM with alpha, bias, residual and ReLU: exact x, then the column op
    A = _bf16_values(rng, (5, 4))
    B = _bf16_values(rng, (4, 3))
    R = _bf16_values(rng, (5, 3))
    bias = _bf16_values(rng, (3,))
    Yg = o.gemm_epilogue_columns(A, B, alpha=0.5, bias=bias, residual=R, act="relu", col_op="rmsnorm",
                                 gamma=gamma[:3], eps=eps)
    E = X.mm(X.mat(A), X.mat(B))
    for j in range(3):
        col = [max(Fraction(1, 2) * E[i][j] + X.F(bias[j]) + X.F(R[i, j]), Fraction(0)) for i in range(5)]
        want = X.rmsnorm_row(col, eps, [gamma[j]] * 5)
        for i in range(5):
            _close_dec(Yg[i, j], want[i], rtol=1e-12, atol=1e-14)


ALL_PINS = [pin_round_bf16, pin_widen_bf16, pin_matmul_exact, pin_stage1_exact, pin_softmax,
            pin_layernorm, pin_rmsnorm, pin_gemm_epilogue_composition, pin_two_outputs, pin_b2b_relu,
            pin_b2b_softmax, pin_b2b_causal, pin_row_statistics, pin_b2b_logsumexp, pin_row_argmax,
            pin_two_stage, pin_row_topk, pin_column_ops]


def run_all(o):
    for p in ALL_PINS:
        p(o)
