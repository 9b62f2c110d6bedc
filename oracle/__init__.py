"""fp64 CPU oracle for the fused GEMM-epilogue and back-to-back GEMM path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``b2bgemm_stage_stream_amd``) never imports it, and the two share no code: no
kernels, headers, helpers or constants. The only common dependency is ``gen``,
which draws the seeded inputs and holds none of this arithmetic.

Source of the method: the pith.science review of arXiv 2608.03537, "ComFuse:
Fusing Complex Memory-Intensive Subgraphs with Compute-Intensive Kernels For
Modern GPU Architectures" (cited below as "ComFuse review"). The page names the
operators (MatMul followed by elementwise ops, softmax, LayerNorm, RMSNorm;
GEMM + elementwise/reduction + GEMM) but prints none of their formulas, so the
oracle is the plain textbook definition of each, evaluated unfused in float64
on the exact stored input values. Fusion and tiling change these results only
by rounding order: per the ComFuse review ("Circularity Check"), Eq. (1) only
bounds which tiles a reduction has to wait for, and Eqs. (3)-(5) cut the second
contraction into segments whose sum is the whole product. So the plain
definition is the oracle.

Readings where the page is silent (each is listed with its reason in the design
notes of this repository):
  * epilogue order: alpha * P, + bias[n], + residual[m, n], activation, row
    operation, affine, cast;
  * LayerNorm uses the biased (1/N) variance and eps inside the square root;
    RMSNorm is x / sqrt(mean(x^2) + eps) * w; softmax subtracts the row max;
  * in the back-to-back GEMM the second contraction takes its left operand in
    bf16: ``round_bf16(F(S))`` for elementwise F, and for the softmax
    ``round_bf16(2**(t - c))`` with ``t = log2(e) * S`` and an integer
    stabiliser ``c = ceil(max_row t)``, divided by the row sum of the unrounded
    ``2**(t - c)``. The result does not depend on which integer c is used.
    The unrounded result (``round_operand=False``) is available beside it.

Parity pins (tests/test_oracle_pins.py) tie every function here to exact
rational / 40-digit decimal brute force on tiny shapes, closed forms and
invariants, not to this code.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "widen_bf16", "round_bf16", "matmul", "elementwise_stage", "relu",
    "row_softmax", "layer_norm", "rms_norm", "gemm_epilogue", "gemm_epilogue_two_stage",
    "softmax_bf16_operand", "b2bgemm", "column_stage", "column_statistics", "gemm_epilogue_columns",
    "gemm_epilogue_column_stats",
]

_LOG2E = 1.0 / math.log(2.0)


# --------------------------------------------------------------------------- storage

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the upper 16 bits of an IEEE binary32 value.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and binary32's exponent range: normal values
    are m * 2**e with 8-bit m; below 2**-126 the spacing is fixed at 2**-133;
    results of magnitude 2**128 or more overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                   # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)         # np.rint: half to even
    tiny = np.abs(x) < 2.0 ** -126
    r = np.where(tiny, np.ldexp(np.rint(np.ldexp(x, 133)), -133), r)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return r


# --------------------------------------------------------------------------- GEMM + stage 1

def matmul(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """P = A . B in float64 (ComFuse review, "Core claim": the GEMM output P that
    is tiled into T_{m,n}). Leading dims broadcast as batches."""
    return np.matmul(np.asarray(A, np.float64), np.asarray(B, np.float64))


def relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0)


def elementwise_stage(P: np.ndarray, alpha: float = 1.0, bias: Optional[np.ndarray] = None,
                      residual: Optional[np.ndarray] = None, act: str = "none") -> np.ndarray:
    """Elementwise nodes that stream over the accumulator tile before the first
    reduction (ComFuse review, "What carries the argument"): scale, bias per
    output column n, residual add, activation."""
    X = float(alpha) * P
    if bias is not None:
        X = X + np.asarray(bias, np.float64)[..., None, :]
    if residual is not None:
        X = X + np.asarray(residual, np.float64)
    if act == "relu":
        X = relu(X)
    elif act != "none":
        raise ValueError(f"unknown activation {act!r}")
    return X


# --------------------------------------------------------------------------- row reductions

def row_softmax(X: np.ndarray) -> np.ndarray:
    """Softmax over the last axis (a single-axis reduction over the strip that
    shares row index m; ComFuse review, "If this is right")."""
    mx = X.max(axis=-1, keepdims=True)
    e = np.exp(X - mx)
    return e / e.sum(axis=-1, keepdims=True)


def layer_norm(X: np.ndarray, gamma: Optional[np.ndarray], beta: Optional[np.ndarray],
               eps: float) -> np.ndarray:
    """LayerNorm over the last axis (ComFuse review, Fig. 3 "MatMul +
    LayerNorm"): two-pass mean and biased variance, eps inside the root."""
    mu = X.mean(axis=-1, keepdims=True)
    d = X - mu
    var = (d * d).mean(axis=-1, keepdims=True)
    Y = d / np.sqrt(var + float(eps))
    if gamma is not None:
        Y = Y * np.asarray(gamma, np.float64)
    if beta is not None:
        Y = Y + np.asarray(beta, np.float64)
    return Y


def rms_norm(X: np.ndarray, weight: Optional[np.ndarray], eps: float) -> np.ndarray:
    """RMSNorm over the last axis (ComFuse review, Fig. 2 "Data Flow in MatMul +
    RMSNorm Subgraph"): x / sqrt(mean(x^2) + eps) * w."""
    ms = (X * X).mean(axis=-1, keepdims=True)
    Y = X / np.sqrt(ms + float(eps))
    if weight is not None:
        Y = Y * np.asarray(weight, np.float64)
    return Y


def gemm_epilogue(A: np.ndarray, B: np.ndarray, *, alpha: float = 1.0,
                  bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                  act: str = "none", row_op: str = "none", gamma: Optional[np.ndarray] = None,
                  beta: Optional[np.ndarray] = None, eps: float = 0.0) -> np.ndarray:
    """GEMM followed by its memory-intensive epilogue, unfused, in float64.

    Stage-Stream order (ComFuse review, "What carries the argument": elementwise
    nodes stream, a reduction is a stage boundary): alpha, bias, residual,
    activation, then one row operation with its affine parameters.
    ``row_op`` is "none", "softmax", "layernorm" or "rmsnorm"; ``gamma`` is the
    RMSNorm weight when row_op is "rmsnorm".
    """
    X = elementwise_stage(matmul(A, B), alpha, bias, residual, act)
    return row_stage(X, row_op, gamma, beta, eps)


def row_stage(X: np.ndarray, row_op: str, gamma: Optional[np.ndarray] = None,
              beta: Optional[np.ndarray] = None, eps: float = 0.0) -> np.ndarray:
    """The stage after the reduction boundary: one row operation on X."""
    if row_op == "none":
        return X
    if row_op == "softmax":
        return row_softmax(X)
    if row_op == "layernorm":
        return layer_norm(X, gamma, beta, eps)
    if row_op == "rmsnorm":
        return rms_norm(X, gamma, eps)
    raise ValueError(f"unknown row_op {row_op!r}")


def row_statistics(X: np.ndarray, row_op: str, eps: float = 0.0) -> np.ndarray:
    """The per-row result of the reduction stage itself (the review's "Reading
    between the lines" names log-sum-exp among the single-axis reductions the
    strip locality covers): for the softmax, ln sum_n exp(x) (the row max plus
    the log of the shifted sum); for LayerNorm, [mean, 1/sqrt(var + eps)] per
    row (last axis of length 2); for RMSNorm, 1/sqrt(mean(x^2) + eps)."""
    if row_op == "softmax":
        mx = X.max(axis=-1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            lse = mx + np.log(np.exp(X - mx).sum(axis=-1, keepdims=True))
        return np.where(np.isneginf(mx), -np.inf, lse)[..., 0]
    if row_op == "layernorm":
        mu = X.mean(axis=-1, keepdims=True)
        var = ((X - mu) * (X - mu)).mean(axis=-1, keepdims=True)
        return np.concatenate([mu, 1.0 / np.sqrt(var + float(eps))], axis=-1)
    if row_op == "rmsnorm":
        return 1.0 / np.sqrt((X * X).mean(axis=-1) + float(eps))
    raise ValueError(f"row_op {row_op!r} has no row statistics")


def row_argmax(X: np.ndarray):
    """(index, value) of each row: the smallest column n with X[m, n] equal to
    the row maximum, and that maximum (the review's "Reading between the lines"
    names max for top-k among the single-axis reductions the strip argument
    covers; top-1 here, ties to the lowest column). A NaN ranks as -inf: it
    never wins over a number, and a row of NaN and -inf only gives column 0."""
    X = np.asarray(X, np.float64)
    key = np.where(np.isnan(X), -np.inf, X)
    idx = np.argmax(key, axis=-1)
    return idx, np.take_along_axis(X, idx[..., None], axis=-1)[..., 0]


def row_topk(X: np.ndarray, k: int):
    """(index, value) of each row's k largest entries, largest first: the
    review's "Reading between the lines" names top-k among the single-axis
    reductions the strip argument covers. Order: value descending, and among
    equal values the smaller column first (so k = 1 is row_argmax); a NaN ranks
    as -inf at its own column. Returns int64 [..., k] and float64 [..., k]."""
    X = np.asarray(X, np.float64)
    n = X.shape[-1]
    if not 1 <= k <= n:
        raise ValueError(f"k = {k} outside 1..{n}")
    key = np.where(np.isnan(X), -np.inf, X)
    # a stable sort on the negated values keeps equal values in column order
    idx = np.argsort(-key, axis=-1, kind="stable")[..., :k]
    return idx, np.take_along_axis(X, idx, axis=-1)


def gemm_epilogue_topk(A: np.ndarray, B: np.ndarray, k: int, *, alpha: float = 1.0,
                       bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                       act: str = "none"):
    """row_topk of the elementwise stage's result X = act(alpha A.B + bias + R)."""
    return row_topk(elementwise_stage(matmul(A, B), alpha, bias, residual, act), k)


def gemm_epilogue_argmax(A: np.ndarray, B: np.ndarray, *, alpha: float = 1.0,
                         bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                         act: str = "none"):
    """row_argmax of the elementwise stage's result X = act(alpha A.B + bias + R)
    (e.g. greedy decoding on an LM head: the logits themselves are not needed)."""
    return row_argmax(elementwise_stage(matmul(A, B), alpha, bias, residual, act))


def gemm_epilogue_row_stats(A: np.ndarray, B: np.ndarray, *, alpha: float = 1.0,
                            bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                            act: str = "none", row_op: str = "softmax", eps: float = 0.0) -> np.ndarray:
    """row_statistics of the elementwise stage's result X = act(alpha A.B + bias + R)."""
    return row_statistics(elementwise_stage(matmul(A, B), alpha, bias, residual, act), row_op, eps)


def gemm_epilogue_with_x(A: np.ndarray, B: np.ndarray, *, alpha: float = 1.0,
                         bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                         act: str = "none", row_op: str = "none", gamma: Optional[np.ndarray] = None,
                         beta: Optional[np.ndarray] = None, eps: float = 0.0):
    """The same epilogue with two stored results, returned as (Y, X): X is the
    elementwise stage's output, the tensor the row operation reads, and Y the
    row operation's output. The review describes the epilogue as chained DAGs
    cut at its reductions (ComFuse review, "What carries the argument"); a DAG
    with a sink on each side of the boundary stores both, as a pre-norm block
    does with its new residual stream X = P + R beside RMSNorm(X). Both are
    float64 and unrounded."""
    X = elementwise_stage(matmul(A, B), alpha, bias, residual, act)
    return row_stage(X, row_op, gamma, beta, eps), X


def gemm_epilogue_two_stage(A: np.ndarray, B: np.ndarray, *, alpha: float = 1.0,
                            bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                            act: str = "none", row_op: str = "none", gamma: Optional[np.ndarray] = None,
                            beta: Optional[np.ndarray] = None, eps: float = 0.0, row_op2: str = "none",
                            gamma2: Optional[np.ndarray] = None, beta2: Optional[np.ndarray] = None,
                            eps2: float = 0.0) -> np.ndarray:
    """An epilogue with two reduction boundaries in sequence. The review
    describes the epilogue as chained DAGs cut at each reduction (ComFuse
    review, "What carries the argument"), and names chains of more than one
    reduction stage as the general case; here the first row operation (with
    gamma, beta, eps) gives Y from the elementwise stage's X, and the second
    (with gamma2, beta2, eps2) acts on Y over the same row."""
    X = elementwise_stage(matmul(A, B), alpha, bias, residual, act)
    Y = row_stage(X, row_op, gamma, beta, eps)
    return row_stage(Y, row_op2, gamma2, beta2, eps2)


# --------------------------------------------------------------------------- column reductions

def column_stage(X: np.ndarray, col_op: str, gamma: Optional[np.ndarray] = None,
                 beta: Optional[np.ndarray] = None, eps: float = 0.0) -> np.ndarray:
    """A reduction along the other dimension: the operation runs over the rows m
    of each column n. The review notes that Eq. (1)'s strip argument covers a
    column-dimension reduction through the complementary strip, the tiles
    T_{m,n} that share n (ComFuse review, Referee Report major comment 1 on
    Sec. III). Textbook forms, as for the rows: softmax over m with the column
    maximum subtracted; LayerNorm with the biased variance over m and eps inside
    the root, then gamma[n] * x_hat + beta[n] (a per-column affine, as a batch
    normalisation over the rows has); RMSNorm x / sqrt(mean_m(x^2) + eps) * w[n]."""
    X = np.asarray(X, np.float64)
    if col_op == "softmax":
        mx = X.max(axis=-2, keepdims=True)
        e = np.exp(X - mx)
        return e / e.sum(axis=-2, keepdims=True)
    if col_op == "layernorm":
        mu = X.mean(axis=-2, keepdims=True)
        d = X - mu
        var = (d * d).mean(axis=-2, keepdims=True)
        Y = d / np.sqrt(var + float(eps))
    elif col_op == "rmsnorm":
        ms = (X * X).mean(axis=-2, keepdims=True)
        Y = X / np.sqrt(ms + float(eps))
        beta = None
    else:
        raise ValueError(f"unknown col_op {col_op!r}")
    if gamma is not None:
        Y = Y * np.asarray(gamma, np.float64)
    if beta is not None:
        Y = Y + np.asarray(beta, np.float64)
    return Y


def column_statistics(X: np.ndarray, col_op: str, eps: float = 0.0) -> np.ndarray:
    """The per-column result of a column reduction: log-sum-exp over m for the
    softmax; [mean, 1/sqrt(var + eps)] for LayerNorm (last axis of length 2);
    1/sqrt(mean_m(x^2) + eps) for RMSNorm."""
    X = np.asarray(X, np.float64)
    if col_op == "softmax":
        mx = X.max(axis=-2)
        return mx + np.log(np.exp(X - mx[..., None, :]).sum(axis=-2))
    if col_op == "layernorm":
        mu = X.mean(axis=-2)
        var = ((X - mu[..., None, :]) ** 2).mean(axis=-2)
        return np.stack([mu, 1.0 / np.sqrt(var + float(eps))], axis=-1)
    if col_op == "rmsnorm":
        return 1.0 / np.sqrt((X * X).mean(axis=-2) + float(eps))
    raise ValueError(f"col_op {col_op!r} has no column statistics")


def gemm_epilogue_columns(A: np.ndarray, B: np.ndarray, *, alpha: float = 1.0,
                          bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                          act: str = "none", col_op: str = "softmax", gamma: Optional[np.ndarray] = None,
                          beta: Optional[np.ndarray] = None, eps: float = 0.0) -> np.ndarray:
    """GEMM, the elementwise stage, then one column reduction (column_stage)."""
    return column_stage(elementwise_stage(matmul(A, B), alpha, bias, residual, act), col_op, gamma, beta, eps)


def gemm_epilogue_column_stats(A: np.ndarray, B: np.ndarray, *, alpha: float = 1.0,
                               bias: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                               act: str = "none", col_op: str = "softmax", eps: float = 0.0) -> np.ndarray:
    """column_statistics of the elementwise stage's result."""
    return column_statistics(elementwise_stage(matmul(A, B), alpha, bias, residual, act), col_op, eps)


# --------------------------------------------------------------------------- back-to-back GEMM

def softmax_bf16_operand(S: np.ndarray):
    """Row softmax of S split into a bf16 numerator operand and a float64
    denominator: returns (round_bf16(2**(t - c)), sum(2**(t - c))) with
    t = log2(e) * S and c = ceil(max_row t), an integer. Dividing the second
    GEMM's result by the denominator gives softmax(S) . B1 with the operand in
    bf16. Because c is an integer and rounding commutes with scaling by a power
    of two, the quotient does not depend on the integer chosen."""
    t = S * _LOG2E
    c = np.ceil(t.max(axis=-1, keepdims=True))
    pt = np.exp2(t - c)
    return round_bf16(pt), pt.sum(axis=-1, keepdims=True)


def causal_visible(M: int, L: int) -> np.ndarray:
    """Boolean [M, L]: key l is visible to query row m iff l <= m + (L - M), the
    M queries being the last M of the L positions (the lower-triangular mask
    when M == L)."""
    return np.arange(L)[None, :] <= np.arange(M)[:, None] + (L - M)


def b2b_logsumexp(A: np.ndarray, B0: np.ndarray, *, alpha: float = 1.0, b0_layout: str = "kl",
                  causal: bool = False) -> np.ndarray:
    """ln sum_l exp(alpha * S[m, l]) over the keys row m sees, S = A . B0 (the
    softmax's own per-row reduction, as attention's backward pass keeps it);
    -inf for a causal row that sees no key. Leading dims broadcast as batches."""
    A = np.asarray(A, np.float64)
    B0 = np.asarray(B0, np.float64)
    if b0_layout == "lk":          # keys stored [L, K]
        B0 = np.moveaxis(B0, -1, -2)
    if A.ndim == 3:
        return np.stack([b2b_logsumexp(A[i], B0[i] if B0.ndim == 3 else B0, alpha=alpha, causal=causal)
                         for i in range(A.shape[0])])
    S = float(alpha) * matmul(A, B0)
    if causal:
        S = np.where(causal_visible(S.shape[0], S.shape[1]), S, -np.inf)
    return row_statistics(S, "softmax")


def b2bgemm(A: np.ndarray, B0: np.ndarray, B1: np.ndarray, *, alpha: float = 1.0,
            bias: Optional[np.ndarray] = None, act: str = "none", row_op: str = "none",
            b0_layout: str = "kl", round_operand: bool = True, causal: bool = False) -> np.ndarray:
    """Back-to-back GEMM O = F(alpha * A . B0 + bias) . B1 (ComFuse review,
    Referee Report major comment 2, paper Sec. IV-A and Eqs. (2)-(5); the
    intermediate S is an [M, L] matrix, L being the page's N1).

    ``B0`` is [K, L] (``b0_layout="kl"``) or [L, K] (``"lk"``, e.g. attention
    keys). F is the activation (``act``) and optionally a row softmax
    (``row_op="softmax"``). With ``round_operand`` the left operand of the second
    GEMM is rounded to bf16 as described in the module docstring; without it
    the whole computation stays in float64. Leading dims broadcast as batches;
    batches are evaluated one at a time to bound memory.

    ``causal`` (softmax only) hides the scores of invisible keys (see
    ``causal_visible``) before the softmax, as causal self-attention does (the
    review's Self-Attention workload, Referee Report major comment 3); a row
    that sees no key (only when M > L) gives 0.
    """
    A = np.asarray(A, np.float64)
    B0 = np.asarray(B0, np.float64)
    B1 = np.asarray(B1, np.float64)
    if b0_layout == "lk":
        B0 = np.swapaxes(B0, -1, -2)
    elif b0_layout != "kl":
        raise ValueError(f"unknown b0_layout {b0_layout!r}")
    if A.ndim == 3:
        return np.stack([
            b2bgemm(A[i], B0[i] if B0.ndim == 3 else B0, B1[i] if B1.ndim == 3 else B1,
                    alpha=alpha, bias=bias, act=act, row_op=row_op, b0_layout="kl",
                    round_operand=round_operand, causal=causal)
            for i in range(A.shape[0])])
    S = elementwise_stage(matmul(A, B0), alpha, bias, None, act)
    if causal and row_op != "softmax":
        raise ValueError("the causal mask applies to the softmax")
    if row_op == "softmax":
        if causal:
            vis = causal_visible(S.shape[0], S.shape[1])
            S = np.where(vis, S, -np.inf)
            empty = ~vis.any(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            if round_operand:
                num, den = softmax_bf16_operand(S)
                O = matmul(num, B1) / den
            else:
                O = matmul(row_softmax(S), B1)
        if causal:
            O[empty] = 0.0
        return O
    if row_op != "none":
        raise ValueError(f"row_op {row_op!r} is not supported between two GEMMs")
    Pm = round_bf16(S) if round_operand else S
    return matmul(Pm, B1)
