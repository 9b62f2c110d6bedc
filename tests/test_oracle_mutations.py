"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins reject every one of them. This shows the pins are strong enough to
catch a dropped term, a wrong sign or index, or a transposed operand."""
import os
import types

import pytest

import pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "__init__.py")

MUTATIONS = {
    "layernorm_unbiased_variance": [(
        "var = (d * d).mean(axis=-1, keepdims=True)",
        "var = (d * d).sum(axis=-1, keepdims=True) / (X.shape[-1] - 1)")],
    "layernorm_eps_outside_root": [(
        "\n    Y = d / np.sqrt(var + float(eps))", "\n    Y = d / (np.sqrt(var) + float(eps))")],
    "layernorm_drops_beta": [(
        "    if beta is not None:\n        Y = Y + np.asarray(beta, np.float64)\n    return Y\n\n\ndef rms_norm",
        "    return Y\n\n\ndef rms_norm")],
    "rmsnorm_drops_eps": [("\n    Y = X / np.sqrt(ms + float(eps))", "\n    Y = X / np.sqrt(ms)")],
    "rmsnorm_centres_rows": [(
        "ms = (X * X).mean(axis=-1, keepdims=True)",
        "ms = ((X - X.mean(axis=-1, keepdims=True)) ** 2).mean(axis=-1, keepdims=True)")],
    "softmax_without_max_shift": [("\n    e = np.exp(X - mx)", "\n    e = np.exp(X)")],
    "bias_per_row": [(
        "X = X + np.asarray(bias, np.float64)[..., None, :]",
        "X = X + np.asarray(bias, np.float64)[..., :, None]")],
    "alpha_dropped": [("X = float(alpha) * P", "X = P")],
    "residual_after_activation": [
        ("        X = X + np.asarray(residual, np.float64)\n", "        pass\n"),
        ("        X = relu(X)\n", "        X = relu(X)\n    if residual is not None:\n"
                                "        X = X + np.asarray(residual, np.float64)\n")],
    "matmul_transposed_b": [(
        "return np.matmul(np.asarray(A, np.float64), np.asarray(B, np.float64))",
        "return np.matmul(np.asarray(A, np.float64), np.swapaxes(np.asarray(B, np.float64), -1, -2))")],
    "round_ties_away_from_zero": [(
        "np.rint(np.ldexp(m, 8))", "np.trunc(np.ldexp(m, 8) + np.copysign(0.5, m))")],
    "round_to_seven_bits": [(
        "r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)", "r = np.ldexp(np.rint(np.ldexp(m, 7)), e - 7)")],
    "widen_wrong_shift": [(".astype(np.uint32) << 16", ".astype(np.uint32) << 15")],
    "softmax_operand_real_stabiliser": [(
        "c = np.ceil(t.max(axis=-1, keepdims=True))", "c = t.max(axis=-1, keepdims=True)")],
    "softmax_operand_rounded_denominator": [(
        "return round_bf16(pt), pt.sum(axis=-1, keepdims=True)",
        "r = round_bf16(pt)\n    return r, r.sum(axis=-1, keepdims=True)")],
    "b2b_operand_not_rounded": [("Pm = round_bf16(S) if round_operand else S", "Pm = S")],
    "b2b_keys_layout_ignored": [("B0 = np.swapaxes(B0, -1, -2)", "B0 = B0")],
    "x_output_after_row_op": [(
        "    return row_stage(X, row_op, gamma, beta, eps), X\n",
        "    Y = row_stage(X, row_op, gamma, beta, eps)\n    return Y, Y\n")],
    "x_output_before_residual": [(
        "    X = elementwise_stage(matmul(A, B), alpha, bias, residual, act)\n    return row_stage(X, row_op, gamma, beta, eps), X\n",
        "    X = elementwise_stage(matmul(A, B), alpha, bias, residual, act)\n"
        "    return row_stage(X, row_op, gamma, beta, eps), elementwise_stage(matmul(A, B), alpha, bias, None, act)\n")],
    "causal_mask_off_by_one": [(
        "return np.arange(L)[None, :] <= np.arange(M)[:, None] + (L - M)",
        "return np.arange(L)[None, :] < np.arange(M)[:, None] + (L - M)")],
    "causal_mask_top_left_aligned": [(
        "return np.arange(L)[None, :] <= np.arange(M)[:, None] + (L - M)",
        "return np.arange(L)[None, :] <= np.arange(M)[:, None]")],
    "causal_mask_ignored": [("            S = np.where(vis, S, -np.inf)\n", "")],
    "logsumexp_without_max": [(
        "lse = mx + np.log(np.exp(X - mx).sum(axis=-1, keepdims=True))",
        "lse = np.log(np.exp(X - mx).sum(axis=-1, keepdims=True))")],
    "layernorm_stats_std_not_inverse": [(
        "return np.concatenate([mu, 1.0 / np.sqrt(var + float(eps))], axis=-1)",
        "return np.concatenate([mu, np.sqrt(var + float(eps))], axis=-1)")],
    "rms_stats_drops_eps": [(
        "return 1.0 / np.sqrt((X * X).mean(axis=-1) + float(eps))",
        "return 1.0 / np.sqrt((X * X).mean(axis=-1))")],
    "b2b_lse_keys_layout_ignored": [("        B0 = np.moveaxis(B0, -1, -2)\n", "        pass\n")],
    "b2b_lse_ignores_alpha": [(
        "    S = float(alpha) * matmul(A, B0)\n", "    S = matmul(A, B0)\n")],
    "argmax_ties_to_last_column": [(
        "    idx = np.argmax(key, axis=-1)\n",
        "    idx = X.shape[-1] - 1 - np.argmax(key[..., ::-1], axis=-1)\n")],
    "argmax_is_argmin": [("    idx = np.argmax(key, axis=-1)\n", "    idx = np.argmin(key, axis=-1)\n")],
    "argmax_nan_wins": [("    idx = np.argmax(key, axis=-1)\n", "    idx = np.argmax(X, axis=-1)\n")],
    "two_stage_second_on_x": [(
        "    return row_stage(Y, row_op2, gamma2, beta2, eps2)\n",
        "    return row_stage(X, row_op2, gamma2, beta2, eps2)\n")],
    "two_stage_order_swapped": [(
        "    Y = row_stage(X, row_op, gamma, beta, eps)\n    return row_stage(Y, row_op2, gamma2, beta2, eps2)\n",
        "    Y = row_stage(X, row_op2, gamma2, beta2, eps2)\n    return row_stage(Y, row_op, gamma, beta, eps)\n")],
    "two_stage_second_affine_from_first": [(
        "    return row_stage(Y, row_op2, gamma2, beta2, eps2)\n",
        "    return row_stage(Y, row_op2, gamma, beta, eps2)\n")],
    "two_stage_second_eps_from_first": [(
        "    return row_stage(Y, row_op2, gamma2, beta2, eps2)\n",
        "    return row_stage(Y, row_op2, gamma2, beta2, eps)\n")],
    "topk_ties_to_last_column": [(
        '    idx = np.argsort(-key, axis=-1, kind="stable")[..., :k]\n',
        '    idx = (n - 1 - np.argsort(-key[..., ::-1], axis=-1, kind="stable"))[..., :k]\n')],
    "topk_ascending": [(
        '    idx = np.argsort(-key, axis=-1, kind="stable")[..., :k]\n',
        '    idx = np.argsort(key, axis=-1, kind="stable")[..., :k]\n')],
    "topk_nan_not_ranked_as_minus_inf": [(
        '    idx = np.argsort(-key, axis=-1, kind="stable")[..., :k]\n',
        '    idx = np.argsort(-X, axis=-1, kind="stable")[..., :k]\n')],
    "topk_one_short": [(
        '    idx = np.argsort(-key, axis=-1, kind="stable")[..., :k]\n',
        '    idx = np.argsort(-key, axis=-1, kind="stable")[..., :max(k - 1, 1)]\n')],
    "column_softmax_over_rows": [(
        "        return e / e.sum(axis=-2, keepdims=True)\n", "        return e / e.sum(axis=-1, keepdims=True)\n")],
    "column_softmax_without_max_shift": [(
        "        mx = X.max(axis=-2, keepdims=True)\n        e = np.exp(X - mx)\n",
        "        mx = X.max(axis=-2, keepdims=True)\n        e = np.exp(X)\n")],
    "column_layernorm_unbiased_variance": [(
        "        var = (d * d).mean(axis=-2, keepdims=True)\n",
        "        var = (d * d).sum(axis=-2, keepdims=True) / (X.shape[-2] - 1)\n")],
    "column_layernorm_mean_over_columns": [(
        "        mu = X.mean(axis=-2, keepdims=True)\n        d = X - mu\n",
        "        mu = X.mean(axis=-1, keepdims=True)\n        d = X - mu\n")],
    "column_rmsnorm_drops_eps": [(
        "        Y = X / np.sqrt(ms + float(eps))\n        beta = None\n",
        "        Y = X / np.sqrt(ms)\n        beta = None\n")],
    "column_affine_per_row": [(
        "    if gamma is not None:\n        Y = Y * np.asarray(gamma, np.float64)\n    if beta is not None:\n"
        "        Y = Y + np.asarray(beta, np.float64)\n    return Y\n\n\ndef column_statistics",
        "    if gamma is not None:\n        Y = Y * np.asarray(gamma, np.float64)[:Y.shape[0], None]\n    if beta is not None:\n"
        "        Y = Y + np.asarray(beta, np.float64)\n    return Y\n\n\ndef column_statistics")],
    "column_stats_lse_drops_max": [(
        "        return mx + np.log(np.exp(X - mx[..., None, :]).sum(axis=-2))",
        "        return np.log(np.exp(X - mx[..., None, :]).sum(axis=-2))")],
    "column_stats_rms_over_rows": [(
        "        return 1.0 / np.sqrt((X * X).mean(axis=-2) + float(eps))",
        "        return 1.0 / np.sqrt((X * X).mean(axis=-1) + float(eps))")],
    "b2b_relu_dropped": [(
        "S = elementwise_stage(matmul(A, B0), alpha, bias, None, act)",
        "S = elementwise_stage(matmul(A, B0), alpha, bias, None, 'none')")],
}


def _mutant(edits):
    src = open(ORACLE_SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(MUTATIONS[name])
    with pytest.raises((AssertionError, ValueError)):
        pins.run_all(mod)


def test_unmutated_copy_passes():
    pins.run_all(_mutant([]))
