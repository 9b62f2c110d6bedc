"""Lowering of traced torch subgraphs to one fused call (no GPU: the plans
only). Each node is placed in the stage stream by its operator and operand
shapes; what has no place, or comes out of order, is rejected."""
import pytest
import torch
import torch.nn.functional as F

from b2bgemm_stage_stream_amd import fuse

M, K, N = 8, 16, 32


def t(*shape):
    return torch.randn(*shape)


def prenorm(x, w, r, g):
    y = x @ w + r
    return F.rms_norm(y, (y.shape[-1],), g, 1e-6), y


def linear_ln(x, w, b, g, be):
    return F.layer_norm(torch.relu(0.5 * (x @ w.t()) + b), (w.shape[0],), g, be, 1e-5)


def attention(q, k, v):
    return torch.softmax(q @ k.transpose(-1, -2) * 0.125, dim=-1) @ v


def mlp(x, w0, w1):
    return torch.relu(x @ w0) @ w1


def test_prenorm_residual_rmsnorm_with_second_output():
    p = fuse.lower(prenorm, t(M, K), t(K, N), t(M, N), t(N)).plan
    assert p.kind == "gemm_epilogue" and not p.b_transposed
    assert p.epi == {"alpha": 1.0, "row_op": "rmsnorm", "eps": 1e-6}
    assert p.tensors == {"residual": 2, "gamma": 3}
    assert p.outputs == ["y", "x"]


def test_linear_bias_relu_layernorm_weight_nk():
    p = fuse.lower(linear_ln, t(M, K), t(N, K), t(N), t(N), t(N)).plan
    assert p.b_transposed and p.tensors == {"bias": 2, "gamma": 3, "beta": 4}
    assert p.epi == {"alpha": 0.5, "act": "relu", "row_op": "layernorm", "eps": 1e-5}


def test_attention_lowers_to_b2bgemm_with_keys_lk():
    p = fuse.lower(attention, t(2, M, K), t(2, 12, K), t(2, 12, K)).plan
    assert p.kind == "b2bgemm" and p.b_transposed and p.b1 == 2
    assert p.epi == {"alpha": 0.125, "row_op": "softmax"}


def test_mlp_lowers_to_b2bgemm_relu():
    p = fuse.lower(mlp, t(M, K), t(K, N), t(N, 4)).plan
    assert p.kind == "b2bgemm" and not p.b_transposed and p.epi == {"alpha": 1.0, "act": "relu"}


def test_plain_gemm_and_division():
    p = fuse.lower(lambda x, w: (x @ w) / 4.0, t(M, K), t(K, N)).plan
    assert p.kind == "gemm_epilogue" and p.epi == {"alpha": 0.25} and p.outputs == ["y"]


@pytest.mark.parametrize("fn,why", [
    (lambda x, w: torch.softmax(x @ w, dim=0), "axis"),
    (lambda x, w: (x @ w).sum(-1), "no place"),
    (lambda x, w: torch.relu(x @ w) * 2.0, "order"),
    (lambda x, w: torch.relu(x @ w) + 1.0, "other than an input"),
    (lambda x, w: torch.softmax(torch.softmax(F.layer_norm(x @ w, (N,)), dim=-1), dim=-1), "no place"),
    (lambda x, w: torch.tanh(x @ w), "no place"),
    (lambda x, w: x + 1.0, "no matrix product"),
])
def test_rejected(fn, why):
    with pytest.raises(fuse.NotFusable, match=why):
        fuse.lower(fn, t(K, K), t(K, N))


def test_two_row_stages():
    # a second row operation on the first one's result: the second boundary
    def fn(x, w, g, be, g2):
        y = F.layer_norm(x @ w, (N,), g, be, 1e-5)
        return F.rms_norm(y, (N,), g2, 1e-6)
    p = fuse.lower(fn, t(M, K), t(K, N), t(N), t(N), t(N)).plan
    assert p.epi == {"alpha": 1.0, "row_op": "layernorm", "eps": 1e-5, "row_op2": "rmsnorm", "eps2": 1e-6}
    assert p.tensors == {"gamma": 2, "beta": 3, "gamma2": 4}
    p = fuse.lower(lambda x, w: torch.softmax(F.rms_norm(x @ w, (N,), None, 1e-6), dim=-1), t(M, K), t(K, N)).plan
    assert p.epi["row_op"] == "rmsnorm" and p.epi["row_op2"] == "softmax"


def test_two_row_stages_first_result_not_stored():
    def fn(x, w):
        y = F.layer_norm(x @ w, (N,))
        return torch.softmax(y, dim=-1), y
    with pytest.raises(fuse.NotFusable, match="beside a second"):
        fuse.lower(fn, t(M, K), t(K, N))


def test_two_row_stages_between_gemms_rejected():
    with pytest.raises(fuse.NotFusable, match="between two GEMMs"):
        fuse.lower(lambda q, k, v: torch.softmax(torch.softmax(q @ k, dim=-1), dim=-1) @ v,
                   t(M, K), t(K, N), t(N, 4))


def test_transposed_left_operand():
    with pytest.raises(fuse.NotFusable, match="stored"):
        fuse.lower(lambda x, w: x.t() @ w, t(K, M), t(K, N))


def test_residual_after_activation_is_out_of_order():
    with pytest.raises(fuse.NotFusable, match="order"):
        fuse.lower(lambda x, w, r: torch.relu(x @ w) + r, t(M, K), t(K, N), t(M, N))


def test_softmax_between_gemms_takes_scores_as_they_are():
    with pytest.raises(fuse.NotFusable, match="as they are"):
        fuse.lower(lambda q, k, v, b: torch.softmax(q @ k + b, dim=-1) @ v, t(M, K), t(K, N), t(N, 4), t(N))
