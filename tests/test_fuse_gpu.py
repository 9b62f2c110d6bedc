"""GPU parity of subgraphs lowered by the front-end (b2bgemm_stage_stream_amd.fuse)
against the fp64 oracle: the lowered call runs the library's fused kernels."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle                                   # noqa: E402
import parity as P                              # noqa: E402
from b2bgemm_stage_stream_amd import fuse       # noqa: E402


def check_bf16(got, ref, what):
    g = P.gpu_to_f64(got)
    P.assert_bf16_within(g, ref, what)
    r, _ = P.metrics(g, oracle.round_bf16(ref))
    assert r <= P.REL_F_BF16, f"{what}: relF vs RNE(oracle) {r:.3e}"


def test_prenorm_block():
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=22, M=300, N=1024, K=512)

    def block(x, wt, r, g):
        y = x @ wt + r
        return F.rms_norm(y, (y.shape[-1],), g, 1e-6), y

    args = (dev["A"], dev["B"], dev["residual"], dev["weight"])
    f = fuse.lower(block, *args)
    y, x = f(*args)
    Yr, Xr = oracle.gemm_epilogue_with_x(ref["A"], ref["B"], residual=ref["residual"], row_op="rmsnorm",
                                         gamma=ref["weight"], eps=1e-6)
    check_bf16(y, Yr, "lowered pre-norm block y")
    check_bf16(x, Xr, "lowered pre-norm block x")


def test_linear_bias_relu_layernorm():
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=23, M=256, N=768, K=256)
    Wt = dev["B"].t().contiguous()       # nn.Linear weight layout [N, K]
    b = torch.linspace(-0.2, 0.2, 768, device="cuda").to(torch.bfloat16)

    def layer(x, wl, bias, g, be):
        return F.layer_norm(torch.relu(0.5 * (x @ wl.t()) + bias), (wl.shape[0],), g, be, 1e-5)

    args = (dev["A"], Wt, b, dev["gamma"], dev["beta"])
    y = fuse.lower(layer, *args)(*args)
    R = oracle.gemm_epilogue(ref["A"], ref["B"], alpha=0.5, bias=P.gpu_to_f64(b), act="relu", row_op="layernorm",
                             gamma=ref["gamma"], beta=ref["beta"], eps=1e-5)
    check_bf16(y, R, "lowered linear + bias + relu + layernorm")


def test_two_row_stages():
    # LayerNorm then softmax over the same rows, lowered to one call with two
    # reduction boundaries
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=25, M=300, N=1024, K=256)

    def block(x, wt, g, be):
        return torch.softmax(F.layer_norm(x @ wt, (wt.shape[1],), g, be, 1e-5), dim=-1)

    args = (dev["A"], dev["B"], dev["gamma"], dev["beta"])
    f = fuse.lower(block, *args)
    assert f.plan.epi["row_op2"] == "softmax"
    y = f(*args, out_dtype=torch.float32)
    R = oracle.gemm_epilogue_two_stage(ref["A"], ref["B"], row_op="layernorm", gamma=ref["gamma"], beta=ref["beta"],
                                       eps=1e-5, row_op2="softmax")
    P.assert_close(P.gpu_to_f64(y), R, P.REL_F_BF16, P.MAX_ABS_BF16, "lowered layernorm -> softmax")


def test_attention():
    w, dev, ref = P.inputs("c5_b2b_attention", seed=24, batch=4, M=256, L=320)

    def attn(q, k, v):
        return torch.softmax(q @ k.transpose(-1, -2) * 0.125, dim=-1) @ v

    args = (dev["A"], dev["B0"], dev["B1"])
    o = fuse.lower(attn, *args)(*args, out_dtype=torch.float32)
    R = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], alpha=0.125, row_op="softmax", b0_layout="lk")
    P.assert_close(P.gpu_to_f64(o), R, P.REL_F_BF16, P.MAX_ABS_BF16, "lowered attention")


def test_mlp():
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=25, M=1000)

    def mlp(x, w0, w1):
        return torch.relu(x @ w0) @ w1

    args = (dev["A"][0], dev["B0"][0], dev["B1"][0])
    o = fuse.lower(mlp, *args)(*args, out_dtype=torch.float32)
    R = oracle.b2bgemm(ref["A"][0], ref["B0"][0], ref["B1"][0], act="relu")
    P.assert_close(P.gpu_to_f64(o)[0] if o.dim() == 3 else P.gpu_to_f64(o), R, P.REL_F_BF16, P.MAX_ABS_BF16,
                   "lowered MLP")
