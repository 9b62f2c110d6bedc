"""The fused calls inside a captured HIP graph (torch.cuda.CUDAGraph): every
replay must equal the eager result bit for bit, with eager work and
synchronisation between replays (the strip exchange's epoch advances across
launches, captured or not), and feature combinations on one call."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import b2bgemm_stage_stream_amd as cf   # noqa: E402
import oracle                           # noqa: E402
import parity as P                      # noqa: E402


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_replays_match_eager():
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=26, M=512, N=2048, K=256)
    e = cf.make_epilogue(row_op="layernorm", gamma=dev["gamma"], beta=dev["beta"], eps=1e-5)
    ws = cf.Workspace("cuda").get(cf.cf_gemm_epilogue_workspace_size(512, 2048, 256, e))
    wa, da, ra = P.inputs("c5_b2b_attention", seed=27, batch=4, M=256, L=256)
    C = torch.empty(512, 2048, dtype=torch.bfloat16, device="cuda")
    O = torch.empty(4, 256, 64, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def calls():
        cf.cf_gemm_epilogue(dev["A"], dev["B"], C, epi=e, workspace=ws)
        cf.cf_b2bgemm(da["A"], da["B0"], da["B1"], O, b0_is_lk=True, alpha=0.125, row_op="softmax",
                      mask="causal")

    with torch.cuda.stream(s):
        calls()                                   # eager, on the capture stream
    torch.cuda.synchronize()
    C_eager, O_eager = C.clone(), O.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    for i in range(4):
        C.zero_()
        O.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(C), bits(C_eager)), f"replay {i}: GEMM output differs"
        assert torch.equal(bits(O), bits(O_eager)), f"replay {i}: attention output differs"
        # eager launches between replays share the workspace
        with torch.cuda.stream(s):
            calls()
        torch.cuda.synchronize()
        assert torch.equal(bits(C), bits(C_eager))
    assert cf.cf_workspace_status(ws) == cf.CF_OK
    R = oracle.gemm_epilogue(ref["A"], ref["B"], row_op="layernorm", gamma=ref["gamma"], beta=ref["beta"], eps=1e-5)
    P.assert_bf16_within(P.gpu_to_f64(C_eager), R, "graph GEMM + LayerNorm")


def test_argmax_with_second_output_and_no_logits():
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=28, M=300, N=1024, K=256)
    idx = torch.empty(300, dtype=torch.int32, device="cuda")
    X = torch.empty(300, 1024, dtype=torch.float32, device="cuda")
    e = cf.make_epilogue(residual=dev["residual"], row_op="argmax", row_index=idx, x_out=X)
    ws = cf.Workspace("cuda").get(cf.cf_gemm_epilogue_workspace_size(300, 1024, 256, e))
    cf.cf_gemm_epilogue(dev["A"], dev["B"], None, epi=e, workspace=ws)
    torch.cuda.synchronize()
    Xr = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]), residual=ref["residual"])
    P.assert_close(P.gpu_to_f64(X), Xr, P.REL_F_BF16, P.MAX_ABS_BF16, "X beside the argmax")
    # the argmax of the stored fp32 X is exactly the kernel's (same values, lowest column on ties)
    assert torch.equal(idx.long().cpu(), torch.argmax(X.cpu(), dim=1)), "argmax differs from that of the stored x"


def test_row_stats_with_second_output():
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=29, M=256, N=768, K=256)
    st = torch.empty(256, dtype=torch.float32, device="cuda")
    X = torch.empty(256, 768, dtype=torch.float32, device="cuda")
    Y = torch.empty(256, 768, dtype=torch.float32, device="cuda")
    e = cf.make_epilogue(residual=dev["residual"], row_op="rmsnorm", gamma=dev["weight"], eps=1e-6,
                         row_stats=st, x_out=X)
    ws = cf.Workspace("cuda").get(cf.cf_gemm_epilogue_workspace_size(256, 768, 256, e))
    cf.cf_gemm_epilogue(dev["A"], dev["B"], Y, epi=e, workspace=ws)
    torch.cuda.synchronize()
    # y = x * rstd * w with the stored x and the stored rstd (fp32 rounding only)
    w32 = dev["weight"].float()
    P.assert_close(P.gpu_to_f64(Y), P.gpu_to_f64(X * st[:, None] * w32), 1e-6, 1e-5, "y from stored x and rstd")
    R = oracle.gemm_epilogue_row_stats(ref["A"], ref["B"], residual=ref["residual"], row_op="rmsnorm", eps=1e-6)
    P.assert_close(P.gpu_to_f64(st), R, 1e-5, 1e-4, "rstd")


def test_launch_stream_is_torch_current_stream():
    # launches without an explicit stream go to torch's current stream, on the
    # default stream and inside a side-stream context
    assert cf._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert cf._stream(None) == s.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert cf._stream(None) == torch.cuda.current_stream().cuda_stream
    assert cf._stream(s) == s.cuda_stream
