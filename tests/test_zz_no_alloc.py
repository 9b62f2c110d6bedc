"""cf_gemm_epilogue_noalloc (the entry point that allocates nothing: its
strip exchange runs in the library's static per-GPU scratch) against
cf_gemm_epilogue with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller problem, each bit-identical to the workspace
entry point and within the parity bars of the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import b2bgemm_stage_stream_amd as cf   # noqa: E402
import oracle                           # noqa: E402
import parity as P                      # noqa: E402

lib = cf._lib


def noalloc(A, B, C, e):
    M, K = A.shape
    N = B.shape[1]
    return lib.cf_gemm_epilogue_noalloc(M, N, K, A.data_ptr(), K, B.data_ptr(), N, 0, cf.CF_BF16,
                                        C.data_ptr(), N, cf._dtype_code(C), ctypes.byref(e),
                                        torch.cuda.current_stream().cuda_stream)


def with_workspace(A, B, C, e):
    M, K = A.shape
    N = B.shape[1]
    nbytes = cf.cf_gemm_epilogue_workspace_size(M, N, K, e)
    ws = cf.Workspace().get(nbytes)
    return lib.cf_gemm_epilogue(M, N, K, A.data_ptr(), K, B.data_ptr(), N, 0, cf.CF_BF16, C.data_ptr(), N,
                                cf._dtype_code(C), ctypes.byref(e), None if ws is None else ws.data_ptr(),
                                nbytes, torch.cuda.current_stream().cuda_stream)


CASES = [
    # (workload, seed, M, N, K): LayerNorm over 16 column tiles, then a smaller
    # residual + RMSNorm problem over 6 tiles with a ragged row strip
    ("c2_gemm_layernorm", 21, 1024, 4096, 512),
    ("c3_gemm_residual_rmsnorm", 22, 300, 1536, 256),
]


def test_noalloc_matches_workspace_entry_two_calls():
    for name, seed, M, N, K in CASES:
        print(f"noalloc case {name} {M}x{N}x{K}", flush=True)
        w, dev, ref = P.inputs(name, seed=seed, M=M, N=N, K=K)
        p = w.params
        g = dev.get("gamma", dev.get("weight"))
        e = cf.make_epilogue(residual=dev.get("residual"), row_op=p["row_op"], gamma=g, beta=dev.get("beta"),
                             eps=p["eps"])
        R = oracle.gemm_epilogue(ref["A"], ref["B"], residual=ref.get("residual"), row_op=p["row_op"],
                                 gamma=ref.get("gamma", ref.get("weight")), beta=ref.get("beta"), eps=p["eps"])
        for dt in (torch.float32, torch.bfloat16):
            C0 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
            C1 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
            assert with_workspace(dev["A"], dev["B"], C0, e) == cf.CF_OK
            assert noalloc(dev["A"], dev["B"], C1, e) == cf.CF_OK
            torch.cuda.synchronize()
            assert torch.equal(C0.view(torch.int16) if dt == torch.bfloat16 else C0.view(torch.int32),
                               C1.view(torch.int16) if dt == torch.bfloat16 else C1.view(torch.int32)), \
                f"{name}: noalloc differs from the workspace entry point ({dt})"
            G = P.gpu_to_f64(C1)
            if dt == torch.float32:
                P.assert_close(G, R, P.REL_F_BF16, P.MAX_ABS_BF16, f"{name} noalloc fp32 out")
            else:
                P.assert_bf16_within(G, R, f"{name} noalloc bf16 out")


def test_noalloc_repeated_calls_stay_exact():
    # the scratch keeps the last call's contents: later calls of other shapes
    # must not read them as current (epoch tags)
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=23, M=512, N=2048, K=128)
    e = cf.make_epilogue(row_op="layernorm", gamma=dev["gamma"], beta=dev["beta"], eps=1e-5)
    C = torch.empty(512, 2048, dtype=torch.float32, device="cuda")
    first = None
    for _ in range(3):
        C.fill_(float("nan"))
        assert noalloc(dev["A"], dev["B"], C, e) == cf.CF_OK
        torch.cuda.synchronize()
        if first is None:
            first = C.clone()
        assert torch.equal(C.view(torch.int32), first.view(torch.int32))
    R = oracle.gemm_epilogue(ref["A"], ref["B"], row_op="layernorm", gamma=ref["gamma"], beta=ref["beta"], eps=1e-5)
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_BF16, P.MAX_ABS_BF16, "noalloc repeated")


def test_noalloc_refuses_beyond_its_scratch():
    # top-8 over 8192 x 4096 needs 16 MiB of slots plus the header: refused
    # before any launch, and the next call still works
    A = torch.zeros(8192, 32, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(32, 4096, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(8192, 8, dtype=torch.int32, device="cuda")
    e = cf.make_epilogue(row_op="topk", topk=8, row_index=idx)
    assert cf.cf_gemm_epilogue_workspace_size(8192, 4096, 32, e) > (16 << 20)
    st = lib.cf_gemm_epilogue_noalloc(8192, 4096, 32, A.data_ptr(), 32, B.data_ptr(), 4096, 0, cf.CF_BF16,
                                      None, 0, cf.CF_BF16, ctypes.byref(e), torch.cuda.current_stream().cuda_stream)
    assert st == cf.CF_ERR_WORKSPACE
    test_noalloc_repeated_calls_stay_exact()
