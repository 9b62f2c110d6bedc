"""GPU parity of cf_gemm_epilogue (the Stage-Stream GEMM + epilogue kernel)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import b2bgemm_stage_stream_amd as cf   # noqa: E402
import oracle                           # noqa: E402
import parity as P                      # noqa: E402

_WS = cf.Workspace()


def run(A, B, out_dtype, *, b_is_nk=False, **epi):
    M = A.shape[0]
    N = B.shape[0] if b_is_nk else B.shape[1]
    e = cf.make_epilogue(**epi)
    ws = _WS.get(cf.cf_gemm_epilogue_workspace_size(M, N, A.shape[1], e))
    C = torch.empty(M, N, dtype=out_dtype, device="cuda")
    cf.cf_gemm_epilogue(A, B, C, b_is_nk=b_is_nk, epi=e, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert cf.cf_workspace_status(ws) == cf.CF_OK
    return C


def oracle_of(w, ref, rows=None):
    p = w.params
    sl = (lambda x: x) if rows is None else (lambda x: x[rows])
    return oracle.gemm_epilogue(
        sl(ref["A"]), ref["B"], alpha=p["alpha"], bias=ref.get("bias"),
        residual=None if "residual" not in ref else sl(ref["residual"]), act=p["act"],
        row_op=p["row_op"], gamma=ref.get("gamma", ref.get("weight")), beta=ref.get("beta"),
        eps=p.get("eps", 0.0))


def epi_of(w, dev):
    p = w.params
    return dict(alpha=p["alpha"], bias=dev.get("bias"), residual=dev.get("residual"), act=p["act"],
                row_op=p["row_op"], gamma=dev.get("gamma", dev.get("weight")), beta=dev.get("beta"),
                eps=p.get("eps", 0.0))


def check_bf16_workload(w, dev, ref, what):
    R = oracle_of(w, ref)
    c32 = run(dev["A"], dev["B"], torch.float32, **epi_of(w, dev))
    r, m = P.assert_close(P.gpu_to_f64(c32), R, P.REL_F_BF16, P.MAX_ABS_BF16, what + " f32-out")
    c16 = run(dev["A"], dev["B"], torch.bfloat16, **epi_of(w, dev))
    P.assert_bf16_consistent(c16, c32, R, what + " bf16-out")
    print(f"{what}: relF {r:.2e} maxabs {m:.2e}", flush=True)


# ---------------------------------------------------------------------------- fp32 path (C1)

def test_c1_softmax_f32_full_size():
    w, dev, ref = P.inputs("c1_gemm_bias_softmax_f32", seed=0)
    R = oracle_of(w, ref)
    C = run(dev["A"], dev["B"], torch.float32, **epi_of(w, dev))
    r, m = P.assert_close(P.gpu_to_f64(C), R, P.REL_F_F32, P.MAX_ABS_F32, "C1")
    assert np.allclose(P.gpu_to_f64(C).sum(1), 1.0, atol=1e-5)
    print(f"C1 relF {r:.2e} maxabs {m:.2e}")


def test_c1_softmax_large_logits():
    # logits scaled x100 exercise the max subtraction
    w, dev, ref = P.inputs("c1_gemm_bias_softmax_f32", seed=1)
    A = dev["A"] * 100.0
    R = oracle.gemm_epilogue(ref["A"] * 100.0, ref["B"], bias=ref["bias"], row_op="softmax")
    C = run(A, dev["B"], torch.float32, bias=dev["bias"], row_op="softmax")
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_F32, P.MAX_ABS_F32, "C1 x100")


@pytest.mark.parametrize("row_op", ["none", "softmax", "layernorm", "rmsnorm"])
def test_f32_row_ops_multi_tile(row_op):
    # fp32 inputs, N spanning several column tiles (strip exchange), ragged M
    w, dev, ref = P.inputs("c1_gemm_bias_softmax_f32", seed=2, M=300, N=768, K=96)
    g = torch.linspace(0.5, 1.5, 768, device="cuda")
    b = torch.linspace(-0.2, 0.2, 768, device="cuda")
    R = oracle.gemm_epilogue(ref["A"], ref["B"], bias=ref["bias"], row_op=row_op,
                             gamma=P.gpu_to_f64(g), beta=P.gpu_to_f64(b), eps=1e-5, act="relu")
    C = run(dev["A"], dev["B"], torch.float32, bias=dev["bias"], row_op=row_op, gamma=g, beta=b,
            eps=1e-5, act="relu")
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_F32, P.MAX_ABS_F32, f"f32 {row_op}")


# ---------------------------------------------------------------------------- bf16 path

def test_c2_layernorm_reduced():
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=0, M=512, K=1024)
    check_bf16_workload(w, dev, ref, "C2 512x4096x1024")


def test_c3_residual_rmsnorm_reduced():
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=0, M=384, K=1088)
    check_bf16_workload(w, dev, ref, "C3 384x4096x1088")


@pytest.mark.parametrize("seed", [1, 2])
def test_c2_seeds(seed):
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=seed, M=256, N=1024, K=512)
    check_bf16_workload(w, dev, ref, f"C2 seed {seed}")


@pytest.mark.parametrize("row_op", ["none", "softmax", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", [(33, 65, 17), (300, 520, 200), (257, 256, 64), (4, 4, 4), (1, 1000, 9)])
def test_ragged_general_path(row_op, shape):
    M, N, K = shape
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=3, M=M, N=N, K=K)
    bias = torch.linspace(-0.3, 0.3, N, device="cuda").to(torch.bfloat16)
    gamma = dev["weight"]
    beta = (torch.linspace(-0.1, 0.1, N, device="cuda")).to(torch.bfloat16)
    R = oracle.gemm_epilogue(ref["A"], ref["B"], alpha=0.5, bias=P.gpu_to_f64(bias), residual=ref["residual"],
                             act="relu", row_op=row_op, gamma=ref["weight"], beta=P.gpu_to_f64(beta), eps=1e-5)
    kw = dict(alpha=0.5, bias=bias, residual=dev["residual"], act="relu", row_op=row_op, gamma=gamma,
              beta=beta, eps=1e-5)
    c32 = run(dev["A"], dev["B"], torch.float32, **kw)
    P.assert_close(P.gpu_to_f64(c32), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"ragged {shape} {row_op}")
    c16 = run(dev["A"], dev["B"], torch.bfloat16, **kw)
    P.assert_bf16_consistent(c16, c32, R, f"ragged {shape} {row_op} bf16")


@pytest.mark.parametrize("row_op", ["none", "softmax", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("N,K", [(264, 256), (1000, 200), (4000, 64)])
def test_ragged_column_tile_fast_path(row_op, N, K):
    # N a multiple of 8, not of 256: whole column tiles take the fast epilogue
    # and each strip's last tile its masked variant (8, 232 and 160 valid
    # columns); K = 256 and 64 stream through the LDS ring, K = 200 takes the
    # register-staged loop; M = 300 leaves a ragged row strip as well
    import dataclasses
    M = 300
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=21, M=M, N=N, K=K)
    bias = torch.linspace(-0.3, 0.3, N, device="cuda").to(torch.bfloat16)
    w2 = dataclasses.replace(w, params={**w.params, "alpha": 0.5, "act": "relu", "row_op": row_op, "eps": 1e-5})
    dev2, ref2 = {**dev, "bias": bias}, {**ref, "bias": P.gpu_to_f64(bias)}
    if row_op == "layernorm":
        beta = torch.linspace(-0.1, 0.1, N, device="cuda").to(torch.bfloat16)
        dev2["beta"], ref2["beta"] = beta, P.gpu_to_f64(beta)
    check_two_outputs(w2, dev2, ref2, epi_of(w2, dev2), f"ragged column tile {M}x{N}x{K} {row_op}")


@pytest.mark.parametrize("row_op", ["layernorm", "softmax"])
def test_ragged_column_tile_b_nk(row_op):
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=22, M=256, N=1000, K=256)
    Bt = dev["B"].t().contiguous()          # [N, K]: rows past N read as zero
    R = oracle.gemm_epilogue(ref["A"], ref["B"], row_op=row_op, gamma=ref["gamma"], beta=ref["beta"], eps=1e-5)
    C = run(dev["A"], Bt, torch.float32, b_is_nk=True, row_op=row_op, gamma=dev["gamma"], beta=dev["beta"],
            eps=1e-5)
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"ragged column tile, B [N,K], {row_op}")


@pytest.mark.parametrize("row_op", ["none", "softmax", "layernorm", "rmsnorm"])
def test_ragged_column_tile_nan_past_n(row_op):
    # B is a [K, N] view of a wider buffer whose extra columns hold NaN, so the
    # ragged tile's accumulators past N are NaN: none of it may reach an output
    # or a row statistic
    M, N, K = 300, 1000, 256
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=24, M=M, N=N, K=K)
    buf = torch.full((K, N + 24), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:, :N] = dev["B"]
    B = buf[:, :N]
    beta_d, beta_r = (dev["beta"], ref["beta"]) if row_op == "layernorm" else (None, None)
    R = oracle.gemm_epilogue(ref["A"], ref["B"], row_op=row_op, gamma=ref["gamma"], beta=beta_r, eps=1e-5)
    c32 = run(dev["A"], B, torch.float32, row_op=row_op, gamma=dev["gamma"], beta=beta_d, eps=1e-5)
    P.assert_close(P.gpu_to_f64(c32), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"NaN past N, {row_op}")
    c16 = run(dev["A"], B, torch.bfloat16, row_op=row_op, gamma=dev["gamma"], beta=beta_d, eps=1e-5)
    P.assert_bf16_consistent(c16, c32, R, f"NaN past N, {row_op} bf16")


# ---------------------------------------------------------------------------- two row stages
def _vec(rng, n, mu, sd):
    return torch.from_numpy(rng.normal(mu, sd, n)).to(torch.bfloat16).cuda()


def _f64(t):
    return None if t is None else P.gpu_to_f64(t)


@pytest.mark.parametrize("op1,op2", [("layernorm", "softmax"), ("softmax", "layernorm"), ("rmsnorm", "rmsnorm"),
                                     ("layernorm", "rmsnorm"), ("softmax", "softmax"), ("rmsnorm", "layernorm")])
@pytest.mark.parametrize("N", [256, 1024, 1000])
def test_two_row_stages(op1, op2, N):
    # a second reduction boundary: z = op2(op1(x)), each stage with its own
    # affine vectors and eps; one column tile (no exchange), four, and four
    # with a ragged last one per strip; M = 300 leaves a ragged row strip
    M, K = 300, 256
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=31, M=M, N=N, K=K)
    rng = np.random.default_rng(32)
    bias = _vec(rng, N, 0.0, 0.3)
    g1 = _vec(rng, N, 1.0, 0.1) if op1 != "softmax" else None
    b1 = _vec(rng, N, 0.0, 0.1) if op1 == "layernorm" else None
    g2 = _vec(rng, N, 1.0, 0.2) if op2 != "softmax" else None
    b2 = _vec(rng, N, 0.0, 0.2) if op2 == "layernorm" else None
    kw = dict(alpha=0.5, bias=bias, residual=dev["residual"], act="relu", row_op=op1, gamma=g1, beta=b1, eps=1e-5,
              row_op2=op2, gamma2=g2, beta2=b2, eps2=1e-3)
    R = oracle.gemm_epilogue_two_stage(ref["A"], ref["B"], alpha=0.5, bias=_f64(bias), residual=ref["residual"],
                                       act="relu", row_op=op1, gamma=_f64(g1), beta=_f64(b1), eps=1e-5, row_op2=op2,
                                       gamma2=_f64(g2), beta2=_f64(b2), eps2=1e-3)
    c32 = run(dev["A"], dev["B"], torch.float32, **kw)
    r, m = P.assert_close(P.gpu_to_f64(c32), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"{op1} -> {op2} N={N}")
    c16 = run(dev["A"], dev["B"], torch.bfloat16, **kw)
    P.assert_bf16_consistent(c16, c32, R, f"{op1} -> {op2} N={N} bf16")
    print(f"{op1} -> {op2} N={N}: relF {r:.2e} maxabs {m:.2e}", flush=True)


def test_two_row_stages_b_nk_with_x_and_stats():
    # B given [N, K]; the second output X (the first stage's input) and the
    # first stage's row statistics beside the two-stage result
    M, N, K = 300, 1024, 512
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=33, M=M, N=N, K=K)
    rng = np.random.default_rng(34)
    g2 = _vec(rng, N, 1.0, 0.2)
    Bt = dev["B"].t().contiguous()
    Xo = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.full((2 * M,), float("nan"), dtype=torch.float32, device="cuda")
    kw = dict(row_op="layernorm", gamma=dev["gamma"], beta=dev["beta"], eps=1e-5, row_op2="rmsnorm", gamma2=g2,
              eps2=1e-6, x_out=Xo, row_stats=st)
    C = run(dev["A"], Bt, torch.float32, b_is_nk=True, **kw)
    R = oracle.gemm_epilogue_two_stage(ref["A"], ref["B"], row_op="layernorm", gamma=ref["gamma"], beta=ref["beta"],
                                       eps=1e-5, row_op2="rmsnorm", gamma2=_f64(g2), eps2=1e-6)
    Xr = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_BF16, P.MAX_ABS_BF16, "LN -> RMS, B [N,K]")
    P.assert_close(P.gpu_to_f64(Xo), Xr, 1e-5, 1e-4, "X beside two stages")
    S = oracle.row_statistics(Xr, "layernorm", 1e-5).reshape(-1)
    P.assert_close(P.gpu_to_f64(st), S, REL_F_STATS, MAX_ABS_STATS, "first-stage statistics beside two stages")


@pytest.mark.parametrize("row_op", ["layernorm", "softmax"])
def test_b_nk_layout(row_op):
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=4, M=256, N=512, K=256)
    Bt = dev["B"].t().contiguous()          # [N, K]
    R = oracle.gemm_epilogue(ref["A"], ref["B"], row_op=row_op, gamma=ref["gamma"], beta=ref["beta"], eps=1e-5)
    C = run(dev["A"], Bt, torch.float32, b_is_nk=True, row_op=row_op, gamma=dev["gamma"], beta=dev["beta"],
            eps=1e-5)
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"B [N,K] {row_op}")


@pytest.mark.parametrize("b_is_nk", [False, True])
@pytest.mark.parametrize("K", [32, 40, 96, 128, 160, 264, 1056])
def test_k_depths_both_layouts(K, b_is_nk):
    # K a multiple of 32: operands stream through the LDS stage ring (1, 3, 4, 5
    # and 33 stages: fewer, as many and more than the ring holds); K = 40 and
    # 264 (multiples of 8 only) take the register-staged loop. M = 300 leaves a
    # ragged last row strip.
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=7, M=300, N=512, K=K)
    B = dev["B"].t().contiguous() if b_is_nk else dev["B"]
    R = oracle_of(w, ref)
    C = run(dev["A"], B, torch.float32, b_is_nk=b_is_nk, **epi_of(w, dev))
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"K={K} nk={b_is_nk}")


def test_fp32_residual_unaligned_ld():
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=5, M=64, N=512, K=128)
    R32 = torch.randn(64, 520, device="cuda")[:, :512]      # fp32 residual, ld 520
    R = oracle.gemm_epilogue(ref["A"], ref["B"], residual=P.gpu_to_f64(R32), row_op="rmsnorm",
                             gamma=ref["weight"], eps=1e-6)
    C = run(dev["A"], dev["B"], torch.float32, residual=R32, row_op="rmsnorm", gamma=dev["weight"], eps=1e-6)
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_BF16, P.MAX_ABS_BF16, "fp32 residual")


def test_k_zero_and_empty():
    A = torch.zeros(8, 0, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda")
    bias = torch.arange(16, dtype=torch.float32, device="cuda")
    C = run(A, B, torch.float32, bias=bias)
    assert torch.equal(C, bias.expand(8, 16))
    E = torch.empty(0, 16, dtype=torch.float32, device="cuda")
    cf.cf_gemm_epilogue(torch.zeros(0, 4, dtype=torch.bfloat16, device="cuda"),
                        torch.zeros(4, 16, dtype=torch.bfloat16, device="cuda"), E)


@pytest.fixture(params=["peer-to-peer", "leader-follower"])
def exchange_mode(request):
    """Runs a test with every strip exchanging peer-to-peer, then with every
    strip of two or more tiles exchanging leader-follower."""
    old = cf.cf_set_exchange_leader_tiles(0 if request.param == "peer-to-peer" else 2)
    yield request.param
    cf.cf_set_exchange_leader_tiles(old)


def test_exchange_timeout_is_reported_and_recoverable(exchange_mode):
    # A zero spin limit (forced from the host) makes a workgroup give up on
    # peers that have not published yet: the launch still completes (every
    # wait is bounded) and the workspace reports the timeout. After a reset and
    # with the normal limit the same call is exact again.
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=13, M=512, K=256)
    e = cf.make_epilogue(**epi_of(w, dev))
    ws = cf.Workspace().get(cf.cf_gemm_epilogue_workspace_size(512, 4096, 256, e))
    C = torch.empty(512, 4096, dtype=torch.float32, device="cuda")
    R = oracle_of(w, ref)
    old = cf.cf_set_exchange_timeout_us(0)
    try:
        seen = set()
        for _ in range(3):
            C.fill_(0.0)
            cf.cf_gemm_epilogue(dev["A"], dev["B"], C, epi=e, workspace=ws)
            st = cf.cf_workspace_status(ws)
            assert st in (cf.CF_OK, cf.CF_ERR_DEVICE_TIMEOUT)
            seen.add(st)
            # a row segment whose peers' statistics never arrived is NaN, every
            # other element is exact; NaN appears exactly when a timeout is reported
            G = P.gpu_to_f64(C)
            nan = np.isnan(G)
            assert nan.any() == (st == cf.CF_ERR_DEVICE_TIMEOUT)
            ok = ~nan
            assert np.abs(G[ok] - R[ok]).max(initial=0.0) <= P.MAX_ABS_BF16
            if st != cf.CF_OK:
                cf.cf_workspace_init(ws)
                assert cf.cf_workspace_status(ws) == cf.CF_OK
    finally:
        cf.cf_set_exchange_timeout_us(old)
    print(f"statuses with a zero spin limit: {sorted(seen)}", flush=True)
    cf.cf_gemm_epilogue(dev["A"], dev["B"], C, epi=e, workspace=ws)
    assert cf.cf_workspace_status(ws) == cf.CF_OK
    P.assert_close(P.gpu_to_f64(C), oracle_of(w, ref), P.REL_F_BF16, P.MAX_ABS_BF16, "after timeout recovery")


# ---------------------------------------------------------------------------- structure

def test_deterministic_and_row_local():
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=6, M=512, N=2048, K=256)
    kw = epi_of(w, dev)
    c1 = run(dev["A"], dev["B"], torch.bfloat16, **kw)
    c2 = run(dev["A"], dev["B"], torch.bfloat16, **kw)
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16)), "not deterministic"
    # Eq. (1) locality: changing row 77 of A changes no other output row
    A2 = dev["A"].clone()
    A2[77] = -A2[77] * 2
    c3 = run(A2, dev["B"], torch.bfloat16, **kw)
    diff = (c3.view(torch.int16) != c1.view(torch.int16)).any(dim=1).cpu().numpy()
    assert diff[77] and diff.sum() == 1


# ---------------------------------------------------------------------------- full sizes, sampled rows

@pytest.mark.parametrize("name", ["c2_gemm_layernorm", "c3_gemm_residual_rmsnorm"])
def test_full_size_all_rows(name):
    # the full workload in the launch configuration bench.py times: every row
    # (every strip of the exchange) against the oracle, fp32 and bf16 outputs
    w, dev, ref = P.inputs(name, seed=0)
    R = oracle_of(w, ref)
    kw = epi_of(w, dev)
    c32 = run(dev["A"], dev["B"], torch.float32, **kw)
    r, m = P.assert_close(P.gpu_to_f64(c32), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"{name} full size")
    c16 = run(dev["A"], dev["B"], torch.bfloat16, **kw)
    P.assert_bf16_consistent(c16, c32, R, f"{name} full size bf16")
    print(f"{name} full: relF {r:.2e} maxabs {m:.2e}", flush=True)


# ---------------------------------------------------------------------------- second output: x before the row op

def run_x(A, B, out_dtype, x_dtype, **epi):
    """Like run(), with X (the elementwise stage's result) stored to a second output."""
    M, N = A.shape[0], B.shape[1]
    Xo = torch.full((M, N), float("nan"), dtype=x_dtype, device="cuda")
    C = run(A, B, out_dtype, x_out=Xo, **epi)
    return C, Xo


def check_two_outputs(w, dev, ref, kw, what):
    p = w.params
    Yr, Xr = oracle.gemm_epilogue_with_x(
        ref["A"], ref["B"], alpha=p["alpha"], bias=ref.get("bias"), residual=ref.get("residual"), act=p["act"],
        row_op=p["row_op"], gamma=ref.get("gamma", ref.get("weight")), beta=ref.get("beta"), eps=p.get("eps", 0.0))
    y_plain = run(dev["A"], dev["B"], torch.bfloat16, **kw)
    y32, x32 = run_x(dev["A"], dev["B"], torch.float32, torch.float32, **kw)
    P.assert_close(P.gpu_to_f64(y32), Yr, P.REL_F_BF16, P.MAX_ABS_BF16, what + " Y f32")
    P.assert_close(P.gpu_to_f64(x32), Xr, P.REL_F_BF16, P.MAX_ABS_BF16, what + " X f32")
    y16, x16 = run_x(dev["A"], dev["B"], torch.bfloat16, torch.bfloat16, **kw)
    # the second sink changes nothing in the first, and stores the same fp32 x rounded once
    assert torch.equal(y16.view(torch.int16), y_plain.view(torch.int16)), what + ": Y changed by storing X"
    P.assert_bf16_consistent(y16, y32, Yr, what + " Y bf16")
    P.assert_bf16_consistent(x16, x32, Xr, what + " X bf16")
    r, m = P.metrics(P.gpu_to_f64(x32), Xr)
    print(f"{what}: X relF {r:.2e} maxabs {m:.2e}", flush=True)


def test_x_out_residual_rmsnorm_fast_path():
    # pre-norm block: the new residual stream X = P + R beside Y = RMSNorm(X)
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=6, M=300, N=1024, K=512)
    check_two_outputs(w, dev, ref, epi_of(w, dev), "C3-shaped 300x1024x512 + X")


@pytest.mark.parametrize("row_op", ["none", "softmax", "layernorm"])
def test_x_out_with_bias_alpha_relu(row_op):
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=7, M=256, N=768, K=256)
    bias = torch.linspace(-0.3, 0.3, 768, device="cuda").to(torch.bfloat16)
    beta = torch.linspace(-0.1, 0.1, 768, device="cuda").to(torch.bfloat16)
    import dataclasses
    w2 = dataclasses.replace(w, params={**w.params, "alpha": 0.5, "act": "relu", "row_op": row_op})
    dev2 = {**dev, "bias": bias, "beta": beta}
    ref2 = {**ref, "bias": P.gpu_to_f64(bias), "beta": P.gpu_to_f64(beta)}
    check_two_outputs(w2, dev2, ref2, epi_of(w2, dev2), f"X with alpha/bias/relu, {row_op}")


@pytest.mark.parametrize("shape", [(33, 65, 17), (300, 520, 200), (1, 1000, 9)])
def test_x_out_general_path(shape):
    M, N, K = shape
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=8, M=M, N=N, K=K)
    check_two_outputs(w, dev, ref, epi_of(w, dev), f"X general path {shape}")


def test_x_out_full_size_all_rows():
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=0)
    p = w.params
    Yr, Xr = oracle.gemm_epilogue_with_x(ref["A"], ref["B"], residual=ref["residual"], row_op="rmsnorm",
                                         gamma=ref["weight"], eps=p["eps"])
    y16, x16 = run_x(dev["A"], dev["B"], torch.bfloat16, torch.bfloat16, **epi_of(w, dev))
    P.assert_bf16_within(P.gpu_to_f64(y16), Yr, "C3 full Y")
    P.assert_bf16_within(P.gpu_to_f64(x16), Xr, "C3 full X")
    assert P.metrics(P.gpu_to_f64(x16), oracle.round_bf16(Xr))[0] <= P.REL_F_BF16


# ---------------------------------------------------------------------------- leader-follower exchange

@pytest.mark.parametrize("N,M", [(512, 300), (4096, 300), (8192, 300), (16384, 300), (65536, 64)])
@pytest.mark.parametrize("row_op", ["softmax", "layernorm", "rmsnorm", "argmax"])
def test_leader_follower_equals_peer_to_peer(N, M, row_op):
    # the two aggregation modes merge the same partials in the same order:
    # bit-identical outputs (and row statistics), both within the oracle's bars
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=19, M=M, N=N, K=128)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    outs = {}
    for mode, tiles in (("p2p", 0), ("lf", 2)):
        old = cf.cf_set_exchange_leader_tiles(tiles)
        try:
            if row_op == "argmax":
                outs[mode] = run_argmax(dev["A"], dev["B"], False)[:2]
            else:
                st = torch.full((M, 2) if row_op == "layernorm" else (M,), float("nan"), device="cuda")
                C = run(dev["A"], dev["B"], torch.float32, row_op=row_op, gamma=dev["gamma"],
                        beta=dev["beta"] if row_op == "layernorm" else None, eps=1e-5, row_stats=st)
                outs[mode] = (C, st)
        finally:
            cf.cf_set_exchange_leader_tiles(old)
    for a, b in zip(outs["p2p"], outs["lf"]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"N={N} {row_op}: modes differ"
    if row_op == "argmax":
        check_argmax(outs["lf"][0], outs["lf"][1], X, f"leader-follower argmax N={N}")
    else:
        R = oracle.row_stage(X, row_op, ref["gamma"], ref["beta"] if row_op == "layernorm" else None, 1e-5)
        P.assert_close(P.gpu_to_f64(outs["lf"][0]), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"leader-follower {row_op} N={N}")


# ---------------------------------------------------------------------------- column reductions

def check_columns(w, dev, ref, col_op, what, b_is_nk=False, **extra):
    """A column reduction (softmax / LayerNorm / RMSNorm over the rows of each
    column) against the oracle: fp32 and bf16 outputs and the per-column
    statistics."""
    M, N = w.dims["M"], w.dims["N"]
    g = dev.get("gamma", dev.get("weight"))
    gr = ref.get("gamma", ref.get("weight"))
    ln = col_op == "layernorm"
    st = torch.full((N, 2) if ln else (N,), float("nan"), dtype=torch.float32, device="cuda")
    kw = dict(row_op=col_op, axis="column", gamma=None if col_op == "softmax" else g,
              beta=dev["beta"] if ln else None, eps=1e-5, row_stats=st, **extra)
    B = dev["B"].t().contiguous() if b_is_nk else dev["B"]
    c32 = run(dev["A"], B, torch.float32, b_is_nk=b_is_nk, **kw)
    rkw = dict(alpha=extra.get("alpha", 1.0), act=extra.get("act", "none"),
               bias=None if extra.get("bias") is None else P.gpu_to_f64(extra["bias"]),
               residual=None if extra.get("residual") is None else P.gpu_to_f64(extra["residual"]))
    R = oracle.gemm_epilogue_columns(ref["A"], ref["B"], col_op=col_op, gamma=None if col_op == "softmax" else gr,
                                     beta=ref["beta"] if ln else None, eps=1e-5, **rkw)
    r, m = P.assert_close(P.gpu_to_f64(c32), R, P.REL_F_BF16, P.MAX_ABS_BF16, what + " f32-out")
    Rs = oracle.gemm_epilogue_column_stats(ref["A"], ref["B"], col_op=col_op, eps=1e-5, **rkw)
    P.assert_close(P.gpu_to_f64(st), Rs, 1e-5, 1e-4, what + " column statistics")
    kw["row_stats"] = None
    c16 = run(dev["A"], B, torch.bfloat16, b_is_nk=b_is_nk, **kw)
    P.assert_bf16_consistent(c16, c32, R, what + " bf16-out")
    print(f"{what}: relF {r:.2e} maxabs {m:.2e}", flush=True)
    return c32


@pytest.mark.parametrize("col_op", ["softmax", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", [(256, 512, 128), (700, 768, 256), (1000, 264, 64), (2048, 1024, 512),
                                   (8192, 512, 64)])
def test_column_reductions(col_op, shape):
    # one row strip, ragged strips and column tiles, 32 strips per tile column
    M, N, K = shape
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=31, M=M, N=N, K=K)
    check_columns(w, dev, ref, col_op, f"column {col_op} {shape}")


@pytest.mark.parametrize("col_op", ["softmax", "layernorm", "rmsnorm"])
def test_column_reductions_with_epilogue_and_nk(col_op):
    # alpha, bias, residual and ReLU before the column reduction; B given [N, K]
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=32, M=600, N=1024, K=256)
    dev["gamma"], ref["gamma"] = dev["weight"], ref["weight"]
    beta = torch.linspace(-0.2, 0.2, 1024, device="cuda").to(torch.bfloat16)
    bias = torch.linspace(-0.5, 0.5, 1024, device="cuda").to(torch.bfloat16)
    dev["beta"], ref["beta"] = beta, P.gpu_to_f64(beta)
    check_columns(w, dev, ref, col_op, f"column {col_op} + alpha/bias/residual/relu, B[N,K]", b_is_nk=True,
                  alpha=0.5, bias=bias, residual=dev["residual"], act="relu")


def test_column_softmax_fp32_inputs_and_large_logits():
    w, dev, ref = P.inputs("c1_gemm_bias_softmax_f32", seed=33, M=700, N=512, K=96)
    dev["A"] = dev["A"] * 40.0
    ref["A"] = P.gpu_to_f64(dev["A"])
    g = torch.ones(512, device="cuda")
    st = torch.empty(512, dtype=torch.float32, device="cuda")
    C = run(dev["A"], dev["B"], torch.float32, row_op="softmax", axis="column", bias=dev["bias"], row_stats=st)
    R = oracle.gemm_epilogue_columns(ref["A"], ref["B"], bias=ref["bias"], col_op="softmax")
    P.assert_close(P.gpu_to_f64(C), R, P.REL_F_F32, P.MAX_ABS_F32, "fp32 column softmax, logits x40")
    del g


def test_column_reduction_modes_and_locality():
    # leader-follower equals peer-to-peer bit for bit; column n of the output
    # depends on column n of B only (the transposed Eq. (1) locality)
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=34, M=4096, N=768, K=256)
    kw = dict(row_op="layernorm", axis="column", gamma=dev["gamma"], beta=dev["beta"], eps=1e-5)
    outs = []
    for tiles in (0, 2):
        old = cf.cf_set_exchange_leader_tiles(tiles)
        try:
            outs.append(run(dev["A"], dev["B"], torch.bfloat16, **kw))
        finally:
            cf.cf_set_exchange_leader_tiles(old)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    B2 = dev["B"].clone()
    B2[:, 77] = -B2[:, 77] * 2
    c2 = run(dev["A"], B2, torch.bfloat16, **kw)
    diff = (c2.view(torch.int16) != outs[0].view(torch.int16)).any(dim=0).cpu().numpy()
    assert diff[77] and diff.sum() == 1


# ---------------------------------------------------------------------------- wide strips

@pytest.mark.parametrize("N", [8192, 16384])
@pytest.mark.parametrize("row_op", ["softmax", "layernorm", "rmsnorm"])
def test_wide_strips(N, row_op):
    # strips of 32 and 64 column tiles: every workgroup of a strip merges that
    # many peers' partial statistics (the C2/C3 strips have 16)
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=9, M=300, N=N, K=128)
    R = oracle.gemm_epilogue(ref["A"], ref["B"], row_op=row_op, gamma=ref["gamma"],
                             beta=ref["beta"] if row_op == "layernorm" else None, eps=1e-5)
    kw = dict(row_op=row_op, gamma=dev["gamma"], beta=dev["beta"] if row_op == "layernorm" else None, eps=1e-5)
    c32 = run(dev["A"], dev["B"], torch.float32, **kw)
    P.assert_close(P.gpu_to_f64(c32), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"N={N} {row_op}")
    c16 = run(dev["A"], dev["B"], torch.bfloat16, **kw)
    P.assert_bf16_consistent(c16, c32, R, f"N={N} {row_op} bf16")


# ---------------------------------------------------------------------------- row statistics of the reduction

REL_F_STATS, MAX_ABS_STATS = 1e-5, 1e-4   # fp32 statistics of the fp32 x


def stats_of(w, dev, ref, row_op, shape_out=torch.bfloat16, **extra):
    M = dev["A"].shape[0]
    st = torch.full((M, 2) if row_op == "layernorm" else (M,), float("nan"), dtype=torch.float32, device="cuda")
    kw = {**epi_of(w, dev), "row_op": row_op, **extra}
    run(dev["A"], dev["B"], shape_out, row_stats=st, **kw)
    p = w.params
    R = oracle.gemm_epilogue_row_stats(ref["A"], ref["B"], alpha=kw.get("alpha", 1.0), bias=ref.get("bias"),
                                       residual=ref.get("residual"), act=kw.get("act", "none"), row_op=row_op,
                                       eps=kw.get("eps", 0.0))
    return P.gpu_to_f64(st), R


@pytest.mark.parametrize("row_op", ["softmax", "layernorm", "rmsnorm"])
def test_row_stats_fast_path(row_op):
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=15, M=300, N=1024, K=256)
    got, R = stats_of(w, dev, ref, row_op, eps=1e-5, beta=None)
    P.assert_close(got, R, REL_F_STATS, MAX_ABS_STATS, f"row stats {row_op}")


@pytest.mark.parametrize("shape", [(33, 65, 17), (300, 520, 200)])
@pytest.mark.parametrize("row_op", ["softmax", "layernorm", "rmsnorm"])
def test_row_stats_general_path(shape, row_op):
    M, N, K = shape
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=16, M=M, N=N, K=K)
    got, R = stats_of(w, dev, ref, row_op, eps=1e-5, beta=None)
    P.assert_close(got, R, REL_F_STATS, MAX_ABS_STATS, f"row stats {row_op} {shape}")


def test_row_stats_f32_softmax_logsumexp():
    w, dev, ref = P.inputs("c1_gemm_bias_softmax_f32", seed=17, M=300, N=768, K=96)
    st = torch.empty(300, dtype=torch.float32, device="cuda")
    C = run(dev["A"] * 30.0, dev["B"], torch.float32, bias=dev["bias"], row_op="softmax", row_stats=st)
    R = oracle.gemm_epilogue_row_stats(ref["A"] * 30.0, ref["B"], bias=ref["bias"], row_op="softmax")
    P.assert_close(P.gpu_to_f64(st), R, REL_F_STATS, MAX_ABS_STATS, "f32 log-sum-exp")
    # consistency with the stored softmax: y = exp(x - lse)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"] * 30.0, ref["B"]), bias=ref["bias"])
    P.assert_close(P.gpu_to_f64(C), np.exp(X - P.gpu_to_f64(st)[:, None]), REL_F_STATS, MAX_ABS_STATS, "y = exp(x - lse)")


# ---------------------------------------------------------------------------- row argmax

def run_argmax(A, B, with_c, **epi):
    M, N = A.shape[0], B.shape[1]
    idx = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    val = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    e = cf.make_epilogue(row_op="argmax", row_index=idx, row_stats=val, **epi)
    ws = _WS.get(cf.cf_gemm_epilogue_workspace_size(M, N, A.shape[1], e))
    C = torch.empty(M, N, dtype=torch.float32, device="cuda") if with_c else None
    cf.cf_gemm_epilogue(A, B, C, epi=e, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert cf.cf_workspace_status(ws) == cf.CF_OK
    return idx, val, C


def check_argmax(idx, val, X, what):
    """The maximum matches; the column is the oracle's wherever the row maximum is
    separated from the runner-up by more than the fp32 rounding bound, and is
    otherwise a column within that bound of the maximum (several answers are then
    correct up to rounding)."""
    oi, ov = oracle.row_argmax(X)
    gi = idx.cpu().numpy().astype(np.int64)
    P.assert_close(P.gpu_to_f64(val), ov, 1e-5, 1e-4, what + " max value")
    tol = 1e-4 * max(1.0, float(np.abs(X).max()))
    rows = np.arange(X.shape[0])
    assert np.all((gi >= 0) & (gi < X.shape[1])), what + ": column out of range"
    srt = np.sort(X, axis=1)
    sep = (srt[:, -1] - srt[:, -2]) > tol if X.shape[1] > 1 else np.ones(X.shape[0], bool)
    bad = int((gi[sep] != oi[sep]).sum())
    assert bad == 0, f"{what}: {bad} rows with a separated maximum disagree"
    assert np.all(X[rows, gi] >= ov - tol), what + ": a chosen column is not a maximum"


@pytest.mark.parametrize("N", [256, 1024, 4096])
def test_argmax_fast_path(N):
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=19, M=300, N=N, K=512)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    idx, val, _ = run_argmax(dev["A"], dev["B"], False)
    check_argmax(idx, val, X, f"argmax N={N}")


@pytest.mark.parametrize("N", [264, 1000])
def test_argmax_ragged_column_tile(N):
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=23, M=300, N=N, K=256)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    idx, val, _ = run_argmax(dev["A"], dev["B"], False)
    check_argmax(idx, val, X, f"argmax ragged column tile N={N}")


@pytest.mark.parametrize("shape", [(33, 65, 17), (300, 520, 200), (1, 1000, 9)])
def test_argmax_general_path_with_logits(shape):
    M, N, K = shape
    w, dev, ref = P.inputs("c3_gemm_residual_rmsnorm", seed=20, M=M, N=N, K=K)
    bias = torch.linspace(-0.3, 0.3, N, device="cuda").to(torch.bfloat16)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]), 0.5, P.gpu_to_f64(bias), ref["residual"], "relu")
    idx, val, C = run_argmax(dev["A"], dev["B"], True, alpha=0.5, bias=bias, residual=dev["residual"], act="relu")
    check_argmax(idx, val, X, f"argmax {shape}")
    P.assert_close(P.gpu_to_f64(C), X, P.REL_F_BF16, P.MAX_ABS_BF16, f"argmax {shape}: C = x")


def run_topk(A, B, k, with_c, b_is_nk=False, **epi):
    M, N = A.shape[0], (B.shape[0] if b_is_nk else B.shape[1])
    idx = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    val = torch.full((M, k), float("nan"), dtype=torch.float32, device="cuda")
    e = cf.make_epilogue(row_op="topk", topk=k, row_index=idx, row_stats=val, **epi)
    ws = _WS.get(cf.cf_gemm_epilogue_workspace_size(M, N, A.shape[1], e))
    C = torch.empty(M, N, dtype=torch.float32, device="cuda") if with_c else None
    cf.cf_gemm_epilogue(A, B, C, b_is_nk=b_is_nk, epi=e, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert cf.cf_workspace_status(ws) == cf.CF_OK
    return idx, val, C


def check_topk(idx, val, X, k, what):
    """The k values match the oracle's rank by rank; the columns are the
    oracle's wherever the k + 1 largest values of the row are separated by more
    than the fp32 rounding bound, and otherwise distinct columns whose exact
    values lie within that bound of the oracle's value of the same rank."""
    oi, ov = oracle.row_topk(X, k)
    gi = idx.cpu().numpy().astype(np.int64)
    P.assert_close(P.gpu_to_f64(val), ov, 1e-5, 1e-4, what + " values")
    tol = 1e-4 * max(1.0, float(np.abs(X).max()))
    assert np.all((gi >= 0) & (gi < X.shape[1])), what + ": column out of range"
    assert all(len(set(r)) == k for r in gi.tolist()), what + ": repeated column"
    rows = np.arange(X.shape[0])[:, None]
    assert np.all(np.abs(X[rows, gi] - ov) <= tol), what + ": a chosen column is not of its rank"
    srt = -np.sort(-X, axis=1)[:, :min(k + 1, X.shape[1])]
    sep = np.all(np.abs(np.diff(srt, axis=1)) > tol, axis=1)
    bad = int((gi[sep] != oi[sep]).any(axis=1).sum())
    assert bad == 0, f"{what}: {bad} rows with separated values disagree"


@pytest.mark.parametrize("k", [1, 2, 4, 5, 8])
@pytest.mark.parametrize("N", [256, 1000, 4096])
def test_topk(N, k):
    # k = 1 runs as the argmax, k <= 4 on lists of 4, k > 4 on lists of 8
    # one column tile per strip (no exchange), four with a ragged one, sixteen
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=41, M=300, N=N, K=256)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    idx, val, _ = run_topk(dev["A"], dev["B"], k, False)
    check_topk(idx, val, X, k, f"top-{k} N={N}")


def test_topk_with_logits_bias_relu():
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=42, M=300, N=1000, K=256)
    bias = torch.linspace(-0.3, 0.3, 1000, device="cuda").to(torch.bfloat16)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]), 0.5, P.gpu_to_f64(bias), None, "relu")
    idx, val, C = run_topk(dev["A"], dev["B"], 5, True, alpha=0.5, bias=bias, act="relu")
    check_topk(idx, val, X, 5, "top-5 of relu logits")
    P.assert_close(P.gpu_to_f64(C), X, P.REL_F_BF16, P.MAX_ABS_BF16, "top-5: C = x")


def test_topk_exact_ties_across_tiles():
    # five equal columns (duplicated B columns, equal bias) that are the row
    # maximum in every row: the top-3 are the three lowest of them, in order
    M, N, K = 256, 4096, 256
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=43, M=M, N=N, K=K)
    cols = (5, 700, 3000, 3001, 4095)
    B = dev["B"].clone()
    for c in cols[1:]:
        B[:, c] = B[:, cols[0]]
    bias = torch.zeros(N, device="cuda").to(torch.bfloat16)
    bias[list(cols)] = 50.0
    idx, val, _ = run_topk(dev["A"], B, 3, False, bias=bias)
    got = idx.cpu().numpy()
    assert np.all(got == np.array(cols[:3])[None, :]), got[:4]
    v = val.cpu().numpy()
    assert np.all(v[:, 0] == v[:, 1]) and np.all(v[:, 1] == v[:, 2])


def test_topk_nonfinite():
    # +inf bias columns rank first, in column order; a NaN row ranks every
    # column as -inf, so its top-k are the lowest columns with value -inf; a row
    # whose only finite values are two columns fills the rest with the lowest
    # -inf columns (empty list entries must give way to real -inf ones, across
    # lanes and column tiles, with a ragged last tile)
    M, N, K = 256, 1000, 256
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=45, M=M, N=N, K=K)
    A = dev["A"].clone()
    A[7] = float("nan")
    bias = torch.zeros(N, device="cuda", dtype=torch.float32)
    bias[[3, 511, 998]] = float("inf")
    idx, val, _ = run_topk(A, dev["B"], 3, False, bias=bias)
    got, v = idx.cpu().numpy(), val.cpu().numpy()
    others = np.arange(M) != 7
    assert np.all(got[others] == np.array([3, 511, 998])[None, :]), got[:2]
    assert np.all(v[others] == np.inf)
    assert list(got[7]) == [0, 1, 2] and np.all(v[7] == -np.inf), (got[7], v[7])

    bias = torch.full((N,), float("-inf"), device="cuda", dtype=torch.bfloat16)
    bias[[17, 900]] = 0.0
    idx, val, _ = run_topk(A, dev["B"], 5, False, bias=bias)
    got, v = idx.cpu().numpy(), val.cpu().numpy()
    Aref = ref["A"].copy()
    Aref[7] = np.nan
    X = oracle.elementwise_stage(oracle.matmul(Aref, ref["B"]), 1.0, P.gpu_to_f64(bias), None, "none")
    oi, ov = oracle.row_topk(X, 5)
    assert np.array_equal(got, oi), np.argwhere(got != oi)[:4]
    fin = np.isfinite(ov)
    assert np.all(np.abs(v[fin] - ov[fin]) <= 1e-4 * np.maximum(1.0, np.abs(ov[fin])))
    assert np.all(v[~fin] == -np.inf)
    assert list(got[7]) == [0, 1, 2, 3, 4]
    assert all(sorted(r[:2]) == [17, 900] and list(r[2:]) == [0, 1, 2] for r in got[others])


@pytest.mark.parametrize("N", [1000, 4096])
def test_topk_relu_zero_ties(N):
    # ReLU clamps all but two columns to exactly 0: the top-8 are those two,
    # then the six lowest zero columns in column order (equal values behind an
    # insertion keep their order within every lane's list)
    M, K = 256, 256
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=47, M=M, N=N, K=K)
    bias = torch.full((N,), -50.0, device="cuda", dtype=torch.bfloat16)
    bias[[17, N - 100]] = 50.0
    idx, val, _ = run_topk(dev["A"], dev["B"], 8, False, bias=bias, act="relu")
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]), 1.0, P.gpu_to_f64(bias), None, "relu")
    oi, ov = oracle.row_topk(X, 8)
    got = idx.cpu().numpy()
    assert np.array_equal(got, oi), np.argwhere(got != oi)[:4]
    assert all(list(r[2:]) == [0, 1, 2, 3, 4, 5] for r in got)
    P.assert_close(P.gpu_to_f64(val), ov, 1e-5, 1e-4, "relu top-8 values")


def test_topk_full_size_all_rows():
    # C2 shape (8192 x 4096 x 4096, sixteen column tiles per strip), top-8 of
    # every row, in the launch configuration bench.py times
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=0)
    idx, val, _ = run_topk(dev["A"], dev["B"], 8, False)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    check_topk(idx, val, X, 8, "top-8 C2 full size")


@pytest.mark.parametrize("k", [3, 8])
def test_topk_b_nk(k):
    # B given [N, K] (the nn.Linear weight layout), ragged last column tile;
    # lists of 4 (k = 3) and of 8
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=48, M=300, N=1000, K=256)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    idx, val, _ = run_topk(dev["A"], dev["B"].t().contiguous(), k, False, b_is_nk=True)
    check_topk(idx, val, X, k, f"top-{k} B[N,K]")


def test_topk_one_is_argmax():
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=44, M=300, N=1000, K=256)
    i1, v1, _ = run_topk(dev["A"], dev["B"], 1, False)
    ia, va, _ = run_argmax(dev["A"], dev["B"], False)
    assert torch.equal(i1[:, 0], ia) and torch.equal(v1[:, 0], va)


@pytest.mark.parametrize("N,cols", [(4096, (5, 700, 3000)), (300, (7, 260, 299))])
def test_argmax_exact_ties_across_tiles(N, cols):
    # equal columns of B and equal bias give bit-identical x in every row; a large
    # bias makes them the row maximum, so the lowest of them must win in every row
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=21, M=260, N=N, K=256)
    B = dev["B"].clone()
    for c in cols[1:]:
        B[:, c] = B[:, cols[0]]
    bias = torch.zeros(N, device="cuda", dtype=torch.bfloat16)
    bias[list(cols)] = 50.0
    idx, val, _ = run_argmax(dev["A"], B, False, bias=bias)
    assert torch.all(idx == cols[0]), f"ties resolved to {torch.unique(idx).tolist()}"


@pytest.mark.parametrize("N", [1000, 300])
def test_argmax_nonfinite(N):
    # a NaN row ranks every column as -inf and names column 0; with -inf bias
    # on all but two columns the maximum is the larger of those two; with -inf
    # everywhere every row names column 0 (never an out-of-range column)
    M, K = 256, 256
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=46, M=M, N=N, K=K)
    A = dev["A"].clone()
    A[7] = float("nan")
    Aref = ref["A"].copy()
    Aref[7] = np.nan
    bias = torch.full((N,), float("-inf"), device="cuda", dtype=torch.bfloat16)
    bias[[17, N - 100]] = 0.0
    idx, val, _ = run_argmax(A, dev["B"], False, bias=bias)
    X = oracle.elementwise_stage(oracle.matmul(Aref, ref["B"]), 1.0, P.gpu_to_f64(bias), None, "none")
    oi, ov = oracle.row_argmax(X)
    got, v = idx.cpu().numpy(), val.cpu().numpy()
    assert np.array_equal(got, oi), np.argwhere(got != oi)[:4]
    assert got[7] == 0 and v[7] == -np.inf
    fin = np.isfinite(ov)
    assert np.all(np.abs(v[fin] - ov[fin]) <= 1e-4 * np.maximum(1.0, np.abs(ov[fin])))
    bias[:] = float("-inf")
    idx, val, _ = run_argmax(A, dev["B"], False, bias=bias)
    assert torch.all(idx == 0) and torch.all(val == float("-inf"))


def test_argmax_full_size_all_rows():
    # C2 shape as an LM-head-like greedy step: no logits written
    w, dev, ref = P.inputs("c2_gemm_layernorm", seed=0)
    idx, val, _ = run_argmax(dev["A"], dev["B"], False)
    X = oracle.elementwise_stage(oracle.matmul(ref["A"], ref["B"]))
    check_argmax(idx, val, X, "argmax C2 full size")
