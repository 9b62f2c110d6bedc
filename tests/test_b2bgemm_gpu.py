"""GPU parity of cf_b2bgemm (back-to-back GEMM, intermediate kept on chip)
against the fp64 oracle, through the C ABI.

The oracle mirrors the one rounding the fused kernel must make: the second
GEMM's left operand in bf16 (round_operand=True). The unrounded oracle is
checked too, against a bar derived from that rounding: round-to-nearest-even
to bf16 (8 significant bits) moves each operand element by at most 2^-9 of
its value, uniformly, so by 2^-9/sqrt(3) = 1.1e-3 of it in the rms; the
second GEMM averages these independent errors over L terms with weights of
both signs, which leaves the relative Frobenius error of O of that order
(measured 1.5e-3 to 1.7e-3). The bar is 3e-3, below any error of twice the
rounding's own size."""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import b2bgemm_stage_stream_amd as cf   # noqa: E402
import oracle                           # noqa: E402
import parity as P                      # noqa: E402

REL_F_UNROUNDED = 3e-3


def run(A, B0, B1, out_dtype, *, b0_is_lk, **epi):
    batch = A.shape[0] if A.dim() == 3 else 1
    M = A.shape[-2]
    N = B1.shape[-1]
    O = torch.empty(batch, M, N, dtype=out_dtype, device="cuda")   # ld = N (element stores when N % 4)
    cf.cf_b2bgemm(A, B0, B1, O, b0_is_lk=b0_is_lk, **epi)
    torch.cuda.synchronize()
    return O


def check(dev, ref, *, lk, what, alpha=1.0, act="none", row_op="none", bias=None, bias_ref=None, causal=False):
    kw = dict(alpha=alpha, act=act, row_op=row_op, bias=bias, mask="causal" if causal else "none")
    R = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], alpha=alpha, act=act, row_op=row_op, bias=bias_ref,
                       b0_layout="lk" if lk else "kl", causal=causal)
    o32 = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=lk, **kw)
    g = P.gpu_to_f64(o32)
    r, m = P.assert_close(g, R, P.REL_F_BF16, P.MAX_ABS_BF16, what + " f32-out")
    Ru = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], alpha=alpha, act=act, row_op=row_op, bias=bias_ref,
                        b0_layout="lk" if lk else "kl", round_operand=False, causal=causal)
    ru, _ = P.metrics(g, Ru)
    assert ru <= REL_F_UNROUNDED, f"{what}: relF vs unrounded oracle {ru:.3e}"
    o16 = run(dev["A"], dev["B0"], dev["B1"], torch.bfloat16, b0_is_lk=lk, **kw)
    P.assert_bf16_consistent(o16, o32, R, what + " bf16-out")
    print(f"{what}: relF {r:.2e} maxabs {m:.2e} (unrounded oracle relF {ru:.2e})", flush=True)
    return o32


def oracle_heads(ref, heads_per_call=16, **kw):
    """oracle.b2bgemm of every (batch, head) problem of ref, evaluated in
    groups of heads on a few host threads (the problems are independent)."""
    nb = ref["A"].shape[0]

    def part(i):
        sl = slice(i, min(nb, i + heads_per_call))
        B0 = ref["B0"][sl] if ref["B0"].ndim == 3 else ref["B0"]
        B1 = ref["B1"][sl] if ref["B1"].ndim == 3 else ref["B1"]
        return oracle.b2bgemm(ref["A"][sl], B0, B1, **kw)

    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
        return np.concatenate(list(ex.map(part, range(0, nb, heads_per_call))))


# ---------------------------------------------------------------------------- the two workloads

def test_c4_mlp_relu_reduced():
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=0, M=2048)
    check(dev, ref, lk=False, act="relu", what="C4 2048 rows")


def test_c5_attention_reduced():
    w, dev, ref = P.inputs("c5_b2b_attention", seed=0, batch=4, M=256, L=256)
    check(dev, ref, lk=True, alpha=0.125, row_op="softmax", what="C5 4x256x256")


@pytest.mark.parametrize("seed", [1, 2])
def test_c5_seeds(seed):
    w, dev, ref = P.inputs("c5_b2b_attention", seed=seed, batch=2, M=128, L=512)
    check(dev, ref, lk=True, alpha=0.125, row_op="softmax", what=f"C5 seed {seed}")


def test_c5_large_logits():
    # logits of several hundred exercise the integer stabiliser's rescaling
    w, dev, ref = P.inputs("c5_b2b_attention", seed=3, batch=2, M=64, L=320)
    dev["A"] = (dev["A"].float() * 6).to(torch.bfloat16)
    ref["A"] = P.gpu_to_f64(dev["A"])
    check(dev, ref, lk=True, alpha=0.125, row_op="softmax", what="C5 x6 logits")


# ---------------------------------------------------------------------------- shapes and layouts

def padded(t: torch.Tensor) -> torch.Tensor:
    """Same values with the row length padded to a multiple of 8 elements (a
    strided view, as the library's 16-byte aligned leading dimensions need)."""
    n = t.shape[-1]
    buf = torch.zeros(*t.shape[:-1], (n + 7) // 8 * 8, dtype=t.dtype, device=t.device)
    buf[..., :n] = t
    return buf[..., :n]


@pytest.mark.parametrize("lk", [False, True])
@pytest.mark.parametrize("row_op,act", [("none", "relu"), ("none", "none"), ("softmax", "none")])
@pytest.mark.parametrize("shape", [(1, 77, 40, 100, 50), (3, 130, 16, 64, 32), (2, 5, 128, 200, 128),
                                   (1, 1, 9, 1, 3), (2, 300, 64, 192, 64)])
def test_shapes(lk, row_op, act, shape):
    # scaled like the workloads (S and O of order one): alpha = K^-1/2, B1 / L^1/2
    batch, M, K, L, N = shape
    w, dev, ref = P.inputs("c5_b2b_attention", seed=4, batch=batch, M=M, K=K, L=L, N=N)
    dev["B1"] = (dev["B1"].float() / np.sqrt(L)).to(torch.bfloat16)
    ref["B1"] = P.gpu_to_f64(dev["B1"])
    if not lk:   # B0 given as [K, L]
        dev["B0"] = dev["B0"].transpose(1, 2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], 1, 2))
    dev = {k: padded(v) for k, v in dev.items()}
    check(dev, ref, lk=lk, alpha=1.0 / np.sqrt(K), act=act, row_op=row_op,
          what=f"{shape} {row_op}/{act} lk={lk}")


@pytest.mark.parametrize("lk", [False, True])
@pytest.mark.parametrize("row_op,act", [("none", "relu"), ("softmax", "none")])
@pytest.mark.parametrize("shape", [(1, 300, 512, 256, 128), (2, 200, 512, 128, 256), (1, 1000, 256, 512, 64),
                                   (2, 77, 200, 150, 300), (1, 130, 130, 64, 129), (3, 65, 1024, 96, 520),
                                   (1, 300, 512, 192, 64), (2, 150, 128, 256, 256), (1, 200, 256, 128, 128),
                                   (1, 257, 256, 320, 256)])
def test_wide_k_and_n(lk, row_op, act, shape):
    # K above 128 and N above 128, among them the pages' DLRM bottom-MLP
    # feature widths 512 / 256 / 128: the streamed kernel for K = 256 or 512
    # with N = 64 or 128 and for K = 128 or 256 with N = 256 (L a multiple of
    # 64), the general kernel (k-blocks and column blocks of 128) otherwise;
    # ragged K, L, N and rows
    batch, M, K, L, N = shape
    w, dev, ref = P.inputs("c5_b2b_attention", seed=15, batch=batch, M=M, K=K, L=L, N=N)
    dev["B1"] = (dev["B1"].float() / np.sqrt(L)).to(torch.bfloat16)
    ref["B1"] = P.gpu_to_f64(dev["B1"])
    if not lk:   # B0 given as [K, L]
        dev["B0"] = dev["B0"].transpose(1, 2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], 1, 2))
    dev = {k: padded(v) for k, v in dev.items()}
    check(dev, ref, lk=lk, alpha=1.0 / np.sqrt(K), act=act, row_op=row_op,
          what=f"wide {shape} {row_op}/{act} lk={lk}")


@pytest.mark.parametrize("causal", [False, True])
def test_wide_attention_logsumexp_and_bias(causal):
    # head dim 256 (K = N = 256): the softmax terms and the log-sum-exp must
    # agree across the two column blocks of O
    w, dev, ref = P.inputs("c5_b2b_attention", seed=16, batch=2, M=192, K=256, L=320, N=256)
    lse = torch.full((2, 192), float("nan"), dtype=torch.float32, device="cuda")
    O = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=True, alpha=1 / 16, row_op="softmax",
            mask="causal" if causal else "none", row_stats=lse)
    R = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], alpha=1 / 16, row_op="softmax", b0_layout="lk",
                       causal=causal)
    P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"head dim 256 causal={causal}")
    Rl = oracle.b2b_logsumexp(ref["A"], ref["B0"], alpha=1 / 16, b0_layout="lk", causal=causal)
    P.assert_close(P.gpu_to_f64(lse), Rl, 1e-5, 1e-4, "head dim 256 log-sum-exp")


@pytest.mark.parametrize("K,N", [(512, 128), (512, 64), (256, 128), (256, 256)])
def test_wide_mlp_with_bias_dlrm_widths(K, N):
    # bottom-MLP layer pairs K -> 256 -> N with a bias and ReLU between (512 ->
    # 256 -> 128 the pages' widths; K = 512 with N = 128 takes the general
    # kernel, the others the streamed one with its bias block).
    # The MLP workload's W0 ~ N(0, 1/8) is scaled for K = 64; alpha = 1/sqrt(8)
    # (sqrt(K / 64) in general) keeps S of the same order at K = 512. (S itself is accumulated in fp32
    # and rounded to bf16 for the second GEMM, as the oracle mirrors; where an
    # fp32 S lies within its rounding error of a bf16 rounding boundary the
    # two roundings pick neighbouring values, and one bf16 step of S grows
    # with |S|, so an unscaled S of order 8 would spend the max-abs bar on such
    # ties alone.)
    batch, M, L = 1, 4096, 256
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=17, batch=batch, M=M, K=K, L=L, N=N)
    rng = np.random.default_rng(17)
    bias = torch.from_numpy(rng.normal(0.0, 0.5, L)).to(torch.bfloat16).cuda()
    check(dev, ref, lk=False, alpha=float(np.float32(1 / np.sqrt(K / 64))), act="relu", bias=bias,
          bias_ref=P.gpu_to_f64(bias), what=f"DLRM {K}-256-{N} + bias")


@pytest.mark.parametrize("lk", [False, True])
@pytest.mark.parametrize("row_op,act", [("softmax", "none"), ("none", "relu")])
@pytest.mark.parametrize("K,N", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_exact_shapes_streamed(K, N, lk, row_op, act):
    # K, N in {64, 128} and L a multiple of 64 take the LDS-ring kernel; L = 320
    # is 5 segments (more than the ring holds), batch 3 spreads over XCDs 0..2
    batch, M, L = 3, 200, 320
    w, dev, ref = P.inputs("c5_b2b_attention", seed=9, batch=batch, M=M, K=K, L=L, N=N)
    dev["B1"] = (dev["B1"].float() / np.sqrt(L)).to(torch.bfloat16)
    ref["B1"] = P.gpu_to_f64(dev["B1"])
    if not lk:
        dev["B0"] = dev["B0"].transpose(1, 2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], 1, 2))
    check(dev, ref, lk=lk, alpha=1.0 / np.sqrt(K), act=act, row_op=row_op,
          what=f"streamed K={K} N={N} lk={lk} {row_op}/{act}")


@pytest.mark.parametrize("bias_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("lk", [False, True])
@pytest.mark.parametrize("K,N,L", [(64, 64, 320), (64, 128, 320), (128, 64, 320), (128, 128, 320), (64, 64, 128)])
def test_bias_streamed(K, N, L, lk, bias_dtype):
    # a bias on the ReLU chain travels with the B0/B1 segments through the
    # LDS ring (per-head weights: streamed; L = 128 with shared weights:
    # resident); bf16 and fp32 bias vectors
    batch, M = 3, 200
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=13, batch=batch, M=M, K=K, L=L, N=N)
    if lk:   # B0 given as [L, K]
        dev["B0"] = dev["B0"].transpose(1, 2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], 1, 2))
    if L == 128:   # one 2-D B0/B1 for the whole batch
        dev["B0"], dev["B1"] = dev["B0"][0], dev["B1"][0]
        ref["B0"], ref["B1"] = ref["B0"][0], ref["B1"][0]
    rng = np.random.default_rng(1000 + K + N + L)
    bias = torch.from_numpy(rng.normal(0.0, 0.5, L)).to(bias_dtype).cuda()
    check(dev, ref, lk=lk, alpha=0.5, act="relu", bias=bias, bias_ref=P.gpu_to_f64(bias),
          what=f"bias {str(bias_dtype)[6:]} K={K} N={N} L={L} lk={lk}")


@pytest.mark.parametrize("bias_dtype", [torch.bfloat16, torch.float32])
def test_bias_unaligned(bias_dtype):
    # a bias one element past an aligned base: fp32 (4-byte aligned) still
    # streams with the ring, bf16 at an odd element takes the general kernel,
    # which reads it element by element
    batch, M, K, L, N = 2, 130, 64, 192, 64
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=14, batch=batch, M=M, K=K, L=L, N=N)
    rng = np.random.default_rng(77)
    buf = torch.from_numpy(rng.normal(0.0, 0.5, L + 1)).to(bias_dtype).cuda()
    bias = buf[1:]
    assert bias.data_ptr() % 16 != 0
    check(dev, ref, lk=False, alpha=0.5, act="relu", bias=bias, bias_ref=P.gpu_to_f64(bias),
          what=f"unaligned bias {str(bias_dtype)[6:]}")


@pytest.mark.parametrize("lk,row_op,act", [(True, "softmax", "none"), (False, "none", "relu")])
def test_two_row_blocks_per_wave(lk, row_op, act):
    # enough 256-row tiles (512 batch entries) for the kernel variant whose
    # waves own 64 rows; M = 200 leaves every tile ragged
    w, dev, ref = P.inputs("c5_b2b_attention", seed=12, batch=512, M=200, K=64, L=128, N=64)
    dev["B1"] = (dev["B1"].float() / np.sqrt(128)).to(torch.bfloat16)
    ref["B1"] = P.gpu_to_f64(dev["B1"])
    if not lk:
        dev["B0"] = dev["B0"].transpose(1, 2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], 1, 2))
    check(dev, ref, lk=lk, alpha=0.125, act=act, row_op=row_op, what=f"512 x 200 rows {row_op}/{act}")


def test_heads_grouped_by_xcd():
    # per-batch B0/B1 with a batch that is a multiple of 8: the row tiles of one
    # batch entry are scheduled together (2 tiles per entry, ragged last tile)
    w, dev, ref = P.inputs("c5_b2b_attention", seed=11, batch=16, M=200, L=192)
    check(dev, ref, lk=True, alpha=0.125, row_op="softmax", what="16 heads x 200 rows")


@pytest.mark.parametrize("L", [128, 640])
def test_shared_weights_streamed(L):
    # 2-D B0/B1 shared by the batch: L = 128 stays resident in LDS, L = 640
    # streams; bias on the ReLU chain, negative alpha on the softmax chain
    batch, M, K, N = 2, 256, 64, 64
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=10, batch=batch, M=M, K=K, L=L, N=N)
    B0, B1 = dev["B0"][0], dev["B1"][0]
    bias = torch.linspace(-0.5, 0.5, L, device="cuda").to(torch.bfloat16)
    R = oracle.b2bgemm(ref["A"], ref["B0"][0], ref["B1"][0], alpha=0.5, act="relu", bias=P.gpu_to_f64(bias))
    O = torch.empty(batch, M, N, dtype=torch.float32, device="cuda")
    cf.cf_b2bgemm(dev["A"], B0, B1, O, alpha=0.5, act="relu", bias=bias)
    torch.cuda.synchronize()
    P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"shared relu+bias L={L}")
    B1s = (B1.float() / np.sqrt(L)).to(torch.bfloat16)
    R = oracle.b2bgemm(ref["A"], ref["B0"][0], P.gpu_to_f64(B1s), alpha=-0.125, row_op="softmax")
    cf.cf_b2bgemm(dev["A"], B0, B1s, O, alpha=-0.125, row_op="softmax")
    torch.cuda.synchronize()
    P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"shared softmax alpha<0 L={L}")


def mlp_inputs(seed, lk, **dims):
    """The MLP workload's inputs; with lk, B0 given as [L, K] (transposed copy)."""
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=seed, **dims)
    if lk:
        dev["B0"] = dev["B0"].transpose(1, 2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], 1, 2))
    return dev, ref


@pytest.mark.parametrize("lk", [False, True])
@pytest.mark.parametrize("K,N,L", [(64, 64, 256), (64, 128, 192), (128, 64, 192), (128, 128, 128)])
def test_mlp_resident_weights_several_tiles_per_workgroup(K, N, L, lk):
    # B0 and B1 resident in LDS (L as long as the ring) with an elementwise F:
    # more 128-row tiles than co-resident workgroups, so a workgroup takes
    # several tiles and loads the next tile's A rows during the current one;
    # the last tile is ragged
    # (alpha = 64 / K, a power of two, keeps the scores at the workload's unit
    # variance when K = 128)
    M = 65536 + 64 * 128 + 37
    dev, ref = mlp_inputs(19, lk, M=M, K=K, L=L, N=N)
    check(dev, ref, lk=lk, alpha=64.0 / K, act="relu", what=f"MLP {M} rows K={K} N={N} L={L} lk={lk}")
    # 2-D weights shared by a batch of 3 (tiles of one workgroup cross batch
    # entries), identity F with alpha != 1
    batch, Mb, alpha = 3, 30005, 0.75 * 64.0 / K
    dev, ref = mlp_inputs(20, lk, batch=batch, M=Mb, K=K, L=L, N=N)
    R = oracle.b2bgemm(ref["A"], ref["B0"][0], ref["B1"][0], alpha=alpha, b0_layout="lk" if lk else "kl")
    O = torch.empty(batch, Mb, N, dtype=torch.float32, device="cuda")
    cf.cf_b2bgemm(dev["A"], dev["B0"][0], dev["B1"][0], O, b0_is_lk=lk, alpha=alpha)
    torch.cuda.synchronize()
    r, m = P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"shared weights, batch {batch}")
    print(f"shared weights batch {batch} x {Mb}: relF {r:.2e} maxabs {m:.2e}", flush=True)


@pytest.mark.parametrize("M", [1, 37, 129])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("act", ["relu", "none"])
def test_mlp_resident_weights_few_rows_and_strided_output(M, out_dtype, act):
    # the MLP kernel on one partial tile (and one full tile plus one row),
    # writing O through a row stride of 67 elements, which takes the element
    # stores instead of the 8- or 16-byte ones; alpha = 1 with and without ReLU
    K, L, N = 64, 256, 64
    dev, ref = mlp_inputs(21, False, M=M, K=K, L=L, N=N)
    R = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], act=act)
    buf = torch.full((1, M, 67), float("nan"), dtype=out_dtype, device="cuda")
    O = buf[..., :N]
    cf.cf_b2bgemm(dev["A"], dev["B0"], dev["B1"], O, act=act)
    torch.cuda.synchronize()
    assert torch.isnan(buf[..., N:].float()).all(), "a store landed past column N"
    if out_dtype == torch.float32:
        P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"MLP {M} rows, strided O")
    else:
        o32 = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=False, act=act)
        P.assert_bf16_consistent(O.contiguous(), o32, R, f"MLP {M} rows, strided bf16 O")


def test_bias_and_shared_weights():
    # a 2-D B0/B1 is shared by every batch; bias per column of S
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=5, batch=3, M=96, K=32, L=96, N=64)
    bias = torch.linspace(-0.5, 0.5, 96, device="cuda").to(torch.bfloat16)
    B0, B1 = dev["B0"][0], dev["B1"][0]
    R = oracle.b2bgemm(ref["A"], ref["B0"][0], ref["B1"][0], alpha=0.5, act="relu", bias=P.gpu_to_f64(bias))
    O = torch.empty(3, 96, 64, dtype=torch.float32, device="cuda")
    cf.cf_b2bgemm(dev["A"], B0, B1, O, alpha=0.5, act="relu", bias=bias)
    torch.cuda.synchronize()
    P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, "bias, shared weights")


def test_identity_b1_matches_single_gemm_epilogue():
    # B1 = I: O is round_bf16(relu(S)), the single-GEMM epilogue followed by bf16 rounding
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=6, M=256, K=64, L=64, N=64)
    eye = torch.eye(64, dtype=torch.bfloat16, device="cuda")
    O = run(dev["A"], dev["B0"], eye[None], torch.float32, b0_is_lk=False, act="relu")
    C = torch.empty(256, 64, dtype=torch.bfloat16, device="cuda")
    cf.cf_gemm_epilogue(dev["A"][0], dev["B0"][0], C, act="relu")
    torch.cuda.synchronize()
    assert torch.equal(O[0], C.float())


def test_identity_v_softmax():
    # V = I: rows are round_bf16(p~) / l, within 2^-8 of softmax(S)
    w, dev, ref = P.inputs("c5_b2b_attention", seed=7, batch=2, M=64, L=64, N=64)
    eye = torch.eye(64, dtype=torch.bfloat16, device="cuda").expand(2, 64, 64).contiguous()
    O = run(dev["A"], dev["B0"], eye, torch.float32, b0_is_lk=True, alpha=0.125, row_op="softmax")
    S = 0.125 * np.matmul(ref["A"], np.swapaxes(ref["B0"], 1, 2))
    Ps = oracle.row_softmax(S)
    assert np.all(np.abs(P.gpu_to_f64(O) - Ps) <= 2.0 ** -8 * Ps + 1e-6)


def test_deterministic():
    w, dev, ref = P.inputs("c5_b2b_attention", seed=8, batch=4, M=128, L=256)
    a = run(dev["A"], dev["B0"], dev["B1"], torch.bfloat16, b0_is_lk=True, alpha=0.125, row_op="softmax")
    b = run(dev["A"], dev["B0"], dev["B1"], torch.bfloat16, b0_is_lk=True, alpha=0.125, row_op="softmax")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------- full sizes, sampled

def test_c4_full_size_all_rows():
    w, dev, ref = P.inputs("c4_b2b_mlp_relu", seed=0)
    O = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=False, act="relu")
    R = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], act="relu")
    r, m = P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, "C4 full size")
    o16 = run(dev["A"], dev["B0"], dev["B1"], torch.bfloat16, b0_is_lk=False, act="relu")
    P.assert_bf16_consistent(o16, O, R, "C4 full size bf16")
    print(f"C4 full: relF {r:.2e} maxabs {m:.2e}", flush=True)


def test_c5_full_size_all_heads():
    w, dev, ref = P.inputs("c5_b2b_attention", seed=0)
    O = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=True, alpha=0.125, row_op="softmax")
    R = oracle_heads(ref, alpha=0.125, row_op="softmax", b0_layout="lk")
    r, m = P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, "C5 full size, all heads")
    o16 = run(dev["A"], dev["B0"], dev["B1"], torch.bfloat16, b0_is_lk=True, alpha=0.125, row_op="softmax")
    P.assert_bf16_consistent(o16, O, R, "C5 full size bf16")
    print(f"C5 full: relF {r:.2e} maxabs {m:.2e}", flush=True)


# ---------------------------------------------------------------------------- causal softmax

@pytest.mark.parametrize("M,L", [(256, 256), (200, 640), (384, 320), (1, 192)])
def test_causal_streamed(M, L):
    # keys [L, K], K = N = 64, L a multiple of 64: the streamed kernel; M < L puts the
    # queries at the end, M > L leaves the first M - L rows with no key (output 0)
    w, dev, ref = P.inputs("c5_b2b_attention", seed=10, batch=3, M=M, L=L)
    o = check(dev, ref, lk=True, alpha=0.125, row_op="softmax", causal=True, what=f"causal {M}x{L}")
    if M > L:
        assert torch.all(o[:, : M - L] == 0)


@pytest.mark.parametrize("K,N", [(64, 128), (128, 64), (128, 128), (256, 128), (512, 64), (128, 256)])
def test_causal_streamed_widths(K, N):
    w, dev, ref = P.inputs("c5_b2b_attention", seed=11, batch=2, M=192, L=256, K=K, N=N)
    check(dev, ref, lk=True, alpha=0.125, row_op="softmax", causal=True, what=f"causal K={K} N={N}")


def test_causal_many_heads_xcd_grouped():
    # 512 heads: enough tiles for every CU, heads grouped by XCD (the causal
    # mask takes 128-row tiles, one row block per wave, at any head count)
    w, dev, ref = P.inputs("c5_b2b_attention", seed=12, batch=512, M=256, L=256)
    check(dev, ref, lk=True, alpha=0.125, row_op="softmax", causal=True, what="causal 512 heads")


def test_causal_negative_alpha_large_logits():
    w, dev, ref = P.inputs("c5_b2b_attention", seed=13, batch=2, M=128, L=320)
    dev["A"] = (dev["A"].float() * 6).to(torch.bfloat16)
    ref["A"] = P.gpu_to_f64(dev["A"])
    check(dev, ref, lk=True, alpha=-0.125, row_op="softmax", causal=True, what="causal alpha<0 x6")


@pytest.mark.parametrize("M,L,lk", [(100, 100, True), (70, 150, True), (130, 90, True), (256, 256, False)])
def test_causal_general_kernel(M, L, lk):
    # L not a multiple of 64, or keys given [K, L]: the general kernel
    w, dev, ref = P.inputs("c5_b2b_attention", seed=14, batch=2, M=M, L=L)
    if not lk:
        dev["B0"] = dev["B0"].transpose(-1, -2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], -1, -2))
    o = check(dev, ref, lk=lk, alpha=0.125, row_op="softmax", causal=True, what=f"causal general {M}x{L} lk={lk}")
    if M > L:
        assert torch.all(o[:, : M - L] == 0)


def test_causal_full_size_all_heads():
    w, dev, ref = P.inputs("c5_b2b_attention", seed=0)
    O = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=True, alpha=0.125, row_op="softmax",
            mask="causal")
    R = oracle_heads(ref, alpha=0.125, row_op="softmax", b0_layout="lk", causal=True)
    P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, "causal C5 full size, all heads")


# ---------------------------------------------------------------------------- log-sum-exp of the attention rows

@pytest.mark.parametrize("M,L,causal", [(256, 512, False), (200, 640, True), (384, 320, True), (100, 150, False)])
def test_attention_logsumexp(M, L, causal):
    w, dev, ref = P.inputs("c5_b2b_attention", seed=18, batch=3, M=M, L=L)
    lse = torch.full((3, M), float("nan"), dtype=torch.float32, device="cuda")
    O = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=True, alpha=0.125, row_op="softmax",
            mask="causal" if causal else "none", row_stats=lse)
    R = oracle.b2b_logsumexp(ref["A"], ref["B0"], alpha=0.125, b0_layout="lk", causal=causal)
    got = P.gpu_to_f64(lse)
    fin = np.isfinite(R)
    assert np.array_equal(np.isfinite(got), fin), "rows without keys must give -inf"
    assert np.all(got[~fin] == -np.inf)
    P.assert_close(got[fin], R[fin], 1e-5, 1e-4, f"attention log-sum-exp {M}x{L} causal={causal}")
    Ro = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], alpha=0.125, row_op="softmax", b0_layout="lk", causal=causal)
    P.assert_close(P.gpu_to_f64(O), Ro, P.REL_F_BF16, P.MAX_ABS_BF16, "output unchanged by storing the statistics")


# ---------------------------------------------------------------------------- ping-pong schedule
# With cf_set_b2b_pingpong(1), the softmax without mask and bias at K = N = 64
# runs with 512-row tiles, two groups of four waves alternating MFMA and
# softmax phases, once there are at least as many 512-row tiles as CUs
# (batch * ceil(M / 512) >= 256 on MI355X).

@pytest.fixture
def pingpong():
    old = cf.cf_set_b2b_pingpong(1)
    yield
    cf.cf_set_b2b_pingpong(old)


def pp_inputs(seed, batch, M, L, lk=True, scale_a=1.0):
    w, dev, ref = P.inputs("c5_b2b_attention", seed=seed, batch=batch, M=M, L=L)
    if scale_a != 1.0:
        dev["A"] = (dev["A"].float() * scale_a).to(torch.bfloat16)
        ref["A"] = P.gpu_to_f64(dev["A"])
    dev["B1"] = (dev["B1"].float() / np.sqrt(L / 64)).to(torch.bfloat16)
    ref["B1"] = P.gpu_to_f64(dev["B1"])
    if not lk:
        dev["B0"] = dev["B0"].transpose(1, 2).contiguous()
        ref["B0"] = np.ascontiguousarray(np.swapaxes(ref["B0"], 1, 2))
    return dev, ref


@pytest.mark.parametrize("lk", [True, False])
@pytest.mark.parametrize("M,L", [(100, 64), (100, 192), (37, 448), (512, 128), (600, 320)])
def test_ping_pong_per_head(pingpong, lk, M, L):
    # ragged 512-row tiles; one segment, several, and more than the ring holds;
    # a workgroup's tiles stream through the ring back to back
    batch = 256 if M <= 512 else 128
    dev, ref = pp_inputs(20, batch, M, L, lk)
    check(dev, ref, lk=lk, alpha=0.125, row_op="softmax", what=f"ping-pong {batch}x{M}x{L} lk={lk}")


@pytest.mark.parametrize("L", [320, 640])
def test_ping_pong_shared_weights(pingpong, L):
    # 2-D B0/B1 shared by the batch: L = 320 stays resident in LDS, L = 640 streams
    batch, M = 256, 96
    dev, ref = pp_inputs(21, batch, M, L)
    R = oracle.b2bgemm(ref["A"], ref["B0"][0], ref["B1"][0], alpha=0.125, row_op="softmax", b0_layout="lk")
    O = run(dev["A"], dev["B0"][0], dev["B1"][0], torch.float32, b0_is_lk=True, alpha=0.125, row_op="softmax")
    P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"ping-pong shared weights L={L}")


@pytest.mark.parametrize("alpha", [0.125, -0.125])
def test_ping_pong_large_logits_and_logsumexp(pingpong, alpha):
    # logits of several hundred: the stabiliser is raised within the stream
    # (the redo of a segment whose terms pass 2^32), either sign of alpha
    batch, M, L = 256, 64, 384
    dev, ref = pp_inputs(22, batch, M, L, scale_a=6.0)
    lse = torch.full((batch, M), float("nan"), dtype=torch.float32, device="cuda")
    O = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=True, alpha=alpha, row_op="softmax",
            row_stats=lse)
    R = oracle.b2bgemm(ref["A"], ref["B0"], ref["B1"], alpha=alpha, row_op="softmax", b0_layout="lk")
    P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, f"ping-pong x6 logits alpha={alpha}")
    Rl = oracle.b2b_logsumexp(ref["A"], ref["B0"], alpha=alpha, b0_layout="lk")
    P.assert_close(P.gpu_to_f64(lse), Rl, 1e-5, 1e-4, f"ping-pong log-sum-exp alpha={alpha}")


def test_ping_pong_full_size_all_heads(pingpong):
    # the attention workload (batch 32 x 16 heads, M = L = 1024) on the ping-pong
    # schedule, every row against the oracle, and against the default schedule
    w, dev, ref = P.inputs("c5_b2b_attention", seed=0)
    O = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=True, alpha=0.125, row_op="softmax")
    R = oracle_heads(ref, alpha=0.125, row_op="softmax", b0_layout="lk")
    r, m = P.assert_close(P.gpu_to_f64(O), R, P.REL_F_BF16, P.MAX_ABS_BF16, "C5 ping-pong, all heads")
    cf.cf_set_b2b_pingpong(0)
    O0 = run(dev["A"], dev["B0"], dev["B1"], torch.float32, b0_is_lk=True, alpha=0.125, row_op="softmax")
    d = float((O - O0).abs().max())
    assert d <= 1e-5, f"schedules differ by {d:.2e} (only the row-sum order may differ)"
    print(f"C5 ping-pong full: relF {r:.2e} maxabs {m:.2e}; max |pp - default| {d:.1e}", flush=True)
