"""The seeded input generator: determinism, shapes, distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

import gen


def test_deterministic_and_seed_dependent():
    a = gen.make("c2_gemm_layernorm", seed=1, M=64, N=128, K=96)
    b = gen.make("c2_gemm_layernorm", seed=1, M=64, N=128, K=96)
    c = gen.make("c2_gemm_layernorm", seed=2, M=64, N=128, K=96)
    for k in a:
        assert np.array_equal(a[k], b[k])
        assert not np.array_equal(a[k], c[k])


def test_only_does_not_change_values():
    full = gen.make("c3_gemm_residual_rmsnorm", seed=0, M=32, N=64, K=48)
    part = gen.make("c3_gemm_residual_rmsnorm", seed=0, only=["residual"], M=32, N=64, K=48)
    assert set(part) == {"residual"}
    assert np.array_equal(full["residual"], part["residual"])


def test_chunking_does_not_change_values(monkeypatch):
    ref = gen.make("c4_b2b_mlp_relu", seed=3, M=300)
    monkeypatch.setattr(gen, "_CHUNK", 1000)
    small = gen.make("c4_b2b_mlp_relu", seed=3, M=300)
    for k in ref:
        assert np.array_equal(ref[k], small[k])


@pytest.mark.parametrize("name", sorted(gen.WORKLOADS))
def test_shapes_and_dtypes(name):
    w = gen.WORKLOADS[name]
    small = {k: max(1, v // 64) if k != "batch" else min(v, 2) for k, v in w.dims.items()}
    out = gen.make(name, seed=0, **small)
    ws = w.with_dims(**small)
    for t in w.tensors:
        assert out[t.name].shape == ws.shape(t)
        assert out[t.name].dtype == (np.uint16 if t.dtype == "bf16" else np.float32)


def test_distributions():
    out = gen.make("c2_gemm_layernorm", seed=0, M=256, K=512, N=512)
    f = {k: gen.bf16_bits_to_f32(v).astype(np.float64) for k, v in out.items()}
    assert abs(f["A"].mean()) < 0.01 and abs(f["A"].std() - 1.0) < 0.01
    assert abs(f["B"].std() - 0.02) < 0.0005
    assert abs(f["gamma"].mean() - 1.0) < 0.005 and abs(f["gamma"].std() - 0.02) < 0.003
    c1 = gen.make("c1_gemm_bias_softmax_f32", seed=0)
    assert abs(c1["A"].std() - 1 / np.sqrt(128)) < 0.003
    assert abs(c1["bias"].std() - 0.1) < 0.02


def test_bf16_bits_match_torch_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = gen.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(gen.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
