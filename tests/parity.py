"""Shared helpers for the GPU parity tests: seeded inputs on the device, the
matching float64 oracle inputs, and the comparison metrics and bars.

Bars (fused GEMM + epilogue and back-to-back GEMM, bf16 inputs): relative
Frobenius error <= 1e-3 and max abs error <= 5e-3 against the fp64 oracle,
checked on the fp32-output instantiation of the kernel; the bf16-output
instantiation must equal round-to-nearest-even of the fp32 output bit for bit,
and lie within 5e-3 + half a bf16 ulp of the rounded oracle element-wise.
fp32 inputs (fp32 MFMA): both metrics <= 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

import gen
import oracle

REL_F_BF16, MAX_ABS_BF16 = 1e-3, 5e-3
REL_F_F32, MAX_ABS_F32 = 1e-5, 1e-5


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_oracle(arr: np.ndarray, dtype: str) -> np.ndarray:
    return oracle.widen_bf16(arr) if dtype == "bf16" else arr.astype(np.float64)


def inputs(name: str, seed: int = 0, **dims):
    """(workload, device tensors, float64 oracle arrays)."""
    w = gen.workload(name, **dims)
    raw = gen.make(w, seed=seed)
    dev = {t.name: to_device(raw[t.name], t.dtype) for t in w.tensors}
    ref = {t.name: to_oracle(raw[t.name], t.dtype) for t in w.tensors}
    return w, dev, ref


def gpu_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def metrics(got: np.ndarray, ref: np.ndarray):
    d = got - ref
    rel_f = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return rel_f, float(np.max(np.abs(d))) if d.size else 0.0


def assert_close(got, ref, rel_f, max_abs, what=""):
    r, m = metrics(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert r <= rel_f and m <= max_abs, f"{what}: relF {r:.3e} (bar {rel_f}), max abs {m:.3e} (bar {max_abs})"
    return r, m


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rne_bits_of_f32(t32: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns of round-to-nearest-even of an fp32 tensor (via gen's rounding)."""
    return gen.f32_to_bf16_bits(t32.detach().cpu().numpy())


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |x| (bf16 keeps 8 significant bits)."""
    return np.ldexp(1.0, np.frexp(np.abs(x))[1] - 9)


def assert_bf16_within(got: np.ndarray, ref: np.ndarray, what=""):
    """|G - R| <= 5e-3 + ulp/2 element-wise against the unrounded oracle R: the
    bound implied by the fp32 bar and one round-to-nearest of the output."""
    bound = MAX_ABS_BF16 + half_ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} bf16 outputs outside 5e-3 + ulp/2 of the oracle"


def assert_bf16_consistent(out_bf16: torch.Tensor, out_f32: torch.Tensor, ref: np.ndarray, what=""):
    """bf16 output == RNE(fp32 output) bit for bit (up to the sign of zero),
    within 5e-3 + ulp/2 of the oracle, and relF <= 1e-3 against RNE(oracle)."""
    a = bf16_bits(out_bf16)
    b = rne_bits_of_f32(out_f32)
    zero = ((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)
    mism = (a != b) & ~zero
    assert not mism.any(), f"{what}: {int(mism.sum())} bf16 outputs differ from RNE(fp32 output)"
    got = gpu_to_f64(out_bf16)
    assert_bf16_within(got, ref, what)
    rel, _ = metrics(got, oracle.round_bf16(ref))
    assert rel <= REL_F_BF16, f"{what}: bf16 relF vs RNE(oracle) {rel:.3e}"
