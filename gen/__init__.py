"""Seeded synthetic inputs for the fused GEMM-epilogue and back-to-back GEMM workloads.

This module only draws random numbers and stores them in the storage dtype
(bf16 as raw uint16 bit patterns, or float32). It holds none of the fused
computation's arithmetic: both the fp64 oracle and the GPU library consume the
exact bytes produced here, each with its own code.

Workloads follow the kinds the ComFuse review page names (pith.science review of
"ComFuse: Fusing Complex Memory-Intensive Subgraphs with Compute-Intensive
Kernels", "The pith" and "If this is right": MatMul followed by softmax /
LayerNorm / RMSNorm, GEMM + ReLU + GEMM, attention as a back-to-back GEMM).
The shapes and value distributions are the five synthetic configurations listed
in the workload table of this repository. ``N(mu, s)`` means mean ``mu`` and
standard deviation ``s``.

Recipe: ``numpy.random.Generator(PCG64(SeedSequence([seed, workload_id])))``,
one child stream per tensor in the order the workload lists them, fp64 standard
normal draws, ``x = mu + s * z``, rounded to float32 (round-to-nearest-even) and,
for bf16 storage, from float32 to bf16 (round-to-nearest-even on the bit pattern).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = ["Tensor", "Workload", "WORKLOADS", "make", "f32_to_bf16_bits", "bf16_bits_to_f32"]


@dataclasses.dataclass(frozen=True)
class Tensor:
    name: str
    shape_keys: Tuple[str, ...]   # symbolic shape, resolved from the workload's dims
    mean: float
    std: float
    dtype: str                    # "bf16" or "f32"


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    kind: str                     # "gemm_epilogue" or "b2bgemm"
    dims: Dict[str, int]
    tensors: Tuple[Tensor, ...]
    params: Dict[str, object]     # epilogue parameters (alpha, eps, act, row_op, ...)
    description: str

    def with_dims(self, **dims) -> "Workload":
        d = dict(self.dims)
        for k, v in dims.items():
            if k not in d:
                raise KeyError(f"{self.name} has no dim {k!r}")
            d[k] = int(v)
        return dataclasses.replace(self, dims=d)

    def shape(self, t: Tensor) -> Tuple[int, ...]:
        return tuple(self.dims[k] if isinstance(k, str) else int(k) for k in t.shape_keys)


def _T(name, shape, mean, std, dtype="bf16"):
    return Tensor(name, tuple(shape), float(mean), float(std), dtype)


WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload):
    WORKLOADS[w.name] = w


_add(Workload(
    1, "c1_gemm_bias_softmax_f32", "gemm_epilogue",
    dict(M=256, K=128, N=256),
    (_T("A", ("M", "K"), 0.0, 1.0 / np.sqrt(128.0), "f32"),
     _T("B", ("K", "N"), 0.0, 1.0 / np.sqrt(128.0), "f32"),
     _T("bias", ("N",), 0.0, 0.1, "f32")),
    dict(alpha=1.0, act="none", row_op="softmax", out_dtype="f32"),
    "fp32 GEMM + bias + row softmax, A[256,128] B[128,256] bias[256]"))

_add(Workload(
    2, "c2_gemm_layernorm", "gemm_epilogue",
    dict(M=8192, K=4096, N=4096),
    (_T("A", ("M", "K"), 0.0, 1.0),
     _T("B", ("K", "N"), 0.0, 0.02),
     _T("gamma", ("N",), 1.0, 0.02),
     _T("beta", ("N",), 0.0, 0.02)),
    dict(alpha=1.0, act="none", row_op="layernorm", eps=1e-5, out_dtype="bf16"),
    "bf16 GEMM + LayerNorm, A[8192,4096] B[4096,4096], eps 1e-5"))

_add(Workload(
    3, "c3_gemm_residual_rmsnorm", "gemm_epilogue",
    dict(M=16384, K=11008, N=4096),
    (_T("A", ("M", "K"), 0.0, 1.0),
     _T("B", ("K", "N"), 0.0, 0.02),
     _T("residual", ("M", "N"), 0.0, 1.0),
     _T("weight", ("N",), 1.0, 0.02)),
    dict(alpha=1.0, act="none", row_op="rmsnorm", eps=1e-6, out_dtype="bf16"),
    "bf16 GEMM + residual add + RMSNorm, A[16384,11008] B[11008,4096], eps 1e-6"))

_add(Workload(
    4, "c4_b2b_mlp_relu", "b2bgemm",
    dict(batch=1, M=65536, K=64, L=256, N=64),
    (_T("A", ("batch", "M", "K"), 0.0, 1.0),
     _T("B0", ("batch", "K", "L"), 0.0, 1.0 / 8.0),
     _T("B1", ("batch", "L", "N"), 0.0, 1.0 / 16.0)),
    dict(alpha=1.0, act="relu", row_op="none", b0_layout="kl", out_dtype="bf16"),
    "B2BGEMM MLP X[65536,64] W0[64,256] ReLU W1[256,64]"))

_add(Workload(
    5, "c5_b2b_attention", "b2bgemm",
    dict(batch=512, M=1024, K=64, L=1024, N=64),
    (_T("A", ("batch", "M", "K"), 0.0, 1.0),      # Q  [B*H, S, D]
     _T("B0", ("batch", "L", "K"), 0.0, 1.0),     # K  [B*H, S, D]  (B0 given as [L, K])
     _T("B1", ("batch", "L", "N"), 0.0, 1.0)),    # V  [B*H, S, D]
    dict(alpha=0.125, act="none", row_op="softmax", b0_layout="lk", out_dtype="bf16"),
    "attention-style B2BGEMM, 32x16 heads, seq 1024, head dim 64, S=QK^T/8, softmax, O=PV"))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


_CHUNK = 1 << 22   # elements drawn per step; draws are sequential, so chunking does not change values


def _draw(rng: np.random.Generator, shape, mean, std, dtype) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        z = rng.standard_normal(e - s)            # fp64
        x32 = (mean + std * z).astype(np.float32)
        out[s:e] = f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    return out.reshape(shape)


def make(workload: str | Workload, seed: int = 0, only: Optional[List[str]] = None,
         **dims) -> Dict[str, np.ndarray]:
    """Draw every tensor of ``workload`` (optionally with overridden dims).

    Returns a dict name -> array: uint16 bf16 bit patterns for bf16 tensors,
    float32 for f32 tensors. ``only`` restricts which tensors are materialised
    (the random streams of the others are still spawned, so values do not depend
    on the selection).
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    if dims:
        w = w.with_dims(**dims)
    ss = np.random.SeedSequence([int(seed), int(w.wid)])
    children = ss.spawn(len(w.tensors))
    out = {}
    for t, child in zip(w.tensors, children):
        if only is not None and t.name not in only:
            continue
        rng = np.random.Generator(np.random.PCG64(child))
        out[t.name] = _draw(rng, w.shape(t), t.mean, t.std, t.dtype)
    return out


def workload(name: str, **dims) -> Workload:
    w = WORKLOADS[name]
    return w.with_dims(**dims) if dims else w
