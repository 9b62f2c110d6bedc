"""Write the oracle's outputs on tiny seeded inputs as text fixtures.

The review page prints no worked numeric example, so these fixtures are a
regression record of the fp64 oracle itself (which is pinned independently by
exact brute force, closed forms and invariants). Only ``gen`` (inputs) and
``oracle`` are called. Run from the repository root:

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import gen      # noqa: E402
import oracle   # noqa: E402

TINY = {
    "c1_gemm_bias_softmax_f32": dict(M=4, K=8, N=6),
    "c2_gemm_layernorm": dict(M=4, K=8, N=6),
    "c3_gemm_residual_rmsnorm": dict(M=4, K=8, N=6),
    "c4_b2b_mlp_relu": dict(M=4, K=8, L=6, N=5),
    "c5_b2b_attention": dict(batch=2, M=3, K=8, L=6, N=5),
}


def tensors(name, dims, seed=0):
    w = gen.workload(name, **dims)
    raw = gen.make(w, seed=seed)
    out = {}
    for t in w.tensors:
        v = raw[t.name]
        out[t.name] = oracle.widen_bf16(v) if t.dtype == "bf16" else v.astype(np.float64)
    return w, out


def golden_output(name, dims, seed=0):
    w, x = tensors(name, dims, seed)
    p = w.params
    if w.kind == "gemm_epilogue":
        return oracle.gemm_epilogue(
            x["A"], x["B"], alpha=p["alpha"], bias=x.get("bias"), residual=x.get("residual"),
            act=p["act"], row_op=p["row_op"], gamma=x.get("gamma", x.get("weight")),
            beta=x.get("beta"), eps=p.get("eps", 0.0))
    return oracle.b2bgemm(x["A"], x["B0"], x["B1"], alpha=p["alpha"], act=p["act"],
                          row_op=p["row_op"], b0_layout=p["b0_layout"])


def main():
    for name, dims in TINY.items():
        y = golden_output(name, dims)
        path = os.path.join(HERE, f"{name}_tiny_seed0.txt")
        with open(path, "w") as f:
            f.write(f"# oracle output for {name} with dims {dims}, seed 0; shape {list(y.shape)}\n")
            f.write("# written by tests/golden/make_golden.py (calls gen and oracle only)\n")
            for v in y.reshape(-1):
                f.write(float(v).hex() + "\n")


if __name__ == "__main__":
    main()
