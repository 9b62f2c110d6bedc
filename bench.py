"""Benchmark of the fused GEMM + epilogue (and back-to-back GEMM) kernels on one
MI355X.

One step = one fused kernel call over the whole workload (inputs already
resident in HBM; consecutive steps cycle through copies of the inputs totalling
at least 512 MiB so that they are read from HBM, not from the last-level
cache). Before the W warmup steps the same calls run untimed for --settle-s
seconds: the shader clock climbs over the first tens of milliseconds of
sustained load (a C2 launch takes 0.33 ms in the first batch and 0.24 ms from
about the 200th on), and the timed steps are meant to see the sustained state.
The K timed launches are captured once into a HIP graph and replayed as one
(--eager: launched one by one from Python), so that a small kernel's time is
not the host's per-call cost.
Prints one JSON line:
  value      algorithmic GEMM TFLOP/s of the workload (2*M*N*K per GEMM)
  roofline   the same kernel against its bound (bf16 dense MFMA peak, or HBM
             bandwidth when the workload's flop/byte is below the ridge point),
             with the mean kernel time from HIP events on the launch stream
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded row sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--store-x] [--causal] [--argmax]
                       [--row2 softmax|layernorm|rmsnorm] [--topk K]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused GEMM+epilogue TFLOP/s, % bf16 MFMA peak, intermediate HBM bytes (=0)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (published)
HBM_GBPS = 8000.0

# the largest workload (16384 x 11008 x 4096 GEMM + residual + RMSNorm)
DEFAULT_WORKLOAD = "c3_gemm_residual_rmsnorm"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-s", type=float, default=0.6,
                    help="untimed seconds of the same calls before the warmup steps, so that the GPU clock has "
                         "left its idle state (0: none)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--b-nk", action="store_true",
                    help="GEMM + epilogue with B stored [N, K] (the nn.Linear weight layout), b_is_nk")
    ap.add_argument("--plain", action="store_true",
                    help="diagnostic: same GEMM with the identity epilogue (not the headline workload)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (written from rocprofv3 counters)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="calibration: time a plain device copy of MIB MiB (for the byte counters)")
    ap.add_argument("--ingest-counters", default=None, metavar="DIR",
                    help="no GPU: read the rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv files under DIR "
                         "(fetch_<workload>/, write_<workload>/, fetch_copy/, write_copy/) and write --traffic")
    ap.add_argument("--store-x", action="store_true",
                    help="GEMM + epilogue workloads: also store x, the input of the row operation, as a second "
                         "bf16 [M, N] output (e.g. the new residual stream of a pre-norm block)")
    ap.add_argument("--topk", type=int, default=0, metavar="K",
                    help="GEMM + epilogue workloads without a residual: replace the row operation by each row's "
                         "K largest (columns and values; no logits written)")
    ap.add_argument("--argmax", action="store_true",
                    help="GEMM + epilogue workloads: replace the row operation by a row argmax and write no "
                         "[M, N] output (a greedy LM-head step)")
    ap.add_argument("--row2", choices=["softmax", "layernorm", "rmsnorm"], default=None,
                    help="GEMM + epilogue workloads: a second row stage on the first one's output (its gamma/beta "
                         "are the workload's own vectors)")
    ap.add_argument("--causal", action="store_true",
                    help="attention workload: causal mask (key l visible to query m iff l <= m + L - M); the "
                         "algorithmic flops count only the visible (query, key) pairs")
    ap.add_argument("--dims", default="",
                    help="diagnostic: override workload dims, e.g. M=2048,N=16384 (the line then names them)")
    ap.add_argument("--column", action="store_true",
                    help="GEMM + epilogue workloads: the row operation over the rows of each column instead "
                         "(cf_epilogue.axis = column; the complementary strip exchange)")
    ap.add_argument("--row-stats", action="store_true",
                    help="GEMM + epilogue workloads: also store the reduction's per-row (per-column) statistics")
    ap.add_argument("--via-fuse", action="store_true",
                    help="time the workload written as a torch function and lowered by fuse.lower onto one fused "
                         "call (the front-end's path) instead of the direct call")
    ap.add_argument("--pingpong", action="store_true",
                    help="attention workload: the ping-pong schedule of the softmax B2BGEMM "
                         "(cf_set_b2b_pingpong; two wave groups per CU alternating MFMA and softmax phases)")
    ap.add_argument("--leader-tiles", type=int, default=-1, metavar="T",
                    help="strips of at least T column tiles exchange leader-follower (0: never; default: the "
                         "library's setting)")
    ap.add_argument("--eager", action="store_true",
                    help="time K eager launches from Python instead of one replay of a HIP graph that holds the "
                         "K launches (the graph removes the host's per-launch cost from the timed region)")
    ap.add_argument("--rotate-mb", type=int, default=512,
                    help="cycle through copies of the inputs totalling at least this many MiB, so that they are "
                         "read from HBM rather than from the 256 MiB last-level cache (0: one set)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the HIP sources: measured traffic is valid only for the kernels it was taken on."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "b2bgemm_stage_stream_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _counter_rows(d: str):
    """(kernel name, counter name, value) of every dispatch in the rocprofv3
    counter-collection csv files under d."""
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                out.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), r.get("Dispatch_Id")))
    return out


def _per_dispatch(d: str, counter: str, match):
    """Mean counter value per dispatch of the kernels whose name satisfies
    `match`, and the most frequent such kernel name."""
    rows = [r for r in _counter_rows(d) if r[1] == counter and match(r[0])]
    if not rows:
        raise SystemExit(f"no {counter} values for the kernel under {d}")
    per = {}
    for name, _, v, disp in rows:
        per.setdefault((name, disp), 0.0)
        per[(name, disp)] += v           # summed over the counter's instances
    names = {}
    for (name, _), _v in per.items():
        names[name] = names.get(name, 0) + 1
    top = max(names, key=names.get)
    vals = [v for (name, _), v in per.items() if name == top]
    return float(np.mean(vals)), top, len(vals)


def ingest_counters(d: str, out_path: str) -> dict:
    """profiles/traffic.json from the FETCH_SIZE / WRITE_SIZE runs: per-dispatch
    KiB of each workload's fused kernel, scaled by what the same counters read
    for a plain copy of known size (copy probe), and the sources they were
    taken on (their hash)."""
    def is_cf(n):
        return "cf::" in n and "workspace_clear" not in n

    def is_copy(n):
        return "cf::" not in n

    probe = json.load(open(os.path.join(d, "copy_probe.json")))
    nbytes = probe["copy_probe_bytes_each_way"]
    fk, _, _ = _per_dispatch(os.path.join(d, "fetch_copy"), "FETCH_SIZE", is_copy)
    wk, _, _ = _per_dispatch(os.path.join(d, "write_copy"), "WRITE_SIZE", is_copy)
    rec = {"kernel_source_hash": kernel_source_hash(),
           "copy_probe": {"bytes_each_way": nbytes, "fetch_kib": fk, "write_kib": wk},
           "factor_fetch": nbytes / (fk * 1024.0), "factor_write": nbytes / (wk * 1024.0),
           "note": "HBM-side bytes per launch = counter KiB * 1024 * factor; the factors make a plain copy of "
                   "known size read and write exactly its size",
           "workloads": {}}
    for sub in sorted(os.listdir(d)):
        if not sub.startswith("fetch_") or sub == "fetch_copy":
            continue
        name = sub[len("fetch_"):]
        f, kname, nd = _per_dispatch(os.path.join(d, sub), "FETCH_SIZE", is_cf)
        w_, kname2, _ = _per_dispatch(os.path.join(d, "write_" + name), "WRITE_SIZE", is_cf)
        rec["workloads"][name] = {"kernel": kname, "dispatches": nd, "fetch_kib": f, "write_kib": w_,
                                  "fetch_bytes": f * 1024.0 * rec["factor_fetch"],
                                  "write_bytes": w_ * 1024.0 * rec["factor_write"]}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


def copy_probe(mib: int, steps: int):
    """A plain copy of a known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "steps": steps}), flush=True)


def visible_pairs(M: int, L: int) -> int:
    """(query, key) pairs a causal mask leaves: row m sees keys 0 .. m + L - M."""
    return int(sum(min(L, max(0, m + L - M + 1)) for m in range(M)))


def flops_of(w, causal: bool = False) -> float:
    d = w.dims
    if w.kind == "gemm_epilogue":
        return 2.0 * d["M"] * d["N"] * d["K"]
    pairs = visible_pairs(d["M"], d["L"]) if causal else d["M"] * d["L"]
    return 2.0 * d["batch"] * pairs * (d["K"] + d["N"])


def bytes_of(w, store_x: bool = False, argmax: bool = False, topk: int = 0) -> float:
    """Algorithmic HBM bytes: every input read once, the output (and X when
    stored) written once; an argmax writes only its index and maximum per row."""
    tot = 0.0
    for t in w.tensors:
        tot += np.prod(w.shape(t)) * (2 if t.dtype == "bf16" else 4)
    d = w.dims
    out_es = 4 if w.params.get("out_dtype") == "f32" else 2
    if w.kind == "gemm_epilogue":
        tot += d["M"] * 8 * (topk or 1) if (argmax or topk) else d["M"] * d["N"] * out_es
        if store_x:
            tot += d["M"] * d["N"] * 2
    else:
        tot += d["batch"] * d["M"] * d["N"] * out_es
    return float(tot)


def output_bytes(w, store_x: bool = False, argmax: bool = False, topk: int = 0) -> float:
    """Bytes the kernel must write: the output (and X when stored); an argmax
    or top-k writes only its indices and values per row."""
    d = w.dims
    out_es = 4 if w.params.get("out_dtype") == "f32" else 2
    if w.kind == "gemm_epilogue":
        tot = d["M"] * 8 * (topk or 1) if (argmax or topk) else d["M"] * d["N"] * out_es
        if store_x:
            tot += d["M"] * d["N"] * 2
        return float(tot)
    return float(d["batch"] * d["M"] * d["N"] * out_es)


def is_f32(w) -> bool:
    return any(t.dtype == "f32" for t in w.tensors if t.name == "A")


def roofline_of(w, kernel_ms: float, store_x: bool = False, causal: bool = False, argmax: bool = False, topk: int = 0):
    """The roofline that bounds the kernel: HBM when the workload's flop/byte is
    below the ridge point (peak flops / HBM bandwidth), the MFMA peak above it.
    Returns (bound, unit, peak, achieved, intensity, ridge)."""
    flops, nbytes = flops_of(w, causal), bytes_of(w, store_x, argmax, topk)
    peak_flops = PEAK_F32_TFLOPS if is_f32(w) else PEAK_BF16_TFLOPS
    intensity = flops / nbytes
    ridge = peak_flops * 1e12 / (HBM_GBPS * 1e9)
    if intensity < ridge:
        return "hbm", "GB/s", HBM_GBPS, nbytes / (kernel_ms * 1e-3) / 1e9, intensity, ridge
    return "mfma", "TFLOP/s", peak_flops, flops / (kernel_ms * 1e-3) / 1e12, intensity, ridge


def fuse_call(w, dev, torch):
    """The workload as a torch function, lowered by fuse.lower; a closure running the lowered call."""
    import torch.nn.functional as F
    from b2bgemm_stage_stream_amd import fuse
    p, d = w.params, w.dims
    if w.name == "c2_gemm_layernorm":
        n, eps = d["N"], p["eps"]

        def fn(a, b, g, be):
            return F.layer_norm(a @ b, (n,), g, be, eps)
        args = (dev["A"], dev["B"], dev["gamma"], dev["beta"])
    elif w.name == "c3_gemm_residual_rmsnorm":
        n, eps = d["N"], p["eps"]

        def fn(a, b, r, g):
            return F.rms_norm(a @ b + r, (n,), g, eps)
        args = (dev["A"], dev["B"], dev["residual"], dev["weight"])
    elif w.name == "c4_b2b_mlp_relu":
        def fn(x, w0, w1):
            return torch.relu(x @ w0) @ w1
        args = (dev["A"], dev["B0"], dev["B1"])
    elif w.name == "c5_b2b_attention":
        alpha = p["alpha"]

        def fn(q, k, v):
            return torch.softmax((q @ k.transpose(-1, -2)) * alpha, dim=-1) @ v
        args = (dev["A"], dev["B0"], dev["B1"])
    else:
        raise SystemExit(f"--via-fuse: no torch form of {w.name}")
    run = fuse.lower(fn, *args)

    def call():
        call.last = run(*args)
    return call


def make_call(w, dev, torch, cf, store_x: bool = False, causal: bool = False, argmax: bool = False, row2=None,
              topk: int = 0, b_nk: bool = False, column: bool = False, row_stats: bool = False):
    """Device tensors + a closure launching one fused kernel on the current stream."""
    p = w.params
    out_dt = torch.float32 if p.get("out_dtype") == "f32" else torch.bfloat16
    stream = None   # torch's current stream at call time (a graph's capture stream while capturing)
    if w.kind == "gemm_epilogue":
        d = w.dims
        X = torch.empty(d["M"], d["N"], dtype=torch.bfloat16, device="cuda") if store_x else None
        if topk:
            idx = torch.empty(d["M"], topk, dtype=torch.int32, device="cuda")
            mx = torch.empty(d["M"], topk, dtype=torch.float32, device="cuda")
            e = cf.make_epilogue(alpha=p["alpha"], bias=dev.get("bias"), act=p["act"], row_op="topk", topk=topk,
                                 row_index=idx, row_stats=mx, x_out=X)
            C = None
        elif argmax:
            idx = torch.empty(d["M"], dtype=torch.int32, device="cuda")
            mx = torch.empty(d["M"], dtype=torch.float32, device="cuda")
            e = cf.make_epilogue(alpha=p["alpha"], bias=dev.get("bias"), residual=dev.get("residual"),
                                 act=p["act"], row_op="argmax", row_index=idx, row_stats=mx, x_out=X)
            C = None
        else:
            idx = None
            g = dev.get("gamma", dev.get("weight"))
            per = (d["N"] if column else d["M"]) * (2 if p["row_op"] == "layernorm" else 1)
            mx = torch.empty(per, dtype=torch.float32, device="cuda") if row_stats else None
            e = cf.make_epilogue(alpha=p["alpha"], bias=dev.get("bias"), residual=dev.get("residual"),
                                 act=p["act"], row_op=p["row_op"], gamma=g, beta=dev.get("beta"),
                                 eps=p.get("eps", 0.0), x_out=X, row_op2=row2 or "none", row_stats=mx,
                                 axis="column" if column else "row",
                                 gamma2=g if row2 in ("layernorm", "rmsnorm") else None,
                                 beta2=dev.get("beta") if row2 == "layernorm" else None,
                                 eps2=p.get("eps", 0.0) if row2 else 0.0)
            C = torch.empty(d["M"], d["N"], dtype=out_dt, device="cuda")
        nbytes = cf.cf_gemm_epilogue_workspace_size(d["M"], d["N"], d["K"], e)
        ws = cf.Workspace("cuda").get(nbytes)

        def call():
            cf.cf_gemm_epilogue(dev["A"], dev["B"], C, b_is_nk=b_nk, epi=e, workspace=ws, stream=stream)
        call.keep = (X, idx, mx)   # the extra outputs live as long as the closure
        return call, C, ws, nbytes
    d = w.dims
    e = cf.make_epilogue(alpha=p["alpha"], act=p["act"], row_op=p["row_op"], mask="causal" if causal else "none")
    O = torch.empty(d["batch"], d["M"], d["N"], dtype=out_dt, device="cuda")
    lk = p["b0_layout"] == "lk"

    def call():
        cf.cf_b2bgemm(dev["A"], dev["B0"], dev["B1"], O, b0_is_lk=lk, epi=e, stream=stream)
    return call, O, None, 0


def host_cpu():
    """CPU model, physical cores and logical CPUs of this host, from /proc/cpuinfo."""
    model, phys = None, set()
    cur = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f.read().splitlines() + [""]:
                if not line.strip():
                    if "core id" in cur:
                        phys.add((cur.get("physical id", "0"), cur["core id"]))
                    cur = {}
                    continue
                k, _, v = line.partition(":")
                cur[k.strip()] = v.strip()
                if k.strip() == "model name" and model is None:
                    model = v.strip()
    except OSError:
        pass
    return {"cpu_model": model, "physical_cores": len(phys) or None, "logical_cpus": os.cpu_count()}


def blas_threads() -> int:
    """Threads numpy's BLAS (the oracle's matmul) runs with."""
    try:
        import threadpoolctl
        n = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(w, raw, target_s: float, causal: bool = False, argmax: bool = False, row2=None, topk: int = 0):
    """The fp64 oracle on a bounded sample of rows (rows are independent). The
    inputs are widened to fp64 once, outside the timed runs."""
    import oracle
    p = w.params
    d = w.dims

    def widen(name):
        t = next(t for t in w.tensors if t.name == name)
        return oracle.widen_bf16(raw[name]) if t.dtype == "bf16" else raw[name].astype(np.float64)

    if w.kind == "gemm_epilogue":
        B = widen("B")
        vec = {k: widen(k) for k in ("bias", "gamma", "beta", "weight") if k in raw}
        A_all = widen("A")
        R_all = widen("residual") if "residual" in raw else None

        def run(rows):
            A = A_all[:rows]
            R = R_all[:rows] if R_all is not None else None
            g = vec.get("gamma", vec.get("weight"))
            if topk:
                oracle.gemm_epilogue_topk(A, B, topk, alpha=p["alpha"], bias=vec.get("bias"), act=p["act"])
            elif argmax:
                oracle.gemm_epilogue_argmax(A, B, alpha=p["alpha"], bias=vec.get("bias"), residual=R, act=p["act"])
            elif row2:
                oracle.gemm_epilogue_two_stage(
                    A, B, alpha=p["alpha"], bias=vec.get("bias"), residual=R, act=p["act"], row_op=p["row_op"],
                    gamma=g, beta=vec.get("beta"), eps=p.get("eps", 0.0), row_op2=row2,
                    gamma2=g if row2 in ("layernorm", "rmsnorm") else None,
                    beta2=vec.get("beta") if row2 == "layernorm" else None, eps2=p.get("eps", 0.0))
            else:
                oracle.gemm_epilogue(A, B, alpha=p["alpha"], bias=vec.get("bias"), residual=R, act=p["act"],
                                     row_op=p["row_op"], gamma=vec.get("gamma", vec.get("weight")),
                                     beta=vec.get("beta"), eps=p.get("eps", 0.0))
        unit_flops = 2.0 * d["N"] * d["K"]          # per row
        total_units = d["M"]
        what = "rows of the output"
    else:
        A, B0, B1 = widen("A"), widen("B0"), widen("B1")

        def run(rows):   # rows = number of (batch) problems
            oracle.b2bgemm(A[:rows], B0[:rows] if B0.shape[0] > 1 else B0, B1[:rows] if B1.shape[0] > 1 else B1,
                           alpha=p["alpha"], act=p["act"], row_op=p["row_op"], b0_layout=p["b0_layout"],
                           causal=causal)
        if d["batch"] > 1:
            unit_flops = flops_of(w, causal) / d["batch"]
            total_units = d["batch"]
            what = "independent (batch, head) problems"
        else:
            # single batch: sample rows of A
            A0 = A

            def run(rows):  # noqa: F811
                oracle.b2bgemm(A0[:, :rows], B0, B1, alpha=p["alpha"], act=p["act"], row_op=p["row_op"],
                               b0_layout=p["b0_layout"])
            unit_flops = 2.0 * (d["K"] * d["L"] + d["L"] * d["N"])
            total_units = d["M"]
            what = "rows of the output"
    # calibrate on a small sample, then time the bounded sample
    n0 = max(1, min(total_units, 64))
    t = time.perf_counter()
    run(n0)
    t0 = time.perf_counter() - t
    n = int(min(total_units, max(n0, n0 * target_s / max(t0, 1e-6))))
    # when the whole workload is quicker than the target, repeat it
    reps, dt = 0, 0.0
    while reps == 0 or (n == total_units and dt < target_s and reps < 100):
        t = time.perf_counter()
        run(n)
        dt += time.perf_counter() - t
        reps += 1
    tflops = reps * n * unit_flops / dt / 1e12
    rep_txt = f" x {reps} runs" if reps > 1 else ""
    return {"value": tflops, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n} of {total_units} {what} of the same workload{rep_txt}, fp64, {dt:.1f} s",
            **host_cpu()}


def main():
    args = parse()
    if args.ingest_counters:
        rec = ingest_counters(args.ingest_counters, args.traffic)
        print(json.dumps(rec["workloads"], indent=1))
        return
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (every box here has one GPU)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import b2bgemm_stage_stream_amd as cf
    import gen
    sys.path.insert(0, os.path.join(ROOT, "tests"))

    dims = {k: int(v) for k, v in (kv.split("=") for kv in args.dims.split(",") if kv)}
    w = gen.workload(args.workload, **dims)
    if args.leader_tiles >= 0:
        cf.cf_set_exchange_leader_tiles(args.leader_tiles)
    if args.pingpong:
        cf.cf_set_b2b_pingpong(1)
    if args.store_x and w.kind != "gemm_epilogue":
        raise SystemExit("--store-x applies to the GEMM + epilogue workloads")
    if args.row2 and (w.kind != "gemm_epilogue" or args.argmax or w.params["row_op"] == "none"):
        raise SystemExit("--row2 applies to the GEMM + epilogue workloads with a row operation, without --argmax")
    if args.topk and (w.kind != "gemm_epilogue" or "residual" in {t.name for t in w.tensors} or args.argmax
                      or args.row2 or not 1 <= args.topk <= 8):
        raise SystemExit("--topk K (1..8) applies to the GEMM + epilogue workloads without a residual, alone")
    if args.via_fuse and (args.store_x or args.causal or args.argmax or args.row2 or args.topk or args.b_nk
                          or args.column or args.row_stats or args.plain or args.dims):
        raise SystemExit("--via-fuse times the workload as it is, with no other variant flag")
    if (args.column or args.row_stats) and (w.kind != "gemm_epilogue" or args.argmax or args.topk or args.row2
                                            or w.params["row_op"] == "none"):
        raise SystemExit("--column and --row-stats apply to the GEMM + epilogue workloads' own row operation")
    if args.argmax and w.kind != "gemm_epilogue":
        raise SystemExit("--argmax applies to the GEMM + epilogue workloads")
    if args.b_nk and w.kind != "gemm_epilogue":
        raise SystemExit("--b-nk applies to the GEMM + epilogue workloads")
    if args.causal and (w.kind != "b2bgemm" or w.params["row_op"] != "softmax"):
        raise SystemExit("--causal applies to the attention (softmax B2BGEMM) workload")
    if args.plain:
        import dataclasses
        w = dataclasses.replace(w, params={**w.params, "row_op": "none", "act": "none"},
                                tensors=tuple(t for t in w.tensors if t.name in ("A", "B", "B0", "B1")))
    raw = gen.make(w, seed=args.seed)

    def to_dev(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    dev = {t.name: to_dev(raw[t.name], t.dtype) for t in w.tensors}
    if args.b_nk:
        dev["B"] = dev["B"].t().contiguous()
    in_bytes = sum(v.numel() * v.element_size() for v in dev.values())
    nset = 1 if args.rotate_mb <= 0 else max(1, min(64, -(-args.rotate_mb * (1 << 20) // in_bytes)))
    devs = [dev] + [{k: v.clone() for k, v in dev.items()} for _ in range(nset - 1)]
    calls = []
    for d_ in devs:
        if args.via_fuse:
            call, ws, ws_bytes = fuse_call(w, d_, torch), None, 0
        else:
            call, out, ws, ws_bytes = make_call(w, d_, torch, cf, args.store_x, args.causal, args.argmax, args.row2,
                                                args.topk, args.b_nk, args.column, args.row_stats)
        calls.append(call)

    # settle: batches of calls (grown to ~20 ms each) until --settle-s has passed
    settle_steps, batch = 0, 4
    t_s = time.perf_counter()
    while time.perf_counter() - t_s < args.settle_s:
        t_b = time.perf_counter()
        for _ in range(batch):
            calls[settle_steps % nset]()
            settle_steps += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t_b < 0.02 and batch < 4096:
            batch *= 2
    settle_s = time.perf_counter() - t_s
    for i in range(max(args.warmup, nset)):
        calls[i % nset]()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        # the K timed launches, captured once (same kernels and arguments as
        # the eager calls) and replayed as one graph on the launch stream
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                calls[i % nset]()
        torch.cuda.synchronize()
        graph.replay()   # untimed first replay
        torch.cuda.synchronize()
    start_ev = torch.cuda.Event(enable_timing=True)
    end_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start_ev.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            calls[i % nset]()
    end_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ws is not None and cf.cf_workspace_status(ws) != cf.CF_OK:
        raise SystemExit("strip exchange timed out during the benchmark")
    kernel_ms = start_ev.elapsed_time(end_ev) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    flops = flops_of(w, args.causal)
    value = flops / (ms_per_step * 1e-3) / 1e12
    in_f32 = is_f32(w)
    bound, unit, peak, achieved, intensity, ridge = roofline_of(w, kernel_ms, args.store_x, args.causal,
                                                                args.argmax, args.topk)
    # HBM-side bytes per launch from the byte counters, when they were taken on
    # these kernel sources and this exact workload; the unfused intermediate's
    # share is what the kernel writes beyond its output and the exchange
    # workspace (0 when the writes come to less: workspace lines still held in
    # the caches when the counters were read)
    traffic = intermediate = None
    out_bytes = output_bytes(w, args.store_x, args.argmax, args.topk)
    if os.path.exists(args.traffic) and not (args.plain or args.store_x or args.causal or args.argmax or args.row2
                                             or args.topk or args.b_nk or args.dims or args.column or args.row_stats
                                             or args.via_fuse):
        try:
            rec = json.load(open(args.traffic))
            if rec.get("kernel_source_hash") == kernel_source_hash():
                t = rec.get("workloads", {}).get(args.workload)
                if t:
                    traffic = round(t["fetch_bytes"] + t["write_bytes"])
                    intermediate = max(0, round(t["write_bytes"] - out_bytes - (ws_bytes or 0)))
        except (OSError, ValueError, KeyError):
            traffic = intermediate = None
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": round(settle_s, 3), "steps": settle_steps},
        "timing": "eager launches" if args.eager else "one HIP graph replay of the K launches",
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if in_f32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + (f"@{args.dims}" if args.dims else "") + ("/identity-epilogue" if args.plain else "")
                   + ("+x_out" if args.store_x else "") + ("/causal" if args.causal else "")
                   + ("/argmax" if args.argmax else "") + (f"/then-{args.row2}" if args.row2 else "")
                   + ("/over-columns" if args.column else "") + ("/row-stats" if args.row_stats else "")
                   + ("/via-fuse" if args.via_fuse else "")
                   + (f"/top-{args.topk}" if args.topk else "") + ("/B[N,K]" if args.b_nk else ""), **w.dims,
                   "out_dtype": w.params.get("out_dtype"), "input_sets": nset, "input_bytes_per_set": in_bytes},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "arithmetic_intensity": round(intensity, 1), "ridge": round(ridge, 1)},
        "kernel_ms": round(kernel_ms, 4),
        "exchange_leader_tiles": cf.cf_set_exchange_leader_tiles(-1),
        "b2b_pingpong": cf.cf_set_b2b_pingpong(-1),
        "algorithmic_bytes": bytes_of(w, args.store_x, args.argmax, args.topk),
        "intermediate_hbm_bytes": intermediate,
        "output_bytes": out_bytes,
        "workspace_bytes": ws_bytes,
    }
    if not args.no_cpu_baseline:
        del dev, devs, calls, out
        line["cpu_baseline"] = cpu_baseline(w, raw, args.cpu_seconds, args.causal, args.argmax, args.row2, args.topk)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
