"""Lowering of a traced torch subgraph to one fused call.

A small analogue of the front-end the ComFuse review describes (the abstract
and "What carries the argument": a compiler that turns tensor subprograms into
fused kernels by itself, through a fusion specification rather than a fixed
table of patterns). Here the subprogram is a torch function traced with
torch.fx; every node is placed by its operator and the shapes of its operands
into the stage stream of one kernel:

  GEMM  P = A . B          (B given [K, N], or [N, K] through a transpose)
  stage 1 (elementwise, in this order, each optional):
        scale by a Python number, + bias [N], + residual [M, N], ReLU
  boundary (optional, last axis): softmax, layer_norm, rms_norm, or a second
        GEMM that consumes the result (back-to-back GEMM; its first stage may
        be a scale, ReLU or softmax)
  second boundary (optional, GEMM + epilogue only): softmax, layer_norm or
        rms_norm of the first one's result

and the stream becomes one ``cf_gemm_epilogue`` or ``cf_b2bgemm`` call. The
stage-1 value may also be an output of the function (it is then stored as the
epilogue's second output). A node that has no place in the stream, or comes
out of order, raises ``NotFusable`` with the reason. This module only
classifies and marshals; every step of the computation runs in the library's
kernels.
"""
from __future__ import annotations

import operator
from dataclasses import dataclass, field
from typing import Any, Callable, Dict, List, Optional, Tuple

import torch
import torch.fx as fx
import torch.nn.functional as F
from torch.fx.passes.shape_prop import ShapeProp

__all__ = ["NotFusable", "Plan", "FusedFunction", "lower"]


class NotFusable(Exception):
    """The traced subgraph does not fit one fused call."""


_MATMUL = {operator.matmul, torch.matmul, torch.mm, torch.bmm}
_RELU = {torch.relu, F.relu}
_SOFTMAX = {torch.softmax, F.softmax}
_STAGES = ("alpha", "bias", "residual", "act")   # the epilogue's fixed order


@dataclass
class Plan:
    kind: str                                   # "gemm_epilogue" or "b2bgemm"
    a: int                                      # placeholder index of A
    b: int                                      # placeholder index of B (B0)
    b_transposed: bool                          # B given [N, K] (B0 given [L, K])
    b1: Optional[int] = None                    # B1 (second GEMM)
    epi: Dict[str, Any] = field(default_factory=dict)      # scalar descriptor fields
    tensors: Dict[str, int] = field(default_factory=dict)  # bias/residual/gamma/beta -> placeholder index
    outputs: List[str] = field(default_factory=list)       # "y" (the result) and/or "x" (stage 1)


def _shape(n) -> Tuple[int, ...]:
    tm = n.meta.get("tensor_meta")
    if tm is None:
        raise NotFusable(f"no shape for {n.name}")
    return tuple(tm.shape)


def _is_matmul(n) -> bool:
    return (n.op == "call_function" and n.target in _MATMUL) or (n.op == "call_method" and n.target in ("matmul", "mm", "bmm"))


def _is_transpose(n) -> bool:
    if n.op == "call_method" and n.target == "t":
        return True
    if n.op == "call_function" and n.target is torch.t:
        return True
    if (n.op == "call_method" and n.target == "transpose") or (n.op == "call_function" and n.target is torch.transpose):
        dims = n.args[1:3]
        nd = len(_shape(n))
        return sorted(d % nd for d in dims) == [nd - 2, nd - 1]
    return n.op == "call_function" and n.target is getattr and n.args[1] == "T"


def _operand(n, placeholders) -> Tuple[int, bool]:
    """(placeholder index, transposed) of a GEMM operand."""
    if n.op == "placeholder":
        return placeholders.index(n), False
    if _is_transpose(n) and n.args[0].op == "placeholder":
        return placeholders.index(n.args[0]), True
    raise NotFusable(f"GEMM operand {n.name} is neither an input nor a transposed input")


def _last_axis(n, dim) -> bool:
    return dim is not None and dim % len(_shape(n)) == len(_shape(n)) - 1


def _shape_query(u) -> bool:
    """A use of a node that reads only its shape (x.shape, x.size(), x.dim())."""
    return (u.op == "call_function" and u.target is getattr and u.args[1] in ("shape", "ndim")) or \
        (u.op == "call_method" and u.target in ("size", "dim"))


def _single_user(n, outputs) -> Optional[fx.Node]:
    users = [u for u in n.users if u.op != "output" and not _shape_query(u)]
    if len(users) > 1:
        raise NotFusable(f"{n.name} feeds {len(users)} nodes; one stream has one consumer per stage")
    return users[0] if users else None


def _place_row_op(u, N, placeholders, plan, stage: str) -> bool:
    """Places u into the descriptor if it is a row operation over the last axis:
    row_op/gamma/beta/eps for the first boundary (stage ""), row_op2/gamma2/
    beta2/eps2 for the second ("2"). False if u is no row operation."""
    if u is None:
        return False
    if (u.op == "call_function" and u.target in _SOFTMAX) or (u.op == "call_method" and u.target == "softmax"):
        dim = u.kwargs.get("dim", u.args[1] if len(u.args) > 1 else None)
        if not _last_axis(u, dim):
            raise NotFusable("softmax over an axis other than the last")
        plan.epi["row_op" + stage] = "softmax"
        return True
    if u.op == "call_function" and u.target in (F.layer_norm, F.rms_norm):
        shape = u.args[1] if len(u.args) > 1 else u.kwargs["normalized_shape"]
        if len(shape) != 1:
            raise NotFusable("the normalisation must be over the last axis only")
        is_ln = u.target is F.layer_norm
        names = ("weight", "bias", "eps") if is_ln else ("weight", "eps")
        vals = dict(zip(names, u.args[2:]))
        vals.update({k: v for k, v in u.kwargs.items() if k in names})
        for k, role in (("weight", "gamma"), ("bias", "beta")):
            t = vals.get(k)
            if t is None:
                continue
            if not (isinstance(t, fx.Node) and t.op == "placeholder" and _shape(t) == (N,)):
                raise NotFusable(f"the {k} of {u.name} must be an input of shape [N]")
            plan.tensors[role + stage] = placeholders.index(t)
        eps = vals.get("eps", 1e-5 if is_ln else None)
        if eps is None:
            raise NotFusable("rms_norm without an explicit eps")
        plan.epi.update({"row_op" + stage: "layernorm" if is_ln else "rmsnorm", "eps" + stage: float(eps)})
        return True
    return False


def lower(fn: Callable, *example_args) -> "FusedFunction":
    """Trace ``fn`` and lower it to one fused call; the example arguments give
    the shapes (any device; shapes are propagated on meta tensors, so nothing
    of ``fn`` is executed)."""
    gm = fx.symbolic_trace(fn)
    metas = [torch.empty(a.shape, dtype=a.dtype, device="meta") if isinstance(a, torch.Tensor) else a
             for a in example_args]
    ShapeProp(gm).propagate(*metas)
    placeholders = [n for n in gm.graph.nodes if n.op == "placeholder"]
    out_node = next(n for n in gm.graph.nodes if n.op == "output")
    outs = out_node.args[0] if isinstance(out_node.args[0], (tuple, list)) else (out_node.args[0],)
    mms = [n for n in gm.graph.nodes if _is_matmul(n)]
    if not mms:
        raise NotFusable("no matrix product in the subgraph")
    mm = mms[0]
    a, a_t = _operand(mm.args[0], placeholders)
    if a_t:
        raise NotFusable("the left operand must be stored [M, K]")
    b, b_t = _operand(mm.args[1], placeholders)
    plan = Plan(kind="gemm_epilogue", a=a, b=b, b_transposed=b_t)
    M, N = _shape(mm)[-2], _shape(mm)[-1]

    alpha, done = 1.0, -1          # index in _STAGES of the last stage placed
    node, x_node = mm, mm
    while True:
        u = _single_user(node, outs)
        if u is None:
            break
        tgt = u.target
        scalar = None
        if u.op == "call_function" and tgt in (operator.mul, torch.mul) and len(u.args) == 2:
            scalar = u.args[1] if u.args[0] is node else u.args[0]
        elif u.op == "call_function" and tgt is operator.truediv and u.args[0] is node:
            scalar = u.args[1]
        if scalar is not None:
            if not isinstance(scalar, (int, float)):
                raise NotFusable(f"{u.name} multiplies by something other than a number")
            if done >= 0:
                raise NotFusable("a scale after a bias, residual or activation is out of the stream's order")
            alpha = alpha / scalar if tgt is operator.truediv else alpha * scalar
        elif u.op == "call_function" and tgt in (operator.add, torch.add) and len(u.args) == 2:
            other = u.args[1] if u.args[0] is node else u.args[0]
            if not (isinstance(other, fx.Node) and other.op == "placeholder"):
                raise NotFusable(f"{u.name} adds something other than an input")
            shp = _shape(other)
            role = "bias" if shp == (N,) else "residual" if shp[-2:] == (M, N) and len(shp) == 2 else None
            if role is None:
                raise NotFusable(f"{u.name} adds a tensor of shape {shp}, neither [N] nor [M, N]")
            if _STAGES.index(role) <= done:
                raise NotFusable(f"{role} after a later stage is out of the stream's order")
            plan.tensors[role] = placeholders.index(other)
            done = _STAGES.index(role)
        elif (u.op == "call_function" and tgt in _RELU) or (u.op == "call_method" and tgt == "relu"):
            if done >= 3:
                raise NotFusable("a second activation")
            plan.epi["act"] = "relu"
            done = 3
        else:
            break
        node = x_node = u

    plan.epi["alpha"] = float(alpha)
    # ---- the boundaries: up to two row reductions over the last axis, and/or a second GEMM
    y_node = node
    u = _single_user(node, outs)
    for stage in ("", "2"):
        if not _place_row_op(u, N, placeholders, plan, stage):
            break
        if stage == "2" and any(o is y_node for o in outs):
            raise NotFusable("the first row stage's result is not stored beside a second one")
        y_node, u = u, _single_user(u, outs)
    if u is not None and _is_matmul(u):
        if u.args[0] is not y_node:
            raise NotFusable("the second GEMM must take the first one's result as its left operand")
        b1, b1_t = _operand(u.args[1], placeholders)
        if b1_t:
            raise NotFusable("the second GEMM's right operand must be stored [L, N]")
        if plan.epi.get("row_op") not in (None, "softmax") or "row_op2" in plan.epi or "residual" in plan.tensors:
            raise NotFusable("between two GEMMs only a scale, bias, ReLU or softmax may stand")
        if plan.epi.get("row_op") == "softmax" and ("bias" in plan.tensors or "act" in plan.epi):
            raise NotFusable("a softmax between two GEMMs takes the scaled scores as they are")
        if any(o is x_node or o is y_node for o in outs):
            raise NotFusable("the intermediate of a back-to-back GEMM is never stored")
        plan.kind, plan.b1 = "b2bgemm", b1
        y_node, u = u, _single_user(u, outs)
    if u is not None:
        raise NotFusable(f"{u.name} ({u.target}) has no place in the stream")
    for o in outs:
        if o is y_node:
            plan.outputs.append("y")
        elif o is x_node and x_node is not y_node:
            plan.outputs.append("x")
        else:
            raise NotFusable(f"output {getattr(o, 'name', o)} is not produced by the stream")
    return FusedFunction(plan)


class FusedFunction:
    """Callable running a lowered plan on new arguments of the traced shapes.

    A row reduction over several column tiles waits for the partial statistics
    of the other workgroups of its row strip. If some of them never run
    alongside (another kernel holds the compute units), the wait gives up after
    the exchange time limit: the rows concerned come out as NaN and the
    workspace records the timeout. ``check=True`` waits for the call and raises
    RuntimeError in that case."""

    def __init__(self, plan: Plan):
        self.plan = plan
        self._ws = None

    def __call__(self, *args, out_dtype=None, check: bool = False):
        from . import (CF_OK, Workspace, cf_b2bgemm, cf_gemm_epilogue, cf_gemm_epilogue_workspace_size,
                       cf_status_string, cf_workspace_status, make_epilogue)
        p = self.plan
        A, B = args[p.a], args[p.b]
        odt = out_dtype or A.dtype
        vec = {k: args[i] for k, i in p.tensors.items()}
        kw = dict(p.epi)
        if p.kind == "b2bgemm":
            B1 = args[p.b1]
            O = torch.empty(*A.shape[:-2], A.shape[-2], B1.shape[-1], dtype=odt, device=A.device)
            cf_b2bgemm(A, B, B1, O, b0_is_lk=p.b_transposed, bias=vec.get("bias"), **kw)
            return O
        M, N = A.shape[0], (B.shape[0] if p.b_transposed else B.shape[1])
        X = torch.empty(M, N, dtype=odt, device=A.device) if "x" in p.outputs else None
        C = torch.empty(M, N, dtype=odt, device=A.device)
        e = make_epilogue(bias=vec.get("bias"), residual=vec.get("residual"), gamma=vec.get("gamma"),
                          beta=vec.get("beta"), gamma2=vec.get("gamma2"), beta2=vec.get("beta2"), x_out=X, **kw)
        if self._ws is None:
            self._ws = Workspace(str(A.device))
        ws = self._ws.get(cf_gemm_epilogue_workspace_size(M, N, A.shape[1], e))
        cf_gemm_epilogue(A, B, C, b_is_nk=p.b_transposed, epi=e, workspace=ws)
        if check and ws is not None:
            st = cf_workspace_status(ws)
            if st != CF_OK:
                raise RuntimeError(f"fused call failed on the device: {cf_status_string(st)}")
        res = {"y": C, "x": X}
        outs = tuple(res[o] for o in p.outputs)
        return outs[0] if len(outs) == 1 else outs
