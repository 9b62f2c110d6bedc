"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments with the documented status before
any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import b2bgemm_stage_stream_amd as cf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cf.h")
lib = cf._lib

# plausible (aligned, non-null) device addresses; never dereferenced here
PA, PB, PC, PW = 0x7F0000000000, 0x7F0000100000, 0x7F0000200000, 0x7F0000300000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cf_[a-z0-9_]+)\s*\(", text)))


def gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "cf_gemm_epilogue" in names and "cf_b2bgemm" in names
    out = subprocess.run(["nm", "-D", "--defined-only", cf.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (cf_[a-z0-9_]+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)
    assert set(cf.EXPORTED) == set(names)


def test_descriptor_layout_matches_header():
    e = cf.cf_epilogue()
    lib.cf_epilogue_init(ctypes.byref(e))
    assert e.struct_size == ctypes.sizeof(cf.cf_epilogue)
    assert e.alpha == 1.0 and e.row_op == 0 and e.act == 0


def test_status_strings_and_version():
    assert cf.cf_status_string(0) == "CF_OK"
    assert cf.cf_status_string(6) == "CF_ERR_DEVICE_TIMEOUT"
    assert cf.cf_status_string(99) == "CF_ERR_UNKNOWN"
    assert "gfx950" in cf.cf_version()
    old = cf.cf_set_exchange_timeout_us(1234)
    assert cf.cf_set_exchange_timeout_us(old) == 1234
    assert cf.cf_set_exchange_leader_tiles(-1) == cf.cf_set_exchange_leader_tiles(-1)
    prev = cf.cf_set_b2b_pingpong(1)
    assert prev == 0   # off unless selected
    assert cf.cf_set_b2b_pingpong(-1) == 1   # a negative value only reads it
    assert cf.cf_set_b2b_pingpong(prev) == 1
    assert cf.cf_set_b2b_pingpong(-1) == 0


def gemm(M=64, N=64, K=64, A=PA, lda=64, B=PB, ldb=64, nk=0, abt=1, C=PC, ldc=64, ct=1, epi=None, ws=None,
         wsb=0):
    return lib.cf_gemm_epilogue(M, N, K, A, lda, B, ldb, nk, abt, C, ldc, ct,
                                ctypes.byref(epi) if epi is not None else None, ws, wsb, None)


def epi(**kw):
    e = cf.cf_epilogue()
    lib.cf_epilogue_init(ctypes.byref(e))
    for k, v in kw.items():
        setattr(e, k, v)
    return e


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(K=-5), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(abt=7), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(ct=3), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(nk=2), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(C=None), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(A=None), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(lda=63), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(ldb=32), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(ldc=10), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(A=PA + 1), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(struct_size=8)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=9)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(act=5)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(eps=-1.0)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(alpha=float("nan"))), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(residual=PW, ld_residual=8)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(N=70000, ldb=70000, ldc=70000, epi=epi(row_op=2)), cf.CF_ERR_UNSUPPORTED),
    (dict(M=1 << 20, K=4096, lda=4096), cf.CF_ERR_UNSUPPORTED),       # 8 GiB A: beyond 32-bit offsets
    (dict(N=4096, ldb=4096, ldc=4096, epi=epi(row_op=2)), cf.CF_ERR_WORKSPACE),   # needs a workspace
    (dict(N=4096, ldb=4096, ldc=4096, epi=epi(row_op=2), ws=PW + 8, wsb=1 << 22), cf.CF_ERR_WORKSPACE),
    (dict(N=4096, ldb=4096, ldc=4096, epi=epi(row_op=2), ws=PW, wsb=4096), cf.CF_ERR_WORKSPACE),
    (dict(epi=epi(x_out=PW, ld_x_out=8)), cf.CF_ERR_INVALID_ARGUMENT),                  # ld below N
    (dict(epi=epi(x_out=PW + 1, ld_x_out=64)), cf.CF_ERR_INVALID_ARGUMENT),             # misaligned bf16
    (dict(epi=epi(x_out=PW + 2, ld_x_out=64, x_out_dtype=0)), cf.CF_ERR_INVALID_ARGUMENT),   # misaligned f32
    (dict(epi=epi(x_out=PW, ld_x_out=64, x_out_dtype=7)), cf.CF_ERR_INVALID_ARGUMENT),  # bad dtype
    (dict(M=1 << 20, epi=epi(x_out=PW, ld_x_out=1024, x_out_dtype=0)), cf.CF_ERR_UNSUPPORTED),  # 4 GiB X
    (dict(epi=epi(row_op=1, mask=1)), cf.CF_ERR_UNSUPPORTED),        # masks belong to the B2B softmax
    (dict(epi=epi(mask=3)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_stats=PW)), cf.CF_ERR_INVALID_ARGUMENT),        # no row op, no statistics
    (dict(epi=epi(row_op=4)), cf.CF_ERR_INVALID_ARGUMENT),            # argmax needs row_index
    (dict(epi=epi(row_op=4, row_index=PW + 2)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=4, row_index=PW, gamma=PB)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=1, row_index=PW)), cf.CF_ERR_INVALID_ARGUMENT),   # row_index belongs to argmax
    (dict(C=None, epi=epi(row_op=3)), cf.CF_ERR_INVALID_ARGUMENT),    # only argmax may omit C
    (dict(epi=epi(row_op=2, row_stats=PW + 1)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op2=1)), cf.CF_ERR_INVALID_ARGUMENT),           # a second stage needs a first
    (dict(epi=epi(row_op=4, row_index=PW, row_op2=1)), cf.CF_ERR_INVALID_ARGUMENT),   # not after argmax
    (dict(epi=epi(row_op=2, row_op2=4)), cf.CF_ERR_INVALID_ARGUMENT),  # argmax is no second stage
    (dict(epi=epi(row_op=2, row_op2=9)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(gamma2=PB)), cf.CF_ERR_INVALID_ARGUMENT),           # second-stage vectors without it
    (dict(epi=epi(eps2=1e-5)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=2, row_op2=1, beta2=PB)), cf.CF_ERR_INVALID_ARGUMENT),   # beta2 belongs to LayerNorm
    (dict(epi=epi(row_op=2, row_op2=2, eps2=-1.0)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=2, row_op2=2, gamma2=PB + 1)), cf.CF_ERR_INVALID_ARGUMENT),   # misaligned bf16
    (dict(K=60, epi=epi(row_op=2, row_op2=1)), cf.CF_ERR_UNSUPPORTED),   # two stages: fast-path layouts only
    (dict(epi=epi(row_op=5, topk=4)), cf.CF_ERR_INVALID_ARGUMENT),            # top-k needs row_index
    (dict(epi=epi(row_op=5, row_index=PW, topk=0)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=5, row_index=PW, topk=9)), cf.CF_ERR_INVALID_ARGUMENT),   # k <= 8
    (dict(N=4, ldb=4, ldc=4, epi=epi(row_op=5, row_index=PW, topk=5)), cf.CF_ERR_INVALID_ARGUMENT),   # k <= N
    (dict(epi=epi(row_op=5, row_index=PW, topk=4, gamma=PB)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=5, row_index=PW, topk=4, residual=PW, ld_residual=64)), cf.CF_ERR_UNSUPPORTED),
    (dict(K=60, epi=epi(row_op=5, row_index=PW, topk=4)), cf.CF_ERR_UNSUPPORTED),   # fast-path layouts only
    (dict(epi=epi(row_op=2, topk=4)), cf.CF_ERR_INVALID_ARGUMENT),            # topk belongs to CF_ROW_TOPK
    (dict(epi=epi(row_op=6)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(epi=epi(row_op=1, axis=5)), cf.CF_ERR_INVALID_ARGUMENT),     # no such axis
    (dict(epi=epi(axis=1)), cf.CF_ERR_INVALID_ARGUMENT),               # a column axis needs a row op
    (dict(epi=epi(row_op=4, row_index=PW, axis=1)), cf.CF_ERR_UNSUPPORTED),   # argmax over columns
    (dict(epi=epi(row_op=2, row_op2=1, axis=1)), cf.CF_ERR_UNSUPPORTED),      # one column stage
    (dict(K=60, epi=epi(row_op=1, axis=1)), cf.CF_ERR_UNSUPPORTED),   # column reductions: fast path only
    (dict(M=70000, epi=epi(row_op=3, axis=1)), cf.CF_ERR_UNSUPPORTED),   # a tile column of more than 256 tiles
    (dict(M=4096, epi=epi(row_op=2, axis=1)), cf.CF_ERR_WORKSPACE),   # 16 strips exchange: needs a workspace
    (dict(M=0), cf.CF_OK),            # empty problems launch nothing
    (dict(N=0), cf.CF_OK),
])
def test_gemm_epilogue_argument_checks(kw, status):
    assert gemm(**kw) == status


def b2b(batch=1, M=64, K=64, L=64, N=64, A=PA, lda=64, sa=0, B0=PB, ldb0=64, sb0=0, lk=0, B1=PC, ldb1=64,
        sb1=0, O=PW, ldo=64, so=0, it=1, ot=1, mid=None):
    return lib.cf_b2bgemm(batch, M, K, L, N, A, lda, sa, B0, ldb0, sb0, lk, B1, ldb1, sb1, O, ldo, so, it, ot,
                          ctypes.byref(mid) if mid is not None else None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(lk=3), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(B1=None), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(lda=32), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(ldo=8), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(sa=-8), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(it=0), cf.CF_ERR_UNSUPPORTED),                            # fp32 inputs
    (dict(lda=68), cf.CF_ERR_UNSUPPORTED),                          # leading dimension not 16-byte aligned
    (dict(mid=epi(row_op=2)), cf.CF_ERR_UNSUPPORTED),               # LayerNorm between two GEMMs
    (dict(mid=epi(residual=PW, ld_residual=64)), cf.CF_ERR_UNSUPPORTED),
    (dict(mid=epi(x_out=PW, ld_x_out=64)), cf.CF_ERR_UNSUPPORTED),   # S is never stored
    (dict(mid=epi(mask=1)), cf.CF_ERR_UNSUPPORTED),                  # causal needs the softmax
    (dict(mid=epi(row_op=1, bias=PW)), cf.CF_ERR_UNSUPPORTED),       # softmax takes alpha * S as it is
    (dict(mid=epi(row_op=1, act=1)), cf.CF_ERR_UNSUPPORTED),
    (dict(mid=epi(row_stats=PW)), cf.CF_ERR_INVALID_ARGUMENT),       # statistics need a row op
    (dict(mid=epi(row_op=1, row_stats=PW + 2)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(mid=epi(row_op=1, mask=2)), cf.CF_ERR_INVALID_ARGUMENT),
    (dict(mid=epi(row_op=4, row_index=PW)), cf.CF_ERR_UNSUPPORTED),   # argmax between two GEMMs
    (dict(mid=epi(row_op=1, row_op2=2)), cf.CF_ERR_UNSUPPORTED),      # one row stage between two GEMMs
    (dict(mid=epi(row_op=5, row_index=PW, topk=2)), cf.CF_ERR_UNSUPPORTED),   # top-k between two GEMMs
    (dict(mid=epi(row_op=1, axis=1)), cf.CF_ERR_UNSUPPORTED),        # S's columns are never all on chip
    (dict(batch=0), cf.CF_OK),
])
def test_b2bgemm_argument_checks(kw, status):
    assert b2b(**kw) == status


def test_workspace_sizes():
    e = epi(row_op=2)
    assert cf.cf_gemm_epilogue_workspace_size(8192, 4096, 4096, e) == 512 + 32 * 16 * 256 * 16
    assert cf.cf_gemm_epilogue_workspace_size(16384, 4096, 11008, epi(row_op=3)) == 512 + 64 * 16 * 256 * 16
    assert cf.cf_gemm_epilogue_workspace_size(8192, 256, 4096, e) == 0        # one column tile per strip
    assert cf.cf_gemm_epilogue_workspace_size(8192, 4096, 4096, epi()) == 0   # no row op
    # top-k exchanges 8 (value, column) pairs per row
    assert cf.cf_gemm_epilogue_workspace_size(8192, 4096, 4096, epi(row_op=5, row_index=PW, topk=4)) == \
        512 + 32 * 16 * 256 * 16 * 8
    # a column reduction exchanges over the tile columns: the same slots
    assert cf.cf_gemm_epilogue_workspace_size(8192, 4096, 4096, epi(row_op=2, axis=1)) == 512 + 32 * 16 * 256 * 16
    assert cf.cf_gemm_epilogue_workspace_size(256, 4096, 4096, epi(row_op=2, axis=1)) == 0   # one strip
    # a second row stage exchanges through a second set of slots
    assert cf.cf_gemm_epilogue_workspace_size(8192, 4096, 4096, epi(row_op=2, row_op2=1)) == \
        512 + 2 * 32 * 16 * 256 * 16
    assert lib.cf_workspace_init(None, 4096, None) == cf.CF_ERR_WORKSPACE
    assert lib.cf_workspace_init(PW + 16, 4096, None) == cf.CF_ERR_WORKSPACE


@pytest.mark.skipif(gpu_present(), reason="would launch on fake pointers; valid calls are covered by the GPU tests")
def test_valid_calls_report_no_device():
    assert gemm(epi=epi(row_op=1, bias=PW)) == cf.CF_ERR_NO_DEVICE
    assert gemm(epi=epi(row_op=3, x_out=PW, ld_x_out=64)) == cf.CF_ERR_NO_DEVICE
    assert gemm(epi=epi(row_op=1, row_stats=PW)) == cf.CF_ERR_NO_DEVICE
    assert gemm(C=None, ldc=0, epi=epi(row_op=4, row_index=PW)) == cf.CF_ERR_NO_DEVICE
    assert b2b(mid=epi(row_op=1, alpha=0.125)) == cf.CF_ERR_NO_DEVICE
    assert b2b(lk=1, mid=epi(row_op=1, alpha=0.125, mask=1)) == cf.CF_ERR_NO_DEVICE
    assert b2b(K=512, lda=512, ldb0=64) == cf.CF_ERR_NO_DEVICE           # K above 128: k-blocks
    assert b2b(N=200, ldb1=200, ldo=200) == cf.CF_ERR_NO_DEVICE          # N above 128: column blocks
    assert lib.cf_workspace_init(PW, 4096, None) == cf.CF_ERR_NO_DEVICE


def noalloc(M=64, N=64, K=64, A=PA, lda=64, B=PB, ldb=64, nk=0, abt=1, C=PC, ldc=64, ct=1, epi=None):
    return lib.cf_gemm_epilogue_noalloc(M, N, K, A, lda, B, ldb, nk, abt, C, ldc, ct,
                                        ctypes.byref(epi) if epi is not None else None, None)


def test_noalloc_argument_checks():
    # the same checks as cf_gemm_epilogue, before any HIP call
    assert noalloc(M=-1) == cf.CF_ERR_INVALID_ARGUMENT
    assert noalloc(lda=63) == cf.CF_ERR_INVALID_ARGUMENT
    assert noalloc(epi=epi(row_op=9)) == cf.CF_ERR_INVALID_ARGUMENT
    assert noalloc(M=0) == cf.CF_OK
    # beyond the 16 MiB scratch: top-8 over 8192 x 4096 needs 16 MiB of slots + the header
    big = epi(row_op=5, row_index=PW, topk=8)
    assert cf.cf_gemm_epilogue_workspace_size(8192, 4096, 64, big) > (16 << 20)
    assert noalloc(M=8192, N=4096, ldb=4096, C=None, ldc=0, epi=big) == cf.CF_ERR_WORKSPACE
    # C3's RMSNorm exchange (4 MiB) fits
    assert cf.cf_gemm_epilogue_workspace_size(16384, 4096, 64, epi(row_op=3)) <= (16 << 20)


@pytest.mark.skipif(gpu_present(), reason="would launch on fake pointers; valid calls are covered by the GPU tests")
def test_noalloc_valid_call_reports_no_device():
    assert noalloc(N=4096, ldb=4096, ldc=4096, epi=epi(row_op=2)) == cf.CF_ERR_NO_DEVICE
