"""Host-side checks of the C ABI (no GPU): exports, the code table, sizes and argument validation.

Every call here fails validation before the library touches HIP, so fake device
addresses are safe: they are compared and range-checked, never dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4lora.h")

nf4 = pytest.importorskip("quantized_lora_fine_amd", reason="libnf4lora.so not built")
lib = nf4._lib


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b((?:nf4|bf16lora)\w*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_match_header():
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(nf4.EXPORTS) == names


def test_abi_version_and_status_strings():
    assert nf4.abi_version() == 5
    for s in range(9):
        assert nf4.status_str(s) and "unknown" not in nf4.status_str(s)
    assert "NONFINITE" in nf4.status_str(nf4.NF4_ERR_NONFINITE)
    assert "unknown" in nf4.status_str(99)


def test_code_table_bit_exact():
    lib_t = nf4.code_table().numpy().astype(np.float32)
    assert np.array_equal(lib_t.view(np.uint32), oracle.nf4_table().view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(1, 64), (512, 512), (4096, 4096), (11008, 4096), (28672, 8192),
                                       (3, 192), (65_000_000_000 // 64, 64)])
@pytest.mark.parametrize("dq", [0, 256])
def test_tensor_bytes(rows, cols, dq):
    assert nf4.tensor_bytes(rows, cols, dq) == oracle.storage_bytes(rows, cols, 64, dq)


def test_protect_count():
    assert nf4.protect_count(0.2, 144) == 29
    assert nf4.protect_count(0.2, 280) == 56
    assert nf4.protect_count(0.0, 10) == 0
    assert nf4.protect_count(1.5, 10) == -1


def test_workspace_sizes():
    for op in (nf4.NF4_OP_FWD, nf4.NF4_OP_BWD):
        a = nf4.workspace_bytes(op, 2048, 4096, 4096, 16)
        b = nf4.workspace_bytes(op, 4096, 4096, 4096, 16)
        assert 0 < a < b
        assert a % 256 == 0
    assert nf4.workspace_bytes(nf4.NF4_OP_ERROR, 0, 4096, 4096, 1) >= 16 * 1024
    with pytest.raises(nf4.NF4Error):
        nf4.workspace_bytes(9, 1, 64, 64, 1)
    with pytest.raises(nf4.NF4Error):
        nf4.workspace_bytes(nf4.NF4_OP_FWD, 1, 64, 64, 0)


# ---------------------------------------------------------------------------
# validation (fake device addresses; every call is rejected before any launch)
# ---------------------------------------------------------------------------
A = 0x10000000          # aligned fake addresses, far apart
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000
F = 0x60000000
G = 0x70000000
H = 0x80000000


def desc(rows=64, cols=64, block=64, dq=0, codes=A, absmax=B, dqs=None):
    return nf4._NF4Tensor(rows, cols, block, dq, codes, absmax, dqs)


def st_quant(d, W=C):
    return lib.nf4_quantize(ctypes.c_void_p(W), ctypes.byref(d) if d is not None else None, None)


def test_quantize_validation():
    assert st_quant(None) == nf4.NF4_ERR_NULL
    assert st_quant(desc(block=32)) == nf4.NF4_ERR_ARG
    assert st_quant(desc(dq=128, dqs=D)) == nf4.NF4_ERR_ARG
    assert st_quant(desc(cols=100)) == nf4.NF4_ERR_SHAPE
    assert st_quant(desc(rows=-1)) == nf4.NF4_ERR_SHAPE
    assert st_quant(desc(codes=None)) == nf4.NF4_ERR_NULL
    assert st_quant(desc(dq=256, dqs=None)) == nf4.NF4_ERR_NULL
    assert st_quant(desc(), W=0) == nf4.NF4_ERR_NULL
    assert st_quant(desc(codes=A + 8)) == nf4.NF4_ERR_ALIGN
    assert st_quant(desc(), W=C + 4) == nf4.NF4_ERR_ALIGN
    assert st_quant(desc(dq=256, dqs=D + 2)) == nf4.NF4_ERR_ALIGN
    # codes inside the input weight
    assert st_quant(desc(codes=C + 64)) == nf4.NF4_ERR_ALIAS
    assert st_quant(desc(absmax=A + 16)) == nf4.NF4_ERR_ALIAS
    # empty tensors are accepted without touching the device
    assert st_quant(desc(rows=0)) == nf4.NF4_OK


def test_dequantize_validation():
    d = desc()
    assert lib.nf4_dequantize(ctypes.byref(d), None, 0, None) == nf4.NF4_ERR_NULL
    assert lib.nf4_dequantize(ctypes.byref(d), ctypes.c_void_p(C + 8), 0, None) == nf4.NF4_ERR_ALIGN
    assert lib.nf4_dequantize(ctypes.byref(d), ctypes.c_void_p(A), 1, None) == nf4.NF4_ERR_ALIAS
    assert lib.nf4_dequantize(ctypes.byref(desc(block=128)), ctypes.c_void_p(C), 0, None) == nf4.NF4_ERR_ARG


def fwd_call(d, X=C, M=16, L1=D, L2=E, r=8, Y=F, T=G, ws=H, ws_bytes=1 << 30):
    return lib.nf4lora_fwd(ctypes.byref(d) if d is not None else None, ctypes.c_void_p(X), M, ctypes.c_void_p(L1),
                           ctypes.c_void_p(L2), r, 2.0, ctypes.c_void_p(Y), ctypes.c_void_p(T) if T else None,
                           ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_fwd_validation():
    d = desc(rows=128, cols=128)
    assert fwd_call(None) == nf4.NF4_ERR_NULL
    assert fwd_call(desc(rows=100, cols=128)) == nf4.NF4_ERR_SHAPE     # rows % 64
    assert fwd_call(d, r=0) == nf4.NF4_ERR_SHAPE
    assert fwd_call(d, r=257) == nf4.NF4_ERR_SHAPE
    assert fwd_call(d, M=-1) == nf4.NF4_ERR_SHAPE
    assert fwd_call(d, X=0) == nf4.NF4_ERR_NULL
    assert fwd_call(d, Y=0) == nf4.NF4_ERR_NULL
    assert fwd_call(d, X=C + 2) == nf4.NF4_ERR_ALIGN
    assert fwd_call(d, T=G + 8) == nf4.NF4_ERR_ALIGN
    assert fwd_call(d, ws=0) == nf4.NF4_ERR_WORKSPACE
    need = nf4.workspace_bytes(nf4.NF4_OP_FWD, 16, 128, 128, 8)
    assert fwd_call(d, ws_bytes=need - 1) == nf4.NF4_ERR_WORKSPACE
    assert fwd_call(d, Y=C) == nf4.NF4_ERR_ALIAS                          # Y == X
    assert fwd_call(d, T=F + 64) == nf4.NF4_ERR_ALIAS                     # T inside Y
    assert fwd_call(d, ws=A) == nf4.NF4_ERR_ALIAS                         # workspace over the codes
    assert fwd_call(d, M=0) == nf4.NF4_OK                                 # empty batch: nothing to do
    # weights beyond the fused kernels' 32-bit buffer ranges are rejected before any launch
    assert fwd_call(desc(rows=(1 << 22) + 64, cols=128)) == nf4.NF4_ERR_SHAPE
    assert fwd_call(desc(rows=128, cols=(1 << 22) + 64)) == nf4.NF4_ERR_SHAPE
    assert fwd_call(desc(rows=1 << 22, cols=(1 << 10) + 64)) == nf4.NF4_ERR_SHAPE   # rows * cols > 2^32
    big = desc(rows=(1 << 22) + 64, cols=128)
    assert lib.nf4_matmul(ctypes.byref(big), 0, ctypes.c_void_p(C), 16, None, None, 0, ctypes.c_void_p(F),
                          None) == nf4.NF4_ERR_SHAPE


def bwd_call(d, X=C, dY=D, M=16, L1=E, L2=F, r=8, T=None, dX=G, dL1=H, dL2=H + 0x1000000, ws=H + 0x2000000,
             ws_bytes=1 << 30):
    v = lambda p: ctypes.c_void_p(p) if p else None
    return lib.nf4lora_bwd(ctypes.byref(d), v(X), v(dY), M, v(L1), v(L2), r, 2.0, v(T), v(dX), v(dL1), v(dL2),
                           v(ws), ws_bytes, None)


def test_bwd_validation():
    d = desc(rows=128, cols=128)
    assert bwd_call(d, dL1=0) == nf4.NF4_ERR_NULL
    assert bwd_call(d, dY=0) == nf4.NF4_ERR_NULL
    assert bwd_call(d, dL2=H + 0x1000004) == nf4.NF4_ERR_ALIGN
    assert bwd_call(d, ws_bytes=16) == nf4.NF4_ERR_WORKSPACE
    assert bwd_call(d, dX=C) == nf4.NF4_ERR_ALIAS
    assert bwd_call(d, dL1=E) == nf4.NF4_ERR_ALIAS
    assert bwd_call(d, T=G) == nf4.NF4_ERR_ALIAS                          # T overlaps dX
    assert bwd_call(desc(rows=128, cols=96)) == nf4.NF4_ERR_SHAPE


def bf16_fwd_call(W=A, rows=128, cols=128, X=C, M=16, Y=F, ws=H, ws_bytes=1 << 30):
    v = lambda p: ctypes.c_void_p(p) if p else None
    return lib.bf16lora_fwd(v(W), rows, cols, v(X), M, v(D), v(E), 8, 2.0, v(Y), v(G), v(ws), ws_bytes, None)


def bf16_bwd_call(W=A, rows=128, cols=128, dX=G, dL1=H, ws_bytes=1 << 30):
    v = lambda p: ctypes.c_void_p(p) if p else None
    return lib.bf16lora_bwd(v(W), rows, cols, v(C), v(D), 16, v(E), v(F), 8, 2.0, None, v(dX), v(dL1),
                            v(H + 0x1000000), v(H + 0x2000000), ws_bytes, None)


def test_bf16_layer_validation():
    assert bf16_fwd_call(W=0) == nf4.NF4_ERR_NULL
    assert bf16_fwd_call(W=A + 2) == nf4.NF4_ERR_ALIGN
    assert bf16_fwd_call(rows=100) == nf4.NF4_ERR_SHAPE
    assert bf16_fwd_call(cols=96) == nf4.NF4_ERR_SHAPE
    assert bf16_fwd_call(rows=1 << 16, cols=1 << 16) == nf4.NF4_ERR_SHAPE   # 2^32 elements: too large
    assert bf16_fwd_call(ws=0) == nf4.NF4_ERR_WORKSPACE
    assert bf16_fwd_call(Y=A + 64) == nf4.NF4_ERR_ALIAS                  # Y inside W
    assert bf16_fwd_call(M=0) == nf4.NF4_OK
    assert bf16_bwd_call(dL1=0) == nf4.NF4_ERR_NULL
    assert bf16_bwd_call(dX=A) == nf4.NF4_ERR_ALIAS                      # dX over W
    assert bf16_bwd_call(ws_bytes=16) == nf4.NF4_ERR_WORKSPACE


def test_error_and_topk_validation():
    v = ctypes.c_void_p
    assert lib.nf4_layer_error(v(C), 64, 64, 64, 0, 0, None, v(D), 1 << 20, None) == nf4.NF4_ERR_NULL
    assert lib.nf4_layer_error(v(C), 64, 65, 64, 0, 0, v(E), v(D), 1 << 20, None) == nf4.NF4_ERR_SHAPE
    assert lib.nf4_layer_error(v(C), 64, 64, 64, 7, 0, v(E), v(D), 1 << 20, None) == nf4.NF4_ERR_ARG
    assert lib.nf4_layer_error(v(C), 64, 64, 64, 0, 0, v(E), None, 0, None) == nf4.NF4_ERR_WORKSPACE
    assert lib.nf4_layer_error(v(C), 64, 64, 64, 0, 0, v(E), v(D), 8, None) == nf4.NF4_ERR_WORKSPACE
    assert lib.nf4_layer_error(v(C), 64, 64, 64, 0, 0, v(C + 16), v(D), 1 << 20, None) == nf4.NF4_ERR_ALIAS
    assert lib.nf4_layer_error(v(C), 64, 64, 64, 0, 3, v(E), v(D), 1 << 20, None) == nf4.NF4_ERR_ARG  # codebook
    assert lib.nf4_topk(v(C), 10, 11, v(D), None) == nf4.NF4_ERR_SHAPE
    assert lib.nf4_topk(v(C), 10, 3, None, None) == nf4.NF4_ERR_NULL
    assert lib.nf4_topk(v(C), 10, 3, v(C + 16), None) == nf4.NF4_ERR_ALIAS
    assert lib.nf4_topk(v(C), 10, 0, None, None) == nf4.NF4_OK


def test_quantize_error_validation():
    v = ctypes.c_void_p

    def call(d, W=C, edq=0, err=E, ws=D, wsb=1 << 20):
        return lib.nf4_quantize_error(v(W), ctypes.byref(d) if d is not None else None, edq, v(err), v(ws), wsb,
                                      None)

    assert call(None) == nf4.NF4_ERR_NULL
    assert call(desc(cols=100)) == nf4.NF4_ERR_SHAPE
    assert call(desc(), edq=256) == nf4.NF4_ERR_ARG                      # no double quant to measure with
    assert call(desc(dq=256, dqs=F), edq=128) == nf4.NF4_ERR_ARG
    d = desc(rows=128, cols=128)
    r = desc(rows=128, cols=128, codes=G, absmax=H)
    d.residual = ctypes.pointer(r)
    assert call(d) == nf4.NF4_ERR_ARG                                    # one stage only
    assert call(desc(), err=0) == nf4.NF4_ERR_NULL
    assert call(desc(), W=0) == nf4.NF4_ERR_NULL
    assert call(desc(), ws=0, wsb=0) == nf4.NF4_ERR_WORKSPACE
    assert call(desc(), wsb=8) == nf4.NF4_ERR_WORKSPACE
    assert call(desc(), W=C + 4) == nf4.NF4_ERR_ALIGN
    assert call(desc(), err=E + 8) == nf4.NF4_ERR_ALIGN
    assert call(desc(), err=C + 16) == nf4.NF4_ERR_ALIAS                 # err inside W
    assert call(desc(), ws=A) == nf4.NF4_ERR_ALIAS                       # workspace over the codes
    assert call(desc(), err=D + 16) == nf4.NF4_ERR_ALIAS                 # err inside the workspace
    assert call(desc(codes=C + 64)) == nf4.NF4_ERR_ALIAS


def test_error_batch_validation():
    v = ctypes.c_void_p
    I64 = ctypes.c_int64

    def arrs(shapes, ptrs):
        n = len(shapes)
        return ((v * max(n, 1))(*ptrs), (I64 * max(n, 1))(*[r for r, _ in shapes]),
                (I64 * max(n, 1))(*[c for _, c in shapes]))

    def call(shapes, ptrs, n=None, dq=0, cb=0, err=E, ws=D, wsb=1 << 20):
        W, R, K = arrs(shapes, ptrs)
        return lib.nf4_layer_error_batch(W, R, K, len(shapes) if n is None else n, dq, cb, v(err), v(ws), wsb, None)

    def wsb(shapes):
        _, R, K = arrs(shapes, [0] * len(shapes))
        b = ctypes.c_size_t()
        st = lib.nf4_error_batch_workspace_bytes(R, K, len(shapes), ctypes.byref(b))
        return st, b.value

    two = [(128, 128), (64, 4096)]
    # 128*128/64 = 256 blocks = 1 group; 64*4096/64 = 4096 blocks = 16 groups: 17 slots of 16 bytes
    assert wsb(two) == (nf4.NF4_OK, 512)
    assert wsb([(128, 100)])[0] == nf4.NF4_ERR_SHAPE
    assert lib.nf4_error_batch_workspace_bytes(None, None, 1, ctypes.byref(ctypes.c_size_t())) == nf4.NF4_ERR_NULL
    assert lib.nf4_error_batch_workspace_bytes(None, None, 0, None) == nf4.NF4_ERR_NULL
    assert call([], [], n=0) == nf4.NF4_OK                                 # nothing to do
    assert call(two, [A, B], n=-1) == nf4.NF4_ERR_ARG
    assert call(two, [A, B], dq=128) == nf4.NF4_ERR_ARG
    assert call(two, [A, B], cb=7) == nf4.NF4_ERR_ARG
    assert call([(128, 128), (64, 100)], [A, B]) == nf4.NF4_ERR_SHAPE
    assert call(two, [A, 0]) == nf4.NF4_ERR_NULL                           # a non-empty linear without W
    assert call(two, [A, B], err=0) == nf4.NF4_ERR_NULL
    assert call(two, [A, B], ws=0, wsb=0) == nf4.NF4_ERR_WORKSPACE
    assert call(two, [A, B], wsb=511) == nf4.NF4_ERR_WORKSPACE
    assert call(two, [A, B + 4]) == nf4.NF4_ERR_ALIGN
    assert call(two, [A, B], ws=D + 8) == nf4.NF4_ERR_ALIGN
    assert call(two, [A, B], err=E + 4) == nf4.NF4_ERR_ALIGN
    assert call(two, [A, B], err=B + 64) == nf4.NF4_ERR_ALIAS              # err inside W[1]
    assert call(two, [A, B], ws=A + 256) == nf4.NF4_ERR_ALIAS              # workspace inside W[0]
    assert call(two, [A, B], err=D + 8) == nf4.NF4_ERR_ALIAS               # err inside the workspace


def test_stack_validation():
    v = ctypes.c_void_p
    d = desc(rows=128, cols=128)
    L = (nf4._NF4Linear * 2)()
    L[0].q = ctypes.pointer(d)
    L[0].r = 8
    L[1].w_bf16, L[1].rows, L[1].cols, L[1].r = v(C), 128, 128, 0
    n = ctypes.c_size_t()
    assert lib.nf4_stack_workspace_bytes(L, 2, 16, ctypes.byref(n)) == nf4.NF4_OK
    assert n.value == max(nf4.workspace_bytes(nf4.NF4_OP_FWD, 16, 128, 128, 8),
                          nf4.workspace_bytes(nf4.NF4_OP_BWD, 16, 128, 128, 8))
    assert lib.nf4_stack_workspace_bytes(L, 2, 16, None) == nf4.NF4_ERR_NULL
    assert lib.nf4_stack_bwd(L, 2, 3, 16, v(H), 1 << 30, None) == nf4.NF4_ERR_SHAPE    # cut > n
    assert lib.nf4_stack_bwd(L, 2, -1, 16, v(H), 1 << 30, None) == nf4.NF4_ERR_SHAPE
    assert lib.nf4_stack_bwd(L, 2, 2, 16, v(H), 1 << 30, None) == nf4.NF4_OK           # cut == n: nothing runs
    L[1].q = ctypes.pointer(d)                                                          # both weights set
    assert lib.nf4_stack_workspace_bytes(L, 2, 16, ctypes.byref(n)) == nf4.NF4_ERR_ARG
    L[1].q = None
    L[1].w_bf16 = None                                                                  # no weight
    assert lib.nf4_stack_fwd(L, 2, 16, v(H), 1 << 30, None) != nf4.NF4_OK
    assert lib.nf4_stack_fwd(None, 1, 16, v(H), 1 << 30, None) == nf4.NF4_ERR_NULL


def test_merge_validation():
    v = ctypes.c_void_p
    d = desc(rows=128, cols=128)
    m = lambda W=C, q=None, rows=128, cols=128, L1=D, L2=E, r=8, out=F, bf=0: lib.nf4lora_merge(
        v(W) if W else None, ctypes.byref(q) if q is not None else None, rows, cols, v(L1) if L1 else None,
        v(L2) if L2 else None, r, 2.0, v(out) if out else None, bf, None)
    assert m(W=None) == nf4.NF4_ERR_NULL                        # neither base
    assert m(cols=100) == nf4.NF4_ERR_SHAPE
    assert m(r=0) == nf4.NF4_ERR_SHAPE
    assert m(W=None, q=d, rows=64) == nf4.NF4_ERR_SHAPE          # q shape differs
    assert m(L1=None) == nf4.NF4_ERR_NULL
    assert m(out=F + 8) == nf4.NF4_ERR_ALIGN
    assert m(out=C + 64) == nf4.NF4_ERR_ALIAS                    # output inside W
    assert m(W=None, q=d, out=A) == nf4.NF4_ERR_ALIAS            # output over the codes
    assert m(rows=0) == nf4.NF4_OK


def test_codebook_values_match_oracle():
    for name in ("nf4", "int4", "fp4"):
        got = nf4.codebook_values(name).numpy()
        assert np.array_equal(got.view(np.uint32), oracle.codebook_table(name).view(np.uint32)), name
    out = (ctypes.c_float * 16)()
    assert lib.nf4_codebook_values(3, out) == nf4.NF4_ERR_ARG
    assert lib.nf4_codebook_values(0, None) == nf4.NF4_ERR_NULL
    # a descriptor naming an unknown codebook is rejected
    d = desc()
    d.codebook = 5
    assert st_quant(d) == nf4.NF4_ERR_ARG



def test_residual_validation():
    d = desc(rows=128, cols=128)
    r = desc(rows=128, cols=128, codes=E, absmax=F)
    d.residual = ctypes.pointer(r)
    bad = desc(rows=64, cols=128, codes=E, absmax=F)
    d.residual = ctypes.pointer(bad)
    assert st_quant(d) == nf4.NF4_ERR_SHAPE                      # residual shape differs
    other = desc(rows=128, cols=128, dq=256, codes=E, absmax=F, dqs=G)
    d.residual = ctypes.pointer(other)
    assert st_quant(d) == nf4.NF4_ERR_SHAPE                      # residual double quant differs
    nested = desc(rows=128, cols=128, codes=E, absmax=F)
    nested.residual = ctypes.pointer(desc(rows=128, cols=128, codes=G, absmax=H))
    d.residual = ctypes.pointer(nested)
    assert st_quant(d) == nf4.NF4_ERR_ARG                        # no residual of a residual
    alias = desc(rows=128, cols=128, codes=A + 64, absmax=F)
    d.residual = ctypes.pointer(alias)
    assert st_quant(d) == nf4.NF4_ERR_ALIAS                      # residual codes inside the first codes
    noptr = desc(rows=128, cols=128, codes=None, absmax=F)
    d.residual = ctypes.pointer(noptr)
    assert st_quant(d) == nf4.NF4_ERR_NULL


def test_check_finite_validation():
    v = ctypes.c_void_p
    ws = nf4.workspace_bytes(nf4.NF4_OP_CHECK, 0, 0, 0, 0)
    assert ws >= 4
    assert lib.nf4_check_finite(v(C), 0, None, 0, None) == nf4.NF4_OK           # nothing to scan
    assert lib.nf4_check_finite(v(C), -1, v(D), ws, None) == nf4.NF4_ERR_SHAPE
    assert lib.nf4_check_finite(None, 16, v(D), ws, None) == nf4.NF4_ERR_NULL
    assert lib.nf4_check_finite(v(C), 16, None, ws, None) == nf4.NF4_ERR_WORKSPACE
    assert lib.nf4_check_finite(v(C), 16, v(D), ws - 1, None) == nf4.NF4_ERR_WORKSPACE
    assert lib.nf4_check_finite(v(C + 4), 16, v(D), ws, None) == nf4.NF4_ERR_ALIGN
    assert lib.nf4_check_finite(v(C), 16, v(C + 32), ws, None) == nf4.NF4_ERR_ALIAS


def test_pass_size_bound():
    """The passes over W accept at most (2^24 - 1) groups of 16384 weights (one launch stays below 2^32
    work-items); storage sizes are still reported beyond that."""
    v = ctypes.c_void_p
    big_rows = (1 << 24) * 256      # x 64 columns = 2^24 groups: one past the bound
    ok_rows = ((1 << 24) - 1) * 256
    assert nf4.tensor_bytes(big_rows, 64, 0)[0] == big_rows * 32
    assert st_quant(desc(rows=big_rows)) == nf4.NF4_ERR_SHAPE
    assert lib.nf4_layer_error(v(C), big_rows, 64, 64, 0, 0, v(E), v(D), 1 << 40, None) == nf4.NF4_ERR_SHAPE
    # one group fewer passes the size check and fails later on the workspace size
    assert lib.nf4_layer_error(v(C), ok_rows, 64, 64, 0, 0, v(E), v(D), 16, None) == nf4.NF4_ERR_WORKSPACE
    rows = (ctypes.c_int64 * 1)(big_rows)
    cols = (ctypes.c_int64 * 1)(64)
    b = ctypes.c_size_t()
    assert lib.nf4_error_batch_workspace_bytes(rows, cols, 1, ctypes.byref(b)) == nf4.NF4_ERR_SHAPE


def test_fwd_noalloc_validation():
    """The allocation-free forward validates like nf4lora_fwd and rejects, before any HIP call, a layer
    whose workspace exceeds its fixed 16 MiB area."""
    v = ctypes.c_void_p

    def call(d, X=C, M=16, L1=D, L2=E, r=8, Y=F, T=G):
        return lib.nf4lora_fwd_noalloc(ctypes.byref(d), v(X), M, v(L1), v(L2), r, 2.0, v(Y),
                                       v(T) if T else None, None)
    assert call(desc(rows=128, cols=128), r=0) == nf4.NF4_ERR_SHAPE
    assert call(desc(rows=100, cols=128)) == nf4.NF4_ERR_SHAPE
    assert call(desc(rows=128, cols=128), M=-1) == nf4.NF4_ERR_SHAPE
    assert call(desc(rows=128, cols=128), M=0) == nf4.NF4_OK
    big = desc(rows=28672, cols=8192, dq=256, dqs=D)
    assert nf4.workspace_bytes(nf4.NF4_OP_FWD, 16384, 28672, 8192, 256) > 16 << 20
    assert call(big, M=16384, r=256) == nf4.NF4_ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    """The binding checks device, dtype, shape and layout before it hands a pointer to the library."""
    import torch
    with pytest.raises(ValueError, match="cuda"):
        nf4._need(torch.zeros(4, 4), torch.float32, (4, 4), "W")
    with pytest.raises(ValueError, match="expected a tensor"):
        nf4._need(None, torch.float32, None, "W")
