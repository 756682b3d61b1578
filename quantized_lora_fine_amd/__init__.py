"""Python binding of libnf4lora (the NF4-LoRA linear layer on MI355X).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current stream; tensors are
passed as raw device pointers.  There is no fallback: if the shared library
is missing this module raises on import, and every call checks the status
the library returns.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# NF4LORA_LIB selects another build of the same library (e.g. a debug build)
LIB_PATH = os.environ.get("NF4LORA_LIB") or os.path.join(_HERE, "libnf4lora.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libnf4lora.so not found at {LIB_PATH}; build it with `python quantized_lora_fine_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

(NF4_OK, NF4_ERR_NULL, NF4_ERR_SHAPE, NF4_ERR_ALIGN, NF4_ERR_WORKSPACE, NF4_ERR_ALIAS, NF4_ERR_HIP, NF4_ERR_ARG,
 NF4_ERR_NONFINITE) = range(9)
NF4_OP_FWD, NF4_OP_BWD, NF4_OP_ERROR, NF4_OP_CHECK = 1, 2, 3, 4
CODEBOOKS = {"nf4": 0, "int4": 1, "fp4": 2}
BLOCK = 64
DQ_GROUP = 256


class _NF4Tensor(ctypes.Structure):
    pass


_NF4Tensor._fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("block", ctypes.c_int32),
                       ("dq_group", ctypes.c_int32), ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                       ("dq_scale", ctypes.c_void_p), ("codebook", ctypes.c_int32),
                       ("residual", ctypes.POINTER(_NF4Tensor))]


class _NF4Linear(ctypes.Structure):
    _fields_ = [("q", ctypes.POINTER(_NF4Tensor)), ("w_bf16", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("r", ctypes.c_int32), ("s", ctypes.c_float), ("L1", ctypes.c_void_p),
                ("L2", ctypes.c_void_p), ("X", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("T", ctypes.c_void_p),
                ("dY", ctypes.c_void_p), ("dX", ctypes.c_void_p), ("dL1", ctypes.c_void_p),
                ("dL2", ctypes.c_void_p)]


_vp, _i64, _i32, _sz, _f32, _f64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                                    ctypes.c_float, ctypes.c_double)
_T = ctypes.POINTER(_NF4Tensor)
_LP = ctypes.POINTER(_NF4Linear)
_SIGS = {
    "nf4_abi_version": ([], ctypes.c_int),
    "nf4_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "nf4_code_table": ([ctypes.POINTER(ctypes.c_float)], None),
    "nf4_tensor_bytes": ([_i64, _i64, _i32, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
                         ctypes.c_int),
    "nf4_quantize": ([_vp, _T, _vp], ctypes.c_int),
    "nf4_dequantize": ([_T, _vp, _i32, _vp], ctypes.c_int),
    "nf4_workspace_bytes": ([_i32, _i64, _i64, _i64, _i32, ctypes.POINTER(_sz)], ctypes.c_int),
    "nf4lora_fwd": ([_T, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "nf4lora_fwd_noalloc": ([_T, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp], ctypes.c_int),
    "nf4lora_bwd": ([_T, _vp, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "bf16lora_fwd": ([_vp, _i64, _i64, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "bf16lora_bwd": ([_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                     ctypes.c_int),
    "nf4_matmul": ([_T, _i32, _vp, _i64, _vp, _vp, _i32, _vp, _vp], ctypes.c_int),
    "nf4_layer_error": ([_vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "nf4_quantize_error": ([_vp, _T, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "nf4_layer_error_batch": ([ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, _i32, _i32,
                               _vp, _vp, _sz, _vp], ctypes.c_int),
    "nf4_error_batch_workspace_bytes": ([ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, ctypes.POINTER(_sz)],
                                        ctypes.c_int),
    "nf4_codebook_values": ([_i32, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
    "nf4_topk": ([_vp, _i32, _i32, _vp, _vp], ctypes.c_int),
    "nf4_check_finite": ([_vp, _i64, _vp, _sz, _vp], ctypes.c_int),
    "nf4_probe_mfma_peak": ([_i32, _i32, _vp, _vp], ctypes.c_int),
    "nf4_protect_count": ([_f64, _i32], _i32),
    "nf4lora_merge": ([_vp, _T, _i64, _i64, _vp, _vp, _i32, _f32, _vp, _i32, _vp], ctypes.c_int),
    "nf4_stack_workspace_bytes": ([_LP, _i32, _i64, ctypes.POINTER(_sz)], ctypes.c_int),
    "nf4_stack_fwd": ([_LP, _i32, _i64, _vp, _sz, _vp], ctypes.c_int),
    "nf4_stack_bwd": ([_LP, _i32, _i32, _i64, _vp, _sz, _vp], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTS = tuple(_SIGS)


class NF4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


def _check(status: int, where: str):
    if status != NF4_OK:
        raise NF4Error(status, where)


def abi_version() -> int:
    return _lib.nf4_abi_version()


def status_str(status: int) -> str:
    return _lib.nf4_status_str(int(status)).decode()


def code_table() -> torch.Tensor:
    out = (ctypes.c_float * 16)()
    _lib.nf4_code_table(out)
    return torch.tensor(list(out), dtype=torch.float32)


def codebook_values(codebook: str = "nf4") -> torch.Tensor:
    """nf4_codebook_values: the 16 code values of a codebook (CPU fp32)."""
    out = (ctypes.c_float * 16)()
    _check(_lib.nf4_codebook_values(CODEBOOKS[codebook], out), "nf4_codebook_values")
    return torch.tensor(list(out), dtype=torch.float32)


def tensor_bytes(rows: int, cols: int, dq_group: int = 0, block: int = BLOCK):
    c, a, d = _sz(), _sz(), _sz()
    _check(_lib.nf4_tensor_bytes(rows, cols, block, dq_group, ctypes.byref(c), ctypes.byref(a), ctypes.byref(d)),
           "nf4_tensor_bytes")
    return c.value, a.value, d.value


def workspace_bytes(op: int, M: int, rows: int, cols: int, r: int) -> int:
    b = _sz()
    _check(_lib.nf4_workspace_bytes(op, M, rows, cols, r, ctypes.byref(b)), "nf4_workspace_bytes")
    return b.value


def protect_count(rho: float, n: int) -> int:
    return int(_lib.nf4_protect_count(float(rho), int(n)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape, name: str):
    """t itself when it is a contiguous tensor of `dtype` on the current cuda device with the given shape
    (entries None are free; shape None: any); else ValueError.  The library sees raw pointers only, so every
    size it reads or writes through them is checked here, before any launch."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor, got {type(t).__name__}")
    if not t.is_cuda or t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: expected a tensor on the current cuda device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and (t.dim() != len(shape) or any(w is not None and n != w for n, w in zip(t.shape, shape))):
        raise ValueError(f"{name}: expected shape {tuple('*' if w is None else w for w in shape)}, "
                         f"got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t


def _need_vec(t, dtype, n: int, name: str):
    """A contiguous 1-D tensor of `dtype` with at least n entries (the library writes the first n)."""
    _need(t, dtype, (None,), name)
    if t.numel() < n:
        raise ValueError(f"{name}: expected at least {n} entries, got {t.numel()}")
    return t


def _need_ws(ws, name: str = "ws"):
    return _need(ws, torch.uint8, None, name)


def _need_q(q, rows: int | None = None, cols: int | None = None, name: str = "q"):
    if not isinstance(q, NF4Weight):
        raise ValueError(f"{name}: expected an NF4Weight, got {type(q).__name__}")
    if (rows is not None and q.rows != rows) or (cols is not None and q.cols != cols):
        raise ValueError(f"{name}: expected a [{rows}][{cols}] weight, got [{q.rows}][{q.cols}]")
    return q


class NF4Weight:
    """A quantized weight: the three device buffers plus the C descriptor."""

    def __init__(self, rows: int, cols: int, dq_group: int = 0, device="cuda", codebook: str = "nf4",
                 residual: bool = False):
        cb, ab, db = tensor_bytes(rows, cols, dq_group)
        self.rows, self.cols, self.dq_group, self.codebook = rows, cols, dq_group, codebook
        self.codes = torch.empty(max(cb, 1), dtype=torch.uint8, device=device)
        self.absmax = torch.empty(max(ab, 1), dtype=torch.uint8, device=device)
        self.dq_scale = torch.empty(max(db, 1), dtype=torch.uint8, device=device) if dq_group else None
        self.desc = _NF4Tensor(rows, cols, BLOCK, dq_group, self.codes.data_ptr(), self.absmax.data_ptr(),
                               self.dq_scale.data_ptr() if dq_group else None, CODEBOOKS[codebook])
        self._cb, self._ab, self._db = cb, ab, db
        # the second quantization stage (quantized residual of this one), when requested
        self.residual = NF4Weight(rows, cols, dq_group, device, codebook) if residual else None
        if self.residual is not None:
            self.desc.residual = ctypes.pointer(self.residual.desc)

    @property
    def absmax_f32(self) -> torch.Tensor:
        return self.absmax[:self._ab].view(torch.float32)

    @property
    def c8(self) -> torch.Tensor:
        return self.absmax[:self._ab]

    @property
    def dq_step(self) -> torch.Tensor:
        return self.dq_scale[:self._db].view(torch.float32)

    @property
    def packed_codes(self) -> torch.Tensor:
        return self.codes[:self._cb]


def quantize(W: torch.Tensor, dq_group: int = 0, out: NF4Weight | None = None, codebook: str = "nf4",
             residual: bool = False) -> NF4Weight:
    """nf4_quantize of a cuda fp32 [rows][cols] tensor (into `out` when given; its codebook and residual stage
    then apply).  residual=True also quantizes what the first stage misses into q.residual."""
    _need(W, torch.float32, (None, None), "W")
    q = _need_q(out, *W.shape, "out") if out is not None else NF4Weight(W.shape[0], W.shape[1], dq_group, W.device,
                                                                        codebook, residual)
    _check(_lib.nf4_quantize(_ptr(W), ctypes.byref(q.desc), _stream()), "nf4_quantize")
    return q


def dequantize(q: NF4Weight, bf16: bool = False, out: torch.Tensor | None = None) -> torch.Tensor:
    """nf4_dequantize into fp32 (or bf16) [rows][cols], into `out` when given."""
    if out is None:
        out = torch.empty(q.rows, q.cols, dtype=torch.bfloat16 if bf16 else torch.float32, device=q.codes.device)
    _need_q(q)
    _need(out, torch.bfloat16 if bf16 else torch.float32, (q.rows, q.cols), "out")
    _check(_lib.nf4_dequantize(ctypes.byref(q.desc), _ptr(out), 1 if bf16 else 0, _stream()), "nf4_dequantize")
    return out


def workspace(op: int, M: int, q: NF4Weight, r: int) -> torch.Tensor:
    n = workspace_bytes(op, M, q.rows, q.cols, r)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.codes.device)


def _fwd_args(o: int, h: int, X, L1, L2, want_T: bool, out, T_out):
    """Checks the forward's tensors against W [o][h]; returns (M, r, Y, T), allocating the outputs not given."""
    M = _need(X, torch.bfloat16, (None, h), "X").shape[0]
    r = _need(L1, torch.bfloat16, (h, None), "L1").shape[1]
    _need(L2, torch.bfloat16, (r, o), "L2")
    Y = _need(out, torch.bfloat16, (M, o), "out") if out is not None else \
        torch.empty(M, o, dtype=torch.bfloat16, device=X.device)
    if T_out is not None:
        T = _need(T_out, torch.bfloat16, (M, r), "T_out")
    else:
        T = torch.empty(M, r, dtype=torch.bfloat16, device=X.device) if want_T else None
    return M, r, Y, T


def _bwd_args(o: int, h: int, X, dY, L1, L2, T, want_dX: bool, outs):
    """Checks the backward's tensors against W [o][h]; returns (M, r, dX, dL1, dL2), allocating the outputs
    when `outs` is None (dX may be None in `outs`: no input gradient)."""
    M = _need(X, torch.bfloat16, (None, h), "X").shape[0]
    r = _need(L1, torch.bfloat16, (h, None), "L1").shape[1]
    _need(L2, torch.bfloat16, (r, o), "L2")
    _need(dY, torch.bfloat16, (M, o), "dY")
    if T is not None:
        _need(T, torch.bfloat16, (M, r), "T")
    if outs is None:
        dX = torch.empty(M, h, dtype=torch.bfloat16, device=X.device) if want_dX else None
        dL1 = torch.empty(h, r, dtype=torch.float32, device=X.device)
        dL2 = torch.empty(r, o, dtype=torch.float32, device=X.device)
    else:
        dX, dL1, dL2 = outs
        if dX is not None:
            _need(dX, torch.bfloat16, (M, h), "dX")
        _need(dL1, torch.float32, (h, r), "dL1")
        _need(dL2, torch.float32, (r, o), "dL2")
    return M, r, dX, dL1, dL2


def fwd(q: NF4Weight, X: torch.Tensor, L1: torch.Tensor, L2: torch.Tensor, s: float, want_T: bool = True,
        ws: torch.Tensor | None = None, out: torch.Tensor | None = None, T_out: torch.Tensor | None = None):
    """nf4lora_fwd: returns (Y bf16 [M][o], T bf16 [M][r] or None)."""
    M, r, Y, T = _fwd_args(_need_q(q).rows, q.cols, X, L1, L2, want_T, out, T_out)
    ws = _need_ws(ws) if ws is not None else workspace(NF4_OP_FWD, M, q, r)
    _check(_lib.nf4lora_fwd(ctypes.byref(q.desc), _ptr(X), M, _ptr(L1), _ptr(L2), r, float(s),
                            _ptr(Y), _ptr(T), _ptr(ws), ws.numel(), _stream()), "nf4lora_fwd")
    return Y, T


def fwd_noalloc(q: NF4Weight, X: torch.Tensor, L1: torch.Tensor, L2: torch.Tensor, s: float, want_T: bool = True,
                out: torch.Tensor | None = None, T_out: torch.Tensor | None = None):
    """nf4lora_fwd_noalloc: nf4lora_fwd on the library's fixed device area (no workspace argument).
    With `out` (and `T_out`) given, the call itself allocates nothing."""
    M, r, Y, T = _fwd_args(_need_q(q).rows, q.cols, X, L1, L2, want_T, out, T_out)
    _check(_lib.nf4lora_fwd_noalloc(ctypes.byref(q.desc), _ptr(X), M, _ptr(L1), _ptr(L2), r,
                                    float(s), _ptr(Y), _ptr(T), _stream()), "nf4lora_fwd_noalloc")
    return Y, T


def bwd(q: NF4Weight, X: torch.Tensor, dY: torch.Tensor, L1: torch.Tensor, L2: torch.Tensor, s: float,
        T: torch.Tensor | None = None, want_dX: bool = True, ws: torch.Tensor | None = None, outs=None):
    """nf4lora_bwd: returns (dX bf16 [M][h] or None, dL1 fp32 [h][r], dL2 fp32 [r][o])."""
    M, r, dX, dL1, dL2 = _bwd_args(_need_q(q).rows, q.cols, X, dY, L1, L2, T, want_dX, outs)
    ws = _need_ws(ws) if ws is not None else workspace(NF4_OP_BWD, M, q, r)
    _check(_lib.nf4lora_bwd(ctypes.byref(q.desc), _ptr(X), _ptr(dY), M, _ptr(L1), _ptr(L2),
                            r, float(s), _ptr(T), _ptr(dX), _ptr(dL1), _ptr(dL2), _ptr(ws), ws.numel(), _stream()),
           "nf4lora_bwd")
    return dX, dL1, dL2


def bf16_workspace(op: int, M: int, W: torch.Tensor, r: int) -> torch.Tensor:
    """Workspace for bf16lora_fwd / bf16lora_bwd on a bf16 weight [o][h]."""
    _need(W, torch.bfloat16, (None, None), "W")
    return torch.empty(workspace_bytes(op, M, W.shape[0], W.shape[1], r), dtype=torch.uint8, device=W.device)


def bf16_fwd(W: torch.Tensor, X: torch.Tensor, L1: torch.Tensor, L2: torch.Tensor, s: float, want_T: bool = True,
             ws: torch.Tensor | None = None, out: torch.Tensor | None = None, T_out: torch.Tensor | None = None):
    """bf16lora_fwd (a protected linear, bf16 W [o][h]): returns (Y, T or None)."""
    o, h = _need(W, torch.bfloat16, (None, None), "W").shape
    M, r, Y, T = _fwd_args(o, h, X, L1, L2, want_T, out, T_out)
    ws = _need_ws(ws) if ws is not None else bf16_workspace(NF4_OP_FWD, M, W, r)
    _check(_lib.bf16lora_fwd(_ptr(W), o, h, _ptr(X), M, _ptr(L1), _ptr(L2), r, float(s),
                             _ptr(Y), _ptr(T), _ptr(ws), ws.numel(), _stream()), "bf16lora_fwd")
    return Y, T


def bf16_bwd(W: torch.Tensor, X: torch.Tensor, dY: torch.Tensor, L1: torch.Tensor, L2: torch.Tensor, s: float,
             T: torch.Tensor | None = None, want_dX: bool = True, ws: torch.Tensor | None = None, outs=None):
    """bf16lora_bwd: returns (dX or None, dL1, dL2)."""
    o, h = _need(W, torch.bfloat16, (None, None), "W").shape
    M, r, dX, dL1, dL2 = _bwd_args(o, h, X, dY, L1, L2, T, want_dX, outs)
    ws = _need_ws(ws) if ws is not None else bf16_workspace(NF4_OP_BWD, M, W, r)
    _check(_lib.bf16lora_bwd(_ptr(W), o, h, _ptr(X), _ptr(dY), M, _ptr(L1), _ptr(L2),
                             r, float(s), _ptr(T), _ptr(dX), _ptr(dL1), _ptr(dL2), _ptr(ws), ws.numel(), _stream()),
           "bf16lora_bwd")
    return dX, dL1, dL2


def layer_error(W: torch.Tensor, dq_group: int = 0, out: torch.Tensor | None = None,
                ws: torch.Tensor | None = None, codebook: str = "nf4") -> torch.Tensor:
    """nf4_layer_error: a cuda float64 tensor of shape [1] (no host sync)."""
    rows, cols = _need(W, torch.float32, (None, None), "W").shape
    err = _need_vec(out, torch.float64, 1, "out") if out is not None else \
        torch.empty(1, dtype=torch.float64, device=W.device)
    if ws is not None:
        _need_ws(ws)
    else:
        n = workspace_bytes(NF4_OP_ERROR, 0, rows, cols, 1)
        ws = torch.empty(n, dtype=torch.uint8, device=W.device)
    _check(_lib.nf4_layer_error(_ptr(W), rows, cols, BLOCK, dq_group, CODEBOOKS[codebook], _ptr(err), _ptr(ws),
                                ws.numel(), _stream()), "nf4_layer_error")
    return err


def _shape_arrays(shapes):
    n = len(shapes)
    rows = (_i64 * max(n, 1))(*[r for r, _ in shapes])
    cols = (_i64 * max(n, 1))(*[c for _, c in shapes])
    return rows, cols


def error_batch_workspace_bytes(shapes) -> int:
    """nf4_error_batch_workspace_bytes for a list of (rows, cols)."""
    rows, cols = _shape_arrays(shapes)
    b = _sz()
    _check(_lib.nf4_error_batch_workspace_bytes(rows, cols, len(shapes), ctypes.byref(b)),
           "nf4_error_batch_workspace_bytes")
    return b.value


def layer_error_batch(Ws, dq_group: int = 0, out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                      codebook: str = "nf4") -> torch.Tensor:
    """nf4_layer_error_batch over a list of cuda fp32 [rows][cols] tensors: a cuda float64 [n] tensor whose
    entry i equals layer_error(Ws[i], dq_group, codebook=codebook) bit for bit (no host sync)."""
    for i, W in enumerate(Ws):
        _need(W, torch.float32, (None, None), f"Ws[{i}]")
    n = len(Ws)
    shapes = [tuple(W.shape) for W in Ws]
    dev = Ws[0].device if n else torch.device("cuda")
    if out is not None:
        err = _need_vec(out, torch.float64, n, "out")
    else:
        err = torch.empty(max(n, 1), dtype=torch.float64, device=dev)
    if ws is not None:
        _need_ws(ws)
    else:
        ws = torch.empty(error_batch_workspace_bytes(shapes), dtype=torch.uint8, device=dev)
    rows, cols = _shape_arrays(shapes)
    ptrs = (_vp * max(n, 1))(*[W.data_ptr() for W in Ws])
    _check(_lib.nf4_layer_error_batch(ptrs, rows, cols, n, dq_group, CODEBOOKS[codebook], _ptr(err), _ptr(ws),
                                      ws.numel(), _stream()), "nf4_layer_error_batch")
    return err[:n]


def quantize_error(W: torch.Tensor, dq_group: int = 0, err_dq_group: int = 0, out: NF4Weight | None = None,
                   err: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                   codebook: str = "nf4") -> tuple[NF4Weight, torch.Tensor]:
    """nf4_quantize_error: (q, err) from one pass over W; q as quantize() gives it (one stage; `out`'s codebook
    applies when given), err a cuda float64 [1] equal to layer_error(W, err_dq_group, codebook=q's)."""
    rows, cols = _need(W, torch.float32, (None, None), "W").shape
    q = _need_q(out, rows, cols, "out") if out is not None else NF4Weight(rows, cols, dq_group, W.device, codebook)
    err = _need_vec(err, torch.float64, 1, "err") if err is not None else \
        torch.empty(1, dtype=torch.float64, device=W.device)
    if ws is not None:
        _need_ws(ws)
    else:
        ws = torch.empty(workspace_bytes(NF4_OP_ERROR, 0, rows, cols, 1), dtype=torch.uint8, device=W.device)
    _check(_lib.nf4_quantize_error(_ptr(W), ctypes.byref(q.desc), err_dq_group, _ptr(err), _ptr(ws), ws.numel(),
                                   _stream()), "nf4_quantize_error")
    return q, err


def matmul(q: NF4Weight, A: torch.Tensor, transpose: bool = False, A2: torch.Tensor | None = None,
           B2: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """nf4_matmul: A * W_hat^T (+ A2 * B2^T), or A * W_hat (+ ...) with transpose=True."""
    _need_q(q)
    K, N = (q.rows, q.cols) if transpose else (q.cols, q.rows)
    M = _need(A, torch.bfloat16, (None, K), "A").shape[0]
    R = 0
    if A2 is not None or B2 is not None:
        if A2 is None or B2 is None:
            raise ValueError("A2 and B2: give both or neither")
        R = _need(A2, torch.bfloat16, (M, None), "A2").shape[1]
        _need(B2, torch.bfloat16, (N, R), "B2")
    C = _need(out, torch.bfloat16, (M, N), "out") if out is not None else \
        torch.empty(M, N, dtype=torch.bfloat16, device=A.device)
    _check(_lib.nf4_matmul(ctypes.byref(q.desc), 1 if transpose else 0, _ptr(A), M,
                           _ptr(A2), _ptr(B2), R, _ptr(C), _stream()), "nf4_matmul")
    return C


def check_finite(W: torch.Tensor, ws: torch.Tensor | None = None) -> bool:
    """nf4_check_finite (synchronizes the stream): True when every value of the cuda fp32 W is finite."""
    _need(W, torch.float32, None, "W")
    if ws is not None:
        _need_ws(ws)
    else:
        ws = torch.empty(workspace_bytes(NF4_OP_CHECK, 0, 0, 0, 0), dtype=torch.uint8, device=W.device)
    st = _lib.nf4_check_finite(_ptr(W), W.numel(), _ptr(ws), ws.numel(), _stream())
    if st == NF4_ERR_NONFINITE:
        return False
    _check(st, "nf4_check_finite")
    return True


def probe_mfma_peak(iters: int, workgroups: int, out: torch.Tensor) -> None:
    """nf4_probe_mfma_peak: 8 * iters bf16 MFMAs (32x32x16) per wave, 8 waves per workgroup (asynchronous)."""
    _need(out, torch.float32, None, "out")
    if out.numel() < workgroups * 512:
        raise ValueError(f"out: expected at least {workgroups * 512} entries, got {out.numel()}")
    _check(_lib.nf4_probe_mfma_peak(int(iters), int(workgroups), _ptr(out), _stream()), "nf4_probe_mfma_peak")


def topk(errors: torch.Tensor, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """nf4_topk over a cuda float64 vector: int32 indices, largest first, ties to the lower index."""
    _need(errors, torch.float64, (None,), "errors")
    if out is not None:
        idx = _need_vec(out, torch.int32, k, "out")
    else:
        idx = torch.empty(max(k, 1), dtype=torch.int32, device=errors.device)
    _check(_lib.nf4_topk(_ptr(errors), errors.numel(), k, _ptr(idx), _stream()), "nf4_topk")
    return idx[:k]


def merge(base, L1: torch.Tensor, L2: torch.Tensor, s: float, bf16: bool = False,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """nf4lora_merge: base (fp32 W tensor [o][h] or NF4Weight) + s (L1 L2)^T, fp32 or bf16 [o][h]."""
    if isinstance(base, NF4Weight):
        W, q, rows, cols, dev = None, ctypes.byref(base.desc), base.rows, base.cols, base.codes.device
    else:
        W, q, (rows, cols), dev = _need(base, torch.float32, (None, None), "base"), None, base.shape, base.device
    r = _need(L1, torch.bfloat16, (cols, None), "L1").shape[1]
    _need(L2, torch.bfloat16, (r, rows), "L2")
    odt = torch.bfloat16 if bf16 else torch.float32
    out = _need(out, odt, (rows, cols), "out") if out is not None else torch.empty(rows, cols, dtype=odt, device=dev)
    _check(_lib.nf4lora_merge(_ptr(W), q, rows, cols, _ptr(L1), _ptr(L2), r, float(s), _ptr(out),
                              1 if bf16 else 0, _stream()), "nf4lora_merge")
    return out


# ---------------------------------------------------------------------------
# stack runner
# ---------------------------------------------------------------------------

class Stack:
    """A list of linears for nf4_stack_fwd / nf4_stack_bwd.

    Each linear is a dict: weight ("q": NF4Weight or "w": bf16 tensor [o][h]),
    optional adapter ("r", "s", "L1", "L2"; r = 0 or absent: none) and the
    buffers "X", "Y", "T", "dY", "dX", "dL1", "dL2" (tensors or None).  The
    tensors must stay alive as long as the Stack is used.
    """

    def __init__(self, linears, M: int):
        self.M = M
        self.linears = linears
        self.arr = (_NF4Linear * len(linears))()
        for i, L in enumerate(linears):
            e = self.arr[i]
            if L.get("q") is not None:
                q = _need_q(L["q"], name=f"linears[{i}].q")
                e.q = ctypes.pointer(q.desc)
                o, h = q.rows, q.cols
            else:
                W = _need(L.get("w"), torch.bfloat16, (None, None), f"linears[{i}].w")
                o, h = W.shape
                e.w_bf16, e.rows, e.cols = _ptr(W), o, h
            e.r, e.s = int(L.get("r", 0)), float(L.get("s", 0.0))
            r = max(e.r, 0)
            shapes = {"L1": (torch.bfloat16, (h, r)), "L2": (torch.bfloat16, (r, o)),
                      "X": (torch.bfloat16, (M, h)), "Y": (torch.bfloat16, (M, o)), "T": (torch.bfloat16, (M, r)),
                      "dY": (torch.bfloat16, (M, o)), "dX": (torch.bfloat16, (M, h)),
                      "dL1": (torch.float32, (h, r)), "dL2": (torch.float32, (r, o))}
            for k, (dt, shp) in shapes.items():
                t = L.get(k)
                if t is not None:
                    _need(t, dt, shp, f"linears[{i}].{k}")
                setattr(e, k, _ptr(t))
        n = _sz()
        _check(_lib.nf4_stack_workspace_bytes(self.arr, len(linears), M, ctypes.byref(n)),
               "nf4_stack_workspace_bytes")
        self.ws = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device="cuda")

    def fwd(self):
        _check(_lib.nf4_stack_fwd(self.arr, len(self.linears), self.M, _ptr(self.ws), self.ws.numel(), _stream()),
               "nf4_stack_fwd")

    def bwd(self, cut: int = 0):
        _check(_lib.nf4_stack_bwd(self.arr, len(self.linears), cut, self.M, _ptr(self.ws), self.ws.numel(),
                                  _stream()), "nf4_stack_bwd")

