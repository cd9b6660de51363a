"""ctypes binding of libq8proj.so (C ABI in include/q8proj.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream, every step of the computation runs in the library's
kernels. There is no CPU fallback: if the library is missing the functions
raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq8proj.so")

LAYOUT_ROW = 0
LAYOUT_PLANE64 = 1
QK = 32

_ERRORS = {0: "Q8_OK", -1: "Q8_EINVAL", -2: "Q8_ESHAPE", -3: "Q8_EALIGN", -4: "Q8_ELAUNCH", -5: "Q8_ENODEV"}


class Q8Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_ERRORS.get(code, code)} ({_lib_strerror(code)})")


WEIGHTS_Q8_0 = 0
WEIGHTS_Q4_K = 1


class _Weights(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("qs", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("format", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library with argument types set. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python int8_quantized_projections_amd/_build.py")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        wp = ctypes.POINTER(_Weights)
        sig = {
            "q8_abi_version": ([], ci),
            "q8_strerror": ([ci], ctypes.c_char_p),
            "q8_act_bytes": ([i64, i64, ci, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)], ci),
            "q8_plane_bytes": ([i64, i64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)], ci),
            "q8_quantize": ([vp, i64, i64, ci, vp, vp, vp], ci),
            "rmsnorm_quant": ([vp, vp, ctypes.c_float, vp, i64, i64, ci, vp, vp, vp], ci),
            "swiglu_quant": ([vp, vp, vp, i64, i64, ci, vp, vp, vp], ci),
            "q8_gemv": ([wp, vp, vp, vp, vp], ci),
            "q8_gemv_f32": ([wp, vp, vp, vp], ci),
            "q8_gemv_shared_multi": ([ci, ctypes.POINTER(wp), vp, vp, ctypes.POINTER(vp), vp], ci),
            "q8_gemv_shared_multi_ex": ([ci, ctypes.POINTER(wp), vp, vp, ctypes.POINTER(vp), ci, vp], ci),
            "q8_gemv_plan": ([i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(ci), ctypes.POINTER(i64)], ci),
            "q8_gemm": ([wp, vp, vp, i64, vp, i64, vp], ci),
            "q4k_gemm": ([ctypes.POINTER(_Q4KWeights), vp, vp, i64, vp, i64, vp], ci),
            "q8_gemm_shared_multi": ([ci, ctypes.POINTER(wp), vp, vp, i64, ctypes.POINTER(vp), ctypes.POINTER(i64), vp],
                                     ci),
            "q8_weights_repack": ([vp, i64, i64, vp, vp, vp], ci),
            "q8_gemv_shared_multi_plus_f32": ([ci, ctypes.POINTER(wp), vp, vp, ctypes.POINTER(vp), wp, vp, vp, vp], ci),
            "rmsnorm_quant_gemv_shared_multi_plus_f32": ([vp, vp, ctypes.c_float, vp, vp, vp, ci, ctypes.POINTER(wp),
                                                          ctypes.POINTER(vp), wp, vp, vp, vp], ci),
            "q8_hbm_read_probe": ([vp, i64, ci, ci, vp, vp], ci),
            "q8_hbm_stream_probe": ([vp, vp, vp, i64, ci, vp, vp], ci),
            "q8_launch_counts": ([ctypes.POINTER(i64), ci], ci),
            "q8_launch_counts_reset": ([], None),
            "q8_launch_counter_name": ([ci], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _lib_strerror(code: int) -> str:
    try:
        return lib().q8_strerror(code).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "?"


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise Q8Error(rc, where)


def _stream(device: torch.device | None = None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("q8lib expects device tensors")
    if not t.is_contiguous():
        raise ValueError("q8lib expects contiguous tensors")
    return t.data_ptr()


# Buffer checks, made before anything reaches the library: a tensor of the wrong
# element type, or one too short for what the kernel reads or writes, is refused
# here (the C ABI sees only a pointer and cannot tell).
_I8 = (torch.int8, torch.uint8)
_I16 = (torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.int16,)
_I32 = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _need(t: torch.Tensor | None, name: str, dtypes, numel: int) -> torch.Tensor | None:
    """t (or None) must have one of `dtypes` and at least `numel` elements."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")
    return t


def _need_act(qs, sd, rows: int, k: int, layout: int, what: str) -> None:
    """Quantized-activation buffers of rows x k in `layout`: int8 qs and 32-bit scale words."""
    nq, ns = act_bytes(rows, k, layout)
    _need(qs, f"{what} qs", _I8, nq)
    _need(sd, f"{what} sd", _I32, ns // 4)


# ---------------------------------------------------------------------------
# Buffers
# ---------------------------------------------------------------------------
def launch_counts() -> dict[str, int]:
    """The library's launch counter of every entry point, by entry-point name (see
    q8_launch_counts in include/q8proj.h)."""
    L = lib()
    n = L.q8_launch_counts(None, 0)  # the number of counters
    if n < 0:
        raise Q8Error(n, "q8_launch_counts")
    buf = (ctypes.c_int64 * n)()
    rc = L.q8_launch_counts(buf, n)
    if rc != n:
        raise Q8Error(rc, "q8_launch_counts")
    return {L.q8_launch_counter_name(i).decode(): int(buf[i]) for i in range(n)}


def launch_counts_reset() -> None:
    lib().q8_launch_counts_reset()


def plane_bytes(t: int, k: int) -> tuple[int, int]:
    """(qs bytes, scale-word bytes) of a PLANE64 activation of t tokens of width k."""
    q = ctypes.c_size_t()
    s = ctypes.c_size_t()
    _check(lib().q8_plane_bytes(t, k, ctypes.byref(q), ctypes.byref(s)), "q8_plane_bytes")
    return q.value, s.value


def act_bytes(rows: int, k: int, layout: int) -> tuple[int, int]:
    q = ctypes.c_size_t()
    s = ctypes.c_size_t()
    _check(lib().q8_act_bytes(rows, k, layout, ctypes.byref(q), ctypes.byref(s)), "q8_act_bytes")
    return q.value, s.value


def alloc_act(rows: int, k: int, layout: int, device="cuda") -> tuple[torch.Tensor, torch.Tensor]:
    """Caller-owned quantized-activation buffers (qs int8, sd int32 holding the uint32 words)."""
    nq, ns = act_bytes(rows, k, layout)
    return (torch.empty(nq, dtype=torch.int8, device=device), torch.empty(ns // 4, dtype=torch.int32, device=device))


@dataclass
class Q8Weights:
    """Q8_0 weights as the library's two planes: qs [N, K] int8 and d [N, K/32] f16 bits (int16)."""
    qs: torch.Tensor
    d: torch.Tensor

    @property
    def n(self) -> int:
        return self.qs.shape[0]

    @property
    def k(self) -> int:
        return self.qs.shape[1]

    def struct(self) -> _Weights:
        if self.qs.dim() != 2 or self.d.dim() != 2:
            raise ValueError("Q8Weights: qs [N, K] and d [N, K/32] must be 2-D")
        _need(self.qs, "Q8Weights.qs", _I8, 0)
        _need(self.d, "Q8Weights.d", _I16, 0)
        if self.k % QK != 0 or tuple(self.d.shape) != (self.n, self.k // QK):
            raise ValueError(f"Q8Weights: d is {tuple(self.d.shape)}, expected ({self.n}, {self.k // QK})")
        return _Weights(self.n, self.k, _ptr(self.qs), _ptr(self.d), WEIGHTS_Q8_0)

    def rows(self, start: int, stop: int) -> "Q8Weights":
        """A band of output rows (a pointer offset and a smaller N)."""
        return Q8Weights(self.qs[start:stop], self.d[start:stop])


class _Q4KWeights(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("blocks", ctypes.c_void_p)]


@dataclass
class Q4KWeights:
    """q4_K weights on the device: uint8 [N, K/256*144] (raw 144-byte super-blocks, row-major)."""
    blocks: torch.Tensor
    k: int

    @property
    def n(self) -> int:
        return self.blocks.shape[0]

    def struct(self) -> _Q4KWeights:
        _need(self.blocks, "Q4KWeights.blocks", torch.uint8, 0)
        if self.k % 256 != 0 or self.blocks.dim() != 2 or self.blocks.shape[1] != self.k // 256 * 144:
            raise ValueError(f"Q4KWeights: blocks {tuple(self.blocks.shape)} do not hold K={self.k} "
                             "in 144-byte super-blocks of 256 values")
        return _Q4KWeights(self.n, self.k, _ptr(self.blocks))

    def q8_struct(self) -> _Weights:
        """The same weights as a q8_weights descriptor of format Q8_WEIGHTS_Q4_K (for q8_gemm)."""
        w = self.struct()
        return _Weights(w.n, w.k, w.blocks, None, WEIGHTS_Q4_K)


def q4k_gemm(W: Q4KWeights, a_qs: torch.Tensor, a_sd: torch.Tensor, t: int, C=None, ldc: int | None = None):
    """C [t, N] = q4_K weights x PLANE64 q8_0 activation (see include/q8proj.h)."""
    if C is None:
        C = torch.empty((t, W.n), dtype=torch.float32, device=a_qs.device)
    if ldc is None:
        ldc = C.shape[-1] if C.dim() > 1 else W.n
    _need_act(a_qs, a_sd, t, W.k, LAYOUT_PLANE64, "q4k_gemm")
    _need(C, "C", torch.float32, (t - 1) * ldc + W.n if t > 0 else 0)
    ws = W.struct()
    _check(lib().q4k_gemm(ctypes.byref(ws), _ptr(a_qs), _ptr(a_sd), t, _ptr(C), ldc, _stream(a_qs.device)),
           "q4k_gemm")
    return C


def q8_weights_repack(blocks: torch.Tensor, n: int, k: int) -> Q8Weights:
    """GGUF Q8_0 blocks (device uint8, N*K/32*34 bytes) -> Q8Weights (one-time, at load)."""
    _need(blocks, "blocks", torch.uint8, n * (k // QK) * 34)
    qs = torch.empty((n, k), dtype=torch.int8, device=blocks.device)
    d = torch.empty((n, k // QK), dtype=torch.int16, device=blocks.device)
    _check(lib().q8_weights_repack(_ptr(blocks), n, k, _ptr(qs), _ptr(d), _stream(blocks.device)),
           "q8_weights_repack")
    return Q8Weights(qs, d)


# ---------------------------------------------------------------------------
# Producers
# ---------------------------------------------------------------------------
def _rows_k(x: torch.Tensor) -> tuple[int, int]:
    """(rows, K) of an activation: [K] is one row, [rows, K] a matrix; other ranks are refused."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(x).__name__}")
    if x.dim() == 1:
        return 1, x.shape[0]
    if x.dim() == 2:
        return x.shape[0], x.shape[1]
    raise ValueError(f"activations are [K] or [rows, K]; got shape {tuple(x.shape)}")


def q8_quantize(x: torch.Tensor, layout: int = LAYOUT_ROW, qs=None, sd=None):
    rows, k = _rows_k(x)
    _need(x, "x", torch.float32, rows * k)
    if qs is None:
        qs, sd = alloc_act(rows, k, layout, x.device)
    _need_act(qs, sd, rows, k, layout, "q8_quantize")
    _check(lib().q8_quantize(_ptr(x), rows, k, layout, _ptr(qs), _ptr(sd), _stream(x.device)), "q8_quantize")
    return qs, sd


def rmsnorm_quant(x: torch.Tensor, w: torch.Tensor, eps: float, layout: int = LAYOUT_ROW, y=None, qs=None, sd=None,
                  quant: bool = True, f32: bool = True):
    """f32=False passes y = NULL: only the quantized activation is written (returned y is None)."""
    rows, k = _rows_k(x)
    _need(x, "x", torch.float32, rows * k)
    _need(w, "w", torch.float32, k)
    if y is None and f32:
        y = torch.empty_like(x)
    if quant and qs is None:
        qs, sd = alloc_act(rows, k, layout, x.device)
    if not quant:
        qs = sd = None
    _need(y, "y", torch.float32, rows * k)
    if qs is not None or sd is not None:
        _need_act(qs, sd, rows, k, layout, "rmsnorm_quant")
    _check(lib().rmsnorm_quant(_ptr(x), _ptr(w), eps, _ptr(y), rows, k, layout, _ptr(qs), _ptr(sd),
                               _stream(x.device)), "rmsnorm_quant")
    return y, qs, sd


def swiglu_quant(gate: torch.Tensor, up: torch.Tensor, layout: int = LAYOUT_ROW, y=None, qs=None, sd=None,
                 quant: bool = True, f32: bool = True):
    """f32=False passes y = NULL: only the quantized activation is written (returned y is None)."""
    rows, k = _rows_k(gate)
    _need(gate, "gate", torch.float32, rows * k)
    _need(up, "up", torch.float32, rows * k)
    if tuple(up.shape) != tuple(gate.shape):
        raise ValueError(f"gate {tuple(gate.shape)} and up {tuple(up.shape)} differ")
    if y is None and f32:
        y = torch.empty_like(gate)
    if quant and qs is None:
        qs, sd = alloc_act(rows, k, layout, gate.device)
    if not quant:
        qs = sd = None
    _need(y, "y", torch.float32, rows * k)
    if qs is not None or sd is not None:
        _need_act(qs, sd, rows, k, layout, "swiglu_quant")
    _check(lib().swiglu_quant(_ptr(gate), _ptr(up), _ptr(y), rows, k, layout, _ptr(qs), _ptr(sd),
                              _stream(gate.device)), "swiglu_quant")
    return y, qs, sd


# ---------------------------------------------------------------------------
# Consumers
# ---------------------------------------------------------------------------
def _need_row_act(a_qs, a_sd, k: int, what: str) -> None:
    _need(a_qs, f"{what} a_qs", _I8, k)
    _need(a_sd, f"{what} a_sd", _I32, k // QK)


def q8_gemv(W: Q8Weights, a_qs: torch.Tensor, a_sd: torch.Tensor, y=None) -> torch.Tensor:
    if y is None:
        y = torch.empty(W.n, dtype=torch.float32, device=a_qs.device)
    _need_row_act(a_qs, a_sd, W.k, "q8_gemv")
    _need(y, "y", torch.float32, W.n)
    ws = W.struct()
    _check(lib().q8_gemv(ctypes.byref(ws), _ptr(a_qs), _ptr(a_sd), _ptr(y), _stream(a_qs.device)), "q8_gemv")
    return y


def q8_gemv_f32(W: Q8Weights, x: torch.Tensor, y=None) -> torch.Tensor:
    """GEMV on an f32 activation [K] quantized inside the launch (K <= 8192)."""
    if y is None:
        y = torch.empty(W.n, dtype=torch.float32, device=x.device)
    _need(x, "x", torch.float32, W.k)
    _need(y, "y", torch.float32, W.n)
    ws = W.struct()
    _check(lib().q8_gemv_f32(ctypes.byref(ws), _ptr(x), _ptr(y), _stream(x.device)), "q8_gemv_f32")
    return y


def _need_members(Ws, ys) -> None:
    """Members of a grouped GEMV: one output per weight matrix, each long enough."""
    if len(Ws) == 0 or len(ys) != len(Ws):
        raise ValueError(f"{len(Ws)} weight matrices and {len(ys)} outputs")
    for i, (W, y) in enumerate(zip(Ws, ys)):
        _need(y, f"y[{i}]", torch.float32, W.n)


def q8_gemv_shared_multi(Ws: list[Q8Weights], a_qs: torch.Tensor, a_sd: torch.Tensor, ys=None,
                         rows_per_wave: int = 0) -> list[torch.Tensor]:
    m = len(Ws)
    if ys is None:
        ys = [torch.empty(W.n, dtype=torch.float32, device=a_qs.device) for W in Ws]
    _need_members(Ws, ys)
    _need_row_act(a_qs, a_sd, Ws[0].k, "q8_gemv_shared_multi")
    structs = [W.struct() for W in Ws]
    wps = (ctypes.POINTER(_Weights) * m)(*[ctypes.pointer(s) for s in structs])
    yps = (ctypes.c_void_p * m)(*[_ptr(y) for y in ys])
    _check(lib().q8_gemv_shared_multi_ex(m, wps, _ptr(a_qs), _ptr(a_sd), yps, rows_per_wave, _stream(a_qs.device)),
           "q8_gemv_shared_multi")
    return ys


def q8_gemv_shared_multi_plus_f32(Ws: list[Q8Weights], a_qs: torch.Tensor, a_sd: torch.Tensor, Wx: Q8Weights,
                                  x: torch.Tensor, ys=None, yx=None) -> tuple[list[torch.Tensor], torch.Tensor]:
    """q8_gemv_shared_multi(Ws, a_qs, a_sd) and q8_gemv_f32(Wx, x) in one launch; returns (ys, yx)."""
    m = len(Ws)
    if ys is None:
        ys = [torch.empty(W.n, dtype=torch.float32, device=a_qs.device) for W in Ws]
    if yx is None:
        yx = torch.empty(Wx.n, dtype=torch.float32, device=x.device)
    _need_members(Ws, ys)
    _need_row_act(a_qs, a_sd, Ws[0].k, "q8_gemv_shared_multi_plus_f32")
    _need(x, "x", torch.float32, Wx.k)
    _need(yx, "yx", torch.float32, Wx.n)
    structs = [W.struct() for W in Ws]
    wps = (ctypes.POINTER(_Weights) * m)(*[ctypes.pointer(st) for st in structs])
    yps = (ctypes.c_void_p * m)(*[_ptr(y) for y in ys])
    wx = Wx.struct()
    _check(lib().q8_gemv_shared_multi_plus_f32(m, wps, _ptr(a_qs), _ptr(a_sd), yps, ctypes.byref(wx), _ptr(x),
                                               _ptr(yx), _stream(a_qs.device)), "q8_gemv_shared_multi_plus_f32")
    return ys, yx


def rmsnorm_quant_gemv_shared_multi_plus_f32(x: torch.Tensor, w: torch.Tensor, eps: float, Ws: list[Q8Weights],
                                             Wx: Q8Weights, x2: torch.Tensor, y=None, a_qs=None, a_sd=None, ys=None,
                                             yx=None, f32: bool = True):
    """rmsnorm_quant of the row x (ROW layout) and q8_gemv_shared_multi_plus_f32 of its consumers, in one
    launch where the shapes allow. Wx = None: no f32-activation GEMV (x2 is ignored, yx is None).
    f32=False passes y = NULL. Returns (y, a_qs, a_sd, ys, yx)."""
    rows, k = _rows_k(x)
    if rows != 1:
        raise ValueError("the decode step normalizes one row")
    if y is None and f32:
        y = torch.empty_like(x)
    if a_qs is None:
        a_qs, a_sd = alloc_act(1, k, LAYOUT_ROW, x.device)
    m = len(Ws)
    if ys is None:
        ys = [torch.empty(W.n, dtype=torch.float32, device=x.device) for W in Ws]
    if yx is None and Wx is not None:
        yx = torch.empty(Wx.n, dtype=torch.float32, device=x.device)
    _need(x, "x", torch.float32, k)
    _need(w, "w", torch.float32, k)
    _need(y, "y", torch.float32, k)
    _need_row_act(a_qs, a_sd, k, "rmsnorm_quant_gemv_shared_multi_plus_f32")
    _need_members(Ws, ys)
    if Wx is not None:
        _need(x2, "x2", torch.float32, Wx.k)
        _need(yx, "yx", torch.float32, Wx.n)
    structs = [W.struct() for W in Ws]
    wps = (ctypes.POINTER(_Weights) * m)(*[ctypes.pointer(st) for st in structs])
    yps = (ctypes.c_void_p * m)(*[_ptr(t) for t in ys])
    wx = ctypes.byref(Wx.struct()) if Wx is not None else None  # None: no f32-activation GEMV
    _check(lib().rmsnorm_quant_gemv_shared_multi_plus_f32(_ptr(x), _ptr(w), eps, _ptr(y), _ptr(a_qs), _ptr(a_sd), m,
                                                          wps, yps, wx, _ptr(x2), _ptr(yx),
                                                          _stream(x.device)),
           "rmsnorm_quant_gemv_shared_multi_plus_f32")
    return y, a_qs, a_sd, ys, yx


def gemv_plan(total_rows: int, k: int, rows_per_wave: int = 0) -> dict:
    lanes = ctypes.c_int()
    rows = ctypes.c_int()
    wg = ctypes.c_int64()
    _check(lib().q8_gemv_plan(total_rows, k, rows_per_wave, ctypes.byref(lanes), ctypes.byref(rows),
                              ctypes.byref(wg)), "q8_gemv_plan")
    return {"lanes_per_row": lanes.value, "rows_per_wave": rows.value, "workgroups": wg.value}


def q8_gemm(W, a_qs: torch.Tensor, a_sd: torch.Tensor, t: int, C=None, ldc: int | None = None):
    """C [t, N] = W x PLANE64 activation; W is Q8Weights, or Q4KWeights (format Q8_WEIGHTS_Q4_K)."""
    if C is None:
        C = torch.empty((t, W.n), dtype=torch.float32, device=a_qs.device)
    if ldc is None:
        ldc = C.shape[-1] if C.dim() > 1 else W.n
    _need_act(a_qs, a_sd, t, W.k, LAYOUT_PLANE64, "q8_gemm")
    _need(C, "C", torch.float32, (t - 1) * ldc + W.n if t > 0 else 0)
    ws = W.q8_struct() if isinstance(W, Q4KWeights) else W.struct()
    _check(lib().q8_gemm(ctypes.byref(ws), _ptr(a_qs), _ptr(a_sd), t, _ptr(C), ldc, _stream(a_qs.device)), "q8_gemm")
    return C


def q8_gemm_shared_multi(Ws: list[Q8Weights], a_qs: torch.Tensor, a_sd: torch.Tensor, t: int, Cs=None,
                         ldcs: list[int] | None = None) -> list[torch.Tensor]:
    """One launch of q8_gemm for every W in Ws over the same PLANE64 activation."""
    m = len(Ws)
    if Cs is None:
        Cs = [torch.empty((t, W.n), dtype=torch.float32, device=a_qs.device) for W in Ws]
    if ldcs is None:
        ldcs = [C.shape[-1] if C.dim() > 1 else W.n for C, W in zip(Cs, Ws)]
    if m == 0 or len(Cs) != m or len(ldcs) != m:
        raise ValueError(f"{m} weight matrices, {len(Cs)} outputs, {len(ldcs)} leading dimensions")
    _need_act(a_qs, a_sd, t, Ws[0].k, LAYOUT_PLANE64, "q8_gemm_shared_multi")
    for i, (W, C, ld) in enumerate(zip(Ws, Cs, ldcs)):
        _need(C, f"C[{i}]", torch.float32, (t - 1) * ld + W.n if t > 0 and W.n > 0 else 0)
    structs = [W.struct() for W in Ws]
    wps = (ctypes.POINTER(_Weights) * m)(*[ctypes.pointer(s) for s in structs])
    cps = (ctypes.c_void_p * m)(*[_ptr(C) for C in Cs])
    lds = (ctypes.c_int64 * m)(*ldcs)
    _check(lib().q8_gemm_shared_multi(m, wps, _ptr(a_qs), _ptr(a_sd), t, cps, lds, _stream(a_qs.device)),
           "q8_gemm_shared_multi")
    return Cs


# ---------------------------------------------------------------------------
# Measurement helper
# ---------------------------------------------------------------------------
def hbm_read_probe(buf: torch.Tensor, workgroups: int, loads_per_lane: int = 1, out=None) -> torch.Tensor:
    """One launch streaming every byte of buf once (the practical HBM read rate; see
    q8_hbm_read_probe in include/q8proj.h). Returns the per-workgroup XOR words."""
    if out is None:
        out = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    _need(out, "out", _I32, workgroups)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().q8_hbm_read_probe(_ptr(buf), nbytes, workgroups, loads_per_lane, _ptr(out), _stream(buf.device)),
           "q8_hbm_read_probe")
    return out


def hbm_stream_probe(nbytes: int, workgroups: int, src0=None, src1=None, dst=None, out=None) -> None:
    """One launch of a plain stream: read nbytes from src0 (and src1), write nbytes to dst (see
    q8_hbm_stream_probe in include/q8proj.h). Every given tensor must hold at least nbytes."""
    for name, t in (("src0", src0), ("src1", src1), ("dst", dst)):
        if t is not None and t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, at least {nbytes} needed")
    if dst is None and out is None:
        raise ValueError("a read-only stream needs out (one int32 per workgroup)")
    if out is not None:
        _need(out, "out", _I32, workgroups)
    dev = next(t for t in (src0, src1, dst) if t is not None).device
    _check(lib().q8_hbm_stream_probe(_ptr(src0), _ptr(src1), _ptr(dst), nbytes, workgroups, _ptr(out), _stream(dev)),
           "q8_hbm_stream_probe")
