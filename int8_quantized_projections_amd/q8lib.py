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


class _Weights(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("qs", ctypes.c_void_p), ("d", ctypes.c_void_p)]


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
        return _Weights(self.n, self.k, _ptr(self.qs), _ptr(self.d))

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
        assert self.blocks.dtype == torch.uint8 and self.blocks.is_contiguous()
        assert self.blocks.shape[1] == self.k // 256 * 144
        return _Q4KWeights(self.n, self.k, _ptr(self.blocks))


def q4k_gemm(W: Q4KWeights, a_qs: torch.Tensor, a_sd: torch.Tensor, t: int, C=None, ldc: int | None = None):
    """C [t, N] = q4_K weights x PLANE64 q8_0 activation (see include/q8proj.h)."""
    if C is None:
        C = torch.empty((t, W.n), dtype=torch.float32, device=a_qs.device)
    if ldc is None:
        ldc = C.shape[-1] if C.dim() > 1 else W.n
    ws = W.struct()
    _check(lib().q4k_gemm(ctypes.byref(ws), _ptr(a_qs), _ptr(a_sd), t, _ptr(C), ldc, _stream(a_qs.device)),
           "q4k_gemm")
    return C


def q8_weights_repack(blocks: torch.Tensor, n: int, k: int) -> Q8Weights:
    """GGUF Q8_0 blocks (device uint8, N*K/32*34 bytes) -> Q8Weights (one-time, at load)."""
    assert blocks.dtype == torch.uint8 and blocks.numel() == n * (k // QK) * 34
    qs = torch.empty((n, k), dtype=torch.int8, device=blocks.device)
    d = torch.empty((n, k // QK), dtype=torch.int16, device=blocks.device)
    _check(lib().q8_weights_repack(_ptr(blocks), n, k, _ptr(qs), _ptr(d), _stream(blocks.device)),
           "q8_weights_repack")
    return Q8Weights(qs, d)


# ---------------------------------------------------------------------------
# Producers
# ---------------------------------------------------------------------------
def _rows_k(x: torch.Tensor) -> tuple[int, int]:
    if x.dim() == 1:
        return 1, x.shape[0]
    return x.shape[0], x.shape[-1]


def q8_quantize(x: torch.Tensor, layout: int = LAYOUT_ROW, qs=None, sd=None):
    rows, k = _rows_k(x)
    if qs is None:
        qs, sd = alloc_act(rows, k, layout, x.device)
    _check(lib().q8_quantize(_ptr(x), rows, k, layout, _ptr(qs), _ptr(sd), _stream(x.device)), "q8_quantize")
    return qs, sd


def rmsnorm_quant(x: torch.Tensor, w: torch.Tensor, eps: float, layout: int = LAYOUT_ROW, y=None, qs=None, sd=None,
                  quant: bool = True, f32: bool = True):
    """f32=False passes y = NULL: only the quantized activation is written (returned y is None)."""
    rows, k = _rows_k(x)
    if y is None and f32:
        y = torch.empty_like(x)
    if quant and qs is None:
        qs, sd = alloc_act(rows, k, layout, x.device)
    if not quant:
        qs = sd = None
    _check(lib().rmsnorm_quant(_ptr(x), _ptr(w), eps, _ptr(y), rows, k, layout, _ptr(qs), _ptr(sd),
                               _stream(x.device)), "rmsnorm_quant")
    return y, qs, sd


def swiglu_quant(gate: torch.Tensor, up: torch.Tensor, layout: int = LAYOUT_ROW, y=None, qs=None, sd=None,
                 quant: bool = True, f32: bool = True):
    """f32=False passes y = NULL: only the quantized activation is written (returned y is None)."""
    rows, k = _rows_k(gate)
    if y is None and f32:
        y = torch.empty_like(gate)
    if quant and qs is None:
        qs, sd = alloc_act(rows, k, layout, gate.device)
    if not quant:
        qs = sd = None
    _check(lib().swiglu_quant(_ptr(gate), _ptr(up), _ptr(y), rows, k, layout, _ptr(qs), _ptr(sd),
                              _stream(gate.device)), "swiglu_quant")
    return y, qs, sd


# ---------------------------------------------------------------------------
# Consumers
# ---------------------------------------------------------------------------
def q8_gemv(W: Q8Weights, a_qs: torch.Tensor, a_sd: torch.Tensor, y=None) -> torch.Tensor:
    if y is None:
        y = torch.empty(W.n, dtype=torch.float32, device=a_qs.device)
    ws = W.struct()
    _check(lib().q8_gemv(ctypes.byref(ws), _ptr(a_qs), _ptr(a_sd), _ptr(y), _stream(a_qs.device)), "q8_gemv")
    return y


def q8_gemv_f32(W: Q8Weights, x: torch.Tensor, y=None) -> torch.Tensor:
    """GEMV on an f32 activation [K] quantized inside the launch (K <= 8192)."""
    if y is None:
        y = torch.empty(W.n, dtype=torch.float32, device=x.device)
    ws = W.struct()
    _check(lib().q8_gemv_f32(ctypes.byref(ws), _ptr(x), _ptr(y), _stream(x.device)), "q8_gemv_f32")
    return y


def q8_gemv_shared_multi(Ws: list[Q8Weights], a_qs: torch.Tensor, a_sd: torch.Tensor, ys=None,
                         rows_per_wave: int = 0) -> list[torch.Tensor]:
    m = len(Ws)
    if ys is None:
        ys = [torch.empty(W.n, dtype=torch.float32, device=a_qs.device) for W in Ws]
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


def q8_gemm(W: Q8Weights, a_qs: torch.Tensor, a_sd: torch.Tensor, t: int, C=None, ldc: int | None = None):
    if C is None:
        C = torch.empty((t, W.n), dtype=torch.float32, device=a_qs.device)
    if ldc is None:
        ldc = C.shape[-1] if C.dim() > 1 else W.n
    ws = W.struct()
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
    structs = [W.struct() for W in Ws]
    wps = (ctypes.POINTER(_Weights) * m)(*[ctypes.pointer(s) for s in structs])
    cps = (ctypes.c_void_p * m)(*[_ptr(C) for C in Cs])
    lds = (ctypes.c_int64 * m)(*ldcs)
    _check(lib().q8_gemm_shared_multi(m, wps, _ptr(a_qs), _ptr(a_sd), t, cps, lds, _stream(a_qs.device)),
           "q8_gemm_shared_multi")
    return Cs
