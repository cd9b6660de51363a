"""CPU oracle for the Q8_0 quantized projection path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library and its binding never
do, and the two share no code.

Thin numpy wrappers over ``q8_oracle.c`` (plain C, see its header for the
page citations). Every function here computes what the pages define, in f64
for floating point except the quantize, which the pages fix in f32.

Parity pins live in ``tests/test_oracle_pins.py``. One reading is pinned
only in part: the bit layout of q4_K's 6-bit scales and mins (the pages name
the decode but not its layout; the GGUF layout is taken, and the pins fix it
up to a permutation of bits), so that assignment is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "q8_oracle.c")

QK = 32
ROW, PLANE64 = 0, 1


def build() -> str:
    """Compile ``liboracle.so`` (always recompiles). No -ffast-math, no FMA contraction."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           SRC_PATH, "-o", LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        sig = {
            "q8o_f32_to_f16": ([ctypes.c_float], ctypes.c_uint16),
            "q8o_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
            "q8o_f32_to_f16_array": ([vp, i64, vp], None),
            "q8o_quantize_rows": ([vp, i64, i64, vp, vp, vp], None),
            "q8o_pack_sd": ([vp, vp, i64, vp], None),
            "q8o_plane_qs_offset": ([i64, i64, i64], i64),
            "q8o_plane_sd_index": ([i64, i64, i64], i64),
            "q8o_encode_plane64": ([vp, vp, vp, i64, i64, vp, vp], None),
            "q8o_decode_plane64": ([vp, vp, i64, i64, vp, vp, vp], i64),
            "q8o_rmsnorm_f64": ([vp, vp, i64, i64, ctypes.c_double, vp], None),
            "q8o_swiglu_f64": ([vp, vp, i64, vp], None),
            "q8o_quantize_weights_gguf": ([vp, i64, i64, vp], None),
            "q8o_gguf_to_planar": ([vp, i64, i64, vp, vp], None),
            "q8o_dot_pairs": ([vp, vp, i64, i64, vp, vp, i64, vp, vp, i64, vp, vp], None),
            "q8o_gemm_full": ([vp, vp, i64, i64, vp, vp, i64, vp, vp], None),
            "q8o_block_isums": ([vp, i64, i64, vp, i64, vp], None),
            "q8o_num_threads": ([], ctypes.c_int),
            "q8o_set_threads": ([ctypes.c_int], None),
            "q4ko_scale_min": ([vp, ctypes.c_int, vp, vp], None),
            "q4ko_decode": ([vp, i64, i64, vp, vp, vp, vp, vp], None),
            "q4ko_dequant_f64": ([vp, i64, i64, vp], None),
            "q4ko_dot_pairs": ([vp, i64, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp], None),
            "q4ko_gemm_full": ([vp, i64, i64, vp, vp, vp, i64, vp, vp], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def num_threads() -> int:
    return lib().q8o_num_threads()


def set_threads(n: int) -> None:
    """Threads of the following calls (results do not depend on it)."""
    lib().q8o_set_threads(n)


# -- f16 ---------------------------------------------------------------------
def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().q8o_f32_to_f16_array(x.ctypes.data, x.size, out.ctypes.data)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    f = lib().q8o_f16_to_f32
    return np.array([f(int(v)) for v in h.reshape(-1)], dtype=np.float32).reshape(h.shape)


def f16_to_f64(h) -> np.ndarray:
    """Exact value of f16 bit patterns (decoded from the format definition, vectorised)."""
    h = np.asarray(h, dtype=np.uint16).astype(np.int64)
    sign = np.where(h & 0x8000, -1.0, 1.0)
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    val = np.where(e == 0, m * 2.0 ** -24, (1024 + m) * np.exp2(e.astype(np.float64) - 25))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


# -- quantize ------------------------------------------------------------------
def quantize(x: np.ndarray):
    """x [rows, K] f32 -> (qs int8 [rows, K], d16 uint16 [rows, K/32], ssum int16 [rows, K/32])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, K = x.shape
    assert K % QK == 0, "K must be a multiple of 32"
    assert np.all(np.isfinite(x)), "oracle inputs must be finite"
    qs = np.empty((rows, K), dtype=np.int8)
    d16 = np.empty((rows, K // QK), dtype=np.uint16)
    ssum = np.empty((rows, K // QK), dtype=np.int16)
    lib().q8o_quantize_rows(x.ctypes.data, rows, K, qs.ctypes.data, d16.ctypes.data, ssum.ctypes.data)
    return qs, d16, ssum


def pack_sd(d16: np.ndarray, ssum: np.ndarray) -> np.ndarray:
    d16 = _c(d16, np.uint16)
    ssum = _c(ssum, np.int16)
    out = np.empty(d16.shape, dtype=np.uint32)
    lib().q8o_pack_sd(d16.ctypes.data, ssum.ctypes.data, d16.size, out.ctypes.data)
    return out


def unpack_sd(sd: np.ndarray):
    sd = np.asarray(sd, dtype=np.uint32)
    return (sd & 0xFFFF).astype(np.uint16), (sd >> 16).astype(np.uint16).view(np.int16)


def plane_sizes(T: int, K: int):
    """(qs bytes, scale-word count) of a PLANE64 activation for T tokens of width K."""
    ntb = (T + 63) // 64
    nchunk = K // QK
    return ntb * nchunk * 2048, ntb * nchunk * 64


def plane_qs_offset(t: int, k: int, K: int) -> int:
    return lib().q8o_plane_qs_offset(t, k, K)


def plane_sd_index(t: int, c: int, K: int) -> int:
    return lib().q8o_plane_sd_index(t, c, K)


def encode_plane64(qs, d16, ssum, T: int, K: int):
    qs = _c(qs, np.int8)
    d16 = _c(d16, np.uint16)
    ssum = _c(ssum, np.int16)
    nq, ns = plane_sizes(T, K)
    pqs = np.empty(nq, dtype=np.int8)
    psd = np.empty(ns, dtype=np.uint32)
    lib().q8o_encode_plane64(qs.ctypes.data, d16.ctypes.data, ssum.ctypes.data, T, K, pqs.ctypes.data,
                             psd.ctypes.data)
    return pqs, psd


def decode_plane64(pqs, psd, T: int, K: int):
    """-> (qs, d16, ssum, tail_nonzero_count)."""
    pqs = _c(pqs, np.int8).reshape(-1)
    psd = _c(psd, np.uint32).reshape(-1)
    nq, ns = plane_sizes(T, K)
    assert pqs.size == nq and psd.size == ns
    qs = np.empty((T, K), dtype=np.int8)
    d16 = np.empty((T, K // QK), dtype=np.uint16)
    ssum = np.empty((T, K // QK), dtype=np.int16)
    bad = lib().q8o_decode_plane64(pqs.ctypes.data, psd.ctypes.data, T, K, qs.ctypes.data, d16.ctypes.data,
                                   ssum.ctypes.data)
    return qs, d16, ssum, int(bad)


# -- producers -------------------------------------------------------------------
def rmsnorm_f64(x, w, eps: float) -> np.ndarray:
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, K = x.shape
    assert w.size == K
    y = np.empty((rows, K), dtype=np.float64)
    lib().q8o_rmsnorm_f64(x.ctypes.data, w.ctypes.data, rows, K, eps, y.ctypes.data)
    return y


def swiglu_f64(g, u) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    assert g.shape == u.shape
    y = np.empty(g.shape, dtype=np.float64)
    lib().q8o_swiglu_f64(g.ctypes.data, u.ctypes.data, g.size, y.ctypes.data)
    return y


# -- weights -----------------------------------------------------------------------
def quantize_weights_gguf(w) -> np.ndarray:
    """f32 [N, K] -> GGUF Q8_0 blocks, uint8 [N, K/32 * 34]."""
    w = _c(w, np.float32)
    N, K = w.shape
    assert K % QK == 0
    assert np.all(np.isfinite(w))
    blocks = np.empty((N, K // QK * 34), dtype=np.uint8)
    lib().q8o_quantize_weights_gguf(w.ctypes.data, N, K, blocks.ctypes.data)
    return blocks


def gguf_to_planar(blocks, N: int, K: int):
    blocks = _c(blocks, np.uint8)
    assert blocks.size == N * (K // QK) * 34
    qs = np.empty((N, K), dtype=np.int8)
    d = np.empty((N, K // QK), dtype=np.uint16)
    lib().q8o_gguf_to_planar(blocks.ctypes.data, N, K, qs.ctypes.data, d.ctypes.data)
    return qs, d


# -- dot products --------------------------------------------------------------------
def dot_pairs(wq, wd, aq, ad, pt, pn):
    """Reference (f64) and norm for output cells (pt[i], pn[i]); activations [T, K]."""
    wq = _c(wq, np.int8)
    wd = _c(wd, np.uint16)
    aq = _c(aq, np.int8)
    ad = _c(ad, np.uint16)
    if aq.ndim == 1:
        aq = aq.reshape(1, -1)
        ad = ad.reshape(1, -1)
    N, K = wq.shape
    T = aq.shape[0]
    pt = _c(pt, np.int64)
    pn = _c(pn, np.int64)
    assert pt.shape == pn.shape
    assert np.all((pt >= 0) & (pt < T)) and np.all((pn >= 0) & (pn < N))
    ref = np.empty(pt.size, dtype=np.float64)
    norm = np.empty(pt.size, dtype=np.float64)
    lib().q8o_dot_pairs(wq.ctypes.data, wd.ctypes.data, N, K, aq.ctypes.data, ad.ctypes.data, T, pt.ctypes.data,
                        pn.ctypes.data, pt.size, ref.ctypes.data, norm.ctypes.data)
    return ref, norm


def gemv(wq, wd, aq, ad):
    """y_ref [N], norm [N] for one activation row."""
    N = wq.shape[0]
    pn = np.arange(N, dtype=np.int64)
    return dot_pairs(wq, wd, aq, ad, np.zeros(N, dtype=np.int64), pn)


def gemm(wq, wd, aq, ad):
    """C_ref [T, N], norm [T, N]."""
    wq = _c(wq, np.int8)
    wd = _c(wd, np.uint16)
    aq = _c(aq, np.int8)
    ad = _c(ad, np.uint16)
    N, K = wq.shape
    T = aq.shape[0]
    ref = np.empty((T, N), dtype=np.float64)
    norm = np.empty((T, N), dtype=np.float64)
    lib().q8o_gemm_full(wq.ctypes.data, wd.ctypes.data, N, K, aq.ctypes.data, ad.ctypes.data, T, ref.ctypes.data,
                        norm.ctypes.data)
    return ref, norm


def block_isums(wq, aq) -> np.ndarray:
    """Exact int32 per-block sums [T, N, K/32]."""
    wq = _c(wq, np.int8)
    aq = _c(aq, np.int8)
    if aq.ndim == 1:
        aq = aq.reshape(1, -1)
    N, K = wq.shape
    T = aq.shape[0]
    out = np.empty((T, N, K // QK), dtype=np.int32)
    lib().q8o_block_isums(wq.ctypes.data, N, K, aq.ctypes.data, T, out.ctypes.data)
    return out


# -- q4_K weights --------------------------------------------------------------------
Q4K_BLOCK = 144   # bytes per 256-value super-block
Q4K_VALUES = 256


def q4k_scale_min(scale_bytes, s: int):
    """(sc, m) of sub-block s from the 12 packed scale bytes."""
    b = _c(np.asarray(scale_bytes, dtype=np.uint8).reshape(12), np.uint8)
    sc, m = ctypes.c_int(), ctypes.c_int()
    lib().q4ko_scale_min(b.ctypes.data, s, ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def q4k_decode(blocks, N: int, K: int):
    """nib [N,K] u8, d and dmin [N,K/256] f16 bits, sc and m [N,K/32] u8."""
    blocks = _c(blocks, np.uint8)
    assert blocks.size == N * (K // Q4K_VALUES) * Q4K_BLOCK
    nib = np.empty((N, K), np.uint8)
    d = np.empty((N, K // Q4K_VALUES), np.uint16)
    dmin = np.empty_like(d)
    sc = np.empty((N, K // QK), np.uint8)
    mn = np.empty_like(sc)
    lib().q4ko_decode(blocks.ctypes.data, N, K, nib.ctypes.data, d.ctypes.data, dmin.ctypes.data, sc.ctypes.data,
                      mn.ctypes.data)
    return nib, d, dmin, sc, mn


def q4k_dequant(blocks, N: int, K: int) -> np.ndarray:
    """Element values [N, K] in f64."""
    blocks = _c(blocks, np.uint8)
    w = np.empty((N, K), np.float64)
    lib().q4ko_dequant_f64(blocks.ctypes.data, N, K, w.ctypes.data)
    return w


def _q4k_args(blocks, N, K, aq, ad, assum):
    blocks = _c(blocks, np.uint8)
    assert blocks.size == N * (K // Q4K_VALUES) * Q4K_BLOCK
    aq, ad, assum = _c(aq, np.int8), _c(ad, np.uint16), _c(assum, np.int16)
    if aq.ndim == 1:
        aq, ad, assum = aq.reshape(1, -1), ad.reshape(1, -1), assum.reshape(1, -1)
    return blocks, aq, ad, assum


def q4k_dot_pairs(blocks, N, K, aq, ad, assum, pt, pn):
    """Reference (f64) and norm of cells (pt[i], pn[i]) for q4_K weights and q8_0 activations."""
    blocks, aq, ad, assum = _q4k_args(blocks, N, K, aq, ad, assum)
    T = aq.shape[0]
    pt, pn = _c(pt, np.int64), _c(pn, np.int64)
    assert np.all((pt >= 0) & (pt < T)) and np.all((pn >= 0) & (pn < N))
    ref = np.empty(pt.size, np.float64)
    norm = np.empty(pt.size, np.float64)
    lib().q4ko_dot_pairs(blocks.ctypes.data, N, K, aq.ctypes.data, ad.ctypes.data, assum.ctypes.data, T,
                         pt.ctypes.data, pn.ctypes.data, pt.size, ref.ctypes.data, norm.ctypes.data)
    return ref, norm


def q4k_gemm(blocks, N, K, aq, ad, assum):
    """C_ref [T, N] and norm [T, N] for q4_K weights and q8_0 activations."""
    blocks, aq, ad, assum = _q4k_args(blocks, N, K, aq, ad, assum)
    T = aq.shape[0]
    ref = np.empty((T, N), np.float64)
    norm = np.empty((T, N), np.float64)
    lib().q4ko_gemm_full(blocks.ctypes.data, N, K, aq.ctypes.data, ad.ctypes.data, assum.ctypes.data, T,
                         ref.ctypes.data, norm.ctypes.data)
    return ref, norm
