"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

Only random numbers live here (see ``synth.c`` for the generator's
definition). The five workloads below give each tensor its shape,
distribution and stream id, after the shapes the three pages use:

* decode at batch 1 with hidden size 7168 (Fusion and the
  Activation-Quantization Discipline, sections 1-2: N=12288 K=7168, N=96,
  K=128 and the four consumers of one normed activation);
* prefill of a 7B-class model at 3325 tokens (r51 producer-fused A-quantize,
  section 2.2: d=3584, nf=18944);
* an LM head of vocabulary 152064 at width 3584.

The pages measured real models; these Gaussian tensors only take their shapes
(no dataset or trained weight is used).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
SRC_PATH = os.path.join(_HERE, "synth.c")

SEED = 0


def build() -> str:
    """Compile ``libsynth.so`` with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", SRC_PATH, "-o", LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_splitmix_at.argtypes = [u64, u64]
        L.synth_splitmix_at.restype = u64
        L.synth_bits.argtypes = [u64, u64, u64]
        L.synth_bits.restype = u64
        L.synth_unit.argtypes = [u64, u64, u64]
        L.synth_unit.restype = dbl
        L.synth_normal_f32.argtypes = [u64, u64, i64, i64, dbl, dbl, vp]
        L.synth_normal_f32.restype = None
        L.synth_uniform_f32.argtypes = [u64, u64, i64, i64, dbl, dbl, vp]
        L.synth_uniform_f32.restype = None
        L.synth_uniform_i8.argtypes = [u64, u64, i64, i64, ctypes.c_int, ctypes.c_int, vp]
        L.synth_uniform_i8.restype = None
        L.synth_bytes.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.synth_bytes.restype = None
        _lib = L
    return _lib


def normal(shape, stream: int, mean: float = 0.0, std: float = 1.0, seed: int = SEED, offset: int = 0,
           out: np.ndarray | None = None) -> np.ndarray:
    """f32 array of N(mean, std^2) draws, element i of the flattened array is index offset+i of the stream."""
    n = int(np.prod(shape))
    a = np.empty(n, dtype=np.float32) if out is None else out.reshape(-1)
    assert a.dtype == np.float32 and a.flags.c_contiguous and a.size == n
    lib().synth_normal_f32(seed, stream, offset, n, mean, std, a.ctypes.data)
    return a.reshape(shape)


def uniform(shape, stream: int, lo: float, hi: float, seed: int = SEED, offset: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    a = np.empty(n, dtype=np.float32)
    lib().synth_uniform_f32(seed, stream, offset, n, lo, hi, a.ctypes.data)
    return a.reshape(shape)


def uniform_i8(shape, stream: int, lo: int, hi: int, seed: int = SEED, offset: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    a = np.empty(n, dtype=np.int8)
    lib().synth_uniform_i8(seed, stream, offset, n, lo, hi, a.ctypes.data)
    return a.reshape(shape)


def random_bytes(n: int, stream: int, seed: int = SEED, offset: int = 0) -> np.ndarray:
    a = np.empty(n, dtype=np.uint8)
    lib().synth_bytes(seed, stream, offset, n, a.ctypes.data)
    return a


def q4k_blocks(N: int, K: int, stream: int, d_exp: int = 2, dmin_exp: int = 5, seed: int = SEED,
               row0: int = 0) -> np.ndarray:
    """q4_K weights [N, K/256 * 144] as raw bytes, rows row0 .. row0+N-1 of the stream: every byte is random
    except the two f16 fields of each 144-byte super-block, whose bit patterns get exponent field d_exp (d)
    and dmin_exp (dmin) with a random 10-bit fraction (d in [2^-13, 2^-12), dmin in [2^-10, 2^-9) by
    default). Any byte pattern is a valid block, so no encoding arithmetic is involved."""
    nsb = K // 256
    rowb = nsb * 144
    raw = random_bytes(N * rowb, stream, seed, offset=row0 * rowb).reshape(N, nsb, 144)
    d = raw[:, :, 0].astype(np.uint16) | ((raw[:, :, 1].astype(np.uint16) & 0x03) << 8) | (d_exp << 10)
    m = raw[:, :, 2].astype(np.uint16) | ((raw[:, :, 3].astype(np.uint16) & 0x03) << 8) | (dmin_exp << 10)
    raw[:, :, 0] = (d & 0xFF).astype(np.uint8)
    raw[:, :, 1] = (d >> 8).astype(np.uint8)
    raw[:, :, 2] = (m & 0xFF).astype(np.uint8)
    raw[:, :, 3] = (m >> 8).astype(np.uint8)
    return raw.reshape(N, rowb)


# ---------------------------------------------------------------------------
# Workloads. Stream ids are fixed per tensor so that any test or benchmark
# draws the same tensor for the same name.
# ---------------------------------------------------------------------------
W_STD = 0.02          # weights ~ N(0, 0.02)
NORM_W_MEAN, NORM_W_STD = 1.0, 0.1   # RMSNorm weight ~ N(1, 0.1)
EPS = 1e-6

WORKLOADS = {
    # 1: single Q8_0 GEMV at batch 1
    "gemv_2048": {
        "desc": "Single Q8_0 GEMV, batch 1: N=2048 K=2048",
        "tensors": {"W": ((2048, 2048), 101, 0.0, W_STD), "x": ((2048,), 102, 0.0, 1.0)},
    },
    # 2: decode projection set at H=7168
    "decode_h7168": {
        "desc": "Decode projection set, batch 1, H=7168: rmsnorm_quant shared by 4 GEMVs "
                "N=4096/512/512/4096, plus GEMVs N=12288 K=7168, N=96 K=7168, N=4096 K=128",
        "tensors": {
            "x": ((7168,), 201, 0.0, 1.0),
            "w_norm": ((7168,), 202, NORM_W_MEAN, NORM_W_STD),
            "Wq": ((4096, 7168), 203, 0.0, W_STD),
            "Wk": ((512, 7168), 204, 0.0, W_STD),
            "Wv": ((512, 7168), 205, 0.0, W_STD),
            "Wg": ((4096, 7168), 206, 0.0, W_STD),
            "W12288": ((12288, 7168), 207, 0.0, W_STD),
            "W96": ((96, 7168), 208, 0.0, W_STD),
            "W128": ((4096, 128), 209, 0.0, W_STD),
            "x128": ((128,), 210, 0.0, 1.0),
        },
    },
    # 3: prefill rms-class
    "prefill_rms": {
        "desc": "Prefill rms-class: T=3325 d=3584, rmsnorm_quant PLANE64 -> q8_gemm N=3584,512,512",
        "tensors": {
            "x": ((3325, 3584), 301, 0.0, 1.0),
            "w_norm": ((3584,), 302, NORM_W_MEAN, NORM_W_STD),
            "Wq": ((3584, 3584), 303, 0.0, W_STD),
            "Wk": ((512, 3584), 304, 0.0, W_STD),
            "Wv": ((512, 3584), 305, 0.0, W_STD),
        },
    },
    # 4: prefill swiglu-class
    "prefill_swiglu": {
        "desc": "Prefill swiglu-class: gate,up [3325 x 18944] -> swiglu_quant PLANE64 -> q8_gemm N=3584 K=18944",
        "tensors": {
            "gate": ((3325, 18944), 401, 0.0, 1.0),
            "up": ((3325, 18944), 402, 0.0, 1.0),
            "Wd": ((3584, 18944), 403, 0.0, W_STD),
        },
    },
    # 5: LM head
    "lm_head": {
        "desc": "LM head: vocab N=152064 K=3584, rmsnorm_quant + q8_gemv at T=1, q8_gemm at T=512",
        "tensors": {
            "W": ((152064, 3584), 501, 0.0, W_STD),
            "x1": ((1, 3584), 502, 0.0, 1.0),
            "x512": ((512, 3584), 503, 0.0, 1.0),
            "w_norm": ((3584,), 504, NORM_W_MEAN, NORM_W_STD),
        },
    },
}


# q4_K weight tensors (raw 144-byte super-blocks): (N, K), stream
Q4K_WEIGHTS = {
    # 6: prefill with q4_K weights: the rms-class plane (T=3325, d=3584) feeding the FFN gate and up
    #    projections N=18944 K=3584 (the q4_K GEMM the pages measure)
    "prefill_q4k": {"Wg": ((18944, 3584), 601), "Wu": ((18944, 3584), 602)},
}


def q4k_tensor(workload: str, name: str, rows: slice | None = None) -> np.ndarray:
    (N, K), stream = Q4K_WEIGHTS[workload][name]
    r0, r1 = (0, N) if rows is None else (rows.start or 0, N if rows.stop is None else rows.stop)
    return q4k_blocks(r1 - r0, K, stream, row0=r0)


def tensor(workload: str, name: str, rows: slice | None = None) -> np.ndarray:
    """Draw one workload tensor (optionally only a range of its leading rows)."""
    shape, stream, mean, std = WORKLOADS[workload]["tensors"][name]
    if rows is None:
        return normal(shape, stream, mean, std)
    start, stop, _ = rows.indices(shape[0])
    row_elems = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    sub = (stop - start,) + tuple(shape[1:])
    return normal(sub, stream, mean, std, offset=start * row_elems)
