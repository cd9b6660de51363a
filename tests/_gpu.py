"""Helpers for the GPU parity tests: uploads, oracle-built inputs, checks."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def ensure_built():
    from int8_quantized_projections_amd import _build
    import synth

    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    if not os.path.exists(synth.LIB_PATH):
        synth.build()


def dev():
    import torch
    return torch.device("cuda:0")


def up(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def poisoned(n, dtype, byte=0x5A):
    """A device buffer whose bytes are all `byte` (so unwritten bytes show)."""
    import torch
    t = torch.empty(n, dtype=dtype, device=dev())
    t.view(torch.uint8).fill_(byte)
    return t


def weights(Wf):
    """f32 weights -> (device Q8Weights via the library's repack, oracle planes (qs, d))."""
    from int8_quantized_projections_amd import q8lib
    N, K = Wf.shape
    blocks = oracle.quantize_weights_gguf(Wf)
    W = q8lib.q8_weights_repack(up(blocks.reshape(-1)), N, K)
    wq, wd = oracle.gguf_to_planar(blocks, N, K)
    return W, wq, wd


def row_act(x):
    """Oracle quantization of x [T, K] as ROW buffers on the device, plus the oracle values."""
    qs, d16, ssum = oracle.quantize(x)
    return up(qs.reshape(-1)), up(oracle.pack_sd(d16, ssum).view(np.int32).reshape(-1)), qs, d16, ssum


def plane_act(x):
    """Oracle quantization of x [T, K] encoded as a PLANE64 activation on the device."""
    T, K = x.shape
    qs, d16, ssum = oracle.quantize(x)
    pq, psd = oracle.encode_plane64(qs, d16, ssum, T, K)
    return up(pq), up(psd.view(np.int32)), qs, d16, ssum


def to_np(t):
    return t.detach().cpu().numpy()


FLT_MIN = 2.0 ** -126  # the smallest normal f32


def assert_rel(y, ref, tol=1e-5, what="", floor=0.0):
    """|y - ref| <= tol |ref| + floor elementwise (floor: a scalar or an array of ref's shape;
    with floor 0, y exactly 0 where ref is 0). The producers' f32 outputs use floor = FLT_MIN
    (RMSNorm) and FLT_MIN * |up| + 2^-149 (SwiGLU): below f32's normal range only an absolute
    bound holds."""
    y = np.asarray(y, dtype=np.float64)
    bad = ~(np.abs(y - ref) <= tol * np.abs(ref) + floor)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements off, e.g. idx {i}: {y.reshape(-1)[i]} vs {ref.reshape(-1)[i]}")


def assert_norm(y, ref, norm, tol=1e-5, what=""):
    """max |y - ref| / norm <= tol (y exactly 0 where norm is 0), NaN-safe."""
    y = np.asarray(y, dtype=np.float64)
    ok = np.abs(y - ref) <= tol * norm
    if not ok.all():
        i = np.flatnonzero(~ok.reshape(-1))[:5]
        raise AssertionError(f"{what}: {(~ok).sum()} outputs off, e.g. idx {i}: {y.reshape(-1)[i]} vs "
                             f"{ref.reshape(-1)[i]} (norm {norm.reshape(-1)[i]})")


def divide_blocks_f32():
    """[n, 32] f32: blocks [amax, x, 0, ...] on which the IEEE quotient x/d and a reciprocal
    multiply round to different integers (tests/golden/quantize_divide_blocks.json)."""
    import json

    with open(os.path.join(ROOT, "tests", "golden", "quantize_divide_blocks.json")) as f:
        pairs = json.load(f)["blocks"]
    x = np.zeros((len(pairs), 32), np.uint32)
    for i, (a, b) in enumerate(pairs):
        x[i, 0], x[i, 1] = int(a, 16), int(b, 16)
    return x.view(np.float32)


def check_row_exact(qs, sd, x, what):
    """The device ROW activation (qs, sd) equals the oracle's quantize of the f32 array x, bit for bit."""
    x = np.asarray(x, np.float32)
    qo, do, so = oracle.quantize(x)
    assert np.array_equal(to_np(qs).reshape(qo.shape), qo), f"{what}: qs differ ({np.sum(to_np(qs).reshape(qo.shape) != qo)})"
    sdo = oracle.pack_sd(do, so).view(np.int32)
    assert np.array_equal(to_np(sd).reshape(sdo.shape), sdo), f"{what}: scale words differ"


def check_plane_exact(qs, sd, x, what):
    """The device PLANE64 activation equals the oracle's quantize of x [T, K], encoded by the
    oracle's plane layout (zero tail included), bit for bit."""
    x = np.asarray(x, np.float32)
    T, K = x.shape
    qo, do, so = oracle.quantize(x)
    pq, psd = oracle.encode_plane64(qo, do, so, T, K)
    gq, gsd = to_np(qs), to_np(sd).view(np.uint32)
    assert np.array_equal(gq, pq), f"{what}: plane qs bytes differ ({np.sum(gq != pq)} bytes)"
    assert np.array_equal(gsd, psd), f"{what}: plane scale words differ ({np.sum(gsd != psd)})"


def check_act_exact(qs, sd, x, layout, what):
    """check_row_exact (layout 0, ROW) or check_plane_exact (layout 1, PLANE64)."""
    x = np.asarray(x, np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    (check_row_exact if layout == 0 else check_plane_exact)(qs, sd, x, what)
