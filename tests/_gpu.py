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


def assert_rel(y, ref, tol=1e-5, what=""):
    """|y - ref| <= tol |ref| elementwise (y exactly 0 where ref is 0)."""
    y = np.asarray(y, dtype=np.float64)
    bad = ~(np.abs(y - ref) <= tol * np.abs(ref))
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
