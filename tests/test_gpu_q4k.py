"""GPU parity of q4k_gemm (q4_K weights x PLANE64 q8_0 activation) against the oracle.

The weights are seeded raw q4_K bytes; the activation is the oracle's PLANE64
encoding of its own quantization of a seeded activation; every expected value
is the oracle's. Bars: every cell within 1e-5 of the oracle's f64 value
relative to its norm (sum of |scale term| + |min term|); cells outside
[0,T) x [0,N) never written; exact bits on the power-of-two-scale case (which
pins the int32 sub-block sums and the ssum min term through the timed kernel).
"""
import numpy as np
import pytest

import oracle
import synth
from _gpu import assert_norm, ensure_built, plane_act, poisoned, to_np, up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
ensure_built()
from int8_quantized_projections_amd import q8lib  # noqa: E402


def dev_weights(blocks, K):
    return q8lib.Q4KWeights(up(np.ascontiguousarray(blocks)), K)


def run(W, pq, ps, T, ldc=None, rows=None):
    ldc = ldc or W.n
    rows = rows or T
    C = poisoned(rows * ldc, torch.float32, 0xFF).view(rows, ldc)
    q8lib.q4k_gemm(W, pq, ps, T, C, ldc)
    return C


# T around the 64-token groups, N around the 128-row tiles, K over 1..14 super-blocks
CASES = [(1, 1, 256), (2, 5, 512), (63, 129, 512), (64, 128, 256), (65, 300, 768), (130, 130, 2048),
         (200, 64, 3584), (17, 257, 1280)]


@pytest.mark.parametrize("T,N,K", CASES)
def test_q4k_gemm_matches_oracle_every_cell(T, N, K):
    blocks = synth.q4k_blocks(N, K, 6100 + N)
    x = synth.normal((T, K), stream=6101 + T)
    pq, ps, qo, do, so = plane_act(x)
    ldc = N + 3
    C = run(dev_weights(blocks, K), pq, ps, T, ldc=ldc, rows=T + 2)
    torch.cuda.synchronize()
    ref, norm = oracle.q4k_gemm(blocks, N, K, qo, do, so)
    Cn = to_np(C)
    assert_norm(Cn[:T, :N], ref, norm, 1e-5, f"q4k_gemm {T}x{N}x{K}")
    assert np.all(np.isnan(Cn[:T, N:])) and np.all(np.isnan(Cn[T:, :]))


@pytest.mark.parametrize("T,N,K", [(70, 129, 512), (64, 128, 256), (3, 200, 512)])
def test_q4k_gemm_exact_power_of_two_scales(T, N, K):
    """d = 2^-10, dmin = 2^-8, activation scale 2^-6 with |q| <= 15: every product and every f32
    partial sum is an exact multiple of 2^-16 below 2^8, so the output equals the oracle exactly."""
    blocks = synth.q4k_blocks(N, K, 6200).reshape(N, K // 256, 144).copy()
    blocks[:, :, 0:2] = [0x00, 0x14]  # d = 2^-10
    blocks[:, :, 2:4] = [0x00, 0x1C]  # dmin = 2^-8
    blocks = blocks.reshape(N, -1)
    h = int(oracle.f32_to_f16_bits(np.float32(2.0 ** -6)).reshape(-1)[0])
    aq = synth.uniform_i8((T, K), stream=6201, lo=-15, hi=15)
    ad = np.full((T, K // 32), h, np.uint16)
    ssum = aq.reshape(T, -1, 32).sum(axis=2).astype(np.int16)
    pq, psd = oracle.encode_plane64(aq, ad, ssum, T, K)
    C = run(dev_weights(blocks, K), up(pq), up(psd.view(np.int32)), T)
    torch.cuda.synchronize()
    ref, norm = oracle.q4k_gemm(blocks, N, K, aq, ad, ssum)
    assert np.array_equal(to_np(C).astype(np.float64), ref)


def test_q4k_gemm_min_term_only():
    """All value nibbles zero: only the ssum min term remains."""
    T, N, K = 66, 130, 512
    blocks = synth.q4k_blocks(N, K, 6300).reshape(N, K // 256, 144).copy()
    blocks[:, :, 16:] = 0
    blocks = blocks.reshape(N, -1)
    x = synth.normal((T, K), stream=6301)
    pq, ps, qo, do, so = plane_act(x)
    C = run(dev_weights(blocks, K), pq, ps, T)
    torch.cuda.synchronize()
    ref, norm = oracle.q4k_gemm(blocks, N, K, qo, do, so)
    assert_norm(to_np(C), ref, norm, 1e-5, "q4k min term only")


def test_q4k_gemm_deterministic():
    T, N, K = 200, 384, 2048
    blocks = synth.q4k_blocks(N, K, 6400)
    pq, ps, *_ = plane_act(synth.normal((T, K), stream=6401))
    W = dev_weights(blocks, K)
    a = run(W, pq, ps, T)
    b = run(W, pq, ps, T)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_q8_gemm_takes_q4k_weights_by_format():
    """q8_gemm with a q8_weights descriptor of format Q8_WEIGHTS_Q4_K runs the q4_K GEMM: the
    same bits as q4k_gemm, counted under q8_gemm, and the oracle's values."""
    T, N, K = 130, 300, 1024
    blocks = synth.q4k_blocks(N, K, 6400)
    pq, ps, qo, do, so = plane_act(synth.normal((T, K), stream=6401))
    W = dev_weights(blocks, K)
    ref_c = run(W, pq, ps, T)
    C = poisoned(T * N, torch.float32, 0xFF).view(T, N)
    torch.cuda.synchronize()
    q8lib.launch_counts_reset()
    q8lib.q8_gemm(W, pq, ps, T, C)
    torch.cuda.synchronize()
    assert {k: v for k, v in q8lib.launch_counts().items() if v} == {"q8_gemm": 1}
    assert torch.equal(C.view(torch.int32), ref_c.view(torch.int32))
    ref, norm = oracle.q4k_gemm(blocks, N, K, qo, do, so)
    assert_norm(to_np(C), ref, norm, 1e-5, "q8_gemm with q4_K weights")
