"""GPU parity of q8_gemm against the oracle, cell by cell.

The A operand is the oracle's PLANE64 encoding of its own quantization of a
seeded activation. Bars: every output cell within 1e-5 of the oracle's f64
value relative to its norm; cells outside [0,T) x [0,N) never written (the
output is poisoned with NaN, so a zero cell or a stray write shows); exact
bits on the power-of-two-scale special case.
"""
import numpy as np
import pytest

import oracle
import synth
from _gpu import assert_norm, ensure_built, plane_act, poisoned, row_act, to_np, up, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
ensure_built()
from int8_quantized_projections_amd import q8lib  # noqa: E402


def run_gemm(W, pq, ps, T, ldc=None, rows=None):
    ldc = ldc or W.n
    rows = rows or T
    C = poisoned(rows * ldc, torch.float32, 0xFF).view(rows, ldc)
    q8lib.q8_gemm(W, pq, ps, T, C, ldc)
    return C


# T around the 64-token groups, N around the 128-row tiles, K around the 8-block stages
CASES = [(1, 1, 32), (2, 5, 64), (15, 127, 256), (16, 128, 288), (63, 129, 640), (64, 300, 3584),
         (65, 33, 96), (129, 256, 1024), (130, 130, 2080)]


@pytest.mark.parametrize("T,N,K", CASES)
def test_gemm_matches_oracle_every_cell(T, N, K):
    x = synth.normal((T, K), stream=5000 + T)
    Wf = synth.normal((N, K), stream=5001 + N, std=0.02)
    W, wq, wd = weights(Wf)
    pq, ps, qo, do, _ = plane_act(x)
    ldc = N + 3
    C = run_gemm(W, pq, ps, T, ldc=ldc, rows=T + 2)
    torch.cuda.synchronize()
    ref, norm = oracle.gemm(wq, wd, qo, do)
    Cn = to_np(C)
    assert_norm(Cn[:T, :N], ref, norm, 1e-5, f"gemm {T}x{N}x{K}")
    # nothing outside the T x N block was written
    assert np.all(np.isnan(Cn[:T, N:])) and np.all(np.isnan(Cn[T:, :]))


@pytest.mark.parametrize("T,N,K", [(70, 129, 18944), (64, 128, 3584), (3, 200, 640)])
def test_gemm_exact_power_of_two_scales(T, N, K):
    h = int(oracle.f32_to_f16_bits(np.float32(2.0 ** -6)).reshape(-1)[0])
    aq = synth.uniform_i8((T, K), stream=5100, lo=-15, hi=15)
    wq = synth.uniform_i8((N, K), stream=5101, lo=-15, hi=15)
    ad = np.full((T, K // 32), h, np.uint16)
    ssum = aq.reshape(T, -1, 32).sum(axis=2).astype(np.int16)
    pq, psd = oracle.encode_plane64(aq, ad, ssum, T, K)
    W = q8lib.Q8Weights(up(wq), up(np.full((N, K // 32), h, np.uint16).view(np.int16)))
    C = run_gemm(W, up(pq), up(psd.view(np.int32)), T)
    torch.cuda.synchronize()
    exact = (aq.astype(np.int64) @ wq.astype(np.int64).T).astype(np.float64) * 2.0 ** -12
    assert np.array_equal(to_np(C).astype(np.float64), exact)


def test_gemm_single_token_matches_gemv():
    K, N = 3584, 500
    x = synth.normal((1, K), stream=5200)
    W, wq, wd = weights(synth.normal((N, K), stream=5201, std=0.02))
    pq, ps, qo, do, _ = plane_act(x)
    aq, asd, *_ = row_act(x)
    C = run_gemm(W, pq, ps, 1)
    y = q8lib.q8_gemv(W, aq, asd)
    torch.cuda.synchronize()
    ref, norm = oracle.gemv(wq, wd, qo[0], do[0])
    assert_norm(to_np(C)[0], ref, norm, 1e-5, "gemm T=1")
    assert_norm(to_np(y), to_np(C)[0].astype(np.float64), norm, 2e-6, "gemv vs gemm")


def test_gemm_on_fused_producer_plane_matches_standalone():
    """rmsnorm_quant's plane and q8_quantize's plane of the same y drive identical GEMMs."""
    T, K, N = 130, 3584, 256
    x = synth.normal((T, K), stream=5300)
    w = synth.normal((K,), stream=5301, mean=1.0, std=0.1)
    W, _, _ = weights(synth.normal((N, K), stream=5302, std=0.02))
    y, pq, ps = q8lib.rmsnorm_quant(up(x), up(w), 1e-6, q8lib.LAYOUT_PLANE64)
    pq2, ps2 = q8lib.q8_quantize(y, q8lib.LAYOUT_PLANE64)
    C1 = run_gemm(W, pq, ps, T)
    C2 = run_gemm(W, pq2, ps2, T)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_gemm_deterministic():
    T, K, N = 200, 2048, 384
    x = synth.normal((T, K), stream=5400)
    W, _, _ = weights(synth.normal((N, K), stream=5401, std=0.02))
    pq, ps, *_ = plane_act(x)
    a = run_gemm(W, pq, ps, T)
    b = run_gemm(W, pq, ps, T)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("K", [3584, 2080])
def test_gemm_scale_plane_two_byte_aligned(K):
    """A weight-scale plane that is only 2-byte aligned (allowed by the interface)
    takes the per-lane scale loads instead of the 4-byte pair copies; the two
    forms give identical bits."""
    T, N = 130, 200
    x = synth.normal((T, K), stream=5500)
    W, wq, wd = weights(synth.normal((N, K), stream=5501, std=0.02))
    pq, ps, qo, do, _ = plane_act(x)
    buf = torch.empty(W.d.numel() + 1, dtype=torch.int16, device=W.d.device)
    buf[1:] = W.d.reshape(-1)
    W2 = q8lib.Q8Weights(W.qs, buf[1:].view(W.d.shape))  # data pointer = 2 mod 4
    assert W2.d.data_ptr() % 4 == 2
    C1 = run_gemm(W, pq, ps, T)
    C2 = run_gemm(W2, pq, ps, T)
    torch.cuda.synchronize()
    ref, norm = oracle.gemm(wq, wd, qo, do)
    assert_norm(to_np(C2), ref, norm, 1e-5, f"gemm 2-byte-aligned scales K={K}")
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("T,K,Ns", [(130, 3584, (3584, 512, 512)), (65, 288, (129, 1, 300, 0, 128)),
                                    (64, 640, (40, 257, 128, 1, 3, 200, 64, 130))])
def test_gemm_shared_multi_matches_separate_and_oracle(T, K, Ns):
    """One grouped launch over several weight matrices equals the separate launches bit for bit, and
    the oracle within the tolerance (members of any N, including 0; K/32 odd takes the register
    form of the weight scales)."""
    x = synth.normal((T, K), stream=5600 + K)
    pq, ps, qo, do, _ = plane_act(x)
    Ws, ref = [], []
    for i, n in enumerate(Ns):
        W, wq, wd = weights(synth.normal((max(n, 1), K), stream=5700 + i, std=0.02))
        if n == 0:
            W = q8lib.Q8Weights(W.qs[:0], W.d[:0])
        Ws.append(W)
        ref.append((wq[:n], wd[:n]))
    ldcs = [n + 5 for n in Ns]
    grouped = [poisoned((T + 1) * ld, torch.float32, 0xFF).view(T + 1, ld) for ld in ldcs]
    q8lib.q8_gemm_shared_multi(Ws, pq, ps, T, grouped, ldcs)
    separate = [run_gemm(W, pq, ps, T, ldc=ld, rows=T + 1) for W, ld in zip(Ws, ldcs)]
    torch.cuda.synchronize()
    for i, n in enumerate(Ns):
        g, sep = to_np(grouped[i]), to_np(separate[i])
        assert np.array_equal(g[:T, :n].view(np.uint32), sep[:T, :n].view(np.uint32)), f"member {i} N={n}"
        assert np.all(np.isnan(g[:T, n:])) and np.all(np.isnan(g[T:, :])), f"member {i}: stray writes"
        if n:
            r, norm = oracle.gemm(ref[i][0], ref[i][1], qo, do)
            assert_norm(g[:T, :n], r, norm, 1e-5, f"grouped member {i} N={n}")


@pytest.mark.parametrize("T", [130, 97])
def test_gemm_half_tile_form_bit_identical_to_full_tiles(T):
    """A launch of at most 128 64-token tiles runs one workgroup per 32-token half of a tile, a larger
    one a workgroup per tile: the same matrix computed both ways (alone, and grouped with a wide
    member that makes the grid large) gives the same bits, and matches the oracle."""
    K = 640
    x = synth.normal((T, K), stream=5900 + T)
    pq, ps, qo, do, _ = plane_act(x)
    small, wq, wd = weights(synth.normal((200, K), stream=5901, std=0.02))
    wide, _, _ = weights(synth.normal((8192, K), stream=5902, std=0.02))
    alone = run_gemm(small, pq, ps, T, ldc=203, rows=T + 1)  # 2 x 3 tiles: halves
    grouped = [poisoned((T + 1) * 203, torch.float32, 0xFF).view(T + 1, 203),
               poisoned(T * 8192, torch.float32, 0xFF).view(T, 8192)]
    q8lib.q8_gemm_shared_multi([small, wide], pq, ps, T, grouped, [203, 8192])  # 66 x 3 tiles: whole tiles
    torch.cuda.synchronize()
    a, g = to_np(alone), to_np(grouped[0])
    assert np.array_equal(a[:T, :200].view(np.uint32), g[:T, :200].view(np.uint32))
    assert np.all(np.isnan(a[:T, 200:])) and np.all(np.isnan(a[T:, :]))
    ref, norm = oracle.gemm(wq, wd, qo, do)
    assert_norm(a[:T, :200], ref, norm, 1e-5, f"gemm half-tile form {T}x200x{K}")
