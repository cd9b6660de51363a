"""The one-launch decode step, rmsnorm_quant_gemv_shared_multi_plus_f32: rmsnorm_quant of one
row and the grouped + f32 GEMVs of its consumers in one launch, each grouped workgroup running
the producer into its own LDS ([P2] s2: the producer writes the quantized activation its
consumers read; [P1] s3: a launch at decode costs more than its bytes).

Bars:
- every output (y, the q8_0 activation, each grouped output, the f32 part) is bit-identical to
  rmsnorm_quant followed by q8_gemv_shared_multi_plus_f32;
- against the oracle, directly: y within 1e-5 of the oracle's f64 RMSNorm; the activation
  bit-exact with the oracle's quantize of the y the launch wrote; every grouped output within
  1e-5 of norm of the oracle's GEMV on that activation, and the f32 part likewise on the
  oracle's quantize of its own input;
- consecutive calls on different rows each give their own row's results;
- the one-launch form counts one launch; other shapes fall back to the two calls;
- graph replays reproduce the eager results, with eager calls and synchronizations between.
"""
import numpy as np
import pytest

import oracle
import synth
from _gpu import assert_norm, assert_rel, check_row_exact, ensure_built, poisoned, to_np, up, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
ensure_built()
from int8_quantized_projections_amd import q8lib  # noqa: E402

ROW = q8lib.LAYOUT_ROW
EPS = 1e-6
STEP = "rmsnorm_quant_gemv_shared_multi_plus_f32"

# (grouped N list, K, f32-part N, its K, one launch?)
CASES = [
    ([4096, 512, 512, 4096, 12288, 96], 7168, 4096, 128, True),  # the decode projection set
    ([300, 200], 3584, 100, 256, True),
    ([129], 2080, 33, 512, True),
    ([5, 0, 70], 4096, 7, 96, True),       # fewer rows than waves: most waves never wait
    ([1000, 24], 8192, 64, 128, True),     # the largest K of the one-launch form
    ([200, 3], 8224, 40, 128, False),      # one block past it: rmsnorm_quant, then the GEMVs
    ([77], 4128, 16, 128, True),
    ([64], 1024, 64, 128, False),          # K too narrow for the pair kernel: the two calls
    ([300], 3584, 0, 128, True),           # empty f32 part
    ([4000, 77], 3584, None, None, True),  # no f32 part (Wx = NULL), as for an LM head
    ([300], 1024, None, None, False),      # no f32 part, K too narrow: rmsnorm_quant + q8_gemv_shared_multi
    ([0, 0], 3584, 40, 128, False),        # empty grouped part
]


def _weights_or_empty(n, K, stream, planes=None):
    W, wq, wd = weights(synth.normal((max(n, 1), K), stream=stream, std=0.02))
    if planes is not None:
        planes.append((wq[:n], wd[:n]))
    return W if n else W.rows(0, 0)


def _inputs(Ns, K, Nx, Kx, base, planes=None):
    """Device weights (and, into `planes`, the oracle's planes of every member, then Wx's)."""
    Ws = [_weights_or_empty(n, K, base + 7 * i, planes) for i, n in enumerate(Ns)]
    Wx = _weights_or_empty(Nx, Kx, base + 50, planes) if Nx is not None else None
    w = synth.normal((K,), stream=base + 51, mean=1.0, std=0.1)
    return Ws, Wx, w


def _reference(x, w, Ws, Wx, x2):
    """rmsnorm_quant, then q8_gemv_shared_multi_plus_f32: the two-call form."""
    y, aq, asd = q8lib.rmsnorm_quant(x, w, EPS, ROW)
    if Wx is None:
        return y, aq, asd, q8lib.q8_gemv_shared_multi(Ws, aq, asd), None
    ys, yx = q8lib.q8_gemv_shared_multi_plus_f32(Ws, aq, asd, Wx, x2)
    return y, aq, asd, ys, yx


class Outs:
    def __init__(self, K, Ws, Wx):
        self.y = poisoned(K, torch.float32, 0xFF).view(1, K)
        nq, ns = q8lib.act_bytes(1, K, ROW)
        self.aq, self.asd = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
        self.ys = [poisoned(max(W.n, 1), torch.float32, 0xFF)[: W.n] for W in Ws]
        self.yx = poisoned(max(Wx.n, 1), torch.float32, 0xFF)[: Wx.n] if Wx is not None else None

    def step(self, x, w, Ws, Wx, x2):
        q8lib.rmsnorm_quant_gemv_shared_multi_plus_f32(x, w, EPS, Ws, Wx, x2, self.y, self.aq, self.asd, self.ys,
                                                       self.yx)

    def all(self):
        return [self.y, self.aq, self.asd, *self.ys] + ([self.yx] if self.yx is not None else [])


def _assert_same(got, ref, what):
    ref = [r for r in ref if r is not None]
    assert len(got) == len(ref)
    names = ["y", "a_qs", "a_sd"] + [f"y[{i}]" for i in range(len(got) - 3)]
    for g, r, n in zip(got, ref, names):
        assert torch.equal(g.reshape(-1).view(torch.int32 if g.dtype == torch.float32 else g.dtype),
                           r.reshape(-1).view(torch.int32 if r.dtype == torch.float32 else r.dtype)), \
            f"{what}: {n} differs from the two-call form"


@pytest.mark.parametrize("Ns,K,Nx,Kx,one", CASES)
def test_step_bit_identical_to_two_calls(Ns, K, Nx, Kx, one):
    planes = []
    Ws, Wx, wh = _inputs(Ns, K, Nx, Kx, 8100 + K + (Kx or 0), planes)
    w = up(wh)
    o = Outs(K, Ws, Wx)
    # three different rows in a row: each call must read its own row's activation
    for r in range(3):
        xh = synth.normal((1, K), stream=8200 + 3 * K + r)
        x2h = synth.normal((Kx,), stream=8300 + Kx + r) if Kx else None
        x, x2 = up(xh), (up(x2h) if Kx else None)
        ref = _reference(x, w, Ws, Wx, x2)
        torch.cuda.synchronize()
        q8lib.launch_counts_reset()
        o.step(x, w, Ws, Wx, x2)
        torch.cuda.synchronize()
        c = {k: v for k, v in q8lib.launch_counts().items() if v}
        if one:
            assert c == {STEP: 1}, c
        else:
            assert c.get(STEP, 0) == 0 and c["rmsnorm_quant"] == 1, c
        _assert_same(o.all(), [ref[0], ref[1], ref[2], *ref[3], ref[4]], f"{Ns}x{K} + {Nx}x{Kx}, row {r}")
        if r != 1:  # every output against the oracle (first and last row)
            y_gpu = to_np(o.y).reshape(1, K)
            assert_rel(y_gpu, oracle.rmsnorm_f64(xh, wh, EPS), 1e-5, f"rmsnorm 1x{K}")
            check_row_exact(o.aq, o.asd, y_gpu, f"step activation 1x{K} vs the oracle's quantize of its y")
            qa, da, _ = oracle.quantize(y_gpu)
            for i, (n, out) in enumerate(zip(Ns, o.ys)):
                wq, wd = planes[i]
                ref, norm = oracle.gemv(wq, wd, qa[0], da[0])
                assert_norm(to_np(out), ref, norm, 1e-5, f"step member {i} ({n}x{K}) vs the oracle")
            if Nx:
                wq, wd = planes[len(Ns)]
                qx, dx, _ = oracle.quantize(x2h.reshape(1, -1))
                ref, norm = oracle.gemv(wq, wd, qx[0], dx[0])
                assert_norm(to_np(o.yx), ref, norm, 1e-5, f"step f32 part ({Nx}x{Kx}) vs the oracle")


def test_step_without_f32_output():
    """y = NULL writes only the quantized activation and the GEMV outputs, with the same bits."""
    Ns, K, Nx, Kx = [4096, 512], 7168, 512, 128
    Ws, Wx, wh = _inputs(Ns, K, Nx, Kx, 8400)
    w = up(wh)
    x, x2 = up(synth.normal((1, K), stream=8401)), up(synth.normal((Kx,), stream=8402))
    a, b = Outs(K, Ws, Wx), Outs(K, Ws, Wx)
    a.step(x, w, Ws, Wx, x2)
    q8lib.rmsnorm_quant_gemv_shared_multi_plus_f32(x, w, EPS, Ws, Wx, x2, None, b.aq, b.asd, b.ys, b.yx, f32=False)
    torch.cuda.synchronize()
    assert torch.all(b.y.view(torch.int32) == -1), "y written although NULL was passed"
    for g, r in zip(b.all()[1:], a.all()[1:]):
        assert torch.equal(g, r)


def test_step_graph_replays_match_eager():
    Ns, K, Nx, Kx = [4096, 512, 512, 4096, 12288, 96], 7168, 4096, 128
    Ws, Wx, wh = _inputs(Ns, K, Nx, Kx, 8500)
    w = up(wh)
    x, x2 = up(synth.normal((1, K), stream=8501)), up(synth.normal((Kx,), stream=8502))
    xo, x2o = up(synth.normal((1, K), stream=8503)), up(synth.normal((Kx,), stream=8504))
    ref = _reference(x, w, Ws, Wx, x2)
    ref = [ref[0], ref[1], ref[2], *ref[3], ref[4]]
    g_out, e_out = Outs(K, Ws, Wx), Outs(K, Ws, Wx)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    q8lib.launch_counts_reset()
    with torch.cuda.graph(g):
        g_out.step(x, w, Ws, Wx, x2)
    assert {k: v for k, v in q8lib.launch_counts().items() if v} == {STEP: 1}
    for i in range(3):
        e_out.step(xo, w, Ws, Wx, x2o)  # eager work on other inputs between replays
        torch.cuda.synchronize()
        for t in g_out.all():
            t.view(torch.uint8).fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        _assert_same(g_out.all(), ref, f"replay {i}")
    assert not torch.equal(e_out.ys[0], ref[3])


def test_step_in_place_norm_runs_as_two_calls():
    """y = x (an in-place norm): the one launch would let one workgroup overwrite x while the
    others read it, so the call takes the two-call path, with the two calls' results."""
    Ns, K, Nx, Kx = [4096, 512], 7168, 512, 128
    Ws, Wx, wh = _inputs(Ns, K, Nx, Kx, 8600)
    w = up(wh)
    xh = synth.normal((1, K), stream=8601)
    x2 = up(synth.normal((Kx,), stream=8602))
    ref = _reference(up(xh), w, Ws, Wx, x2)
    xin = up(xh)
    o = Outs(K, Ws, Wx)
    torch.cuda.synchronize()
    q8lib.launch_counts_reset()
    q8lib.rmsnorm_quant_gemv_shared_multi_plus_f32(xin, w, EPS, Ws, Wx, x2, xin, o.aq, o.asd, o.ys, o.yx)
    torch.cuda.synchronize()
    c = {k: v for k, v in q8lib.launch_counts().items() if v}
    assert c.get(STEP, 0) == 0 and c["rmsnorm_quant"] == 1, c
    _assert_same([xin, o.aq, o.asd, *o.ys, o.yx], [ref[0], ref[1], ref[2], *ref[3], ref[4]], "in place")


def test_step_row_with_overflowing_sum_of_squares():
    """A row whose f32 sum of squares overflows takes the producer's rescaled second pass in
    every workgroup of the one launch: the same bits as the two calls, and y within 1e-5 of the
    oracle's f64 RMSNorm."""
    Ns, K, Nx, Kx = [300, 200], 3584, 100, 256
    planes = []
    Ws, Wx, wh = _inputs(Ns, K, Nx, Kx, 8700, planes)
    w = up(wh)
    rng = np.random.default_rng(8701)
    xh = (np.where(rng.integers(0, 2, K) == 0, -1.0, 1.0) * np.exp2(rng.uniform(60, 127, K))).astype(np.float32)
    xh = xh.reshape(1, K)
    x, x2 = up(xh), up(synth.normal((Kx,), stream=8702))
    ref = _reference(x, w, Ws, Wx, x2)
    o = Outs(K, Ws, Wx)
    o.step(x, w, Ws, Wx, x2)
    torch.cuda.synchronize()
    _assert_same(o.all(), [ref[0], ref[1], ref[2], *ref[3], ref[4]], "overflowing row")
    y_gpu = to_np(o.y).reshape(1, K)
    assert_rel(y_gpu, oracle.rmsnorm_f64(xh, wh, EPS), 1e-5, "rmsnorm of an overflowing row", floor=2.0 ** -126)
    check_row_exact(o.aq, o.asd, y_gpu, "activation of an overflowing row")
