"""Launch economy of the projection path ([P1] section 3: a tiny kernel's cost is
its launch count; section 5: count launches and check the count against the
model's structure): the library's launch counters, and HIP graph capture of the
per-token decode sequence.

Every count below is predicted from the structure of the computation before
anything runs, and the measured counters must equal it exactly:
- the unfused decode layer (H=7168) is rmsnorm_quant, a grouped GEMV over the
  four attention/gate consumers, two single GEMVs, q8_quantize and q8_gemv: 6;
- the grouped layer is rmsnorm_quant, one grouped GEMV over the six K=7168
  consumers and q8_gemv_f32 for the K=128 consumer: 3;
- the paired layer is rmsnorm_quant and q8_gemv_shared_multi_plus_f32, both
  GEMVs in one launch: 2;
- the one-launch layer is rmsnorm_quant_gemv_shared_multi_plus_f32: 1;
- the savings are therefore exactly 3, 4 and 5 launches per layer, and all four
  forms give identical outputs.
Launches captured into a graph count once, at capture; replays count nothing
and reproduce the eager results bit for bit, with eager work and
synchronizations between the replays.
"""
import numpy as np
import pytest

import synth
from _gpu import ensure_built, up, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
ensure_built()
from int8_quantized_projections_amd import q8lib  # noqa: E402

ROW, PLANE = q8lib.LAYOUT_ROW, q8lib.LAYOUT_PLANE64
EPS = synth.EPS
WL = "decode_h7168"
H = 7168
GROUP = ["Wq", "Wk", "Wv", "Wg", "W12288", "W96"]
LAYERS = 4


def counts():
    return {k: v for k, v in q8lib.launch_counts().items() if v}


@pytest.fixture(scope="module")
def decode():
    ws = {n: weights(synth.tensor(WL, n))[0] for n in GROUP + ["W128"]}
    x = up(synth.tensor(WL, "x").reshape(1, H))
    w = up(synth.tensor(WL, "w_norm"))
    x128 = up(synth.tensor(WL, "x128"))
    return ws, x, w, x128


class Buffers:
    def __init__(self, ws):
        self.y = torch.empty((1, H), device="cuda")
        self.aq, self.asd = q8lib.alloc_act(1, H, ROW)
        self.bq, self.bsd = q8lib.alloc_act(1, 128, ROW)
        self.out = {n: torch.full((ws[n].n,), float("nan"), device="cuda") for n in ws}

    def outputs(self):
        return [self.out[n].clone() for n in GROUP + ["W128"]]


def fused_layer(ws, x, w, x128, B):
    q8lib.rmsnorm_quant(x, w, EPS, ROW, B.y, B.aq, B.asd)
    q8lib.q8_gemv_shared_multi([ws[n] for n in GROUP], B.aq, B.asd, [B.out[n] for n in GROUP])
    q8lib.q8_gemv_f32(ws["W128"], x128, B.out["W128"])


def paired_layer(ws, x, w, x128, B):
    q8lib.rmsnorm_quant(x, w, EPS, ROW, B.y, B.aq, B.asd)
    q8lib.q8_gemv_shared_multi_plus_f32([ws[n] for n in GROUP], B.aq, B.asd, ws["W128"], x128,
                                        [B.out[n] for n in GROUP], B.out["W128"])


def step_layer(ws, x, w, x128, B):
    q8lib.rmsnorm_quant_gemv_shared_multi_plus_f32(x, w, EPS, [ws[n] for n in GROUP], ws["W128"], x128, B.y, B.aq,
                                                   B.asd, [B.out[n] for n in GROUP], B.out["W128"])


def unfused_layer(ws, x, w, x128, B):
    q8lib.rmsnorm_quant(x, w, EPS, ROW, B.y, B.aq, B.asd)
    q8lib.q8_gemv_shared_multi([ws[n] for n in GROUP[:4]], B.aq, B.asd, [B.out[n] for n in GROUP[:4]])
    q8lib.q8_gemv(ws["W12288"], B.aq, B.asd, B.out["W12288"])
    q8lib.q8_gemv(ws["W96"], B.aq, B.asd, B.out["W96"])
    q8lib.q8_quantize(x128.view(1, 128), ROW, B.bq, B.bsd)
    q8lib.q8_gemv(ws["W128"], B.bq, B.bsd, B.out["W128"])


FUSED = {"rmsnorm_quant": 1, "q8_gemv_shared_multi": 1, "q8_gemv_f32": 1}
PAIRED = {"rmsnorm_quant": 1, "q8_gemv_shared_multi_plus_f32": 1}
STEP = {"rmsnorm_quant_gemv_shared_multi_plus_f32": 1}
UNFUSED = {"rmsnorm_quant": 1, "q8_gemv_shared_multi": 1, "q8_gemv": 3, "q8_quantize": 1}


def test_decode_launch_counts_match_model_arithmetic(decode):
    ws, x, w, x128 = decode
    Bf, Bp, Bs, Bu = Buffers(ws), Buffers(ws), Buffers(ws), Buffers(ws)
    torch.cuda.synchronize()
    measured = {}
    for name, layer, B in (("fused", fused_layer, Bf), ("paired", paired_layer, Bp), ("step", step_layer, Bs),
                           ("unfused", unfused_layer, Bu)):
        q8lib.launch_counts_reset()
        for _ in range(LAYERS):
            layer(ws, x, w, x128, B)
        measured[name] = counts()
    torch.cuda.synchronize()
    assert measured["fused"] == {k: LAYERS * v for k, v in FUSED.items()}
    assert measured["paired"] == {k: LAYERS * v for k, v in PAIRED.items()}
    assert measured["step"] == {k: LAYERS * v for k, v in STEP.items()}
    assert measured["unfused"] == {k: LAYERS * v for k, v in UNFUSED.items()}
    # the predicted savings, as counts: 3, 4 and 5 launches per layer
    total = {k: sum(v.values()) for k, v in measured.items()}
    assert total["unfused"] - total["fused"] == 3 * LAYERS
    assert total["unfused"] - total["paired"] == 4 * LAYERS
    assert total["unfused"] - total["step"] == 5 * LAYERS
    for a, b, c, d, n in zip(Bf.outputs(), Bp.outputs(), Bs.outputs(), Bu.outputs(), GROUP + ["W128"]):
        assert not torch.isnan(a).any(), n
        assert torch.equal(a, b) and torch.equal(a, c) and torch.equal(a, d), f"{n}: the layer forms differ"
    assert torch.equal(Bs.y, Bp.y) and torch.equal(Bs.aq, Bp.aq) and torch.equal(Bs.asd, Bp.asd)


def test_graph_capture_counts_once_and_replays_match_eager(decode):
    ws, x, w, x128 = decode
    # eager reference of the captured inputs
    Be = Buffers(ws)
    paired_layer(ws, x, w, x128, Be)
    ref = Be.outputs()
    # other inputs for the eager work between replays
    x2 = up(synth.normal((1, H), stream=7301))
    x128b = up(synth.normal((128,), stream=7302))
    Bo = Buffers(ws)
    Bg = Buffers(ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    q8lib.launch_counts_reset()
    with torch.cuda.graph(g):
        paired_layer(ws, x, w, x128, Bg)
    assert counts() == PAIRED, "capture records each launch once"
    for i in range(3):
        paired_layer(ws, x2, w, x128b, Bo)  # eager work between replays
        torch.cuda.synchronize()
        for t in Bg.out.values():
            t.fill_(float("nan"))
        Bg.aq.fill_(0x55)
        g.replay()
        torch.cuda.synchronize()
        for a, b, n in zip(Bg.outputs(), ref, GROUP + ["W128"]):
            assert torch.equal(a, b), f"replay {i}: {n} differs from the eager result"
        assert torch.equal(Bg.aq, Be.aq) and torch.equal(Bg.asd, Be.asd), f"replay {i}: activation differs"
    # replays add nothing; the three eager layers add theirs
    assert counts() == {k: 4 * v for k, v in PAIRED.items()}
    # the eager layers on the other inputs computed something else
    assert not torch.equal(Bo.out["Wq"], ref[0])


def test_prefill_slices_launch_counts():
    """Per layer: rmsnorm_quant + one grouped q/k/v GEMM (2); swiglu_quant in plane-only
    mode + the down GEMM (2); rmsnorm_quant + two q4_K GEMMs (3)."""
    T, d, nf, nkv = 130, 256, 512, 128
    x = up(synth.normal((T, d), stream=7310))
    wn = up(np.ones(d, np.float32))
    Wq, Wk, Wv = (weights(synth.normal((n, d), stream=7311 + i, std=0.02))[0] for i, n in enumerate((d, nkv, nkv)))
    Wd = weights(synth.normal((d, nf), stream=7314, std=0.02))[0]
    gate = up(synth.normal((T, nf), stream=7315))
    upv = up(synth.normal((T, nf), stream=7316))
    Wg4 = q8lib.Q4KWeights(up(np.ascontiguousarray(synth.q4k_blocks(nf, d, 7317))), d)
    Wu4 = q8lib.Q4KWeights(up(np.ascontiguousarray(synth.q4k_blocks(nf, d, 7318))), d)
    pq, ps = q8lib.alloc_act(T, d, PLANE)
    gq, gs = q8lib.alloc_act(T, nf, PLANE)
    torch.cuda.synchronize()
    q8lib.launch_counts_reset()
    for _ in range(LAYERS):
        q8lib.rmsnorm_quant(x, wn, EPS, PLANE, None, pq, ps, f32=False)
        q8lib.q8_gemm_shared_multi([Wq, Wk, Wv], pq, ps, T)
        q8lib.swiglu_quant(gate, upv, PLANE, None, gq, gs, f32=False)
        q8lib.q8_gemm(Wd, gq, gs, T)
        q8lib.rmsnorm_quant(x, wn, EPS, PLANE, None, pq, ps, f32=False)
        q8lib.q4k_gemm(Wg4, pq, ps, T)
        q8lib.q4k_gemm(Wu4, pq, ps, T)
    torch.cuda.synchronize()
    assert counts() == {"rmsnorm_quant": 2 * LAYERS, "q8_gemm_shared_multi": LAYERS, "swiglu_quant": LAYERS,
                        "q8_gemm": LAYERS, "q4k_gemm": 2 * LAYERS}
