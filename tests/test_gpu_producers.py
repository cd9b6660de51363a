"""GPU parity of the producers against the oracle: q8_quantize, rmsnorm_quant,
swiglu_quant (ROW and PLANE64), and the weight repack.

Bars: quantized planes bit-exact with the oracle's quantize of the same f32
input; producer f32 outputs within 1e-5 relative of the oracle's f64 value;
fused planes bit-identical to the standalone quantize of the f32 output the
same call wrote; padded plane tails zero on poisoned buffers.
"""
import numpy as np
import pytest

import oracle
import synth
from _gpu import (FLT_MIN, assert_rel, check_act_exact, check_plane_exact, check_row_exact, dev, divide_blocks_f32,
                  ensure_built, poisoned, to_np, up, weights)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
ensure_built()
from int8_quantized_projections_amd import q8lib  # noqa: E402

ROW, PLANE = q8lib.LAYOUT_ROW, q8lib.LAYOUT_PLANE64


def quantize_dev(x_dev, rows, K, layout):
    nq, ns = q8lib.act_bytes(rows, K, layout)
    qs = poisoned(nq, torch.int8)
    sd = poisoned(ns // 4, torch.int32)
    q8lib.q8_quantize(x_dev, layout, qs, sd)
    return qs, sd


def test_repack_matches_oracle_planes():
    for N, K in ((5, 64), (97, 2080), (3, 32)):
        Wf = synth.normal((N, K), stream=3000 + N, std=0.02)
        W, wq, wd = weights(Wf)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(W.qs), wq)
        assert np.array_equal(to_np(W.d).view(np.uint16), wd)


@pytest.mark.parametrize("rows,K", [(1, 32), (1, 128), (3, 2048), (7, 640), (5, 2080), (2, 7168), (4, 18944)])
def test_quantize_row_bit_exact(rows, K):
    x = synth.normal((rows, K), stream=3100 + K)
    qs, sd = quantize_dev(up(x), rows, K, ROW)
    torch.cuda.synchronize()
    check_row_exact(qs, sd, x, f"q8_quantize ROW {rows}x{K}")


@pytest.mark.parametrize("T,K", [(1, 32), (63, 96), (64, 640), (65, 896), (129, 256), (130, 3584)])
def test_quantize_plane64_bit_exact_and_tail(T, K):
    x = synth.normal((T, K), stream=3200 + T)
    qs, sd = quantize_dev(up(x), T, K, PLANE)
    torch.cuda.synchronize()
    check_plane_exact(qs, sd, x, f"q8_quantize PLANE64 {T}x{K}")


@pytest.mark.parametrize("T,K", [(2000, 16480), (2048, 16384), (1250, 12320)])
def test_quantize_plane64_wide_bit_exact_and_tail(T, K):
    """Wide activations (1024 or more work items of 16 rows x 32 chunks) take the
    4 KB-run kernel: a ragged last group and a partial last 32-chunk column,
    and an exact fit, bit-exact with the oracle on poisoned buffers."""
    x = synth.normal((T, K), stream=3290 + T)
    qs, sd = quantize_dev(up(x), T, K, PLANE)
    torch.cuda.synchronize()
    check_plane_exact(qs, sd, x, f"q8_quantize PLANE64 {T}x{K}")
    # the same plane from the fused producer's path (k_elementwise writes it for swiglu_quant
    # with an f32 output; the plane-only swiglu_quant takes the run order)
    u = np.ones_like(x)
    y, q2, s2 = q8lib.swiglu_quant(up(x), up(u), PLANE)
    q3, s3 = quantize_dev(y, T, K, PLANE)
    nq, ns = q8lib.act_bytes(T, K, PLANE)
    q4, s4 = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
    q8lib.swiglu_quant(up(x), up(u), PLANE, None, q4, s4, f32=False)
    torch.cuda.synchronize()
    check_plane_exact(q2, s2, to_np(y), f"swiglu_quant PLANE64 {T}x{K} vs the oracle's quantize of its y")
    assert torch.equal(q2, q3) and torch.equal(s2, s3), "run-order plane differs from the fused producer's"
    assert torch.equal(q2, q4) and torch.equal(s2, s4), "plane-only swiglu_quant differs from the fused one"


def test_quantize_edge_values_bit_exact():
    """Ties, near-ties, zero blocks, f16-subnormal scales, f32-subnormal inputs."""
    rng = np.random.default_rng(7)
    blocks = []
    # exact half-integers on a power-of-two scale (ties to even decide)
    for k in (-8, 0, 3):
        m = rng.integers(-126, 127, size=32) + 0.5
        m[0] = 127.0
        blocks.append(m * 2.0 ** k)
    # values one f32 ulp either side of half-integers
    base = (rng.integers(-120, 121, size=32) + 0.5).astype(np.float32)
    base[0] = 127.0
    blocks.append(np.nextafter(base, np.float32(np.inf)))
    blocks.append(np.nextafter(base, np.float32(-np.inf)))
    # zero block, single nonzero, negative amax
    blocks.append(np.zeros(32))
    z = np.zeros(32)
    z[17] = -3.0
    blocks.append(z)
    # tiny scales: f16-subnormal d, f32-subnormal d, amax/127 underflowing to zero
    for scale in (1e-6, 1e-38, 1e-42, 1e-45):
        blocks.append(rng.standard_normal(32) * scale)
    # random blocks at many magnitudes
    for e in range(-30, 16, 3):
        blocks.append(rng.standard_normal(32) * 2.0 ** e)
    x = np.concatenate(blocks).astype(np.float32)
    x = np.concatenate([x, np.zeros((-x.size) % 256, np.float32)]).reshape(1, -1)
    qs, sd = quantize_dev(up(x), 1, x.shape[1], ROW)
    torch.cuda.synchronize()
    check_row_exact(qs, sd, x, "edge values")


@pytest.mark.parametrize("layout", [ROW, PLANE])
def test_quantize_ieee_division_blocks(layout):
    """Blocks on which rint of the correctly rounded quotient x/d and rint of x times the
    rounded reciprocal 1/d differ: the q8_quantize kernels, and the fused SwiGLU producer on an
    input whose y is exactly those values (gate 32 makes silu(gate) exactly 32 in f32, and up =
    x/32 is exact), match the oracle bit for bit."""
    blocks = divide_blocks_f32()
    for x in (blocks.reshape(1, -1), blocks):  # one row of several blocks; several one-block rows
        rows, K = x.shape
        qs, sd = quantize_dev(up(x), rows, K, layout)
        g = np.full_like(x, 32.0)
        u = (x / np.float32(32.0)).astype(np.float32)
        assert np.array_equal(u * np.float32(32.0), x)
        y, fq, fsd = q8lib.swiglu_quant(up(g), up(u), layout)
        nq, ns = q8lib.act_bytes(rows, K, layout)
        pq, psd = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
        q8lib.swiglu_quant(up(g), up(u), layout, None, pq, psd, f32=False)
        torch.cuda.synchronize()
        check_act_exact(qs, sd, x, layout, f"q8_quantize divide blocks {rows}x{K}")
        assert np.array_equal(to_np(y), x), "swiglu_quant: y is not exactly 32 * up"
        check_act_exact(fq, fsd, x, layout, f"swiglu_quant divide blocks {rows}x{K}")
        check_act_exact(pq, psd, x, layout, f"plane-only swiglu_quant divide blocks {rows}x{K}")


@pytest.mark.parametrize("layout", [ROW, PLANE])
def test_quantize_amax_sweep_bit_exact(layout):
    """The block maximum swept over f32's whole range (65,536 bit patterns from the smallest
    subnormal to the largest finite value, so the scale d = amax/127 takes every exponent:
    f32-subnormal, f16-subnormal, ordinary and f16-overflowing), each block's other 31 values a
    random fraction of it: bit-exact with the oracle (the division by 127, the reciprocal path
    and its IEEE fallback, the f16 rounding of d)."""
    rng = np.random.default_rng(4242)
    n = 65536
    bits = rng.integers(1, 0x7F7FFFFF, size=n, dtype=np.uint32)
    # and the ends of each range: the smallest subnormals, the subnormal/normal boundary,
    # the largest finite value
    bits[:6] = [0x00000001, 0x00000002, 0x007FFFFF, 0x00800000, 0x00800001, 0x7F7FFFFF]
    amax = np.sort(bits).view(np.float32)
    frac = rng.uniform(-1.0, 1.0, size=(n, 32))
    x = (amax[:, None].astype(np.float64) * frac).astype(np.float32)
    pos = rng.integers(0, 32, size=n)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    x[np.arange(n), pos] = amax * sign
    assert np.all(np.abs(x).max(axis=1) == amax)
    x = x.reshape(2048, 1024)
    qs, sd = quantize_dev(up(x), 2048, 1024, layout)
    torch.cuda.synchronize()
    check_act_exact(qs, sd, x, layout, f"amax sweep layout {layout}")


def test_quantize_random_many_rows_bit_exact():
    x = synth.normal((333, 3584), stream=3300, std=3.0)
    qs, sd = quantize_dev(up(x), 333, 3584, ROW)
    pq, ps = quantize_dev(up(x), 333, 3584, PLANE)
    torch.cuda.synchronize()
    check_row_exact(qs, sd, x, "ROW 333x3584")
    check_plane_exact(pq, ps, x, "PLANE64 333x3584")


def test_quantize_zero_rows_is_noop_and_zero_row_is_zero_block():
    qs = poisoned(64, torch.int8)
    sd = poisoned(2, torch.int32)
    x = torch.zeros(64, device=dev())
    rc = q8lib.lib().q8_quantize(x.data_ptr(), 0, 64, ROW, qs.data_ptr(), sd.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == 0 and torch.all(qs.view(torch.uint8) == 0x5A) and torch.all(sd.view(torch.uint8) == 0x5A)
    q8lib.q8_quantize(x, ROW, qs, sd)
    torch.cuda.synchronize()
    assert torch.count_nonzero(qs) == 0 and torch.count_nonzero(sd) == 0


def report_plane_vs_reference(qs, sd, y_ref, layout, what):
    """Diagnostic only: how many blocks of the GPU's quantized output differ from the oracle's
    quantize of the f32 rounding of the oracle's own f64 reference (last-bit differences in y
    can move a block by one step). The bar is the exact check on the y the call wrote."""
    T, K = y_ref.shape
    gq, gsd = to_np(qs), to_np(sd).view(np.uint32)
    if layout == PLANE:
        q, d16, s, bad = oracle.decode_plane64(gq, gsd, T, K)
        assert bad == 0, f"{what}: padded tail not zero"
    else:
        q = gq.reshape(T, K)
        d16, s = oracle.unpack_sd(gsd.reshape(T, K // 32))
    qo, do, so = oracle.quantize(y_ref.astype(np.float32))
    blk_diff = np.any(q.reshape(T, -1, 32) != qo.reshape(T, -1, 32), axis=2) | (d16 != do)
    print(f"{what}: {blk_diff.sum()} of {blk_diff.size} blocks differ from the quantize of the f32-rounded "
          f"f64 reference (max step {np.abs(q.astype(int) - qo.astype(int)).max()})")


def _rms_case(rows, K, layout, stream):
    x = synth.normal((rows, K), stream=stream)
    w = synth.normal((K,), stream=stream + 1, mean=1.0, std=0.1)
    nq, ns = q8lib.act_bytes(rows, K, layout)
    qs, sd = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
    y = poisoned(rows * K, torch.float32).view(rows, K)
    q8lib.rmsnorm_quant(up(x), up(w), 1e-6, layout, y, qs, sd)
    y2 = poisoned(rows * K, torch.float32).view(rows, K)
    q8lib.rmsnorm_quant(up(x), up(w), 1e-6, layout, y2, quant=False)
    q2, s2 = quantize_dev(y, rows, K, layout)
    # plane only (y = NULL): nothing but the quantized output is written
    q3, s3 = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
    q8lib.rmsnorm_quant(up(x), up(w), 1e-6, layout, None, q3, s3, f32=False)
    torch.cuda.synchronize()
    assert torch.equal(qs, q3) and torch.equal(sd, s3), "plane-only call differs from the call that writes y"
    return x, w, y, qs, sd, y2, q2, s2


# rows <= 16 run one 1024-thread workgroup per row (K/4 > 8192 float4: the two-pass form), more rows 4 or 2
# waves per row; from 1024 rows, PLANE64 with 4 or 8 float4 per lane (K in (1024, 4096]) takes the form
# with the plane staged in LDS: up to 4096 padded rows dealt evenly to 512 workgroups (even counts of 2 to
# 8 rows, runs that cross 64-token groups; 1027 and 1030 rows: ragged, padded to 1088; 2049 rows: 2112,
# 4 or 6 rows per workgroup; 2500 rows: 2560; 4033 rows: 4096, 8 rows each), beyond that 8 rows per
# workgroup (4097 rows)
@pytest.mark.parametrize("rows,K,layout", [(1, 7168, ROW), (1, 3584, ROW), (3, 640, ROW), (70, 896, PLANE),
                                           (130, 3584, PLANE), (64, 256, PLANE), (3, 9216, ROW), (65, 18944, PLANE),
                                           (2, 40960, ROW), (16, 2048, PLANE), (17, 2048, PLANE), (1, 32, ROW),
                                           (1027, 2048, PLANE), (1030, 2080, PLANE), (1100, 4096, PLANE),
                                           (1025, 992, PLANE), (1024, 4128, PLANE), (1027, 3584, ROW),
                                           (2049, 2048, PLANE), (2500, 4096, PLANE), (4033, 1056, PLANE),
                                           (4097, 2048, PLANE)])
def test_rmsnorm_quant(rows, K, layout):
    x, w, y, qs, sd, y2, q2, s2 = _rms_case(rows, K, layout, 3400 + K + rows)
    ref = oracle.rmsnorm_f64(x, w, 1e-6)
    assert_rel(to_np(y), ref, 1e-5, f"rmsnorm y {rows}x{K}")
    # fused quantize == standalone quantize of the y this call wrote (bit for bit)
    assert torch.equal(qs, q2) and torch.equal(sd, s2), "fused plane differs from q8_quantize(y)"
    # the f32-only call writes the same y bits
    assert torch.equal(y, y2), "f32-only call differs"
    # the quantized output is the oracle's quantize of the y the same call wrote, bit for bit
    check_act_exact(qs, sd, to_np(y), layout, f"rmsnorm_quant {rows}x{K}")
    report_plane_vs_reference(qs, sd, ref, layout, f"rmsnorm quant {rows}x{K}")


def _swiglu_case(rows, K, layout, stream):
    g = synth.normal((rows, K), stream=stream)
    u = synth.normal((rows, K), stream=stream + 1)
    nq, ns = q8lib.act_bytes(rows, K, layout)
    qs, sd = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
    y = poisoned(rows * K, torch.float32).view(rows, K)
    q8lib.swiglu_quant(up(g), up(u), layout, y, qs, sd)
    y2 = poisoned(rows * K, torch.float32).view(rows, K)
    q8lib.swiglu_quant(up(g), up(u), layout, y2, quant=False)
    q2, s2 = quantize_dev(y, rows, K, layout)
    q3, s3 = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
    q8lib.swiglu_quant(up(g), up(u), layout, None, q3, s3, f32=False)
    torch.cuda.synchronize()
    assert torch.equal(qs, q3) and torch.equal(sd, s3), "plane-only call differs from the call that writes y"
    return g, u, y, qs, sd, y2, q2, s2


@pytest.mark.parametrize("rows,K,layout", [(1, 128, ROW), (3, 640, ROW), (63, 896, PLANE), (64, 18944, PLANE),
                                           (129, 2048, PLANE), (17, 96, ROW)])
def test_swiglu_quant(rows, K, layout):
    g, u, y, qs, sd, y2, q2, s2 = _swiglu_case(rows, K, layout, 3500 + K + rows)
    ref = oracle.swiglu_f64(g, u)
    assert_rel(to_np(y), ref, 1e-5, f"swiglu y {rows}x{K}")
    assert torch.equal(qs, q2) and torch.equal(sd, s2), "fused plane differs from q8_quantize(y)"
    assert torch.equal(y, y2), "f32-only call differs"
    check_act_exact(qs, sd, to_np(y), layout, f"swiglu_quant {rows}x{K}")
    report_plane_vs_reference(qs, sd, ref, layout, f"swiglu quant {rows}x{K}")


def test_swiglu_closed_form_points():
    g = np.zeros((1, 32), np.float32)
    u = np.ones((1, 32), np.float32)
    g[0, 1] = 40.0
    u[0, 2] = 0.0
    g[0, 2] = 3.0
    y, _, _ = q8lib.swiglu_quant(up(g), up(u), ROW, quant=False)
    torch.cuda.synchronize()
    yv = to_np(y)[0]
    assert yv[0] == 0.0 and yv[2] == 0.0
    assert abs(yv[1] - 40.0) <= 1e-5 * 40.0


# Gate values across f32's range: silu(g) underflows below about -87.3 (the old e^-g form
# overflowed there), its f32 value turns denormal, then zero; large positive g gives g.
DOMAIN_GATES = [-3e38, -1e30, -1e4, -200.0, -110.0, -104.0, -103.0, -100.0, -97.0, -95.0, -92.0, -90.0, -89.0,
                -88.72, -88.7, -88.0, -87.4, -87.3, -87.0, -86.0, -80.0, -40.0, -20.0, -1.0, -1e-30, -1e-40, -0.0,
                0.0, 1e-40, 1e-30, 1.0, 20.0, 40.0, 87.5, 88.0, 89.0, 100.0, 1e4, 1e30, 3e38]


@pytest.mark.parametrize("layout", [ROW, PLANE])
def test_swiglu_input_domain(layout):
    """SwiGLU over the whole finite f32 range of the gate, with |up| from 3e-30 to 1e20 (each
    pair chosen so that |y| stays below f32's maximum): y within 1e-5 relative of the oracle's
    f64 value plus FLT_MIN * |up| + 2^-149 absolute (silu(g) itself is only held to FLT_MIN once
    it leaves f32's normal range, and a product below that range rounds to f32's denormal
    step), and the plane bit-exact with the oracle's quantize of that y."""
    gates = np.array(DOMAIN_GATES, np.float32)
    rows = []
    for u in (1.0, -2.5, 1e20, 3e-30):
        g = np.where(np.abs(gates.astype(np.float64) * u) < 1e38, gates, np.float32(0.0))
        rows.append((g, np.full(g.size, u, np.float32)))
    K = 64
    g = np.zeros((len(rows), K), np.float32)
    u = np.zeros((len(rows), K), np.float32)
    for i, (gr, ur) in enumerate(rows):
        g[i, : gr.size], u[i, : ur.size] = gr, ur
    y, qs, sd = q8lib.swiglu_quant(up(g), up(u), layout)
    torch.cuda.synchronize()
    yg = to_np(y)
    assert np.all(np.isfinite(yg))
    ref = oracle.swiglu_f64(g, u)
    # silu(g) in f32 holds to FLT_MIN below the normal range; times up, plus the final rounding
    # of a product below f32's normal range (half its denormal step)
    assert_rel(yg, ref, 1e-5, "swiglu domain", floor=FLT_MIN * np.abs(u.astype(np.float64)) + 2.0 ** -149)
    check_act_exact(qs, sd, yg, layout, "swiglu domain plane")


def _domain_rows(K):
    """RMSNorm rows across f32's range: sums of squares that overflow f32 (the rescaled
    second pass), one huge element among normal ones, squares that underflow, denormal
    inputs, a zero row and an ordinary row."""
    rng = np.random.default_rng(K)
    sign = np.where(rng.integers(0, 2, K) == 0, -1.0, 1.0)
    rows = [
        sign * 3e38,                                             # every square overflows
        np.full(K, 2e19),                                        # x^2 = 4e38 overflows
        sign * np.exp2(rng.uniform(60, 127, K)),                 # 1e18 .. 1.7e38 mixed
        np.concatenate([[1e25], rng.standard_normal(K - 1)]),    # one huge element
        np.full(K, 1.7e19 / np.sqrt(K)) * sign,                  # the sum just below f32's maximum
        np.full(K, 1.95e19 / np.sqrt(K)) * sign,                 # and just above it
        sign * 1e-30,                                            # squares underflow: eps dominates
        sign * 1e-40,                                            # denormal inputs
        np.zeros(K),
        rng.standard_normal(K),
    ]
    return np.array(rows, np.float32)


@pytest.mark.parametrize("K,copies,layout", [(256, 1, ROW), (7168, 1, PLANE), (40960, 1, ROW), (256, 120, PLANE),
                                              (2048, 120, PLANE)])
def test_rmsnorm_input_domain(K, copies, layout):
    """RMSNorm over f32's range: y within 1e-5 relative of the oracle's f64 value plus FLT_MIN,
    the plane bit-exact with the oracle's quantize of that y, and rows with a finite sum of
    squares bit-identical to the same rows normalized among ordinary ones. copies > 1 gives
    1080 rows, two rows per workgroup (four or six with the plane staged, at K = 2048), so overflowing and
    ordinary rows share workgroups (the rows <= 16 and K = 40960 cases take the 16-wave and the
    two-pass forms)."""
    x = np.tile(_domain_rows(K), (copies, 1))
    w = synth.normal((K,), stream=3700 + K, mean=1.0, std=0.1)
    y, qs, sd = q8lib.rmsnorm_quant(up(x), up(w), 1e-6, layout)
    torch.cuda.synchronize()
    yg = to_np(y)
    assert np.all(np.isfinite(yg))
    ref = oracle.rmsnorm_f64(x, w, 1e-6)
    assert_rel(yg, ref, 1e-5, f"rmsnorm domain {x.shape}", floor=FLT_MIN)
    check_act_exact(qs, sd, yg, layout, f"rmsnorm domain plane {x.shape}")
    # rows whose f32 sum of squares is finite keep the first pass's bits
    finite = np.isfinite((x.astype(np.float32) ** 2).sum(axis=1, dtype=np.float32))
    plain = np.tile(synth.normal((1, K), stream=3701), (x.shape[0], 1))
    plain[finite] = x[finite]
    y2, _, _ = q8lib.rmsnorm_quant(up(plain), up(w), 1e-6, layout)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y2)[finite], yg[finite])


def test_producers_deterministic():
    a = _rms_case(130, 3584, PLANE, 3600)
    b = _rms_case(130, 3584, PLANE, 3600)
    assert torch.equal(a[2], b[2]) and torch.equal(a[3], b[3]) and torch.equal(a[4], b[4])


def test_rmsnorm_plane64_forms_bit_identical():
    """From 1024 rows, rmsnorm_quant PLANE64 deals up to 4096 padded rows evenly to the CUs and takes 8
    rows per workgroup beyond. Every row's bits depend on the row, K and the waves per row (two in both
    forms) only: the first rows of one input give the same y, quantized blocks and scales whether the
    call has 1100 or 3325 rows (balanced) or 4200 rows (8-row workgroups)."""
    K = 2048
    x = synth.normal((4200, K), stream=3810)
    w = synth.normal((K,), stream=3811, mean=1.0, std=0.1)
    out = {}
    for n in (4200, 3325, 1100):
        y, qs, sd = q8lib.rmsnorm_quant(up(x[:n]), up(w), 1e-6, PLANE)
        torch.cuda.synchronize()
        q, d16, s, bad = oracle.decode_plane64(to_np(qs), to_np(sd).view(np.uint32), n, K)
        assert bad == 0, f"{n} rows: padded tail not zero"
        out[n] = (to_np(y), q, d16, s)
    for n in (3325, 1100):
        for a, b, what in zip(out[n], out[4200], ("y", "qs", "d", "ssum")):
            assert np.array_equal(a.view(np.uint8) if a.dtype == np.float32 else a,
                                  (b[:n].view(np.uint8) if b.dtype == np.float32 else b[:n])), f"{n} rows: {what}"
