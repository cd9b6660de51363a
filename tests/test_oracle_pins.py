"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the pages or the mathematics fix:
worked values, closed forms, invariants, special cases with an exact answer,
brute force on tiny inputs, or an independent library routine. Together
they are chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, round-half-away instead of
half-even, d = amax/128, a missing scale) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def page_numbers():
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# IEEE binary16 conversion
# ---------------------------------------------------------------------------
def test_f16_worked_values():
    # 1/127 = 0.00787401...: 2^-7 * 1.00787 -> fraction 8/1024 -> 0x2008
    assert oracle.f32_to_f16_bits(np.float32(1.0) / np.float32(127.0)) == 0x2008
    assert oracle.f32_to_f16_bits(np.float32(1.0)) == 0x3C00
    assert oracle.f32_to_f16_bits(np.float32(65504.0)) == 0x7BFF
    assert oracle.f32_to_f16_bits(np.float32(65520.0)) == 0x7C00  # halfway to 2^16 rounds to even -> inf
    assert oracle.f32_to_f16_bits(np.float32(2.0 ** -24)) == 0x0001  # smallest subnormal
    assert oracle.f32_to_f16_bits(np.float32(2.0 ** -25)) == 0x0000  # exact half of it: ties to even (0)
    assert oracle.f32_to_f16_bits(np.float32(3 * 2.0 ** -25)) == 0x0002  # 1.5 steps -> 2 (even)
    assert oracle.f32_to_f16_bits(np.float32(-0.0)) == 0x8000


def test_f16_conversion_exhaustive():
    """Every f32 bit pattern against the host's IEEE conversion (torch on x86 uses the F16C
    instruction), and every 64th pattern against numpy's float16 cast. NaNs: only NaN-ness."""
    import torch

    chunk = 1 << 24
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        f = bits.view(np.float32)
        ours = oracle.f32_to_f16_bits(f)
        ref = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        assert np.array_equal(ours[~nan], ref[~nan]), hex(start)
        assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x3FF) != 0)
        sub = f[::64]
        with np.errstate(over="ignore", invalid="ignore"):
            ref_np = sub.astype(np.float16).view(np.uint16)
        keep = ~np.isnan(sub)
        assert np.array_equal(ours[::64][keep], ref_np[keep]), hex(start)


def test_f16_decode_exhaustive_against_numpy():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    ours = oracle.f16_to_f64(h)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    dec32 = oracle.f16_bits_to_f32(h[fin][::97])
    assert np.array_equal(dec32.astype(np.float64), ref[fin][::97])


# ---------------------------------------------------------------------------
# Quantize: worked examples and invariants
# ---------------------------------------------------------------------------
def test_quantize_worked_block_ties_to_even():
    # amax = 127 gives d = 1 exactly (f16 0x3C00), so q = rint(x), half to even.
    x = np.zeros(32, dtype=np.float32)
    x[:8] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -1.5]
    qs, d16, ssum = oracle.quantize(x)
    assert d16[0, 0] == 0x3C00
    assert list(qs[0, :8]) == [127, 2, 4, -2, 0, 2, 0, -2]  # roundf would give 3, 4, -3, 1, 2, -1, -2
    assert ssum[0, 0] == 127 + 2 + 4 - 2 + 0 + 2 + 0 - 2
    assert np.all(qs[0, 8:] == 0)


def test_quantize_negative_amax_and_zero_block():
    x = np.zeros(64, dtype=np.float32)
    x[0] = -254.0
    x[1] = 127.0   # = 0.5 * 254 -> exactly 63.5 in units of d=2 -> 64 (even)
    x[2] = 1.0     # 0.5 -> 0
    qs, d16, ssum = oracle.quantize(x)
    assert d16[0, 0] == 0x4000  # d = 2
    assert list(qs[0, :3]) == [-127, 64, 0]
    assert d16[0, 1] == 0 and np.all(qs[0, 32:] == 0) and ssum[0, 1] == 0


def test_quantize_underflowing_scale_gives_zero_block():
    x = np.zeros(32, dtype=np.float32)
    x[5] = np.float32(1e-45)  # smallest subnormal: amax/127 underflows to 0
    qs, d16, ssum = oracle.quantize(x)
    assert d16[0, 0] == 0 and np.all(qs == 0) and ssum[0, 0] == 0


def _invariants(x, qs, d16, ssum):
    rows, K = x.shape
    nb = K // 32
    xb = x.reshape(rows, nb, 32).astype(np.float64)
    qb = qs.reshape(rows, nb, 32).astype(np.int64)
    amax = np.abs(xb).max(axis=2)
    d_true = amax / 127.0
    d16v = oracle.f16_to_f64(d16)
    # |q| <= 127 and the amax element reaches 127 whenever d is a normal f32
    assert np.abs(qb).max() <= 127
    normal = d_true >= 2.0 ** -126
    assert np.all(np.abs(qb).max(axis=2)[normal] == 127)
    # the stored d is the f16 rounding of amax/127 (relative 2^-11 for f16 normals)
    f16n = (d16v >= 2.0 ** -14) & np.isfinite(d16v)
    assert np.all(np.abs(d16v - d_true)[f16n] <= d_true[f16n] * (2.0 ** -11 + 2.0 ** -23))
    # ssum is the integer sum of the block's q
    assert np.array_equal(ssum.astype(np.int64), qb.sum(axis=2))
    # round trip with the exact d: |x - d q| <= d/2 (1 + 2^-16)
    err = np.abs(xb - d_true[..., None] * qb)
    assert np.all(err <= (d_true[..., None] / 2) * (1 + 2.0 ** -16) + 1e-300)
    # round trip with the stored f16 d: <= 0.5625 d_true (f16-normal d)
    err16 = np.abs(xb - d16v[..., None] * qb)
    assert np.all((err16 <= 0.5625 * d_true[..., None])[f16n])


@pytest.mark.parametrize("K,std", [(2048, 1.0), (3584, 1.0), (7168, 0.02), (640, 3.0)])
def test_quantize_invariants_random(K, std):
    x = synth.normal((37, K), stream=900 + K, std=std)
    qs, d16, ssum = oracle.quantize(x)
    _invariants(x, qs, d16, ssum)


def test_quantize_invariants_wide_dynamic_range():
    # blocks spanning many binades, including f16-subnormal scales
    x = synth.normal((16, 1024), stream=950)
    scale = np.exp2(np.repeat(np.arange(-40, 24, 2), 32)).astype(np.float32)  # the top blocks overflow f16 d
    x = (x * scale[: x.shape[1]]).astype(np.float32)
    qs, d16, ssum = oracle.quantize(x)
    _invariants(x, qs, d16, ssum)


def test_quantize_scale_and_sign_invariance():
    x = synth.normal((8, 512), stream=960)
    q0, d0, s0 = oracle.quantize(x)
    for k in (-6, -1, 3, 9):
        qk, dk, sk = oracle.quantize((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(qk, q0) and np.array_equal(sk, s0)
        assert np.array_equal(oracle.f16_to_f64(dk), oracle.f16_to_f64(d0) * 2.0 ** k)
    qn, dn, sn = oracle.quantize(-x)
    assert np.array_equal(qn, -q0) and np.array_equal(dn, d0) and np.array_equal(sn, -s0)


def test_quantize_is_nearest_integer_on_exact_scale_grid():
    # x = d * (m + f) with d a power of two: x/d is exact, so q must be the nearest
    # integer to m + f, ties to even -- checked against Python's round(), which is half-even.
    rng = np.random.default_rng(1)
    m = rng.integers(-120, 121, size=(64, 32))
    f = rng.choice([0.0, 0.25, 0.5, -0.5, 0.75, -0.25], size=(64, 32))
    v = (m + f).astype(np.float64)
    v[:, 0] = 127.0  # pin amax so that d = 1 * 2^k exactly
    for k in (-3, 0, 5):
        x = (v * 2.0 ** k).astype(np.float32).reshape(1, -1)
        qs, d16, _ = oracle.quantize(x)
        want = np.vectorize(lambda a: int(round(a)))(np.clip(v, -127, 127))
        assert np.array_equal(qs.reshape(64, 32).astype(np.int64), want)
        assert np.all(oracle.f16_to_f64(d16) == 2.0 ** k)


def divide_blocks():
    """(amax bits, x bits) of blocks [amax, x, 0, ...] on which the IEEE quotient and a
    reciprocal multiply round to different integers (tests/golden/quantize_divide_blocks.json)."""
    with open(os.path.join(GOLDEN, "quantize_divide_blocks.json")) as f:
        return [(int(a, 16), int(b, 16)) for a, b in json.load(f)["blocks"]]


DIVIDE_BLOCKS = divide_blocks()


def _bits_f32(b: int) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def _round_f32(r):
    """The binary32 value nearest to the rational r, ties to even, from the format's
    definition: 24 significant bits at or above 2^-126, a fixed step of 2^-149 below
    (the values here stay far from overflow)."""
    from fractions import Fraction

    if r == 0:
        return Fraction(0)
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (max(e, -126) - 23)
    m = round(a / step)  # Fraction.__round__ is half-even
    return (m * step) if r > 0 else -(m * step)


def _q_exact(amax_bits: int, x_bits: int):
    """(q with the IEEE divide, q with a reciprocal multiply) for value x of a block whose
    largest magnitude is amax: d = fl(amax/127), q = rint(fl(x/d)) ties to even, clamped."""
    from fractions import Fraction

    amax, x = Fraction(float(_bits_f32(amax_bits))), Fraction(float(_bits_f32(x_bits)))
    d = _round_f32(amax / 127)
    q_div = round(_round_f32(x / d))
    q_rcp = round(_round_f32(x * _round_f32(1 / d)))
    clamp = lambda q: max(-127, min(127, q))  # noqa: E731
    return clamp(q_div), clamp(q_rcp), d


def test_quantize_uses_ieee_division_not_reciprocal():
    """The quantize divides (q = rint(x/d) with the correctly rounded f32 quotient), as the
    activation-quantize definition states it; a multiply by the rounded reciprocal 1/d lands
    one step away on every block below, so an oracle that multiplied would fail here."""
    x = np.zeros((len(DIVIDE_BLOCKS), 32), np.float32)
    for i, (a, b) in enumerate(DIVIDE_BLOCKS):
        x[i, 0], x[i, 1] = _bits_f32(a), _bits_f32(b)
        assert abs(x[i, 1]) <= x[i, 0]
    qs, d16, ssum = oracle.quantize(x.reshape(1, -1))
    qs = qs.reshape(len(DIVIDE_BLOCKS), 32)
    for i, (a, b) in enumerate(DIVIDE_BLOCKS):
        q_div, q_rcp, d = _q_exact(a, b)
        assert q_div != q_rcp, "the block does not tell the two forms apart"
        q_amax, _, _ = _q_exact(a, a)
        assert q_amax == 127
        assert int(qs[i, 1]) == q_div, f"block {i}: q {qs[i, 1]}, exact divide {q_div}, reciprocal {q_rcp}"
        assert int(qs[i, 0]) == 127 and not qs[i, 2:].any()
        assert int(ssum[0, i]) == 127 + q_div
        # the stored scale is the f16 rounding of the same d
        assert oracle.f16_to_f64(d16[0, i]) == float(np.float16(float(d)))


# ---------------------------------------------------------------------------
# Layouts
# ---------------------------------------------------------------------------
def _last_digit(printed: float) -> float:
    """One unit in the last digit the page printed (e.g. 1.49 -> 0.01)."""
    txt = repr(printed)
    return 10.0 ** -(len(txt.split(".")[1]) if "." in txt else 0) + 1e-9


def test_plane_byte_counts_match_pages():
    pn = page_numbers()
    tile = pn["plane_tile"]
    for key in ("rms_class", "swiglu_class"):
        c = pn[key]
        K = c.get("d", c.get("nf"))
        T = c["T"]
        nq, ns = oracle.plane_sizes(T, K)
        assert K // 32 == c["nchunk"]
        assert nq == ((T + 63) // 64) * c["nchunk"] * tile["qs_bytes_per_group_chunk"]
        assert ns * 4 == ((T + 63) // 64) * c["nchunk"] * tile["scale_bytes_per_group_chunk"]
        assert abs(nq / 1e6 - c["qs_MB"]) <= _last_digit(c["qs_MB"])
        assert abs(ns * 4 / 1e6 - c["sda_MB"]) <= _last_digit(c["sda_MB"])
        assert abs(T * K * 4 / 1e6 - c["f32_MB"]) <= _last_digit(c["f32_MB"])
    assert pn["rms_class"]["ntb"] == (3325 + 63) // 64
    dw = pn["decode_weight"]
    assert round(dw["N"] * dw["K"] // 32 * pn["q8_0_block"]["block_bytes"] / 1e6) == dw["weight_MB"]
    lm = pn["lm_head"]
    assert abs(lm["N"] * lm["K"] // 32 * 34 / 1e9 - lm["weight_GB"]) < 0.005


def test_plane_tile_offsets_are_a_bijection():
    K = 96
    seen = np.zeros(oracle.plane_sizes(64, K)[0], dtype=np.int64)
    for t in range(64):
        for k in range(K):
            seen[oracle.plane_qs_offset(t, k, K)] += 1
    assert np.all(seen == 1)
    # each token's 32 bytes of a chunk stay inside its own 32-byte row of the tile
    for t in range(64):
        offs = {oracle.plane_qs_offset(t, k, K) % 2048 // 32 for k in range(32)}
        assert offs == {t}
    # 4-byte groups of consecutive elements stay contiguous
    for t in (0, 5, 13, 63):
        for k0 in range(0, 32, 4):
            o = [oracle.plane_qs_offset(t, k0 + i, K) for i in range(4)]
            assert o == list(range(o[0], o[0] + 4)) and o[0] % 4 == 0


@pytest.mark.parametrize("T,K", [(1, 32), (63, 64), (64, 96), (65, 640), (130, 896)])
def test_plane_encode_decode_roundtrip_and_zero_tail(T, K):
    x = synth.normal((T, K), stream=970 + T)
    qs, d16, ssum = oracle.quantize(x)
    pqs, psd = oracle.encode_plane64(qs, d16, ssum, T, K)
    q2, d2, s2, bad = oracle.decode_plane64(pqs, psd, T, K)
    assert bad == 0
    assert np.array_equal(q2, qs) and np.array_equal(d2, d16) and np.array_equal(s2, ssum)
    # the tail tokens of the last group are zero bytes
    tpad = (T + 63) // 64 * 64
    for t in range(T, tpad, 7):
        for k in range(0, K, 11):
            assert pqs[oracle.plane_qs_offset(t, k, K)] == 0


def test_gguf_block_layout():
    # hand-built row of two blocks: block b starts at 34*b, f16 d little-endian at +0, qs at +2
    blk = np.zeros((1, 68), dtype=np.uint8)
    blk[0, 0:2] = [0x00, 0x3C]        # d = 1.0
    blk[0, 2:34] = np.arange(32)
    blk[0, 34:36] = [0x08, 0x20]      # d = 0x2008
    blk[0, 36:68] = (np.arange(32) - 16).astype(np.int8).view(np.uint8)
    qs, d = oracle.gguf_to_planar(blk, 1, 64)
    assert list(d[0]) == [0x3C00, 0x2008]
    assert list(qs[0, :32]) == list(range(32))
    assert list(qs[0, 32:]) == list(range(-16, 16))
    # the weight quantizer writes that layout
    w = synth.normal((3, 64), stream=980, std=0.02)
    g = oracle.quantize_weights_gguf(w)
    q, dd, _ = oracle.quantize(w)
    q2, d2 = oracle.gguf_to_planar(g, 3, 64)
    assert np.array_equal(q, q2) and np.array_equal(dd, d2)
    assert np.array_equal(g.reshape(3, 2, 34)[:, :, 2:].reshape(3, 64).view(np.int8), q)


# ---------------------------------------------------------------------------
# Producers
# ---------------------------------------------------------------------------
def test_rmsnorm_constant_vector_closed_form():
    K = 256
    w = synth.normal((K,), stream=990, mean=1.0, std=0.1)
    for c, eps in ((3.0, 1e-6), (1e-3, 1e-6), (-2.0, 0.5)):
        x = np.full(K, c, dtype=np.float32)
        y = oracle.rmsnorm_f64(x, w, eps)[0]
        cc = float(np.float32(c))
        want = w.astype(np.float64) * cc / math.sqrt(cc * cc + eps)
        assert np.allclose(y, want, rtol=1e-14, atol=0)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    x = synth.normal((5, 3584), stream=991)
    y = oracle.rmsnorm_f64(x, np.ones(3584, np.float32), 0.0)
    assert np.allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-13)
    y2 = oracle.rmsnorm_f64((x * np.float32(4.0)).astype(np.float32), np.ones(3584, np.float32), 0.0)
    assert np.array_equal(y, y2)
    w = synth.normal((3584,), stream=992, mean=1.0, std=0.1)
    yw = oracle.rmsnorm_f64(x, w, 0.0)
    assert np.allclose(yw, y * w.astype(np.float64), rtol=1e-15)


def test_swiglu_closed_forms():
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, 2.0, -2.0], dtype=np.float32)
    u = np.array([5.0, 2.0, 2.0, 3.0, 1.0, 1.0], dtype=np.float32)
    y = oracle.swiglu_f64(g, u)
    gl = float(np.float32(math.log(3.0)))
    assert y[0] == 0.0
    assert math.isclose(y[1], gl / (1 + math.exp(-gl)) * 2.0, rel_tol=1e-15)
    assert math.isclose(y[1], 0.75 * gl * 2.0, rel_tol=1e-7)   # sigmoid(ln 3) = 3/4
    assert math.isclose(y[2], 0.25 * -gl * 2.0, rel_tol=1e-7)  # sigmoid(-ln 3) = 1/4
    assert math.isclose(y[3], 120.0, rel_tol=1e-15)            # silu(g) -> g for large g
    assert math.isclose(y[4] - y[5], 2.0, rel_tol=1e-15)       # silu(g) - silu(-g) = g
    assert oracle.swiglu_f64(np.float32([1.5]), np.float32([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# Block-scaled dot products
# ---------------------------------------------------------------------------
def _quantized_pair(T, N, K, stream):
    x = synth.normal((T, K), stream=stream)
    w = synth.normal((N, K), stream=stream + 1, std=0.02)
    aq, ad, _ = oracle.quantize(x)
    wq, wd, _ = oracle.quantize(w)
    return aq, ad, wq, wd


@pytest.mark.parametrize("T,N,K", [(1, 1, 32), (2, 3, 64), (3, 5, 96)])
def test_dot_brute_force_tiny(T, N, K):
    aq, ad, wq, wd = _quantized_pair(T, N, K, 1000 + K)
    ref, norm = oracle.gemm(wq, wd, aq, ad)
    for t in range(T):
        for n in range(N):
            s = 0.0
            a = 0.0
            for b in range(K // 32):
                isum = sum(int(aq[t, 32 * b + j]) * int(wq[n, 32 * b + j]) for j in range(32))
                term = float(oracle.f16_to_f64(wd[n, b])) * float(oracle.f16_to_f64(ad[t, b])) * isum
                s += term
                a += abs(term)
            assert math.isclose(ref[t, n], s, rel_tol=0, abs_tol=1e-12 * max(a, 1e-300))
            assert math.isclose(norm[t, n], a, rel_tol=1e-15)


def test_dot_matches_dequantized_matmul():
    T, N, K = 7, 33, 2080  # 65 blocks
    aq, ad, wq, wd = _quantized_pair(T, N, K, 1100)
    ref, norm = oracle.gemm(wq, wd, aq, ad)
    A = aq.astype(np.float64) * np.repeat(oracle.f16_to_f64(ad), 32, axis=1)
    W = wq.astype(np.float64) * np.repeat(oracle.f16_to_f64(wd), 32, axis=1)
    lib_ref = A @ W.T
    assert np.all(np.abs(ref - lib_ref) <= 1e-12 * norm)
    # pairs and single-row entry points agree with the full product
    pt = np.array([0, 6, 3, 6]), np.array([0, 32, 17, 1])
    r2, n2 = oracle.dot_pairs(wq, wd, aq, ad, *pt)
    assert np.array_equal(r2, ref[pt]) and np.array_equal(n2, norm[pt])
    yv, nv = oracle.gemv(wq, wd, aq[2], ad[2])
    assert np.array_equal(yv, ref[2])


def test_dot_exact_power_of_two_scales():
    # every d = 2^-6, |q| <= 15: every partial sum is an exact multiple of 2^-12, so the
    # result is exactly (integer dot product) * 2^-12 whatever the summation order.
    T, N, K = 4, 9, 18944
    aq = synth.uniform_i8((T, K), stream=1200, lo=-15, hi=15)
    wq = synth.uniform_i8((N, K), stream=1201, lo=-15, hi=15)
    d = np.full((1,), 2.0 ** -6, np.float32)
    h = oracle.f32_to_f16_bits(d)[0]
    ad = np.full((T, K // 32), h, np.uint16)
    wd = np.full((N, K // 32), h, np.uint16)
    ref, _ = oracle.gemm(wq, wd, aq, ad)
    exact = (aq.astype(np.int64) @ wq.astype(np.int64).T).astype(np.float64) * 2.0 ** -12
    assert np.array_equal(ref, exact)


def test_block_isums_exact_and_consistent():
    T, N, K = 3, 4, 2048
    aq, ad, wq, wd = _quantized_pair(T, N, K, 1300)
    isum = oracle.block_isums(wq, aq)
    assert isum.dtype == np.int32
    full = aq.astype(np.int64) @ wq.astype(np.int64).T
    assert np.array_equal(isum.astype(np.int64).sum(axis=2), full)
    # brute force one block
    t, n, b = 2, 3, 17
    assert isum[t, n, b] == int(np.dot(aq[t, 32 * b:32 * b + 32].astype(np.int64),
                                       wq[n, 32 * b:32 * b + 32].astype(np.int64)))
    # sums bounded by 32 * 127 * 127
    assert np.abs(isum).max() <= 32 * 127 * 127


# ---------------------------------------------------------------------------
# Input generator
# ---------------------------------------------------------------------------
def test_generator_splitmix64_reference_outputs():
    # SplitMix64 seeded with 0: its first three published outputs
    L = synth.lib()
    assert L.synth_splitmix_at(0, 0) == 0xE220A8397B1DCDAF
    assert L.synth_splitmix_at(0, 1) == 0x6E789E6AA1B965F4
    assert L.synth_splitmix_at(0, 2) == 0x06C45D188009454F


def test_generator_moments_and_offsets():
    z = synth.normal((1 << 20,), stream=7)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    part = synth.normal((1000,), stream=7, offset=5000)
    assert np.array_equal(part, z[5000:6000])
    i8 = synth.uniform_i8((1 << 16,), stream=8, lo=-15, hi=15)
    assert i8.min() == -15 and i8.max() == 15


# -- q4_K weights ([P3] s2-s3: 144-byte super-blocks, w = d*sc*nib - dmin*m) -----------------------
Q4K_SCALE_BYTES = [0xC1, 0x02, 0x83, 0x44, 0x05, 0x46, 0x87, 0xC8, 0x21, 0x43, 0x65, 0x87]
# (sc, m) of sub-blocks 0..7 for the bytes above, worked out by hand from the 6-bit layout:
# s < 4 takes the low six bits of bytes s and s+4; s >= 4 takes the nibbles of byte s+4 and the
# top two bits of bytes s-4 (scale) and s (min) as bits 4..5.
Q4K_SCALE_EXPECT = [(1, 5), (2, 6), (3, 7), (4, 8), (49, 2), (3, 20), (37, 38), (23, 56)]


def test_q4k_scale_min_worked_example():
    for s, expect in enumerate(Q4K_SCALE_EXPECT):
        assert oracle.q4k_scale_min(Q4K_SCALE_BYTES, s) == expect, s


def test_q4k_scale_packing_uses_every_bit_once():
    """Flipping any one of the 96 bits changes exactly one of the 16 six-bit fields, by a power of
    two: the packing is a bijection between 12 bytes and 8 (scale, min) pairs."""
    rng = np.random.default_rng(11)
    base = rng.integers(0, 256, 12).astype(np.uint8)
    fields = lambda b: [v for s in range(8) for v in oracle.q4k_scale_min(b, s)]
    f0 = fields(base)
    assert all(0 <= v < 64 for v in f0)
    hit = set()
    for bit in range(96):
        b = base.copy()
        b[bit // 8] ^= np.uint8(1 << (bit % 8))
        diff = [(i, abs(a - c)) for i, (a, c) in enumerate(zip(f0, fields(b))) if a != c]
        assert len(diff) == 1 and diff[0][1] in (1, 2, 4, 8, 16, 32), (bit, diff)
        hit.add((diff[0][0], diff[0][1]))
    assert len(hit) == 96  # each (field, bit) pair is reached by exactly one byte bit


def _q4k_worked_block():
    blk = np.zeros(144, np.uint8)
    blk[0:2] = [0x00, 0x3C]  # d = 1.0
    blk[2:4] = [0x00, 0x38]  # dmin = 0.5
    blk[4:16] = Q4K_SCALE_BYTES
    blk[16:] = np.arange(128, dtype=np.uint8)  # value byte i = i
    return blk


def test_q4k_values_worked_example():
    """Values of a hand-made block (d = 1, dmin = 0.5, value bytes 0..127), worked out by hand:
    sub-block s, value j reads byte 32*(s//2) + j, low nibble for even s, high for odd s."""
    w = oracle.q4k_dequant(_q4k_worked_block(), 1, 256)[0]
    cases = {  # (s, j): d*sc*nib - dmin*m
        (0, 5): 1 * 5 - 0.5 * 5,      # byte 5, low nibble 5
        (1, 5): 2 * 0 - 0.5 * 6,      # byte 5, high nibble 0
        (3, 31): 4 * 3 - 0.5 * 8,     # byte 63 = 0x3F, high nibble 3
        (4, 17): 49 * 1 - 0.5 * 2,    # byte 81 = 0x51, low nibble 1
        (6, 31): 37 * 15 - 0.5 * 38,  # byte 127 = 0x7F, low nibble 15
        (7, 0): 23 * 6 - 0.5 * 56,    # byte 96 = 0x60, high nibble 6
    }
    for (s, j), v in cases.items():
        assert w[32 * s + j] == v, (s, j, w[32 * s + j], v)
    nib, d, dmin, sc, mn = oracle.q4k_decode(_q4k_worked_block(), 1, 256)
    assert d[0, 0] == 0x3C00 and dmin[0, 0] == 0x3800
    assert [(int(a), int(b)) for a, b in zip(sc[0], mn[0])] == Q4K_SCALE_EXPECT
    assert nib[0, 32 * 2 + 10] == (32 + 10) & 15 and nib[0, 32 * 5 + 3] == (64 + 3) >> 4


def test_q4k_dot_equals_dequantized_matmul():
    """The block-scaled form with the activation's ssum carrying the min term equals the plain f64
    matmul of the dequantized weights and the dequantized activation (da * qa)."""
    N, K, T = 5, 768, 3
    blocks = synth.q4k_blocks(N, K, 950)
    x = synth.normal((T, K), stream=951)
    qa, da, ssum = oracle.quantize(x)
    ref, norm = oracle.q4k_gemm(blocks, N, K, qa, da, ssum)
    a = qa.astype(np.float64) * np.repeat(oracle.f16_to_f64(da), 32, axis=1)
    direct = a @ oracle.q4k_dequant(blocks, N, K).T
    assert np.all(np.abs(ref - direct) <= 1e-12 * norm)
    # and one cell by pure-Python loops over the dequantized values
    w = oracle.q4k_dequant(blocks, N, K)
    s = 0.0
    for k in range(K):
        s += float(w[2, k]) * float(a[1, k])
    assert abs(ref[1, 2] - s) <= 1e-12 * norm[1, 2]
    pr, pn = oracle.q4k_dot_pairs(blocks, N, K, qa, da, ssum, np.array([1, 0]), np.array([2, 4]))
    assert pr[0] == ref[1, 2] and pr[1] == ref[0, 4] and pn[0] == norm[1, 2]


def test_q4k_degenerate_blocks():
    """All-zero values leave only the min term -dmin*m*ssum; dmin = 0 leaves only d*sc*isum."""
    K = 256
    x = synth.normal((1, K), stream=952)
    qa, da, ssum = oracle.quantize(x)
    blk = _q4k_worked_block()
    zero_vals = blk.copy()
    zero_vals[16:] = 0
    ref, _ = oracle.q4k_gemm(zero_vals, 1, K, qa, da, ssum)
    expect = -sum(float(oracle.f16_to_f64(da[0, s])) * 0.5 * m * int(ssum[0, s])
                  for s, (_, m) in enumerate(Q4K_SCALE_EXPECT))
    assert ref[0, 0] == pytest.approx(expect, rel=1e-14, abs=0)
    no_min = blk.copy()
    no_min[2:4] = 0
    ref2, _ = oracle.q4k_gemm(no_min, 1, K, qa, da, ssum)
    w = oracle.q4k_dequant(no_min, 1, K)[0]
    a = qa[0].astype(np.float64) * np.repeat(oracle.f16_to_f64(da[0]), 32)
    assert ref2[0, 0] == pytest.approx(float(np.dot(w, a)), rel=1e-13)


# ---------------------------------------------------------------------------
# Thread count
# ---------------------------------------------------------------------------


def test_oracle_results_do_not_depend_on_thread_count():
    """The oracle's parallel loops split work over rows, columns or blocks only; every output is
    computed by one thread in a fixed order, so one thread and all of them give the same bits
    (the benchmark times it both ways)."""
    x = synth.normal((70, 640), stream=9100)
    w = synth.normal((640,), stream=9101, mean=1.0, std=0.1)
    wq, wd = oracle.gguf_to_planar(oracle.quantize_weights_gguf(synth.normal((200, 640), stream=9102, std=0.02)),
                                   200, 640)
    blocks = synth.q4k_blocks(64, 512, 9103)
    x4 = synth.normal((70, 512), stream=9104)

    def run():
        q, d, s = oracle.quantize(x)
        y = oracle.rmsnorm_f64(x, w, 1e-6)
        g = oracle.gemv(wq, wd, q[3], d[3])
        c = oracle.gemm(wq, wd, q, d)
        q4, d4, s4 = oracle.quantize(x4)
        k = oracle.q4k_gemm(blocks, 64, 512, q4, d4, s4)
        return [q, d, s, y, g[0], c[0], k[0]]

    n = oracle.num_threads()
    try:
        oracle.set_threads(1)
        one = run()
        oracle.set_threads(max(n, 4))
        many = run()
    finally:
        oracle.set_threads(n)
    for i, (a, b) in enumerate(zip(one, many)):
        a, b = np.asarray(a), np.asarray(b)
        assert a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"output {i}"
