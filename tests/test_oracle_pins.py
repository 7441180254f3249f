"""Pins for the CPU oracle, against facts that do not come from the oracle.

Each test ties one oracle step to something independent: exhaustive
enumeration against the web page's own formulation of a step, exact rational
arithmetic, a closed form, a second bit-level formulation, torch's bf16 cast,
or brute force. Source of the method: web page "mlx-bun 0.2.0 -> 0.4.0" (npm
diff, page 57), section src/model/trellis-wide-prefill.ts (kernel body and
host wrapper).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
C_NORM = Fraction(147.800537109375)


# ---- exact helpers (independent of the oracle) ----------------------------

def f32_bits(f) -> int:
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0])


def rn_f32(q: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (ties to even)."""
    f0 = np.float32(float(q))
    best = None
    for f in (np.nextafter(f0, np.float32(-np.inf)), f0, np.nextafter(f0, np.float32(np.inf))):
        d = abs(Fraction(float(f)) - q)
        key = (d, f32_bits(f) & 1)
        if best is None or key < best[0]:
            best = (key, f)
    return np.float32(best[1])


def torch_bf16_bits(a) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- constants ------------------------------------------------------------

def test_reciprocal_is_correctly_rounded():
    # The page writes the reciprocal as 1.0f/147.800537109375f. IEEE division
    # gives the correctly rounded float32 of the exact quotient.
    r = oracle.reciprocal()
    assert np.float32(r) == rn_f32(1 / C_NORM)
    assert f32_bits(r) == 0x3BDDB447


def test_normaliser_constants_are_byte_sum_moments():
    # 510 is the mean of a sum of four uniform bytes (4 * 127.5) and
    # 147.800537109375 is float32(sqrt(21845)), 21845 = 4 * (256^2 - 1) / 12
    # being that sum's variance: the code is centred and scaled to unit
    # variance. Checked exactly: C is a float32 whose rounding interval
    # contains sqrt(21845).
    assert 4 * Fraction(255, 2) == 510
    var = 4 * Fraction(256 ** 2 - 1, 12)
    assert var == 21845
    c = np.float32(147.800537109375)
    assert Fraction(float(c)) == C_NORM
    ulp = Fraction(float(np.nextafter(c, np.float32(np.inf)))) - C_NORM
    lo, hi = C_NORM - ulp / 2, C_NORM + ulp / 2
    assert lo * lo < var < hi * hi


# ---- hash and byte sum: all 4096 windows ------------------------------------

def page_swar_code(win: int) -> int:
    """The page's own formulation: a byte-pair SWAR add of the hash."""
    z = (win * 34038481 + 76625530) & 0xFFFFFFFF
    p = (z & 0x00FF00FF) + ((z >> 8) & 0x00FF00FF)
    return (p & 0xFFFF) + (p >> 16) - 510


def test_code_matches_page_swar_form_exhaustively():
    codes = [oracle.code(w) for w in range(4096)]
    assert codes == [page_swar_code(w) for w in range(4096)]
    assert min(codes) >= -510 and max(codes) <= 510
    # Observed image of the 4096 windows.
    assert (min(codes), max(codes), len(set(codes))) == (-448, 454, 713)


def test_code_golden_points():
    rows = []
    with open(os.path.join(GOLDEN, "decode_points.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                w, z, c = line.split()
                rows.append((int(w), int(z, 16), int(c)))
    assert len(rows) >= 3
    for w, z, c in rows:
        assert (w * 34038481 + 76625530) % 2 ** 32 == z
        assert oracle.code(w) == c


def test_code_mean_and_variance_are_near_standard():
    vals = np.array([oracle.value(oracle.code(w)) for w in range(4096)])
    assert abs(vals.mean()) < 0.02
    assert abs(vals.var() - 1.0) < 0.02


# ---- normalisation: all 1021 codes ------------------------------------------

def test_value_is_correctly_rounded_quotient_for_every_code():
    # The fused refinement reaches the correctly rounded float32 of code/C
    # for every reachable code.
    for c in range(-510, 511):
        assert f32_bits(oracle.value(c)) == f32_bits(rn_f32(Fraction(c) / C_NORM)), c


def test_plain_product_differs_so_refinement_is_observable():
    # Negative control: rounding c*r once (no refinement) disagrees with the
    # quotient for many codes, so the test above would catch a dropped step.
    r = np.float32(oracle.reciprocal())
    cs = np.arange(-510, 511, dtype=np.float32)
    plain = (cs * r).astype(np.float32)
    exact = np.array([rn_f32(Fraction(int(c)) / C_NORM) for c in cs], dtype=np.float32)
    assert int(np.sum(plain != exact)) == 398


def test_value_closed_form_window_zero():
    # window 0 -> code -185 -> -185 / 147.800537109375 = -1.2516869...
    assert f32_bits(oracle.value(oracle.code(0))) == 0xBFA03747
    assert abs(oracle.value(-185) - (-185 / 147.800537109375)) < 2e-7


# ---- bf16 rounding ----------------------------------------------------------

def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(7)
    vals = [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 1e-40, -3e-39, 3.4e38, 1.0e-45]
    # exact ties: odd and even kept halves
    for h in (0x3F80, 0x3F81, 0xBF82, 0x0001, 0x7F7F):
        vals.append(np.array([(h << 16) | 0x8000], dtype=np.uint32).view(np.float32)[0])
    vals = np.array(vals, dtype=np.float32)
    rnd = rng.standard_normal(20000).astype(np.float32) * np.float32(0.05)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    raw = bits.view(np.float32)
    raw = raw[np.isfinite(raw)]
    allv = np.concatenate([vals, rnd, raw]).astype(np.float32)
    ours = np.array([oracle.f32_to_bf16(float(v)) for v in allv], dtype=np.uint16)
    assert np.array_equal(ours, torch_bf16_bits(allv))


def test_bf16_widening_is_exact():
    hs = np.arange(0, 65536, 97, dtype=np.uint32)
    for h in hs:
        v = oracle.bf16_to_f32(int(h))
        if np.isnan(v):
            continue
        assert f32_bits(v) == int(h) << 16


# ---- windows: three formulations, rotation, single-bit probes ----------------

def bigint_window(block: np.ndarray, bits: int, t: int) -> int:
    """Block as one integer; cyclic read by concatenating it with itself."""
    nbits = 256 * bits
    s = 0
    for i, w in enumerate(block.tolist()):
        s |= int(w) << (32 * i)
    ss = s | (s << nbits)
    return (ss >> ((255 - t) * bits)) & 0xFFF


def page_word_window(block: np.ndarray, bits: int, t: int) -> int:
    """The page's word-shift formulation (shift one word, OR in the next
    word of the same block when the window straddles, wrap to word 0)."""
    wpb = 256 * bits // 32
    pos = (255 - t) * bits
    wi, off = pos >> 5, pos & 31
    win = int(block[wi]) >> off
    if off + 12 > 32:
        nxt = 0 if wi + 1 == wpb else wi + 1
        win |= (int(block[nxt]) << (32 - off)) & 0xFFFFFFFF
    return win & 0xFFF


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_window_three_formulations_agree(bits):
    rng = np.random.default_rng(100 + bits)
    for _ in range(6):
        block = rng.integers(0, 2 ** 32, 256 * bits // 32, dtype=np.uint32)
        for t in range(256):
            w = oracle.window(block, bits, t)
            assert w == bigint_window(block, bits, t)
            assert w == page_word_window(block, bits, t)


def rotate_stream(block: np.ndarray, bits: int, by: int) -> np.ndarray:
    """New stream bit j = old stream bit (j + by) mod 256*bits."""
    nbits = 256 * bits
    s = 0
    for i, w in enumerate(block.tolist()):
        s |= int(w) << (32 * i)
    by %= nbits
    s = ((s >> by) | (s << (nbits - by))) & ((1 << nbits) - 1)
    return np.array([(s >> (32 * i)) & 0xFFFFFFFF for i in range(block.size)], dtype=np.uint32)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_window_rotation_invariant(bits):
    # Rotating the cyclic stream by k bits moves every weight by one slot:
    # W'[t] = W[(t - 1) mod 256].
    rng = np.random.default_rng(200 + bits)
    block = rng.integers(0, 2 ** 32, 256 * bits // 32, dtype=np.uint32)
    rot = rotate_stream(block, bits, bits)
    w = [oracle.window(block, bits, t) for t in range(256)]
    w2 = [oracle.window(rot, bits, t) for t in range(256)]
    assert w2 == [w[(t - 1) % 256] for t in range(256)]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_window_single_bit_probes(bits):
    # Setting one stream bit j lights exactly the windows whose cyclic span
    # covers j, each at bit (j - pos) mod 256k (LSB-first, tail-biting).
    nbits = 256 * bits
    words = 256 * bits // 32
    for j in list(range(0, 40)) + list(range(nbits - 40, nbits)) + [nbits // 2, nbits // 3]:
        block = np.zeros(words, dtype=np.uint32)
        block[j >> 5] = np.uint32(1 << (j & 31))
        for t in range(256):
            pos = (255 - t) * bits
            d = (j - pos) % nbits
            expect = (1 << d) if d < 12 else 0
            assert oracle.window(block, bits, t) == expect, (j, t)


@pytest.mark.parametrize("bits,wrapping", [(2, 5), (3, 3), (4, 2)])
def test_wrap_count(bits, wrapping):
    # Windows that run past the end of the block: t = 0 .. ceil(12/k) - 2.
    nbits = 256 * bits
    assert sum(1 for t in range(256) if (255 - t) * bits + 12 > nbits) == wrapping
    block = np.zeros(256 * bits // 32, dtype=np.uint32)
    block[0] = 1  # stream bit 0 only
    lit = [t for t in range(256) if oracle.window(block, bits, t)]
    assert lit == list(range(wrapping)) + [255]


# ---- scale and rounding: all windows x all 257 reachable scales --------------

def reachable_scales() -> np.ndarray:
    # bf16 RNE image of U[0.005, 0.02]: 0x3BA4 (0.0050048828125) .. 0x3CA4.
    lo = int(torch_bf16_bits([0.005])[0])
    hi = int(torch_bf16_bits([0.02])[0])
    assert (lo, hi) == (0x3BA4, 0x3CA4)
    return np.arange(lo, hi + 1, dtype=np.uint16)


def test_weight_exhaustive_against_exact_double_rounding():
    # W = bf16_RNE(RN_f32(value * scale)), value = RN_f32(code / C). The
    # product of a 24-bit and an 8-bit significand is exact in float64, so
    # numpy's float64 -> float32 cast is the single float32 rounding; torch's
    # cast is the bf16 rounding.
    scales = reachable_scales()
    assert scales.size == 257
    vals = np.array([rn_f32(Fraction(oracle.code(w)) / C_NORM) for w in range(4096)],
                    dtype=np.float32)
    prod = (vals[None, :].astype(np.float64) * bf16_value(scales)[:, None].astype(np.float64))
    expect = torch_bf16_bits(prod.astype(np.float32))
    got = np.empty((257, 4096), dtype=np.uint16)
    for i, s in enumerate(scales):
        for w in range(4096):
            got[i, w] = oracle.weight(w, int(s))
    assert np.array_equal(got, expect)


def test_weight_power_of_two_scales():
    # scale 1.0 gives bf16(value); scale 2^-6 gives bf16(value) * 2^-6 exactly.
    for w in range(0, 4096, 7):
        v = np.float32(oracle.value(oracle.code(w)))
        b = int(torch_bf16_bits([v])[0])
        assert oracle.weight(w, 0x3F80) == b
        scaled = bf16_value(oracle.weight(w, 0x3C80))[()]
        assert scaled == np.float32(bf16_value(b)[()] * np.float32(2.0 ** -6))
    assert bf16_value(oracle.weight(0, 0x3C80))[()] == np.float32(-0.01953125)


# ---- row layout ---------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decode_rows_block_layout(bits):
    rng = np.random.default_rng(300 + bits)
    n, k = 4, 768
    wpb = 256 * bits // 32
    codes = rng.integers(0, 2 ** 32, (n, k * bits // 32), dtype=np.uint32)
    scales = rng.integers(0x3BA4, 0x3CA5, n).astype(np.uint16)
    w = oracle.decode_rows(codes, scales, k, bits)
    for r in range(n):
        for b in range(k // 256):
            blk = codes[r, b * wpb:(b + 1) * wpb]
            for t in range(0, 256, 17):
                win = bigint_window(blk, bits, t)
                assert w[r, 256 * b + t] == oracle.weight(win, int(scales[r]))
    # a sub-range of rows decodes to the same rows
    assert np.array_equal(oracle.decode_rows(codes, scales, k, bits, 1, 2), w[1:3])


# ---- contraction --------------------------------------------------------------

def test_contraction_brute_force_exact():
    from workloads import generate

    x, codes, scales = generate(5, 256, 4, 3, seed=11)
    w = oracle.decode(codes, scales, 256, 3)
    y, a = oracle.prefill(x, codes, scales, 256, 3)
    xv = bf16_value(x).astype(np.float64)
    wv = bf16_value(w).astype(np.float64)
    for i in range(5):
        for n in range(4):
            exact = sum(Fraction(float(wv[n, kk])) * Fraction(float(xv[i, kk])) for kk in range(256))
            absum = sum(abs(Fraction(float(wv[n, kk])) * Fraction(float(xv[i, kk]))) for kk in range(256))
            bound = 256 * 2.0 ** -53 * float(absum)
            assert abs(Fraction(y[i, n]) - exact) <= Fraction(bound)
            assert abs(Fraction(a[i, n]) - absum) <= Fraction(bound)


def test_prefill_equals_contract_of_decode():
    from workloads import generate

    x, codes, scales = generate(7, 512, 8, 4, seed=12)
    w = oracle.decode(codes, scales, 512, 4)
    y1, a1 = oracle.prefill(x, codes, scales, 512, 4)
    y2, a2 = oracle.contract(x, w)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)
    y3, _ = oracle.prefill_rows(x, codes, scales, 512, 4, [5, 1, 2, 7])
    assert np.array_equal(y3, y1[:, [5, 1, 2, 7]])


def test_one_hot_rows_select_weights():
    from workloads import generate

    _, codes, scales = generate(5, 512, 12, 2, seed=13)
    m, k = 6, 512
    js = [0, 1, 255, 256, 300, 511]
    x = np.zeros((m, k), dtype=np.uint16)
    for i, j in enumerate(js):
        x[i, j] = 0x3F80  # 1.0
    w = oracle.decode(codes, scales, k, 2)
    y, a = oracle.prefill(x, codes, scales, k, 2)
    for i, j in enumerate(js):
        assert np.array_equal(y[i], bf16_value(w[:, j]).astype(np.float64))
        assert np.array_equal(a[i], np.abs(y[i]))


def test_zero_codes_closed_form():
    # All-zero codes: every window is 0, every weight is bf16(v0 * s_n) with
    # v0 = RN_f32(-185 / C), so y[m, n] = w0(n) * sum_k x[m, k].
    from workloads import generate

    x, _, scales = generate(5, 512, 8, 4, seed=14)
    codes = np.zeros((8, 512 * 4 // 32), dtype=np.uint32)
    y, _ = oracle.prefill(x, codes, scales, 512, 4)
    v0 = rn_f32(Fraction(-185) / C_NORM)
    w0 = bf16_value(torch_bf16_bits(
        (np.float64(v0) * bf16_value(scales).astype(np.float64)).astype(np.float32)))
    xs = bf16_value(x).astype(np.float64)
    for i in range(5):
        for n in range(8):
            exact = Fraction(float(w0[n])) * sum(Fraction(float(v)) for v in xs[i])
            assert abs(Fraction(y[i, n]) - exact) <= Fraction(512 * 2.0 ** -52) * abs(exact) + Fraction(2.0 ** -80)


# ---- acceptance bound helper ---------------------------------------------------

def test_ulp_bf16():
    v = np.array([1.0, 1.5, 2.0, -3.0, 0.0, 2.0 ** -126, 0.0078125], dtype=np.float64)
    assert np.array_equal(oracle.ulp_bf16(v),
                          [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133, 2.0 ** -14])
    out = torch_bf16_bits([1.0, 2.0])
    assert oracle.within_tolerance(out, np.array([1.0 + 2 ** -7, 2.0 - 2 ** -6]), np.zeros(2)).all()
    assert not oracle.within_tolerance(out, np.array([1.0 + 2 ** -6, 2.0]), np.zeros(2))[0]


# ---- gate/up tail (silu(gate) * up) ------------------------------------------

def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly; silu(0) = 0;
    # silu(x) - silu(-x) = x for every x; silu(x) -> x and -> 0 at the ends.
    ln3 = np.log(3.0)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(ln3) - 0.75 * ln3) <= 1e-15
    assert abs(oracle.silu(-ln3) + 0.25 * ln3) <= 1e-15
    xs = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(xs) - oracle.silu(-xs), xs, rtol=0, atol=1e-13)
    assert abs(oracle.silu(60.0) - 60.0) <= 1e-20 * 60 + 1e-12
    assert abs(oracle.silu(-800.0)) == 0.0
    # minimum of silu: about -0.2785 at x about -1.2785 (x = -1 - W(1/e))
    grid = np.linspace(-3, 0, 300001)
    assert abs(oracle.silu(grid).min() + 0.27846454276) < 1e-9


def test_gate_up_rows_one_hot_and_zero_codes():
    # One-hot x rows: g = Wg[n, j], u = Wu[n, j], so h = silu(Wg[n, j]) * Wu[n, j];
    # all-zero up codes: u = w0(n) * sum(x) as in the prefill closed form.
    from workloads import generate

    k, n = 512, 12
    _, cg, sg = generate(5, k, n, 4, seed=21)
    _, cu, su = generate(5, k, n, 4, seed=22)
    js = [0, 7, 256, 511]
    x = np.zeros((len(js), k), dtype=np.uint16)
    x[np.arange(len(js)), js] = 0x3F80
    h, g, ag, u, au = oracle.gate_up_rows(x, cg, sg, cu, su, k, 4, range(n))
    wg = bf16_value(oracle.decode(cg, sg, k, 4)).astype(np.float64)
    wu = bf16_value(oracle.decode(cu, su, k, 4)).astype(np.float64)
    for i, j in enumerate(js):
        assert np.array_equal(g[i], wg[:, j]) and np.array_equal(u[i], wu[:, j])
        assert np.allclose(h[i], wg[:, j] / (1 + np.exp(-wg[:, j])) * wu[:, j], rtol=1e-15, atol=0)
    xr, _, _ = generate(3, k, n, 4, seed=23)
    hz, gz, _, uz, _ = oracle.gate_up_rows(xr, cg, sg, np.zeros_like(cu), su, k, 4, range(n))
    yz, _ = oracle.prefill(xr, np.zeros_like(cu), su, k, 4)
    assert np.array_equal(uz, yz)


def test_gate_up_tolerance_accepts_the_chain_and_rejects_a_slip():
    # The bf16 chain applied to bf16-rounded g, u lies inside the bound; an
    # output one bf16 step from it for |h| well above the bound does not.
    rng = np.random.default_rng(31)
    g = rng.normal(0, 2, 2000)
    u = rng.normal(0, 2, 2000)
    ag = np.abs(g) * 3
    au = np.abs(u) * 3
    gb = bf16_value(torch_bf16_bits(g.astype(np.float32))).astype(np.float64)
    ub = bf16_value(torch_bf16_bits(u.astype(np.float32))).astype(np.float64)
    sig = bf16_value(torch_bf16_bits((1 / (1 + np.exp(-gb))).astype(np.float32))).astype(np.float64)
    silu_b = bf16_value(torch_bf16_bits((gb * sig).astype(np.float32))).astype(np.float64)
    hb = torch_bf16_bits((silu_b * ub).astype(np.float32))
    h = oracle.silu(g) * u
    assert oracle.gate_up_within_tolerance(hb, h, g, ag, u, au).all()
    # the rounding terms alone cover the chain (no accumulation error here)
    assert oracle.gate_up_within_tolerance(hb, h, g, np.zeros_like(ag), u, np.zeros_like(au)).all()
    far = torch_bf16_bits((bf16_value(hb).astype(np.float64) * 1.25).astype(np.float32))
    # where silu is not tiny next to its slope (gate >= 0.5) the bound is a
    # few percent of |h|, so a 25% slip must fail
    sel = (g >= 0.5) & (np.abs(h) > 0.5)
    assert sel.sum() > 100
    assert not oracle.gate_up_within_tolerance(far, h, g, np.zeros_like(ag), u, np.zeros_like(au))[sel].any()


# ---- bf16 chain of the gate/up tail ------------------------------------------
# Page "mlx-bun 0.0.4" (npm, page 62), section src/model/minicpm5.ts, MLP
# forward: sigmoid(gate), gate * sigmoid(gate) and that times up are each a
# bf16 array. oracle.gate_up_chain rounds each exact step once; it is pinned
# here against exact rational rounding and a 40-digit decimal sigmoid.

def _bf16_round_fraction(q: Fraction) -> int:
    """bf16 bits of the exact rational q, to nearest, ties to even (integer
    arithmetic on q's numerator and denominator; finite, |q| < 2^128)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    num, den = a.numerator, a.denominator
    e = num.bit_length() - den.bit_length()          # 2^e <= a < 2^(e+2)
    if Fraction(num, den) < Fraction(2) ** e:
        e -= 1
    if Fraction(num, den) >= Fraction(2) ** (e + 1):
        e += 1
    qexp = max(e - 7, -133)                            # quantum of a's binade
    scaled = a / (Fraction(2) ** qexp)
    r, rem = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * rem
    if twice > scaled.denominator or (twice == scaled.denominator and r & 1):
        r += 1
    val = Fraction(r) * Fraction(2) ** qexp
    bits = int(np.array([float(val)], dtype=np.float32).view(np.uint32)[0]) >> 16
    return sign | bits


def test_f64_to_bf16_is_exact_single_rounding():
    rng = np.random.default_rng(41)
    vals = list(rng.normal(0, 1, 3000) * np.exp2(rng.integers(-140, 127, 3000)))
    # exact midpoints between neighbouring bf16 values and their f64 neighbours
    for b in rng.integers(0x0001, 0x7F7F, 600):
        lo = float(bf16_value([b])[0])
        hi = float(bf16_value([b + 1])[0])
        mid = (lo + hi) / 2
        vals += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), -mid]
    for v in vals:
        want = _bf16_round_fraction(Fraction(float(v)))
        got = oracle.f64_to_bf16(float(v))
        assert got == want, (v, hex(got), hex(want))
    # a value one float32 rounding would push onto a tie: 1 + 2^-8 + 2^-40
    # rounds up in one step (and to even, down, after a float32 rounding)
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.f64_to_bf16(float(np.float32(1.0 + 2.0 ** -8 + 2.0 ** -40))) == 0x3F80


def _chain_reference(gate_bits: int, up_bits: int, drop: str = ""):
    """The page's chain with a 40-digit decimal sigmoid and exact rational
    products; `drop` skips one rounding ("sig" or "silu") for the negative
    controls below."""
    from decimal import Decimal, localcontext

    g = Fraction(float(bf16_value([gate_bits])[0]))
    u = Fraction(float(bf16_value([up_bits])[0]))
    with localcontext() as ctx:
        ctx.prec = 40
        ctx.Emax = 10 ** 6
        ctx.Emin = -10 ** 6
        dg = Decimal(g.numerator) / Decimal(g.denominator)
        sig = Fraction(Decimal(1) / (Decimal(1) + (-dg).exp()))
    sig_r = sig if drop == "sig" else Fraction(float(bf16_value([_bf16_round_fraction(sig)])[0]))
    silu = g * sig_r
    silu_r = silu if drop == "silu" else Fraction(float(bf16_value([_bf16_round_fraction(silu)])[0]))
    return _bf16_round_fraction(silu_r * u)


def test_gate_up_chain_exhaustive_gates_against_decimal():
    # every bf16 gate with |gate| < 2^11 (beyond that sigmoid is 0 or 1 in
    # every format) against one up with a full 8-bit significand, so the
    # final rounding is exercised too
    gates = np.array([b for b in range(0x10000) if (b & 0x7FFF) < 0x4500], dtype=np.uint16)
    up = np.full(gates.shape, 0xBFB5, dtype=np.uint16)   # -1.4140625
    h, amb = oracle.gate_up_chain(gates, up)
    want = np.array([_chain_reference(int(g), 0xBFB5) for g in gates], dtype=np.uint16)
    same = (h == want) | ((h & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
    assert same.all(), [(hex(g), hex(a), hex(b)) for g, a, b in zip(gates[~same][:5], h[~same][:5], want[~same][:5])]
    # the ambiguity flag is rare (sigmoid within 2^-21 of a bf16 midpoint)
    assert amb.sum() < 40


def test_gate_up_chain_closed_forms():
    one, two, zero = 0x3F80, 0x4000, 0x0000
    # gate = 0: sigmoid 1/2, silu 0, h = 0
    h, _ = oracle.gate_up_chain(np.array([zero], np.uint16), np.array([two], np.uint16))
    assert (h[0] & 0x7FFF) == 0
    # gate = ln 3 rounded: sigmoid close to 3/4 -> bf16 0.75 exactly when the
    # rounded gate keeps the sigmoid within half an ulp of 0.75
    g = oracle.f64_to_bf16(np.log(3.0))
    gv = float(bf16_value([g])[0])
    s = 1 / (1 + np.exp(-gv))
    assert abs(s - 0.75) < 2 ** -10
    h, _ = oracle.gate_up_chain(np.array([g], np.uint16), np.array([one], np.uint16))
    assert h[0] == oracle.f64_to_bf16(gv * 0.75)
    # large gates: sigmoid rounds to 1 (gate >= 2^4 is enough) so h = bf16(gate*up)
    big = np.array([0x4180, 0x4200, 0x4380], np.uint16)     # 16, 32, 256
    upv = np.array([0x3FB5, 0xC0A1, 0x3E01], np.uint16)
    h, _ = oracle.gate_up_chain(big, upv)
    for i in range(3):
        gv = float(bf16_value([big[i]])[0])
        uv = float(bf16_value([upv[i]])[0])
        assert h[i] == oracle.f64_to_bf16(gv * uv)
    # very negative gates: silu underflows to (-)0
    h, _ = oracle.gate_up_chain(np.array([0xC400, 0xC2C8], np.uint16), np.array([one, one], np.uint16))
    assert ((h & 0x7FFF) == 0).all()


@pytest.mark.parametrize("drop", ["sig", "silu"])
def test_gate_up_chain_each_rounding_is_observable(drop):
    # One-hot x turns the device's gate and up into single decoded weights
    # times a power of two, so a bit-exact comparison against the chain sees
    # any missing rounding: on gates and ups of that kind, dropping the
    # rounding of sigmoid(gate) or of gate * sigmoid(gate) changes a sizeable
    # share of the outputs.
    rng = np.random.default_rng(53)
    w = rng.normal(0, 0.02, 1500).astype(np.float32)
    p = np.exp2(rng.integers(0, 9, 1500)).astype(np.float32)
    gates = torch_bf16_bits(w * p)
    ups = torch_bf16_bits(rng.normal(0, 0.02, 1500).astype(np.float32) * 16)
    h, _ = oracle.gate_up_chain(gates, ups)
    diff = sum(int(h[i]) != _chain_reference(int(gates[i]), int(ups[i]), drop) for i in range(len(gates)))
    assert diff > 100, diff
