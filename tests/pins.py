"""Pins of the oracle: checks of ``oracle.post`` against things other than
itself (textbook attention, closed forms, exact rational brute force, a
library routine, hand-derived fixtures).

Each ``pin_*`` raises AssertionError when the oracle is wrong. They look the
oracle's functions up at call time through the module object, so the mutation
tests can plant a mistake in one function and check that some pin fails.
"""

from __future__ import annotations

import bisect
import os
from fractions import Fraction

import numpy as np
import torch

import oracle.post as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MIDS4 = (1, 3, 5, 7, 10, 14, 20)  # 4x the midpoints between adjacent E2M1 magnitudes


# ---------------------------------------------------------------- helpers


def torch_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """torch's CPU float32 -> bfloat16 cast, a library RNE routine."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_from_f32(x) -> np.ndarray:
    return torch_bf16_bits(np.asarray(x, dtype=np.float32))


_POS_BF16 = None


def positive_bf16_table():
    """All positive finite bf16 values, ascending, as (Fraction list, bits)."""
    global _POS_BF16
    if _POS_BF16 is None:
        bits = np.arange(0x0001, 0x7F80, dtype=np.uint32)
        vals = (bits << 16).view(np.float32).astype(np.float64)
        _POS_BF16 = ([Fraction(float(v)) for v in vals], bits.astype(np.uint16))
    return _POS_BF16


def brute_rne_bf16(v: Fraction) -> int:
    """RNE to bf16 by search over every finite bf16 value (tiny cases)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    vals, bits = positive_bf16_table()
    maxv = vals[-1]
    half_ulp_top = (Fraction(2) ** 127) * Fraction(1, 2**8)  # half a quantum at the top binade
    if a >= maxv + half_ulp_top:
        return sign | 0x7F80
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | int(bits[i])
    lo_v, lo_b = (Fraction(0), 0) if i == 0 else (vals[i - 1], int(bits[i - 1]))
    hi_v, hi_b = (vals[i], int(bits[i])) if i < len(vals) else (Fraction(2) ** 128, 0x7F80)
    dl, dh = a - lo_v, hi_v - a
    if dl < dh:
        return sign | lo_b
    if dh < dl:
        return sign | hi_b
    return sign | (lo_b if lo_b % 2 == 0 else hi_b)


def attention_split(rng, n_kv, d, dv, sizes):
    """Brute-force softmax attention of one query, unsplit and split into KV
    chunks of the given sizes; returns (full [dv], partial outs [C, dv],
    natural-log LSEs [C]). An empty chunk gets LSE -inf and a NaN output."""
    q = rng.standard_normal(d)
    K = rng.standard_normal((n_kv, d))
    V = rng.standard_normal((n_kv, dv))
    s = K @ q / np.sqrt(d)
    p = np.exp(s - s.max())
    full = (p / p.sum()) @ V
    outs, lses, at = [], [], 0
    for c in sizes:
        if c == 0:
            outs.append(np.full(dv, np.nan))
            lses.append(-np.inf)
            continue
        sc = s[at : at + c]
        pc = np.exp(sc - sc.max())
        outs.append((pc / pc.sum()) @ V[at : at + c])
        lses.append(sc.max() + np.log(pc.sum()))
        at += c
    assert at == n_kv
    return full, np.array(outs), np.array(lses)


def load_golden_blocks():
    rows = []
    with open(os.path.join(GOLDEN, "mxfp4_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, code, elems, out = [p.strip() for p in line.split(";")]
            x = np.zeros(32, dtype=np.uint16)
            for tok in elems.split():
                i, v = tok.split(":")
                if i == "*":
                    x[:] = int(v, 16)
                else:
                    x[int(i)] = int(v, 16)
            rows.append((name, int(code), x, np.array([int(b, 16) for b in out.split()], dtype=np.uint8)))
    return rows


def load_e2m1_table():
    tab = {}
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                tab[int(c)] = float(v)
    return tab


def _dense_case(rng, n, T, lse_lo=-4.0, lse_hi=16.0):
    o = bf16_bits_from_f32(rng.standard_normal((n, T, O.NH, O.KVL)).astype(np.float32))
    lse = rng.uniform(lse_lo, lse_hi, size=(n, T, O.NH)).astype(np.float32)
    return o, lse


def _random_wv(rng):
    w = bf16_bits_from_f32((rng.standard_normal((O.NH, O.VD, O.KVL)) / np.sqrt(512)).astype(np.float32))
    return O.quantize_mxfp4(w)


def _gate(rng, T):
    return bf16_bits_from_f32(rng.random((T, O.NH * O.VD)).astype(np.float32))


# ---------------------------------------------------------------- merge pins


def pin_textbook_attention():
    """I1: merging the chunk partials of a brute-force softmax attention gives
    the unsplit attention (flash-decoding identity), in float64 exactly up to
    rounding, and within 2^-8 max|V| when the partials are bf16."""
    rng = np.random.default_rng(11)
    chunkings = [(0, 5, 12, 20), (37,), (1, 1, 35), (20, 0, 0, 17), (9, 9, 9, 10)]
    T = 4
    for sizes in chunkings:
        outs = np.zeros((len(sizes), T, O.NH, 16))
        lses = np.zeros((len(sizes), T, O.NH))
        fulls = np.zeros((T, O.NH, 16))
        for t in range(T):
            for h in range(O.NH):
                full, oc, lc = attention_split(rng, 37, 8, 16, sizes)
                fulls[t, h] = full
                outs[:, t, h] = oc
                lses[:, t, h] = lc
        x, _ = O.merge_values(outs, lses)
        scale = np.abs(fulls).max()
        assert np.all(np.abs(x - fulls) <= 1e-12 * scale), f"merge != unsplit attention for {sizes}"
        # the same through bf16 partials and float32 LSEs
        ob = bf16_bits_from_f32(np.nan_to_num(outs, nan=0.0).astype(np.float32))
        ob = np.where(np.isnan(outs), np.uint16(0x7FC0), ob)
        xb, _ = O.merge_values(O.bf16_to_f64(ob), lses.astype(np.float32))
        assert np.all(np.abs(xb - fulls) <= 2.0**-8 * scale), f"bf16 partials drift for {sizes}"


def pin_single_partial_identity():
    """I2: one partial with a finite LSE is returned bit for bit; with an LSE
    of -inf, NaN or +inf it is dropped and the latents are +0. Without an LSE
    the row itself is the latent row."""
    rng = np.random.default_rng(12)
    o, lse = _dense_case(rng, 1, 3)
    codes, scales = _random_wv(rng)
    g = _gate(rng, 3)
    r = O.mla_post(o, lse, codes, scales, g)
    assert np.array_equal(r["lat"], o[0]), "single finite partial must be the identity"
    r0 = O.mla_post(o, None, codes, scales, g)
    assert np.array_equal(r0["lat"], o[0]), "no-LSE row must be the identity"
    assert np.array_equal(r0["core"], r["core"])
    for bad in (-np.inf, np.nan, np.inf):
        rb = O.mla_post(o, np.full_like(lse, bad), codes, scales, g)
        assert np.all(rb["lat"] == 0), f"single partial with LSE {bad} must give +0 latents"


def pin_all_empty_zero():
    """I3: when every LSE of a (t, h) is -inf, NaN or +inf the latents and that
    head's 128 core columns are exactly +0, and the scale code is 1."""
    rng = np.random.default_rng(13)
    o, lse = _dense_case(rng, 4, 3)
    choices = np.array([-np.inf, np.nan, np.inf], dtype=np.float32)
    lse[:, 1, 5] = choices[rng.integers(0, 3, size=4)]
    lse[:, 2, :] = -np.inf
    codes, scales = _random_wv(rng)
    r = O.mla_post(o, lse, codes, scales, _gate(rng, 3))
    for t, hs in ((1, [5]), (2, range(12))):
        for h in hs:
            assert np.all(r["lat"][t, h] == 0)
            assert np.all(r["codes"][t, h] == 0) and np.all(r["scales"][t, h] == 1)
            assert np.all(r["core"][t, 128 * h : 128 * h + 128] == 0)
    assert np.any(r["lat"][0] != 0)
    # the weights themselves: all zero (not NaN) when every partial is empty
    for row in ([-np.inf] * 4, [-np.inf]):
        w, e = O.merge_weights(np.array(row))
        assert np.all(w == 0.0) and np.all(e == 0.0), "an all-empty row must give zero weights"


def pin_permutation():
    """I4: permuting the partials (rows together with their LSEs) changes the
    float64 merge only by rounding; the bf16 latents agree in >= 99.99% and
    are never more than 1 ulp apart."""
    rng = np.random.default_rng(14)
    o, lse = _dense_case(rng, 8, 16)
    lse[rng.random(lse.shape) < 0.1] = -np.inf
    perm = rng.permutation(8)
    x1, mag = O.merge(o, lse)
    x2, _ = O.merge(o[perm], lse[perm])
    assert np.all(np.abs(x1 - x2) <= 1e-14 * np.maximum(mag, 1e-300))
    l1, l2 = O.rne_bf16(x1), O.rne_bf16(x2)
    eq = np.mean(l1 == l2)
    assert eq >= 0.9999
    d = np.abs(O.bf16_to_f64(l1) - O.bf16_to_f64(l2))
    assert np.all(d <= O.ulp_bf16(np.maximum(np.abs(x1), np.abs(x2))))


def pin_shift_invariance():
    """I5: adding one constant to all LSEs of a (t, h) leaves the merge
    unchanged up to rounding."""
    rng = np.random.default_rng(15)
    o, lse = _dense_case(rng, 6, 8)
    lse[rng.random(lse.shape) < 0.15] = -np.inf
    x0, mag = O.merge(o, lse)
    for c in (-50.0, 3.7, 60.0):
        x1, _ = O.merge(o, lse.astype(np.float64) + c)
        assert np.all(np.abs(x1 - x0) <= 1e-12 * np.maximum(mag, 1e-300)), f"shift {c}"


def pin_equal_weights_average():
    """I6: two partials with equal finite LSEs merge to their exact average."""
    rng = np.random.default_rng(16)
    o, lse = _dense_case(rng, 2, 4)
    lse[1] = lse[0]
    x, _ = O.merge(o, lse)
    expect = (O.bf16_to_f64(o[0]) + O.bf16_to_f64(o[1])) / 2.0  # exact in float64
    assert np.array_equal(x, expect)
    assert np.array_equal(O.rne_bf16(x), O.rne_bf16(expect))


def pin_nan_inf_as_neg_inf():
    """I7: a NaN or +inf LSE behaves exactly as -inf."""
    rng = np.random.default_rng(17)
    o, lse = _dense_case(rng, 5, 6)
    mask = rng.random(lse.shape) < 0.3
    ref = lse.copy()
    ref[mask] = -np.inf
    for bad in (np.nan, np.inf):
        alt = lse.copy()
        alt[mask] = bad
        x0, _ = O.merge(o, ref)
        x1, _ = O.merge(o, alt)
        assert np.array_equal(x0, x1), f"LSE {bad} differs from -inf"


def pin_dead_rows_ignored():
    """I8: NaN or inf stored in partials of weight 0 does not reach the result."""
    rng = np.random.default_rng(18)
    o, lse = _dense_case(rng, 4, 6)
    lse[1] = -np.inf
    lse[2, :, ::2] = np.nan
    x0, _ = O.merge(o, lse)
    o2 = o.copy()
    o2[1] = 0x7FC0  # NaN
    o2[2, :, ::2] = 0x7F80  # +inf
    x1, _ = O.merge(o2, lse)
    assert np.array_equal(x0, x1)
    assert np.all(np.isfinite(x1))


def pin_dcp_gather_view():
    """The decode-context-parallel view: rank r's partial of local head h is
    gathered head r*12 + h, read through (sj, st, sh) strides; checked against
    an explicit loop over the gathered buffer."""
    import synth

    w = synth.dcp_gathered("t", 3, 5, seed=1, head_stride_rows=40, dead_from=4)
    v = w.o_view()
    buf = w.o_buf
    for r in range(3):
        for t in range(5):
            for h in range(12):
                assert np.array_equal(v[r, t, h], buf[t, r * 12 + h])
    lv = w.lse_view()
    for r in range(3):
        for t in range(5):
            for h in range(12):
                a, b = lv[r, t, h], w.lse_buf[t, r * 12 + h]
                assert (a == b) or (np.isnan(a) and np.isnan(b))


# ---------------------------------------------------------------- bf16 pins


def pin_rne_bf16_vs_torch():
    """rne_bf16 agrees with torch's CPU float32 -> bfloat16 cast on structured
    patterns around every tie and on random float32 bit patterns, for every
    exponent including subnormals and overflow."""
    exps = np.arange(0, 255, dtype=np.uint32)
    low = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    mid = np.array([0x00, 0x01, 0x7E, 0x7F], dtype=np.uint32)
    pats = (exps[:, None, None] << 23) | (mid[None, :, None] << 16) | low[None, None, :]
    pats = pats.reshape(-1)
    pats = np.concatenate([pats, pats | 0x80000000])
    rng = np.random.default_rng(19)
    rnd = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    rnd = rnd[((rnd >> 23) & 0xFF) != 0xFF]
    allp = np.concatenate([pats, rnd])
    f = allp.view(np.float32)
    got = O.rne_bf16(f.astype(np.float64))
    ref = torch_bf16_bits(f)
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} mismatches vs torch"
    # bf16 -> float64 -> bf16 is the identity on every non-NaN pattern
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ok = ~np.isnan(O.bf16_to_f64(b))
    assert np.array_equal(O.rne_bf16(O.bf16_to_f64(b))[ok], b[ok])


def pin_rne_bf16_exact_rational():
    """On float64 inputs that are not float32 values (where torch's cast cannot
    be used without double rounding), rne_bf16 and rne_bf16_fraction agree with
    a search over every finite bf16 value using exact rational distances."""
    rng = np.random.default_rng(20)
    vals = []
    for _ in range(300):
        e = int(rng.integers(-140, 130))
        m = 1.0 + rng.random()
        vals.append(np.ldexp(m, e) * (1 if rng.random() < 0.5 else -1))
    # exact ties and near-ties in float64
    for e in (-133, -130, -126, -1, 0, 5, 127):
        for k in (1, 3, 255):
            base = np.ldexp(float(k) + 0.5, e - 7)
            vals += [base, np.nextafter(base, np.inf), np.nextafter(base, -np.inf)]
    vals += [3.4e38, 3.39e38, -1e-45, 0.0, -0.0]
    x = np.array(vals, dtype=np.float64)
    got = O.rne_bf16(x)
    for v, g in zip(x, got):
        ref = brute_rne_bf16(Fraction(float(v)))
        if v == 0:
            ref = 0x8000 if np.signbit(v) else 0
        assert int(g) == ref, f"rne_bf16({v!r}) = {int(g):#06x}, brute {ref:#06x}"
        if v != 0:
            assert O.rne_bf16_fraction(Fraction(float(v))) == ref


# ---------------------------------------------------------------- quantiser pins


def _expected_nibbles_integer(bits: np.ndarray, code: int) -> np.ndarray:
    """Nibble of x / 2^(code-127) by exact integer comparisons of 4|y| with 4x
    the E2M1 midpoints (a formulation independent of the oracle's)."""
    b = bits.astype(np.int64)
    eb = (b >> 7) & 0xFF
    m = b & 0x7F
    N = np.where(eb > 0, 128 + m, m)
    sh = np.where(eb > 0, eb - 134, -133) + 127 - code + 2  # 4y = N * 2^sh
    nib = np.zeros(b.shape, dtype=np.int64)
    for k, mu in enumerate(MIDS4):  # midpoint between codes k and k+1
        upper_even = (k + 1) % 2 == 0
        pos = sh >= 0
        lhs = np.where(pos, N << np.minimum(np.maximum(sh, 0), 40), N)
        rhs = np.where(pos, mu, mu << np.minimum(np.maximum(-sh, 0), 50))
        passed = (lhs > rhs) | ((lhs == rhs) & upper_even)
        nib += passed
    return (nib | (((b >> 15) & 1) << 3)).astype(np.uint8)


def pin_e2m1_exhaustive():
    """Q1: for every finite bf16 pattern and every scale code 1..254 the
    oracle's element encoder equals the integer-midpoint formulation; a random
    sample also equals nearest-by-exact-rational-distance."""
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    x = O.bf16_to_f64(b)
    for code in range(1, 255):
        got = O.e2m1_nibble(x / np.ldexp(1.0, code - 127))
        exp = _expected_nibbles_integer(b, code)
        assert np.array_equal(got, exp), f"code {code}: {np.sum(got != exp)} mismatches"
    rng = np.random.default_rng(21)
    grid = [Fraction(v).limit_denominator(4) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    for _ in range(3000):
        bit = int(rng.choice(b))
        code = int(rng.integers(1, 255))
        v = Fraction(float(O.bf16_to_f64(np.uint16(bit)))) / (Fraction(2) ** (code - 127))
        a = abs(v)
        d = [abs(a - g) for g in grid]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        idx = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        expect = idx | (8 if (bit >> 15) & 1 else 0)
        got = int(O.e2m1_nibble(np.float64(v))[()])
        assert got == expect, f"bits {bit:#06x} code {code}: {got} vs {expect}"


def pin_scale_rule_closed_form():
    """Q2: over all 32768 bf16 magnitude patterns (as the block maximum), the
    scale code equals max(1, 125 + floor(log2(8 amax / 7))) computed with exact
    rationals (8/7 amax reaches the next power of two exactly when the mantissa
    fraction is >= 0.75), and the largest scaled magnitude of an unclamped
    block lies in [3.5, 7)."""
    mags = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    blocks = np.zeros((mags.size, 32), dtype=np.uint16)
    blocks[:, 7] = mags
    blocks[:, 3] = mags >> 1  # a smaller element must not matter
    got = O.e8m0_even(blocks)
    vals = O.bf16_to_f64(mags)
    for i in range(mags.size):
        a = Fraction(float(vals[i]))
        if a == 0:
            exp = 1
        else:
            t = a * 8 / 7
            e = t.numerator.bit_length() - t.denominator.bit_length()
            if Fraction(2) ** e > t:
                e -= 1
            exp = max(1, 125 + e)
        assert int(got[i]) == exp, f"amax {mags[i]:#06x}: {int(got[i])} vs {exp}"
        if exp > 1:
            y = a / (Fraction(2) ** (exp - 127))
            assert Fraction(7, 2) <= y < 7


def pin_round_trip_and_bound():
    """Q3: E2M1 grid values times a power-of-two scale survive quantise ->
    dequantise exactly. Q4: otherwise the error is at most half the grid step
    at that magnitude times the scale (1 scale unit in the (6, 7) band)."""
    rng = np.random.default_rng(22)
    tab = load_e2m1_table()
    for code in (3, 100, 125, 140, 250):
        s = 2.0 ** (code - 127)
        nib = rng.integers(0, 16, size=(64, 32))
        nib[:, 0] = 7  # put 6 in every block so the scale is this code
        vals = np.array([[tab[int(c)] for c in row] for row in nib]) * s
        bits = O.rne_bf16(vals)
        assert np.array_equal(O.bf16_to_f64(bits), vals)
        codes, scales = O.quantize_mxfp4(bits)
        # 6*s has fraction 0.5: code = E + 0 - 2 with 6 = 1.5 * 2^2 -> the block code
        assert np.all(scales == code)
        assert np.array_equal(O.dequant_mxfp4(codes, scales), vals)
    x = rng.standard_normal((256, 512)) * np.exp(rng.uniform(-8, 8, size=(256, 1)))
    bits = O.rne_bf16(x)
    codes, scales = O.quantize_mxfp4(bits)
    deq = O.dequant_mxfp4(codes, scales)
    xb = O.bf16_to_f64(bits)
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    y = np.abs(xb) / s
    halfstep = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    assert np.all(np.abs(deq - xb) <= halfstep * s)
    assert np.all(np.sign(deq) * np.sign(xb) >= 0)


def pin_quant_golden():
    """Q5: hand-derived blocks (tests/golden/mxfp4_blocks.txt) and the E2M1
    table (tests/golden/e2m1_table.txt)."""
    for name, code, x, out in load_golden_blocks():
        c, s = O.quantize_mxfp4(x[None])
        assert int(s[0, 0]) == code, f"{name}: scale {int(s[0, 0])} vs {code}"
        assert np.array_equal(c[0], out), f"{name}: codes {c[0]} vs {out}"
    tab = load_e2m1_table()
    codes = np.array([[c | (c << 4) for c in range(16)]], dtype=np.uint8)  # byte = same code twice
    v2 = O.e2m1_twice(codes)[0]
    deq = O.dequant_mxfp4(np.array([[c | (c << 4) for c in range(16)]], np.uint8), np.array([127], np.uint8))[0]
    for c in range(16):
        assert v2[2 * c] == v2[2 * c + 1] == int(round(2 * tab[c])), f"code {c}"
        assert deq[2 * c] == tab[c], f"code {c}"


# ---------------------------------------------------------------- W_UV and gate pins


def pin_wuv_vs_blas():
    """U1: the exact block-scaled contraction agrees with a float64 BLAS matmul
    of the dequantised operands (a library routine); its bf16 rounding equals
    the rounding of the matmul except at ties, and is never 1 ulp off."""
    rng = np.random.default_rng(23)
    T = 6
    lat = O.rne_bf16(rng.standard_normal((T, O.NH, O.KVL)) * np.exp(rng.uniform(-3, 3, size=(T, O.NH, 1))))
    lc, ls = O.quantize_mxfp4(lat)
    wc, ws = _random_wv(rng)
    acc_bf, acc = O.wuv_exact(lc, ls, wc, ws)
    Ld = O.dequant_mxfp4(lc, ls)  # [T,12,512]
    Wd = O.dequant_mxfp4(wc, ws)  # [12,128,512]
    ref = np.stack([Ld[:, h, :] @ Wd[h].T for h in range(O.NH)], axis=1)  # [T,12,128]
    absum = np.stack([np.abs(Ld[:, h, :]) @ np.abs(Wd[h]).T for h in range(O.NH)], axis=1)
    assert np.all(np.abs(acc - ref) <= 1e-13 * absum + 1e-300)
    rb = O.rne_bf16(ref)
    assert np.mean(rb == acc_bf) > 0.999
    d = np.abs(O.bf16_to_f64(rb) - O.bf16_to_f64(acc_bf))
    assert np.all(d <= O.ulp_bf16(ref))


def pin_wuv_one_hot():
    """U2: W_V rows that are one-hot (value 1.0 at position k(h, v)) pick the
    dequantised latent at k(h, v): pins the nibble order of W_V, its row and
    head mapping and the scale exponent bias. An all-zero W_V gives +0."""
    rng = np.random.default_rng(24)
    T = 3
    lat = O.rne_bf16(rng.standard_normal((T, O.NH, O.KVL)))
    lc, ls = O.quantize_mxfp4(lat)
    Ld = O.dequant_mxfp4(lc, ls)
    wc = np.zeros((O.NH, O.VD, O.KVL // 2), dtype=np.uint8)
    ws = np.full((O.NH, O.VD, O.KVL // 32), 127, dtype=np.uint8)
    ks = np.zeros((O.NH, O.VD), dtype=np.int64)
    for h in range(O.NH):
        for v in range(O.VD):
            k = (h * 37 + v * 11) % O.KVL
            ks[h, v] = k
            wc[h, v, k // 2] = 0x2 if k % 2 == 0 else 0x20  # code 2 = 1.0
    acc_bf, _ = O.wuv_exact(lc, ls, wc, ws)
    for h in range(O.NH):
        for v in range(O.VD):
            assert np.array_equal(O.bf16_to_f64(acc_bf[:, h, v]), Ld[:, h, ks[h, v]])
    ws2 = ws.copy()
    ws2[:, :, :] = 129  # scale 4
    acc4, _ = O.wuv_exact(lc, ls, wc, ws2)
    assert np.array_equal(O.bf16_to_f64(acc4), 4 * O.bf16_to_f64(acc_bf))
    z, _ = O.wuv_exact(lc, ls, np.zeros_like(wc), ws)
    assert np.all(z == 0)
    # a hand-computed case: latents 1.0 (code 125, element code 6 = 4, 4 * 2^-2 = 1),
    # W_V all 1.0 -> every output is 512 = bf16 0x4400
    lc1, ls1 = O.quantize_mxfp4(np.full((1, O.NH, O.KVL), 0x3F80, dtype=np.uint16))
    wc1 = np.full((O.NH, O.VD, O.KVL // 2), 0x22, dtype=np.uint8)
    a1, _ = O.wuv_exact(lc1, ls1, wc1, ws)
    assert np.all(a1 == 0x4400)


def pin_gate_core():
    """U3: core column 128 h + v holds W_UV output (h, v) times the gate there;
    a gate of 1 returns the W_UV result, doubling the gate doubles core, and
    the hand case 512 * 0.5 = 256 (bf16 0x4380)."""
    rng = np.random.default_rng(25)
    T = 5
    acc = O.rne_bf16(rng.standard_normal((T, O.NH, O.VD)))
    ones = np.full((T, O.NH * O.VD), 0x3F80, dtype=np.uint16)
    c1 = O.gate_core(acc, ones)
    for c in range(O.NH * O.VD):
        assert np.array_equal(c1[:, c], acc[:, c // 128, c % 128])
    g = O.rne_bf16(rng.random((T, O.NH * O.VD)))
    g2 = O.rne_bf16(2.0 * O.bf16_to_f64(g))
    assert np.array_equal(O.bf16_to_f64(O.gate_core(acc, g2)), 2.0 * O.bf16_to_f64(O.gate_core(acc, g)))
    hand = O.gate_core(np.full((1, O.NH, O.VD), 0x4400, np.uint16), np.full((1, O.NH * O.VD), 0x3F00, np.uint16))
    assert np.all(hand == 0x4380)


def pin_ulp_bf16_brute():
    """The tolerance helper's bf16 spacing against the gaps between adjacent
    bf16 values: for every non-negative finite bf16 pattern b, the value of
    b + 1 minus the value of b (past the largest finite value, the gap to
    2^128), at the value itself, strictly inside the gap (its midpoint) and
    for the negative value; zero has the smallest subnormal's spacing,
    2^-133."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)  # +0 .. the largest finite value
    vals = (bits << 16).view(np.float32).astype(np.float64)
    nxt = np.append(vals[1:], 2.0**128)
    gap = nxt - vals
    assert np.array_equal(O.ulp_bf16(vals), gap)
    assert np.array_equal(O.ulp_bf16(vals + gap / 2), gap)
    assert np.array_equal(O.ulp_bf16(-vals), gap)
    assert O.ulp_bf16(0.0) == 2.0**-133 and O.ulp_bf16(-0.0) == 2.0**-133
    # hand values: 1 and 1.5 lie in [1, 2), spacing 2^-7; 2 starts the next binade
    assert np.array_equal(O.ulp_bf16(np.array([1.0, 1.5, 2.0, 2.0**-126, 2.0**-130])),
                          np.array([2.0**-7, 2.0**-7, 2.0**-6, 2.0**-133, 2.0**-133]))


def pin_end_to_end_small():
    """The whole oracle on a tiny case equals a scalar walk-through built from
    the pinned pieces (BLAS for the contraction), per token and head."""
    rng = np.random.default_rng(26)
    o, lse = _dense_case(rng, 3, 2)
    lse[0, 0, 0] = -np.inf
    wc, ws = _random_wv(rng)
    g = _gate(rng, 2)
    r = O.mla_post(o, lse, wc, ws, g)
    Wd = O.dequant_mxfp4(wc, ws)
    for t in range(2):
        for h in range(O.NH):
            ls = [float(lse[j, t, h]) for j in range(3)]
            m = max(ls)
            e = [np.exp(v - m) for v in ls]
            w = [v / sum(e) for v in e]
            x = sum(w[j] * O.bf16_to_f64(o[j, t, h]) for j in range(3) if w[j] > 0)
            lat = O.rne_bf16(x)
            assert np.array_equal(lat, r["lat"][t, h])
            lc, lsc = O.quantize_mxfp4(lat[None])
            acc = Wd[h] @ O.dequant_mxfp4(lc, lsc)[0]
            # the float64 BLAS sum of the dequantised products is exact here:
            # every product is a multiple of the smallest block's quantum and
            # the blocks' scales span far less than 53 bits
            core = O.rne_bf16(O.bf16_to_f64(O.rne_bf16(acc)) * O.bf16_to_f64(g[t, 128 * h : 128 * h + 128]))
            assert np.array_equal(core, r["core"][t, 128 * h : 128 * h + 128])


def pin_request_major_gather():
    """The page's request-major split layout: token t takes slices
    (t // q) * per + j, checked against explicit loops; with one request the
    gather is the identity; slices of other requests (NaN-filled) are never
    read by the merge."""
    rng = np.random.default_rng(27)
    for P, S, q in ((6, 6, 2), (8, 4, 4), (12, 12, 3), (5, 5, 5)):
        R = S // q
        per = P // R
        o_all = rng.standard_normal((P, S, 2, 3))
        l_all = rng.standard_normal((P, S, 2))
        o, l = O.gather_request_major(o_all, l_all, q)
        assert o.shape == (per, S, 2, 3) and l.shape == (per, S, 2)
        for j in range(per):
            for t in range(S):
                assert np.array_equal(o[j, t], o_all[(t // q) * per + j, t])
                assert np.array_equal(l[j, t], l_all[(t // q) * per + j, t])
        if R == 1:
            assert np.array_equal(o, o_all)
    # foreign slices poisoned with NaN: the merged latents stay finite
    P, S, q = 8, 8, 2
    R, per = S // q, P // (S // q)
    o_all = np.full((P, S, O.NH, O.KVL), 0x7FC0, dtype=np.uint16)
    lse_all = np.full((P, S, O.NH), np.nan, dtype=np.float32)
    vals = bf16_bits_from_f32(rng.standard_normal((per, S, O.NH, O.KVL)).astype(np.float32))
    lv = rng.uniform(-2, 6, size=(per, S, O.NH)).astype(np.float32)
    for t in range(S):
        for j in range(per):
            o_all[(t // q) * per + j, t] = vals[j, t]
            lse_all[(t // q) * per + j, t] = lv[j, t]
    o, l = O.gather_request_major(o_all, lse_all, q)
    x, _ = O.merge(o, l)
    x_ref, _ = O.merge(vals, lv)
    assert np.array_equal(x, x_ref) and np.all(np.isfinite(x))


def pin_push_mask():
    """Push-side masking: a partial whose request has no KV there, or a token
    past the batch, merges exactly as if its LSE were -inf; checked against
    loops; tokens past the batch give +0 latents."""
    rng = np.random.default_rng(28)
    n, S, q = 3, 12, 4
    R = S // q
    o, lse = _dense_case(rng, n, S)
    kv = rng.integers(0, 3, size=(n, R)).astype(np.int32)  # zeros mark requests without KV
    qsl = np.array([0, 4, 8, 10], dtype=np.int32)  # 10 live tokens of 12
    m = O.push_mask(lse, q, kv, qsl)
    ref = lse.astype(np.float64).copy()
    for j in range(n):
        for t in range(S):
            if kv[j, t // q] == 0 or t >= qsl[R]:
                ref[j, t] = -np.inf
    assert np.array_equal(m, ref)
    x, _ = O.merge(o, m)
    assert np.all(O.rne_bf16(x)[10:] == 0)
    assert np.array_equal(O.push_mask(lse, q), lse.astype(np.float64))  # no masks: unchanged


# ---------------------------------------------------------------- o_proj


def _oproj_case(rng, S, D, K, sigma=1.0):
    core = bf16_bits_from_f32(rng.standard_normal((S, K)) * sigma)
    w = bf16_bits_from_f32(rng.standard_normal((D, K)) / np.sqrt(K))
    return core, w


def pin_oproj_exact_rational():
    """o_proj against exact rational arithmetic: every output of a small
    case is the exact sum of its K products of bf16 values (Fractions),
    rounded to bf16 by search over every bf16 value; includes a case whose
    products span more than 37 binades (values from 2^-40 to 2^30)."""
    from oracle.oproj import oproj

    rng = np.random.default_rng(40)
    cases = [_oproj_case(rng, 3, 5, 64)]
    core = bf16_bits_from_f32(rng.standard_normal((2, 32)) * np.exp2(rng.integers(-40, 30, size=(2, 32))))
    w = bf16_bits_from_f32(rng.standard_normal((3, 32)))
    cases.append((core, w))
    for core, w in cases:
        r = oproj(core, w)
        a, b = O.bf16_to_f64(core), O.bf16_to_f64(w)
        for t in range(core.shape[0]):
            for d in range(w.shape[0]):
                exact = sum((Fraction(float(a[t, k])) * Fraction(float(b[d, k])) for k in range(core.shape[1])), Fraction(0))
                assert int(r["out"][t, d]) == brute_rne_bf16(exact), (t, d)
                assert abs(Fraction(float(r["y"][t, d])) - exact) <= Fraction(1, 2**50) * abs(Fraction(float(r["mag"][t, d])))


def pin_oproj_known_answers():
    """One-hot rows of W_O pick a column of core exactly (row d of W_O = 1.0
    at k = (7 d) mod K); a zero core row gives +0; doubling core doubles
    every output; out[t, d] takes row t of core and row d of W_O (a
    transposed operand fails on a non-square case)."""
    from oracle.oproj import oproj

    rng = np.random.default_rng(41)
    S, D, K = 4, 6, 96
    core, w = _oproj_case(rng, S, D, K)
    core[2] = 0
    one = np.zeros((D, K), np.uint16)
    for d in range(D):
        one[d, (7 * d) % K] = 0x3F80
    r = oproj(core, one)
    for d in range(D):
        assert np.array_equal(r["out"][:, d], core[:, (7 * d) % K])
    r = oproj(core, w)
    assert np.all(r["out"][2] == 0)
    c2 = O.rne_bf16(2.0 * O.bf16_to_f64(core))
    assert np.array_equal(O.bf16_to_f64(oproj(c2, w)["out"]), 2.0 * O.bf16_to_f64(r["out"]))
    # a row of W_O with a single 2.0 at k = 0 and a core row of ones except
    # k = 0: only the product at k = 0 counts
    w2 = np.zeros((D, K), np.uint16)
    w2[3, 0] = 0x4000
    c3 = np.full((S, K), 0x3F80, np.uint16)
    c3[:, 0] = O.rne_bf16(np.arange(S, dtype=np.float64) + 1)
    r3 = oproj(c3, w2)
    assert np.array_equal(O.bf16_to_f64(r3["out"][:, 3]), 2.0 * (np.arange(S) + 1))
    assert np.all(r3["out"][:, [0, 1, 2, 4, 5]] == 0)


# ---------------------------------------------------------------- the split-KV attention (producer)


def _attn_case(rng, lens, q, sigma_q=1.0):
    import oracle.attention as A

    R = len(lens)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    kv = bf16_bits_from_f32(rng.standard_normal((int(indptr[-1]), A.DQK)))
    qry = bf16_bits_from_f32(rng.standard_normal((R * q, A.NH, A.DQK)) * sigma_q)
    return qry, kv, indptr


def pin_attention_split_equals_unsplit():
    """Merging a request's split partials (float64, the merge's own
    definition) gives its unsplit attention, for split counts that leave some
    splits empty; the unsplit attention equals a scalar walk-through (scores,
    softmax, weighted sum of the 512 value dims) written out with loops."""
    import oracle.attention as A

    rng = np.random.default_rng(50)
    qry, kv, indptr = _attn_case(rng, [7, 0, 3, 20], q=2)
    scale = 1.0 / np.sqrt(192.0)
    one = A.attention_partials(qry, kv, indptr, 2, 1, scale)
    for per in (2, 3, 5, 9):
        sp = A.attention_partials(qry, kv, indptr, 2, per, scale)
        R = indptr.size - 1
        for r in range(R):
            x, _ = O.merge_values(sp["o"][r], sp["lse"][r])  # [q, 12, 512]
            ref = one["o"][r, 0]
            assert np.all(np.abs(x - ref) <= 1e-12 * max(1.0, np.abs(ref).max())), (per, r)
    # scalar walk-through for request 2 (3 rows), token 1, heads 0 and 7
    qv, kvv = O.bf16_to_f64(qry), O.bf16_to_f64(kv)
    for h in (0, 7):
        t = 2 * 2 + 1
        rows = range(int(indptr[2]), int(indptr[3]))
        sc = [scale * sum(qv[t, h, d] * kvv[i, d] for d in range(A.DQK)) for i in rows]
        mx = max(sc)
        ws = [np.exp(v - mx) for v in sc]
        out = [sum(ws[n] * kvv[i, d] for n, i in enumerate(rows)) / sum(ws) for d in range(A.KVL)]
        assert np.allclose(one["o"][2, 0, 1, h], out, rtol=1e-12, atol=1e-12)
        assert abs(one["lse"][2, 0, 1, h] - (mx + np.log(sum(ws)))) <= 1e-12


def pin_attention_bounds_empty_single():
    """Split bounds are floor(j L / per) (hand values); a split without rows
    has LSE -inf and a zero partial; a split of one row returns that row's
    latent part exactly, with its score as LSE."""
    import oracle.attention as A

    assert list(A.split_bounds(10, 4)) == [0, 2, 5, 7, 10]
    assert list(A.split_bounds(3, 5)) == [0, 0, 1, 1, 2, 3]
    assert list(A.split_bounds(0, 2)) == [0, 0, 0]
    rng = np.random.default_rng(51)
    qry, kv, indptr = _attn_case(rng, [3], q=1)
    p = A.attention_partials(qry, kv, indptr, 1, 5, 0.1)
    for j, n in enumerate(np.diff(A.split_bounds(3, 5))):
        if n == 0:
            assert np.all(p["lse"][0, j] == -np.inf) and np.all(p["o"][0, j] == 0)
        else:
            i = int(A.split_bounds(3, 5)[j])
            assert np.array_equal(p["o_bits"][0, j, 0], np.broadcast_to(kv[i, : A.KVL], (A.NH, A.KVL)))
            s = 0.1 * O.bf16_to_f64(qry)[0] @ O.bf16_to_f64(kv)[i]
            assert np.allclose(p["lse"][0, j, 0], s, rtol=0, atol=1e-12)


def pin_attention_rotary_dims_and_scale():
    """The 64 rotary dims enter the scores but never the values: with the
    query's rotary dims zero, changing the cache's rotary dims changes
    nothing; with them set, it changes the LSEs. Doubling the scale equals
    doubling the query."""
    import oracle.attention as A

    rng = np.random.default_rng(52)
    qry, kv, indptr = _attn_case(rng, [6, 9], q=2)
    q0 = qry.copy()
    q0[..., A.KVL :] = 0
    kv2 = kv.copy()
    kv2[:, A.KVL :] = bf16_bits_from_f32(rng.standard_normal((kv.shape[0], A.DQK - A.KVL)) * 5)
    a = A.attention_partials(q0, kv, indptr, 2, 2, 0.07)
    b = A.attention_partials(q0, kv2, indptr, 2, 2, 0.07)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    c = A.attention_partials(qry, kv, indptr, 2, 2, 0.07)
    d = A.attention_partials(qry, kv2, indptr, 2, 2, 0.07)
    assert not np.allclose(c["lse"], d["lse"])
    q2 = O.rne_bf16(2.0 * O.bf16_to_f64(qry))
    e = A.attention_partials(q2, kv, indptr, 2, 2, 0.07)
    f = A.attention_partials(qry, kv, indptr, 2, 2, 0.14)
    assert np.allclose(e["o"], f["o"], rtol=1e-12, atol=1e-13) and np.allclose(e["lse"], f["lse"], rtol=1e-12)


ALL_PINS = [
    pin_textbook_attention,
    pin_single_partial_identity,
    pin_all_empty_zero,
    pin_permutation,
    pin_shift_invariance,
    pin_equal_weights_average,
    pin_nan_inf_as_neg_inf,
    pin_dead_rows_ignored,
    pin_dcp_gather_view,
    pin_rne_bf16_vs_torch,
    pin_rne_bf16_exact_rational,
    pin_e2m1_exhaustive,
    pin_scale_rule_closed_form,
    pin_round_trip_and_bound,
    pin_quant_golden,
    pin_wuv_vs_blas,
    pin_wuv_one_hot,
    pin_gate_core,
    pin_end_to_end_small,
    pin_ulp_bf16_brute,
    pin_request_major_gather,
    pin_push_mask,
    pin_oproj_exact_rational,
    pin_oproj_known_answers,
    pin_attention_split_equals_unsplit,
    pin_attention_bounds_empty_single,
    pin_attention_rotary_dims_and_scale,
]
