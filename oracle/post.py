"""Plain float64 CPU oracle of the MLA decode post-attention step (``mla_post``).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table or
constant with the HIP library; only the seeded input generators in ``synth``
serve both sides.

Source of truth: the vLLM API-docs page for the module
``vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back``.
Citations below have the form ``[mla_back: <section>]``, where the section is
the page's module docstring or one of the functions whose source it shows.

What is computed, for every token t and head h (12 heads, latent 512, 128
value rows per head):

1. the LSE-weighted merge of the N bf16 partial rows o[j, t, h, :] (natural-log
   LSEs, NaN and +inf treated as -inf, a zero-weight row contributes nothing);
   with N == 1 and no LSE the single row is the attention output itself;
2. round-to-nearest-even to bf16 latents;
3. MXFP4 quantisation of each block of 32 latents (E8M0 block scale chosen by
   the "even" rule, E2M1 elements rounded to nearest, ties to the even code,
   saturating at 6);
4. the exact block-scaled FP4 dot product with W_V[h] (128 x 512, MXFP4);
5. bf16 rounding of that dot product, times the bf16 gate, rounded to bf16:
   ``core[t, 128 h + v]``.

All arithmetic is float64 or exact integer arithmetic; bf16 values are carried
as their uint16 bit patterns. Readings of steps the page leaves open (the scale
rule, the element rounding, nibble order, RNE everywhere) are stated where they
are used. Every function here has a pin in ``tests/pins.py`` that
checks it against something other than itself.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

NH = 12  # heads per rank            [mla_back: mla_post] (core is [S, 1536] = 12 x 128)
KVL = 512  # latent width            [mla_back: module docstring] (o [S, ranks x 12, 512])
VD = 128  # value rows per head      [mla_back: mla_post] (w_v (12, 128, 256))
BLK = 32  # MXFP4 block              (OCP microscaling: 32 elements share one E8M0 scale)
NBLK = KVL // BLK  # 16 scale blocks along the latent

# E2M1 magnitudes indexed by the 3-bit code (OCP MX v1.0, element type FP4 E2M1).
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# --------------------------------------------------------------------------
# bf16 <-> float64
# --------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def rne_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even), exactly.

    Reading: every bf16 rounding on the page (the packed latents in
    [mla_back: combine_ranks], [mla_back: combine_splits]; the rounding of the
    MFMA result and of the gated product in [mla_back: stage_uv]) is IEEE
    round-to-nearest-even with gradual underflow and overflow to infinity.

    The value is split as a * 2^q, with q the quantum of bf16 at |x| (8
    significant bits, or 2^-133 below the normal range); a is then an exactly
    representable float64 < 512 and ``np.rint`` rounds it half-to-even.
    Negative inputs keep their sign, so a negative value that rounds to zero
    gives -0. NaN maps to the quiet NaN 0x7FC0 (sign kept).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    a = np.abs(np.where(nan, 0.0, x))
    _, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    q = np.maximum(e - 8, -133)  # quantum exponent
    r = np.rint(np.ldexp(a, -q))  # exact scaling, then round half to even
    val = np.ldexp(r, q)
    with np.errstate(over="ignore"):
        f32 = val.astype(np.float32)  # exact for bf16 values; >= 2^128 -> inf
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    sign = np.signbit(x).astype(np.uint16) << 15
    out[...] = bits | sign
    out[nan] = np.uint16(0x7FC0) | sign[nan]
    return out


def rne_bf16_fraction(v: Fraction) -> int:
    """Scalar exact RNE of a rational to a bf16 bit pattern (fallback for
    exact sums whose span does not fit a float64)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 7, -133)
    scaled = a / (Fraction(2) ** q)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * (Fraction(2) ** q)
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = int(np.float32(float(val)).view(np.uint32)) >> 16
    return sign | bits


# --------------------------------------------------------------------------
# Step 1: LSE sanitising and merge weights
# --------------------------------------------------------------------------


def sanitize_lse(lse) -> np.ndarray:
    """NaN and +inf LSEs become -inf ([mla_back: sane]); float64 out."""
    v = np.asarray(lse, dtype=np.float64).copy()
    v[np.isnan(v) | (v == np.inf)] = -np.inf
    return v


def merge_weights(lse) -> tuple[np.ndarray, np.ndarray]:
    """Merge weights over the last axis of sanitised natural-log LSEs.

    [mla_back: combine_ranks] and [mla_back: combine_splits]: m is the largest
    LSE, replaced by 0 when every LSE is -inf; e_j = exp(lse_j - m) (the page
    evaluates it as exp2 of (lse_j - m) * log2(e), i.e. natural-log LSEs);
    the weight is e_j / sum(e); a partial with e_j == 0 gets weight 0, and
    when the sum is 0 (every partial empty) all weights are 0.

    Returns (w, e), both float64 with the input's shape.
    """
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(axis=-1, keepdims=True)
    m = np.where(m == -np.inf, 0.0, m)
    e = np.exp(lse - m)  # exp(-inf) == 0 exactly
    tot = e.sum(axis=-1, keepdims=True)
    safe = np.where(tot == 0.0, 1.0, tot)
    w = np.where((tot == 0.0) | (e == 0.0), 0.0, e / safe)
    return w, e


def merge_values(o, lse):
    """Step 1 on float64 partial values o [N, T, 12, K] and LSEs [N, T, 12].

    x[k] = sum over j with w_j > 0 of w_j * o_j[k]. Rows of weight 0 are
    excluded outright, so NaN or inf stored in an empty partial cannot reach
    the result ([mla_back: combine_ranks] masks such rows;
    [mla_back: combine_splits] relies on empty splits holding zeros; one rule
    covers both).

    The sum starts at +0, as the page's float32 accumulators do, so a merge
    whose terms are all zero (every weight 0, or live rows holding +-0) is +0.

    Returns (x, mag): x [T, 12, K] float64, and mag = sum_j w_j |o_j[k]|, the
    size of the terms the merge cancels (used by tolerances).
    """
    o = np.asarray(o, dtype=np.float64)
    w, _ = merge_weights(np.moveaxis(sanitize_lse(lse), 0, -1))  # [T, 12, N]
    w = np.moveaxis(w, -1, 0)[..., None]  # [N, T, 12, 1]
    live = w > 0.0
    oz = np.where(live, o, 0.0)
    x = 0.0 + np.where(live, w * oz, 0.0).sum(axis=0)
    mag = np.where(live, w * np.abs(oz), 0.0).sum(axis=0)
    return x, mag


def merge(o_bits, lse):
    """Step 1 on bf16 partials: o_bits uint16 [N, T, 12, 512], lse [N, T, 12]
    or None.

    With ``lse is None`` (N must be 1) the row is the attention output itself
    and is returned unchanged ([mla_back: stage_combine], the copy taken when
    there is one rank and no splits). Otherwise ``merge_values``.
    """
    o = bf16_to_f64(o_bits)
    if lse is None:
        if o.shape[0] != 1:
            raise ValueError("without LSEs there must be exactly one partial")
        return o[0].copy(), np.abs(o[0])
    return merge_values(o, lse)


# --------------------------------------------------------------------------
# Step 3: MXFP4 quantisation of bf16 rows
# --------------------------------------------------------------------------


def e8m0_even(block_bits) -> np.ndarray:
    """E8M0 scale code of a block of 32 bf16 values (the last axis).

    [mla_back: stage_uv]: the block maximum is taken over the 15-bit bf16
    magnitude patterns, the code is the page's "even" scale of that maximum,
    and codes below 1 are raised to 1. The page does not show the even rule.
    Reading (the common "even" mode of MXFP4 scale selection): write the
    maximum as (1 + f) 2^E; the maximum is first rounded up to the next power
    of two when f >= 0.75, then E2M1's largest exponent (2) is taken off:
    code = E_biased + [f >= 0.75] - 2. In bit form, adding 0x20 to the
    magnitude pattern carries into the exponent exactly when the top two of the
    seven mantissa bits are set.
    """
    mag = (np.asarray(block_bits, dtype=np.uint16) & 0x7FFF).astype(np.int64)
    amax = mag.max(axis=-1)
    code = ((amax + 0x20) >> 7) - 2
    return np.maximum(code, 1)


def e2m1_nibble(y) -> np.ndarray:
    """E2M1 code (4-bit nibble) of exact float64 quotients y = x / scale.

    Reading of the page's packed bf16 -> FP4 conversion ([mla_back: stage_uv]):
    the magnitude goes to the nearest E2M1 value, a tie goes to the value with
    the even code, values above 6 saturate to 6 (E2M1 has no inf or NaN), and
    the sign bit is the sign bit of x, so a negative value that rounds to zero
    gives the code 0x8 (-0).
    """
    y = np.asarray(y, dtype=np.float64)
    # Every magnitude >= 6 has 6 as its nearest value, so clamping at 8 changes
    # no result; it keeps the distances below exact (for huge |y| the float64
    # differences |y| - g would all round to |y| and fake a tie).
    a = np.minimum(np.abs(y), 8.0)
    d = np.abs(a[..., None] - E2M1_MAG)  # distance to each of the 8 magnitudes
    best = d.min(axis=-1, keepdims=True)
    hit = d == best  # one, or (at a midpoint) two adjacent codes
    codes = np.arange(8)
    # at a tie the two candidates are adjacent codes: keep the even one
    even_hit = hit & (codes % 2 == 0)
    idx = np.where(even_hit.any(axis=-1), np.argmax(even_hit, axis=-1), np.argmax(hit, axis=-1))
    return (idx | (np.signbit(y).astype(np.int64) << 3)).astype(np.uint8)


def quantize_mxfp4(bits):
    """Step 3: bf16 rows (last axis a multiple of 32) -> (codes, scales).

    Per block of 32: the E8M0 code c (``e8m0_even``), the scale 2^(c - 127),
    each element's E2M1 nibble of x / scale (exact in float64: x is bf16 and
    the scale a power of two). Packing: element 2i goes to the low nibble of
    byte i, element 2i+1 to the high nibble (the OCP order; on the page a
    16-byte W_V operand carries 32 consecutive latent positions,
    [mla_back: wv_loads]).

    Returns codes uint8 [..., K/2] and scales uint8 [..., K/32].
    """
    bits = np.asarray(bits, dtype=np.uint16)
    K = bits.shape[-1]
    if K % BLK:
        raise ValueError("row length must be a multiple of 32")
    blocks = bits.reshape(bits.shape[:-1] + (K // BLK, BLK))
    code = e8m0_even(blocks)  # [..., K/32]
    scale = np.ldexp(1.0, code - 127)[..., None]
    nib = e2m1_nibble(bf16_to_f64(blocks) / scale).reshape(bits.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, code.astype(np.uint8)


def e2m1_twice(codes) -> np.ndarray:
    """Unpack MXFP4 code bytes to 2 * element value as int64 (exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    nib = np.stack([c & 0xF, c >> 4], axis=-1).reshape(c.shape[:-1] + (2 * c.shape[-1],))
    mag2 = (2 * E2M1_MAG).astype(np.int64)[nib & 7]
    return np.where(nib & 8, -mag2, mag2)


def dequant_mxfp4(codes, scales) -> np.ndarray:
    """MXFP4 codes and E8M0 scales -> float64 values (exact)."""
    v2 = e2m1_twice(codes).astype(np.float64)
    K = v2.shape[-1]
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (v2.reshape(v2.shape[:-1] + (K // BLK, BLK)) * 0.5 * s[..., None]).reshape(v2.shape)


# --------------------------------------------------------------------------
# Step 4: W_UV, the block-scaled FP4 contraction, computed exactly
# --------------------------------------------------------------------------


def wuv_exact(lat_codes, lat_scales, w_codes, w_scales):
    """acc2[t, h, v] = sum_k W_V[h, v, k] * L[t, h, k] with both operands
    MXFP4, computed exactly; returns its bf16 rounding (uint16) and, for
    diagnostics, a float64 approximation of the exact value.

    [mla_back: stage_uv] runs this as scaled FP4 MFMAs of W_V[h]'s rows
    against the quantised latents; the module docstring names the op
    _v_up_proj. Per block b the integer dot product of the doubled E2M1
    values (at most 32 * 12 * 12 in size) is scaled by
    2^(sw - 127) * 2^(c - 127) / 4. The blocks are summed at a common exponent;
    when that integer fits a float64 mantissa the sum is exact in float64 and
    rounded once to bf16, otherwise the element is summed with Python integers.

    lat_codes [T, 12, 256] u8, lat_scales [T, 12, 16] u8,
    w_codes [12, 128, 256] u8, w_scales [12, 128, 16] u8.
    """
    L2 = e2m1_twice(lat_codes).reshape(lat_codes.shape[:-1] + (NBLK, BLK))  # [T,12,16,32]
    W2 = e2m1_twice(w_codes).reshape(w_codes.shape[:-1] + (NBLK, BLK))  # [12,128,16,32]
    # P[t, h, v, b] = sum_{k in b} W2[h, v, b, k] * L2[t, h, b, k]: integers < 2^13,
    # so the float64 matmul is exact whatever order BLAS sums in
    Lb = np.transpose(L2, (1, 2, 0, 3)).astype(np.float64)  # [12,16,T,32]
    Wb = np.transpose(W2, (0, 2, 3, 1)).astype(np.float64)  # [12,16,32,128]
    P = np.transpose(np.matmul(Lb, Wb), (2, 0, 3, 1))  # [T,12,128,16]
    P = np.rint(P).astype(np.int64)
    ex = (
        np.asarray(w_scales, dtype=np.int64)[None, :, :, :]
        + np.asarray(lat_scales, dtype=np.int64)[:, :, None, :]
        - 254
        - 2
    )  # [T,12,128,16]: block b contributes P * 2^ex
    big = np.where(P != 0, ex, np.iinfo(np.int64).max)
    emin = big.min(axis=-1, keepdims=True)
    emin = np.where(emin == np.iinfo(np.int64).max, 0, emin)
    span = np.where(P != 0, ex - emin, 0)
    safe = span.max(axis=-1) <= 36  # 16 * 2^13 * 2^36 < 2^53
    sh = np.where(safe[..., None], span, 0)
    Ssum = (P * (np.int64(1) << sh)).sum(axis=-1)  # exact int64
    approx = np.ldexp(Ssum.astype(np.float64), emin[..., 0])
    acc_bf = rne_bf16(approx)  # single rounding: approx is exact where safe
    if not safe.all():
        for idx in zip(*np.nonzero(~safe)):
            tot = Fraction(0)
            for b in range(NBLK):
                p = int(P[idx + (b,)])
                if p:
                    tot += Fraction(p) * (Fraction(2) ** int(ex[idx + (b,)]))
            acc_bf[idx] = rne_bf16_fraction(tot)
            approx[idx] = float(tot)
    return acc_bf, approx


def gate_core(acc_bf, gate_bits) -> np.ndarray:
    """Step 5: core[t, 128 h + v] = bf16(acc_bf[t, h, v] * gate[t, 128 h + v]).

    [mla_back: stage_uv]: the MFMA result is rounded to bf16, multiplied by
    the gate element of column h * 128 + v and packed to bf16. The product of
    two bf16 values is exact in float64, so one rounding remains.
    """
    T = acc_bf.shape[0]
    a = bf16_to_f64(acc_bf).reshape(T, NH * VD)
    g = bf16_to_f64(gate_bits).reshape(T, NH * VD)
    return rne_bf16(a * g)


# --------------------------------------------------------------------------
# Request-major split partials and push-side masking
# --------------------------------------------------------------------------


def gather_request_major(o_all, lse_all, q: int):
    """The page's split layout ([mla_back: combine_splits]): the partials of
    all requests sit in one dense tensor of P split slices, o_all
    [P, S, 12, 512] and lse_all [P, S, 12], request-major; with R = S / q
    requests of q tokens and per = P / R splits each, token t merges slices
    (t // q) * per + j for j < per. Returns the per-token views o [per, S,
    12, 512] and lse [per, S, 12] that ``mla_post`` takes.
    """
    P, S = o_all.shape[0], o_all.shape[1]
    if S % q:
        raise ValueError("S must be a whole number of requests")
    R = S // q
    if P % R:
        raise ValueError("the split slices must divide evenly among the requests")
    per = P // R
    t = np.arange(S)
    idx = (t // q)[None, :] * per + np.arange(per)[:, None]  # [per, S]
    o = np.asarray(o_all)[idx, t[None, :]]
    lse = np.asarray(lse_all)[idx, t[None, :]]
    return o, lse


def push_mask(lse, q: int, kv_lens=None, qsl=None):
    """Push-side masking of partial LSEs ([mla_back: stage_push]): the partial
    of token t is empty, its LSE -inf, when the request t // q has no KV in
    that partial (kv_lens[j, t // q] == 0; kv_lens [n, R], one row per
    partial) or when t lies past the batch (t >= qsl[S // q], qsl the R + 1
    query start offsets). Returns a float64 copy of lse [n, S, 12].
    """
    v = np.asarray(lse, dtype=np.float64).copy()
    n, S = v.shape[0], v.shape[1]
    t = np.arange(S)
    if kv_lens is not None:
        kv = np.asarray(kv_lens).reshape(n, -1)
        empty = kv[:, t // q] == 0  # [n, S]
        v[empty] = -np.inf
    if qsl is not None:
        rows = int(np.asarray(qsl)[S // q])
        v[:, t >= rows] = -np.inf
    return v


# --------------------------------------------------------------------------
# The whole step
# --------------------------------------------------------------------------


def mla_post(o_bits, lse, w_codes, w_scales, gate_bits, tokens=None) -> dict:
    """The oracle for one ``mla_post`` call (steps 1-5).

    o_bits   uint16 [N, S, 12, 512]  bf16 partials (any numpy strides; for the
             decode-context-parallel layout, rank r's partial of local head h
             is gathered head r * 12 + h, [mla_back: stage_push])
    lse      float32 [N, S, 12] natural-log LSEs, or None when N == 1 and the
             single row is the final attention output
    w_codes  uint8 [12, 128, 256] MXFP4 W_V; w_scales uint8 [12, 128, 16]
    gate     uint16 [S, 1536] bf16
    tokens   optional token indices: only those rows are computed

    Returns a dict of per-stage results for the selected tokens:
    x (float64 merge), mag, lat (bf16 bits), codes, scales, acc_bf (bf16 bits
    of the W_UV result), acc (float64), core (bf16 bits [T, 1536]).
    """
    if tokens is not None:
        tokens = np.asarray(tokens)
        o_bits = o_bits[:, tokens]
        lse = None if lse is None else lse[:, tokens]
        gate_bits = gate_bits[tokens]
    x, mag = merge(o_bits, lse)
    if lse is None:
        lat = np.asarray(o_bits[0], dtype=np.uint16).copy()  # identity, bit for bit
    else:
        lat = rne_bf16(x)
    codes, scales = quantize_mxfp4(lat)
    acc_bf, acc = wuv_exact(codes, scales, w_codes, w_scales)
    core = gate_core(acc_bf, gate_bits)
    return dict(x=x, mag=mag, lat=lat, codes=codes, scales=scales, acc_bf=acc_bf, acc=acc, core=core)


def ulp_bf16(a) -> np.ndarray:
    """Spacing of bf16 values at magnitude |a| (float64): 2^(e - 7) for |a| in
    [2^e, 2^(e+1)) with e >= -126, and 2^-133 below 2^-126 (the subnormal
    range, zero included). Used by the acceptance tolerances.

    ``np.frexp`` gives exponent 0 for a zero input, which would read as the
    spacing at 0.5; zero takes the subnormal spacing explicitly.
    """
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(a)
    e = np.where(a == 0.0, -133 + 8, e)
    return np.ldexp(1.0, np.maximum(e - 8, -133))


__all__ = [
    "NH",
    "KVL",
    "VD",
    "BLK",
    "E2M1_MAG",
    "bf16_to_f64",
    "rne_bf16",
    "rne_bf16_fraction",
    "sanitize_lse",
    "merge_weights",
    "merge_values",
    "merge",
    "e8m0_even",
    "e2m1_nibble",
    "quantize_mxfp4",
    "e2m1_twice",
    "dequant_mxfp4",
    "wuv_exact",
    "gate_core",
    "gather_request_major",
    "push_mask",
    "mla_post",
    "ulp_bf16",
]
