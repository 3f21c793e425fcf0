"""Planted mistakes in the oracle (CPU only): each must make one of the named
pins fail, which shows the pins can see that kind of mistake."""

import numpy as np
import pytest

import oracle.post as O
import pins

_orig = {n: getattr(O, n) for n in dir(O) if callable(getattr(O, n))}

import oracle.oproj as OP  # noqa: E402

_orig_oproj = OP.oproj


def _sanitize_no_posinf(lse):
    v = np.asarray(lse, dtype=np.float64).copy()
    v[np.isnan(v)] = -np.inf
    return v


def _sanitize_no_nan(lse):
    v = np.asarray(lse, dtype=np.float64).copy()
    v[v == np.inf] = -np.inf
    return v


def _weights_no_m_reset(lse):
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.exp(lse - m)
    tot = e.sum(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        w = np.where(e == 0.0, 0.0, e / tot)
    return w, e


def _weights_exp2(lse):
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(axis=-1, keepdims=True)
    m = np.where(m == -np.inf, 0.0, m)
    e = np.exp2(lse - m)
    tot = e.sum(axis=-1, keepdims=True)
    safe = np.where(tot == 0.0, 1.0, tot)
    return np.where((tot == 0.0) | (e == 0.0), 0.0, e / safe), e


def _weights_unnormalised(lse):
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(axis=-1, keepdims=True)
    m = np.where(m == -np.inf, 0.0, m)
    e = np.exp(lse - m)
    return e, e


def _merge_values_no_mask(o, lse):
    o = np.asarray(o, dtype=np.float64)
    w, _ = O.merge_weights(np.moveaxis(O.sanitize_lse(lse), 0, -1))
    w = np.moveaxis(w, -1, 0)[..., None]
    with np.errstate(invalid="ignore"):
        return (w * o).sum(axis=0), (w * np.abs(o)).sum(axis=0)


def _rne_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _rne_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint16) << 15
    a = np.abs(x)
    _, e = np.frexp(a)
    q = np.maximum(e - 8, -133)
    s = np.ldexp(a, -q)
    r = np.floor(s + 0.5)
    with np.errstate(over="ignore"):
        f32 = np.ldexp(r, q).astype(np.float32)
    return ((f32.view(np.uint32) >> 16).astype(np.uint16)) | sign


def _e8m0_floor(block_bits):
    mag = (np.asarray(block_bits, dtype=np.uint16) & 0x7FFF).astype(np.int64)
    return np.maximum((mag.max(axis=-1) >> 7) - 2, 1)


def _e8m0_no_clamp(block_bits):
    mag = (np.asarray(block_bits, dtype=np.uint16) & 0x7FFF).astype(np.int64)
    return np.maximum(((mag.max(axis=-1) + 0x20) >> 7) - 2, 0)


def _e2m1_ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 8.0)
    d = np.abs(a[..., None] - O.E2M1_MAG)
    best = d.min(axis=-1, keepdims=True)
    hit = d == best
    idx = 7 - np.argmax(hit[..., ::-1], axis=-1)  # the larger candidate
    return (idx | (np.signbit(y).astype(np.int64) << 3)).astype(np.uint8)


def _e2m1_plus_zero(y):
    n = _orig["e2m1_nibble"](y)
    return np.where((n & 7) == 0, 0, n).astype(np.uint8)


def _quant_swapped_nibbles(bits):
    c, s = _orig["quantize_mxfp4"](bits)
    return ((c >> 4) | (c << 4)).astype(np.uint8), s


def _wuv_bias_off(lc, ls, wc, ws):
    return _orig["wuv_exact"](lc, ls, wc, np.minimum(np.asarray(ws, np.int64) + 1, 254).astype(np.uint8))


def _wuv_rows_reversed(lc, ls, wc, ws):
    return _orig["wuv_exact"](lc, ls, wc[:, ::-1], ws[:, ::-1])


def _gate_transposed(acc_bf, gate_bits):
    T = acc_bf.shape[0]
    a = O.bf16_to_f64(acc_bf).transpose(0, 2, 1).reshape(T, O.NH * O.VD)
    return O.rne_bf16(a * O.bf16_to_f64(gate_bits).reshape(T, -1))


def _gather_shifted(o_all, lse_all, q):
    P, S = o_all.shape[0], o_all.shape[1]
    per = P // (S // q)
    t = np.arange(S)
    idx = np.minimum(((t + 1) // q)[None, :] * per + np.arange(per)[:, None], P - 1)
    return np.asarray(o_all)[idx, t[None, :]], np.asarray(lse_all)[idx, t[None, :]]


def _push_mask_token_index(lse, q, kv_lens=None, qsl=None):
    v = np.asarray(lse, dtype=np.float64).copy()
    n, S = v.shape[0], v.shape[1]
    t = np.arange(S)
    if kv_lens is not None:
        kv = np.asarray(kv_lens).reshape(n, -1)
        v[kv[:, np.minimum(t, kv.shape[1] - 1)] == 0] = -np.inf  # request index taken as t
    if qsl is not None:
        v[:, t >= int(np.asarray(qsl)[S // q])] = -np.inf
    return v


def _ulp_frexp_at_zero(a):
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(a)  # exponent 0 for a zero input: reads as the spacing at 0.5
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def _ulp_exponent_off_by_one(a):
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(a)
    e = np.where(a == 0.0, -125, e)
    return np.ldexp(1.0, np.maximum(e - 7, -133))


def _oproj_w_transposed(core_bits, w_bits, rows=None):
    w = np.asarray(w_bits)
    return _orig_oproj(core_bits, w.reshape(w.shape[1], w.shape[0]).T.copy(), rows)


def _oproj_truncated(core_bits, w_bits, rows=None):
    r = _orig_oproj(core_bits, w_bits, rows)
    f = r["y"].astype(np.float32)
    r["out"] = (f.view(np.uint32) >> 16).astype(np.uint16)
    return r


def _oproj_f32_products(core_bits, w_bits, rows=None):
    r = _orig_oproj(core_bits, w_bits, rows)
    r["out"] = O.rne_bf16(r["y"].astype(np.float16).astype(np.float64))  # a half-precision sum
    return r


MUTATIONS = [
    ("sanitize misses +inf", "sanitize_lse", _sanitize_no_posinf, [pins.pin_nan_inf_as_neg_inf]),
    ("sanitize misses NaN", "sanitize_lse", _sanitize_no_nan, [pins.pin_nan_inf_as_neg_inf]),
    ("max not reset when all empty", "merge_weights", _weights_no_m_reset, [pins.pin_all_empty_zero]),
    ("base-2 LSEs", "merge_weights", _weights_exp2, [pins.pin_textbook_attention]),
    ("weights not normalised", "merge_weights", _weights_unnormalised, [pins.pin_textbook_attention]),
    ("dead rows not masked", "merge_values", _merge_values_no_mask, [pins.pin_dead_rows_ignored]),
    ("bf16 by truncation", "rne_bf16", _rne_truncate, [pins.pin_rne_bf16_vs_torch]),
    ("bf16 ties away", "rne_bf16", _rne_ties_away, [pins.pin_rne_bf16_vs_torch]),
    ("floor scale rule", "e8m0_even", _e8m0_floor, [pins.pin_scale_rule_closed_form, pins.pin_quant_golden]),
    ("scale not raised to 1", "e8m0_even", _e8m0_no_clamp, [pins.pin_quant_golden]),
    ("E2M1 ties away", "e2m1_nibble", _e2m1_ties_away, [pins.pin_quant_golden]),
    ("E2M1 loses -0", "e2m1_nibble", _e2m1_plus_zero, [pins.pin_quant_golden]),
    ("nibble order swapped", "quantize_mxfp4", _quant_swapped_nibbles, [pins.pin_quant_golden]),
    ("scale bias off by one", "wuv_exact", _wuv_bias_off, [pins.pin_wuv_one_hot]),
    ("W_V rows reversed", "wuv_exact", _wuv_rows_reversed, [pins.pin_wuv_one_hot]),
    ("gate columns transposed", "gate_core", _gate_transposed, [pins.pin_gate_core]),
    ("request index off by one", "gather_request_major", _gather_shifted, [pins.pin_request_major_gather]),
    ("mask uses token not request", "push_mask", _push_mask_token_index, [pins.pin_push_mask]),
    ("ulp of zero from frexp", "ulp_bf16", _ulp_frexp_at_zero, [pins.pin_ulp_bf16_brute]),
    ("ulp exponent off by one", "ulp_bf16", _ulp_exponent_off_by_one, [pins.pin_ulp_bf16_brute]),
]

import oracle.attention as AT  # noqa: E402

_orig_attn = AT.attention_partials
_orig_bounds = AT.split_bounds


def _attn_rope_values(qry_bits, kv_bits, indptr, q, per, scale):
    kv = np.asarray(kv_bits).copy()
    kv[:, : AT.KVL] = np.concatenate([kv[:, AT.DQK - AT.KVL :]], axis=1)  # values read from the last 512 dims
    r = _orig_attn(qry_bits, kv_bits, indptr, q, per, scale)
    r2 = _orig_attn(qry_bits, kv, indptr, q, per, scale)
    r["o"], r["o_bits"] = r2["o"], r2["o_bits"]
    return r


def _attn_lse_base2(qry_bits, kv_bits, indptr, q, per, scale):
    r = _orig_attn(qry_bits, kv_bits, indptr, q, per, scale)
    r["lse"] = r["lse"] / np.log(2.0)
    r["lse_f32"] = r["lse"].astype(np.float32)
    return r


def _bounds_ceil(L, per):
    return np.array([-((-j * L) // per) for j in range(per + 1)], dtype=np.int64)


def _attn_no_scale(qry_bits, kv_bits, indptr, q, per, scale):
    return _orig_attn(qry_bits, kv_bits, indptr, q, per, 1.0)


ATTN_MUTATIONS = [
    ("values from the rotary end", "attention_partials", _attn_rope_values, [pins.pin_attention_rotary_dims_and_scale]),
    ("LSE in base 2", "attention_partials", _attn_lse_base2, [pins.pin_attention_split_equals_unsplit]),
    ("split bounds rounded up", "split_bounds", _bounds_ceil, [pins.pin_attention_bounds_empty_single]),
    ("scale ignored", "attention_partials", _attn_no_scale, [pins.pin_attention_rotary_dims_and_scale]),
]


@pytest.mark.parametrize("name,attr,fn,catchers", ATTN_MUTATIONS, ids=[m[0] for m in ATTN_MUTATIONS])
def test_attention_mutation_is_caught(monkeypatch, name, attr, fn, catchers):
    monkeypatch.setattr(AT, attr, fn)
    caught = []
    for pin in catchers:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{name}' passed every pin in {[p.__name__ for p in catchers]}"


OPROJ_MUTATIONS = [
    ("W_O read transposed", _oproj_w_transposed, [pins.pin_oproj_known_answers]),
    ("o_proj rounded by truncation", _oproj_truncated, [pins.pin_oproj_exact_rational]),
    ("o_proj summed in half precision", _oproj_f32_products, [pins.pin_oproj_exact_rational]),
]


@pytest.mark.parametrize("name,attr,fn,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, attr, fn, catchers):
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in catchers:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{name}' passed every pin in {[p.__name__ for p in catchers]}"


@pytest.mark.parametrize("name,fn,catchers", OPROJ_MUTATIONS, ids=[m[0] for m in OPROJ_MUTATIONS])
def test_oproj_mutation_is_caught(monkeypatch, name, fn, catchers):
    monkeypatch.setattr(OP, "oproj", fn)
    caught = []
    for pin in catchers:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{name}' passed every pin in {[p.__name__ for p in catchers]}"
