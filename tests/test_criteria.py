"""The acceptance criteria themselves (CPU only): planted GPU-side mistakes
that each check must reject, on a small oracle case whose own outputs pass.

The 'GPU results' here are the oracle's own stage outputs with one element
changed, so each test shows that a criterion sees that kind of wrong value
(a NaN, a small value where the merge is exactly zero, a flipped sign)."""

import numpy as np
import pytest

import criteria as C
import oracle.post as O
import synth


@pytest.fixture(scope="module")
def case():
    # 24 splits, 90% of the LSEs -inf: many (token, head) pairs have no live partial
    w = synth.dense_splits("criteria", 24, 6, seed=3, p_neg_inf=0.9)
    wc, ws = O.quantize_mxfp4(w.wv_bits)
    ref = O.mla_post(w.o_view(), w.lse_view(), wc, ws, w.gate)
    assert np.any(np.all(ref["mag"] == 0, axis=-1)), "the case must hold all-empty heads"
    return w, wc, ws, ref


def _all(case, lat=None, core=None):
    w, wc, ws, ref = case
    lat = ref["lat"] if lat is None else lat
    codes, scales = O.quantize_mxfp4(lat)
    core = ref["core"] if core is None else core
    C.check_t1(lat, ref)
    C.check_t2(lat, codes, scales)
    C.check_t3(core, codes, scales, wc, ws, w.gate)
    C.check_t4(core, ref, lat, codes, scales)


def test_oracle_outputs_pass(case):
    _all(case)


def _live_index(ref):
    t, h, k = np.argwhere(ref["mag"] > 0)[0]
    return t, h, k


def _empty_index(ref):
    t, h = np.argwhere(np.all(ref["mag"] == 0, axis=-1))[0]
    return t, h


def test_t1_rejects_nan_latent(case):
    ref = case[3]
    lat = ref["lat"].copy()
    lat[_live_index(ref)] = 0x7FC0
    with pytest.raises(AssertionError, match="T1"):
        C.check_t1(lat, ref)


def test_t1_rejects_small_value_in_empty_head(case):
    ref = case[3]
    lat = ref["lat"].copy()
    t, h = _empty_index(ref)
    lat[t, h, :] = O.rne_bf16(np.full(512, 0.003))
    with pytest.raises(AssertionError, match="T1"):
        C.check_t1(lat, ref)


def test_t1_rejects_negative_zero_in_empty_head(case):
    ref = case[3]
    lat = ref["lat"].copy()
    t, h = _empty_index(ref)
    lat[t, h, 5] = 0x8000
    with pytest.raises(AssertionError, match="T1"):
        C.check_t1(lat, ref)


def test_t3_rejects_nan_core(case):
    w, wc, ws, ref = case
    core = ref["core"].copy()
    t, h, _ = _live_index(ref)
    core[t, 128 * h + 3] = 0x7FC0
    with pytest.raises(AssertionError, match="T3"):
        C.check_t3(core, ref["codes"], ref["scales"], wc, ws, w.gate)


def test_t4_rejects_nan_core(case):
    ref = case[3]
    core = ref["core"].copy()
    t, h, _ = _live_index(ref)
    core[t, 128 * h + 3] = 0x7FC0
    with pytest.raises(AssertionError, match="T4"):
        C.check_t4(core, ref, ref["lat"], ref["codes"], ref["scales"])


def test_t4_rejects_nonzero_core_in_empty_head(case):
    ref = case[3]
    core = ref["core"].copy()
    t, h = _empty_index(ref)
    core[t, 128 * h + 7] = 0x0001  # the smallest subnormal: far inside 2e-2 RMS of the row
    with pytest.raises(AssertionError, match="T4"):
        C.check_t4(core, ref, ref["lat"], ref["codes"], ref["scales"])


def test_t5_accepts_float32_sums_and_rejects_mistakes():
    """T5 (o_proj): a float32 sum rounded to bf16 (numpy's float32 matrix
    product, another summation order) passes; a NaN, an output missing its
    largest product, a transposed result and a truncating final rounding
    fail."""
    from oracle.oproj import oproj

    rng = np.random.default_rng(5)
    S, D, K = 9, 40, 1536
    core = synth.f32_to_bf16_bits(rng.standard_normal((S, K), dtype=np.float32))
    w = synth.f32_to_bf16_bits(rng.standard_normal((D, K), dtype=np.float32) / np.float32(40))
    ref = oproj(core, w)
    a, b = O.bf16_to_f64(core), O.bf16_to_f64(w)
    f32 = a.astype(np.float32) @ b.astype(np.float32).T
    got = synth.f32_to_bf16_bits(f32)
    C.check_t5(got, ref, K)
    bad = got.copy()
    bad[2, 3] = 0x7FC0
    with pytest.raises(AssertionError, match="T5"):
        C.check_t5(bad, ref, K)
    bad = got.copy()
    terms = a[4] * b[5]
    kmax = int(np.argmax(np.abs(terms)))
    bad[4, 5] = O.rne_bf16(ref["y"][4, 5] - terms[kmax])
    with pytest.raises(AssertionError, match="T5"):
        C.check_t5(bad, ref, K)
    sq = oproj(core, w[:S])  # square S x S
    t = synth.f32_to_bf16_bits((a.astype(np.float32) @ b[:S].astype(np.float32).T).T)
    with pytest.raises(AssertionError, match="T5"):
        C.check_t5(t, sq, K)
    trunc = (f32.view(np.uint32) >> 16).astype(np.uint16)
    with pytest.raises(AssertionError, match="T5"):
        C.check_t5(trunc, ref, K)
