"""Acceptance criteria of the HIP path against the CPU oracle.

T1  latents: |lat_gpu - x| <= ulp_bf16(max(|x|, 2^-8 M)) per element, x the
    oracle's exact float64 merge and M = sum_j w_j |o_j| (the floor covers
    cancellation: float32 accumulation error is about (n + 6) 2^-24 M, which
    exceeds one bf16 ulp of a nearly cancelled |x|). Where M == 0 (every
    term of the merge is zero: a (token, head) whose partials are all empty)
    the latent must be +0 bit for bit, as the merge's sum starts at +0.
    Without LSEs: exact.

Every comparison is written so that a NaN on the GPU side counts as a
failure: an element passes only when its error is known to be within the
bound.
T2  MXFP4 codes and scales: the oracle's quantiser applied to the GPU's own
    latents reproduces the GPU's codes and scales bit for bit.
T3  core given the GPU's codes: the oracle's exact W_UV + gate on the GPU's
    codes/scales; every element within max(2e-2 RMS_row, 1 ulp_bf16(|ref|))
    (float32 accumulation order inside the MFMA can move the bf16 rounding
    of the dot product by one ulp).
T4  core end to end (oracle from o and lse): global relative RMS error
    <= 2e-2, and each row over 2e-2 RMS_row must hold a block whose GPU and
    oracle latents differ and whose codes differ (a 1-ulp latent difference
    that crosses an E2M1 rounding boundary moves the whole block). With
    ``strict`` every row must be within 2e-2 RMS_row.
"""

from __future__ import annotations

import numpy as np

import oracle.post as O


def rms_rows(core_bits: np.ndarray) -> np.ndarray:
    v = O.bf16_to_f64(core_bits)
    return np.sqrt(np.mean(v * v, axis=-1))


def check_t1(lat_gpu, ref, exact: bool = False) -> dict:
    x, mag = ref["x"], ref["mag"]
    g = O.bf16_to_f64(lat_gpu)
    if exact:
        bad = lat_gpu != ref["lat"]
        assert not bad.any(), f"T1 exact: {int(bad.sum())} latents differ"
        return {"t1_bad": 0, "t1_strict_ulp": 0}
    tol = O.ulp_bf16(np.maximum(np.abs(x), 2.0**-8 * mag))
    with np.errstate(invalid="ignore"):
        err = np.abs(g - x)
        bad = ~(err <= tol)
        strict = ~(np.abs(g - O.bf16_to_f64(ref["lat"])) <= O.ulp_bf16(x))
    assert not bad.any(), f"T1: {int(bad.sum())} latents outside tolerance (max err/tol {float(np.nanmax(err / tol)):.3g})"
    zero = mag == 0
    zbad = zero & (np.asarray(lat_gpu, dtype=np.uint16) != 0)
    assert not zbad.any(), f"T1: {int(zbad.sum())} latents of all-zero merges are not +0"
    return {"t1_bad": 0, "t1_strict_ulp": int(strict.sum()), "t1_diff_latents": int((lat_gpu != ref["lat"]).sum()),
            "t1_zero_latents": int(zero.sum())}


def check_t2(lat_gpu, codes_gpu, scales_gpu) -> dict:
    c, s = O.quantize_mxfp4(lat_gpu)
    bs = s != scales_gpu
    bc = c != codes_gpu
    assert not bs.any(), f"T2: {int(bs.sum())} scale codes differ"
    assert not bc.any(), f"T2: {int(bc.sum())} code bytes differ"
    return {"t2_blocks": int(s.size)}


def check_t3(core_gpu, codes_gpu, scales_gpu, w_codes, w_scales, gate) -> dict:
    acc_bf, _ = O.wuv_exact(codes_gpu, scales_gpu, w_codes, w_scales)
    ref = O.gate_core(acc_bf, gate)
    rv, gv = O.bf16_to_f64(ref), O.bf16_to_f64(core_gpu)
    rms = rms_rows(ref)[:, None]
    tol = np.maximum(2e-2 * rms, O.ulp_bf16(rv))
    with np.errstate(invalid="ignore"):
        err = np.abs(gv - rv)
        bad = ~(err <= tol)
    assert not bad.any(), f"T3: {int(bad.sum())} core elements outside tolerance"
    ulps = np.where(err > 0, err / O.ulp_bf16(rv), 0)
    return {
        "t3_exact_frac": float(np.mean(core_gpu == ref)),
        "t3_max_ulp": float(ulps.max()) if ulps.size else 0.0,
        "t3_needed_ulp_term": int(np.sum(err > 2e-2 * rms)),
    }


def check_t4(core_gpu, ref, lat_gpu=None, codes_gpu=None, scales_gpu=None, strict: bool = False) -> dict:
    rv, gv = O.bf16_to_f64(ref["core"]), O.bf16_to_f64(core_gpu)
    rms = rms_rows(ref["core"])
    with np.errstate(invalid="ignore"):
        err = np.abs(gv - rv)
    zero_rows = rms == 0
    assert np.all(err[zero_rows] == 0), "T4: rows the oracle makes exactly zero must be exactly zero"
    # a (token, head) whose merge is all zero (all partials empty) has +0
    # latents, codes 0 and scale code 1, so its 128 columns are bf16(+0 x gate):
    # the oracle's bits exactly
    empty = np.all(ref["mag"] == 0, axis=-1)  # [T, 12]
    if empty.any():
        cg = np.asarray(core_gpu, dtype=np.uint16).reshape(empty.shape + (O.VD,))
        cr = np.asarray(ref["core"], dtype=np.uint16).reshape(empty.shape + (O.VD,))
        ebad = empty & np.any(cg != cr, axis=-1)
        assert not ebad.any(), f"T4: {int(ebad.sum())} all-empty (token, head) slices of core are not exact"
    with np.errstate(invalid="ignore"):
        row_bad = np.any(~(err <= 2e-2 * rms[:, None]), axis=-1) & ~zero_rows
    denom = np.sqrt(np.mean(rv * rv))
    rel_rms = float(np.sqrt(np.mean((gv - rv) ** 2)) / denom) if denom > 0 else 0.0
    assert rel_rms <= 2e-2, f"T4: global relative RMS error {rel_rms:.3g}"
    if strict:
        assert not row_bad.any(), f"T4 strict: {int(row_bad.sum())} rows over 2e-2 RMS"
    elif row_bad.any():
        assert lat_gpu is not None and codes_gpu is not None, "T4: rows over tolerance and no stage outputs to explain them"
        for t in np.nonzero(row_bad)[0]:
            with np.errstate(invalid="ignore"):
                cols = np.nonzero(~(err[t] <= 2e-2 * rms[t]))[0]
            for h in np.unique(cols // 128):
                lat_diff = (lat_gpu[t, h] != ref["lat"][t, h]).reshape(16, 32).any(-1)
                code_diff = (codes_gpu[t, h] != ref["codes"][t, h]).reshape(16, 16).any(-1)
                if scales_gpu is not None:
                    code_diff |= scales_gpu[t, h] != ref["scales"][t, h]
                assert np.any(lat_diff & code_diff), f"T4: token {t} head {h} off with no flipped code"
    return {"t4_rows_over": int(row_bad.sum()), "t4_rel_rms": rel_rms, "t4_empty_heads": int(empty.sum())}


def check_all(o, lse, w_codes, w_scales, gate, g, exact_t1: bool = False, strict_t4: bool = False,
              max_elems: int = 1 << 23) -> dict:
    """T1-T4 on every token of a call, the oracle run over consecutive token
    chunks so that host memory stays bounded (at most about max_elems
    partial values, float64, per chunk).

    o, lse      the oracle's inputs (per-token partials [n, S, 12, 512] as
                bf16 bits, LSEs [n, S, 12] or None)
    g           the GPU's stage outputs: dict of core, lat, codes, scales
    Returns summed statistics; T4's relative RMS is also checked over the
    whole call.
    """
    n, S = o.shape[0], o.shape[1]
    chunk = max(1, min(S, max_elems // (n * O.NH * O.KVL)))
    tot = {}
    se = sq = 0.0
    for s0 in range(0, S, chunk):
        tok = np.arange(s0, min(S, s0 + chunk))
        sl = slice(s0, s0 + len(tok))
        ref = O.mla_post(o, lse, w_codes, w_scales, gate, tokens=tok)
        lat, codes, scales, core = g["lat"][sl], g["codes"][sl], g["scales"][sl], g["core"][sl]
        st = {}
        st.update(check_t1(lat, ref, exact=exact_t1))
        st.update(check_t2(lat, codes, scales))
        st.update(check_t3(core, codes, scales, w_codes, w_scales, gate[sl]))
        st.update(check_t4(core, ref, lat, codes, scales, strict=strict_t4))
        rv, gv = O.bf16_to_f64(ref["core"]), O.bf16_to_f64(core)
        se += float(np.sum((gv - rv) ** 2))
        sq += float(np.sum(rv * rv))
        for k, v in st.items():
            if k in ("t3_exact_frac", "t4_rel_rms"):
                continue
            tot[k] = max(tot.get(k, 0), v) if k == "t3_max_ulp" else tot.get(k, 0) + v
    rel = (se / sq) ** 0.5 if sq > 0 else 0.0
    assert rel <= 2e-2, f"T4: global relative RMS error {rel:.3g}"
    tot["t4_rel_rms"] = rel
    tot["tokens"] = S
    return tot


# ---------------------------------------------------------------- o_proj


def check_t5(out_gpu, ref, K: int, min_exact: float = 0.9) -> dict:
    """T5, o_proj: out = bf16(sum_k core[t, k] W_O[d, k]) with float32
    accumulation. Every product of two bf16 values is exact in float32, so
    in any order of float32 additions the sum's error is at most
    g = gamma_K M, gamma_K = K u / (1 - K u), u = 2^-24, M = sum_k |core W_O|
    (the standard bound for recursive summation); one rounding to bf16 adds
    at most half a bf16 ulp of the float32 sum. The bound per element:
    |out - y| <= g + ulp_bf16(|y| + g), y the exact sum. A NaN fails.
    That bound is the worst case; a float32 sum is typically about sqrt(K)
    times closer, so nearly every output is RNE(y) itself: at least
    min_exact of them must be (a statistical check, which a wrong final
    rounding, such as truncation, fails). Also reported: the largest error
    in units of the bound."""
    u = 2.0**-24
    gam = K * u / (1 - K * u)
    g = gam * ref["mag"]
    y = ref["y"]
    tol = g + O.ulp_bf16(np.abs(y) + g)
    with np.errstate(invalid="ignore"):
        err = np.abs(O.bf16_to_f64(out_gpu) - y)
        bad = ~(err <= tol)
    assert not bad.any(), f"T5: {int(bad.sum())} o_proj outputs outside the float32 summation bound"
    exact = float(np.mean(out_gpu == ref["out"])) if out_gpu.size else 1.0
    assert exact >= min_exact, f"T5: only {exact:.3f} of the outputs are the exact sum's bf16 rounding"
    return {"t5_exact_frac": exact, "t5_max_err_over_bound": float(np.max(err / tol)) if err.size else 0.0}


# ---------------------------------------------------------------- the split-KV attention (producer)


def check_t0(o_gpu, lse_gpu, ref, nrows) -> dict:
    """T0, the producer's partials against the float64 attention oracle.

    o_gpu bf16 bits [R, n, q, 12, 512] and lse_gpu float32 [R, n, q, 12]
    from the workspace; ref = oracle.attention.attention_partials; nrows
    [R, n] the rows of each split. An empty split must give exactly +0
    partials and an LSE of -inf. Otherwise, with rows the split's rows and
    the score error e = (gamma_576 + 2^-22) smag (576 exact float32 products
    summed in float32, then scaled; smag = scale max_i sum_d |q_d c_id|):
      |lse_gpu - lse| <= 2 e + rows 2^-22 + 2^-20 (1 + |lse|)
    (every score and the running maximum off by at most e; the float32 sum
    of rows exponentials and the base-2 logarithm), and
      |o_gpu - o| <= (2^-8 + 4 e + rows 2^-22) mag + ulp_bf16(|o|)
    (each weight off by a relative 2e from the scores and 2^-9 from rounding
    the probabilities to bf16 for the value product, the float32 sums, one
    bf16 rounding; mag = the softmax-weighted mean of |value|). A NaN
    fails."""
    u = 2.0**-24
    g576 = 576 * u / (1 - 576 * u)
    e = (g576 + 2.0**-22) * ref["smag"]
    rows = np.asarray(nrows, dtype=np.float64)[:, :, None, None]
    empty = np.broadcast_to(rows == 0, ref["lse"].shape)
    lg = np.asarray(lse_gpu, dtype=np.float64)
    assert np.all(lg[empty] == -np.inf), "T0: an empty split's LSE is not -inf"
    assert np.all(np.asarray(o_gpu)[empty] == 0), "T0: an empty split's partial is not +0"
    live = ~empty
    lr = ref["lse"]
    with np.errstate(invalid="ignore"):
        dl = np.abs(lg - lr)
        tl = 2 * e + rows * 2.0**-22 + 2.0**-20 * (1 + np.abs(lr))
        bad = live & ~(dl <= tl)
    assert not bad.any(), f"T0: {int(bad.sum())} LSEs outside tolerance"
    og = O.bf16_to_f64(o_gpu)
    with np.errstate(invalid="ignore"):
        do = np.abs(og - ref["o"])
        to = (2.0**-8 + 4 * e[..., None] + rows[..., None] * 2.0**-22) * ref["mag"] + O.ulp_bf16(ref["o"])
        bad = live[..., None] & ~(do <= to)
    assert not bad.any(), f"T0: {int(bad.sum())} partial values outside tolerance"
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(live[..., None], do / np.maximum(to, 1e-300), 0)
    return {"t0_partials": int(live.sum()), "t0_max_err_over_tol": float(rel.max()) if rel.size else 0.0,
            "t0_exact_frac": float(np.mean((np.asarray(o_gpu) == ref["o_bits"])[np.broadcast_to(live[..., None], og.shape)])) if live.any() else 1.0}
