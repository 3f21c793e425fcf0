"""Acceptance criteria of the HIP path against the CPU oracle.

T1  latents: |lat_gpu - x| <= ulp_bf16(max(|x|, 2^-8 M)) per element, x the
    oracle's exact float64 merge and M = sum_j w_j |o_j| (the floor covers
    cancellation: float32 accumulation error is about (n + 6) 2^-24 M, which
    exceeds one bf16 ulp of a nearly cancelled |x|). Without LSEs: exact.
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
    err = np.abs(g - x)
    bad = err > tol
    strict = np.abs(g - O.bf16_to_f64(ref["lat"])) > O.ulp_bf16(x)
    assert not bad.any(), f"T1: {int(bad.sum())} latents outside tolerance (max err/tol {float((err / tol).max()):.3g})"
    return {"t1_bad": 0, "t1_strict_ulp": int(strict.sum()), "t1_diff_latents": int((lat_gpu != ref["lat"]).sum())}


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
    err = np.abs(gv - rv)
    bad = err > tol
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
    err = np.abs(gv - rv)
    zero_rows = rms == 0
    assert np.all(err[zero_rows] == 0), "T4: rows the oracle makes exactly zero must be exactly zero"
    row_bad = np.any(err > 2e-2 * rms[:, None], axis=-1) & ~zero_rows
    denom = np.sqrt(np.mean(rv * rv))
    rel_rms = float(np.sqrt(np.mean((gv - rv) ** 2)) / denom) if denom > 0 else 0.0
    assert rel_rms <= 2e-2, f"T4: global relative RMS error {rel_rms:.3g}"
    if strict:
        assert not row_bad.any(), f"T4 strict: {int(row_bad.sum())} rows over 2e-2 RMS"
    elif row_bad.any():
        assert lat_gpu is not None and codes_gpu is not None, "T4: rows over tolerance and no stage outputs to explain them"
        for t in np.nonzero(row_bad)[0]:
            cols = np.nonzero(err[t] > 2e-2 * rms[t])[0]
            for h in np.unique(cols // 128):
                lat_diff = (lat_gpu[t, h] != ref["lat"][t, h]).reshape(16, 32).any(-1)
                code_diff = (codes_gpu[t, h] != ref["codes"][t, h]).reshape(16, 16).any(-1)
                if scales_gpu is not None:
                    code_diff |= scales_gpu[t, h] != ref["scales"][t, h]
                assert np.any(lat_diff & code_diff), f"T4: token {t} head {h} off with no flipped code"
    return {"t4_rows_over": int(row_bad.sum()), "t4_rel_rms": rel_rms}
