"""Moving seeded workloads to the GPU and reading results back (tests only)."""

from __future__ import annotations

import numpy as np
import torch

import oracle.post as O


def bf16_to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def device_inputs(w, dev="cuda", w_codes=None, w_scales=None) -> dict:
    """Device tensors for workload ``w``: o and lse as the same strided views
    of their device buffers, W_V in MXFP4 (the oracle's quantiser of the bf16
    W_V draw unless given), gate."""
    if w_codes is None:
        w_codes, w_scales = O.quantize_mxfp4(w.wv_bits)
    o_buf = bf16_to_dev(w.o_buf, dev)
    o = torch.as_strided(o_buf, (w.n, w.S, 12, 512), tuple(w.o_strides) + (1,))
    lse = None
    if w.lse_buf is not None:
        lse_buf = torch.from_numpy(np.ascontiguousarray(w.lse_buf)).to(dev)
        lse = torch.as_strided(lse_buf, (w.n, w.S, 12), tuple(w.lse_strides))
    return {
        "o_buf": o_buf,
        "o": o,
        "lse": lse,
        "w_v": torch.from_numpy(np.ascontiguousarray(w_codes)).to(dev),
        "w_v_scale": torch.from_numpy(np.ascontiguousarray(w_scales)).to(dev),
        "gate": bf16_to_dev(w.gate, dev),
        "w_codes": w_codes,
        "w_scales": w_scales,
        "layout": layout_kwargs(w, dev),
    }


def layout_kwargs(w, dev="cuda") -> dict:
    """Request-major and masking arguments of workload w for the binding."""
    kw = {}
    if w.q != 1 or w.o_sr or w.l_sr:
        kw.update(q=w.q, o_sr=w.o_sr, l_sr=w.l_sr)
    if w.kv_lens is not None:
        kw["kv_lens"] = torch.from_numpy(np.ascontiguousarray(w.kv_lens)).to(dev)
    if w.qsl is not None:
        kw["qsl"] = torch.from_numpy(np.ascontiguousarray(w.qsl)).to(dev)
    return kw


def run_debug(m, d) -> dict:
    """One launch with stage outputs; results as host arrays."""
    core, lat, codes, scales = m.mla_post(
        d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], debug=True, **d.get("layout", {})
    )
    torch.cuda.synchronize()
    return {
        "core": to_bits(core),
        "lat": to_bits(lat),
        "codes": codes.cpu().numpy(),
        "scales": scales.cpu().numpy(),
    }
