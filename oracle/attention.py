"""Plain float64 CPU oracle of the split-KV decode attention that produces
mla_post's partials.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library.

The vLLM API-docs page for module
``vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back`` names
the producer of the split partials (module docstring: M1c's mla_attn writes
o / lse per split, dense [splits, S, 12, 512] bf16 and [splits, S, 12] f32;
``combine_splits``: a token merges its request's splits, request-major; K2
runs M1c in the same launch as the merge and W_UV, polling M1c's per-split
ready flags). It does not show M1c itself. This module takes the plainest
reading of a split-KV MLA decode attention whose outputs have exactly those
shapes (each point a reading, "parity unpinned" against the real M1c):

A1  MLA in the absorbed form: the query of token t and head h is
    q[t, h, 0:576] (512 latent dims and 64 rotary dims); row i of the KV
    cache is c[i, 0:576], shared by all heads; the score is
    scale * (q . c_i) over all 576 dims; the value is the latent part
    c_i[0:512], so a partial lives in the 512-wide latent space the merge and
    W_UV consume.
A2  Request r owns the KV rows indptr[r] .. indptr[r + 1] - 1 (the page's
    per-request local KV lengths); each of its q query tokens attends to all
    of them.
A3  Split j of per covers the request's rows floor(j L / per) ..
    floor((j + 1) L / per) - 1 (L its length): contiguous, near-even shares.
    A split without rows is empty: LSE -inf and a zero partial (the page: an
    empty split has weight 0 and its o is 0).
A4  The partial is the softmax-weighted mean of the split's value rows,
    rounded to bf16 (round to nearest even); its LSE is the natural log of
    the sum of exp(score) over the split, as float32.
"""

from __future__ import annotations

import numpy as np

from .post import bf16_to_f64, rne_bf16

NH = 12
DQK = 576  # query / key width: 512 latent + 64 rotary
KVL = 512  # value width (the latent part)


def split_bounds(L: int, per: int) -> np.ndarray:
    """Row offsets (within the request) where the per splits start, and L."""
    return np.array([(j * L) // per for j in range(per + 1)], dtype=np.int64)


def attention_partials(qry_bits, kv_bits, indptr, q: int, per: int, scale: float) -> dict:
    """Partials of every (request, split, token, head).

    qry_bits uint16 [S, 12, 576] bf16 (S = R q, token t of request t // q);
    kv_bits uint16 [rows, 576] bf16; indptr int [R + 1].
    Returns o (float64 [R, per, q, 12, 512]), lse (float64 [R, per, q, 12]),
    o_bits (bf16 bits, A4) and lse_f32 (float32); for tolerances also mag
    (the softmax-weighted mean of |value|, per element of o) and smag
    (scale times the largest sum over the dims of |q c| among the split's
    rows, per (token, head): the size of the terms a score sums).
    """
    qv = bf16_to_f64(qry_bits)
    kv = bf16_to_f64(kv_bits)
    indptr = np.asarray(indptr, dtype=np.int64)
    R = indptr.size - 1
    if qv.shape[0] != R * q:
        raise ValueError("S must be R * q")
    o = np.zeros((R, per, q, NH, KVL))
    mag = np.zeros((R, per, q, NH, KVL))
    smag = np.zeros((R, per, q, NH))
    lse = np.full((R, per, q, NH), -np.inf)
    for r in range(R):
        rows = kv[indptr[r] : indptr[r + 1]]
        b = split_bounds(rows.shape[0], per)
        qr = qv[r * q : (r + 1) * q]  # [q, 12, 576]
        for j in range(per):
            c = rows[b[j] : b[j + 1]]
            if c.shape[0] == 0:
                continue
            s = scale * np.einsum("thd,id->thi", qr, c)  # [q, 12, n]
            m = s.max(axis=-1, keepdims=True)
            p = np.exp(s - m)
            tot = p.sum(axis=-1)
            o[r, j] = np.einsum("thi,id->thd", p, c[:, :KVL]) / tot[..., None]
            mag[r, j] = np.einsum("thi,id->thd", p, np.abs(c[:, :KVL])) / tot[..., None]
            smag[r, j] = abs(scale) * np.einsum("thd,id->thi", np.abs(qr), np.abs(c)).max(axis=-1)
            lse[r, j] = m[..., 0] + np.log(tot)
    return {"o": o, "lse": lse, "o_bits": rne_bf16(o), "lse_f32": lse.astype(np.float32), "mag": mag, "smag": smag}


def token_partials(parts):
    """Per-token views of attention_partials' bf16 partials and float32 LSEs
    for mla_post: o [per, S, 12, 512] (token t = r q + tt takes split j of its
    request) and lse [per, S, 12]."""
    ob, lf = parts["o_bits"], parts["lse_f32"]
    R, per, q = ob.shape[0], ob.shape[1], ob.shape[2]
    o = np.ascontiguousarray(np.transpose(ob, (1, 0, 2, 3, 4)).reshape(per, R * q, NH, KVL))
    lse = np.ascontiguousarray(np.transpose(lf, (1, 0, 2, 3)).reshape(per, R * q, NH))
    return o, lse


__all__ = ["NH", "DQK", "KVL", "split_bounds", "attention_partials", "token_partials"]
