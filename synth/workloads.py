"""Seeded synthetic inputs for mla_post, shared by the oracle and the HIP path.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no merge, no quantisation, no contraction). bf16 inputs
are made by torch's CPU float32 -> bfloat16 cast (round to nearest even) of
float32 draws. W_V is handed out as bf16 values; turning it into MXFP4 is the
caller's job (the oracle's quantiser in the tests, the library's quantiser in
the benchmark), so no quantiser lives here.

Workloads follow the shapes of the Kimi-K3 decode step at 8-way tensor
parallelism on the vLLM page for module
``vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back``: 12
local heads, latent 512, W_V[h] of 128 x 512, gate/core [S, 1536]. Each
partial row o[j, t, h, :] is 512 contiguous bf16 at element offset
``off + j*sj + t*st + h*sh`` of its buffer, the strided-view convention of the
page's host launcher.

Draw order inside a workload: o, lse, mask uniforms, W_V, gate.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

NH, KVL, VD = 12, 512, 128
NAN_BF16 = np.uint16(0x7FC0)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """torch CPU cast float32 -> bfloat16 (RNE), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, sigma: float, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, sigma) float32 draws rounded to bf16, drawn in flat chunks (same
    stream as one big draw) to bound host memory for the large case."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        d = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            d *= np.float32(sigma)
        out[s:e] = f32_to_bf16_bits(d)
    return out.reshape(shape)


@dataclass
class Workload:
    """One mla_post call's inputs, host side."""

    name: str
    n: int  # partials per (token, head): splits or ranks
    S: int  # tokens
    o_buf: np.ndarray  # uint16, the allocation holding the partials
    o_strides: tuple  # (sj, st, sh) in elements; innermost stride 1
    lse_buf: np.ndarray | None  # float32 allocation, or None (one partial, no LSE)
    lse_strides: tuple | None  # (sj, st, sh) in elements
    wv_bits: np.ndarray  # uint16 [12, 128, 512]: bf16 of the W_V draw
    gate: np.ndarray  # uint16 [S, 1536]
    seed: int = 0
    notes: dict = field(default_factory=dict)
    # request-major slices: row (j, t, h) also moves by (t // q) * o_sr elements
    q: int = 1
    o_sr: int = 0
    l_sr: int = 0
    kv_lens: np.ndarray | None = None  # int32 [n, S // q]: 0 marks an empty partial
    qsl: np.ndarray | None = None  # int32 [S // q + 1]

    def o_view(self) -> np.ndarray:
        """[N, S, 12, 512] numpy view into o_buf."""
        sj, st, sh = self.o_strides
        b = self.o_buf.itemsize
        return np.lib.stride_tricks.as_strided(
            self.o_buf, shape=(self.n, self.S, NH, KVL), strides=(sj * b, st * b, sh * b, b), writeable=False
        )

    def lse_view(self) -> np.ndarray | None:
        """[N, S, 12] numpy view into lse_buf (None without LSEs)."""
        if self.lse_buf is None:
            return None
        sj, st, sh = self.lse_strides
        b = self.lse_buf.itemsize
        return np.lib.stride_tricks.as_strided(
            self.lse_buf, shape=(self.n, self.S, NH), strides=(sj * b, st * b, sh * b), writeable=False
        )


def _wv_gate(rng, S):
    wv = _normal_bf16(rng, (NH, VD, KVL), 1.0 / np.sqrt(KVL))
    gate = f32_to_bf16_bits(rng.random((S, NH * VD), dtype=np.float32))
    return wv, gate


def dense_splits(
    name: str,
    n: int,
    S: int,
    seed: int,
    o_sigma: float = 1.0,
    lse_uniform: tuple | None = (-4.0, 16.0),
    lse_normal: tuple | None = None,
    p_neg_inf: float = 0.0,
    p_nan: float = 0.0,
    p_pos_inf: float = 0.0,
    n_neg_inf_exact: int = 0,
) -> Workload:
    """Split-KV partials in a dense [N, S, 12, 512] buffer with LSE [N, S, 12].

    LSE draws: U(lo, hi) (``lse_uniform``) or N(mean, sd) (``lse_normal``).
    Per-entry masks from one uniform draw u: u < p_neg_inf -> -inf, the next
    p_nan -> NaN, the next p_pos_inf -> +inf. ``n_neg_inf_exact`` instead sets
    that many entries, picked with ``rng.integers``, to -inf.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    o = _normal_bf16(rng, (n, S, NH, KVL), o_sigma)
    if lse_normal is not None:
        lse = rng.normal(lse_normal[0], lse_normal[1], size=(n, S, NH)).astype(np.float32)
    else:
        lse = rng.uniform(lse_uniform[0], lse_uniform[1], size=(n, S, NH)).astype(np.float32)
    if p_neg_inf or p_nan or p_pos_inf:
        u = rng.random((n, S, NH))
        lse[u < p_neg_inf] = -np.inf
        lse[(u >= p_neg_inf) & (u < p_neg_inf + p_nan)] = np.nan
        lse[(u >= p_neg_inf + p_nan) & (u < p_neg_inf + p_nan + p_pos_inf)] = np.inf
    if n_neg_inf_exact:
        flat = lse.reshape(-1)
        for _ in range(n_neg_inf_exact):
            flat[int(rng.integers(0, flat.size))] = -np.inf
    wv, gate = _wv_gate(rng, S)
    return Workload(
        name,
        n,
        S,
        o,
        (S * NH * KVL, NH * KVL, KVL),
        lse,
        (S * NH, NH, 1),
        wv,
        gate,
        seed,
    )


def single_partial(name: str, S: int, seed: int, o_sigma: float = 1.0) -> Workload:
    """One partial per (token, head) and no LSE: o [S, 12, 512] is the final
    attention output (decode-context-parallel group of one, no splits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    o = _normal_bf16(rng, (S, NH, KVL), o_sigma)
    wv, gate = _wv_gate(rng, S)
    return Workload(name, 1, S, o, (0, NH * KVL, KVL), None, None, wv, gate, seed)


def dcp_gathered(
    name: str,
    R: int,
    S: int,
    seed: int,
    head_stride_rows: int,
    dead_from: int,
    p_neg_inf: float = 0.05,
    p_nan: float = 0.005,
    p_pos_inf: float = 0.005,
) -> Workload:
    """Decode-context-parallel partials gathered on one GPU.

    Buffer o [S, head_stride_rows, 512]; rank r's partial of local head h is
    gathered head r * 12 + h, so (sj, st, sh) = (12*512, head_stride_rows*512,
    512). Heads past R * 12 are padding, poisoned with NaN (never read).
    lse [S, R*12] dense: (sj, st, sh) = (12, R*12, 1), U(-4, 16) with per-entry
    -inf / NaN / +inf masks, and every LSE of tokens t >= dead_from is -inf.
    """
    assert head_stride_rows >= R * NH
    rng = np.random.Generator(np.random.PCG64(seed))
    o = _normal_bf16(rng, (S, head_stride_rows, KVL), 1.0)
    o[:, R * NH :, :] = NAN_BF16
    lse = rng.uniform(-4.0, 16.0, size=(S, R * NH)).astype(np.float32)
    u = rng.random((S, R * NH))
    lse[u < p_neg_inf] = -np.inf
    lse[(u >= p_neg_inf) & (u < p_neg_inf + p_nan)] = np.nan
    lse[(u >= p_neg_inf + p_nan) & (u < p_neg_inf + p_nan + p_pos_inf)] = np.inf
    lse[dead_from:, :] = -np.inf
    wv, gate = _wv_gate(rng, S)
    return Workload(
        name,
        R,
        S,
        o,
        (NH * KVL, head_stride_rows * KVL, KVL),
        lse,
        (NH, R * NH, 1),
        wv,
        gate,
        seed,
    )


def request_major(
    name: str,
    per: int,
    q: int,
    S: int,
    seed: int,
    compact: bool = False,
    p_neg_inf: float = 0.1,
    kv_zero: float = 0.0,
    batch_rows: int | None = None,
    o_sigma: float = 1.0,
    lse_normal: tuple | None = None,
) -> Workload:
    """Split partials laid out request-major, R = S / q requests of q tokens,
    per splits each.

    compact=False: the page's layout, one dense tensor of P = per * R slices,
    o [P, S, 12, 512] and lse [P, S, 12]; token t's splits are slices
    (t // q) * per + j. Only those (slice, token) rows are filled; every other
    row is NaN and every other LSE NaN (never to be read).
    compact=True: o [R, per, q, 12, 512], lse [R, per, q, 12]: no unused rows.

    kv_zero: fraction of (partial, request) pairs whose KV length is 0
    (kv_lens [per, R], otherwise lengths 1..64); batch_rows: qsl[R] (tokens
    from there on are past the batch; qsl evenly spaced otherwise).
    """
    assert S % q == 0
    R = S // q
    rng = np.random.Generator(np.random.PCG64(seed))
    vals = _normal_bf16(rng, (per, S, NH, KVL), o_sigma)
    if lse_normal is not None:
        lv = rng.normal(lse_normal[0], lse_normal[1], size=(per, S, NH)).astype(np.float32)
    else:
        lv = rng.uniform(-4.0, 16.0, size=(per, S, NH)).astype(np.float32)
    u = rng.random((per, S, NH))
    lv[u < p_neg_inf] = -np.inf
    kv = rng.integers(1, 65, size=(per, R)).astype(np.int32)
    kv[rng.random((per, R)) < kv_zero] = 0
    qsl = (np.arange(R + 1, dtype=np.int32) * q).astype(np.int32)
    if batch_rows is not None:
        qsl[R] = batch_rows
    wv, gate = _wv_gate(rng, S)
    t = np.arange(S)
    if compact:
        o = np.empty((R, per, q, NH, KVL), dtype=np.uint16)
        lse = np.empty((R, per, q, NH), dtype=np.float32)
        for j in range(per):
            o[t // q, j, t % q] = vals[j]
            lse[t // q, j, t % q] = lv[j]
        o_strides = (q * NH * KVL, NH * KVL, KVL)
        o_sr = (per - 1) * q * NH * KVL
        l_strides = (q * NH, NH, 1)
        l_sr = (per - 1) * q * NH
    else:
        P = per * R
        o = np.full((P, S, NH, KVL), NAN_BF16, dtype=np.uint16)
        lse = np.full((P, S, NH), np.nan, dtype=np.float32)
        for j in range(per):
            o[(t // q) * per + j, t] = vals[j]
            lse[(t // q) * per + j, t] = lv[j]
        o_strides = (S * NH * KVL, NH * KVL, KVL)
        o_sr = per * S * NH * KVL
        l_strides = (S * NH, NH, 1)
        l_sr = per * S * NH
    w = Workload(name, per, S, o, o_strides, lse, l_strides, wv, gate, seed)
    w.q, w.o_sr, w.l_sr = q, o_sr, l_sr
    w.notes["o_logical"], w.notes["lse_logical"] = vals, lv  # what token t's split j holds
    w.kv_lens = kv if kv_zero > 0 else None
    w.qsl = qsl if batch_rows is not None else None
    return w


# ---- the five standard workloads -------------------------------------------


def tiny() -> Workload:
    """S=4, 2 splits, o ~N(0,1), lse ~U(-4,12) with one entry -inf; seed 0."""
    return dense_splits("tiny", 2, 4, seed=0, lse_uniform=(-4.0, 12.0), n_neg_inf_exact=1)


def no_merge() -> Workload:
    """S=64, one partial, no LSE (W_UV + gate alone); seed 1."""
    return single_partial("no_merge", 64, seed=1)


def split_merge() -> Workload:
    """32 requests x 4 tokens (S=128), 8 splits, lse ~U(-4,16), 10% -inf; seed 2."""
    return dense_splits("split_merge", 8, 128, seed=2, p_neg_inf=0.10)


def dcp8() -> Workload:
    """R=8 gathered rank partials, S=256, head-row stride 104, lse ~U(-4,16)
    with 5% -inf / 0.5% NaN / 0.5% +inf, tokens >= 240 all -inf; seed 3."""
    return dcp_gathered("dcp8", 8, 256, seed=3, head_stride_rows=104, dead_from=240)


def large_decode() -> Workload:
    """1024 requests x 4 tokens (S=4096), 16 splits, o ~N(0,2), lse ~N(8,6)
    with 5% -inf; seed 4. 805 MB of partials."""
    return dense_splits("large_decode", 16, 4096, seed=4, o_sigma=2.0, lse_normal=(8.0, 6.0), p_neg_inf=0.05)


def large_decode_request_major() -> Workload:
    """The large decode batch's sizes and distributions (S=4096, 1024
    requests x 4 tokens, 16 splits, o ~N(0,2), lse ~N(8,6) with 5% -inf) in
    the compact request-major layout [1024, 16, 4, 12, 512]; seed 5."""
    return request_major(
        "large_decode_request_major", per=16, q=4, S=4096, seed=5, compact=True, p_neg_inf=0.05,
        o_sigma=2.0, lse_normal=(8.0, 6.0),
    )


# ---- inputs of the split-KV decode attention that produces the partials ----

DQK = 576  # query / cache row width: 512 latent + 64 rotary


@dataclass
class DecodeInputs:
    """One fused decode call's inputs, host side: queries of R requests of q
    tokens, the KV cache rows of every request back to back, W_V (bf16, to be
    put into MXFP4 by the caller) and the gate."""

    name: str
    R: int
    q: int
    n: int  # KV splits per request
    qry: np.ndarray  # uint16 [R q, 12, 576]
    kv: np.ndarray  # uint16 [sum of lengths, 576]
    indptr: np.ndarray  # int32 [R + 1]
    wv_bits: np.ndarray  # uint16 [12, 128, 512]
    gate: np.ndarray  # uint16 [R q, 1536]
    scale: float

    @property
    def S(self) -> int:
        return self.R * self.q


def decode_inputs(name: str, lens, q: int, n: int, seed: int, q_sigma: float = 1.0, kv_sigma: float = 1.0,
                  scale: float = 1.0 / np.sqrt(192.0)) -> DecodeInputs:
    """Seeded draws: per-request KV lengths `lens`, queries ~ N(0, q_sigma)
    and cache rows ~ N(0, kv_sigma) in bf16, W_V ~ N(0, 1/sqrt(512)), gate
    ~ U(0, 1). Draw order: queries, cache, W_V, gate. The default scale is
    1/sqrt(192), a DeepSeek-V3-style query-key head width of 128 + 64."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    R = lens.size
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qry = _normal_bf16(rng, (R * q, NH, DQK), q_sigma)
    kv = _normal_bf16(rng, (int(indptr[-1]), DQK), kv_sigma)
    wv, gate = _wv_gate(rng, R * q)
    return DecodeInputs(name, R, q, n, qry, kv, indptr, wv, gate, float(scale))


STANDARD = {
    "tiny": tiny,
    "no_merge": no_merge,
    "split_merge": split_merge,
    "dcp8": dcp8,
    "large_decode": large_decode,
}

EXTRA = {"large_decode_request_major": large_decode_request_major}
