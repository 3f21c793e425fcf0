"""Plain float64 CPU oracle of o_proj, the consumer of ``core``.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library.

The vLLM API-docs page for the module
``vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back`` names
the step after the path only as its consumer: its module docstring describes
the path as running from AITER's decode output to o_proj's input, and
``core`` [S, 1536] is that input. The page states nothing else about it, so
this module takes the plainest reading (every point is a reading, and the
model's real o_proj is "parity unpinned" against it):

* o_proj is a linear layer without bias over the 1536 columns of core that
  one tensor-parallel rank holds (12 heads x 128): out[t, d] = sum_k
  core[t, k] * W_O[d, k], with W_O stored [D, K] row-major in bf16 (a linear
  layer's weight layout) and D the model's hidden size. Under tensor
  parallelism each rank's product is a partial sum that an all-reduce across
  the ranks completes; on one GPU that reduction is out of scope.
* The sum is rounded once to bf16, round to nearest even.

The sum is formed in float64 with a library matrix product. Every product of
two bf16 values is exact in float64, and the sum of K of them is exact
whenever the products' exponents span fewer than 53 - 16 bits. Otherwise the
error is below K * 2^-53 of sum |core * W_O|, far inside the criterion's
bound, so the result is the exact sum for every purpose here. A pin checks it
against exact rational arithmetic.
"""

from __future__ import annotations

import numpy as np

from .post import bf16_to_f64, rne_bf16


def oproj(core_bits, w_bits, rows=None) -> dict:
    """out = bf16(core @ W_O^T).

    core_bits uint16 [S, K] bf16 bits; w_bits uint16 [D, K] bf16 bits;
    rows: optional token indices (only those rows are computed).
    Returns y (float64 [T, D], the sum), mag (float64 [T, D], sum_k
    |core[t, k] * W_O[d, k]|, the size of the terms a float32 sum rounds)
    and out (bf16 bits [T, D]).
    """
    c = np.asarray(core_bits, dtype=np.uint16)
    if rows is not None:
        c = c[np.asarray(rows)]
    a = bf16_to_f64(c)
    w = bf16_to_f64(np.asarray(w_bits, dtype=np.uint16))
    if a.shape[-1] != w.shape[-1]:
        raise ValueError("core and W_O must have the same K")
    y = a @ w.T
    mag = np.abs(a) @ np.abs(w).T
    return {"y": y, "mag": mag, "out": rne_bf16(y)}


__all__ = ["oproj"]
