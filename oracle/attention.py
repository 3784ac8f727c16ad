"""fp64 decode attention of the agents' rows over their own KV caches.

TEST INFRASTRUCTURE ONLY (the oracle): used by the tests, the smoke check and the
benchmark's CPU-baseline leg; the HIP library never imports it.

OpenJet multi-agent serving page, section on moving the weights only once: the
weights are shared by the stacked rows, but every agent reads its own KV cache,
and attention grows with the number of agents.  Each agent's step has
`rows` query rows (its current token and its drafts) at positions L, L + 1, ...
of its sequence, whose keys and values are already in its cache.  Row i
attends to positions 0 .. L + i (causal), with grouped heads: query head hq
uses key/value head hq // (Hq / Hkv).  The scores are q.k / sqrt(d); the
weights are their softmax; the output is the weighted sum of the values.
Everything below is that definition in fp64 on the exact bf16 inputs.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16 or int16 array)."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, lengths,
                     mutant: int = 0) -> np.ndarray:
    """q [A, rows, Hq, d], caches [A, cap, Hkv, d] (bf16 bit patterns), lengths [A]
    = cached positions before the step's rows.  Returns fp64 [A, rows, Hq, d].
    ``mutant`` != 0 plants one deliberate mistake, for the pin tests only:
    1 drops the 1/sqrt(d) scale, 2 lets row i see one position too many, 3 maps
    query heads to key/value heads round-robin instead of in groups."""
    A, rows, Hq, d = q_bits.shape
    _, cap, Hkv, d2 = k_bits.shape
    if d2 != d or v_bits.shape != k_bits.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    group = Hq // Hkv
    out = np.empty((A, rows, Hq, d), dtype=np.float64)
    for a in range(A):
        L = int(lengths[a])
        if L + rows > cap:
            raise ValueError("cache too short for the step's rows")
        K = bf16_to_f64(k_bits[a, :L + rows])            # [L + rows, Hkv, d]
        V = bf16_to_f64(v_bits[a, :L + rows])
        Q = bf16_to_f64(q_bits[a])                        # [rows, Hq, d]
        for hq in range(Hq):
            h = hq % Hkv if mutant == 3 else hq // group
            s = Q[:, hq, :] @ K[:, h, :].T                # [rows, L + rows]
            if mutant != 1:
                s /= np.sqrt(d)
            for i in range(rows):
                s[i, L + i + 1 + (1 if mutant == 2 else 0):] = -np.inf   # row i sees positions 0 .. L + i
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[a, :, hq, :] = p @ V[:, h, :]
    return out
