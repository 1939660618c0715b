"""Elementwise error scale for the gradient parity tests.

A gradient element is a sum of products, and the rounding of its inputs and
partial results is bounded by the same sum over absolute values (the standard
bound |fl(x.y) - x.y| <= c u |x|.|y| for a dot product in unit roundoff u).
Each gradient element therefore gets its own scale, the "magnitude companion"
of its sum:

  dV = P^T dO                    A_dV = P^T |dO|
  dS = P * (dP - D)              A_dS = |dS| + P * (|dO_i| . |O_i|)
  dQ = scale dS K                A_dQ = scale A_dS |K|
  dK = scale dS^T Q              A_dK = scale A_dS^T |Q|

A_dS covers the two places 16-bit rounding enters dS in the kernels: dS
itself is rounded to the input type before the products with K and Q, and
D_i = dO_i . O_i uses the forward's O, rounded to the input type (error at
most u |dO_i| . |O_i|).  O and the log-sum-exp come from the fp64 oracle;
P and dP are formed from them the way the oracle forms them, with its masks
and causal alignment (bottom-right causal, per-batch lengths, GQA sums over
the query heads of a KV head).  Every companion bounds its reference from
above, which the tests also check.

fp16 has a narrow exponent range: below 2^-14 it keeps a fixed absolute step
of 2^-24, so rounding a value x costs at most u |x| + 2^-25 (u = 2^-11).
`floor` is that absolute part in units of u (2^-14 for fp16, 0 otherwise);
it enters wherever a rounded P or dS element is nonzero.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import _f64, _mask64, sdpa_reference


def grad_magnitudes(q, k, v, dout, *, scale: float, causal: bool = False, mask=None, sinks=None,
                    seqlens_q=None, seqlens_k=None, floor: float = 0.0):
    """(A_dQ, A_dK, A_dV) in float64, shaped like dQ, dK, dV."""
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Lq, _ = Q.shape
    Hkv, Lk = K.shape[1], K.shape[2]
    G = Hq // Hkv
    M = None if mask is None else np.broadcast_to(_mask64(mask), (B, Hq, Lq, Lk))
    O, LSE = sdpa_reference(q, k, v, scale=scale, causal=causal, mask=mask, sinks=sinks,
                            seqlens_q=seqlens_q, seqlens_k=seqlens_k)
    aQ, aK, aV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        lq = Lq if seqlens_q is None else min(max(int(_f64(seqlens_q)[b]), 0), Lq)
        lk = Lk if seqlens_k is None else min(max(int(_f64(seqlens_k)[b]), 0), Lk)
        if lq == 0:
            continue
        rows = np.arange(lq)
        for hq in range(Hq):
            g = hq // G
            Qb, dOb, Ob, Lb = Q[b, hq, :lq], dO[b, hq, :lq], O[b, hq, :lq], LSE[b, hq, :lq]
            Kb, Vb = K[b, g, :lk], V[b, g, :lk]
            live = np.isfinite(Lb)
            S = scale * (Qb @ Kb.T)
            if M is not None:
                S = S + M[b, hq, :lq, :lk]
            if causal:
                S = np.where(np.arange(lk)[None, :] > rows[:, None] + (lk - lq), -np.inf, S)
            P = np.where(live[:, None], np.exp(S - np.where(live, Lb, 0.0)[:, None]), 0.0)
            Di = np.sum(dOb * Ob, axis=1)
            dS = P * (dOb @ Vb.T - Di[:, None])
            nz = floor * (P > 0)
            adS = np.abs(dS) + P * np.sum(np.abs(dOb) * np.abs(Ob), axis=1)[:, None] + nz
            aQ[b, hq, :lq] = scale * (adS @ np.abs(Kb))
            aK[b, g, :lk] += scale * (adS.T @ np.abs(Qb))
            aV[b, g, :lk] += (P + nz).T @ np.abs(dOb)
    return aQ, aK, aV
