"""fp64 CPU oracle for the gradients of scaled-dot-product attention (test
infrastructure).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it.

Given the forward O = softmax(S) V with S = scale * Q K^T + mask (masked and
causal entries -inf, an optional sink logit in the denominator, optional
per-batch lengths), and an upstream gradient dO, it returns dQ, dK, dV and the
gradient of the sink logits.  The steps follow the two backward kernels of the
rustytorch "flash_attention.metal" page ("Flash Attention backward kernel for
dQ" and "... for dK and dV"), written here as whole matrices:

  1. P[i, j] = exp(S[i, j] - LSE_i), LSE_i the natural log of the full
     denominator (sink term included), so P is the softmax itself;
  2. D_i = sum_d dO[i, d] O[i, d]            (= sum_j P[i, j] dP[i, j]);
  3. dP = dO V^T;   dS = P * (dP - D)        (elementwise, "softmax_grad");
  4. dQ = scale dS K;   dK = scale dS^T Q;   dV = P^T dO;
  5. a sink s_h enters only the denominator, so dO . dO_i/ds_h = -p_sink,i D_i
     with p_sink,i = exp(s_h - LSE_i):  dsink_h = -sum_{b, i} p_sink,i D_i.

The attribute set (scale, bottom-right causal mask, additive bias, sink token,
the forward's O and log-sum-exp statistics as inputs) is that of
build_sdpa_backward_graph on the "mlx 0.30.7 -- backend/cuda/
scaled_dot_product_attention.cpp" page.  Query head hq reads KV head
hq // (Hq / Hkv), so dK and dV of a KV head sum over its query heads.  The
mask is treated as a constant (no gradient).  Rows that see no key have P = 0
and contribute nothing; padding rows and keys (per-batch lengths) get zero
gradients.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import _f64, _mask64, sdpa_reference


def sdpa_backward_reference(q, k, v, dout, *, scale: float, causal: bool = False,
                            mask=None, sinks=None, seqlens_q=None, seqlens_k=None
                            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Gradients (dQ, dK, dV, dsinks) in float64; dsinks is None without sinks.

    Shapes as in sdpa_reference; dout has the shape of the output o,
    [B, Hq, Lq, Dv] (Dv, the head dim of v, may differ from that of q, k)."""
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Lq, D = Q.shape
    Hkv, Lk = K.shape[1], K.shape[2]
    G = Hq // Hkv
    M = None if mask is None else np.broadcast_to(_mask64(mask), (B, Hq, Lq, Lk))
    SK = None if sinks is None else _f64(sinks).reshape(Hq)
    # the forward: O and LSE of the same definition
    O, LSE = sdpa_reference(q, k, v, scale=scale, causal=causal, mask=mask, sinks=sinks,
                            seqlens_q=seqlens_q, seqlens_k=seqlens_k)

    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dsink = None if SK is None else np.zeros(Hq)
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
            # step 1: the softmax probabilities from the scores and the LSE
            S = scale * (Qb @ Kb.T)
            if M is not None:
                S = S + M[b, hq, :lq, :lk]
            if causal:
                S = np.where(np.arange(lk)[None, :] > rows[:, None] + (lk - lq), -np.inf, S)
            P = np.where(live[:, None], np.exp(S - np.where(live, Lb, 0.0)[:, None]), 0.0)
            # step 2: D_i = dO_i . O_i
            Di = np.sum(dOb * Ob, axis=1)
            # step 3
            dP = dOb @ Vb.T
            dS = P * (dP - Di[:, None])
            # step 4 (GQA: the query heads of a group add into one KV head)
            dQ[b, hq, :lq] = scale * (dS @ Kb)
            dK[b, g, :lk] += scale * (dS.T @ Qb)
            dV[b, g, :lk] += P.T @ dOb
            # step 5
            if SK is not None:
                psink = np.where(live, np.exp(SK[hq] - np.where(live, Lb, 0.0)), 0.0)
                dsink[hq] -= float(np.sum(psink * Di))
    return dQ, dK, dV, dsink
