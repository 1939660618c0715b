"""fp64 CPU oracle for fused scaled-dot-product attention (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it; it imports nothing from the HIP package.

What it computes is the plain definition of the operation, written out with an
explicit score matrix (the "unfused" composition the pages compare their fused
kernels against):

    O = softmax(scale * Q K^T + mask) V

with the feature set of the cuDNN SDPA graph built on the "mlx 0.30.7 --
backend/cuda/scaled_dot_product_attention.cpp" page (``build_sdpa_graph``:
attention scale, generated statistics = log-sum-exp, bottom-right causal mask,
additive bias, sink token) and the grouped-query shapes of the "Add D512
support to Metal vector attention" page (query heads ``h``, KV heads ``hk``).

Readings adopted where the pages are silent (each also listed in the design
notes):
  * causal is bottom-right aligned: key j is visible to query i iff
    j <= i + (Lk - Lq) (``set_causal_mask_bottom_right``);
  * query head hq reads KV head hq // (Hq / Hkv) (contiguous groups);
  * a sink is a raw per-query-head logit (not multiplied by ``scale``) that
    adds exp(sink) to the softmax denominator only;
  * the log-sum-exp output is natural-log and includes the sink term;
  * a row with no visible key and no sink yields O = 0 and LSE = -inf;
  * scale multiplies the dot product (in fp64 here), then the mask is added;
  * per-batch lengths (the padding mask that ``build_sdpa_graph`` turns on
    with ``set_seq_len_q`` / ``set_seq_len_kv``): batch b has its first
    seq_len_q[b] query rows and seq_len_kv[b] keys (clamped to [0, Lq] and
    [0, Lk]); the rest is padding.  A padding key is seen by no row; a
    padding row sees no key (so it is written as an empty row); bottom-right
    causal alignment uses the batch's own lengths:
    j <= i + (seq_len_kv[b] - seq_len_q[b]).

Steps per (b, hq), g = hq // G, in the order of the definition:
  1. convert the inputs exactly to fp64;
  2. S[i, j] = scale * sum_d Q[i, d] K[j, d]  (+ mask[i, j]);  S = -inf where
     causal hides the key;
  3. m_i = max(max_j S[i, j], sink);
  4. e[i, j] = exp(S[i, j] - m_i);  den_i = sum_j e[i, j] + exp(sink - m_i);
  5. O[i] = sum_j e[i, j] V[j] / den_i,  LSE_i = m_i + log(den_i);
     rows with m_i = -inf give O = 0, LSE = -inf.
The online (running max / running sum) recurrence that the fused kernels use
(rustytorch ``flash_attention.metal``, forward kernel, "Online softmax update")
reaches this same result up to rounding order, so the oracle needs no blocking.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact conversion of a numpy array or CPU torch tensor to float64."""
    if hasattr(x, "detach"):                     # torch tensor (any float dtype)
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _mask64(mask) -> np.ndarray:
    """An additive mask in float64; a boolean mask (True = the key takes part,
    the MLX convention) becomes 0 where True and -inf where False."""
    m = mask.detach().cpu().numpy() if hasattr(mask, "detach") else np.asarray(mask)
    if m.dtype == np.bool_:
        return np.where(m, 0.0, -np.inf)
    return np.asarray(m, dtype=np.float64)


def sdpa_reference(q, k, v, *, scale: float, causal: bool = False,
                   mask=None, sinks=None, rows: Optional[Sequence[int]] = None,
                   heads: Optional[Sequence[Tuple[int, int]]] = None,
                   seqlens_q=None, seqlens_k=None
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Naive attention in fp64.

    q: [B, Hq, Lq, D]; k: [B, Hkv, Lk, D]; v: [B, Hkv, Lk, Dv] (Dv may differ
    from D; O then has head dim Dv); mask: anything broadcastable to
    [B, Hq, Lq, Lk], additive (may hold -inf) or boolean (False hides the
    key); sinks: [Hq] or None;
    seqlens_q, seqlens_k: per-batch valid lengths [B] or None (= Lq, Lk).
    Padding entries of q, k and v are never read, so they may hold anything.

    ``rows`` restricts the computation to those query indices (same for every
    head); ``heads`` restricts it to those (b, hq) pairs.  The result then has
    the restricted shape [len(heads) or B*Hq ..., len(rows), D] -- see below.

    Returns (O, LSE) in float64 with shapes [B, Hq, Lq', Dv] and [B, Hq, Lq']
    (Lq' = len(rows) when ``rows`` is given).  With ``heads`` the leading two
    dims are replaced by one dim over the listed pairs: [n, Lq', D], [n, Lq'].
    """
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, D = Q.shape
    Bk, Hkv, Lk, Dk = K.shape
    Dv = V.shape[3]                                  # value / output head dim (may differ from D)
    if Bk != B or Dk != D or V.shape[:3] != K.shape[:3]:
        raise ValueError("q/k/v shapes disagree")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    M = None if mask is None else np.broadcast_to(_mask64(mask), (B, Hq, Lq, Lk))
    S_ = None if sinks is None else _f64(sinks).reshape(Hq)
    row_idx = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)

    O = np.zeros((len(pairs), len(row_idx), Dv))
    LSE = np.full((len(pairs), len(row_idx)), -np.inf)

    def lengths(b):
        lq = Lq if seqlens_q is None else min(max(int(_f64(seqlens_q)[b]), 0), Lq)
        lk = Lk if seqlens_k is None else min(max(int(_f64(seqlens_k)[b]), 0), Lk)
        return lq, lk

    for n, (b, hq) in enumerate(pairs):
        g = hq // G                                   # KV head of this query head
        lq, lk = lengths(b)
        real = row_idx < lq                           # non-padding query rows
        # step 2: explicit score matrix over the batch's own keys; padding
        # rows see no key
        S = scale * (np.where(real[:, None], Q[b, hq, row_idx, :], 0.0) @ K[b, g, :lk].T)
        if M is not None:
            S = S + M[b, hq][row_idx, :lk]
        hidden = ~real[:, None] & np.ones((1, lk), dtype=bool)
        if causal:
            # bottom-right aligned on the batch's lengths: j <= i + (lk - lq)
            hidden |= np.arange(lk)[None, :] > (row_idx[:, None] + (lk - lq))
        S = np.where(hidden, -np.inf, S)
        if lk == 0:
            S = np.full((len(row_idx), 1), -np.inf)    # no key at all
        # step 3: row max, including the sink logit
        m = S.max(axis=1)
        if S_ is not None:
            m = np.maximum(m, S_[hq])
        live = np.isfinite(m)                         # m = -inf: nothing visible
        m_safe = np.where(live, m, 0.0)
        # step 4: max-subtracted exponentials and the denominator
        e = np.exp(S - m_safe[:, None])               # exp(-inf) = 0
        den = e.sum(axis=1)
        if S_ is not None:
            den = den + np.exp(S_[hq] - m_safe)
        # step 5: normalise; empty rows stay O = 0, LSE = -inf
        Vb = V[b, g, :lk] if lk > 0 else np.zeros((1, Dv))
        with np.errstate(divide="ignore", invalid="ignore"):
            O[n] = np.where(live[:, None], (e @ Vb) / den[:, None], 0.0)
            LSE[n] = np.where(live, m_safe + np.log(den), -np.inf)

    if heads is None:
        O = O.reshape(B, Hq, len(row_idx), Dv)
        LSE = LSE.reshape(B, Hq, len(row_idx))
    return O, LSE


def allclose_report(got, ref, atol: float, rtol: float) -> dict:
    """Elementwise |got - ref| <= atol + rtol * |ref| (the allclose form of the
    reproducer's numerical check on the D512 page), plus normwise error.

    -inf entries (empty-row LSE) must match exactly."""
    g = _f64(got)
    r = _f64(ref)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    inf_r = np.isinf(r)
    inf_ok = bool(np.all(g[inf_r] == r[inf_r])) if inf_r.any() else True
    fin = ~inf_r
    diff = np.abs(g[fin] - r[fin])
    bound = atol + rtol * np.abs(r[fin])
    ok_elem = bool(np.all(diff <= bound)) and bool(np.all(np.isfinite(g[fin])))
    nref = float(np.linalg.norm(r[fin])) if fin.any() else 0.0
    nerr = float(np.linalg.norm(g[fin] - r[fin])) if fin.any() else 0.0
    worst = int(np.argmax(diff - bound)) if diff.size else -1
    return {
        "ok": ok_elem and inf_ok,
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "max_excess": float((diff - bound).max()) if diff.size else 0.0,
        "worst_index": worst,
        "norm_rel": nerr / nref if nref > 0 else nerr,
        "inf_ok": inf_ok,
        "n": int(r.size),
    }
