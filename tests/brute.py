"""Arbitrary-precision brute-force attention for tiny inputs (test helper).

Independent of the oracle's formulation: no max subtraction (mpmath has an
unbounded exponent range), the visible key set is enumerated explicitly
instead of being masked with -inf, a sink is one extra term exp(sink) in the
denominator, and everything runs at 50 significant digits with pure-Python
loops.  Used only to pin the fp64 oracle on tiny shapes.
"""
import math

import mpmath as mp
import numpy as np


def _np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def brute_attention(q, k, v, scale, causal=False, mask=None, sinks=None, dps=50,
                    seqlens_q=None, seqlens_k=None):
    mp.mp.dps = dps
    Q, K, V = _np(q), _np(k), _np(v)
    B, Hq, Lq, D = Q.shape
    Hkv, Lk = K.shape[1], K.shape[2]
    group = Hq // Hkv
    if mask is not None and str(getattr(mask, "dtype", "")).endswith("bool"):
        # a boolean mask lists the keys that take part
        keep = np.broadcast_to(np.asarray(mask.cpu() if hasattr(mask, "cpu") else mask), (B, Hq, Lq, Lk))
        M = np.where(keep, 0.0, -math.inf)
    else:
        M = None if mask is None else np.broadcast_to(_np(mask), (B, Hq, Lq, Lk))
    SK = _np(sinks)
    Dv = V.shape[3]
    O = np.zeros((B, Hq, Lq, Dv))
    LSE = np.zeros((B, Hq, Lq))
    sc = mp.mpf(float(scale))
    for b in range(B):
        # this batch's query block and key block (the leading rows / keys)
        nq = Lq if seqlens_q is None else sorted((0, int(seqlens_q[b]), Lq))[1]
        nk = Lk if seqlens_k is None else sorted((0, int(seqlens_k[b]), Lk))[1]
        for h in range(Hq):
            kv = h // group
            for i in range(Lq):
                weights = []
                for j in range(nk if i < nq else 0):
                    # a query at position i (counted from the end of the query
                    # block) may look at keys no later than its own position
                    # counted from the end of the key block
                    if causal and (nk - 1 - j) < (nq - 1 - i):
                        continue
                    add = mp.mpf(0)
                    if M is not None:
                        if M[b, h, i, j] == -math.inf:
                            continue
                        add = mp.mpf(float(M[b, h, i, j]))
                    z = sc * mp.fsum(mp.mpf(float(Q[b, h, i, d])) * mp.mpf(float(K[b, kv, j, d]))
                                     for d in range(D)) + add
                    weights.append((j, mp.e ** z))
                den = mp.fsum(w for _, w in weights)
                if SK is not None:
                    den += mp.e ** mp.mpf(float(SK[h]))
                if den == 0:
                    LSE[b, h, i] = -math.inf
                    continue
                for d in range(Dv):
                    O[b, h, i, d] = float(mp.fsum(w * mp.mpf(float(V[b, kv, j, d]))
                                                  for j, w in weights) / den)
                LSE[b, h, i] = float(mp.log(den))
    return O, LSE
