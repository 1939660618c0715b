"""Pins for the fp64 gradient oracle (oracle/backward.py), each against
something other than the oracle itself:

* central finite differences of the scalar sum(dO * O) computed with the
  forward oracle (which is pinned on its own), for every element of Q, K, V
  and the sink logits, on tiny shapes covering GQA, bottom-right causal with
  Lq != Lk, an additive mask with -inf entries, sinks and per-batch lengths;
* torch's CPU fp64 autograd through F.scaled_dot_product_attention (GQA,
  additive mask, causal with Lq == Lk);
* closed forms: without sinks the rows of dS sum to zero, so sum_j dK_j = 0,
  and the rows of P sum to one, so sum_j dV_j = sum_i dO_i.

Planted mistakes in a copy of the oracle's source must each break a pin.
"""
import inspect

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.backward as bwd_mod
from oracle import sdpa_backward_reference, sdpa_reference
from workloads import random_case


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b).max() if a.size else 0.0
    scale = max(1.0, np.abs(b).max() if b.size else 1.0)
    assert err <= tol * scale, f"{what}: max err {err:.3e}"


FD_CASES = [
    # (B, Hq, Hkv, Lq, Lk, D, causal, mask, sinks, seqlens_q, seqlens_k, Dv)
    (1, 2, 2, 3, 4, 3, False, False, False, None, None, None),
    (2, 4, 2, 3, 5, 2, True, False, True, None, None, None),       # GQA, causal Lq < Lk, sinks
    (1, 2, 1, 4, 3, 2, True, True, True, None, None, None),        # Lq > Lk, mask with -inf
    (2, 2, 1, 3, 4, 2, True, False, True, [3, 2], [4, 1], None),   # per-batch lengths
    (1, 2, 1, 3, 4, 2, True, False, True, None, None, 3),          # value head dim 3 != 2
]


def _loss(q, k, v, dout, sinks, kw):
    O, _ = sdpa_reference(q, k, v, sinks=sinks, **kw)
    return float(np.sum(O * dout))


def pin_finite_differences(ref):
    h = 1e-6
    for n, (B, Hq, Hkv, Lq, Lk, D, causal, mask, sinks, sq, sk, Dv) in enumerate(FD_CASES):
        x = random_case(500 + n, B, Hq, Hkv, Lq, Lk, D, "fp32", mask=mask, sinks=sinks,
                        sink_scale=1.5, mask_neg_inf_frac=0.25, Dv=Dv)
        q, k, v = (x[t].double().numpy() for t in ("q", "k", "v"))
        s = None if x["sinks"] is None else x["sinks"].double().numpy()
        dout = np.random.default_rng(600 + n).standard_normal(q.shape[:3] + v.shape[3:])
        kw = dict(scale=0.9, causal=causal, mask=x["mask"],
                  seqlens_q=None if sq is None else np.array(sq),
                  seqlens_k=None if sk is None else np.array(sk))
        dq, dk, dv, ds = ref(q, k, v, dout, sinks=s, **kw)
        for name, arr, got in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                a0 = arr[idx]
                arr[idx] = a0 + h
                lp = _loss(q, k, v, dout, s, kw)
                arr[idx] = a0 - h
                lm = _loss(q, k, v, dout, s, kw)
                arr[idx] = a0
                fd[idx] = (lp - lm) / (2 * h)
            _close(got, fd, 1e-7, f"fd case {n} d{name}")
        if s is not None:
            fd = np.zeros_like(s)
            for i in range(len(s)):
                s0 = s[i]
                s[i] = s0 + h
                lp = _loss(q, k, v, dout, s, kw)
                s[i] = s0 - h
                lm = _loss(q, k, v, dout, s, kw)
                s[i] = s0
                fd[i] = (lp - lm) / (2 * h)
            _close(ds, fd, 1e-7, f"fd case {n} dsinks")
        else:
            assert ds is None


def pin_torch_autograd(ref):
    cases = [
        dict(seed=31, B=2, Hq=4, Hkv=2, Lq=5, Lk=7, D=8, causal=False, mask=True),
        dict(seed=32, B=1, Hq=2, Hkv=2, Lq=9, Lk=9, D=4, causal=True, mask=False),
        dict(seed=33, B=1, Hq=6, Hkv=3, Lq=6, Lk=6, D=8, causal=True, mask=False),
    ]
    for c in cases:
        x = random_case(c["seed"], c["B"], c["Hq"], c["Hkv"], c["Lq"], c["Lk"], c["D"], "fp32",
                        mask=c["mask"])
        q, k, v = (x[t].double().requires_grad_(True) for t in ("q", "k", "v"))
        m = None if x["mask"] is None else x["mask"].double()
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=m, is_causal=c["causal"], scale=0.7,
                                           enable_gqa=True)
        dout = torch.from_numpy(np.random.default_rng(c["seed"]).standard_normal(o.shape))
        o.backward(dout)
        dq, dk, dv, _ = ref(q.detach(), k.detach(), v.detach(), dout, scale=0.7,
                            causal=c["causal"], mask=m)
        _close(dq, q.grad.numpy(), 1e-12, f"autograd dq {c['seed']}")
        _close(dk, k.grad.numpy(), 1e-12, f"autograd dk {c['seed']}")
        _close(dv, v.grad.numpy(), 1e-12, f"autograd dv {c['seed']}")


def pin_closed_forms(ref):
    x = random_case(40, 2, 4, 4, 6, 9, 5, "fp32", mask=True, mask_neg_inf_frac=0.2)
    dout = np.random.default_rng(41).standard_normal(x["q"].shape)
    dq, dk, dv, _ = ref(x["q"], x["k"], x["v"], dout, scale=0.6, mask=x["mask"])
    # sum over keys of dK is scale * sum_i (sum_j dS_ij) Q_i = 0
    _close(dk.sum(axis=2), np.zeros_like(dk.sum(axis=2)), 1e-12, "sum_j dK_j")
    # sum over keys of dV is sum_i (sum_j P_ij) dO_i = sum_i dO_i (every row sees a key)
    _close(dv.sum(axis=2), dout.sum(axis=2), 1e-12, "sum_j dV_j")


PINS = [pin_finite_differences, pin_torch_autograd, pin_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_oracle_pin(pin):
    pin(sdpa_backward_reference)


MUTANTS = {
    "dq_without_scale": ("dQ[b, hq, :lq] = scale * (dS @ Kb)", "dQ[b, hq, :lq] = (dS @ Kb)"),
    "dk_without_scale": ("dK[b, g, :lk] += scale * (dS.T @ Qb)", "dK[b, g, :lk] += (dS.T @ Qb)"),
    "dk_from_p": ("dK[b, g, :lk] += scale * (dS.T @ Qb)", "dK[b, g, :lk] += scale * (P.T @ Qb)"),
    "dv_from_ds": ("dV[b, g, :lk] += P.T @ dOb", "dV[b, g, :lk] += dS.T @ dOb"),
    "d_sign": ("dS = P * (dP - Di[:, None])", "dS = P * (dP + Di[:, None])"),
    "d_dropped": ("dS = P * (dP - Di[:, None])", "dS = P * dP"),
    "dp_from_keys": ("dP = dOb @ Vb.T", "dP = dOb @ Kb.T"),
    "head_map_modulo": ("            g = hq // G\n", "            g = hq % Hkv\n"),
    "dsink_sign": ("dsink[hq] -= float", "dsink[hq] += float"),
    "p_without_lse": ("np.exp(S - np.where(live, Lb, 0.0)[:, None])", "np.exp(S)"),
    "causal_top_left": ("rows[:, None] + (lk - lq)", "rows[:, None]"),
}


def _mutant(old, new):
    src = inspect.getsource(bwd_mod)
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    ns = {"__name__": "oracle.backward_mutant", "__package__": "oracle"}
    exec(compile(src.replace(old, new), "oracle_backward_mutant", "exec"), ns)
    return ns["sdpa_backward_reference"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_backward_mistake_is_caught(name):
    fn = _mutant(*MUTANTS[name])
    failures = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except Exception as e:
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"mutant {name} passed every pin"
