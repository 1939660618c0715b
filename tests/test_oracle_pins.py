"""Pins for the fp64 oracle: it is checked against things other than itself.

* hand-derived closed forms (tests/golden/hand_examples.json, each cited);
* an arbitrary-precision brute force with a different formulation (tests/brute.py);
* library routines for the special cases they cover: torch's CPU fp64
  scaled_dot_product_attention (GQA, additive mask, top-left causal when
  Lq == Lk, and sinks expressed as one extra zero-valued key whose mask entry
  is the sink logit) and torch's CPU flash-attention op for the log-sum-exp;
* invariants and closed forms of the mathematics (row sums, identical keys,
  dominant logit, causal rows, sink shrink factor, mask shift, key deletion,
  head grouping, key permutation, split/merge of the key range).

The mutation test at the end plants plausible mistakes in a copy of the
oracle's source and checks that every one of them breaks at least one pin.
"""
import inspect
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as oracle_mod
from oracle import sdpa_reference
from tests.brute import brute_attention
from workloads import random_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN = {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4), "ln8": math.log(8),
      "ln3/2": math.log(3) / 2, "-inf": -math.inf}


def _num(x):
    if isinstance(x, list):
        return [_num(y) for y in x]
    return LN[x] if isinstance(x, str) else float(x)


def _t(x):
    return torch.as_tensor(x, dtype=torch.float64)


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    inf = np.isinf(b)
    assert np.array_equal(np.isinf(a), inf), f"{what}: inf pattern differs"
    assert np.all(a[inf] == b[inf]), f"{what}: inf sign differs"
    fin = ~inf
    err = np.abs(a[fin] - b[fin]).max() if fin.any() else 0.0
    scale = max(1.0, np.abs(b[fin]).max() if fin.any() else 1.0)
    assert err <= tol * scale, f"{what}: max err {err:.3e}"


# ---------------------------------------------------------------------------
# individual pins, each taking the oracle function under test
# ---------------------------------------------------------------------------

def pin_hand_examples(ref):
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        scale = _num(c["scale"])
        O, L = ref(_t(_num(c["q"])), _t(_num(c["k"])), _t(_num(c["v"])), scale=scale,
                   causal=c["causal"],
                   mask=_t(_num(c["mask"])) if "mask" in c else None,
                   sinks=_t(_num(c["sinks"])) if "sinks" in c else None)
        _close(O, _num(c["O"]), 1e-13, c["name"] + " O")
        _close(L, _num(c["LSE"]), 1e-13, c["name"] + " LSE")


BRUTE_CASES = [
    # (B, Hq, Hkv, Lq, Lk, D, causal, mask, sinks, -inf fraction)
    (1, 2, 2, 3, 5, 4, False, False, False, 0.0),
    (2, 4, 2, 3, 3, 5, True, False, False, 0.0),
    (1, 4, 1, 2, 6, 3, True, True, True, 0.3),
    (1, 2, 1, 5, 3, 4, True, False, True, 0.0),      # Lq > Lk: leading rows empty (sink only)
    (1, 3, 3, 4, 2, 2, True, False, False, 0.0),     # Lq > Lk without sinks: O = 0, LSE = -inf
    (2, 2, 1, 1, 7, 8, False, True, True, 0.5),      # decode shape
]


def pin_brute_force(ref):
    for n, (B, Hq, Hkv, Lq, Lk, D, causal, mask, sinks, frac) in enumerate(BRUTE_CASES):
        x = random_case(100 + n, B, Hq, Hkv, Lq, Lk, D, "fp32", mask=mask, sinks=sinks,
                        sink_scale=2.0, mask_neg_inf_frac=frac)
        scale = 0.7
        Ob, Lb = brute_attention(x["q"], x["k"], x["v"], scale, causal, x["mask"], x["sinks"])
        Oo, Lo = ref(x["q"], x["k"], x["v"], scale=scale, causal=causal, mask=x["mask"],
                     sinks=x["sinks"])
        _close(Oo, Ob, 1e-12, f"brute case {n} O")
        _close(Lo, Lb, 1e-12, f"brute case {n} LSE")


def _sinks_as_extra_key(q, k, v, mask, sinks):
    """Sinks == one extra key with zero key/value vectors whose mask entry is the
    sink logit (scale * q.0 = 0, plus the mask).  Returns augmented k, v, mask."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    k2 = torch.cat([k, torch.zeros(B, Hkv, 1, D, dtype=k.dtype)], dim=2)
    v2 = torch.cat([v, torch.zeros(B, Hkv, 1, D, dtype=v.dtype)], dim=2)
    base = torch.zeros(B, Hq, Lq, Lk, dtype=torch.float64) if mask is None else \
        torch.broadcast_to(mask.double(), (B, Hq, Lq, Lk))
    col = sinks.double().view(1, Hq, 1, 1).expand(B, Hq, Lq, 1)
    return k2, v2, torch.cat([base, col], dim=3)


def pin_torch_sdpa(ref):
    # (a) GQA + additive mask, Lq != Lk, non-causal
    x = random_case(7, 2, 6, 2, 5, 9, 16, "fp32", mask=True)
    q, k, v, m = (x[n].double() for n in ("q", "k", "v", "mask"))
    o_t = F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=0.3, enable_gqa=True)
    O, _ = ref(q, k, v, scale=0.3, mask=m)
    _close(O, o_t.numpy(), 1e-12, "torch sdpa gqa+mask")
    # (b) causal with Lq == Lk (top-left and bottom-right coincide)
    x = random_case(8, 1, 4, 4, 11, 11, 8, "fp32")
    q, k, v = (x[n].double() for n in ("q", "k", "v"))
    o_t = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.5)
    O, _ = ref(q, k, v, scale=0.5, causal=True)
    _close(O, o_t.numpy(), 1e-12, "torch sdpa causal")
    # (c) sinks as an extra zero-valued key carrying the sink logit in the mask
    x = random_case(9, 1, 4, 2, 3, 6, 8, "fp32", mask=True, sinks=True, sink_scale=3.0)
    q, k, v, m, s = (x[n].double() for n in ("q", "k", "v", "mask", "sinks"))
    k2, v2, m2 = _sinks_as_extra_key(q, k, v, m, s)
    o_t = F.scaled_dot_product_attention(q, k2, v2, attn_mask=m2, scale=0.4, enable_gqa=True)
    O, _ = ref(q, k, v, scale=0.4, mask=m, sinks=s)
    _close(O, o_t.numpy(), 1e-12, "torch sdpa sinks")


def pin_torch_lse(ref):
    flash = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu
    x = random_case(10, 2, 3, 3, 4, 7, 8, "fp32", mask=True)
    q, k, v, m = (x[n].double() for n in ("q", "k", "v", "mask"))
    o_t, l_t = flash(q, k, v, 0.0, False, attn_mask=m, scale=0.6)
    O, L = ref(q, k, v, scale=0.6, mask=m)
    _close(O, o_t.numpy(), 1e-12, "flash cpu O")
    _close(L, l_t.numpy(), 1e-12, "flash cpu LSE")
    x = random_case(11, 1, 2, 2, 9, 9, 4, "fp32")
    q, k, v = (x[n].double() for n in ("q", "k", "v"))
    o_t, l_t = flash(q, k, v, 0.0, True, scale=0.9)
    O, L = ref(q, k, v, scale=0.9, causal=True)
    _close(L, l_t.numpy(), 1e-12, "flash cpu causal LSE")
    # sinks: LSE = log-sum-exp over the keys plus the extra sink column
    x = random_case(12, 1, 2, 1, 3, 5, 4, "fp32", sinks=True, sink_scale=2.0)
    q, k, v, s = (x[n].double() for n in ("q", "k", "v", "sinks"))
    k2, v2, m2 = _sinks_as_extra_key(q, k, v, None, s)
    _, l_t = flash(q, k2, v2, 0.0, False, attn_mask=m2, scale=0.8)
    _, L = ref(q, k, v, scale=0.8, sinks=s)
    _close(L, l_t.numpy(), 1e-12, "flash cpu sink LSE")


def pin_probabilities(ref):
    """With V = identity (D = Lk), O is the attention-probability matrix: rows sum
    to 1 - exp(sink - LSE); log-ratios of probabilities equal logit differences."""
    B, Hq, Lq, Lk = 1, 2, 4, 6
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, Hq, Lq, Lk))
    k = rng.standard_normal((B, Hq, Lk, Lk))
    v = np.broadcast_to(np.eye(Lk), (B, Hq, Lk, Lk)).copy()
    sinks = np.array([0.5, -1.0])
    for sk in (None, sinks):
        P, L = ref(q, k, v, scale=0.8, sinks=sk)
        tot = P.sum(-1)
        expect = np.ones_like(tot) if sk is None else 1 - np.exp(sk[None, :, None] - L)
        _close(tot, expect, 1e-13, "row sums")
        # log p_ij - log p_i0 = scale * q_i . (k_j - k_0)
        lr = np.log(P) - np.log(P[..., :1])
        dz = 0.8 * np.einsum("bhid,bhjd->bhij", q, k - k[:, :, :1])
        _close(lr, dz, 1e-12, "logit differences")


def pin_invariants(ref):
    rng = np.random.default_rng(3)
    B, Hq, Lq, Lk, D = 1, 2, 5, 7, 6
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hq, Lk, D))
    v = rng.standard_normal((B, Hq, Lk, D))

    # identical keys: O = mean of the visible V rows (causal: the first i+off+1)
    k_same = np.broadcast_to(k[:, :, :1], k.shape).copy()
    O, _ = ref(q, k_same, v, scale=0.9)
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), 1e-13, "identical keys")
    O, _ = ref(q, k_same, v, scale=0.9, causal=True)
    off = Lk - Lq
    for i in range(Lq):
        _close(O[:, :, i], v[:, :, :i + off + 1].mean(axis=2), 1e-13, "identical keys causal")

    # one dominant logit selects that V row
    jstar = 4
    kd = k.copy()
    kd[:, :, jstar] = 60.0 * q[:, :, 1]
    O, _ = ref(q[:, :, 1:2], kd, v, scale=1.0)
    _close(O[:, :, 0], v[:, :, jstar], 1e-9, "dominant logit")

    # causal with Lq == Lk: row 0 is V[0]; the last row equals the non-causal row
    O_c, _ = ref(q[:, :, :5], k[:, :, :5], v[:, :, :5], scale=0.7, causal=True)
    O_n, _ = ref(q[:, :, :5], k[:, :, :5], v[:, :, :5], scale=0.7)
    _close(O_c[:, :, 0], v[:, :, 0], 1e-15, "causal row 0")
    _close(O_c[:, :, -1], O_n[:, :, -1], 1e-13, "causal last row")

    # sinks only shrink: O_s = sigmoid(LSE - sink) O,  LSE_s = logaddexp(LSE, sink)
    sinks = np.array([0.3, 2.5])
    O0, L0 = ref(q, k, v, scale=0.9)
    O1, L1 = ref(q, k, v, scale=0.9, sinks=sinks)
    sig = 1.0 / (1.0 + np.exp(sinks[None, :, None] - L0))
    _close(O1, sig[..., None] * O0, 1e-13, "sink shrink")
    _close(L1, np.logaddexp(L0, sinks[None, :, None]), 1e-13, "sink LSE")
    O2, L2 = ref(q, k, v, scale=0.9, sinks=np.array([-np.inf, -np.inf]))
    _close(O2, O0, 1e-15, "sink -inf")
    _close(L2, L0, 1e-15, "sink -inf LSE")

    # one key: O = V[0]; with a sink: sigmoid(s0 - sink) V[0]
    O, L = ref(q, k[:, :, :1], v[:, :, :1], scale=0.5)
    _close(O, np.broadcast_to(v[:, :, :1], O.shape), 1e-15, "Lk = 1")
    s0 = 0.5 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0])
    _close(L, s0, 1e-14, "Lk = 1 LSE")
    O, _ = ref(q, k[:, :, :1], v[:, :, :1], scale=0.5, sinks=sinks)
    sig = 1.0 / (1.0 + np.exp(sinks[None, :, None] - s0))
    _close(O, sig[..., None] * v[:, :, :1], 1e-14, "Lk = 1 sink")

    # scale 0: uniform weights; LSE = log Lk
    O, L = ref(q, k, v, scale=0.0)
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), 1e-14, "scale 0")
    _close(L, np.full(L.shape, math.log(Lk)), 1e-14, "scale 0 LSE")

    # a constant additive mask moves LSE by c and leaves O unchanged
    O3, L3 = ref(q, k, v, scale=0.9, mask=np.full((1, 1, 1, Lk), 3.25))
    _close(O3, O0, 1e-13, "mask shift O")
    _close(L3, L0 + 3.25, 1e-13, "mask shift LSE")

    # a -inf mask on a key set is the same as deleting those keys
    keep = np.array([0, 2, 3, 6])
    m = np.full((1, 1, 1, Lk), -np.inf)
    m[..., keep] = 0.0
    O4, L4 = ref(q, k, v, scale=0.9, mask=m)
    O5, L5 = ref(q, k[:, :, keep], v[:, :, keep], scale=0.9)
    _close(O4, O5, 1e-13, "mask delete O")
    _close(L4, L5, 1e-13, "mask delete LSE")

    # Q -> a Q is the same as scale -> a scale
    O6, L6 = ref(2.5 * q, k, v, scale=0.4)
    O7, L7 = ref(q, k, v, scale=1.0)
    _close(O6, O7, 1e-13, "q scaling")
    _close(L6, L7, 1e-13, "q scaling LSE")

    # permuting keys and values together leaves non-causal results unchanged
    perm = rng.permutation(Lk)
    O8, L8 = ref(q, k[:, :, perm], v[:, :, perm], scale=0.9)
    _close(O8, O0, 1e-13, "key permutation")
    _close(L8, L0, 1e-13, "key permutation LSE")


def pin_gqa_equals_repeat(ref):
    x = random_case(21, 2, 8, 2, 3, 5, 4, "fp32", mask=True, sinks=True)
    q, k, v, m, s = (x[n] for n in ("q", "k", "v", "mask", "sinks"))
    O, L = ref(q, k, v, scale=0.6, mask=m, sinks=s, causal=True)
    kr = k.repeat_interleave(4, dim=1)
    vr = v.repeat_interleave(4, dim=1)
    O2, L2 = ref(q, kr, vr, scale=0.6, mask=m, sinks=s, causal=True)
    _close(O, O2, 1e-14, "gqa vs repeat")
    _close(L, L2, 1e-14, "gqa vs repeat LSE")


def pin_split_merge(ref):
    """The log-sum-exp merge of two key ranges equals the whole: the algebra
    that a split-K decode uses to combine its partial results."""
    x = random_case(22, 1, 4, 2, 1, 12, 8, "fp32", mask=True, mask_neg_inf_frac=0.2)
    q, k, v, m = (x[n].double() for n in ("q", "k", "v", "mask"))
    O, L = ref(q, k, v, scale=0.5, mask=m)
    Oa, La = ref(q, k[:, :, :5], v[:, :, :5], scale=0.5, mask=m[..., :5])
    Ob, Lb = ref(q, k[:, :, 5:], v[:, :, 5:], scale=0.5, mask=m[..., 5:])
    Lm = np.logaddexp(La, Lb)
    wa = np.exp(La - Lm)[..., None]
    wb = np.exp(Lb - Lm)[..., None]
    _close(Lm, L, 1e-13, "merge LSE")
    _close(wa * Oa + wb * Ob, O, 1e-13, "merge O")


SEQLEN_CASES = [
    # (B, Hq, Hkv, Lq, Lk, D, causal, mask, sinks, seqlens_q, seqlens_k)
    (3, 2, 1, 4, 6, 3, True, False, False, [4, 2, 3], [6, 3, 5]),
    (3, 2, 2, 3, 5, 4, False, True, True, [3, 0, 1], [0, 5, 2]),   # empty batches
    (2, 4, 2, 1, 7, 4, False, False, True, [1, 1], [7, 4]),         # decode shape
    (2, 2, 1, 5, 4, 2, True, False, True, [5, 2], [2, 4]),          # lq_b > lk_b
]


def pin_seqlens(ref):
    """Per-batch lengths (padding masks): brute force on tiny shapes, padding
    equal to truncation, and padding contents never read."""
    for n, (B, Hq, Hkv, Lq, Lk, D, causal, mask, sinks, sq, sk) in enumerate(SEQLEN_CASES):
        x = random_case(150 + n, B, Hq, Hkv, Lq, Lk, D, "fp32", mask=mask, sinks=sinks,
                        sink_scale=2.0, mask_neg_inf_frac=0.2)
        sq_, sk_ = np.array(sq), np.array(sk)
        kw = dict(scale=0.8, causal=causal, mask=x["mask"], sinks=x["sinks"])
        O, L = ref(x["q"], x["k"], x["v"], seqlens_q=sq_, seqlens_k=sk_, **kw)
        Ob, Lb = brute_attention(x["q"], x["k"], x["v"], 0.8, causal, x["mask"], x["sinks"],
                                 seqlens_q=sq, seqlens_k=sk)
        _close(O, Ob, 1e-12, f"seqlens brute {n} O")
        _close(L, Lb, 1e-12, f"seqlens brute {n} LSE")
        for b in range(B):
            lq, lk = sq[b], sk[b]
            if lq == 0 or lk == 0:
                continue
            m = None if x["mask"] is None else x["mask"][b:b + 1, :, :lq, :lk]
            Ot, Lt = ref(x["q"][b:b + 1, :, :lq], x["k"][b:b + 1, :, :lk], x["v"][b:b + 1, :, :lk],
                         scale=0.8, causal=causal, mask=m, sinks=x["sinks"])
            _close(O[b, :, :lq], Ot[0], 1e-14, f"seqlens truncation {n}.{b} O")
            _close(L[b, :, :lq], Lt[0], 1e-14, f"seqlens truncation {n}.{b} LSE")
        # padding rows are empty rows: O = 0, LSE = sink or -inf
        for b in range(B):
            assert np.all(O[b, :, sq[b]:] == 0.0)
            want = -np.inf if x["sinks"] is None else np.asarray(x["sinks"], np.float64)[:, None]
            _close(L[b, :, sq[b]:], np.broadcast_to(want, L[b, :, sq[b]:].shape), 0, "padding row LSE")
        # garbage in the padding changes nothing
        q2, k2, v2 = x["q"].clone(), x["k"].clone(), x["v"].clone()
        for b in range(B):
            q2[b, :, sq[b]:] = float("nan")
            k2[b, :, sk[b]:] = 1e30
            v2[b, :, sk[b]:] = float("nan")
        O2, L2 = ref(q2, k2, v2, seqlens_q=sq_, seqlens_k=sk_, **kw)
        _close(O2, O, 0, f"seqlens garbage {n} O")
        _close(L2, L, 0, f"seqlens garbage {n} LSE")
    # lengths at the tensor extents equal no lengths at all
    x = random_case(160, 2, 2, 2, 4, 6, 3, "fp32", mask=True, sinks=True)
    kw = dict(scale=0.8, causal=True, mask=x["mask"], sinks=x["sinks"])
    O, L = ref(x["q"], x["k"], x["v"], **kw)
    O2, L2 = ref(x["q"], x["k"], x["v"], seqlens_q=np.array([4, 9]), seqlens_k=np.array([6, 6]), **kw)
    _close(O2, O, 0, "full lengths O")
    _close(L2, L, 0, "full lengths LSE")


def pin_bool_mask(ref):
    """A boolean mask (True = the key takes part) against the brute force,
    which enumerates the listed keys, with causal masking and sinks, and a
    row whose keys are all hidden."""
    for n, (causal, sinks) in enumerate(((False, False), (True, True))):
        x = random_case(170 + n, 2, 4, 2, 5, 7, 3, "fp32", sinks=sinks, sink_scale=2.0)
        keep = np.random.default_rng(180 + n).random((2, 1, 5, 7)) < 0.6
        keep[0, 0, 2, :] = False
        mb = torch.from_numpy(keep)
        O, L = ref(x["q"], x["k"], x["v"], scale=0.7, causal=causal, mask=mb, sinks=x["sinks"])
        Ob, Lb = brute_attention(x["q"], x["k"], x["v"], 0.7, causal, mb, x["sinks"])
        _close(O, Ob, 1e-12, f"bool mask {n} O")
        _close(L, Lb, 1e-12, f"bool mask {n} LSE")


def pin_value_head_dim(ref):
    """Values with a head dim other than the keys' (D_v != D_qk): brute force,
    and the output columns are those of V alone (splitting V by columns
    splits O the same way)."""
    x = random_case(190, 2, 4, 2, 4, 6, 3, "fp32", sinks=True, sink_scale=1.5)
    v5 = torch.from_numpy(np.random.default_rng(191).standard_normal((2, 2, 6, 5)).astype(np.float32))
    O, L = ref(x["q"], x["k"], v5, scale=0.8, causal=True, sinks=x["sinks"])
    Ob, Lb = brute_attention(x["q"], x["k"], v5, 0.8, True, None, x["sinks"])
    _close(O, Ob, 1e-12, "Dv != D O")
    _close(L, Lb, 1e-12, "Dv != D LSE")
    O2, _ = ref(x["q"], x["k"], v5[..., 1:4], scale=0.8, causal=True, sinks=x["sinks"])
    _close(O[..., 1:4], O2, 1e-14, "value columns")


PINS = [pin_hand_examples, pin_brute_force, pin_torch_sdpa, pin_torch_lse,
        pin_probabilities, pin_invariants, pin_gqa_equals_repeat, pin_split_merge,
        pin_seqlens, pin_bool_mask, pin_value_head_dim]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(sdpa_reference)


def test_oracle_rows_and_heads_subsets():
    """The sampled-row / sampled-head modes used at full sizes agree with the
    full computation."""
    x = random_case(30, 2, 4, 2, 9, 13, 8, "fp32", mask=True, sinks=True)
    O, L = sdpa_reference(x["q"], x["k"], x["v"], scale=0.3, causal=True,
                          mask=x["mask"], sinks=x["sinks"])
    rows = [0, 4, 8]
    heads = [(0, 1), (1, 3)]
    Os, Ls = sdpa_reference(x["q"], x["k"], x["v"], scale=0.3, causal=True,
                            mask=x["mask"], sinks=x["sinks"], rows=rows, heads=heads)
    for n, (b, h) in enumerate(heads):
        _close(Os[n], O[b, h, rows], 0, "rows subset O")
        _close(Ls[n], L[b, h, rows], 0, "rows subset LSE")


def test_d512_grid_covers_page_cases():
    import workloads
    with open(os.path.join(GOLDEN, "d512_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        hits = [w for w in workloads.GQA_DECODE
                if (w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, w.dtype, w.sinks)
                == (c["b"], c["h"], c["hk"], c["ql"], c["kl"], c["d"], c["dtype"], c["sinks"])]
        assert hits, c["name"]


# ---------------------------------------------------------------------------
# mutation test: a plausible mistake anywhere in the oracle breaks some pin
# ---------------------------------------------------------------------------

MUTANTS = {
    "causal_top_left": ("(row_idx[:, None] + (lk - lq))", "(row_idx[:, None])"),
    "causal_off_by_one": ("hidden |= np.arange(lk)[None, :] >", "hidden |= np.arange(lk)[None, :] >="),
    "causal_on_tensor_extents": ("(row_idx[:, None] + (lk - lq))", "(row_idx[:, None] + (Lk - Lq))"),
    "padding_rows_see_keys": ("real = row_idx < lq ", "real = row_idx < Lq "),
    "padding_keys_seen": ("int(_f64(seqlens_k)[b])", "int(_f64(seqlens_k)[b]) + 1"),
    "bool_mask_inverted": ("np.where(m, 0.0, -np.inf)", "np.where(m, -np.inf, 0.0)"),
    "sink_not_in_denominator": ("den = den + np.exp(S_[hq] - m_safe)", "den = den"),
    "sink_not_in_max": ("m = np.maximum(m, S_[hq])", "m = m"),
    "head_map_modulo": ("        g = hq // G ", "        g = hq % Hkv "),
    "scale_dropped": ("S = scale * (", "S = ("),
    "mask_sign": ("S = S + M[b, hq][row_idx, :lk]", "S = S - M[b, hq][row_idx, :lk]"),
    "lse_without_max": ("m_safe + np.log(den), -np.inf", "np.log(den), -np.inf"),
    "values_from_keys": ("Vb = V[b, g, :lk]", "Vb = K[b, g, :lk]"),
    "exp_sign": ("e = np.exp(S - m_safe[:, None])", "e = np.exp(m_safe[:, None] - S)"),
    "lse_log2": ("m_safe + np.log(den)", "m_safe + np.log2(den)"),
}


def _mutant(old, new):
    src = inspect.getsource(oracle_mod)
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    ns = {"__name__": "oracle_mutant"}
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), ns)
    return ns["sdpa_reference"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    fn = _mutant(*MUTANTS[name])
    failures = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except Exception as e:   # AssertionError, or a crash caused by the mistake
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"mutant {name} passed every pin"
