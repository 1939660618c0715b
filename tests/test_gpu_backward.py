"""GPU parity of the attention gradients (sdpa_prefill_backward through the C
ABI) against the fp64 gradient oracle: a grid of small cases spanning several
tiles with ragged tails (GQA, bottom-right causal with Lq != Lk, rows without
keys, additive mask with -inf entries, sinks and their gradient, per-batch
lengths with NaN in the padding) for fp32 / fp16 / bf16 and D = 64 / 128, head dims
that are multiples of 8 up to 128 with Dv != D, plus the
autograd wrapper.

Tolerance: gradients are linear in dO, so the forward's elementwise bound
(abs 2e-3, rel 1e-2 for 16-bit inputs) is applied with the absolute part
scaled by the tensor's largest reference magnitude (at least 1):
|got - ref| <= 2e-3 * max(1, max|ref|) + 1e-2 * |ref| (fp32: 1e-5 * max(1, max|ref|),
the forward's fp32 bound scaled the same way).  The 16-bit kernels round P
and dS to the input type (unit roundoff 2^-11 fp16, 2^-8 bf16) before the
second products and accumulate in fp32, which stays inside this bound."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_prefill_amd as sdpa
from oracle import allclose_report, sdpa_backward_reference
from tests.gpu_util import say, to_dev
from tests.grad_bound import grad_magnitudes
from workloads import DTYPES, random_case

pytestmark = pytest.mark.gpu


# unit roundoff of the input type; the elementwise gate's multiple of it
# (measured worst over these tests: bf16 0.66, fp16 0.72, fp32 19.6); the
# absolute rounding step of a result stored below fp16's normal range (2^-14
# and down: step 2^-24, error at most 2^-25)
UNIT = {"fp32": 2.0 ** -24, "fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
C_ELEM = {"fp32": 64.0, "fp16": 4.0, "bf16": 2.0}
OUT_FLOOR = {"fp32": 0.0, "fp16": 2.0 ** -25, "bf16": 0.0}


def _report(got, ref, what, dtype="bf16", mag=None):
    """Three gates: |got - ref| <= atol max(1, max|ref|) + rtol |ref|; the
    normwise relative error; and, with the magnitude companion `mag` of each
    element's sum, |got - ref| <= C u mag + u |ref| + (fp16: 2^-25) element
    by element (a small element of a tensor with a large maximum gets its
    own scale; the last two terms are the rounding of the stored result)."""
    ref = np.asarray(ref, dtype=np.float64)
    s = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    atol, rtol, nrel = (1e-5, 0.0, 1e-5) if dtype == "fp32" else (2e-3, 1e-2, 1e-2)
    g = got.float().cpu().numpy().astype(np.float64)
    rep = allclose_report(g, ref, atol * s, rtol)
    ok = rep["ok"] and rep["norm_rel"] <= nrel
    elem = ""
    if mag is not None:
        mag = np.asarray(mag, dtype=np.float64)
        assert np.all(np.abs(ref) <= mag * (1 + 1e-9) + 1e-300), f"{what}: companion below its reference"
        u = UNIT[dtype]
        excess = np.abs(g - ref) - u * np.abs(ref) - OUT_FLOOR[dtype]
        zero = mag == 0
        ratio = float(np.max(excess[~zero] / (u * mag[~zero]))) if np.any(~zero) else 0.0
        ok_zero = bool(np.all(excess[zero] <= 0)) if np.any(zero) else True
        ok = ok and ratio <= C_ELEM[dtype] and ok_zero
        rep["elem_ratio"], rep["elem_zero_ok"] = ratio, ok_zero
        elem = f" elem_ratio={ratio:.3g} (gate {C_ELEM[dtype]:g}) zero_ok={ok_zero}"
        if ratio > C_ELEM[dtype] or not ok_zero:
            rr = np.where(zero, 0.0, excess / np.maximum(u * mag, 1e-300))
            idx = np.unravel_index(np.argmax(rr), rr.shape)
            sl = tuple(idx[:3])
            say(f"    worst {idx}: got={g[idx]:.6e} ref={ref[idx]:.6e} mag={mag[idx]:.3e} "
                f"row |ref| max={np.abs(ref[sl]).max():.3e} row mag max={mag[sl].max():.3e} "
                f"over the gate: {int(np.sum(rr > C_ELEM[dtype]))}")
    say(f"  {what}: max_abs={rep['max_abs']:.3e} (scale {s:.3g}) norm_rel={rep['norm_rel']:.3e}{elem} ok={ok}")
    return None if ok else f"{what}: {rep}"


def _check_all(pairs, dtype="bf16", mags=None):
    """Report every gradient, then fail on the first mismatch.  mags: the
    magnitude companions of the first three pairs (dq, dk, dv)."""
    bad = [m for m in (_report(g, r, w, dtype, mags[i] if mags is not None and i < 3 else None)
                       for i, (g, r, w) in enumerate(pairs)) if m]
    assert not bad, bad


def _reference(q, k, v, dout, **kw):
    """The oracle's gradients and their magnitude companions (with fp16's
    absolute rounding floor below its normal range)."""
    floor = 2.0 ** -14 if q.dtype == torch.float16 else 0.0
    return sdpa_backward_reference(q, k, v, dout, **kw), grad_magnitudes(q, k, v, dout, floor=floor, **kw)


def _dout(seed, shape, dtype):
    g = np.random.default_rng([2, seed]).standard_normal(shape, dtype=np.float32)
    return torch.from_numpy(g).to(DTYPES[dtype])


def _run(x, dout, dtype, causal, sq=None, sk=None, want_dsinks=False):
    d = to_dev(x)
    D = x["q"].shape[-1]
    sc = 1.0 / math.sqrt(D)
    o, lse = sdpa.prefill(d["q"], d["k"], d["v"], scale=sc, causal=causal, mask=d["mask"], sinks=d["sinks"],
                          return_lse=True, seqlens_q=sq, seqlens_k=sk)
    res = sdpa.prefill_backward(d["q"], d["k"], d["v"], o, lse, dout.cuda(), scale=sc, causal=causal,
                                mask=d["mask"], sinks=d["sinks"], seqlens_q=sq, seqlens_k=sk,
                                want_dsinks=want_dsinks)
    torch.cuda.synchronize()
    return res, sc


# (B, Hq, Hkv, Lq, Lk, causal, mask, sinks)
GRID = [
    (1, 2, 2, 200, 333, False, False, False),   # ragged non-causal
    (2, 4, 2, 300, 300, True, False, False),    # causal Lq == Lk, GQA
    (1, 2, 1, 100, 357, True, False, True),     # bottom-right causal Lq < Lk, sinks
    (1, 2, 2, 260, 130, True, False, False),    # Lq > Lk: leading rows see nothing
    (1, 3, 1, 129, 257, False, True, True),     # mask with -inf entries and sinks
    (2, 2, 2, 64, 64, True, True, False),       # causal + mask together
]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", range(len(GRID)))
def test_backward_grid(dtype, D, case):
    B, Hq, Hkv, Lq, Lk, causal, mask, sinks = GRID[case]
    say(f"backward {dtype} D={D} case={GRID[case]}")
    x = random_case(5000 + 10 * case + D, B, Hq, Hkv, Lq, Lk, D, dtype, mask=mask, sinks=sinks,
                    sink_scale=2.0, mask_neg_inf_frac=0.1)
    dout = _dout(5000 + case, x["q"].shape, dtype)
    (dq, dk, dv, ds), sc = _run(x, dout, dtype, causal, want_dsinks=True)
    (rq, rk, rv, rs), mags = _reference(x["q"], x["k"], x["v"], dout, scale=sc, causal=causal,
                                             mask=x["mask"], sinks=x["sinks"])
    pairs = [(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")]
    if sinks:
        pairs.append((ds, rs, "dsinks"))
    else:
        assert ds is None
    _check_all(pairs, dtype, mags)


# (D, Dv): head dims that are multiples of 8 up to 128, run at kernel dim 64
# or 128 with zero chunks past the real dims
BWD_DIMS = [(8, 8), (40, 40), (96, 96), (112, 112), (128, 64), (64, 120)]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("dims", BWD_DIMS, ids=lambda d: f"{d[0]}x{d[1]}")
@pytest.mark.parametrize("causal", [False, True])
def test_backward_head_dims(dtype, dims, causal):
    D, Dv = dims
    B, Hq, Hkv, Lq, Lk = 2, 4, 2, 150, 211
    say(f"backward head dims {dtype} D={D} Dv={Dv} causal={causal}")
    x = random_case(5300 + D + Dv, B, Hq, Hkv, Lq, Lk, D, dtype, Dv=Dv, sinks=causal, sink_scale=2.0)
    dout = _dout(5300 + D, (B, Hq, Lq, Dv), dtype)
    (dq, dk, dv, ds), sc = _run(x, dout, dtype, causal, want_dsinks=True)
    assert dq.shape == x["q"].shape and dk.shape == x["k"].shape and dv.shape == x["v"].shape
    (rq, rk, rv, rs), mags = _reference(x["q"], x["k"], x["v"], dout, scale=sc, causal=causal,
                                             sinks=x["sinks"])
    pairs = [(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")]
    if causal:
        pairs.append((ds, rs, "dsinks"))
    _check_all(pairs, dtype, mags)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_backward_seqlens(dtype):
    B, Hq, Hkv, Lq, Lk, D = 3, 4, 2, 300, 333, 128
    sq, sk = [300, 129, 0], [333, 200, 3]
    x = random_case(5100, B, Hq, Hkv, Lq, Lk, D, dtype, sinks=True, sink_scale=2.0)
    dout = _dout(5100, x["q"].shape, dtype)
    y = dict(x)
    y["q"], y["k"], y["v"] = x["q"].clone(), x["k"].clone(), x["v"].clone()
    dpad = dout.clone()
    for b in range(B):
        y["q"][b, :, sq[b]:] = float("nan")
        dpad[b, :, sq[b]:] = float("nan")
        y["k"][b, :, sk[b]:] = float("nan")
        y["v"][b, :, sk[b]:] = float("nan")
    (dq, dk, dv, ds), sc = _run(y, dpad, dtype, True, sq, sk, want_dsinks=True)
    (rq, rk, rv, rs), mags = _reference(x["q"], x["k"], x["v"], dout, scale=sc, causal=True,
                                             sinks=x["sinks"], seqlens_q=np.array(sq), seqlens_k=np.array(sk))
    _check_all([(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv"), (ds, rs, "dsinks")], dtype, mags)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_backward_seqlens_keys_end_early(dtype):
    """Per-batch key lengths that end several 256-key blocks before Lk, under
    causal masking: those key blocks have no query tile at all while their
    first visible query tile lies past the batch's queries, and must load
    nothing.  D = 104 leaves chunks past the real head dim in every row."""
    B, Hq, Hkv, Lq, Lk, D = 3, 8, 2, 200, 1100, 104
    sq, sk = [200, 66, 133], [1100, 962, 404]
    x = random_case(5150, B, Hq, Hkv, Lq, Lk, D, dtype, sinks=True, sink_scale=2.0)
    dout = _dout(5150, x["q"].shape, dtype)
    (dq, dk, dv, ds), sc = _run(x, dout, dtype, True, sq, sk, want_dsinks=True)
    (rq, rk, rv, rs), mags = _reference(x["q"], x["k"], x["v"], dout, scale=sc, causal=True,
                                             sinks=x["sinks"], seqlens_q=np.array(sq), seqlens_k=np.array(sk))
    _check_all([(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv"), (ds, rs, "dsinks")], dtype, mags)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("G", [4, 8])
def test_backward_gqa_head_groups(dtype, G):
    """GQA with several 256-key dK / dV blocks and a ragged key tail: the
    blocks are split over query-head groups (each group's dK, dV in fp32,
    summed by a reduction pass), so every key row sums the groups of every
    head of its KV head."""
    B, Hkv, L, D = 1, 2, 1100, 128
    Hq = G * Hkv
    x = random_case(5250 + G, B, Hq, Hkv, L, L, D, dtype, sinks=True, sink_scale=2.0)
    dout = _dout(5250 + G, x["q"].shape, dtype)
    (dq, dk, dv, ds), sc = _run(x, dout, dtype, True, None, None, want_dsinks=True)
    (rq, rk, rv, rs), mags = _reference(x["q"], x["k"], x["v"], dout, scale=sc, causal=True,
                                             sinks=x["sinks"])
    _check_all([(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv"), (ds, rs, "dsinks")], dtype, mags)


def test_autograd_wrapper_matches_entry_point():
    x = to_dev(random_case(5200, 2, 4, 2, 150, 150, 64, "bf16", sinks=True))
    q, k, v = (x[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    s = x["sinks"].clone().requires_grad_(True)
    o = sdpa.attention(q, k, v, causal=True, sinks=s)
    dout = _dout(5200, o.shape, "bf16").cuda()
    o.backward(dout)
    o2, lse = sdpa.prefill(x["q"], x["k"], x["v"], causal=True, sinks=x["sinks"], return_lse=True)
    dq, dk, dv, ds = sdpa.prefill_backward(x["q"], x["k"], x["v"], o2, lse, dout, causal=True,
                                           sinks=x["sinks"], want_dsinks=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for a, b_ in ((q.grad, dq), (k.grad, dk), (v.grad, dv), (s.grad, ds)):
        assert torch.equal(a, b_)


def test_backward_rejects_unsupported():
    x = to_dev(random_case(5300, 1, 2, 2, 8, 8, 136, "fp16"))   # head dim above 128
    o, lse = sdpa.prefill(x["q"], x["k"], x["v"], return_lse=True)
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.prefill_backward(x["q"], x["k"], x["v"], o, lse, o)
    assert e.value.status == sdpa.Status.ERR_UNSUPPORTED


@pytest.mark.timeout(600)
def test_causal_full_size_sampled_heads():
    """The causal bf16 workload (B1 H32 L4096 D128) at full size, in the launch
    configuration bench.py times; heads 0 and 31 (independent problems, one KV
    head each) against the oracle, every element of dQ, dK, dV."""
    import workloads
    w = workloads.CAUSAL_BWD
    say("backward full size", w)
    x = workloads.make_inputs(w)
    d = to_dev(x)
    o, lse = sdpa.prefill(d["q"], d["k"], d["v"], scale=w.scale, causal=True, return_lse=True)
    dq, dk, dv = sdpa.prefill_backward(d["q"], d["k"], d["v"], o, lse, d["dout"], scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for h in (0, 31):
        sl = slice(h, h + 1)
        (rq, rk, rv, _), mags = _reference(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["dout"][:, sl],
                                                scale=w.scale, causal=True)
        _check_all([(dq[:, sl], rq, f"dq head {h}"), (dk[:, sl], rk, f"dk head {h}"),
                    (dv[:, sl], rv, f"dv head {h}")], "bf16", mags)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_backward_bool_mask(dtype):
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 200, 190, 128
    x = random_case(5400, B, Hq, Hkv, Lq, Lk, D, dtype, sinks=True, sink_scale=2.0)
    keep = np.random.default_rng(5400).random((B, Hq, Lq, Lk)) < 0.7
    keep[0, 1, 7, :] = False
    x["mask"] = torch.from_numpy(keep)
    dout = _dout(5400, x["q"].shape, dtype)
    (dq, dk, dv, ds), sc = _run(x, dout, dtype, True, want_dsinks=True)
    (rq, rk, rv, rs), mags = _reference(x["q"], x["k"], x["v"], dout, scale=sc, causal=True,
                                             mask=x["mask"], sinks=x["sinks"])
    _check_all([(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv"), (ds, rs, "dsinks")], dtype, mags)
