"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
HIP library through its binding, compare with the fp64 oracle."""
import sys

import numpy as np
import torch

from oracle import allclose_report, sdpa_reference

# elementwise |gpu - ref| <= atol + rtol * |ref|
TOL = {"fp32": (1e-5, 0.0), "fp16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
# normwise ||gpu - ref||_2 / ||ref||_2 over the finite entries.  With N(0,1)
# inputs a long key range makes |O| small (about sqrt(e / Lk)), so the
# elementwise atol alone would accept an output that lost a whole block of
# keys; the normwise bound does not.
NORM_REL = {"fp32": 1e-5, "fp16": 1e-2, "bf16": 1e-2}
# log-sum-exp: absolute error bound in natural-log units, every dtype (the
# fp32 elementwise bound above is tighter still)
LSE_MAX_ABS = 1e-3
DT_NAME = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}
# elementwise against each output element's magnitude companion
# A_i = sum_j P_ij |V_j| (the oracle's output for |V| in place of V: the same
# weights, P >= 0), the scale of the rounding of P, the row sum and the
# scores a kernel makes:  |gpu - ref| <= C u A + u |ref| (+ 2^-25 for fp16,
# whose results below 2^-14 are stored with a fixed step of 2^-24), u the
# unit roundoff of the input type.  A small element of an output with a
# large maximum gets its own scale.  Computed where the oracle's extra pass
# is cheap (at most MAG_PAIRS_MAX query-key pairs, or sampled rows).
# C, measured worst over the GPU tests: bf16 0.32; fp16 1.3, and 8.5 in the
# tests with scores up to 200 (the fp16 kernels multiply Q by the scale in
# fp16, which moves each score by up to about u |S|); fp32 39.
UNIT = {"fp32": 2.0 ** -24, "fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
C_ELEM = {"fp32": 160.0, "fp16": 32.0, "bf16": 2.0}
OUT_FLOOR = {"fp32": 0.0, "fp16": 2.0 ** -25, "bf16": 0.0}
MAG_PAIRS_MAX = 1 << 26


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return {k: (v.cuda() if v is not None else None) for k, v in x.items()}


def elem_gate(got, ref, mag, dtype_name):
    """The magnitude-companion gate: (passed, worst ratio of the rounding
    excess to u A).  Elements with A = 0 must match to the stored rounding."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    a = np.asarray(mag, dtype=np.float64)
    fin = np.isfinite(r) & np.isfinite(a)
    u = UNIT[dtype_name]
    excess = np.abs(g[fin] - r[fin]) - u * np.abs(r[fin]) - OUT_FLOOR[dtype_name]
    pos = a[fin] > 0
    ratio = float(np.max(excess[pos] / (u * a[fin][pos]))) if pos.any() else 0.0
    zero_ok = bool(np.all(excess[~pos] <= 0)) if (~pos).any() else True
    return ratio <= C_ELEM[dtype_name] and zero_ok and bool(np.all(np.isfinite(g[fin]))), ratio


def gate(got, ref, dtype_name, lse=False, mag=None):
    """All parity gates for one output tensor: elementwise allclose, normwise
    relative error, for a log-sum-exp output the absolute bound, and with a
    magnitude companion `mag` the elementwise gate scaled by it.
    Returns (passed, report)."""
    atol, rtol = TOL[dtype_name]
    rep = allclose_report(got, ref, atol, rtol)
    rep["norm_ok"] = rep["norm_rel"] <= NORM_REL[dtype_name]
    rep["lse_ok"] = (not lse) or rep["max_abs"] <= LSE_MAX_ABS
    rep["mag_ok"], rep["elem_ratio"] = elem_gate(got, ref, mag, dtype_name) if mag is not None else (True, None)
    return rep["ok"] and rep["norm_ok"] and rep["lse_ok"] and rep["mag_ok"], rep


def check(got, ref, dtype_name, what, lse=False, mag=None):
    ok, rep = gate(got, ref, dtype_name, lse=lse, mag=mag)
    er = "" if rep["elem_ratio"] is None else f" elem_ratio={rep['elem_ratio']:.3g}"
    say(f"  {what}{' lse' if lse else ''} [{dtype_name}]: max_abs={rep['max_abs']:.3e} "
        f"norm_rel={rep['norm_rel']:.3e}{er} elem_ok={rep['ok']} norm_ok={rep['norm_ok']} "
        f"lse_ok={rep['lse_ok']} mag_ok={rep['mag_ok']}")
    assert ok, f"{what}: {rep}"
    return rep


def _abs(t):
    return t.abs() if isinstance(t, torch.Tensor) else np.abs(t)


def compare_full(out, lse, x, scale, dtype_name, what, causal=False, **kw):
    O, L = sdpa_reference(x["q"], x["k"], x["v"], scale=scale, causal=causal,
                          mask=x["mask"], sinks=x["sinks"], **kw)
    B, Hq, Lq = x["q"].shape[:3]
    mag = None
    if B * Hq * Lq * x["k"].shape[2] <= MAG_PAIRS_MAX:
        mag, _ = sdpa_reference(x["q"], x["k"], _abs(x["v"]), scale=scale, causal=causal,
                                mask=x["mask"], sinks=x["sinks"], **kw)
    check(out.float().cpu(), O, dtype_name, what, mag=mag)
    if lse is not None:
        check(lse.cpu(), L, dtype_name, what, lse=True)


def compare_sampled(out, lse, x_cpu, scale, dtype_name, what, heads, rows, causal=False, **kw):
    """Compare selected (b, hq) pairs and query rows against the oracle."""
    O, L = sdpa_reference(x_cpu["q"], x_cpu["k"], x_cpu["v"], scale=scale, causal=causal,
                          mask=x_cpu["mask"], sinks=x_cpu["sinks"], rows=rows, heads=heads, **kw)
    mag, _ = sdpa_reference(x_cpu["q"], x_cpu["k"], _abs(x_cpu["v"]), scale=scale, causal=causal,
                            mask=x_cpu["mask"], sinks=x_cpu["sinks"], rows=rows, heads=heads, **kw)
    got = np.stack([out[b, h, rows].float().cpu().numpy() for b, h in heads])
    check(got, O, dtype_name, what, mag=mag)
    if lse is not None:
        gl = np.stack([lse[b, h, rows].cpu().numpy() for b, h in heads])
        check(gl, L, dtype_name, what, lse=True)
