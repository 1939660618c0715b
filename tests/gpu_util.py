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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return {k: (v.cuda() if v is not None else None) for k, v in x.items()}


def gate(got, ref, dtype_name, lse=False):
    """All parity gates for one output tensor: elementwise allclose, normwise
    relative error and, for a log-sum-exp output, the absolute bound.
    Returns (passed, report)."""
    atol, rtol = TOL[dtype_name]
    rep = allclose_report(got, ref, atol, rtol)
    rep["norm_ok"] = rep["norm_rel"] <= NORM_REL[dtype_name]
    rep["lse_ok"] = (not lse) or rep["max_abs"] <= LSE_MAX_ABS
    return rep["ok"] and rep["norm_ok"] and rep["lse_ok"], rep


def check(got, ref, dtype_name, what, lse=False):
    ok, rep = gate(got, ref, dtype_name, lse=lse)
    say(f"  {what}{' lse' if lse else ''}: max_abs={rep['max_abs']:.3e} "
        f"norm_rel={rep['norm_rel']:.3e} elem_ok={rep['ok']} norm_ok={rep['norm_ok']} "
        f"lse_ok={rep['lse_ok']}")
    assert ok, f"{what}: {rep}"
    return rep


def compare_full(out, lse, x, scale, dtype_name, what, causal=False, **kw):
    O, L = sdpa_reference(x["q"], x["k"], x["v"], scale=scale, causal=causal,
                          mask=x["mask"], sinks=x["sinks"], **kw)
    check(out.float().cpu(), O, dtype_name, what)
    if lse is not None:
        check(lse.cpu(), L, dtype_name, what, lse=True)


def compare_sampled(out, lse, x_cpu, scale, dtype_name, what, heads, rows, causal=False, **kw):
    """Compare selected (b, hq) pairs and query rows against the oracle."""
    O, L = sdpa_reference(x_cpu["q"], x_cpu["k"], x_cpu["v"], scale=scale, causal=causal,
                          mask=x_cpu["mask"], sinks=x_cpu["sinks"], rows=rows, heads=heads, **kw)
    got = np.stack([out[b, h, rows].float().cpu().numpy() for b, h in heads])
    check(got, O, dtype_name, what)
    if lse is not None:
        gl = np.stack([lse[b, h, rows].cpu().numpy() for b, h in heads])
        check(gl, L, dtype_name, what, lse=True)
