"""The elementwise error scale of the gradient tests (tests/grad_bound.py),
checked on the CPU: every magnitude companion bounds its oracle reference; a
simulated 16-bit kernel (the oracle's gradients with the roundings a bf16
kernel makes: O, P and dS rounded to bf16, results stored in bf16) stays
within the gate the GPU tests use; and plausible mistakes in a kernel (D_i
dropped from dS, the scale dropped from dK, P.V summed over the wrong key
range) exceed it by far."""
import numpy as np
import torch

from oracle import sdpa_backward_reference
from oracle.attention import sdpa_reference
from tests.grad_bound import grad_magnitudes
from workloads import random_case

U_BF16 = 2.0 ** -8
C_BF16 = 2.0  # the gate of test_gpu_backward for bf16


def _bf(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _ratio(got, ref, mag):
    excess = np.abs(got - ref) - U_BF16 * np.abs(ref)
    nz = mag > 0
    assert np.all(excess[~nz] <= 0)
    return float(np.max(excess[nz] / (U_BF16 * mag[nz])))


def _kernel_like(x, dout, scale, lq, lk, mistake=None):
    """dQ, dK, dV of one head (H = 1) the way a bf16 kernel rounds them."""
    Q, K, V = (x[n][0, 0].double().numpy() for n in ("q", "k", "v"))
    dO = dout[0, 0].double().numpy()
    O, L = sdpa_reference(x["q"], x["k"], x["v"], scale=scale, causal=True, sinks=x["sinks"])
    O, L = O[0, 0], L[0, 0]
    S = scale * Q @ K.T
    S = np.where(np.arange(lk)[None, :] > np.arange(lq)[:, None] + (lk - lq), -np.inf, S)
    P = np.exp(S - L[:, None])
    Di = np.sum(dO * _bf(O), axis=1)
    if mistake == "no_D":
        Di = 0 * Di
    dS = _bf(P * (dO @ V.T - Di[:, None]))
    ks = 1.0 if mistake == "no_scale_dk" else scale
    dq, dk = _bf(scale * dS @ K), _bf(ks * dS.T @ Q)
    Pb = _bf(P)
    if mistake == "keys_shifted":
        Pb = np.roll(Pb, 1, axis=1)
    return dq, dk, _bf(Pb.T @ dO)


def test_companions_bound_and_gate():
    lq, lk, D = 48, 80, 32
    x = random_case(7100, 1, 1, 1, lq, lk, D, "bf16", sinks=True, sink_scale=2.0)
    dout = torch.from_numpy(np.random.default_rng(7100).standard_normal((1, 1, lq, D)).astype(np.float32))
    dout = dout.to(torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    kw = dict(scale=scale, causal=True, sinks=x["sinks"])
    refs = sdpa_backward_reference(x["q"], x["k"], x["v"], dout, **kw)[:3]
    mags = grad_magnitudes(x["q"], x["k"], x["v"], dout, **kw)
    for r, m in zip(refs, mags):
        assert np.all(np.abs(r) <= m * (1 + 1e-12))
    refs = [r[0, 0] for r in refs]
    mags = [m[0, 0] for m in mags]
    good = _kernel_like(x, dout, scale, lq, lk)
    worst = max(_ratio(g, r, m) for g, r, m in zip(good, refs, mags))
    assert worst <= C_BF16, worst
    for mistake, which in (("no_D", 0), ("no_scale_dk", 1), ("keys_shifted", 2)):
        bad = _kernel_like(x, dout, scale, lq, lk, mistake)
        assert _ratio(bad[which], refs[which], mags[which]) > 10 * C_BF16, mistake


def test_floor_covers_fp16_subnormal_rounding():
    # with floor > 0 every element with a visible pair gets at least that much
    lq, lk, D = 16, 24, 16
    x = random_case(7101, 1, 1, 1, lq, lk, D, "fp16")
    dout = torch.zeros(1, 1, lq, D, dtype=torch.float16)
    kw = dict(scale=0.25, causal=False)
    a0 = grad_magnitudes(x["q"], x["k"], x["v"], dout, **kw)
    a1 = grad_magnitudes(x["q"], x["k"], x["v"], dout, floor=2.0 ** -14, **kw)
    for m0, m1 in zip(a0, a1):
        assert np.all(m0 == 0)           # dO = 0: no gradient, no magnitude
    assert np.all(a1[0] > 0) and np.all(a1[1] > 0)   # rounded dS entries may be nonzero
    assert np.all(a1[2] == 0)                          # dV = P^T dO stays 0 with dO = 0
