"""Seeded random configurations through all three entry points (prefill,
decode, gradients) against the fp64 oracles: every combination the fixed
grids do not pin down by hand -- odd head counts and group sizes, head dims
that are any multiple of 8 with Dv != D, ragged lengths around the tile
sizes, additive or boolean masks with hidden entries, sinks, per-batch
lengths and split counts -- drawn from one generator so that each run checks
the same cases.  Sizes stay small enough for the oracle to finish in
seconds."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_prefill_amd as sdpa
from oracle import allclose_report, sdpa_backward_reference
from tests.gpu_util import compare_full, say, to_dev
from workloads import DTYPES, random_case

pytestmark = pytest.mark.gpu

N_PREFILL, N_DECODE, N_BACKWARD = 48, 32, 32


def _draw(seed, decode=False, backward=False):
    r = np.random.default_rng([7, seed, decode, backward])
    dtype = ["fp32", "fp16", "bf16"][int(r.integers(3))]
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 8]))
    B = int(r.integers(1, 4))
    hmax = 128 if backward else 512
    D = 8 * int(r.integers(1, hmax // 8 + 1))
    Dv = D if r.random() < 0.6 else 8 * int(r.integers(1, hmax // 8 + 1))
    Lq = int(r.integers(1, 17)) if decode else int(r.choice([1, 31, 64, 65, 127, 129, 200, 257]))
    Lk = int(r.choice([1, 7, 63, 64, 65, 300, 513, 1100]))
    causal = bool(r.random() < 0.5)
    mask = ["none", "add", "bool"][int(r.integers(3))]
    sinks = bool(r.random() < 0.5)
    lens = bool(r.random() < 0.4)
    sq = [int(r.integers(0, Lq + 1)) for _ in range(B)] if lens else None
    sk = [int(r.integers(0, Lk + 1)) for _ in range(B)] if lens else None
    if sq is not None:
        sq[0], sk[0] = Lq, Lk   # one full batch
    return dict(dtype=dtype, B=B, Hq=Hkv * G, Hkv=Hkv, Lq=Lq, Lk=Lk, D=D, Dv=Dv, causal=causal, mask=mask,
                sinks=sinks, sq=sq, sk=sk, splits=int(r.choice([0, 0, 1, 3])))


def _inputs(seed, c):
    x = random_case(9100 + seed, c["B"], c["Hq"], c["Hkv"], c["Lq"], c["Lk"], c["D"], c["dtype"],
                    mask=c["mask"] == "add", sinks=c["sinks"], sink_scale=2.0, mask_neg_inf_frac=0.1,
                    mask_shape=(c["B"], 1, c["Lq"], c["Lk"]), Dv=c["Dv"])
    if c["mask"] == "bool":
        keep = np.random.default_rng([8, seed]).random((c["B"], c["Hq"], c["Lq"], c["Lk"])) < 0.8
        x["mask"] = torch.from_numpy(keep)
    return x


def _lens(c):
    return dict(seqlens_q=None if c["sq"] is None else np.array(c["sq"]),
                seqlens_k=None if c["sk"] is None else np.array(c["sk"]))


@pytest.mark.parametrize("seed", range(N_PREFILL))
def test_random_prefill(seed):
    c = _draw(seed)
    say(f"random prefill {seed}: {c}")
    x = _inputs(seed, c)
    d = to_dev(x)
    sc = 1.0 / math.sqrt(c["D"])
    # odd seeds ask for no log-sum-exp (fp16 then runs the pre-scaled-Q kernels)
    want_lse = seed % 2 == 0
    r = sdpa.prefill(d["q"], d["k"], d["v"], scale=sc, causal=c["causal"], mask=d["mask"],
                     sinks=d["sinks"], return_lse=want_lse, seqlens_q=c["sq"], seqlens_k=c["sk"])
    out, lse = r if want_lse else (r, None)
    torch.cuda.synchronize()
    compare_full(out, lse, x, sc, c["dtype"], f"random prefill {seed}", causal=c["causal"], **_lens(c))


@pytest.mark.parametrize("seed", range(N_DECODE))
def test_random_decode(seed):
    c = _draw(seed, decode=True)
    say(f"random decode {seed}: {c}")
    x = _inputs(seed, c)
    d = to_dev(x)
    sc = 1.0 / math.sqrt(c["D"])
    out, lse = sdpa.decode(d["q"], d["k"], d["v"], scale=sc, causal=c["causal"], mask=d["mask"],
                           sinks=d["sinks"], return_lse=True, num_splits=min(c["splits"], c["Lk"]),
                           seqlens_q=c["sq"], seqlens_k=c["sk"])
    torch.cuda.synchronize()
    compare_full(out, lse, x, sc, c["dtype"], f"random decode {seed}", causal=c["causal"], **_lens(c))


@pytest.mark.parametrize("seed", range(N_BACKWARD))
def test_random_backward(seed):
    c = _draw(seed, backward=True)
    say(f"random backward {seed}: {c}")
    x = _inputs(seed, c)
    d = to_dev(x)
    sc = 1.0 / math.sqrt(c["D"])
    g = np.random.default_rng([9, seed]).standard_normal((c["B"], c["Hq"], c["Lq"], c["Dv"]), dtype=np.float32)
    dout = torch.from_numpy(g).to(DTYPES[c["dtype"]])
    o, lse = sdpa.prefill(d["q"], d["k"], d["v"], scale=sc, causal=c["causal"], mask=d["mask"], sinks=d["sinks"],
                          return_lse=True, seqlens_q=c["sq"], seqlens_k=c["sk"])
    res = sdpa.prefill_backward(d["q"], d["k"], d["v"], o, lse, dout.cuda(), scale=sc, causal=c["causal"],
                                mask=d["mask"], sinks=d["sinks"], seqlens_q=c["sq"], seqlens_k=c["sk"],
                                want_dsinks=c["sinks"])
    torch.cuda.synchronize()
    ref = sdpa_backward_reference(x["q"], x["k"], x["v"], dout, scale=sc, causal=c["causal"], mask=x["mask"],
                                  sinks=x["sinks"], **_lens(c))
    names = ("dq", "dk", "dv", "dsinks")
    fp32 = c["dtype"] == "fp32"
    bad = []
    for got, want, name in zip(res, ref, names):
        if want is None:
            continue
        want = np.asarray(want, dtype=np.float64)
        s = max(1.0, float(np.abs(want).max()) if want.size else 1.0)
        atol, rtol, nrel = (1e-5, 0.0, 1e-5) if fp32 else (2e-3, 1e-2, 1e-2)
        rep = allclose_report(got.float().cpu().numpy(), want, atol * s, rtol)
        ok = rep["ok"] and rep["norm_rel"] <= nrel
        say(f"  {name}: max_abs={rep['max_abs']:.3e} (scale {s:.3g}) norm_rel={rep['norm_rel']:.3e} ok={ok}")
        if not ok:
            bad.append((name, rep))
    assert not bad, bad
