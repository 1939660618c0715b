"""The parity gates can fail.  On the long-context decode shape (B=8, Hq=32,
Hkv=8, D=128, Lk=131072, trailing tenth of the keys masked, bf16), an output
that lost one 2048-key split of the 64 the decode kernel uses, or six, is
rejected, although the elementwise allclose bound alone accepts it (|O| is
about sqrt(e / Lk) = 0.0046 there, half of it below atol).  The "wrong"
outputs come from the oracle itself with those keys hidden, i.e. what a merge
that skipped a split would produce.  And the magnitude-companion gate rejects
a head of small values that lost keys, which the other two gates accept.
CPU only."""
import functools

import numpy as np
import torch

import workloads
from oracle import allclose_report, sdpa_reference
from tests.gpu_util import TOL, gate

W = workloads.LONG_DECODE
SPLIT = 2048        # keys per split at 64 splits


@functools.lru_cache(maxsize=1)
def _group(b=0, hk=0):
    """Inputs of one (batch, KV head) group of the long-decode workload."""
    G = W.Hq // W.Hkv
    dt = W.torch_dtype
    q = torch.stack([workloads.slice_normal(W.cfg_id, workloads.TENSOR_Q, b, hk * G + i, 1, W.D, dt)
                     for i in range(G)])[None]
    k = workloads.slice_normal(W.cfg_id, workloads.TENSOR_K, b, hk, W.Lk, W.D, dt)[None, None]
    v = workloads.slice_normal(W.cfg_id, workloads.TENSOR_V, b, hk, W.Lk, W.D, dt)[None, None]
    mask = workloads.tail_mask(1, W.Lk)
    return q, k, v, mask


def _bf16(x):
    """Round an fp64 result the way the kernel stores O (bf16)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _outputs(dropped_splits):
    q, k, v, mask = _group()
    O, L = sdpa_reference(q, k, v, scale=W.scale, mask=mask)
    m2 = mask.clone()
    for s in dropped_splits:
        m2[..., s * SPLIT:(s + 1) * SPLIT] = -np.inf
    Ob, Lb = sdpa_reference(q, k, v, scale=W.scale, mask=m2)
    return O, L, Ob, Lb


def test_correct_output_passes():
    O, L, _, _ = _outputs([])
    ok, rep = gate(_bf16(O), O, "bf16")
    assert ok, rep
    ok, rep = gate(L.astype(np.float32), L, "bf16", lse=True)
    assert ok, rep


def test_one_dropped_split_fails_the_gate():
    O, L, Ob, Lb = _outputs([10])
    atol, rtol = TOL["bf16"]
    assert allclose_report(_bf16(Ob), O, atol, rtol)["ok"]      # the elementwise bound alone accepts it
    ok, rep = gate(_bf16(Ob), O, "bf16")
    assert not ok and not rep["norm_ok"], rep
    assert rep["norm_rel"] > 0.05


def test_six_dropped_splits_fail_the_lse_gate():
    O, L, Ob, Lb = _outputs([3, 11, 20, 33, 40, 50])
    atol, rtol = TOL["bf16"]
    assert allclose_report(Lb, L, atol, rtol)["ok"]             # LSE within rtol * |LSE| alone
    ok, rep = gate(Lb, L, "bf16", lse=True)
    assert not ok and not rep["lse_ok"], rep



def test_companion_gate_scales_small_heads():
    """The magnitude-companion gate (|gpu - ref| <= C u A + u |ref|, A_i =
    sum_j P_ij |V_j|) gives each element its own scale: in a tensor whose
    second head has values 1000 times smaller, that head losing four of its
    64 keys passes the allclose bound and the normwise bound, and fails it."""
    g = torch.Generator().manual_seed(71)
    q, k, v = (torch.randn(1, 2, 64, 32, generator=g).to(torch.bfloat16) for _ in range(3))
    v[:, 1] = (v[:, 1].float() * 1e-3).to(torch.bfloat16)
    sc = 32 ** -0.5
    O, _ = sdpa_reference(q, k, v, scale=sc)
    A, _ = sdpa_reference(q, k, v.abs(), scale=sc)
    assert np.all(np.abs(O) <= A * (1 + 1e-12))
    ok, rep = gate(_bf16(O), O, "bf16", mag=A)
    assert ok and rep["mag_ok"], rep
    m = torch.zeros(1, 2, 64, 64)
    m[0, 1, :, 10:14] = -np.inf
    Ob, _ = sdpa_reference(q, k, v, scale=sc, mask=m)
    ok, rep = gate(_bf16(Ob), O, "bf16")
    assert ok, rep                                     # allclose and normwise accept it
    ok, rep = gate(_bf16(Ob), O, "bf16", mag=A)
    assert not ok and not rep["mag_ok"] and rep["elem_ratio"] > 5, rep
