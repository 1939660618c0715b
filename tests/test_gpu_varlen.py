"""GPU parity of per-batch lengths (the padding mask of the cuDNN SDPA graph:
seq_len_q / seq_len_kv) and of fixed-capacity KV caches, for prefill and
decode, against the fp64 oracle.  Padding rows and keys hold NaN on the
device, so any read of them into a result shows up as a mismatch."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_prefill_amd as sdpa
from tests.gpu_util import compare_full, say, to_dev
from workloads import random_case

pytestmark = pytest.mark.gpu


def _poison(x, sq, sk):
    """Copy of the inputs with NaN in every padding row of q and key of k, v."""
    y = dict(x)
    y["q"], y["k"], y["v"] = x["q"].clone(), x["k"].clone(), x["v"].clone()
    for b in range(len(sq)):
        y["q"][b, :, sq[b]:] = float("nan")
        y["k"][b, :, sk[b]:] = float("nan")
        y["v"][b, :, sk[b]:] = float("nan")
    return y


# (Hq, Hkv, Lq, Lk, seqlens_q, seqlens_k, causal, mask, sinks)
PREFILL_CASES = [
    (4, 2, 300, 333, [300, 129, 0], [333, 200, 3], True, False, False),
    (4, 2, 300, 333, [300, 129, 64], [333, 200, 1], False, False, True),
    (2, 1, 260, 257, [260, 100, 7], [130, 257, 0], True, False, True),   # rows without keys
    (3, 3, 129, 190, [129, 1, 65], [190, 64, 65], False, True, False),
    (2, 2, 70, 70, [70, 33, 64], [70, 70, 64], True, True, True),
]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_seqlens(dtype, D, case):
    Hq, Hkv, Lq, Lk, sq, sk, causal, mask, sinks = PREFILL_CASES[case]
    say(f"prefill seqlens {dtype} D={D} case={PREFILL_CASES[case]}")
    x = random_case(4000 + 10 * case + D, 3, Hq, Hkv, Lq, Lk, D, dtype, mask=mask, sinks=sinks,
                    sink_scale=2.0, mask_neg_inf_frac=0.1)
    d = to_dev(_poison(x, sq, sk))
    sc = 1.0 / math.sqrt(D)
    out, lse = sdpa.prefill(d["q"], d["k"], d["v"], scale=sc, causal=causal, mask=d["mask"],
                            sinks=d["sinks"], return_lse=True, seqlens_q=sq, seqlens_k=sk)
    torch.cuda.synchronize()
    compare_full(out, lse, x, sc, dtype, f"seqlens{case}-{dtype}-D{D}", causal=causal,
                 seqlens_q=np.array(sq), seqlens_k=np.array(sk))
    if dtype == "fp16":   # no log-sum-exp requested: the pre-scaled-Q kernels
        out = sdpa.prefill(d["q"], d["k"], d["v"], scale=sc, causal=causal, mask=d["mask"],
                           sinks=d["sinks"], seqlens_q=sq, seqlens_k=sk)
        torch.cuda.synchronize()
        compare_full(out, None, x, sc, dtype, f"seqlens{case}-{dtype}-D{D} O only", causal=causal,
                     seqlens_q=np.array(sq), seqlens_k=np.array(sk))


def test_prefill_full_lengths_equal_no_lengths():
    x = to_dev(random_case(4100, 2, 4, 2, 200, 300, 128, "bf16"))
    a = sdpa.prefill(x["q"], x["k"], x["v"], causal=True)
    b = sdpa.prefill(x["q"], x["k"], x["v"], causal=True, seqlens_q=[200, 900], seqlens_k=[300, 300])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# (Hq, Hkv, Lq, Lk, D, seqlens_q, seqlens_k, causal, sinks)
DECODE_CASES = [
    (8, 2, 1, 5000, 128, [1, 1, 1], [5000, 1234, 0], False, False),
    (8, 2, 1, 5000, 128, [1, 0, 1], [4097, 4096, 17], False, True),
    (32, 4, 1, 3000, 512, [1, 1, 1], [3000, 1, 1500], False, True),
    (8, 2, 4, 2000, 128, [4, 2, 4], [2000, 999, 3], True, False),
    (32, 4, 4, 1024, 512, [4, 1, 3], [1024, 700, 0], True, True),
]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_seqlens(dtype, case):
    Hq, Hkv, Lq, Lk, D, sq, sk, causal, sinks = DECODE_CASES[case]
    say(f"decode seqlens {dtype} case={DECODE_CASES[case]}")
    x = random_case(4200 + case, 3, Hq, Hkv, Lq, Lk, D, dtype, sinks=sinks, sink_scale=2.0)
    d = to_dev(_poison(x, sq, sk))
    sc = 1.0 / math.sqrt(D)
    for ns in (0, 1, 7):
        out, lse = sdpa.decode(d["q"], d["k"], d["v"], scale=sc, causal=causal, sinks=d["sinks"],
                               return_lse=True, num_splits=ns, seqlens_q=sq, seqlens_k=sk)
        torch.cuda.synchronize()
        compare_full(out, lse, x, sc, dtype, f"decode seqlens{case}-{dtype} splits={ns}",
                     causal=causal, seqlens_q=np.array(sq), seqlens_k=np.array(sk))


def test_decode_whole_cache_equals_slices():
    """A fixed-capacity cache passed whole with fill levels gives, per batch,
    the result of the sliced cache."""
    B, Hq, Hkv, T, D = 3, 16, 2, 4096, 128
    fill = [4096, 1000, 2500]
    x = to_dev(random_case(4300, B, Hq, Hkv, 1, T, D, "bf16", sinks=True))
    whole = sdpa.decode(x["q"], x["k"], x["v"], sinks=x["sinks"], seqlens_k=fill)
    for b in range(B):
        part = sdpa.decode(x["q"][b:b + 1], x["k"][b:b + 1, :, :fill[b]], x["v"][b:b + 1, :, :fill[b]],
                           sinks=x["sinks"])
        torch.cuda.synchronize()
        err = (whole[b:b + 1].float() - part.float()).abs().max().item()
        say(f"  batch {b} fill {fill[b]}: max diff {err:.3e}")
        assert err <= 2e-3


@pytest.mark.timeout(600)
def test_kvcache_ragged_full_size():
    """The ragged KV-cache decode workload at full size (B8 Hq32 Hkv8 D128, a
    131072-slot cache per (batch, KV head) with per-batch fill levels), every
    output row against the oracle, in the launch configuration bench.py times."""
    import workloads
    w = workloads.KVCACHE_DECODE
    say("decode full size", w, "fill", list(w.seqlens_k()))
    x = workloads.make_inputs(w)
    d = to_dev(x)
    out, lse = sdpa.decode(d["q"], d["k"], d["v"], scale=w.scale, return_lse=True,
                           seqlens_k=d["seqlens_k"])
    torch.cuda.synchronize()
    compare_full(out, lse, x, w.scale, w.dtype, w.name, seqlens_k=w.seqlens_k())
