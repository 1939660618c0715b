"""sdpa_decode_noalloc (split partials in the library's static per-GPU
scratch) against sdpa_decode (caller workspace) through the C ABI: the same
kernels and split plan, so the outputs must be identical, and both within the
oracle's parity gates.  Two calls in a row, the second with a smaller input,
so the second reads nothing the first left in the scratch."""
import math

import pytest
import torch

import scaled_dot_product_prefill_amd as sdpa
from tests.gpu_util import compare_full, say, to_dev
from workloads import random_case

pytestmark = pytest.mark.gpu


def _both(x, num_splits, causal=False):
    d = to_dev(x)
    D = x["q"].shape[-1]
    sc = 1 / math.sqrt(D)
    ns = sdpa.decode_num_splits(d["q"], d["k"], d["v"], num_splits=num_splits)
    need = sdpa.decode_workspace_bytes(d["q"], d["k"], d["v"], num_splits=num_splits)
    assert 0 < need <= sdpa.DECODE_SCRATCH_BYTES
    a, la = sdpa.decode(d["q"], d["k"], d["v"], scale=sc, causal=causal, mask=d["mask"], sinks=d["sinks"],
                        return_lse=True, num_splits=num_splits)
    b, lb = sdpa.decode_noalloc(d["q"], d["k"], d["v"], scale=sc, causal=causal, mask=d["mask"],
                                sinks=d["sinks"], return_lse=True, num_splits=num_splits)
    torch.cuda.synchronize()
    say(f"  splits {ns}, partials {need} bytes")
    assert torch.equal(a, b) and torch.equal(la, lb)
    compare_full(b, lb, x, sc, {torch.float16: "fp16", torch.bfloat16: "bf16", torch.float32: "fp32"}[x["q"].dtype],
                 f"noalloc splits={ns}", causal=causal)


def test_noalloc_matches_workspace_decode_twice():
    # first call: a large request (long keys, mask, sinks, GQA-4, bf16)
    say("noalloc call 1")
    x1 = random_case(4100, 4, 32, 8, 1, 20000, 128, "bf16", mask=True, sinks=True,
                     mask_shape=(4, 1, 1, 20000), mask_neg_inf_frac=0.05)
    _both(x1, 0)
    # second call: smaller, fewer splits, another dtype and head dim
    say("noalloc call 2")
    x2 = random_case(4101, 1, 8, 2, 1, 3000, 64, "fp16", sinks=True)
    _both(x2, 5)


def test_noalloc_multi_query_and_single_pass():
    x = random_case(4102, 2, 16, 2, 4, 2500, 512, "fp16", sinks=True)
    _both(x, 7, causal=True)
    d = to_dev(x)
    a = sdpa.decode(d["q"], d["k"], d["v"], causal=True, sinks=d["sinks"], num_splits=1)
    b = sdpa.decode_noalloc(d["q"], d["k"], d["v"], causal=True, sinks=d["sinks"], num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_noalloc_rejects_oversize():
    x = to_dev(random_case(4103, 8, 32, 8, 1, 8192, 128, "bf16"))
    assert sdpa.decode_workspace_bytes(x["q"], x["k"], x["v"], num_splits=128) > sdpa.DECODE_SCRATCH_BYTES
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.decode_noalloc(x["q"], x["k"], x["v"], num_splits=128)
    assert e.value.status == sdpa.Status.ERR_WORKSPACE
