"""GPU parity of the decode kernels (sdpa_decode through the C ABI: single-pass,
and two-pass split-K + merge) against the fp64 oracle: the whole GQA-8 D=512
grid (Lk 1k/8k/32k, B 1/2, fp16/bf16/fp32, with and without sinks), the
long-context masked batch at full size, edge cases (fully masked splits,
all keys masked, KV-cache slices, every head dim and group size) and
multi-query decode (Lq <= 16, causal within the block)."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_prefill_amd as sdpa
import workloads
from tests.gpu_util import check, compare_full, say, to_dev
from workloads import random_case

pytestmark = pytest.mark.gpu


def _decode(d, scale, num_splits):
    out, l = sdpa.decode(d["q"], d["k"], d["v"], scale=scale, mask=d["mask"], sinks=d["sinks"],
                         return_lse=True, num_splits=num_splits)
    torch.cuda.synchronize()
    return out, l


@pytest.mark.timeout(300)
@pytest.mark.parametrize("w", workloads.GQA_DECODE, ids=lambda w: w.name)
def test_gqa8_d512_grid(w):
    say("decode", w)
    x = workloads.make_inputs(w)
    d = to_dev(x)
    ns = sdpa.decode_num_splits(d["q"], d["k"], d["v"])
    for num_splits in (0, 1):
        out, l = _decode(d, w.scale, num_splits)
        compare_full(out, l, x, w.scale, w.dtype, f"{w.name} splits={num_splits}->"
                     f"{ns if num_splits == 0 else 1}")


@pytest.mark.timeout(900)
def test_long_context_masked_full_size():
    w = workloads.LONG_DECODE
    say("decode full size", w)
    x = workloads.make_inputs(w)
    d = to_dev(x)
    ns = sdpa.decode_num_splits(d["q"], d["k"], d["v"])
    say(f"  auto splits: {ns}")
    out, l = _decode(d, w.scale, 0)
    compare_full(out, l, x, w.scale, w.dtype, f"{w.name} auto")
    # 64 splits of 2048 keys: the last 6 splits see only -inf keys
    out2, l2 = _decode(d, w.scale, 64)
    compare_full(out2, l2, x, w.scale, w.dtype, f"{w.name} 64 splits")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_head_dims_and_groups(dtype, D, G):
    Hkv = 2
    x = random_case(3000 + D + G, 2, Hkv * G, Hkv, 1, 777, D, dtype, sinks=(G == 4))
    d = to_dev(x)
    sc = 1 / math.sqrt(D)
    for ns in (0, 1, 5):
        out, l = _decode(d, sc, ns)
        compare_full(out, l, x, sc, dtype, f"D{D} G{G} splits={ns}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fully_masked_splits_and_rows(dtype):
    B, Hq, Hkv, Lk, D = 2, 8, 2, 1000, 128
    x = random_case(3100, B, Hq, Hkv, 1, Lk, D, dtype, mask=True, mask_shape=(B, 1, 1, Lk))
    x["mask"][..., 600:] = -math.inf                  # trailing splits fully masked
    x["mask"][1] = -math.inf                          # batch 1 sees no key at all
    d = to_dev(x)
    sc = 1 / math.sqrt(D)
    for ns in (1, 4, 10, 0):
        out, l = _decode(d, sc, ns)
        assert torch.all(out[1] == 0) and torch.all(torch.isneginf(l[1]))
        compare_full(out, l, x, sc, dtype, f"masked splits={ns}")
    # with sinks the empty batch gets O = 0 and LSE = sink
    x["sinks"] = torch.linspace(-2, 2, Hq)
    d = to_dev(x)
    for ns in (1, 7):
        out, l = _decode(d, sc, ns)
        compare_full(out, l, x, sc, dtype, f"masked+sinks splits={ns}")


def test_kv_cache_slice():
    # K / V are the first Lk rows of a larger cache (row stride Lk_max * D per head)
    B, Hq, Hkv, Lmax, Lk, D = 2, 16, 2, 4096, 3000, 128
    x = random_case(3200, B, Hq, Hkv, 1, Lmax, D, "bf16")
    d = to_dev(x)
    k, v = d["k"][:, :, :Lk], d["v"][:, :, :Lk]
    assert not k.is_contiguous()
    out, l = sdpa.decode(d["q"], k, v, return_lse=True)
    torch.cuda.synchronize()
    xs = dict(x, k=x["k"][:, :, :Lk], v=x["v"][:, :, :Lk])
    compare_full(out, l, xs, 1 / math.sqrt(D), "bf16", "kv-cache slice")


def test_single_pass_matches_two_pass_and_prefill():
    x = to_dev(random_case(3300, 1, 32, 4, 1, 4096, 128, "fp16", sinks=True))
    a = sdpa.decode(x["q"], x["k"], x["v"], sinks=x["sinks"], num_splits=1)
    b = sdpa.decode(x["q"], x["k"], x["v"], sinks=x["sinks"], num_splits=16)
    c = sdpa.prefill(x["q"], x["k"], x["v"], sinks=x["sinks"])
    torch.cuda.synchronize()
    for name, y in (("two-pass", b), ("prefill", c)):
        err = (a.float() - y.float()).abs().max().item()
        say(f"  single-pass vs {name}: {err:.3e}")
        assert err <= 2e-3


def test_decode_errors():
    x = to_dev(random_case(3400, 1, 4, 2, 17, 64, 128, "fp16"))
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.decode(x["q"], x["k"], x["v"])                # Lq = 17 > 16
    assert e.value.status == sdpa.Status.ERR_UNSUPPORTED
    x = to_dev(random_case(3401, 1, 4, 2, 1, 64, 520, "fp16"))
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.decode(x["q"], x["k"], x["v"])                # D = 520 > 512
    assert e.value.status == sdpa.Status.ERR_UNSUPPORTED


# Multi-query decode (Lq query rows per head, speculative / chunked decoding):
# the rows and the G heads of a KV head are the columns of 16-column matrix
# tiles, 16, 32 or 64 columns per workgroup (Lq * G of 16, 32, 51 and 64
# below); causal is bottom-right within the block.
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("Lq,G", [(2, 8), (4, 8), (8, 8), (8, 4), (16, 1), (3, 17)])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_query(dtype, Lq, G, causal):
    Hkv, D, Lk = 2, (512 if G == 8 else 128), 1500
    x = random_case(3500 + 17 * Lq + G, 2, Hkv * G, Hkv, Lq, Lk, D, dtype, mask=True,
                    mask_neg_inf_frac=0.05, sinks=(Lq == 4))
    d = to_dev(x)
    sc = 1 / math.sqrt(D)
    for ns in (0, 1, 7):
        out, l = sdpa.decode(d["q"], d["k"], d["v"], scale=sc, causal=causal, mask=d["mask"],
                             sinks=d["sinks"], return_lse=True, num_splits=ns)
        torch.cuda.synchronize()
        compare_full(out, l, x, sc, dtype, f"Lq{Lq} G{G} causal={causal} splits={ns}", causal=causal)


def test_multi_query_more_rows_than_keys():
    # causal with Lq > Lk: the first Lq - Lk rows see no key (O = 0, LSE = -inf,
    # or LSE = sink when sinks are given)
    for sinks in (False, True):
        x = random_case(3600 + sinks, 1, 8, 2, 12, 5, 128, "bf16", sinks=sinks)
        d = to_dev(x)
        for ns in (1, 3):
            out, l = sdpa.decode(d["q"], d["k"], d["v"], causal=True, sinks=d["sinks"],
                                 return_lse=True, num_splits=ns)
            torch.cuda.synchronize()
            assert torch.all(out[:, :, :7] == 0)
            compare_full(out, l, x, 1 / math.sqrt(128), "bf16", f"Lq>Lk sinks={sinks} splits={ns}",
                         causal=True)


def test_multi_query_matches_prefill():
    x = to_dev(random_case(3700, 2, 32, 4, 8, 4096, 128, "fp16", sinks=True))
    a = sdpa.decode(x["q"], x["k"], x["v"], causal=True, sinks=x["sinks"])
    c = sdpa.prefill(x["q"], x["k"], x["v"], causal=True, sinks=x["sinks"])
    torch.cuda.synchronize()
    err = (a.float() - c.float()).abs().max().item()
    say(f"  multi-query decode vs prefill: {err:.3e}")
    assert err <= 2e-3


@pytest.mark.timeout(600)
def test_multi_query_full_size():
    # the bench workload (4 causal query rows, GQA-8 D512, Lk 32768) in the
    # launch configuration bench.py times (automatic splits), all heads
    w = workloads.MQ_DECODE
    say("multi-query decode full size", w)
    x = workloads.make_inputs(w)
    d = to_dev(x)
    out, l = sdpa.decode(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, return_lse=True)
    torch.cuda.synchronize()
    compare_full(out, l, x, w.scale, w.dtype, f"{w.name} auto", causal=w.causal)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_bool_mask(dtype, num_splits):
    """Boolean [B,1,1,Lk] mask (the trailing tenth hidden, plus scattered
    holes) through the single-pass and split-K decode kernels."""
    B, Hq, Hkv, Lk, D = 2, 16, 2, 3000, 128
    x = random_case(2400, B, Hq, Hkv, 1, Lk, D, dtype, sinks=True)
    keep = np.random.default_rng(2400).random((B, 1, 1, Lk)) < 0.9
    keep[..., Lk - Lk // 10:] = False
    x["mask"] = torch.from_numpy(keep)
    d = to_dev(x)
    out, l = _decode(d, 1 / math.sqrt(D), num_splits)
    compare_full(out, l, x, 1 / math.sqrt(D), dtype, f"decode bool mask splits={num_splits}")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("dims", [(8, 8), (80, 80), (96, 64), (192, 128), (320, 320), (512, 448)],
                         ids=lambda d: f"{d[0]}x{d[1]}")
def test_head_dims(dtype, dims):
    """Head dims that are multiples of 8 (D_v may differ from D_qk), single
    pass and split-K."""
    D, Dv = dims
    x = random_case(2600 + D + Dv, 2, 16, 4, 1, 1500, D, dtype, Dv=Dv, sinks=True)
    d = to_dev(x)
    for ns in (0, 1):
        out, l = _decode(d, 1 / math.sqrt(D), ns)
        assert out.shape[-1] == Dv
        compare_full(out, l, x, 1 / math.sqrt(D), dtype, f"decode head dims {D}x{Dv} splits={ns}")
