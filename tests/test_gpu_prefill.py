"""GPU parity of the prefill kernel (sdpa_prefill through the C ABI) against the
fp64 oracle: the tiny, DiT and causal workloads at full size (every row of
every head),
a grid of small cases spanning several tiles with ragged tails, and the
edge cases of the method (empty rows, fully masked rows, sinks, GQA,
non-contiguous layouts, one key)."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_prefill_amd as sdpa
import workloads
from tests.gpu_util import check, compare_full, compare_sampled, say, to_dev
from workloads import random_case

pytestmark = pytest.mark.gpu


def _run(x, dtype_name, causal=False, scale=None, lse=True):
    """One prefill call; with lse=False the call itself asks for no
    log-sum-exp (fp16 then takes the pre-scaled-Q kernels)."""
    d = to_dev(x)
    D = x["q"].shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    r = sdpa.prefill(d["q"], d["k"], d["v"], scale=scale, causal=causal, mask=d["mask"],
                     sinks=d["sinks"], return_lse=lse)
    out, l = r if lse else (r, None)
    torch.cuda.synchronize()
    return out, l, scale


def test_tiny_fp32_full():
    w = workloads.TINY
    say("tiny fp32", w)
    x = workloads.make_inputs(w)
    out, l, sc = _run(x, w.dtype)
    compare_full(out, l, x, sc, w.dtype, w.name)


# (B, Hq, Hkv, Lq, Lk, D, sinks): 128-row tile counts just past a multiple of
# 256, so that the workspace form runs the last tiles as two key pieces each
# and merges them (4 or 8 tail tiles, ragged last pieces and rows)
TAIL = [
    (1, 65, 65, 512, 512, 64, False),     # 260 tiles, pieces of 256 keys
    (1, 65, 13, 500, 700, 128, True),     # GQA-5, sinks, pieces of 384 and 316 keys
    (2, 33, 33, 512, 300, 64, True),      # 264 tiles, pieces of 192 and 108 keys
    (1, 130, 130, 256, 4250, 64, False),  # pieces of 2176 and 2074 keys
]


@pytest.mark.parametrize("dtype,lse", [("fp16", False), ("fp16", True), ("bf16", True)])
@pytest.mark.parametrize("case", range(len(TAIL)))
def test_prefill_tail_pieces(dtype, lse, case):
    B, Hq, Hkv, Lq, Lk, D, sinks = TAIL[case]
    say(f"prefill tail pieces {dtype} lse={lse} case={TAIL[case]}")
    x = random_case(5000 + 10 * case, B, Hq, Hkv, Lq, Lk, D, dtype, sinks=sinks, sink_scale=2.0)
    d = to_dev(x)
    sc = 1.0 / math.sqrt(D)
    assert sdpa.prefill_workspace_bytes(d["q"], d["k"], d["v"]) > 0  # the split applies
    runs = []
    for split in (True, True, False):
        r = sdpa.prefill(d["q"], d["k"], d["v"], scale=sc, sinks=d["sinks"], return_lse=lse, split_tail=split)
        runs.append(r if lse else (r, None))
    torch.cuda.synchronize()
    out, l = runs[0]
    compare_full(out, l, x, sc, dtype, f"tail{case}-{dtype}-lse{int(lse)}")
    # no atomics: the same call gives the same bits
    assert torch.equal(runs[0][0], runs[1][0])
    # and the one-pass form agrees within the gates: each piece rounds its
    # probabilities against its own running max (bf16: 8 bits), so the row
    # sums, and the LSE, differ in their last bits
    torch.testing.assert_close(out.float(), runs[2][0].float(), atol=2e-3, rtol=1e-2)
    if lse:
        torch.testing.assert_close(l, runs[2][1], atol=1e-3, rtol=0)


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
def test_prefill_grid(dtype, D, case):
    B, Hq, Hkv, Lq, Lk, causal, mask, sinks = GRID[case]
    say(f"prefill grid {dtype} D={D} case={GRID[case]}")
    x = random_case(1000 + 10 * case + D, B, Hq, Hkv, Lq, Lk, D, dtype, mask=mask, sinks=sinks,
                    sink_scale=2.0, mask_neg_inf_frac=0.1)
    out, l, sc = _run(x, dtype, causal=causal)
    compare_full(out, l, x, sc, dtype, f"grid{case}-{dtype}-D{D}", causal=causal)
    if dtype == "fp16":   # no log-sum-exp requested: the pre-scaled-Q kernels
        out, _, sc = _run(x, dtype, causal=causal, lse=False)
        compare_full(out, None, x, sc, dtype, f"grid{case}-{dtype}-D{D} O only", causal=causal)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", range(len(GRID)))
def test_prefill_grid_d256(dtype, case):
    # head dim 256: 16-bit inputs only
    B, Hq, Hkv, Lq, Lk, causal, mask, sinks = GRID[case]
    say(f"prefill grid {dtype} D=256 case={GRID[case]}")
    x = random_case(3000 + 10 * case, B, Hq, Hkv, Lq, Lk, 256, dtype, mask=mask, sinks=sinks,
                    sink_scale=2.0, mask_neg_inf_frac=0.1)
    out, l, sc = _run(x, dtype, causal=causal)
    compare_full(out, l, x, sc, dtype, f"grid{case}-{dtype}-D256", causal=causal)
    if dtype == "fp16":
        out, _, sc = _run(x, dtype, causal=causal, lse=False)
        compare_full(out, None, x, sc, dtype, f"grid{case}-{dtype}-D256 O only", causal=causal)


def test_d256_long_causal_sampled():
    # head dim 256 over 32 key tiles: steady state, rescales, ragged causal edge
    w = workloads.CAUSAL.with_(name="causal_bf16_d256", B=1, Hq=4, Hkv=2, Lq=2048, Lk=2048, D=256)
    _full_size(w, heads=[(0, 0), (0, 3)], rows=[0, 1, 63, 64, 127, 128, 1000, 2047])


def _full_size(w, heads, rows):
    say("full size", w)
    x = workloads.make_inputs(w)
    out, l, sc = _run(x, w.dtype, causal=w.causal)
    compare_sampled(out, l, x, sc, w.dtype, w.name, heads, rows, causal=w.causal)


def _full_size_every_row(w):
    """The workload at its full size, in the launch configuration the
    benchmark times (log-sum-exp output only where the workload asks for
    it), compared with the oracle on every row of every head."""
    say("full size, every row", w)
    x = workloads.make_inputs(w)
    out, l, sc = _run(x, w.dtype, causal=w.causal, lse=w.lse)
    compare_full(out, l, x, sc, w.dtype, w.name, causal=w.causal)


@pytest.mark.timeout(600)
def test_dit_fp16_full_size():
    _full_size_every_row(workloads.DIT_FP16)


@pytest.mark.timeout(600)
def test_dit_fp32_full_size():
    _full_size_every_row(workloads.DIT_FP32)


@pytest.mark.timeout(600)
def test_causal_bf16_full_size():
    _full_size_every_row(workloads.CAUSAL)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_one_key_and_one_query(dtype):
    x = random_case(2001, 1, 2, 2, 1, 1, 64, dtype, sinks=True)
    out, l, sc = _run(x, dtype)
    compare_full(out, l, x, sc, dtype, "Lq=Lk=1")
    x = random_case(2002, 1, 2, 1, 70, 1, 128, dtype)
    out, l, sc = _run(x, dtype, causal=True)          # Lq > Lk: only the last row sees the key
    compare_full(out, l, x, sc, dtype, "Lk=1 causal", causal=True)


@pytest.mark.parametrize("dtype", ["fp32", "fp16"])
def test_fully_masked_rows(dtype):
    x = random_case(2003, 1, 2, 2, 130, 90, 64, dtype, mask=True)
    x["mask"][:, :, 5] = -math.inf                    # row 5 sees nothing
    x["mask"][:, :, 100:] = -math.inf                 # rows 100.. see nothing
    out, l, sc = _run(x, dtype)
    assert torch.all(out[:, :, 5] == 0) and torch.all(out[:, :, 100:] == 0)
    assert torch.all(torch.isneginf(l[:, :, 5]))
    compare_full(out, l, x, sc, dtype, "masked rows")
    # with sinks: O = 0 and LSE = sink on the empty rows
    x["sinks"] = torch.tensor([0.5, -1.25])
    out, l, sc = _run(x, dtype)
    compare_full(out, l, x, sc, dtype, "masked rows + sinks")


def test_large_sinks_and_scale():
    x = random_case(2004, 2, 4, 2, 150, 200, 128, "bf16", sinks=True, sink_scale=10.0)
    out, l, sc = _run(x, "bf16", causal=True, scale=0.3)
    compare_full(out, l, x, sc, "bf16", "10x sinks", causal=True)


@pytest.mark.parametrize("dtype", ["fp32", "fp16"])
def test_dominant_logit_and_identical_keys(dtype):
    x = random_case(2005, 1, 1, 1, 40, 300, 64, dtype)
    k = x["k"].float()
    k[0, 0, 77] = 4.0 * x["q"][0, 0, 3].float()       # key 77 dominates query 3
    k[0, 0, 200:] = k[0, 0, 200]                      # identical tail keys
    x["k"] = k.to(x["q"].dtype)
    out, l, sc = _run(x, dtype)
    compare_full(out, l, x, sc, dtype, "dominant/identical")
    # without the log-sum-exp (fp16: Q pre-multiplied by the exponent scale);
    # the dominant score is 4 |q_3|^2 / 8, about 32
    out, _, sc = _run(x, dtype, lse=False)
    compare_full(out, None, x, sc, dtype, "dominant/identical, O only")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_running_max_moves(dtype, D):
    # a score offset that grows along the keys (a shared direction in q and
    # k) moves the reference max past the rescale slack again and again
    # inside the steady loop, while tens of keys still share each row
    x = random_case(2010 + D, 1, 2, 2, 256, 1024, D, dtype)
    q, k = x["q"].float(), x["k"].float()
    q[..., 0] = 8.0
    k[..., 0] = torch.linspace(0.0, 25.0, 1024)
    x["q"], x["k"] = q.to(x["v"].dtype), k.to(x["v"].dtype)
    out, l, sc = _run(x, dtype)
    compare_full(out, l, x, sc, dtype, f"moving max {dtype} D{D}")
    out, _, sc = _run(x, dtype, lse=False)
    compare_full(out, None, x, sc, dtype, f"moving max {dtype} D{D} O only")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("jump", [10.0, 30.0, 200.0])
def test_fp16_score_jump_inside_the_steady_tiles(causal, D, jump):
    # Without a log-sum-exp, fp16 takes the steady tiles without a row max
    # and checks each tile's row sum afterwards.  Key 150 (a steady tile of
    # every workgroup, causal or not) is made to lift the score of query 300
    # by `jump` nats over its first tile's maximum; along that direction it
    # also moves the other rows' scores by up to several times as much, either
    # way.  Rows whose tile sum passes 2^14 but stays finite move the
    # reference max in the fast pass; rows whose probabilities overflow fp16
    # (or, at 200, fp32's exponential) send their workgroup through the
    # tiles again with the max taken first.
    x = random_case(2020 + D, 1, 2, 2, 640, 640, D, "fp16")
    q, k = x["q"].float(), x["k"].float()
    i, j = 300, 150
    qn = q[0, 0, i] / q[0, 0, i].norm()
    # score(i, j) = scale q_i . k_j = jump + (a typical first-tile maximum)
    target = jump + 3.0
    k[0, 0, j] = qn * target * math.sqrt(D) / q[0, 0, i].norm()
    x["k"] = k.half()
    x["q"] = q.half()
    out, _, sc = _run(x, "fp16", causal=causal, lse=False)
    compare_full(out, None, x, sc, "fp16", f"score jump {jump} D{D} causal={causal}", causal=causal)


@pytest.mark.parametrize("causal", [False, True])
def test_fp16_scale_above_one_log2_unit(causal):
    # |scale| log2(e) > 1: Q is not pre-multiplied and every tile takes the
    # general path
    x = random_case(2012, 1, 2, 2, 200, 700, 64, "fp16")
    x["q"] = (x["q"].float() * 0.25).half()
    out, l, sc = _run(x, "fp16", causal=causal, scale=1.5)
    compare_full(out, l, x, sc, "fp16", f"scale 1.5 causal={causal}", causal=causal)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("tail", [1, 31, 33, 64, 65, 96, 97])
def test_tail_workgroup_waves(dtype, tail):
    # the last 128-row workgroup of each head holds `tail` real rows, so 0 to 3
    # of its 32-row waves hold none (they still stream K / V with the others)
    Lq = 256 + tail
    x = random_case(2100 + tail, 2, 2, 1, Lq, 300, 64, dtype, sinks=True)
    out, l, sc = _run(x, dtype, causal=tail % 2 == 1)
    compare_full(out, l, x, sc, dtype, f"tail {tail}", causal=tail % 2 == 1)
    out, _, sc = _run(x, dtype, causal=tail % 2 == 1, lse=False)
    compare_full(out, None, x, sc, dtype, f"tail {tail} O only", causal=tail % 2 == 1)


def test_non_contiguous_layouts():
    # q, k, v, o stored as [B, L, H, D] and viewed as [B, H, L, D]
    B, H, L, D = 2, 4, 150, 128
    g = torch.Generator().manual_seed(7)
    mk = lambda: torch.randn(B, L, H, D, generator=g).to(torch.bfloat16)
    qs, ks, vs = mk(), mk(), mk()
    x = {"q": qs.transpose(1, 2), "k": ks.transpose(1, 2), "v": vs.transpose(1, 2),
         "mask": None, "sinks": None}
    dq, dk, dv = (t.cuda().transpose(1, 2) for t in (qs, ks, vs))
    o_store = torch.empty(B, L, H, D, dtype=torch.bfloat16, device="cuda")
    out = sdpa.prefill(dq, dk, dv, causal=True, out=o_store.transpose(1, 2))
    torch.cuda.synchronize()
    compare_full(o_store.transpose(1, 2), None, x, 1 / math.sqrt(D), "bf16", "strided", causal=True)


def test_deterministic():
    x = to_dev(random_case(2006, 2, 4, 4, 333, 333, 128, "fp16"))
    a = sdpa.prefill(x["q"], x["k"], x["v"], causal=True)
    b = sdpa.prefill(x["q"], x["k"], x["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gqa_equals_repeated_kv():
    x = to_dev(random_case(2007, 1, 8, 2, 200, 260, 64, "bf16"))
    a = sdpa.prefill(x["q"], x["k"], x["v"], causal=True)
    b = sdpa.prefill(x["q"], x["k"].repeat_interleave(4, 1), x["v"].repeat_interleave(4, 1), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_rejects_unsupported():
    for dt in ("fp16", "fp32"):
        x = to_dev(random_case(2008, 1, 2, 2, 8, 8, 520, dt))   # D = 520 > 512
        with pytest.raises(sdpa.SdpaError) as e:
            sdpa.prefill(x["q"], x["k"], x["v"])
        assert e.value.status == sdpa.Status.ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bool_mask(dtype, causal):
    """Boolean mask (one byte per entry, True = the key takes part), broadcast
    over heads, with rows whose keys are all hidden."""
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 150, 211, 128 if dtype != "fp32" else 64
    x = random_case(2300 + causal, B, Hq, Hkv, Lq, Lk, D, dtype, sinks=causal, sink_scale=2.0)
    keep = np.random.default_rng(2300).random((B, 1, Lq, Lk)) < 0.7
    keep[0, 0, 5, :] = False
    keep[1, 0, 100:110, :] = False
    x["mask"] = torch.from_numpy(keep)
    out, l, sc = _run(x, dtype, causal=causal)
    compare_full(out, l, x, sc, dtype, f"bool mask {dtype} causal={causal}", causal=causal)


# (D, Dv): head dims that are multiples of 8, run in the next kernel size up
HEAD_DIMS = [(8, 8), (40, 40), (80, 80), (96, 96), (112, 64), (64, 120), (128, 96)]
HEAD_DIMS_16 = [(160, 160), (192, 128), (256, 200)]
# kernel head dim 512 (and 256 in fp32): 16 columns per workgroup
HEAD_DIMS_WIDE = [(512, 512), (264, 512), (512, 320), (136, 136)]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("dims", HEAD_DIMS + HEAD_DIMS_16 + HEAD_DIMS_WIDE, ids=lambda d: f"{d[0]}x{d[1]}")
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims(dtype, dims, causal):
    D, Dv = dims
    say(f"prefill head dims {dtype} D={D} Dv={Dv} causal={causal}")
    x = random_case(2500 + D + Dv, 2, 4, 2, 150, 211, D, dtype, Dv=Dv, sinks=causal, sink_scale=2.0)
    out, l, sc = _run(x, dtype, causal=causal)
    assert out.shape[-1] == Dv
    compare_full(out, l, x, sc, dtype, f"head dims {D}x{Dv}", causal=causal)


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_d512_gqa_causal_sampled(dtype):
    """Head dim 512 with GQA-8 (the decode workload's heads) over 2048 causal
    rows: 16 columns = 2 query rows x 8 heads per workgroup; LSE and sinks."""
    w = workloads.CAUSAL.with_(name=f"causal_{dtype}_d512", B=1, Hq=16, Hkv=2, Lq=2048, Lk=2048, D=512,
                               dtype=dtype, sinks=True)
    _full_size(w, heads=[(0, 0), (0, 7), (0, 8), (0, 15)], rows=[0, 1, 2, 15, 16, 1000, 2046, 2047])



@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("mask", [False, True])
def test_d512_eight_wave_workgroups_sampled(dtype, mask):
    """Head dim 512 with a grid large enough for the 128-column (eight-wave)
    workgroups: B=8, GQA-8 over 1024 causal rows; additive mask with -inf
    entries broadcast over heads, and sinks."""
    B, Hq, Hkv, Lq, Lk, D = 8, 16, 2, 1024, 1100, 512
    x = random_case(2700 + mask, B, Hq, Hkv, Lq, Lk, D, dtype, mask=mask, sinks=True,
                    mask_neg_inf_frac=0.05, mask_shape=(B, 1, Lq, Lk))
    say(f"prefill d512 eight-wave {dtype} mask={mask}")
    out, l, sc = _run(x, dtype, causal=True)
    compare_sampled(out, l, x, sc, dtype, f"d512 w8 {dtype} mask={mask}",
                    [(0, 0), (3, 9), (7, 15)], [0, 1, 127, 128, 500, 1023], causal=True)


def test_binding_rejects_bad_buffers():
    # caller-supplied outputs, LSE and workspaces that the kernels could not
    # write safely are refused in the binding, before any launch
    say("binding: bad out / lse / workspace buffers")
    dev = torch.device("cuda")
    B, H, L, D = 1, 2, 64, 64
    q, k, v = (torch.randn(B, H, L, D, device=dev).half() for _ in range(3))
    bad_outs = [torch.empty(B, H, L, D, dtype=torch.float16),                     # host memory
                torch.empty(B, H, L, D, dtype=torch.bfloat16, device=dev),        # dtype
                torch.empty(B, H, L + 1, D, dtype=torch.float16, device=dev),     # shape
                torch.empty(B, H, L, D + 1, dtype=torch.float16, device=dev)[..., :D]]  # 130-byte rows
    for o in bad_outs:
        with pytest.raises(ValueError):
            sdpa.prefill(q, k, v, out=o)
        with pytest.raises(ValueError):
            sdpa.decode(q[:, :, :1], k, v, out=o[:, :, :1] if o.shape[2] == L else o)
    qd = q[:, :, :1].contiguous()
    with pytest.raises(ValueError):
        sdpa.decode(qd, k, v, num_splits=4, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        sdpa.decode(qd, k, v, num_splits=4,
                    workspace=torch.empty(2, 1 << 20, dtype=torch.uint8, device=dev)[:, ::2])
    with pytest.raises(ValueError):
        sdpa.decode_noalloc(qd, k, v, return_lse=True,
                            lse=torch.empty(B, 2 * H, 1, device=dev)[:, ::2])
    with pytest.raises(ValueError):
        sdpa.prefill(q, k.cpu().cuda(), v.cpu(), causal=True)
    o, lse = sdpa.prefill(q, k, v, causal=True, return_lse=True)
    with pytest.raises(ValueError):
        sdpa.prefill_backward(q, k, v, o, lse.cpu(), torch.randn_like(o), causal=True)
    with pytest.raises(ValueError):
        sdpa.prefill_backward(q, k, v, o.cpu(), lse, torch.randn_like(o), causal=True)
    torch.cuda.synchronize()
