"""The work counts behind bench.py's roofline figures, checked on the CPU:
visible (query, key) pairs against a brute-force count of the bottom-right
causal rule, flops and bytes per launch of the benchmarked shapes against
their closed forms, the one-GPU guard, and that traffic figures taken on other
kernel sources are not reported."""
import subprocess
import sys

import pytest

import bench
import workloads


def _brute_pairs(Lq, Lk, causal):
    # key j is visible to query i iff j <= i + (Lk - Lq) under causal masking
    return sum(1 for i in range(Lq) for j in range(Lk) if not causal or j <= i + Lk - Lq)


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (1, 7), (7, 1), (5, 5), (3, 11), (11, 3), (64, 65), (130, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_brute_force(Lq, Lk, causal):
    assert bench.visible_pairs(Lq, Lk, causal) == _brute_pairs(Lq, Lk, causal)


def test_visible_pairs_square_causal_is_triangle():
    assert bench.visible_pairs(4096, 4096, True) == 4096 * 4097 // 2


def test_prefill_flops_of_benchmarked_shapes():
    # DiT: 4 * D * Lq * Lk * B * H, every pair visible
    assert bench.prefill_flops(workloads.DIT_FP16) == 4 * 64 * 4250 * 4250 * 2 * 38 == 351_424_000_000
    # causal L4096 D128 H32: the lower triangle with its diagonal only
    assert bench.prefill_flops(workloads.CAUSAL) == 4 * 128 * (4096 * 4097 // 2) * 32 == 137_472_507_904
    # gradients: 10 * D per visible pair (2.5x the forward)
    assert bench.backward_flops(workloads.CAUSAL_BWD) == 137_472_507_904 * 5 // 2


def test_decode_bytes_of_benchmarked_shapes():
    # long decode: K + V (4 GiB bf16) + fp32 mask [8, 131072] + Q and O (bf16)
    kv = 2 * 8 * 8 * 131072 * 128 * 2
    assert kv == 4 << 30
    assert bench.decode_bytes(workloads.LONG_DECODE) == kv + 4 * 8 * 131072 + 2 * 8 * 32 * 128 * 2 == 4_299_292_672
    # GQA-8 D512 B2 Lk32k fp16: K + V once per (batch, KV head), no mask
    w = workloads.ALL["gqa8_decode_b2_lk32768_fp16"]
    assert bench.decode_bytes(w) == 2 * 2 * 32768 * 4 * 512 * 2 + 2 * 2 * 32 * 512 * 2
    # ragged cache: only the filled keys of each batch count
    kc = workloads.KVCACHE_DECODE
    fill = [int(x) for x in kc.seqlens_k()]
    assert bench.decode_bytes(kc) == 2 * sum(fill) * 8 * 128 * 2 + 2 * 8 * 32 * 128 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_from_other_sources_is_not_reported(monkeypatch):
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.load_traffic("prefill_dit_fp16") is None
    assert bench.load_traffic("no_such_kernel") is None


def test_drift_ratio():
    # first 7 steps at 1.0 ms, last 8 at 1.1 ms: a 10 % slow-down across the run
    assert bench.drift([1.0] * 7 + [1.1] * 8) == pytest.approx(1.1)
    assert bench.drift([2.0] * 30) == 1.0
    assert bench.drift([1.0] * 14) is None


def test_settle_stops_when_chunks_agree():
    seq = iter([[2.0], [1.5], [1.2], [1.1], [1.1], [1.1]])
    r = bench.settle(None, lambda: next(seq), min_s=0.0, max_s=10.0)
    assert r["settled"] and r["chunks"] == 5


def test_settle_gives_up_at_its_limit():
    vals = iter((1.0, 1.1)[x % 2] for x in range(10 ** 9))   # 10 % apart, never settles
    r = bench.settle(None, lambda: [next(vals)], min_s=0.0, max_s=0.05)
    assert r["settled"] is False and r["chunks"] >= 2


def test_settle_disabled():
    assert bench.settle(None, lambda: 1 / 0, min_s=0.0, max_s=0.0)["chunks"] == 0


def test_cpu_oracle_one_thread():
    r = bench.cpu_oracle_1thread()
    assert set(r) == {"tiny_fp32", "gqa8_decode_b1_lk1024_fp16"}
    for v in r.values():
        assert v["cores"] == 1 and v["value"] > 0 and v["kind"] == "oracle"
    assert bench.cpu_model()
