"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic.  It only draws the tensors that
both sides of every comparison (the fp64 oracle and the HIP path) consume, and
names the workload shapes.

Recipe (the same for every tensor):
  * each (batch b, head h) slice of tensor ``t`` (q=0, k=1, v=2) is drawn as
    iid N(0, 1) in float32 from ``numpy.random.default_rng([0, cfg, t, b, h])``
    with shape [L, D], so any slice can be regenerated on the host without
    copying device data back;
  * the float32 draw is rounded to nearest-even into the working dtype
    (float16 / bfloat16 / float32).  Both sides then see exactly the same
    representable values;
  * sinks (one logit per query head) are float32 N(0, 1) from
    ``default_rng([0, cfg, 3])`` (times ``sink_scale``);
  * the long-context decode mask is float32 [B, 1, 1, Lk]: 0 for the leading
    keys and -inf for the trailing floor(Lk / 10) keys of every batch;
  * ragged KV-cache fill levels (per-batch key counts) are uniform integers
    in [Lk / 8, Lk] from ``default_rng([0, cfg, 4])``;
  * the upstream gradient dO of a gradient workload is drawn like q with
    tensor id 5.

Seed 0 follows the reproducer script on the "Add D512 support to Metal vector
attention" page (its ``SEED``); the shapes follow the pages' workloads (the
SD3-style B=2, H=38, D=64 self-attention of the "Metal shaders for memory
efficient self attention on large sequences" page and the D=512, 32/4-head
decode cases of the D512 page's table).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np
import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_SINKS, TENSOR_FILL, TENSOR_DOUT = 0, 1, 2, 3, 4, 5

DTYPES = {
    "fp32": torch.float32,
    "fp16": torch.float16,
    "bf16": torch.bfloat16,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: sizes, dtype and which optional inputs it has."""

    name: str
    cfg_id: int          # seed component; distinct per workload family
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    dtype: str           # "fp32" | "fp16" | "bf16"
    causal: bool = False
    mask: Optional[str] = None     # None | "tail10" (decode mask, trailing 10 % of keys = -inf)
    sinks: bool = False
    sink_scale: float = 1.0
    lse: bool = False
    decode: bool = False           # run through sdpa_decode (always so when Lq == 1)
    fill: Optional[str] = None     # None | "ragged" (per-batch KV-cache fill levels)
    grad: bool = False             # time the gradients (sdpa_prefill_backward) instead

    @property
    def is_decode(self) -> bool:
        return self.decode or self.Lq == 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def seqlens_k(self) -> Optional[np.ndarray]:
        """Per-batch key counts (int32 [B]) of a ragged KV cache, else None."""
        if self.fill != "ragged":
            return None
        rng = np.random.default_rng([0, self.cfg_id, TENSOR_FILL])
        return rng.integers(self.Lk // 8, self.Lk + 1, size=self.B).astype(np.int32)


# The five workload families.  Sizes are the ones the pages measure on; the
# decode family is expanded over its Lk / B / dtype / sinks grid.
TINY = Workload("tiny_fp32", 1, B=1, Hq=2, Hkv=2, Lq=128, Lk=128, D=64, dtype="fp32")
DIT_FP16 = Workload("dit_fp16", 2, B=2, Hq=38, Hkv=38, Lq=4250, Lk=4250, D=64, dtype="fp16")
DIT_FP32 = DIT_FP16.with_(name="dit_fp32", dtype="fp32")
CAUSAL = Workload("causal_bf16", 3, B=1, Hq=32, Hkv=32, Lq=4096, Lk=4096, D=128,
                  dtype="bf16", causal=True, lse=True)
LONG_DECODE = Workload("long_decode_bf16", 5, B=8, Hq=32, Hkv=8, Lq=1, Lk=131072, D=128,
                       dtype="bf16", mask="tail10")


def gqa_decode(B: int, Lk: int, dtype: str, sinks: bool) -> Workload:
    return Workload(f"gqa8_decode_b{B}_lk{Lk}_{dtype}{'_sinks' if sinks else ''}", 4,
                    B=B, Hq=32, Hkv=4, Lq=1, Lk=Lk, D=512, dtype=dtype, sinks=sinks)


GQA_DECODE = [gqa_decode(B, Lk, dt, s)
              for Lk in (1024, 8192, 32768) for B in (1, 2)
              for dt in ("fp16", "bf16", "fp32") for s in (False, True)]

# Multi-query decode (next-row extension, not one of the five families): the
# GQA-8 D512 shape with a block of 4 query rows per head, causal within the
# block -- the qL4 control of the D512 page, i.e. speculative decoding.
MQ_DECODE = Workload("mq4_gqa8_decode_b1_lk32768_fp16", 6, B=1, Hq=32, Hkv=4, Lq=4, Lk=32768,
                     D=512, dtype="fp16", causal=True, decode=True)

# Ragged KV cache (next-row extension): the long-context decode shape as a
# fixed-capacity cache of 131072 slots per (batch, KV head) whose batches are
# filled to different levels (the padding mask of the cuDNN graph, with
# per-batch seq_len_kv).
KVCACHE_DECODE = Workload("kvcache_ragged_decode_bf16", 7, B=8, Hq=32, Hkv=8, Lq=1, Lk=131072,
                          D=128, dtype="bf16", fill="ragged")

# Gradients of the causal prefill (next-row extension): same inputs, plus dO.
CAUSAL_BWD = CAUSAL.with_(name="causal_bf16_bwd", grad=True)

# Prefill at head dim 512 (next-row extension): the GQA-8 D512 heads of the
# decode family over a 4096-token causal prompt.
PREFILL_D512 = CAUSAL.with_(name="causal_gqa8_d512_bf16", Hq=32, Hkv=4, D=512)

ALL: Dict[str, Workload] = {w.name: w for w in
                            [TINY, DIT_FP16, DIT_FP32, CAUSAL, LONG_DECODE, *GQA_DECODE, MQ_DECODE,
                             KVCACHE_DECODE, CAUSAL_BWD, PREFILL_D512]}


# ---- generators --------------------------------------------------------------

def _round_to(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 numpy -> torch tensor in ``dtype`` (round to nearest even)."""
    t = torch.from_numpy(x)
    return t if dtype == torch.float32 else t.to(dtype)


def slice_normal(cfg_id: int, tensor_id: int, b: int, h: int, L: int, D: int,
                 dtype: torch.dtype) -> torch.Tensor:
    """The [L, D] slice (b, h) of tensor ``tensor_id`` as a CPU tensor in ``dtype``."""
    rng = np.random.default_rng([0, cfg_id, tensor_id, b, h])
    return _round_to(rng.standard_normal((L, D), dtype=np.float32), dtype)


def tensor_normal(cfg_id: int, tensor_id: int, B: int, H: int, L: int, D: int,
                  dtype: torch.dtype, device="cpu") -> torch.Tensor:
    """Full [B, H, L, D] tensor assembled slice by slice (device optional)."""
    out = torch.empty((B, H, L, D), dtype=dtype, device=device)
    for b in range(B):
        for h in range(H):
            out[b, h].copy_(slice_normal(cfg_id, tensor_id, b, h, L, D, dtype))
    return out


def sinks_normal(cfg_id: int, Hq: int, scale: float = 1.0) -> torch.Tensor:
    rng = np.random.default_rng([0, cfg_id, TENSOR_SINKS])
    return torch.from_numpy((rng.standard_normal(Hq, dtype=np.float32) * np.float32(scale)))


def tail_mask(B: int, Lk: int) -> torch.Tensor:
    """[B, 1, 1, Lk] float32: 0 for keys j < Lk - floor(Lk/10), -inf after."""
    m = torch.zeros((B, 1, 1, Lk), dtype=torch.float32)
    m[..., Lk - Lk // 10:] = float("-inf")
    return m


def make_inputs(w: Workload, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of workload ``w``: q, k, v (dtype), mask and sinks (fp32) or None."""
    dt = w.torch_dtype
    q = tensor_normal(w.cfg_id, TENSOR_Q, w.B, w.Hq, w.Lq, w.D, dt, device)
    k = tensor_normal(w.cfg_id, TENSOR_K, w.B, w.Hkv, w.Lk, w.D, dt, device)
    v = tensor_normal(w.cfg_id, TENSOR_V, w.B, w.Hkv, w.Lk, w.D, dt, device)
    mask = tail_mask(w.B, w.Lk).to(device) if w.mask == "tail10" else None
    sinks = sinks_normal(w.cfg_id, w.Hq, w.sink_scale).to(device) if w.sinks else None
    out = {"q": q, "k": k, "v": v, "mask": mask, "sinks": sinks}
    fill = w.seqlens_k()
    if fill is not None:
        out["seqlens_k"] = torch.from_numpy(fill).to(device)
    if w.grad:
        out["dout"] = tensor_normal(w.cfg_id, TENSOR_DOUT, w.B, w.Hq, w.Lq, w.D, dt, device)
    return out


def random_case(seed: int, B: int, Hq: int, Hkv: int, Lq: int, Lk: int, D: int,
                dtype: str = "fp32", *, mask: bool = False, sinks: bool = False,
                sink_scale: float = 1.0, mask_neg_inf_frac: float = 0.0,
                mask_shape: Tuple[int, int, int, int] | None = None, Dv: Optional[int] = None
                ) -> Dict[str, Optional[torch.Tensor]]:
    """Small seeded case for tests: N(0,1) q/k/v (v with head dim Dv when
    given), optional N(0,1) additive mask (a fraction of entries set to -inf)
    and optional sinks."""
    rng = np.random.default_rng([1, seed])
    dt = DTYPES[dtype]
    q = _round_to(rng.standard_normal((B, Hq, Lq, D), dtype=np.float32), dt)
    k = _round_to(rng.standard_normal((B, Hkv, Lk, D), dtype=np.float32), dt)
    v = _round_to(rng.standard_normal((B, Hkv, Lk, Dv or D), dtype=np.float32), dt)
    m = None
    if mask:
        shp = mask_shape or (B, Hq, Lq, Lk)
        mm = rng.standard_normal(shp, dtype=np.float32)
        if mask_neg_inf_frac > 0:
            mm[rng.random(shp) < mask_neg_inf_frac] = -np.inf
        m = torch.from_numpy(mm)
    s = None
    if sinks:
        s = torch.from_numpy(rng.standard_normal(Hq, dtype=np.float32) * np.float32(sink_scale))
    return {"q": q, "k": k, "v": v, "mask": m, "sinks": s}
