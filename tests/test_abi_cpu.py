"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/*.h, the ctypes mirror of sdpa_args has the C layout, and
every validation error is reachable through the host-only *_check entry
points (no kernel is ever launched here)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import scaled_dot_product_prefill_amd as sdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sdpa.library_path):
        from scaled_dot_product_prefill_amd import build_lib
        build_lib.build()
    return sdpa.library()


def _declared_functions():
    names = []
    for fn in os.listdir(HEADER_DIR):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            names += re.findall(r"SDPA_API\s+[\w\s\*]+?\b(sdpa_\w+)\s*\(", text)
    return names


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 9, names
    out = subprocess.run(["nm", "-D", "--defined-only", sdpa.library_path],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert b"gfx950" in lib.sdpa_version()


def test_struct_layout_matches_c():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "sdpa_mi355x.h"
#define F(f) printf("%s %zu\n", #f, offsetof(sdpa_args, f));
int main(void) {
  printf("sizeof %zu\n", sizeof(sdpa_args));
  F(B) F(Hq) F(Hkv) F(Lq) F(Lk) F(D) F(dtype) F(causal) F(scale) F(mask_kind)
  F(q) F(q_stride) F(k) F(k_stride) F(v) F(v_stride) F(o) F(o_stride)
  F(mask) F(mask_stride) F(sinks) F(lse) F(seqlens_q) F(seqlens_k) F(Dv)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "layout.c")
        exe = os.path.join(td, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", HEADER_DIR, c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(l.split() for l in out.strip().splitlines())
    assert int(got.pop("sizeof")) == ctypes.sizeof(sdpa.SdpaArgs)
    for name, off in got.items():
        assert getattr(sdpa.SdpaArgs, name).offset == int(off), name


def _args(**kw):
    a = sdpa.SdpaArgs()
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.D = 2, 8, 2, 64, 64, 128
    a.dtype, a.causal, a.scale, a.mask_kind = sdpa.BF16, 0, 0.125, 0
    # fake, aligned, non-overlapping host addresses: validation never dereferences them
    base = 1 << 40
    for i, n in enumerate(("q", "k", "v", "o")):
        setattr(a, n, base + i * (1 << 32))
    for n, L, H in (("q", 64, 8), ("k", 64, 2), ("v", 64, 2), ("o", 64, 8)):
        st = getattr(a, n + "_stride")
        st[0], st[1], st[2] = H * L * 128, L * 128, 128
    for k, v in kw.items():
        if isinstance(v, tuple):
            arr = getattr(a, k)
            for i, x in enumerate(v):
                arr[i] = x
        else:
            setattr(a, k, v)
    return a


def _prefill(lib, **kw):
    return lib.sdpa_prefill_check(ctypes.byref(_args(**kw)))


def _decode(lib, num_splits=0, ws=1 << 44, ws_bytes=1 << 30, **kw):
    kw.setdefault("Lq", 1)
    a = _args(**kw)
    for n in ("q_stride", "o_stride"):
        st = getattr(a, n)
        st[0], st[1], st[2] = 8 * 128, 128, 128
    return lib.sdpa_decode_check(ctypes.byref(a), num_splits, ws, ws_bytes)


S = sdpa.Status


def test_prefill_validation(lib):
    assert _prefill(lib) == S.OK
    assert lib.sdpa_prefill_check(None) == S.ERR_NULL
    assert _prefill(lib, q=None) == S.ERR_NULL
    assert _prefill(lib, Lq=0) == S.ERR_SHAPE
    assert _prefill(lib, Hq=7) == S.ERR_SHAPE                 # not a multiple of Hkv
    assert _prefill(lib, D=96) == S.OK                          # runs in the D = 128 kernel
    assert _prefill(lib, D=100) == S.ERR_UNSUPPORTED            # not a multiple of 8
    assert _prefill(lib, Dv=64) == S.OK
    assert _prefill(lib, Dv=-8) == S.ERR_SHAPE
    assert _prefill(lib, D=64, Dv=136) == S.ERR_ARG             # o rows (stride 128) overlap
    assert _prefill(lib, dtype=sdpa.F32, D=136, q_stride=(8 * 64 * 136, 64 * 136, 136),
                    k_stride=(2 * 64 * 136, 64 * 136, 136), v_stride=(2 * 64 * 136, 64 * 136, 136),
                    o_stride=(8 * 64 * 136, 64 * 136, 136)) == S.OK   # 16-column kernel
    assert _prefill(lib, D=520, q_stride=(8 * 64 * 520, 64 * 520, 520),
                    k_stride=(2 * 64 * 520, 64 * 520, 520), v_stride=(2 * 64 * 520, 64 * 520, 520),
                    o_stride=(8 * 64 * 520, 64 * 520, 520)) == S.ERR_UNSUPPORTED   # above 512
    assert _prefill(lib, dtype=7) == S.ERR_UNSUPPORTED
    assert _prefill(lib, q=(1 << 40) + 8) == S.ERR_ALIGN
    assert _prefill(lib, k_stride=(2 * 64 * 128, 64 * 128, 100)) == S.ERR_ALIGN
    assert _prefill(lib, scale=float("nan")) == S.ERR_ARG
    assert _prefill(lib, scale=float("inf")) == S.ERR_ARG
    assert _prefill(lib, causal=2) == S.ERR_ARG
    assert _prefill(lib, mask_kind=2) == S.ERR_ARG
    assert _prefill(lib, mask=(1 << 45) + 1, mask_kind=1, mask_stride=(0, 0, 64, 1)) == S.OK   # bytes
    assert _prefill(lib, mask=(1 << 45) + 1, mask_kind=0, mask_stride=(0, 0, 64, 1)) == S.ERR_ALIGN
    assert _prefill(lib, o=(1 << 40) + 4096) == S.ERR_ARG     # o overlaps q
    assert _prefill(lib, mask=(1 << 45) + 2) == S.ERR_ALIGN
    assert _prefill(lib, mask=1 << 45, mask_stride=(0, 0, -1, 1)) == S.ERR_ARG
    assert _prefill(lib, lse=(1 << 40) + 16) == S.ERR_ARG     # lse overlaps q
    big = (1 << 22) + 8                                        # 8 MiB + 16 B per bf16 row
    assert _prefill(lib, k_stride=(2 * 64 * big, 64 * big, big)) == S.ERR_UNSUPPORTED
    assert _prefill(lib, v_stride=(2 * 64 * big, 64 * big, big)) == S.ERR_UNSUPPORTED
    assert _prefill(lib, seqlens_q=(1 << 46), seqlens_k=(1 << 46) + 64) == S.OK
    assert _prefill(lib, seqlens_k=(1 << 46) + 2) == S.ERR_ALIGN
    assert _prefill(lib, seqlens_q=(1 << 46) + 1) == S.ERR_ALIGN
    assert _prefill(lib, seqlens_k=(1 << 40) + 64) == S.OK             # inputs may overlap
    assert _prefill(lib, seqlens_k=(1 << 40) + 3 * (1 << 32) + 64) == S.ERR_ARG   # inside o
    assert _prefill(lib, D=64, causal=1, Lq=100, Lk=7) == S.OK

    msg = lib.sdpa_last_error()
    assert msg == b""
    _prefill(lib, D=100)
    assert b"multiples of 8" in lib.sdpa_last_error()


def test_decode_validation(lib):
    assert _decode(lib) == S.OK
    assert _decode(lib, Lq=17) == S.ERR_UNSUPPORTED           # multi-query decode: Lq <= 16
    assert _decode(lib, D=96) == S.OK
    assert _decode(lib, D=100) == S.ERR_UNSUPPORTED
    assert _decode(lib, num_splits=-1) == S.ERR_ARG
    assert _decode(lib, num_splits=65) == S.ERR_ARG           # more splits than keys
    assert _decode(lib, num_splits=4, ws=None) == S.ERR_WORKSPACE
    assert _decode(lib, num_splits=4, ws_bytes=16) == S.ERR_WORKSPACE
    assert _decode(lib, num_splits=4, ws=(1 << 44) + 4) == S.ERR_ALIGN
    assert _decode(lib, num_splits=1, ws=None, ws_bytes=0) == S.OK   # single pass needs none
    for st in range(8):
        assert lib.sdpa_status_string(st)


def _sizes(B, Hq, Hkv, Lk, D, dtype, Lq=1):
    a = sdpa.SdpaArgs()
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.D, a.dtype, a.scale = B, Hq, Hkv, Lq, Lk, D, dtype, 1.0
    return a


def test_split_plan(lib):
    # long-context batch: B*Hkv = 64 units start at 4 splits (256 workgroups)
    # and double until a split holds <= 32 tiles of 64 keys: 64 splits of 2048
    a = _sizes(8, 32, 8, 131072, 128, sdpa.BF16)
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 0) == 64
    assert lib.sdpa_decode_workspace_bytes(ctypes.byref(a), 0) == 8 * 32 * 64 * 130 * 4
    # GQA-8 D512, B2, Lk=32768 (2048 tiles of 16 keys): 16-bit head dim 512
    # stays at one workgroup per CU (the four-stage ring): 8 units x 32 splits
    a = _sizes(2, 32, 4, 32768, 512, sdpa.F16)
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 0) == 32
    # ... and three units aim at floor(256 / 3) = 85 splits: 2048 tiles give
    # ceil(2048 / 85) = 25 tiles (400 keys) per split, 82 splits, 246 workgroups
    a = _sizes(1, 24, 3, 32768, 512, sdpa.BF16)
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 0) == 82
    # fp32 at head dim 512 keeps doubling: 32 -> 64 splits
    a = _sizes(2, 32, 4, 32768, 512, sdpa.F32)
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 0) == 64
    # GQA-8 D=512, B=1, Lk=1024: one 16-key tile per split
    a = _sizes(1, 32, 4, 1024, 512, sdpa.F16)
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 0) == 64
    # multi-query decode: Lq * G = 4 * 8 columns = 2 chunks of 16 per KV head
    # -> 8 units start at 32 splits, doubled once to 32 tiles per split;
    # partials are kept per query row
    a = _sizes(1, 32, 4, 32768, 512, sdpa.F16, Lq=4)
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 0) == 64
    assert lib.sdpa_decode_workspace_bytes(ctypes.byref(a), 0) == 1 * 32 * 4 * 64 * 514 * 4
    a = _sizes(1, 32, 4, 1024, 512, sdpa.F16)
    # forced counts and single pass
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 1) == 1
    assert lib.sdpa_decode_workspace_bytes(ctypes.byref(a), 1) == 0
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 7) == 7
    a = _sizes(1, 8, 1, 10, 128, sdpa.F32)
    assert lib.sdpa_decode_num_splits(ctypes.byref(a), 6) == 5   # ceil(10/6)=2 keys -> 5 splits
    # every split count covers the key range exactly once
    for Lk in (1, 31, 32, 33, 1000, 131072):
        for ns in (0, 2, 3, 17):
            if ns > Lk:
                continue
            a = _sizes(1, 4, 1, Lk, 128, sdpa.BF16)
            n = lib.sdpa_decode_num_splits(ctypes.byref(a), ns)
            assert n >= 1
            if ns >= 2:
                ln = -(-Lk // ns)
                assert n == -(-Lk // ln) and (n - 1) * ln < Lk <= n * ln


def test_python_binding_has_no_cpu_path():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError, match="GPU tensors"):
        sdpa.prefill(x, x, x)


def test_backward_struct_layout_matches_c():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "sdpa_mi355x.h"
#define F(f) printf("%s %zu\n", #f, offsetof(sdpa_bwd_args, f));
int main(void) {
  printf("sizeof %zu\n", sizeof(sdpa_bwd_args));
  F(dout) F(dout_stride) F(dq) F(dq_stride) F(dk) F(dk_stride) F(dv) F(dv_stride) F(dsinks)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "layout.c")
        exe = os.path.join(td, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", HEADER_DIR, c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(l.split() for l in out.strip().splitlines())
    assert int(got.pop("sizeof")) == ctypes.sizeof(sdpa.SdpaBwdArgs)
    for name, off in got.items():
        assert getattr(sdpa.SdpaBwdArgs, name).offset == int(off), name


def _bwd(lib, ws=1 << 45, ws_bytes=1 << 30, gkw=None, **kw):
    kw.setdefault("lse", 1 << 44)
    a = _args(**kw)
    g = sdpa.SdpaBwdArgs()
    base = 1 << 41
    for i, n in enumerate(("dout", "dq", "dk", "dv")):
        setattr(g, n, base + i * (1 << 32))
        st = getattr(g, n + "_stride")
        L, H = (64, 8) if n in ("dout", "dq") else (64, 2)
        st[0], st[1], st[2] = H * L * 128, L * 128, 128
    for k_, v_ in (gkw or {}).items():
        if isinstance(v_, tuple):
            arr = getattr(g, k_)
            for i, x in enumerate(v_):
                arr[i] = x
        else:
            setattr(g, k_, v_)
    return lib.sdpa_prefill_backward_check(ctypes.byref(a), ctypes.byref(g), ws, ws_bytes)


def test_backward_validation(lib):
    assert _bwd(lib) == S.OK
    assert _bwd(lib, dtype=sdpa.F32) == S.OK                      # fp32 matrix cores
    assert _bwd(lib, dtype=sdpa.F32, gkw={"dq_stride": (8 * 64 * 128, 64 * 128, 130)}) == S.ERR_ALIGN
    assert _bwd(lib, D=96) == S.OK                               # runs at kernel dim 128
    assert _bwd(lib, Dv=64) == S.OK                              # D = 128, Dv = 64
    assert _bwd(lib, D=100) == S.ERR_UNSUPPORTED                 # not a multiple of 8
    assert _bwd(lib, D=136, q_stride=(8 * 64 * 136, 64 * 136, 136), k_stride=(2 * 64 * 136, 64 * 136, 136),
                v_stride=(2 * 64 * 136, 64 * 136, 136), o_stride=(8 * 64 * 136, 64 * 136, 136),
                gkw={"dq_stride": (8 * 64 * 136, 64 * 136, 136), "dk_stride": (2 * 64 * 136, 64 * 136, 136),
                     "dv_stride": (2 * 64 * 136, 64 * 136, 136),
                     "dout_stride": (8 * 64 * 136, 64 * 136, 136)}) == S.ERR_UNSUPPORTED   # above 128
    assert _bwd(lib, Dv=64, gkw={"dv_stride": (2 * 64 * 56, 64 * 56, 56)}) == S.ERR_ARG  # dv rows overlap
    assert _bwd(lib, lse=None) == S.ERR_NULL
    assert _bwd(lib, gkw={"dq": None}) == S.ERR_NULL
    assert _bwd(lib, gkw={"dk": (1 << 41) + 8}) == S.ERR_ALIGN
    assert _bwd(lib, gkw={"dv_stride": (2 * 64 * 128, 64 * 128, 100)}) == S.ERR_ALIGN
    assert _bwd(lib, gkw={"dk": (1 << 41) + (1 << 32) + 64}) == S.ERR_ARG      # dk inside dq
    assert _bwd(lib, gkw={"dq": (1 << 40) + 64}) == S.ERR_ARG                  # dq inside q
    assert _bwd(lib, gkw={"dsinks": (1 << 46) + 2}) == S.ERR_ALIGN
    assert _bwd(lib, ws=None) == S.ERR_WORKSPACE
    assert _bwd(lib, ws_bytes=64) == S.ERR_WORKSPACE
    assert _bwd(lib, ws=(1 << 45) + 8) == S.ERR_ALIGN
    assert _bwd(lib, ws=(1 << 41) + 64) == S.ERR_ARG                           # workspace inside dout
    a = _args()
    # D_i and LSE rows (B * Hq * Lq * 2 floats), then -- GQA-4 over one
    # 256-key block for 2 x 2 (batch, KV head) units -- the fp32 dK / dV shares
    # of 4 head groups: 4 * B * Hkv * Lk rows of 2 * 128 floats
    assert lib.sdpa_prefill_backward_workspace_bytes(ctypes.byref(a)) == 2 * 8 * 64 * 2 * 4 + 4 * 2 * 2 * 64 * 256 * 4


def test_backward_head_split_plan(lib):
    # The dK / dV key blocks (256 keys) of a GQA call are split over query-head
    # groups: the largest divisor of Hq / Hkv keeping the grid within 512
    # workgroups (two per compute unit).  MHA and fp32 never split.
    def ws(**kw):
        a = _args(**kw)
        return lib.sdpa_prefill_backward_workspace_bytes(ctypes.byref(a))
    base = lambda B, Hq, Lq: ((B * Hq * Lq * 2 * 4 + 15) // 16) * 16
    part = lambda hs, B, Hkv, Lk, kd: hs * B * Hkv * Lk * 2 * kd * 4
    # MHA: no shares
    assert ws(Hkv=8) == base(2, 8, 64)
    # fp32: one workgroup per key block and KV head
    assert ws(dtype=sdpa.F32) == base(2, 8, 64)
    # GQA-4, B1 Hkv8 L4096: 8 x 16 = 128 units -> 4 groups (512 workgroups)
    assert ws(B=1, Hq=32, Hkv=8, Lq=4096, Lk=4096) == base(1, 32, 4096) + part(4, 1, 8, 4096, 128)
    # GQA-4, B4 Hkv8 L4096: 512 units already -> no split
    assert ws(B=4, Hq=32, Hkv=8, Lq=4096, Lk=4096) == base(4, 32, 4096)
    # GQA-8, B1 Hkv4 L4096, D64: 64 units -> 8 groups
    assert ws(B=1, Hq=32, Hkv=4, Lq=4096, Lk=4096, D=64) == base(1, 32, 4096) + part(8, 1, 4, 4096, 64)
    # GQA-6, 3 units: the largest divisor of 6 within 512 workgroups is 6; odd row count rounds up
    assert ws(B=1, Hq=6, Hkv=1, Lq=7, Lk=700) == base(1, 6, 7) + part(6, 1, 1, 700, 128)


def test_prefill_tail_plan(lib):
    # The workspace form of prefill runs the r 128-row tiles past the last
    # multiple of 256 (r <= 128) as two key pieces of whole 64-key tiles each;
    # 16-bit, non-causal, no mask or per-batch lengths, kernel head dim <= 128.
    # Workspace: per piece 128 rows of kernel-dim numerators plus (max, sum),
    # fp32.
    def ws(**kw):
        a = _args(**kw)
        return lib.sdpa_prefill_workspace_bytes(ctypes.byref(a))
    part = lambda r, kd: r * 2 * 128 * (kd + 2) * 4
    dit = dict(B=2, Hq=38, Hkv=38, Lq=4250, Lk=4250, D=64, dtype=sdpa.F16)
    assert ws(**dit) == part(24, 64)  # 2584 tiles: 24 past 2560
    assert ws(**{**dit, "dtype": sdpa.BF16}) == part(24, 64)
    assert ws(**{**dit, "Hq": 42, "Hkv": 42}) == part(40, 64)  # 2856 tiles: 40 past 2816
    assert ws(**{**dit, "causal": 1}) == 0
    assert ws(**{**dit, "dtype": sdpa.F32}) == 0
    assert ws(**{**dit, "D": 256}) == 0
    assert ws(**{**dit, "mask": 1 << 41}) == 0
    assert ws(**{**dit, "seqlens_k": 1 << 41}) == 0
    assert ws(**{**dit, "Hq": 36, "Hkv": 36}) == 0  # 2448 tiles: 144 past 2304, more than 128
    assert ws(B=1, Hq=32, Hkv=32, Lq=4096, Lk=4096, D=128) == 0  # 1024 tiles
    assert ws(B=1, Hq=2, Hkv=2, Lq=128, Lk=128, D=64) == 0  # fewer tiles than compute units
    assert ws(B=1, Hq=257, Hkv=257, Lq=128, Lk=64, D=64) == 0  # one key tile: nothing to split
    # the GPU test cases
    assert ws(B=1, Hq=65, Hkv=65, Lq=512, Lk=512, D=64, dtype=sdpa.F16) == part(4, 64)
    assert ws(B=2, Hq=33, Hkv=33, Lq=512, Lk=300, D=64, dtype=sdpa.F16) == part(8, 64)
    assert ws(B=1, Hq=65, Hkv=13, Lq=500, Lk=700, D=128, dtype=sdpa.F16) == part(4, 128)
    assert ws(B=1, Hq=130, Hkv=130, Lq=256, Lk=4250, D=64, dtype=sdpa.F16) == part(4, 64)


def test_noalloc_decode_rejects_partials_beyond_the_static_scratch(lib):
    # long-context decode shape at 128 splits: 8*32*1*128*(128+2)*4 bytes of
    # partials > 16 MiB; rejected by validation before any HIP call
    B, Hq, Hkv, Lk, D = 8, 32, 8, 131072, 128
    a = _args(B=B, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lk, D=D)
    for n, L, H in (("q", 1, Hq), ("k", Lk, Hkv), ("v", Lk, Hkv), ("o", 1, Hq)):
        st = getattr(a, n + "_stride")
        st[0], st[1], st[2] = H * L * D, L * D, D
    need = lib.sdpa_decode_workspace_bytes(ctypes.byref(a), 128)
    assert need == B * Hq * 128 * (D + 2) * 4 > 16 << 20
    assert lib.sdpa_decode_noalloc(ctypes.byref(a), 128, None) == S.ERR_WORKSPACE
    assert b"static scratch" in lib.sdpa_last_error()
    # invalid arguments are still reported as such
    a.Hq = 30
    assert lib.sdpa_decode_noalloc(ctypes.byref(a), 0, None) == S.ERR_SHAPE
