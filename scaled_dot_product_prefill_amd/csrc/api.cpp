// Host side of libsdpa_mi355x.so: argument validation, decode split choice,
// workspace layout and the extern "C" entry points declared in sdpa_mi355x.h.
//
// Validation happens entirely before any HIP call, so the *_check entry
// points (and every error path of the launching entry points) run without a
// GPU.  Unsupported requests return SDPA_ERR_UNSUPPORTED instead of taking a
// slower path, the convention of the force_fused check on the "Add D512
// support to Metal vector attention" page.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "sdpa_internal.hpp"
#include "sdpa_mi355x.h"

// Split partials of sdpa_decode_noalloc: one copy per GPU, alive until the
// process ends, shared by every call on that GPU.
static __device__ __align__(256) unsigned char scratch[SDPA_DECODE_SCRATCH_BYTES];

namespace sdpa {
namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SDPA_OK;
}

int elem_bytes(int dtype) { return dtype == SDPA_F32 ? 4 : 2; }

constexpr int64_t kMaxInt = 2147483647LL;
constexpr int64_t kMaxRowBytes = 1LL << 23;  // 8 MiB: 256 rows stay below 2^31 bytes

struct Extent {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool valid = false;
};

Extent tensor_extent(const void* p, const int64_t* st, int64_t n0, int64_t n1, int64_t n2,
                     int64_t inner, int es) {
  Extent e;
  if (!p) return e;
  const int64_t last = (n0 - 1) * st[0] + (n1 - 1) * st[1] + (n2 - 1) * st[2] + inner;
  e.lo = (uintptr_t)p;
  e.hi = e.lo + (uintptr_t)(last * es);
  e.valid = true;
  return e;
}

bool overlaps(const Extent& a, const Extent& b) {
  return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi;
}

// Head dim of v and o (0 in the argument block means the q / k head dim).
int64_t dv_of(const sdpa_args* a) { return a->Dv ? a->Dv : a->D; }

// The kernels' head dim: the real dims rounded up to 64, 128, 256 or 512
// (0 beyond 512).  Chunks past the real dims are zero-filled on load and not
// stored.
int kernel_dim(const sdpa_args* a) {
  const int64_t d = a->D > dv_of(a) ? a->D : dv_of(a);
  for (int k : {64, 128, 256, 512})
    if (d <= k) return k;
  return 0;
}

// Size and scalar checks (no pointers examined).
int check_sizes(const sdpa_args* a) {
  if (!a) return fail(SDPA_ERR_NULL, "args is NULL");
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Lq < 1 || a->Lk < 1 || a->D < 1)
    return fail(SDPA_ERR_SHAPE, "B, Hq, Hkv, Lq, Lk, D must all be >= 1 (got %lld %lld %lld %lld %lld %lld)",
                (long long)a->B, (long long)a->Hq, (long long)a->Hkv, (long long)a->Lq,
                (long long)a->Lk, (long long)a->D);
  if (a->Hq % a->Hkv != 0)
    return fail(SDPA_ERR_SHAPE, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)a->Hq,
                (long long)a->Hkv);
  if (a->Dv < 0) return fail(SDPA_ERR_SHAPE, "Dv must be >= 0 (0 = D), got %lld", (long long)a->Dv);
  if (a->D % 8 != 0 || dv_of(a) % 8 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "head dims must be multiples of 8, got D=%lld Dv=%lld", (long long)a->D,
                (long long)dv_of(a));
  if (a->Lq > kMaxInt / 2 || a->Lk > kMaxInt / 2 || a->B * a->Hq > kMaxInt / 2)
    return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond the 32-bit index range of the kernels");
  if (a->dtype != SDPA_F32 && a->dtype != SDPA_F16 && a->dtype != SDPA_BF16)
    return fail(SDPA_ERR_UNSUPPORTED, "dtype %d is not one of SDPA_F32, SDPA_F16, SDPA_BF16", a->dtype);
  if (a->causal != 0 && a->causal != 1) return fail(SDPA_ERR_ARG, "causal must be 0 or 1");
  if (a->mask_kind != SDPA_MASK_ADD_F32 && a->mask_kind != SDPA_MASK_BOOL)
    return fail(SDPA_ERR_ARG, "mask_kind must be SDPA_MASK_ADD_F32 or SDPA_MASK_BOOL");
  if (!std::isfinite(a->scale)) return fail(SDPA_ERR_ARG, "scale must be finite");
  return SDPA_OK;
}

// Checks shared by both launching entry points.
int check_common(const sdpa_args* a) {
  int st = check_sizes(a);
  if (st != SDPA_OK) return st;
  if (!a->q || !a->k || !a->v || !a->o) return fail(SDPA_ERR_NULL, "q, k, v and o must be non-NULL");
  const int es = elem_bytes(a->dtype);
  const void* ptrs[4] = {a->q, a->k, a->v, a->o};
  const int64_t* strides[4] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t) {
    if ((uintptr_t)ptrs[t] % 16 != 0) return fail(SDPA_ERR_ALIGN, "%s is not 16-byte aligned", names[t]);
    for (int d = 0; d < 3; ++d) {
      if (strides[t][d] < 0) return fail(SDPA_ERR_ARG, "%s stride %d is negative", names[t], d);
      if ((strides[t][d] * es) % 16 != 0)
        return fail(SDPA_ERR_ALIGN, "%s stride %d (%lld elements) is not a multiple of 16 bytes",
                    names[t], d, (long long)strides[t][d]);
    }
  }
  if (a->o_stride[2] < dv_of(a)) return fail(SDPA_ERR_ARG, "o rows overlap (o_stride[2] < Dv)");
  // key/value tiles are addressed with 32-bit byte offsets from the tile's first row
  if (a->k_stride[2] * es > kMaxRowBytes || a->v_stride[2] * es > kMaxRowBytes)
    return fail(SDPA_ERR_UNSUPPORTED, "k/v row stride above %lld bytes", (long long)kMaxRowBytes);
  const int mask_es = a->mask_kind == SDPA_MASK_BOOL ? 1 : 4;
  if (a->mask) {
    if ((uintptr_t)a->mask % mask_es != 0) return fail(SDPA_ERR_ALIGN, "mask is not 4-byte aligned");
    for (int d = 0; d < 4; ++d)
      if (a->mask_stride[d] < 0) return fail(SDPA_ERR_ARG, "mask stride %d is negative", d);
  }
  if (a->sinks && (uintptr_t)a->sinks % 4 != 0) return fail(SDPA_ERR_ALIGN, "sinks is not 4-byte aligned");
  if (a->seqlens_q && (uintptr_t)a->seqlens_q % 4 != 0)
    return fail(SDPA_ERR_ALIGN, "seqlens_q is not 4-byte aligned");
  if (a->seqlens_k && (uintptr_t)a->seqlens_k % 4 != 0)
    return fail(SDPA_ERR_ALIGN, "seqlens_k is not 4-byte aligned");
  if (a->lse && (uintptr_t)a->lse % 4 != 0) return fail(SDPA_ERR_ALIGN, "lse is not 4-byte aligned");

  // the output must not overlap any input or the other output
  const Extent eo = tensor_extent(a->o, a->o_stride, a->B, a->Hq, a->Lq, dv_of(a), es);
  const Extent eq = tensor_extent(a->q, a->q_stride, a->B, a->Hq, a->Lq, a->D, es);
  const Extent ek = tensor_extent(a->k, a->k_stride, a->B, a->Hkv, a->Lk, a->D, es);
  const Extent ev = tensor_extent(a->v, a->v_stride, a->B, a->Hkv, a->Lk, dv_of(a), es);
  Extent em;
  if (a->mask) {
    const int64_t last = (a->B - 1) * a->mask_stride[0] + (a->Hq - 1) * a->mask_stride[1] +
                         (a->Lq - 1) * a->mask_stride[2] + (a->Lk - 1) * a->mask_stride[3] + 1;
    em.lo = (uintptr_t)a->mask;
    em.hi = em.lo + (uintptr_t)(last * mask_es);
    em.valid = true;
  }
  Extent es_, el, esq, esk;
  if (a->sinks) { es_.lo = (uintptr_t)a->sinks; es_.hi = es_.lo + a->Hq * 4; es_.valid = true; }
  if (a->lse) { el.lo = (uintptr_t)a->lse; el.hi = el.lo + a->B * a->Hq * a->Lq * 4; el.valid = true; }
  if (a->seqlens_q) { esq.lo = (uintptr_t)a->seqlens_q; esq.hi = esq.lo + a->B * 4; esq.valid = true; }
  if (a->seqlens_k) { esk.lo = (uintptr_t)a->seqlens_k; esk.hi = esk.lo + a->B * 4; esk.valid = true; }
  if (overlaps(eo, eq) || overlaps(eo, ek) || overlaps(eo, ev) || overlaps(eo, em) ||
      overlaps(eo, es_) || overlaps(eo, el) || overlaps(eo, esq) || overlaps(eo, esk))
    return fail(SDPA_ERR_ARG, "o overlaps an input or lse");
  if (overlaps(el, eq) || overlaps(el, ek) || overlaps(el, ev) || overlaps(el, em) || overlaps(el, es_) ||
      overlaps(el, esq) || overlaps(el, esk))
    return fail(SDPA_ERR_ARG, "lse overlaps an input");
  return SDPA_OK;
}

// Decode: the Lq query rows times the G heads of a KV head are the columns of
// 16-wide matrix tiles; each chunk of 16 columns is one workgroup per key split.
int64_t decode_chunks(const sdpa_args* a) {
  const int64_t cols = a->Lq * (a->Hq / a->Hkv);
  const int64_t w = 16 * decode_cpw(a->dtype, cols);
  return (cols + w - 1) / w;
}

// Prefill head dims the 128-row prefill kernels do not hold (kernel head dim
// 512, or above 128 in fp32: a 32-row wave's O accumulator alone would fill
// the register file) run on the 16-column kernels of the decode path, one
// pass over the keys per workgroup: in 16-bit each wave owns 16 columns of
// its own, in fp32 the four waves share 16.
bool prefill_narrow(const sdpa_args* a) {
  const int kd = kernel_dim(a);
  return kd == 512 || (a->dtype == SDPA_F32 && kd > 128);
}

int check_prefill(const sdpa_args* a) {
  int st = check_common(a);
  if (st != SDPA_OK) return st;
  if (kernel_dim(a) == 0)
    return fail(SDPA_ERR_UNSUPPORTED, "prefill supports head dims up to 512, got D=%lld Dv=%lld",
                (long long)a->D, (long long)dv_of(a));
  const int64_t grid = prefill_narrow(a) ? decode_chunks(a) * a->B * a->Hkv : ((a->Lq + 127) / 128) * a->B * a->Hq;
  if (grid > kMaxInt) return fail(SDPA_ERR_UNSUPPORTED, "grid too large");
  return SDPA_OK;
}

// Decode: the Lq query rows times the G heads of a KV head are the columns of
// 16-wide matrix tiles (multi-query decode, e.g. speculative or chunked
// decoding); each chunk of 16 columns is one workgroup per key split
// (decode_chunks).
constexpr int kMaxDecodeLq = 16;
struct SplitPlan {
  int nsplit = 1;
  int split_len = 0;
};

// Split of the key range for decode.  Automatic: start from one workgroup per
// compute unit (MI355X: 256), then double the split count while a split would
// still hold more than 32 key tiles (up to 16 workgroups per CU); never more
// splits than tiles, each split a whole number of tiles.  16-bit kernels at
// head dim 256 / 512 with one 16-column block stop at one workgroup per CU
// instead: such a grid runs with a four-stage load ring (three tiles in
// flight), which streams faster than two workgroups of two stages each
// (GQA-8 D512 B2 Lk32768 fp16, cold: 32 splits 100 us, 64 splits 102 us).
// Measured on the GQA-8 D512 and long-context D128 decode shapes, this is
// within a few percent of the best fixed split count for each.
constexpr int64_t kDecodeCUs = 256;
constexpr int64_t kDecodeMaxTilesPerSplit = 32;

// Prefill tail split (16-bit, non-causal, no mask, no per-batch lengths,
// kernel head dim <= 128).  The query tiles take about equal time, and the
// kernel runs as long as the compute unit that gets the most of them:
// ceil(tiles / 256) tiles' worth (a sweep of the head count at B2 L4250 D64
// moves in those steps).  The r = tiles % 256 tiles past the last multiple of
// 256 therefore run as two key pieces each (pieces of a whole number of
// 64-key tiles; needs r <= 128), so that they spread over 2 r compute units
// and add half a tile's time instead of a whole one; a merge kernel combines
// the pieces.  More pieces per tile (up to 8) measured slower on the DiT
// shape (B2 H38 L4250 D64, r = 24; same box, fp16 one pass 377 us: 2 pieces
// 364 us, 4 pieces 368 us, 8 pieces 375 us): each piece pays the start of a
// tile loop and writes a whole partial.  Not without a workspace
// (sdpa_prefill).
constexpr int64_t kTailPieces = 2;
struct TailPlan {
  int64_t tiles = 0;
  int64_t tail = 0;
  int k = 1;
  int64_t chunk = 0;
};
TailPlan plan_tail(const sdpa_args* a) {
  TailPlan t;
  if (a->dtype == SDPA_F32 || a->causal || a->mask || a->seqlens_q || a->seqlens_k) return t;
  if (prefill_narrow(a) || kernel_dim(a) > 128) return t;
  const int64_t tiles = (a->Lq + 127) / 128 * a->B * a->Hq;
  const int64_t r = tiles % kDecodeCUs;
  if (tiles < kDecodeCUs || r == 0) return t;
  const int64_t k0 = std::min<int64_t>(kTailPieces, kDecodeCUs / r);
  if (k0 < 2) return t;
  const int64_t chunk = ((a->Lk + k0 - 1) / k0 + 63) / 64 * 64;
  const int64_t k = (a->Lk + chunk - 1) / chunk;
  if (k != kTailPieces) return t;  // the merge kernel takes exactly two pieces
  t.tiles = tiles;
  t.tail = r;
  t.k = (int)k;
  t.chunk = chunk;
  return t;
}
// partial numerators [piece][128][kernel head dim] and (max, sum) [piece][128][2]
size_t tail_workspace(const sdpa_args* a, const TailPlan& t) {
  if (t.tail == 0) return 0;
  return (size_t)t.tail * t.k * 128 * (size_t)(kernel_dim(a) + 2) * sizeof(float);
}

SplitPlan plan_splits(const sdpa_args* a, int num_splits) {
  SplitPlan sp;
  const int64_t Lk = a->Lk;
  if (num_splits == 1) {
    sp.nsplit = 1;
    sp.split_len = (int)Lk;
    return sp;
  }
  int64_t len;
  if (num_splits >= 2) {
    len = (Lk + num_splits - 1) / num_splits;
  } else {
    const int64_t tk = decode_tile_keys(a->dtype, kernel_dim(a), decode_cpw(a->dtype, a->Lq * (a->Hq / a->Hkv)));
    const int64_t tiles = (Lk + tk - 1) / tk;
    const int64_t units = a->B * a->Hkv * decode_chunks(a);
    const bool deep = a->dtype != SDPA_F32 && kernel_dim(a) >= 256 &&
                      decode_cpw(a->dtype, a->Lq * (a->Hq / a->Hkv)) == 1;
    int64_t ns = deep ? kDecodeCUs / units : (kDecodeCUs + units - 1) / units;
    while (!deep && (tiles + ns - 1) / ns > kDecodeMaxTilesPerSplit && ns * units < 16 * kDecodeCUs) ns *= 2;
    if (ns > tiles) ns = tiles;
    if (ns < 1) ns = 1;
    const int64_t tiles_per = (tiles + ns - 1) / ns;
    len = tiles_per * tk;
  }
  sp.split_len = (int)len;
  sp.nsplit = (int)((Lk + len - 1) / len);
  return sp;
}

size_t workspace_for(const sdpa_args* a, const SplitPlan& sp) {
  if (sp.nsplit <= 1) return 0;
  return (size_t)a->B * a->Hq * a->Lq * sp.nsplit * (kernel_dim(a) + 2) * sizeof(float);
}

// static_scratch: the partials go to the library's static device array
// (sdpa_decode_noalloc) instead of the caller's workspace.
int check_decode(const sdpa_args* a, int num_splits, const void* ws, size_t ws_bytes, SplitPlan* out,
                 bool static_scratch = false) {
  int st = check_common(a);
  if (st != SDPA_OK) return st;
  if (a->Lq > kMaxDecodeLq)
    return fail(SDPA_ERR_UNSUPPORTED, "decode supports 1 <= Lq <= %d, got %lld", kMaxDecodeLq, (long long)a->Lq);
  if (kernel_dim(a) == 0)
    return fail(SDPA_ERR_UNSUPPORTED, "decode supports head dims up to 512, got D=%lld Dv=%lld", (long long)a->D,
                (long long)dv_of(a));
  if (num_splits < 0 || num_splits > a->Lk)
    return fail(SDPA_ERR_ARG, "num_splits must be in [0, Lk], got %d", num_splits);
  SplitPlan sp = plan_splits(a, num_splits);
  if ((int64_t)sp.nsplit * decode_chunks(a) * a->Hkv * a->B > kMaxInt)
    return fail(SDPA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = workspace_for(a, sp);
  if (static_scratch) {
    if (need > SDPA_DECODE_SCRATCH_BYTES)
      return fail(SDPA_ERR_WORKSPACE,
                  "the %d-split partials need %zu bytes, above the %zu-byte static scratch of "
                  "sdpa_decode_noalloc (pass fewer splits, or sdpa_decode with a workspace)",
                  sp.nsplit, need, (size_t)SDPA_DECODE_SCRATCH_BYTES);
  } else if (need > 0) {
    if (!ws) return fail(SDPA_ERR_WORKSPACE, "two-pass decode needs a workspace of %zu bytes", need);
    if ((uintptr_t)ws % 16 != 0) return fail(SDPA_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < need)
      return fail(SDPA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  }
  if (out) *out = sp;
  return SDPA_OK;
}

// Backward: the forward's checks (o and lse are inputs), 16-bit only,
// D in {64, 128}, and the gradient outputs.
// Query-head groups a 16-bit dK / dV key block is split over (GQA): the
// largest divisor of Hq / Hkv that keeps the grid within two workgroups per
// compute unit.  Each group's workgroup accumulates its heads' share in
// fp32; a reduction pass adds the groups up.
int bwd_head_split(const sdpa_args* a) {
  if (a->dtype == SDPA_F32 || a->Hkv <= 0) return 1;
  const int64_t g = a->Hq / a->Hkv;
  const int64_t units = a->B * a->Hkv * ((a->Lk + kBwdKeyBlock - 1) / kBwdKeyBlock);
  int hs = 1;
  for (int64_t d = 2; d <= g; ++d)
    if (g % d == 0 && units * d <= 2 * kDecodeCUs) hs = (int)d;
  return hs;
}
size_t backward_workspace(const sdpa_args* a) {
  // D_i and LSE rows, rounded up to 16 bytes, then the head groups' shares
  size_t n = ((size_t)a->B * a->Hq * a->Lq * 2 * sizeof(float) + 15) / 16 * 16;
  const int hs = bwd_head_split(a);
  if (hs > 1) n += (size_t)hs * a->B * a->Hkv * a->Lk * 2 * kernel_dim(a) * sizeof(float);
  return n;
}

int check_backward(const sdpa_args* a, const sdpa_bwd_args* g, const void* ws, size_t ws_bytes) {
  int st = check_common(a);
  if (st != SDPA_OK) return st;
  if (!g) return fail(SDPA_ERR_NULL, "gradient arguments are NULL");
  const int es = a->dtype == SDPA_F32 ? 4 : 2;  // element bytes of every tensor
  const int kd = kernel_dim(a);
  if (kd != 64 && kd != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "backward supports head dims up to 128, got D=%lld Dv=%lld", (long long)a->D,
                (long long)dv_of(a));
  if (!a->lse) return fail(SDPA_ERR_NULL, "backward needs the forward's lse");
  if (!g->dout || !g->dq || !g->dk || !g->dv) return fail(SDPA_ERR_NULL, "dout, dq, dk and dv must be non-NULL");
  const void* ptrs[4] = {g->dout, g->dq, g->dk, g->dv};
  const int64_t* strides[4] = {g->dout_stride, g->dq_stride, g->dk_stride, g->dv_stride};
  const char* names[4] = {"dout", "dq", "dk", "dv"};
  for (int t = 0; t < 4; ++t) {
    if ((uintptr_t)ptrs[t] % 16 != 0) return fail(SDPA_ERR_ALIGN, "%s is not 16-byte aligned", names[t]);
    for (int d = 0; d < 3; ++d) {
      if (strides[t][d] < 0) return fail(SDPA_ERR_ARG, "%s stride %d is negative", names[t], d);
      if ((strides[t][d] * es) % 16 != 0)
        return fail(SDPA_ERR_ALIGN, "%s stride %d (%lld elements) is not a multiple of 16 bytes", names[t], d,
                    (long long)strides[t][d]);
    }
  }
  if (g->dout_stride[2] * es > kMaxRowBytes)
    return fail(SDPA_ERR_UNSUPPORTED, "dout row stride above %lld bytes", (long long)kMaxRowBytes);
  if (a->q_stride[2] * es > kMaxRowBytes)
    return fail(SDPA_ERR_UNSUPPORTED, "q row stride above %lld bytes", (long long)kMaxRowBytes);
  if (g->dq_stride[2] < a->D || g->dk_stride[2] < a->D || g->dv_stride[2] < dv_of(a))
    return fail(SDPA_ERR_ARG, "gradient rows overlap (row stride below the head dim)");
  if (g->dsinks && (uintptr_t)g->dsinks % 4 != 0) return fail(SDPA_ERR_ALIGN, "dsinks is not 4-byte aligned");
  const size_t need = backward_workspace(a);
  if (!ws) return fail(SDPA_ERR_WORKSPACE, "backward needs a workspace of %zu bytes", need);
  if ((uintptr_t)ws % 16 != 0) return fail(SDPA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < need) return fail(SDPA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);

  // outputs: disjoint from each other, from every input and from the workspace
  const Extent outs[4] = {tensor_extent(g->dq, g->dq_stride, a->B, a->Hq, a->Lq, a->D, es),
                          tensor_extent(g->dk, g->dk_stride, a->B, a->Hkv, a->Lk, a->D, es),
                          tensor_extent(g->dv, g->dv_stride, a->B, a->Hkv, a->Lk, dv_of(a), es), Extent{}};
  Extent eds;
  if (g->dsinks) { eds.lo = (uintptr_t)g->dsinks; eds.hi = eds.lo + a->Hq * 4; eds.valid = true; }
  Extent ews;
  ews.lo = (uintptr_t)ws; ews.hi = ews.lo + need; ews.valid = true;
  Extent ins[12];
  int n = 0;
  ins[n++] = tensor_extent(a->q, a->q_stride, a->B, a->Hq, a->Lq, a->D, es);
  ins[n++] = tensor_extent(a->k, a->k_stride, a->B, a->Hkv, a->Lk, a->D, es);
  ins[n++] = tensor_extent(a->v, a->v_stride, a->B, a->Hkv, a->Lk, dv_of(a), es);
  ins[n++] = tensor_extent(a->o, a->o_stride, a->B, a->Hq, a->Lq, dv_of(a), es);
  ins[n++] = tensor_extent(g->dout, g->dout_stride, a->B, a->Hq, a->Lq, dv_of(a), es);
  { Extent e; e.lo = (uintptr_t)a->lse; e.hi = e.lo + a->B * a->Hq * a->Lq * 4; e.valid = true; ins[n++] = e; }
  if (a->mask) {
    const int64_t last = (a->B - 1) * a->mask_stride[0] + (a->Hq - 1) * a->mask_stride[1] +
                         (a->Lq - 1) * a->mask_stride[2] + (a->Lk - 1) * a->mask_stride[3] + 1;
    const int mes = a->mask_kind == SDPA_MASK_BOOL ? 1 : 4;
    Extent e; e.lo = (uintptr_t)a->mask; e.hi = e.lo + (uintptr_t)(last * mes); e.valid = true; ins[n++] = e;
  }
  if (a->sinks) { Extent e; e.lo = (uintptr_t)a->sinks; e.hi = e.lo + a->Hq * 4; e.valid = true; ins[n++] = e; }
  if (a->seqlens_q) { Extent e; e.lo = (uintptr_t)a->seqlens_q; e.hi = e.lo + a->B * 4; e.valid = true; ins[n++] = e; }
  if (a->seqlens_k) { Extent e; e.lo = (uintptr_t)a->seqlens_k; e.hi = e.lo + a->B * 4; e.valid = true; ins[n++] = e; }
  ins[n++] = ews;
  Extent all_out[4] = {outs[0], outs[1], outs[2], eds};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(all_out[i], all_out[j])) return fail(SDPA_ERR_ARG, "gradient outputs overlap each other");
    for (int j = 0; j < n; ++j)
      if (overlaps(all_out[i], ins[j])) return fail(SDPA_ERR_ARG, "a gradient output overlaps an input or the workspace");
  }
  for (int j = 0; j + 1 < n; ++j)
    if (overlaps(ews, ins[j])) return fail(SDPA_ERR_ARG, "workspace overlaps an input");
  const int64_t grid = ((a->Lq + 127) / 128) * a->B * a->Hq;
  const int64_t gridk = ((a->Lk + 127) / 128) * a->B * a->Hkv;
  if (grid > kMaxInt || gridk > kMaxInt) return fail(SDPA_ERR_UNSUPPORTED, "grid too large");
  return SDPA_OK;
}

int launch_status(hipError_t e) {
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Device address of the static decode scratch on the current device, looked
// up once per device (each GPU holds its own copy of the array).  In host code
// the array's name only stands for the symbol; kernels get this address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int scratch_address(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SDPA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch covers", dev,
                kMaxDevices);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return fail(SDPA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(SDPA_ERR_ARG, "stream belongs to device %d, the current device is %d", (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SDPA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SDPA_OK;
}

}  // namespace

AttnParams make_params(const sdpa_args& a) {
  AttnParams p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o;
  for (int d = 0; d < 3; ++d) {
    p.qs[d] = a.q_stride[d]; p.ks[d] = a.k_stride[d];
    p.vs[d] = a.v_stride[d]; p.os[d] = a.o_stride[d];
  }
  p.mask = a.mask;
  p.mask_bool = a.mask_kind == SDPA_MASK_BOOL;
  for (int d = 0; d < 4; ++d) p.ms[d] = a.mask_stride[d];
  p.sinks = a.sinks;
  p.lse = a.lse;
  p.B = (int)a.B; p.Hq = (int)a.Hq; p.Hkv = (int)a.Hkv;
  p.Lq = (int)a.Lq; p.Lk = (int)a.Lk;
  p.D = kernel_dim(&a);
  p.Dqk = (int)a.D;
  p.Dv = (int)dv_of(&a);
  p.group = (int)(a.Hq / a.Hkv);
  p.causal = a.causal;
  p.seqlens_q = a.seqlens_q;
  p.seqlens_k = a.seqlens_k;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.nsplit = 1;
  p.nchunk = 1;
  p.split_len = (int)a.Lk;
  p.tiles = 0;
  p.tail_tiles = 0;
  p.tail_k = 1;
  p.tail_chunk = (int)a.Lk;
  return p;
}

}  // namespace sdpa

extern "C" {

int sdpa_prefill_check(const sdpa_args* args) {
  int st = sdpa::check_prefill(args);
  return st == SDPA_OK ? sdpa::ok() : st;
}

int sdpa_prefill(const sdpa_args* args, void* stream) {
  int st = sdpa::check_prefill(args);
  if (st != SDPA_OK) return st;
  sdpa::AttnParams p = sdpa::make_params(*args);
  if (sdpa::prefill_narrow(args)) {
    p.nsplit = 1;
    p.split_len = (int)args->Lk;
    if (args->dtype != SDPA_F32)
      return sdpa::launch_status(sdpa::launch_prefill_wide(p, args->dtype, (hipStream_t)stream));
    p.nchunk = (int)sdpa::decode_chunks(args);
    return sdpa::launch_status(sdpa::launch_decode(p, args->dtype, (hipStream_t)stream));
  }
  return sdpa::launch_status(sdpa::launch_prefill(p, args->dtype, args->causal != 0, (hipStream_t)stream));
}

size_t sdpa_prefill_workspace_bytes(const sdpa_args* args) {
  // sizes only (like the decode query): pointers and strides are not needed
  if (sdpa::check_sizes(args) != SDPA_OK || sdpa::kernel_dim(args) == 0) return 0;
  return sdpa::tail_workspace(args, sdpa::plan_tail(args));
}

int sdpa_prefill_ws(const sdpa_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  int st = sdpa::check_prefill(args);
  if (st != SDPA_OK) return st;
  const sdpa::TailPlan t = sdpa::plan_tail(args);
  const size_t need = sdpa::tail_workspace(args, t);
  if (need == 0) return sdpa_prefill(args, stream);
  if (workspace == nullptr || workspace_bytes < need)
    return sdpa::fail(SDPA_ERR_WORKSPACE, "prefill workspace: need %zu bytes, got %zu%s", need, workspace_bytes,
                      workspace ? "" : " (null)");
  if (((uintptr_t)workspace & 15) != 0) return sdpa::fail(SDPA_ERR_WORKSPACE, "prefill workspace not 16-byte aligned");
  sdpa::AttnParams p = sdpa::make_params(*args);
  p.tail_tiles = (int)t.tail;
  p.tail_k = t.k;
  p.tail_chunk = (int)t.chunk;
  p.part_o = (float*)workspace;
  p.part_ml = p.part_o + (size_t)t.tail * t.k * 128 * sdpa::kernel_dim(args);
  return sdpa::launch_status(sdpa::launch_prefill(p, args->dtype, false, (hipStream_t)stream));
}

int sdpa_decode_check(const sdpa_args* args, int num_splits, const void* workspace, size_t workspace_bytes) {
  int st = sdpa::check_decode(args, num_splits, workspace, workspace_bytes, nullptr);
  return st == SDPA_OK ? sdpa::ok() : st;
}

int sdpa_decode_num_splits(const sdpa_args* args, int num_splits) {
  if (sdpa::check_sizes(args) != SDPA_OK) return 0;
  if (num_splits < 0 || num_splits > args->Lk) return 0;
  return sdpa::plan_splits(args, num_splits).nsplit;
}

size_t sdpa_decode_workspace_bytes(const sdpa_args* args, int num_splits) {
  if (sdpa::check_sizes(args) != SDPA_OK) return 0;
  if (num_splits < 0 || num_splits > args->Lk) return 0;
  return sdpa::workspace_for(args, sdpa::plan_splits(args, num_splits));
}

int sdpa_decode(const sdpa_args* args, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  sdpa::SplitPlan sp;
  int st = sdpa::check_decode(args, num_splits, workspace, workspace_bytes, &sp);
  if (st != SDPA_OK) return st;
  sdpa::AttnParams p = sdpa::make_params(*args);
  p.nsplit = sp.nsplit;
  p.split_len = sp.split_len;
  p.nchunk = (int)sdpa::decode_chunks(args);
  if (sp.nsplit > 1) {
    float* ws = (float*)workspace;
    p.part_o = ws;
    p.part_ml = ws + (size_t)args->B * args->Hq * args->Lq * sp.nsplit * sdpa::kernel_dim(args);
  }
  return sdpa::launch_status(sdpa::launch_decode(p, args->dtype, (hipStream_t)stream));
}

int sdpa_decode_noalloc(const sdpa_args* args, int num_splits, void* stream) {
  sdpa::SplitPlan sp;
  int st = sdpa::check_decode(args, num_splits, nullptr, 0, &sp, /*static_scratch=*/true);
  if (st != SDPA_OK) return st;
  sdpa::AttnParams p = sdpa::make_params(*args);
  p.nsplit = sp.nsplit;
  p.split_len = sp.split_len;
  p.nchunk = (int)sdpa::decode_chunks(args);
  if (sp.nsplit > 1) {
    void* base = nullptr;
    st = sdpa::scratch_address(stream, &base);
    if (st != SDPA_OK) return st;
    float* ws = (float*)base;
    p.part_o = ws;
    p.part_ml = ws + (size_t)args->B * args->Hq * args->Lq * sp.nsplit * sdpa::kernel_dim(args);
  }
  return sdpa::launch_status(sdpa::launch_decode(p, args->dtype, (hipStream_t)stream));
}

int sdpa_prefill_backward_check(const sdpa_args* fwd, const sdpa_bwd_args* grad, const void* workspace,
                                size_t workspace_bytes) {
  int st = sdpa::check_backward(fwd, grad, workspace, workspace_bytes);
  return st == SDPA_OK ? sdpa::ok() : st;
}

size_t sdpa_prefill_backward_workspace_bytes(const sdpa_args* fwd) {
  if (sdpa::check_sizes(fwd) != SDPA_OK) return 0;
  return sdpa::backward_workspace(fwd);
}

int sdpa_prefill_backward(const sdpa_args* fwd, const sdpa_bwd_args* grad, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int st = sdpa::check_backward(fwd, grad, workspace, workspace_bytes);
  if (st != SDPA_OK) return st;
  sdpa::AttnParams p = sdpa::make_params(*fwd);
  return sdpa::launch_status(sdpa::launch_backward(p, *grad, fwd->scale, (float*)workspace, fwd->dtype,
                                                   fwd->causal != 0, sdpa::bwd_head_split(fwd), (hipStream_t)stream));
}

const char* sdpa_status_string(int status) {
  switch (status) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_NULL: return "required pointer is NULL";
    case SDPA_ERR_SHAPE: return "inconsistent sizes";
    case SDPA_ERR_UNSUPPORTED: return "unsupported request (no kernel covers it)";
    case SDPA_ERR_ALIGN: return "pointer or stride alignment";
    case SDPA_ERR_WORKSPACE: return "workspace missing or too small";
    case SDPA_ERR_ARG: return "invalid argument";
    case SDPA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sdpa_last_error(void) { return sdpa::g_last_error.c_str(); }

const char* sdpa_version(void) { return "sdpa_mi355x abi 2, gfx950 (CDNA4)"; }

}  // extern "C"
