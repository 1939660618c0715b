// Host <-> kernel interface of the library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa_mi355x.h"

namespace sdpa {

// Kernel parameters, passed by value.  Strides are in elements.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t qs[3], ks[3], vs[3], os[3];
  const void* mask;  // fp32 additive, or uint8 boolean when mask_bool
  int64_t ms[4];
  int mask_bool;
  const float* sinks;
  float* lse;
  int B, Hq, Hkv, Lq, Lk, D;  // D: the kernel's head dim (the real dims rounded up)
  int Dqk, Dv;                  // real head dims of q / k and of v / o (multiples of 8)
  int group;         // Hq / Hkv
  int causal;        // bottom-right causal masking (decode; prefill has it as a template flag)
  const int32_t* seqlens_q;  // optional [B] real query rows per batch
  const int32_t* seqlens_k;  // optional [B] real keys per batch
  float scale_log2;  // scale * log2(e)
  // decode only
  int nsplit;        // number of key-range splits (1 = single pass)
  int nchunk;        // decode: 16-column chunks of the Lq * G (query row, head) columns
  int split_len;     // keys per split
  float* part_o;     // [B*Hq*Lq, nsplit, D]  fp32 partial numerators
  float* part_ml;    // [B*Hq*Lq, nsplit, 2]  fp32 (running max in log2 units, sum)
  // 16-bit prefill work list: `tiles` query tiles (128 rows x one (b, hq));
  // the last tail_tiles of them run as tail_k pieces of tail_chunk keys each,
  // whose partials (part_o: [piece][128 rows][D], part_ml: [piece][128][2])
  // a merge kernel combines (0 tail tiles: one pass per tile)
  int tiles;
  int tail_tiles;
  int tail_k;
  int tail_chunk;
};

AttnParams make_params(const sdpa_args& a);

// Kernel launchers: return hipSuccess or the launch error.  launch_prefill
// sets p.tiles itself; a tail split (p.tail_tiles > 0, non-causal 16-bit
// without a mask, kernel head dim <= 128) also enqueues the merge.
hipError_t launch_prefill(const AttnParams& p, int dtype, bool causal, hipStream_t s);
hipError_t launch_decode(const AttnParams& p, int dtype, hipStream_t s);
// 16-bit prefill at kernel head dim 512 (sets its own column chunks), one pass
hipError_t launch_prefill_wide(const AttnParams& p, int dtype, hipStream_t s);
// Gradients: ws holds 2 * B * Hq * Lq floats (D_i, then the LSE in log2
// units) and, with head_split > 1, from the next 16-byte boundary on,
// head_split * B * Hkv * Lk rows of 2 * kernel head dim floats (each head
// group's fp32 dK, dV).
hipError_t launch_backward(const AttnParams& p, const sdpa_bwd_args& g, float scale, float* ws, int dtype,
                           bool causal, int head_split, hipStream_t s);
// The dK / dV kernel's keys per workgroup (16-bit).
constexpr int kBwdKeyBlock = 256;

// Decode tiling shared by the host heuristics and the kernels.  The Lq * G
// (query row, head) columns of a KV head form 16-column blocks; in 16-bit up
// to four blocks share one pass over K / V (one workgroup per chunk and split).
inline int decode_cpw(int dtype, int64_t cols) {
  return dtype == SDPA_F32 ? 1 : (cols > 32 ? 4 : (cols > 16 ? 2 : 1));
}
int decode_tile_keys(int dtype, int D, int cpw);

}  // namespace sdpa
