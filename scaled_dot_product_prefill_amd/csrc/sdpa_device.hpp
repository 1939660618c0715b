// Device-side building blocks shared by the prefill and decode kernels
// (gfx950 / CDNA4 only).
//
// Matrix-core operand layouts used throughout (wave64, lane l, register r):
//   v_mfma_f32_32x32x16_{bf16,f16}: A[m][k] m = l%32, k = 8*(l/32)+e (e = 0..7)
//                                   B[k][n] n = l%32, k = 8*(l/32)+e
//                                   C[m][n] n = l%32, m = 8*(r/4)+4*(l/32)+r%4 (r = 0..15)
//   v_mfma_f32_32x32x2_f32:        A m = l%32, k = l/32;  B n = l%32, k = l/32;  C as above
//   v_mfma_f32_16x16x32_{bf16,f16}: A m = l%16, k = 8*(l/16)+e;  B n = l%16, k = 8*(l/16)+e
//                                   C n = l%16, m = 4*(l/16)+r (r = 0..3)
//   v_mfma_f32_16x16x4_f32:        A m = l%16, k = l/16;  B n = l%16, k = l/16;  C as above
// A reduction index k may be assigned to any element of the contraction as
// long as A and B agree; the kernels use that freedom to read operands as
// 16-byte vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// element types: storage is raw bits; arithmetic is always fp32
// ---------------------------------------------------------------------------
struct TF32 {
  using storage = float;
  static constexpr int kBytes = 4;
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static inline float to_f32(storage x) { return x; }
  __device__ static inline storage from_f32(float x) { return x; }
};
struct TF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kVec = 8;
  __device__ static inline float to_f32(storage x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
  __device__ static inline storage from_f32(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
  }
  // pack two fp32 into one dword (lo in bits 0..15)
  __device__ static inline uint32_t pack2(float lo, float hi) {
    return (uint32_t)from_f32(lo) | ((uint32_t)from_f32(hi) << 16);
  }
};
struct TBF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kVec = 8;
  __device__ static inline float to_f32(storage x) {
    return __builtin_bit_cast(float, (uint32_t)x << 16);
  }
  __device__ static inline storage from_f32(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    return (uint32_t)from_f32(lo) | ((uint32_t)from_f32(hi) << 16);
  }
  // p = hi + lo with hi = bf16(p) and lo = bf16(p - hi): a matrix product with
  // both halves carries p to ~16 significant bits instead of 8.
  __device__ static inline void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const storage ha = from_f32(a), hb = from_f32(b);
    hi = (uint32_t)ha | ((uint32_t)hb << 16);
    lo = pack2(a - to_f32(ha), b - to_f32(hb));
  }
};

// Scalar reinterpretation.  Arguments are taken by value: a bit-cast applied
// directly to an element of an ext_vector_type expression does not select the
// element on this compiler, so vector elements are always copied out first.
__device__ inline float as_float(uint32_t x) { return __uint_as_float(x); }
__device__ inline uint32_t as_uint(float x) { return __float_as_uint(x); }

// ---------------------------------------------------------------------------
// matrix-core wrappers (operands as raw dwords)
// ---------------------------------------------------------------------------
__device__ inline f32x16 mma32(TBF16, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline f32x16 mma32(TF16, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// fp32: one 16-byte vector holds the operands of four consecutive k-steps
__device__ inline f32x16 mma32(TF32, u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(as_float(a[t]), as_float(b[t]), c, 0, 0, 0);
  return c;
}

// 16x16x16: A m = l%16, k = 4*(l/16)+e; B n = l%16, k = 4*(l/16)+e (e = 0..3)
__device__ inline f32x4 mma16k16(TBF16, u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                   __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
}
__device__ inline f32x4 mma16k16(TF16, u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                               __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

__device__ inline f32x4 mma16(TBF16, u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mma16(TF16, u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mma16(TF32, u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(as_float(a[t]), as_float(b[t]), c, 0, 0, 0);
  return c;
}

// Two fp32 values -> one dword of two 16-bit values (round to nearest even;
// v_cvt_pk_{bf16,f16}_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t cvt_pk(TBF16, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ inline uint32_t cvt_pk(TF16, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------
__device__ inline u32x4 ldg16(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ inline u32x4 ldg16_cached(const void* p) { return *(const u32x4*)p; }

// Mask entry idx (element index from the caller's strides) as an additive
// term: the fp32 value, or 0 / -inf for a boolean (uint8) mask.
__device__ inline float mask_val(const void* mask, int is_bool, int64_t idx) {
  if (is_bool) return ((const uint8_t*)mask)[idx] ? 0.f : kNegInf;
  return ((const float*)mask)[idx];
}

// Real rows of batch b along an extent of L rows: lens[b] clamped to [0, L],
// or L when there is no per-batch length array.
__device__ inline int batch_len(const int32_t* lens, int b, int L) {
  return lens ? min(max(lens[b], 0), L) : L;
}

// Per-lane offset of a direct load that must read nothing (a chunk past the
// real head dim): 1 GiB, above every tile's byte count (at most 64 rows of
// 8 MiB), so the range check returns zero; with a tile's scalar offset added
// it stays below 2^31.
constexpr uint32_t kNoLoad = 0x40000000u;

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// Direct HBM -> LDS load: lane l's 16 bytes at voff land at lds + 16*l (lds is
// wave-uniform, written to M0).  Completion is tracked by vmcnt only.
__device__ inline void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                      uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(lds), 16, (int)voff, (int)soff, 0, 0);
}

// The same direct load, issued so that the compiler does not track it: its
// wait-count pass otherwise cannot tell that a later LDS read of a different
// ring stage is independent of the load and waits for every load in flight
// (vmcnt(0)) before that read, which serialises the prefetch.  Callers order
// it themselves: wait_vmcnt<> then lds_barrier() before reading the stage.
// The descriptor is built by hand (base, stride 0, num_records, the same
// format word as make_rsrc); M0 holds the wave-uniform LDS destination, set
// at least one wait state before the load.
// base, bytes, soff and lds_addr are wave-uniform; they are pinned to scalar
// registers (readfirstlane) so the "s" operands never see a vector register.
// A vector instruction that writes a scalar register needs five wait states
// before a buffer instruction reads it, and the compiler does not see inside
// the asm, so it opens with s_nop 4 (which also covers the M0 write).
__device__ inline void dma16(const void* base, uint32_t bytes, uint32_t lds_addr, uint32_t voff,
                             uint32_t soff) {
  const uint64_t a = (uint64_t)base;
  const u32x4 rsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
                      (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
  soff = (uint32_t)__builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr));
}
// A wave-uniform pointer pinned to scalar registers, so that addresses built
// from it stay in scalar arithmetic.
template <class P>
__device__ inline P* uniform_ptr(P* ptr) {
  const uint64_t a = (uint64_t)ptr;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (P*)(lo | (hi << 32));
}
// LDS byte address of a pointer into shared memory
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

// Workgroup barrier without the implied memory fence of __syncthreads: the
// fence would wait for every outstanding load (vmcnt(0)), including direct
// LDS loads of later tiles.  Callers wait for what they need explicitly.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane r names 4 consecutive
// 16-bit values (a "row"); lane r receives element (r % 4) of the rows named by
// lanes r/4, 4 + r/4, 8 + r/4, 12 + r/4.  With lane r pointing at
// X[k0 + r/4][c0 + 4*(r%4)] of a row-major 16-bit matrix X, lane r receives
// X[k0 + e][c0 + r] for e = 0..3: a 4 x 16 block read transposed.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline u32x2 lds_read_tr16(const void* p) {
  // address-space cast (not an integer cast): generic LDS address -> LDS offset
  auto lp = (__attribute__((address_space(3))) s16x4*)(const_cast<void*>(p));
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}
__device__ inline u32x4 lds_read16(const void* p) { return *(const u32x4*)p; }
__device__ inline void lds_write16(void* p, u32x4 v) { *(u32x4*)p = v; }
__device__ inline void lds_write8(void* p, u32x2 v) { *(u32x2*)p = v; }

// byte-select of two dwords: result bytes = sel over {b (bytes 0..3), a (bytes 4..7)}
__device__ inline uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(a, b, sel);
}
// low / high 16-bit halves of (b, a) joined: lo(b) | lo(a) << 16, hi(b) | hi(a) << 16
__device__ inline uint32_t join_lo(uint32_t a, uint32_t b) { return perm(a, b, 0x05040100u); }
__device__ inline uint32_t join_hi(uint32_t a, uint32_t b) { return perm(a, b, 0x07060302u); }

// Workgroups are dispatched round-robin over the 8 XCDs (block i -> XCD i % 8),
// each with its own L2.  Map block i to work item w so that every XCD walks a
// contiguous range of the work list (a bijection on [0, n)).
constexpr int kNumXcd = 8;
__device__ inline int xcd_work_index(int i, int n) {
  const int x = i % kNumXcd, local = i / kNumXcd;
  const int q = n / kNumXcd, r = n % kNumXcd;
  return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

// Prefill workgroup -> (query tile, batch*head).  Causal: tiles differ in
// work, so the heaviest (last) query tiles go first; when the head count is a
// multiple of 8, head h lives on XCD h % 8 (its K / V stay in one L2) and each
// XCD runs its heads' tiles heaviest first.  Non-causal: tiles are equal, each
// XCD walks whole heads in turn.
__device__ inline void prefill_tile(int i, int n, int nqt, int nbh, bool causal, int& qt, int& bh) {
  if (causal) {
    if (nbh % kNumXcd == 0) {
      const int per = nbh / kNumXcd, local = i / kNumXcd;
      qt = nqt - 1 - local / per;
      bh = i % kNumXcd + kNumXcd * (local % per);
    } else {
      qt = nqt - 1 - i / nbh;
      bh = i % nbh;
    }
  } else {
    const int w = xcd_work_index(i, n);
    qt = w % nqt;
    bh = w / nqt;
  }
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine each lane with lane l ^ 32 (v_permlane32_swap: the two halves of
// the wave trade places, no LDS round trip).
__device__ inline float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_uint(v), as_uint(v), false, false);
  return fmaxf(as_float(r[0]), as_float(r[1]));
}
__device__ inline float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_uint(v), as_uint(v), false, false);
  return as_float(r[0]) + as_float(r[1]);
}

// v itself, as a value the compiler cannot trace back: what a loop derives
// from the result is computed where it is used instead of being kept (or,
// short of registers, spilled to scratch and reloaded) across iterations
__device__ inline int fresh(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
// A fresh copy of the lane index.  The mask restores what the compiler knew
// of it (0..63), so that swizzled LDS offsets derived from it still fold into
// per-lane bases plus immediate offsets.
__device__ inline int fresh_lane(int lane) { return fresh(lane) & 63; }

// exchange with lane l ^ 32 (the other half of the wave)
__device__ inline float xor32(float v) { return __shfl_xor(v, 32, 64); }
__device__ inline float xor16(float v) { return __shfl_xor(v, 16, 64); }

}  // namespace sdpa
