// Prefill / full self-attention forward for gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V with the online softmax of the
// rustytorch "flash_attention.metal" page (forward kernel, "Online softmax
// update": running max m, running sum l, O rescaled by exp(m_old - m_new)),
// never forming the Lq x Lk score matrix in memory, and finishes as its
// "Write final output" step (O = acc / l, LSE = m + log l) extended with the
// sink term and the empty-row convention of the C ABI header.
//
// Work decomposition: one workgroup of 4 waves per (query tile of 128 rows,
// query head, batch).  Each wave owns 32 query rows.  The key range is
// streamed in tiles of BN keys through LDS: K row-major, V transposed so the
// P.V product can read it as a matrix-core operand.  The next tile is
// prefetched into registers while the current one is consumed.
//
// Per wave and tile the products are formed transposed,
//     S^T (keys x queries) = K . Q^T      and      O^T += V^T . P^T,
// so that in the 32x32 accumulator layout every lane holds the scores of ONE
// query (lane % 32) for 16 keys of each 32-key block: the row max and row sum
// are in-lane reductions plus one exchange with lane ^ 32, and the lane's
// probabilities are directly the B operand of the P.V product.
#include <type_traits>

#include "sdpa_device.hpp"
#include "sdpa_internal.hpp"

namespace sdpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup

template <class T, int D>
struct PrefillCfg {
  static constexpr int ES = T::kBytes;
  static constexpr int VEC = T::kVec;            // elements per 16-byte chunk
  static constexpr int NCH = D / VEC;            // chunks per row
  static constexpr bool F32 = (ES == 4);
  // keys per tile: keep the K + V^T tile near 32 KiB
  static constexpr int BN = F32 ? (D == 128 ? 32 : 64) : (D == 128 ? 64 : 128);
  static constexpr int NKB = BN / 32;            // 32-key blocks per tile
  static constexpr int KP = D * ES + 16;         // K row pitch (bytes), padded
  static constexpr int VP = BN * ES + 16;        // V^T row pitch (bytes), padded
  static constexpr int K_BYTES = BN * KP;
  static constexpr int V_BYTES = D * VP;
  static constexpr int NQ = D * ES / 32;         // 16-byte Q vectors per lane
  static constexpr int K_IT = BN * NCH / kThreads;        // K chunks per thread
  static constexpr int V_IT = (BN / 4) * NCH / kThreads;  // 4-key V groups per thread
  static constexpr int NMB = D / 32;             // 32-row blocks of O^T
  static_assert(K_IT >= 1 && BN * NCH % kThreads == 0, "K tile split");
  static_assert(V_IT >= 1 && (BN / 4) * NCH % kThreads == 0, "V tile split");
};

// V^T row (in LDS) holding head-dim element d = VEC*c + e of chunk c.
// Rows are permuted so that the 16 lanes writing chunk c = 0..15 of one
// element e hit consecutive rows (no bank conflicts on the transposing
// stores); the matrix-core row m of block mb reads LDS row 32*mb + m.
template <int NCH>
__device__ constexpr int vt_row(int c, int e) { return c + NCH * e; }
template <int NCH, int VEC>
__device__ constexpr int vt_row_to_d(int rho) { return VEC * (rho % NCH) + rho / NCH; }

// Position of key group kg (4 keys, within a 32-key block) in the V^T row.
// 16-bit: the P.V k-slots of lane half g are keys {16t + 8a + 4g + c}, stored
// contiguously at slot 16t + 8g + 4a + c (swap bits 0 and 1 of kg).
// fp32: natural order.
template <bool F32>
__device__ constexpr int vt_group_slot(int kg) {
  return F32 ? kg : ((kg & ~3) | ((kg & 1) << 1) | ((kg & 2) >> 1));
}

// fp32 inputs: fp32 matrix cores (32x32x2), V transposed into LDS by the
// loading threads.
template <class T, int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 2) void prefill_f32_kernel(AttnParams p) {
  using C = PrefillCfg<T, D>;
  using S = typename T::storage;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::K_BYTES + C::V_BYTES];
  uint8_t* Ks = smem;
  uint8_t* Vt = smem + C::K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // heaviest (last) query tiles first: with the causal mask their key range
  // is the longest
  const int nqt = (p.Lq + kBM - 1) / kBM;
  int qt, bh;
  prefill_tile((int)blockIdx.x, (int)gridDim.x, nqt, p.B * p.Hq, CAUSAL, qt, bh);
  const int b = bh / p.Hq;
  const int hq = bh % p.Hq;
  const int hk = hq / p.group;

  const int i0 = qt * kBM;            // first query row of the workgroup
  const int iw = i0 + 32 * wave;      // first query row of this wave
  const int my_i = iw + l32;          // this lane's query row
  // real query rows and keys of this batch; bottom-right causal offset
  const int lq = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_q, b, p.Lq));
  const int lk = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_k, b, p.Lk));
  const int coff = lk - lq;

  const S* qp = (const S*)p.q + b * p.qs[0] + hq * p.qs[1];
  const S* kp = (const S*)p.k + b * p.ks[0] + hk * p.ks[1];
  const S* vp = (const S*)p.v + b * p.vs[0] + hk * p.vs[1];

  // ---- Q row of this lane as B operands: vector s holds chunk 2s + g ----
  u32x4 qreg[C::NQ];
  {
    const bool ok = my_i < lq;
    const S* row = qp + (int64_t)(ok ? my_i : 0) * p.qs[2];
    const int nqk = p.Dqk / C::VEC;  // real chunks of a q / k row; the rest is zero
#pragma unroll
    for (int s = 0; s < C::NQ; ++s) {
      u32x4 v = ldg16_cached(row + min(2 * s + g, nqk - 1) * C::VEC);
      qreg[s] = ok && 2 * s + g < nqk ? v : u32x4{0, 0, 0, 0};
    }
  }

  // key range of the workgroup's real rows (bottom-right causal)
  int kend = i0 < lq ? lk : 0;
  if (CAUSAL) kend = min(kend, min(i0 + kBM, lq) + coff);
  const int ntiles = kend > 0 ? (kend + C::BN - 1) / C::BN : 0;
  const int wave_last_key = CAUSAL ? iw + 31 + coff : lk - 1;
  // bf16 probabilities carry 8 significant bits; rows that average few keys
  // would show that rounding directly in O, so such workgroups feed P.V with
  // P = hi + lo (two bf16 products).  Many-key rows average it away.
  const bool split_p = std::is_same<T, TBF16>::value && (MASK || kend <= 1024);

  f32x16 acc[C::NMB];
#pragma unroll
  for (int mb = 0; mb < C::NMB; ++mb) acc[mb] = f32x16{};
  float m_run = kNegInf;  // running max (log2 units)
  float l_run = 0.f;      // running sum, this lane's half of the keys

  // ---- register prefetch of one K / V tile ----
  u32x4 kpre[C::K_IT];
  u32x4 vpre[C::V_IT][4];
  auto prefetch = [&](int j0) {
#pragma unroll
    for (int it = 0; it < C::K_IT; ++it) {
      const int u = tid + kThreads * it;
      const int key = u / C::NCH, c = u % C::NCH;
      const int j = j0 + key;
      kpre[it] = j < lk && c * C::VEC < p.Dqk ? ldg16_cached(kp + (int64_t)j * p.ks[2] + c * C::VEC)
                                              : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < C::V_IT; ++it) {
      const int u = tid + kThreads * it;
      const int kg = u / C::NCH, c = u % C::NCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * kg + r;
        vpre[it][r] = j < lk && c * C::VEC < p.Dv ? ldg16_cached(vp + (int64_t)j * p.vs[2] + c * C::VEC)
                                                  : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::K_IT; ++it) {
      const int u = tid + kThreads * it;
      const int key = u / C::NCH, c = u % C::NCH;
      lds_write16(Ks + key * C::KP + c * 16, kpre[it]);
    }
#pragma unroll
    for (int it = 0; it < C::V_IT; ++it) {
      const int u = tid + kThreads * it;
      const int kg = u / C::NCH, c = u % C::NCH;
      const int slot4 = (kg & ~7) | vt_group_slot<C::F32>(kg & 7);  // within 32-key blocks
      if constexpr (C::F32) {
        // 4 keys x 4 elements: element e of the 4 keys -> one 16-byte store
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 w = {vpre[it][0][e], vpre[it][1][e], vpre[it][2][e], vpre[it][3][e]};
          lds_write16(Vt + vt_row<C::NCH>(c, e) * C::VP + slot4 * 16, w);
        }
      } else {
        // 4 keys x 8 elements: element e of the 4 keys -> one 8-byte store
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dw = e >> 1;
          uint32_t lo, hi;
          if (e & 1) {
            lo = join_hi(vpre[it][1][dw], vpre[it][0][dw]);
            hi = join_hi(vpre[it][3][dw], vpre[it][2][dw]);
          } else {
            lo = join_lo(vpre[it][1][dw], vpre[it][0][dw]);
            hi = join_lo(vpre[it][3][dw], vpre[it][2][dw]);
          }
          lds_write8(Vt + vt_row<C::NCH>(c, e) * C::VP + slot4 * 8, u32x2{lo, hi});
        }
      }
    }
  };

  if (ntiles > 0) prefetch(0);

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * C::BN;
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();  // tile visible
    if (t + 1 < ntiles) prefetch(j0 + C::BN);

    if (j0 > wave_last_key) continue;  // nothing visible to this wave's rows
    const bool edge = (j0 + C::BN > lk) || (CAUSAL && j0 + C::BN - 1 > iw + coff);

    // ---- S^T = K . Q^T for the tile ----
    f32x16 sc[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      sc[kb] = f32x16{};
      const uint8_t* krow = Ks + (32 * kb + l32) * C::KP + g * 16;
#pragma unroll
      for (int s = 0; s < C::NQ; ++s) sc[kb] = mma32(T{}, lds_read16(krow + s * 32), qreg[s], sc[kb]);
    }

    // ---- scale, mask, running max ----
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sc[kb][r] * p.scale_log2;
        const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (MASK) {
          const int ii = my_i < lq ? my_i : lq - 1;
          const int jj = j < lk ? j : lk - 1;
          x += kLog2e * mask_val(p.mask, p.mask_bool,
                                 b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] + (int64_t)jj * p.ms[3]);
        }
        if (edge) {
          const bool vis = (j < lk) && (!CAUSAL || j <= my_i + coff);
          x = vis ? x : kNegInf;
        }
        sc[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float corr = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= corr;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) acc[mb] *= corr;

    // ---- P = exp2(S - m), row sum, O^T += V^T . P^T ----
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(sc[kb][r] - m_use);
        sc[kb][r] = pr;
        l_run += pr;
      }
      if constexpr (C::F32) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          u32x4 pb = {as_uint(sc[kb][4 * u + 0]),
                      as_uint(sc[kb][4 * u + 1]),
                      as_uint(sc[kb][4 * u + 2]),
                      as_uint(sc[kb][4 * u + 3])};
          const uint8_t* vcol = Vt + l32 * C::VP + (32 * kb + 8 * u + 4 * g) * 4;
#pragma unroll
          for (int mb = 0; mb < C::NMB; ++mb)
            acc[mb] = mma32(T{}, lds_read16(vcol + 32 * mb * C::VP), pb, acc[mb]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint8_t* vcol = Vt + l32 * C::VP + (32 * kb + 16 * u + 8 * g) * 2;
          if constexpr (std::is_same<T, TBF16>::value) {
            if (split_p) {
              u32x4 hi, lo;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                uint32_t h, l;
                T::split2(sc[kb][8 * u + 2 * e], sc[kb][8 * u + 2 * e + 1], h, l);
                hi[e] = h;
                lo[e] = l;
              }
#pragma unroll
              for (int mb = 0; mb < C::NMB; ++mb) {
                const u32x4 va = lds_read16(vcol + 32 * mb * C::VP);
                acc[mb] = mma32(T{}, va, hi, acc[mb]);
                acc[mb] = mma32(T{}, va, lo, acc[mb]);
              }
              continue;
            }
          }
          u32x4 pb = {T::pack2(sc[kb][8 * u + 0], sc[kb][8 * u + 1]),
                      T::pack2(sc[kb][8 * u + 2], sc[kb][8 * u + 3]),
                      T::pack2(sc[kb][8 * u + 4], sc[kb][8 * u + 5]),
                      T::pack2(sc[kb][8 * u + 6], sc[kb][8 * u + 7])};
#pragma unroll
          for (int mb = 0; mb < C::NMB; ++mb)
            acc[mb] = mma32(T{}, lds_read16(vcol + 32 * mb * C::VP), pb, acc[mb]);
        }
      }
    }
  }

  // ---- epilogue: normalise, sink, LSE.  Padding rows see no key. ----
  float l_tot = l_run + xor32(l_run);
  if (my_i >= lq) {
    m_run = kNegInf;
    l_tot = 0.f;
  }
  float M = m_run;
  float Ltot = l_tot;
  if (p.sinks) {
    const float sk = p.sinks[hq] * kLog2e;
    M = fmaxf(m_run, sk);
    if (M != kNegInf) {
      Ltot = l_tot * fast_exp2(m_run - M) + fast_exp2(sk - M);
    }
  }
  float scale_o = 0.f;
  float lse = kNegInf;
  if (M != kNegInf && Ltot > 0.f) {
    const float inv = 1.f / Ltot;
    scale_o = (p.sinks ? fast_exp2(m_run - M) : 1.f) * inv;
    lse = (M + fast_log2(Ltot)) * kLn2;
  }
  if (my_i < p.Lq) {
    S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)my_i * p.os[2];
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rho = 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
        const int d = vt_row_to_d<C::NCH, C::VEC>(rho);
        if (d < p.Dv) orow[d] = T::from_f32(acc[mb][r] * scale_o);
      }
    }
    if (p.lse && g == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Lq + my_i] = lse;
  }
}


// ---------------------------------------------------------------------------
// 16-bit inputs (fp16 / bf16)
// ---------------------------------------------------------------------------
template <int D, int NW>
struct Cfg16 {
  static constexpr int BN = 64;                 // keys per tile
  static constexpr int NKB = BN / 32;           // 32-key blocks per tile
  static constexpr int RB = D * 2;              // row bytes (unpadded)
  static constexpr int NCH = D / 8;             // 16-byte chunks per row
  static constexpr int TILE = BN * RB;          // bytes of one K (or V) tile
  static constexpr int LINES = TILE / 1024;     // 1 KiB direct-load lines per tile
  static constexpr int LPW = LINES / NW;        // lines per wave per tile (K or V)
  static constexpr int STEP_ROWS = NW * 64 / NCH;  // rows between a wave's lines
  static constexpr int NQ = D / 16;             // 16-byte Q vectors per lane
  static constexpr int NMB = D / 32;            // 32-row blocks of O^T
  static_assert(LINES % NW == 0, "tile lines");
  // lines i and i + KVAR of a wave share the K swizzle (period 16 rows)
  static constexpr int KVAR = STEP_ROWS % 16 == 0 ? 1 : 16 / STEP_ROWS;
  static_assert(KVAR == 1 || KVAR == 2, "swizzle period");
  static_assert(STEP_ROWS % 4 == 0, "V swizzle period");
};

// The reference max is only moved (and O, l rescaled) when a row's tile max
// exceeds it by more than this many log2 units; probabilities then stay
// below 2^8, and O = sum(p v) / sum(p) is unchanged by which max is used.
constexpr float kRescaleSlack = 8.f;

// Fast pass of the pre-scaled fp16 form (steady tiles only): no row max is
// taken before the exponentials; each tile's row sum is checked afterwards.
// Every probability is at most that sum, so a finite sum means each was a
// finite fp16 value.  A row sum of kFastSumMax or more moves the reference
// max by its log2; one that is not finite sends the workgroup through the
// tiles again with the max taken before every exponential.
constexpr float kFastSumMax = 16384.f;

// 16-byte chunk swizzles of the unpadded LDS rows (low chunk bits ^= f(row)):
// K: the Q.K^T operand read touches 16 consecutive rows in one chunk;
// V: a transposed read touches 8 rows x 4 consecutive chunks.
template <int NCH>
__device__ constexpr int swz_k(int row) { return NCH >= 16 ? (row & 15) : ((row >> 1) & 7); }
template <int NCH>
__device__ constexpr int swz_v(int row) { return NCH >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// Two packed fp16 values.  By value: a bit-cast applied directly to an
// element of an ext_vector_type expression does not select the element on
// this compiler.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ inline h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }

// max(a, b) over this lane and lane ^ 32, written out so that no operand is
// first quietened (fmaxf would add one move per operand): the two halves of
// the wave trade places with v_permlane32_swap.
__device__ inline float max2_xor32(float a, float b) {
  float m, t;
  asm volatile(
      "v_max_f32 %0, %2, %3\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1"
      : "=&v"(m), "=&v"(t)
      : "v"(a), "v"(b));
  return m;
}

// Row-sum contribution of one packed pair of probabilities, in fp32: a v_dot2
// of the packed (rounded) values P.V multiplies against ones.  The steady
// loop of steady_slots picks its own form per type and masking.
__device__ inline float row_sum2(TF16, uint32_t pk, float acc) {
  return __builtin_amdgcn_fdot2(as_h2(pk), as_h2(0x3C003C00u), acc, false);
}
__device__ inline float row_sum2(TBF16, uint32_t pk, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                         acc, false);
}

// Lead, in slots, of a matrix-core operand's LDS read over its product.  Two
// slots (two products, 64+ cycles) cover the LDS latency; each further slot
// holds 4 more registers per lane, which at three waves per SIMD (D = 64)
// only pushes values into scratch (measured: 2 is 0.9 % faster than 4 on the
// DiT shape, 0.7 % on causal bf16 D = 128).
#ifndef SDPA_PF_WIN
#define SDPA_PF_WIN 2
#endif

// Per wave (32 queries) and tile (64 keys), software-pipelined:
//   S(t+1) = K(t+1) . Q^T  on the matrix cores  ||  P(t) = exp2(S(t) c - m)  on the VALU
//   O^T   += V(t)^T . P(t)^T on the matrix cores  ||  row max of S(t+1) on the VALU
// (the pre-scaled form's fast pass drops the row max and checks each tile's
// row sum instead, see kFastSumMax).
// K and V tiles arrive by direct buffer -> LDS loads into two-stage rings, one
// tile ahead, with one fence-free barrier per tile.  V^T is read with
// ds_read_b64_tr_b16.  Interior tiles (every key visible to the whole
// workgroup, no mask) skip per-element masking.
// REL (fp16 only): Q is pre-multiplied by the exponent scale and the scores
// are kept relative to the reference max (below); the host selects it for
// calls without a log-sum-exp output.
template <class T, int D, bool CAUSAL, bool MASK, int NW, bool REL>
__device__ __forceinline__ void prefill16_body(const AttnParams& p) {
  using C = Cfg16<D, NW>;
  constexpr int BM = 32 * NW;  // query rows per workgroup
  using S = uint16_t;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * C::TILE];
  uint8_t* const Kring = smem;               // stages 0, 1
  uint8_t* const Vring = smem + 2 * C::TILE;  // stages 0, 1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int nqt = (p.Lq + BM - 1) / BM;
  // Work item: a query tile of the work list, or (non-causal, no mask) one
  // key piece of a tail tile.  The tiles' count per compute unit sets the
  // kernel's time (each runs about as long as the others), so the tiles past
  // the last multiple of the compute units run as pieces spread over several
  // units, and a merge kernel combines their partials.
  int item = (int)blockIdx.x, piece = -1;
  if constexpr (!CAUSAL && !MASK) {
    const int first = p.tiles - p.tail_tiles;
    if (item >= first) {
      piece = (item - first) % p.tail_k;
      item = first + (item - first) / p.tail_k;
    }
  }
  int qt, bh;
  prefill_tile(item, p.tiles, nqt, p.B * p.Hq, CAUSAL, qt, bh);
  const int b = bh / p.Hq;
  const int hq = bh % p.Hq;
  const int hk = hq / p.group;

  const int i0 = qt * BM;
  const int iw = i0 + 32 * wave;
  const int my_i = iw + l32;
  // real query rows and keys of this batch (a piece: its own key range, from
  // key kbeg on); bottom-right causal offset
  const int lq = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_q, b, p.Lq));
  const int kbeg = piece >= 0 ? piece * p.tail_chunk : 0;
  const int lk = __builtin_amdgcn_readfirstlane(
      piece >= 0 ? min(p.Lk - kbeg, p.tail_chunk) : batch_len(p.seqlens_k, b, p.Lk));
  const int coff = lk - lq;

  // exponent scale c = |scale| log2(e); a negative scale is moved into Q.
  // REL (fp16, c <= 1, no log-sum-exp output): Q is multiplied by c once (it
  // cannot overflow; each element takes one more rounding, 2^-11 relative, so
  // a score moves by at most 2^-11 c sum_d |q_d k_d|), the matrix cores
  // deliver c S itself and the steady loop, which also starts its score
  // accumulators at -m, feeds the exponential without any per-score
  // arithmetic.  Calls that return the log-sum-exp keep the exact fp32 scale:
  // that error would reach the LSE undamped at large logits.  (bf16 would
  // round c Q to 8 bits, which shows in rows that average few keys, so bf16
  // never takes this form.)  cs is the factor the scores still owe.
  static_assert(!REL || std::is_same<T, TF16>::value, "pre-scaled Q is fp16 only");
  constexpr bool kRel = REL;
  const float c = fabsf(p.scale_log2);
  const bool pre = kRel && c <= 1.f;
  const float cs = pre ? 1.f : c;
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  u32x4 qreg[C::NQ];
  {
    const bool ok = my_i < lq;
    const S* row = (const S*)p.q + b * p.qs[0] + hq * p.qs[1] + (int64_t)(ok ? my_i : 0) * p.qs[2];
    const int nqk = p.Dqk / 8;  // real 16-byte chunks of a q / k row; the rest is zero
#pragma unroll
    for (int s = 0; s < C::NQ; ++s) {
      u32x4 v = ldg16_cached(row + min(2 * s + g, nqk - 1) * 8);
      v ^= qflip;
      if (pre) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = v[e];
          v[e] = cvt_pk(T{}, T::to_f32((uint16_t)(w & 0xffffu)) * c, T::to_f32((uint16_t)(w >> 16)) * c);
        }
      }
      qreg[s] = ok && 2 * s + g < nqk ? v : u32x4{0, 0, 0, 0};
    }
  }

  // key range of the workgroup's real rows (bottom-right causal)
  int kend = i0 < lq ? lk : 0;
  if (CAUSAL) kend = min(kend, min(i0 + BM, lq) + coff);
  const int ntiles = kend > 0 ? (kend + C::BN - 1) / C::BN : 0;
  // tiles [0, n_int) have every key visible to every row of the workgroup
  int n_int = 0;
  if (!MASK) {
    int full = lk;
    if (CAUSAL) full = min(full, i0 + 1 + coff);
    n_int = full > 0 ? min(ntiles, full / C::BN) : 0;
  }
  // bf16 probabilities carry 8 significant bits; rows that average few keys
  // would show that rounding directly in O, so such workgroups feed P.V with
  // P = hi + lo (two bf16 products).  Rows past 256 keys average it away
  // (the row sum adds the same rounded probabilities, so only the relative
  // weights are perturbed, by ~2^-9 / sqrt(keys)).
  const bool split_p = std::is_same<T, TBF16>::value && (MASK || kend <= 256);

  // ---- direct buffer -> LDS loads.  Wave w fills lines w, w + NW, ... of a
  // tile; line i of a wave sits i * STEP_ROWS rows below line 0 and both
  // swizzles repeat every 16 rows: one per-lane offset plus a uniform step.
  const S* kbase = uniform_ptr((const S*)p.k + b * p.ks[0] + hk * p.ks[1] + (int64_t)kbeg * p.ks[2]);
  const S* vbase = uniform_ptr((const S*)p.v + b * p.vs[0] + hk * p.vs[1] + (int64_t)kbeg * p.vs[2]);
  // A lane whose chunk lies past the real head dim loads nothing (kNoLoad).
  uint32_t koff[C::KVAR], voff;
  {
    const int pos = wave * 64 + lane;  // 16-byte slot of line 0
    const int row = pos / C::NCH, pch = pos % C::NCH;
#pragma unroll
    for (int k = 0; k < C::KVAR; ++k) {
      const int rk = row + k * C::STEP_ROWS;  // a line KVAR steps further repeats it
      const int lch = pch ^ swz_k<C::NCH>(rk);
      koff[k] = lch * 8 < p.Dqk ? (uint32_t)(row * p.ks[2] * 2 + lch * 16) : kNoLoad;
    }
    const int lch = pch ^ swz_v<C::NCH>(row);
    voff = lch * 8 < p.Dv ? (uint32_t)(row * p.vs[2] * 2 + lch * 16) : kNoLoad;
  }
  const uint32_t krow = __builtin_amdgcn_readfirstlane((uint32_t)(p.ks[2] * 2));
  const uint32_t vrow = __builtin_amdgcn_readfirstlane((uint32_t)(p.vs[2] * 2));
  const uint32_t kstep = __builtin_amdgcn_readfirstlane(C::STEP_ROWS * krow);
  const uint32_t vstep = __builtin_amdgcn_readfirstlane(C::STEP_ROWS * vrow);
  // bytes of a tile that hold real keys: rows from lk on (and, since the row
  // stride is at least the real row, everything past the last real row) read
  // as zero
  auto tile_bytes = [&](int j0, uint32_t rowb, uint32_t real_rb) -> uint32_t {
    const int rows = min(lk - j0, C::BN);
    return (uint32_t)(rows - 1) * rowb + real_rb;
  };
  // a full tile's byte count, once (uniform)
  const uint32_t kfull = __builtin_amdgcn_readfirstlane((C::BN - 1) * krow + 2 * p.Dqk);
  const uint32_t vfull = __builtin_amdgcn_readfirstlane((C::BN - 1) * vrow + 2 * p.Dv);
  auto issue = [&](const S* base, int64_t rs, uint32_t rowb, uint32_t real_rb, uint32_t full, const uint32_t* off,
                   int noff, uint32_t step, uint8_t* st, int t) {
    const int j0 = t * C::BN;
    const S* tb = base + (int64_t)j0 * rs;
    const uint32_t nb = j0 + C::BN <= lk ? full : tile_bytes(j0, rowb, real_rb);
    const uint32_t la = lds_addr(st) + wave * 1024;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) dma16(tb, nb, la + NW * i * 1024, off[i % noff], i * step);
  };
  auto issue_k = [&](int t, uint8_t* st) {
    issue(kbase, p.ks[2], krow, 2 * p.Dqk, kfull, koff, C::KVAR, kstep, st, t);
  };
  auto issue_v = [&](int t, uint8_t* st) { issue(vbase, p.vs[2], vrow, 2 * p.Dv, vfull, &voff, 1, vstep, st, t); };

  // ---- per-lane LDS read offsets
  const uint32_t k_lane = l32 * C::RB;                 // + (32 kb) rows
  const int k_swz = swz_k<C::NCH>(l32);
  const int r16 = lane & 15, dh = (lane >> 4) & 1;
  const int v_row = 4 * g + (r16 >> 2);                // + (32 kb + 16 u + 8 a) rows
  const int v_swz = swz_v<C::NCH>(v_row);
  const uint32_t v_lane = v_row * C::RB + (r16 & 1) * 8;
  const int v_ch = 2 * dh + ((r16 >> 1) & 1);          // + 4 mb

  f32x16 acc[C::NMB];
#pragma unroll
  for (int mb = 0; mb < C::NMB; ++mb) acc[mb] = f32x16{};
  float m_run = kNegInf;   // reference max of the scaled scores (log2 units)
  float l_run = 0.f;       // running sum over this lane's half of the keys

  // At D = 256 (one wave per SIMD, every tile on this path) both product
  // loops below read each LDS operand two products ahead, with a fence on
  // each side of every product: with no other wave to cover it, a read issued
  // just before its product left every product waiting out the LDS latency
  // (bf16 non-causal 732 -> 650 us, causal 396 -> 352 us, fp16 678 -> 666
  // us; three ahead measured the same within 2 %).
  constexpr bool kReadAhead = D >= 256;
  auto qk = [&](const uint8_t* Kst, f32x16* sc) {
    const uint8_t* Ks = Kst + k_lane;
    if constexpr (kReadAhead) {
      auto kread = [&](int i) {  // i = kb * NQ + s
        return lds_read16(Ks + 32 * (i / C::NQ) * C::RB + (((2 * (i % C::NQ) + g) ^ k_swz) * 16));
      };
      constexpr int N = C::NKB * C::NQ;
      constexpr int LA = 2;
      u32x4 kr[LA];
#pragma unroll
      for (int j = 0; j < LA; ++j) kr[j] = kread(j < N ? j : 0);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int kb = i / C::NQ, s = i % C::NQ;
        const u32x4 ka = kr[i % LA];
        if (i + LA < N) kr[i % LA] = kread(i + LA);
        __builtin_amdgcn_sched_barrier(0);
        sc[kb] = mma32(T{}, ka, qreg[s], s == 0 ? f32x16{} : sc[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < C::NQ; ++s)
          sc[kb] = mma32(T{}, lds_read16(Ks + 32 * kb * C::RB + (((2 * s + g) ^ k_swz) * 16)), qreg[s], sc[kb]);
      }
    }
  };
  // row max of tile t (scaled log2 units), masking first on edge tiles
  auto tile_max = [&](int t, f32x16* sc, auto edge_tag) -> float {
    constexpr bool EDGE = decltype(edge_tag)::value;
    float mx;
    if constexpr (!EDGE) {
      mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = max_xor32(mx) * cs;
    } else {
      const int j0 = t * C::BN;
      const int ii = my_i < lq ? my_i : lq - 1;
      mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          float x = sc[kb][r] * cs;
          if (MASK) {
            const int jj = j < lk ? j : lk - 1;
            x += kLog2e * mask_val(p.mask, p.mask_bool,
                                 b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] + (int64_t)jj * p.ms[3]);
          }
          const bool vis = (j < lk) && (!CAUSAL || j <= my_i + coff);
          x = vis ? x : kNegInf;
          sc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = max_xor32(mx);
    }
    return mx;
  };
  // move the reference max when some row's tile max exceeds it by the slack
  auto update_max = [&](float mx) {
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = m_new > m_run ? fast_exp2(m_run - m_new) : 1.f;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) acc[mb] *= corr;
      l_run *= corr;
      m_run = m_new;
    }
  };
  // P = exp2(S cs - m) (interior) or exp2(S - m) (edge, already scaled), left
  // in sc and packed as the B operands of P.V: k-step u of block kb <->
  // accumulator rows 8u..8u+7.  The row sum adds the packed values (bf16:
  // the rounded values P.V multiplies).
  auto probs = [&](f32x16* sc, u32x4 (&pk)[C::NKB][2], auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const float m_use = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sc[kb][r] = EDGE ? fast_exp2(sc[kb][r] - m_use) : fast_exp2(fmaf(sc[kb][r], cs, -m_use));
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[kb][u][e] = cvt_pk(T{}, sc[kb][8 * u + 2 * e], sc[kb][8 * u + 2 * e + 1]);
          l_run = row_sum2(T{}, pk[kb][u][e], l_run);
        }
    }
  };
  // O^T += V^T P^T for one packed P
  auto pv = [&](const uint8_t* Vst, const u32x4 (&pk)[C::NKB][2]) {
    const uint8_t* Vs = Vst + v_lane;
    // product i = (2 kb + u) NMB + mb
    auto vread = [&](int i) {
      const int kb = i / (2 * C::NMB), u = (i / C::NMB) % 2, mb = i % C::NMB;
      const uint8_t* vb = Vs + (32 * kb + 16 * u) * C::RB;
      const uint32_t ch = ((4 * mb + v_ch) ^ v_swz) * 16;
      const u32x2 a0 = lds_read_tr16(vb + ch);
      const u32x2 a1 = lds_read_tr16(vb + 8 * C::RB + ch);
      return u32x4{a0[0], a0[1], a1[0], a1[1]};
    };
    constexpr int N = C::NKB * 2 * C::NMB;
    if constexpr (kReadAhead) {
      constexpr int LA = 2;
      u32x4 vr[LA];
#pragma unroll
      for (int j = 0; j < LA; ++j) vr[j] = vread(j < N ? j : 0);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const u32x4 va = vr[i % LA];
        if (i + LA < N) vr[i % LA] = vread(i + LA);
        __builtin_amdgcn_sched_barrier(0);
        acc[i % C::NMB] = mma32(T{}, va, pk[i / (2 * C::NMB)][(i / C::NMB) % 2], acc[i % C::NMB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i)
        acc[i % C::NMB] = mma32(T{}, vread(i), pk[i / (2 * C::NMB)][(i / C::NMB) % 2], acc[i % C::NMB]);
    }
  };

  // One steady-state tile as a fixed sequence of slots.  fp16 holds scores
  // relative to the reference max: S'(t) = c S(t) - m, the accumulators of
  // S(t+1) starting at -m (mneg), so P(t) = exp2(S'(t)); bf16 holds the raw
  // S(t) and P(t) = exp2(c S(t) - m).  Slot i holds
  //   - the LDS operand read of matrix-core op i + W (W ops of lead time),
  //   - matrix-core op i: ops [0, NQK) form S(t+1) = K(t+1).Q^T (kb-major),
  //     the rest O^T += V(t)^T.P(t)^T in (kb, u) groups of NMB,
  //   - its share of the VALU work: "EC" items (two probabilities of P(t),
  //     exponentials, packing, row sum) before the P.V ops that consume them,
  //     then "X" items (row max of S(t+1), two scores each) once it exists
  //     (none in the fast pass, whose slots there hold the row-sum check).
  // Returns the row max of c S(t+1): relative to m for fp16, absolute for
  // bf16; the fast pass moves the reference max itself and returns -inf.
  // A full scheduling fence closes every slot.  A wave whose matrix ops are
  // spaced by a few VALU ops lets both units run at once; a run of
  // back-to-back matrix ops stalls the VALU of the other wave on the SIMD.
  f32x16 mneg;
  bool bad = false;  // fast pass: a tile's row sum was not finite (wave-uniform)
  // update_max in relative units; S'(t+1) follows the moved max
  auto rel_move = [&](float mx, f32x16* nxt) {
    if (__any(mx > kRescaleSlack)) {
      const float d = fmaxf(mx, 0.f);
      const float corr = fast_exp2(-d);
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) acc[mb] *= corr;
      l_run *= corr;
      m_run += d;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) nxt[kb] -= d;
      mneg = -m_run;
    }
  };
  auto steady_slots = [&](auto fast_tag, const uint8_t* Kst, const uint8_t* Vst, f32x16* cur,
                          f32x16* nxt) -> float {
    constexpr bool kFast = decltype(fast_tag)::value;
    constexpr int NQK = C::NKB * C::NQ;
    constexpr int GOPS = C::NMB;
    constexpr int NOPS = NQK + C::NKB * 2 * GOPS;
    constexpr int W = SDPA_PF_WIN;
    constexpr int NEC = C::NKB * 8;            // EC items: (kb, u, e)
    constexpr int NX = C::NKB * 8;             // X items: (kb, pair of rows)
    // EC items occupy slots [0, EC_END).  The fast pass at D = 64 has no X
    // items: its EC items spread over all but the last 3 slots (which hold
    // the row-sum check), 0.7 % faster than leaving 6.
    constexpr int EC_END = NOPS - (D == 64 ? (kRel ? 3 : 6) : 8);
    constexpr int X_BEG = EC_END;                     // X items occupy [X_BEG, NOPS)
    static_assert(EC_END >= NQK + 2, "X items need S(t+1) complete");
    u32x4 opnd[NOPS];
    u32x4 hi[C::NKB][2];
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    auto load_op = [&](int i) {
      if (i < NQK) {
        const int kb = i / C::NQ, s = i % C::NQ;
        opnd[i] = lds_read16(Kst + k_lane + 32 * kb * C::RB + (((2 * s + g) ^ k_swz) * 16));
      } else {
        const int j = i - NQK, grp = j / GOPS, w = j % GOPS;
        const int kb = grp / 2, u = grp % 2;
        if (w < C::NMB) {
          const uint8_t* vb = Vst + v_lane + (32 * kb + 16 * u) * C::RB + ((4 * w + v_ch) ^ v_swz) * 16;
          const u32x2 a0 = lds_read_tr16(vb);
          const u32x2 a1 = lds_read_tr16(vb + 8 * C::RB);
          opnd[i] = u32x4{a0[0], a0[1], a1[0], a1[1]};
        }
      }
    };
    auto do_op = [&](int i) {
      if (i < NQK) {
        const int kb = i / C::NQ, s = i % C::NQ;
        nxt[kb] = mma32(T{}, opnd[i], qreg[s], s == 0 ? (kRel ? mneg : f32x16{}) : nxt[kb]);
      } else {
        const int j = i - NQK, grp = j / GOPS, w = j % GOPS;
        const int kb = grp / 2, u = grp % 2;
        acc[w] = mma32(T{}, opnd[i], hi[kb][u], acc[w]);
      }
    };
    // EC item = two probabilities: (a) bf16 only: scaled score minus max,
    // (b) exp2, (c) pack + row sum.  The stages of one item run in consecutive
    // slots (a two slots ahead of c), so each slot mixes independent work of
    // several items instead of one dependent chain.
    float xs[NEC][2], ps[NEC][2];
    auto ec_a = [&](int it) {
      if constexpr (!kRel) {
        const int kb = it / 8, u = (it % 8) / 4, e = it % 4;
        xs[it][0] = fmaf(cur[kb][8 * u + 2 * e], c, -m_use);
        xs[it][1] = fmaf(cur[kb][8 * u + 2 * e + 1], c, -m_use);
      }
    };
    auto ec_b = [&](int it) {
      const int kb = it / 8, u = (it % 8) / 4, e = it % 4;
      ps[it][0] = fast_exp2(kRel ? cur[kb][8 * u + 2 * e] : xs[it][0]);
      ps[it][1] = fast_exp2(kRel ? cur[kb][8 * u + 2 * e + 1] : xs[it][1]);
    };
    // Row sum.  Without causal masking fp16 takes the cheapest VALU form:
    // the exact-scale path adds the two fp32 probabilities themselves
    // (against the fp16-rounded values P.V multiplies they differ by at most
    // 2^-11 relative per term); the pre-scaled path sums the packed fp16
    // probabilities in two fp16 pairs (one add per two probabilities),
    // folded into the fp32 row sum once per tile: 16 values of at most 2^8
    // per pair, each add rounded to 11 bits (at most 2^-11 x 16 relative on a
    // tile's sum, about 2^-11 / sqrt(keys) on the row's after the rounding of
    // independent tiles averages).  With causal masking one v_dot2 of the
    // packed pair against ones into the fp32 sum measured 3-4 % faster on
    // both paths (the masked kernel schedules the slots differently), and
    // bf16 always sums the rounded values that way: its 2^-9 rounding would
    // otherwise show in rows of a few hundred keys.
    h2 lh[2];
    float lsum = 0.f;  // fast pass under causal masking: this tile's row sum
    auto ec_c = [&](int it) {
      const int kb = it / 8, u = (it % 8) / 4, e = it % 4;
      hi[kb][u][e] = cvt_pk(T{}, ps[it][0], ps[it][1]);
      if constexpr (kRel && !CAUSAL) {
        if (it < 2) lh[it] = as_h2(hi[kb][u][e]);
        else lh[it & 1] += as_h2(hi[kb][u][e]);
      }
      else if constexpr (std::is_same<T, TF16>::value && !CAUSAL) l_run += ps[it][0] + ps[it][1];
      else if constexpr (kFast) lsum = row_sum2(T{}, hi[kb][u][e], lsum);
      else l_run = row_sum2(T{}, hi[kb][u][e], l_run);
    };
    // v_max3 written out: fmaxf on matrix-core results would first quieten
    // each operand (two extra VALU ops), and volatile keeps it in its slot.
    // Two running maxima halve the dependent chain.
    float mx2[2] = {kNegInf, kNegInf};
    auto x_item = [&](int it) {
      if constexpr (kFast) return;
      const int kb = it / 8, r = 2 * (it % 8);
      float& m = mx2[it & 1];
      asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(m), "v"(nxt[kb][r]), "v"(nxt[kb][r + 1]));
    };
    // item ranges: EC items finish (stage c) evenly over slots [0, EC_END),
    // X items run over [X_BEG, NOPS)
    auto ec_begin = [](int i) { return i >= EC_END ? NEC : (i * NEC + EC_END - 1) / EC_END; };
    auto x_begin = [](int i) {
      return i <= X_BEG ? 0 : (i >= NOPS ? NX : ((i - X_BEG) * NX + (NOPS - X_BEG) - 1) / (NOPS - X_BEG));
    };
    // this tile's row sum over the lane's keys, once every EC item is done
    float lt = 0.f;
    unsigned long long trig = 0;  // fast pass: lanes whose sum reached kFastSumMax
    auto tile_sum = [&]() {
      if constexpr (kRel && !CAUSAL) {
        const h2 t = lh[0] + lh[1];
        lt = (float)t[0] + (float)t[1];
      } else {
        lt = lsum;
      }
    };
#pragma unroll
    for (int i = 0; i < W && i < NOPS; ++i) load_op(i);
#pragma unroll
    for (int it = 0; it < ec_begin(2); ++it) ec_a(it);
#pragma unroll
    for (int it = 0; it < ec_begin(1); ++it) ec_b(it);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NOPS; ++i) {
      if (i + W < NOPS) load_op(i + W);
      do_op(i);
#pragma unroll
      for (int it = ec_begin(i + 2); it < ec_begin(i + 3); ++it) ec_a(it);
#pragma unroll
      for (int it = ec_begin(i + 1); it < ec_begin(i + 2); ++it) ec_b(it);
#pragma unroll
      for (int it = ec_begin(i); it < ec_begin(i + 1); ++it) ec_c(it);
#pragma unroll
      for (int it = x_begin(i); it < x_begin(i + 1); ++it) x_item(it);
      // fast pass: the sum and its check in the slots the row max would
      // take; after the last slot only a scalar branch remains
      if constexpr (kFast) {
        if (i == X_BEG) tile_sum();
        if (i == X_BEG + 1) l_run += lt;
        if (i == X_BEG + 2) trig = __ballot(!(lt < kFastSumMax));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!kFast) tile_sum();
    if constexpr (kFast) {
      static_assert(X_BEG + 2 < NOPS, "slots for the fast pass's check");
      if (__builtin_expect(trig != 0, 0)) {
        // (rare) the reference max moves by log2 of the row's tile sum, the
        // same for both halves of a row, so that the tile's sum becomes 1
        const float lr = lt + __shfl_xor(lt, 32, 64);
        if (__any(!(lr < -kNegInf))) bad = true;
        rel_move(fast_log2(lr), nxt);
      }
      return kNegInf;  // nothing left for the caller to move
    }
    if constexpr (kRel && !CAUSAL) l_run += lt;
    const float mx = max2_xor32(mx2[0], mx2[1]);
    return kRel ? mx : mx * c;
  };

  // ---- pipeline.  Tile t lives in stage t & 1 of both rings.  Iteration t
  // waits for K(t+1) and V(t) (issued one iteration earlier), then refills the
  // stages that K(t) and V(t-1) occupied, whose last reads precede the barrier.
  // A wave whose 32 rows all lie past the batch's real rows (the ragged last
  // workgroup of a head) computes nothing: it only keeps its share of the K /
  // V loads and the workgroup's barriers, in the same order as the others,
  // and leaves its rows empty.  Its SIMD time goes to the waves beside it.
  const bool idle = iw >= lq;
  // The pre-scaled form at D <= 128 takes the fast pass first; a workgroup
  // where it met a tile out of range (kFastSumMax) takes the checked pass.
  constexpr bool kTwoPass = kRel && D <= 128;
  __shared__ int wg_bad;
  if (kTwoPass && tid == 0) wg_bad = 0;  // ordered before any vote by the tile barriers
  // K(0), K(1) and V(0) in flight and landed
  auto prologue = [&]() {
    issue_k(0, Kring);
    if (ntiles > 1) issue_k(1, Kring + C::TILE);
    issue_v(0, Vring);
    wait_vmcnt<0>();
    lds_barrier();
  };
  auto idle_pass = [&]() {
    if (ntiles > 0) prologue();
    for (int t = 0; t < ntiles; ++t) {
      const int par = t & 1;
      wait_vmcnt<0>();
      lds_barrier();
      if (t + 1 < ntiles) issue_v(t + 1, Vring + (par ^ 1) * C::TILE);
      if (t + 2 < ntiles) issue_k(t + 2, Kring + par * C::TILE);
    }
  };
  f32x16 sa[C::NKB], sb[C::NKB];
  auto first_tile = [&]() {
    if (ntiles > 0) {
      prologue();
      qk(Kring, sa);
      update_max(0 < n_int ? tile_max(0, sa, std::false_type{}) : tile_max(0, sa, std::true_type{}));
    }
  };
  auto general = [&](int t, auto edge_tag) {
    const int par = t & 1;
    wait_vmcnt<0>();
    lds_barrier();
    if (t + 1 < ntiles) issue_v(t + 1, Vring + (par ^ 1) * C::TILE);
    if (t + 2 < ntiles) issue_k(t + 2, Kring + par * C::TILE);
    // The bf16 hi + lo split is a branch per tile around its own products:
    // a runtime choice inside probs / pv put a branch around every product,
    // so each product was a block of its own and nothing was scheduled
    // across them (bf16 at D = 256, whose tiles all take this path, ran 43 %
    // slower than fp16).
    u32x4 hi[C::NKB][2];
    probs(sa, hi, edge_tag);
    if constexpr (std::is_same<T, TBF16>::value) {
      if (split_p) {
        // P = hi + lo: lo is the rounding hi left, as a second set of
        // products; the row sum adds it too
        u32x4 lo[C::NKB][2];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t h = hi[kb][u][e];
              lo[kb][u][e] = TBF16::pack2(sa[kb][8 * u + 2 * e] - TBF16::to_f32((uint16_t)(h & 0xffffu)),
                                          sa[kb][8 * u + 2 * e + 1] - TBF16::to_f32((uint16_t)(h >> 16)));
              l_run = row_sum2(T{}, lo[kb][u][e], l_run);
            }
        pv(Vring + par * C::TILE, lo);
      }
    }
    pv(Vring + par * C::TILE, hi);
    if (t + 1 < ntiles) {
      qk(Kring + (par ^ 1) * C::TILE, sa);
      update_max(t + 1 < n_int ? tile_max(t + 1, sa, std::false_type{})
                               : tile_max(t + 1, sa, std::true_type{}));
    }
  };
  if (idle) {
    idle_pass();
  } else {
    first_tile();
    // steady state (tiles t, t+1 interior, tile t+2 exists, single bf16 P): no
    // branch between the barrier and the max update, stage offsets fixed by
    // the parity of t, so matrix-core and VALU work of the two tiles interleave
    auto steady = [&](auto fast_tag, int t, auto par_tag, f32x16* cur, f32x16* nxt) {
      constexpr int PAR = decltype(par_tag)::value;
      wait_vmcnt<0>();
      lds_barrier();
      issue_v(t + 1, Vring + (PAR ^ 1) * C::TILE);
      issue_k(t + 2, Kring + PAR * C::TILE);
      const float mx = steady_slots(fast_tag, Kring + (PAR ^ 1) * C::TILE, Vring + PAR * C::TILE, cur, nxt);
      if constexpr (!kRel) update_max(mx);
      else if constexpr (!decltype(fast_tag)::value) rel_move(mx, nxt);  // the fast pass moved it itself
    };
    int t = 0;
    if constexpr (D <= 128) {
      const int n_steady = split_p || (kRel && !pre) ? 0 : max(0, min(n_int - 1, ntiles - 2));
      if (kRel && n_steady > 0) {
        // tile 0 was interior, so m_run is finite
        mneg = -m_run;
  #pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) sa[kb] += mneg;
      }
      auto run_steady = [&](auto fast_tag) {
        for (; t + 1 < n_steady; t += 2) {
          steady(fast_tag, t, std::integral_constant<int, 0>{}, sa, sb);
          steady(fast_tag, t + 1, std::integral_constant<int, 1>{}, sb, sa);
        }
        if (t < n_steady) {
          steady(fast_tag, t, std::integral_constant<int, 0>{}, sa, sb);
    #pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) sa[kb] = sb[kb];
          ++t;
        }
      };
      if constexpr (kTwoPass) run_steady(std::true_type{});
      else run_steady(std::false_type{});
      if (kRel && n_steady > 0) {
  #pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) sa[kb] += m_run;
      }
    }
    for (; t < n_int; ++t) general(t, std::false_type{});
    for (; t < ntiles; ++t) general(t, std::true_type{});
  }
  if constexpr (kTwoPass) {
    if (bad && lane == 0) wg_bad = 1;
    __syncthreads();  // also: every wave is past its last read of the rings
    if (wg_bad) {
      // the checked pass: every tile again, on the general path (row max first)
  #pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) acc[mb] = f32x16{};
      m_run = kNegInf;
      l_run = 0.f;
      if (idle) {
        idle_pass();
      } else {
        first_tile();
        int t = 0;
        for (; t < n_int; ++t) general(t, std::false_type{});
        for (; t < ntiles; ++t) general(t, std::true_type{});
      }
    }
  }

  // ---- epilogue (padding rows see no key) ----
  float l_tot = sum_xor32(l_run);
  if (my_i >= lq) {
    m_run = kNegInf;
    l_tot = 0.f;
  }
  if constexpr (!CAUSAL && !MASK) {
    if (piece >= 0) {
      // a piece's partial: the unnormalised numerators, the reference max
      // (log2 units) and the row sum; the sink enters at the merge
      const int part = (int)blockIdx.x - (p.tiles - p.tail_tiles);
      const int row = 32 * wave + l32;
      float* po = p.part_o + ((int64_t)part * BM + row) * D;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(f32x4*)(po + 32 * mb + 8 * q4 + 4 * g) =
              f32x4{acc[mb][4 * q4], acc[mb][4 * q4 + 1], acc[mb][4 * q4 + 2], acc[mb][4 * q4 + 3]};
      if (g == 0) *(f32x2*)(p.part_ml + ((int64_t)part * BM + row) * 2) = f32x2{m_run, l_tot};
      return;
    }
  }
  float M = m_run, Ltot = l_tot;
  if (p.sinks) {
    const float sk = p.sinks[hq] * kLog2e;
    M = fmaxf(m_run, sk);
    if (M != kNegInf) Ltot = l_tot * fast_exp2(m_run - M) + fast_exp2(sk - M);
  }
  float scale_o = 0.f, lse = kNegInf;
  if (M != kNegInf && Ltot > 0.f) {
    scale_o = (p.sinks ? fast_exp2(m_run - M) : 1.f) / Ltot;
    lse = (M + fast_log2(Ltot)) * kLn2;
  }
  if (my_i < p.Lq) {
    S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)my_i * p.os[2];
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // rows 8*q4 + 4g + (0..3) of block mb: four consecutive head-dim elements
        const u32x2 w = {cvt_pk(T{}, acc[mb][4 * q4] * scale_o, acc[mb][4 * q4 + 1] * scale_o),
                         cvt_pk(T{}, acc[mb][4 * q4 + 2] * scale_o, acc[mb][4 * q4 + 3] * scale_o)};
        if (32 * mb + 8 * q4 + 4 * g < p.Dv) *(u32x2*)(orow + 32 * mb + 8 * q4 + 4 * g) = w;
      }
    if (p.lse && g == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Lq + my_i] = lse;
  }
}

// D = 64: three waves per SIMD (168 registers; the few values that do not fit
// are parked in scratch outside the tile loop), which measured 3-4 % faster
// than two.  D = 128: two waves per SIMD.  D = 256: one.  The masked variants
// keep a second score tile plus the mask gathers live across the pipeline and
// get the whole register file.
template <class T, int D, bool CAUSAL, int NW, bool REL>
__global__ __launch_bounds__(64 * NW, D >= 256 ? 1 : (D == 64 ? 3 : 2)) void prefill16_kernel(AttnParams p) {
  prefill16_body<T, D, CAUSAL, false, NW, REL>(p);
}
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void prefill16_mask_kernel(AttnParams p) {
  prefill16_body<T, D, CAUSAL, true, kWaves, false>(p);
}

// The tail tiles' pieces, merged: workgroup = (tail tile, quarter of its 128
// rows), 8 threads per row, each over D/8 columns.  Per row: M = the larger
// piece max (and the sink), each piece weighted by 2^(m - M), the sink added
// to the denominator, as the one-pass epilogue does; the pieces are summed in
// piece order, so the result does not depend on which finished first.  Two
// pieces per tile (the host's plan): every load is issued before the first
// use, the kernel being a few dependent memory round trips long.
constexpr int kMergeRowsThreads = 256;
constexpr int kTailPiecesK = 2;
template <class T, int D>
__global__ __launch_bounds__(kMergeRowsThreads) void prefill_tail_merge_kernel(AttnParams p) {
  using S = uint16_t;
  constexpr int BM = kBM, ROWS = BM / 4, TPR = kMergeRowsThreads / ROWS, CPT = D / TPR, K = kTailPiecesK;
  static_assert(CPT % 4 == 0, "merge columns");
  const int tile = (int)blockIdx.x / 4, quarter = (int)blockIdx.x % 4;
  const int item = p.tiles - p.tail_tiles + tile;
  int qt, bh;
  prefill_tile(item, p.tiles, (p.Lq + BM - 1) / BM, p.B * p.Hq, false, qt, bh);
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int row = quarter * ROWS + (int)threadIdx.x / TPR, c0 = ((int)threadIdx.x % TPR) * CPT;
  const int i = qt * BM + row;
  if (i >= p.Lq) return;
  const int64_t base = (int64_t)tile * K;
  f32x2 ml[K];
  f32x4 v[K][CPT / 4];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    ml[j] = *(const f32x2*)(p.part_ml + ((base + j) * BM + row) * 2);
#pragma unroll
    for (int c = 0; c < CPT / 4; ++c) v[j][c] = *(const f32x4*)(p.part_o + ((base + j) * BM + row) * D + c0 + 4 * c);
  }
  const float sk = p.sinks ? p.sinks[hq] * kLog2e : kNegInf;
  float M = sk;
#pragma unroll
  for (int j = 0; j < K; ++j) M = fmaxf(M, ml[j][0]);
  float w[K], L = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    w[j] = (M != kNegInf && ml[j][0] != kNegInf) ? fast_exp2(ml[j][0] - M) : 0.f;
    L += ml[j][1] * w[j];
  }
  if (p.sinks && M != kNegInf) L += fast_exp2(sk - M);
  const float inv = (M != kNegInf && L > 0.f) ? 1.f / L : 0.f;
  S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)i * p.os[2];
#pragma unroll
  for (int c = 0; c < CPT / 4; ++c) {
    f32x4 o = f32x4{};
#pragma unroll
    for (int j = 0; j < K; ++j) o += v[j][c] * (w[j] * inv);
    const int col = c0 + 4 * c;
    if (col < p.Dv) *(u32x2*)(orow + col) = u32x2{cvt_pk(T{}, o[0], o[1]), cvt_pk(T{}, o[2], o[3])};
  }
  if (p.lse && c0 == 0)
    p.lse[((int64_t)b * p.Hq + hq) * p.Lq + i] = (M != kNegInf && L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

template <class T, int D>
hipError_t launch_t(const AttnParams& p, bool causal, hipStream_t s) {
  const bool mask = p.mask != nullptr;
  if constexpr (std::is_same<T, TF32>::value) {
    const int nqt = (p.Lq + kBM - 1) / kBM;
    const dim3 grid((unsigned)(nqt * p.B * p.Hq));
    const dim3 block(kThreads);
    if (causal) {
      if (mask) hipLaunchKernelGGL((prefill_f32_kernel<T, D, true, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((prefill_f32_kernel<T, D, true, false>), grid, block, 0, s, p);
    } else {
      if (mask) hipLaunchKernelGGL((prefill_f32_kernel<T, D, false, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((prefill_f32_kernel<T, D, false, false>), grid, block, 0, s, p);
    }
  } else {
    // 4-wave workgroups of 128 query rows.  (2-wave workgroups for D = 64 shrink
    // the idle tail of the last round but double the K/V tile traffic into
    // LDS, and measure slower.)
    AttnParams q = p;
    q.tiles = (p.Lq + kBM - 1) / kBM * p.B * p.Hq;
    const dim3 grid((unsigned)(q.tiles + q.tail_tiles * (q.tail_k - 1)));
    const dim3 block(kThreads);
    // pre-scaled Q: fp16, exponent scale at most 1, no log-sum-exp output
    const bool rel = std::is_same<T, TF16>::value && fabsf(p.scale_log2) <= 1.f && p.lse == nullptr;
    if (mask) {
      if (causal) hipLaunchKernelGGL((prefill16_mask_kernel<T, D, true>), grid, block, 0, s, q);
      else hipLaunchKernelGGL((prefill16_mask_kernel<T, D, false>), grid, block, 0, s, q);
    } else if (rel) {
      if constexpr (std::is_same<T, TF16>::value) {
        if (causal) hipLaunchKernelGGL((prefill16_kernel<T, D, true, kWaves, true>), grid, block, 0, s, q);
        else hipLaunchKernelGGL((prefill16_kernel<T, D, false, kWaves, true>), grid, block, 0, s, q);
      }
    } else {
      if (causal) hipLaunchKernelGGL((prefill16_kernel<T, D, true, kWaves, false>), grid, block, 0, s, q);
      else hipLaunchKernelGGL((prefill16_kernel<T, D, false, kWaves, false>), grid, block, 0, s, q);
    }
    if (q.tail_tiles > 0) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((prefill_tail_merge_kernel<T, D>), dim3((unsigned)(q.tail_tiles * 4)), dim3(kMergeRowsThreads),
                         0, s, q);
    }
  }
  return hipGetLastError();
}

template <class T>
hipError_t launch_d(const AttnParams& p, bool causal, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_t<T, 64>(p, causal, s);
    case 128: return launch_t<T, 128>(p, causal, s);
    default:
      if constexpr (std::is_same<T, TF32>::value) return hipErrorInvalidValue;  // rejected by the API
      else return launch_t<T, 256>(p, causal, s);
  }
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, int dtype, bool causal, hipStream_t s) {
  switch (dtype) {
    case SDPA_F32: return launch_d<TF32>(p, causal, s);
    case SDPA_F16: return launch_d<TF16>(p, causal, s);
    default: return launch_d<TBF16>(p, causal, s);
  }
}

}  // namespace sdpa
