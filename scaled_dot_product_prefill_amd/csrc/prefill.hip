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

  const S* qp = (const S*)p.q + b * p.qs[0] + hq * p.qs[1];
  const S* kp = (const S*)p.k + b * p.ks[0] + hk * p.ks[1];
  const S* vp = (const S*)p.v + b * p.vs[0] + hk * p.vs[1];

  // ---- Q row of this lane as B operands: vector s holds chunk 2s + g ----
  u32x4 qreg[C::NQ];
  {
    const bool ok = my_i < p.Lq;
    const S* row = qp + (int64_t)(ok ? my_i : 0) * p.qs[2];
#pragma unroll
    for (int s = 0; s < C::NQ; ++s) {
      u32x4 v = ldg16_cached(row + (2 * s + g) * C::VEC);
      qreg[s] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }

  // key range of the workgroup (bottom-right causal)
  int kend = p.Lk;
  if (CAUSAL) kend = min(kend, i0 + kBM + p.causal_off);
  const int ntiles = kend > 0 ? (kend + C::BN - 1) / C::BN : 0;
  const int wave_last_key = CAUSAL ? iw + 31 + p.causal_off : p.Lk - 1;
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
      kpre[it] = j < p.Lk ? ldg16_cached(kp + (int64_t)j * p.ks[2] + c * C::VEC)
                          : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < C::V_IT; ++it) {
      const int u = tid + kThreads * it;
      const int kg = u / C::NCH, c = u % C::NCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * kg + r;
        vpre[it][r] = j < p.Lk ? ldg16_cached(vp + (int64_t)j * p.vs[2] + c * C::VEC)
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
    const bool edge = (j0 + C::BN > p.Lk) || (CAUSAL && j0 + C::BN - 1 > iw + p.causal_off);

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
          const int ii = my_i < p.Lq ? my_i : p.Lq - 1;
          const int jj = j < p.Lk ? j : p.Lk - 1;
          x += kLog2e * p.mask[b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] +
                               (int64_t)jj * p.ms[3]];
        }
        if (edge) {
          const bool vis = (j < p.Lk) && (!CAUSAL || j <= my_i + p.causal_off);
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

  // ---- epilogue: normalise, sink, LSE ----
  const float l_tot = l_run + xor32(l_run);
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
        orow[vt_row_to_d<C::NCH, C::VEC>(rho)] = T::from_f32(acc[mb][r] * scale_o);
      }
    }
    if (p.lse && g == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Lq + my_i] = lse;
  }
}


// ---------------------------------------------------------------------------
// 16-bit inputs (fp16 / bf16)
// ---------------------------------------------------------------------------
template <int D>
struct Cfg16 {
  static constexpr int BN = 64;                 // keys per tile
  static constexpr int NKB = BN / 32;           // 32-key blocks per tile
  static constexpr int NCH = D / 8;             // 16-byte chunks per row
  static constexpr int KP = D * 2 + 16;         // K row pitch (bytes)
  static constexpr int VP = D * 2 + 64;         // V row pitch (bytes): 4 rows tile 256 B
  static constexpr int STAGE = BN * KP + BN * VP;
  static constexpr int NQ = D / 16;             // 16-byte Q vectors per lane
  static constexpr int IT = BN * NCH / kThreads;  // K (and V) chunks per thread
  static constexpr int NMB = D / 32;            // 32-row blocks of O^T
  // D = 64: the per-row sum of P runs on the matrix cores as one more
  // 32-row block whose V^T rows are all ones (the VALU is the scarcer unit)
  static constexpr bool SUM_MFMA = (D == 64);
  static_assert(IT >= 1 && BN * NCH % kThreads == 0, "tile split");
};

// The running max is only moved (and O, l rescaled) when a row's tile max
// exceeds it by more than this many log2 units; probabilities then stay
// below 2^8, and O = sum(p v) / sum(p) is unchanged by which max is used.
constexpr float kRescaleSlack = 8.f;

// Per wave and tile (BN = 64 keys, 32 queries):
//   S^T = K . Q^T        (NKB x NQ 32x32x16 matrix-core ops, K from LDS)
//   online softmax       (in-lane over 32 keys, one exchange with lane ^ 32)
//   O^T += V^T . P^T     (V^T read with ds_read_b64_tr_b16 from row-major V)
// Interior tiles (every key visible, no mask) take a path with no per-element
// visibility test; the scale is folded into the exponent, exp2(s*c - m).
// The running max only rescales O and l when it grows for some lane.
template <class T, int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 2) void prefill16_kernel(AttnParams p) {
  using C = Cfg16<D>;
  using S = uint16_t;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int nqt = (p.Lq + kBM - 1) / kBM;
  int qt, bh;
  prefill_tile((int)blockIdx.x, (int)gridDim.x, nqt, p.B * p.Hq, CAUSAL, qt, bh);
  const int b = bh / p.Hq;
  const int hq = bh % p.Hq;
  const int hk = hq / p.group;

  const int i0 = qt * kBM;
  const int iw = i0 + 32 * wave;
  const int my_i = iw + l32;

  // exponent scale c = |scale| log2(e); a negative scale is moved into Q
  const float c = fabsf(p.scale_log2);
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  u32x4 qreg[C::NQ];
  {
    const bool ok = my_i < p.Lq;
    const S* row = (const S*)p.q + b * p.qs[0] + hq * p.qs[1] + (int64_t)(ok ? my_i : 0) * p.qs[2];
#pragma unroll
    for (int s = 0; s < C::NQ; ++s) {
      u32x4 v = ldg16_cached(row + (2 * s + g) * 8);
      v ^= qflip;
      qreg[s] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }

  int kend = p.Lk;
  if (CAUSAL) kend = min(kend, i0 + kBM + p.causal_off);
  const int ntiles = kend > 0 ? (kend + C::BN - 1) / C::BN : 0;
  const int wave_last_key = CAUSAL ? iw + 31 + p.causal_off : p.Lk - 1;
  // bf16 probabilities carry 8 significant bits; rows that average few keys
  // would show that rounding directly in O, so such workgroups feed P.V with
  // P = hi + lo (two bf16 products).  Many-key rows average it away.
  const bool split_p = std::is_same<T, TBF16>::value && (MASK || kend <= 1024);

  f32x16 acc[C::NMB];
#pragma unroll
  for (int mb = 0; mb < C::NMB; ++mb) acc[mb] = f32x16{};
  f32x16 lacc = f32x16{};  // row sums from the matrix cores (SUM_MFMA)
  float m_run = kNegInf;  // reference max of the scaled scores (log2 units)
  float l_run = 0.f;      // running sum over this lane's half of the keys
  constexpr uint32_t kOnes = std::is_same<T, TBF16>::value ? 0x3F803F80u : 0x3C003C00u;
  const u32x4 ones = {kOnes, kOnes, kOnes, kOnes};
  auto rescale = [&](float corr) {
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb) acc[mb] *= corr;
    if constexpr (C::SUM_MFMA) lacc *= corr;
    else l_run *= corr;
  };

  // ---- K / V tile loads: buffer resources clip the key range (loads past
  //      the last key return zeros); per-thread byte offsets are fixed ----
  const S* kbase = (const S*)p.k + b * p.ks[0] + hk * p.ks[1];
  const S* vbase = (const S*)p.v + b * p.vs[0] + hk * p.vs[1];
  uint32_t koff[C::IT], voff[C::IT], lds_off[C::IT];
#pragma unroll
  for (int it = 0; it < C::IT; ++it) {
    const int u = tid + kThreads * it;
    const int key = u / C::NCH, ch = u % C::NCH;
    koff[it] = (uint32_t)(key * p.ks[2] * 2 + ch * 16);
    voff[it] = (uint32_t)(key * p.vs[2] * 2 + ch * 16);
    lds_off[it] = key * C::KP + ch * 16;
  }
  auto valid_bytes = [&](int j0, int64_t stride) -> uint32_t {
    const int64_t n = (int64_t)(p.Lk - j0 - 1) * stride * 2 + D * 2;
    return n > 0xffffffffLL ? 0xffffffffu : (uint32_t)n;
  };
  u32x4 kpre[C::IT], vpre[C::IT];
  auto prefetch = [&](int j0) {
    const auto rk = make_rsrc(kbase + (int64_t)j0 * p.ks[2], valid_bytes(j0, p.ks[2]));
    const auto rv = make_rsrc(vbase + (int64_t)j0 * p.vs[2], valid_bytes(j0, p.vs[2]));
#pragma unroll
    for (int it = 0; it < C::IT; ++it) {
      kpre[it] = buf_load16(rk, koff[it]);
      vpre[it] = buf_load16(rv, voff[it]);
    }
  };
  auto store = [&](uint8_t* st) {
#pragma unroll
    for (int it = 0; it < C::IT; ++it) {
      lds_write16(st + lds_off[it], kpre[it]);
      // V rows use the V pitch: the same (key, chunk) position
      const int u = tid + kThreads * it;
      lds_write16(st + C::BN * C::KP + (u / C::NCH) * C::VP + (u % C::NCH) * 16, vpre[it]);
    }
  };

  // lane part of the transposed V read: row 4g + r/4, columns 16*dh + 4*(r%4)
  const int r16 = lane & 15;
  const int dh = (lane >> 4) & 1;
  const uint32_t vtr_lane = (4 * g + (r16 >> 2)) * C::VP + (16 * dh + 4 * (r16 & 3)) * 2;

  auto compute = [&](const uint8_t* st, int j0, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const uint8_t* Ks = st;
    const uint8_t* Vs = st + C::BN * C::KP;
    f32x16 sc[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      sc[kb] = f32x16{};
      const uint8_t* krow = Ks + (32 * kb + l32) * C::KP + g * 16;
#pragma unroll
      for (int s = 0; s < C::NQ; ++s) sc[kb] = mma32(T{}, lds_read16(krow + s * 32), qreg[s], sc[kb]);
    }
    float m_use;
    if constexpr (!EDGE) {
      // every key visible: max over raw scores, scale applied once per row
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = max_xor32(mx) * c;
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        rescale(fast_exp2(m_run - m_new));
        m_run = m_new;
      }
      m_use = m_run;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(sc[kb][r], c, -m_use));
          sc[kb][r] = pr;
          if constexpr (!C::SUM_MFMA) l_run += pr;
        }
    } else {
      float mx = kNegInf;
      const int ii = my_i < p.Lq ? my_i : p.Lq - 1;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          float x = sc[kb][r] * c;
          if (MASK) {
            const int jj = j < p.Lk ? j : p.Lk - 1;
            x += kLog2e * p.mask[b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] + (int64_t)jj * p.ms[3]];
          }
          const bool vis = (j < p.Lk) && (!CAUSAL || j <= my_i + p.causal_off);
          x = vis ? x : kNegInf;
          sc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = max_xor32(mx);
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        // rows that still see nothing (both -inf) keep corr = 1
        rescale(m_new > m_run ? fast_exp2(m_run - m_new) : 1.f);
        m_run = m_new;
      }
      m_use = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(sc[kb][r] - m_use);
          sc[kb][r] = pr;
          if constexpr (!C::SUM_MFMA) l_run += pr;
        }
    }
    // ---- O^T += V^T . P^T; k-step u of block kb covers keys 32kb + 16u + [0, 16):
    //      B element e <-> key 16u + 8(e/4) + 4g + e%4 (the accumulator rows)
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 hi, lo;
        bool two = false;
        if constexpr (std::is_same<T, TBF16>::value) {
          if (split_p) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              uint32_t h, l;
              T::split2(sc[kb][8 * u + 2 * e], sc[kb][8 * u + 2 * e + 1], h, l);
              hi[e] = h;
              lo[e] = l;
            }
            two = true;
          }
        }
        if (!two) {
#pragma unroll
          for (int e = 0; e < 4; ++e) hi[e] = cvt_pk(T{}, sc[kb][8 * u + 2 * e], sc[kb][8 * u + 2 * e + 1]);
        }
        const uint8_t* vb = Vs + vtr_lane + (32 * kb + 16 * u) * C::VP;
#pragma unroll
        for (int mb = 0; mb < C::NMB; ++mb) {
          const u32x2 a0 = lds_read_tr16(vb + 64 * mb);
          const u32x2 a1 = lds_read_tr16(vb + 8 * C::VP + 64 * mb);
          const u32x4 va = {a0[0], a0[1], a1[0], a1[1]};
          acc[mb] = mma32(T{}, va, hi, acc[mb]);
          if (two) acc[mb] = mma32(T{}, va, lo, acc[mb]);
        }
        if constexpr (C::SUM_MFMA) {
          lacc = mma32(T{}, ones, hi, lacc);
          if (two) lacc = mma32(T{}, ones, lo, lacc);
        }
      }
    }
  };

  // Tiles [0, n_int) are interior for every wave of the workgroup (all keys
  // visible to all 128 rows, no mask); they run a loop with a single path.
  // The remaining tiles (causal diagonal, key tail, or every tile when a mask
  // is given) run the masking path.
  int n_int = 0;
  if (!MASK) {
    int last_full = p.Lk;                                   // keys [0, last_full) are in range
    if (CAUSAL) last_full = min(last_full, i0 + 1 + p.causal_off);  // visible to row i0
    n_int = last_full > 0 ? min(ntiles, last_full / C::BN) : 0;
  }
  if (ntiles > 0) {
    prefetch(0);
    store(smem);
  }
  __syncthreads();
  int t = 0;
  for (; t < n_int; ++t) {
    const int j0 = t * C::BN;
    if (t + 1 < ntiles) prefetch(j0 + C::BN);
    compute(smem + (t & 1) * C::STAGE, j0, std::false_type{});
    if (t + 1 < ntiles) store(smem + ((t + 1) & 1) * C::STAGE);
    __syncthreads();
  }
  for (; t < ntiles; ++t) {
    const int j0 = t * C::BN;
    if (t + 1 < ntiles) prefetch(j0 + C::BN);
    if (j0 <= wave_last_key) compute(smem + (t & 1) * C::STAGE, j0, std::true_type{});
    if (t + 1 < ntiles) store(smem + ((t + 1) & 1) * C::STAGE);
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = C::SUM_MFMA ? lacc[0] : sum_xor32(l_run);
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
        *(u32x2*)(orow + 32 * mb + 8 * q4 + 4 * g) = w;
      }
    if (p.lse && g == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Lq + my_i] = lse;
  }
}

template <class T, int D>
hipError_t launch_t(const AttnParams& p, bool causal, hipStream_t s) {
  const int nqt = (p.Lq + kBM - 1) / kBM;
  const dim3 grid((unsigned)(nqt * p.B * p.Hq));
  const dim3 block(kThreads);
  const bool mask = p.mask != nullptr;
  if constexpr (std::is_same<T, TF32>::value) {
    if (causal) {
      if (mask) hipLaunchKernelGGL((prefill_f32_kernel<T, D, true, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((prefill_f32_kernel<T, D, true, false>), grid, block, 0, s, p);
    } else {
      if (mask) hipLaunchKernelGGL((prefill_f32_kernel<T, D, false, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((prefill_f32_kernel<T, D, false, false>), grid, block, 0, s, p);
    }
  } else {
    if (causal) {
      if (mask) hipLaunchKernelGGL((prefill16_kernel<T, D, true, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((prefill16_kernel<T, D, true, false>), grid, block, 0, s, p);
    } else {
      if (mask) hipLaunchKernelGGL((prefill16_kernel<T, D, false, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((prefill16_kernel<T, D, false, false>), grid, block, 0, s, p);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, int dtype, bool causal, hipStream_t s) {
  switch (dtype) {
    case SDPA_F32: return p.D == 64 ? launch_t<TF32, 64>(p, causal, s) : launch_t<TF32, 128>(p, causal, s);
    case SDPA_F16: return p.D == 64 ? launch_t<TF16, 64>(p, causal, s) : launch_t<TF16, 128>(p, causal, s);
    default: return p.D == 64 ? launch_t<TBF16, 64>(p, causal, s) : launch_t<TBF16, 128>(p, causal, s);
  }
}

}  // namespace sdpa
