// Single-query ("vector") decode attention for gfx950: single-pass and
// two-pass split-K forms, grouped-query head mapping, optional per-head sinks,
// optional additive mask and log-sum-exp output.
//
// The two forms are the single-pass and two-pass vector kernels of the "Add
// D512 support to Metal vector attention" page.  Both use the running-max /
// running-sum recurrence of the rustytorch "flash_attention.metal" forward
// kernel ("Online softmax update") over their key range.  The two-pass form
// writes, per (batch, query head, split), the unnormalised partial
// (m_s, l_s, o_s = sum_j 2^(s_j - m_s) v_j); the merge pass combines them with
//     M = max(max_s m_s, sink),  L = sum_s l_s 2^(m_s - M) + 2^(sink - M),
//     O = sum_s o_s 2^(m_s - M) / L,   LSE = (M + log2 L) ln 2
// (scores in log2 units), giving splits with m_s = -inf weight zero.
//
// Work decomposition: one workgroup (4 waves) per (split, KV head, batch).
// The G <= 16 query heads that share the KV head are the 16 columns of
// 16x16 matrix-core tiles, so every K / V element is read from HBM once per
// (batch, KV head) and used for all G heads:
//     S^T (keys x heads) = K . Q^T     (contraction over the head dim, split
//                                      across the waves, partials summed in LDS)
//     O^T (dims x heads) += V^T . P^T  (each wave owns a quarter of the dims)
// K / V tiles stream HBM -> registers (next tile prefetched) -> LDS.
#include <type_traits>

#include "sdpa_device.hpp"
#include "sdpa_internal.hpp"

namespace sdpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <class T, int D>
struct DecodeCfg {
  static constexpr int ES = T::kBytes;
  static constexpr int VEC = T::kVec;
  static constexpr int NCH = D / VEC;                  // 16-byte chunks per row
  static constexpr bool F32 = (ES == 4);
  static constexpr int TK = F32 ? (D >= 256 ? 16 : 4096 / D) : (D >= 256 ? 32 : 8192 / D);
  static constexpr int NBLK = TK / 16;                 // 16-key blocks per tile
  static constexpr int KP = D * ES + 16;               // K row pitch (bytes)
  static constexpr int VP = TK * ES + 16;              // V^T row pitch (bytes)
  static constexpr int K_BYTES = TK * KP;
  static constexpr int V_BYTES = D * VP;
  static constexpr int NS = D * ES / 64;               // 16-byte Q vectors per head row / 4
  static constexpr int QSPLIT = NS < kWaves ? NS : kWaves;  // waves sharing Q.K^T
  static constexpr int NSW = NS / QSPLIT;              // Q vectors per wave
  static constexpr int X_BYTES = QSPLIT * NBLK * 64 * 16;  // partial-score exchange
  static constexpr int NOB = D / 16 / kWaves;          // 16-row blocks of O^T per wave
  static constexpr int K_IT = TK * NCH / kThreads;
  static constexpr int V_IT = (TK / 4) * NCH / kThreads;
  static_assert(NS % QSPLIT == 0, "Q split");
  static_assert(NOB >= 1, "O split");
  static_assert(K_IT >= 1 && TK * NCH % kThreads == 0, "K tile split");
  static_assert(V_IT >= 1 && (TK / 4) * NCH % kThreads == 0, "V tile split");
  static_assert(F32 ? TK % 16 == 0 : TK % 32 == 0, "tile keys");
};

template <int NCH>
__device__ constexpr int vt_row(int c, int e) { return c + NCH * e; }
template <int NCH, int VEC>
__device__ constexpr int vt_row_to_d(int rho) { return VEC * (rho % NCH) + rho / NCH; }

// Slot of key group kg (4 keys) inside a 32-key block of a V^T row.  16-bit:
// lane group g4 of the P.V product supplies keys {16a + 4*g4 + c} (a: which
// 16-key score block, c = 0..3) as its 8 contiguous k-slots 8*g4 + 4a + c.
// fp32: natural order.
template <bool F32>
__device__ constexpr int vt_group_slot(int kg) {
  return F32 ? kg : ((kg & ~7) | (2 * (kg & 3) + ((kg >> 2) & 1)));
}

template <class T, int D, bool MASK, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(AttnParams p) {
  using C = DecodeCfg<T, D>;
  using S = typename T::storage;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::K_BYTES + C::V_BYTES + C::X_BYTES];
  uint8_t* Ks = smem;
  uint8_t* Vt = smem + C::K_BYTES;
  f32x4* Sx = (f32x4*)(smem + C::K_BYTES + C::V_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;   // head column of the 16x16 tiles
  const int g4 = lane >> 4;  // lane group

  const int split = blockIdx.x % p.nsplit;
  const int bk = blockIdx.x / p.nsplit;
  const int hk = bk % p.Hkv;
  const int b = bk / p.Hkv;
  const int hq = hk * p.group + n;  // query head of this lane's column
  const bool head_ok = n < p.group;

  const int kbeg = split * p.split_len;
  const int kend = min(p.Lk, kbeg + p.split_len);
  const int ntiles = kend > kbeg ? (kend - kbeg + C::TK - 1) / C::TK : 0;

  const S* kp = (const S*)p.k + b * p.ks[0] + hk * p.ks[1];
  const S* vp = (const S*)p.v + b * p.vs[0] + hk * p.vs[1];

  // ---- Q^T operand: this wave's share of the head dim; vector s = chunk 4*(s0+s) + g4
  u32x4 qreg[C::NSW];
  {
    const int s0 = wave < C::QSPLIT ? wave * C::NSW : 0;
    const S* row = (const S*)p.q + b * p.qs[0] + (int64_t)(head_ok ? hq : hk * p.group) * p.qs[1];
#pragma unroll
    for (int s = 0; s < C::NSW; ++s) {
      u32x4 v = ldg16_cached(row + (4 * (s0 + s) + g4) * C::VEC);
      qreg[s] = head_ok ? v : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 acc[C::NOB];
#pragma unroll
  for (int i = 0; i < C::NOB; ++i) acc[i] = f32x4{};
  float m_run = kNegInf;
  float l_run = 0.f;

  u32x4 kpre[C::K_IT];
  u32x4 vpre[C::V_IT][4];
  auto prefetch = [&](int j0) {
#pragma unroll
    for (int it = 0; it < C::K_IT; ++it) {
      const int u = tid + kThreads * it;
      const int key = u / C::NCH, c = u % C::NCH;
      const int j = j0 + key;
      kpre[it] = j < kend ? ldg16(kp + (int64_t)j * p.ks[2] + c * C::VEC) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < C::V_IT; ++it) {
      const int u = tid + kThreads * it;
      const int kg = u / C::NCH, c = u % C::NCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * kg + r;
        vpre[it][r] = j < kend ? ldg16(vp + (int64_t)j * p.vs[2] + c * C::VEC) : u32x4{0, 0, 0, 0};
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
      const int slot4 = vt_group_slot<C::F32>(kg);
      if constexpr (C::F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 w = {vpre[it][0][e], vpre[it][1][e], vpre[it][2][e], vpre[it][3][e]};
          lds_write16(Vt + vt_row<C::NCH>(c, e) * C::VP + slot4 * 16, w);
        }
      } else {
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

  if (ntiles > 0) prefetch(kbeg);

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = kbeg + t * C::TK;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) prefetch(j0 + C::TK);

    // ---- partial S^T over this wave's share of the head dim ----
    if (wave < C::QSPLIT) {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        f32x4 s = f32x4{};
        const uint8_t* krow = Ks + (16 * blk + n) * C::KP + (4 * wave * C::NSW + g4) * 16;
#pragma unroll
        for (int ss = 0; ss < C::NSW; ++ss) s = mma16(T{}, lds_read16(krow + ss * 64), qreg[ss], s);
        Sx[(wave * C::NBLK + blk) * 64 + lane] = s;
      }
    }
    __syncthreads();

    // ---- full scores, scale, mask, tail, running max (identical in all waves)
    f32x4 sc[C::NBLK];
    float mx = kNegInf;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
      f32x4 s = Sx[blk * 64 + lane];
#pragma unroll
      for (int w = 1; w < C::QSPLIT; ++w) s += Sx[(w * C::NBLK + blk) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 16 * blk + 4 * g4 + r;
        float x = s[r] * p.scale_log2;
        if (MASK) {
          const int jj = j < kend ? j : kend - 1;
          const int hh = head_ok ? hq : hk * p.group;
          x += kLog2e * p.mask[b * p.ms[0] + hh * p.ms[1] + (int64_t)jj * p.ms[3]];
        }
        x = j < kend ? x : kNegInf;
        sc[blk][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float corr = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < C::NOB; ++i) acc[i] *= corr;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = fast_exp2(sc[blk][r] - m_use);
        sc[blk][r] = pr;
        l_run += pr;
      }
    }

    // ---- O^T += V^T . P^T on this wave's rows ----
    if constexpr (C::F32) {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        u32x4 pb = {as_uint(sc[blk][0]), as_uint(sc[blk][1]),
                    as_uint(sc[blk][2]), as_uint(sc[blk][3])};
#pragma unroll
        for (int i = 0; i < C::NOB; ++i) {
          const int row = 16 * (wave * C::NOB + i) + n;
          acc[i] = mma16(T{}, lds_read16(Vt + row * C::VP + (16 * blk + 4 * g4) * 4), pb, acc[i]);
        }
      }
    } else {
#pragma unroll
      for (int pp = 0; pp < C::NBLK / 2; ++pp) {
        if constexpr (std::is_same<T, TBF16>::value) {
          // bf16 P carries 8 significant bits: feed P = hi + lo (the matrix
          // cores have ample headroom in this bandwidth-bound kernel)
          u32x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t h, l;
            T::split2(sc[2 * pp + (e >> 1)][2 * (e & 1)], sc[2 * pp + (e >> 1)][2 * (e & 1) + 1], h, l);
            hi[e] = h;
            lo[e] = l;
          }
#pragma unroll
          for (int i = 0; i < C::NOB; ++i) {
            const int row = 16 * (wave * C::NOB + i) + n;
            const u32x4 va = lds_read16(Vt + row * C::VP + (32 * pp + 8 * g4) * 2);
            acc[i] = mma16(T{}, va, hi, acc[i]);
            acc[i] = mma16(T{}, va, lo, acc[i]);
          }
        } else {
          u32x4 pb = {T::pack2(sc[2 * pp][0], sc[2 * pp][1]), T::pack2(sc[2 * pp][2], sc[2 * pp][3]),
                      T::pack2(sc[2 * pp + 1][0], sc[2 * pp + 1][1]),
                      T::pack2(sc[2 * pp + 1][2], sc[2 * pp + 1][3])};
#pragma unroll
          for (int i = 0; i < C::NOB; ++i) {
            const int row = 16 * (wave * C::NOB + i) + n;
            acc[i] = mma16(T{}, lds_read16(Vt + row * C::VP + (32 * pp + 8 * g4) * 2), pb, acc[i]);
          }
        }
      }
    }
  }

  // ---- epilogue ----
  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
  const int64_t bh = (int64_t)b * p.Hq + hq;
  if constexpr (SPLIT) {
    if (head_ok) {
      float* po = p.part_o + (bh * p.nsplit + split) * D;
#pragma unroll
      for (int i = 0; i < C::NOB; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rho = 16 * (wave * C::NOB + i) + 4 * g4 + r;
          po[vt_row_to_d<C::NCH, C::VEC>(rho)] = acc[i][r];
        }
      }
      if (wave == 0 && g4 == 0) {
        float* pml = p.part_ml + (bh * p.nsplit + split) * 2;
        pml[0] = m_run;
        pml[1] = l_tot;
      }
    }
  } else {
    float M = m_run, Ltot = l_tot;
    if (p.sinks) {
      const float sk = p.sinks[head_ok ? hq : 0] * kLog2e;
      M = fmaxf(m_run, sk);
      if (M != kNegInf) Ltot = l_tot * fast_exp2(m_run - M) + fast_exp2(sk - M);
    }
    float so = 0.f, lse = kNegInf;
    if (M != kNegInf && Ltot > 0.f) {
      so = (p.sinks ? fast_exp2(m_run - M) : 1.f) / Ltot;
      lse = (M + fast_log2(Ltot)) * kLn2;
    }
    if (head_ok) {
      S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1];
#pragma unroll
      for (int i = 0; i < C::NOB; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rho = 16 * (wave * C::NOB + i) + 4 * g4 + r;
          orow[vt_row_to_d<C::NCH, C::VEC>(rho)] = T::from_f32(acc[i][r] * so);
        }
      }
      if (p.lse && wave == 0 && g4 == 0) p.lse[bh] = lse;
    }
  }
}

// Merge pass.  Workgroup (b, hq, 64-element slice of the head dim): the
// reference max M and the total L are reduced over the splits by all 256
// threads, then thread (split group sg, element quad dq) sums its splits'
// weighted partial O for four head-dim elements and the 16 split groups are
// combined in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 64;  // head-dim elements per workgroup

template <class T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnParams p) {
  using S = typename T::storage;
  constexpr int NDQ = (D < kMergeCols ? D : kMergeCols) / 4;  // float4 columns per workgroup
  constexpr int NSG = kMergeThreads / NDQ;                      // split groups
  __shared__ float red[kMergeThreads / 64];
  __shared__ f32x4 part[NSG][NDQ];
  const int tid = threadIdx.x;
  const int nslice = D / (NDQ * 4);
  const int64_t bh = blockIdx.x / nslice;
  const int d0 = (blockIdx.x % nslice) * NDQ * 4;
  const int hq = (int)(bh % p.Hq);
  const int b = (int)(bh / p.Hq);
  const float* pml = p.part_ml + bh * p.nsplit * 2;
  const float* po = p.part_o + bh * p.nsplit * D;
  const float sk = p.sinks ? p.sinks[hq] * kLog2e : kNegInf;

  // M = max(max_s m_s, sink)
  float M = kNegInf;
  for (int s = tid; s < p.nsplit; s += kMergeThreads) M = fmaxf(M, pml[2 * s]);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  M = fmaxf(M, sk);
  __syncthreads();
  // L = sum_s l_s 2^(m_s - M) + 2^(sink - M); splits with m_s = -inf weigh 0
  float L = 0.f;
  if (M != kNegInf)
    for (int s = tid; s < p.nsplit; s += kMergeThreads) {
      const float ms = pml[2 * s];
      if (ms != kNegInf) L += pml[2 * s + 1] * fast_exp2(ms - M);
    }
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = L;
  __syncthreads();
  L = red[0] + red[1] + red[2] + red[3];
  if (p.sinks && M != kNegInf) L += fast_exp2(sk - M);
  const bool live = M != kNegInf && L > 0.f;

  // weighted partial numerators
  const int dq = tid % NDQ, sg = tid / NDQ;
  f32x4 o = f32x4{};
  if (live)
    for (int s = sg; s < p.nsplit; s += NSG) {
      const float ms = pml[2 * s];
      if (ms != kNegInf) o += fast_exp2(ms - M) * *(const f32x4*)(po + (int64_t)s * D + d0 + 4 * dq);
    }
  part[sg][dq] = o;
  __syncthreads();
  if (sg == 0) {
    for (int g = 1; g < NSG; ++g) o += part[g][dq];
    const float inv = live ? 1.f / L : 0.f;
    S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1] + d0 + 4 * dq;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = T::from_f32(o[e] * inv);
    if (p.lse && blockIdx.x % nslice == 0 && dq == 0)
      p.lse[bh] = live ? (M + fast_log2(L)) * kLn2 : kNegInf;
  }
}

template <class T, int D>
hipError_t launch_t(const AttnParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.nsplit * p.Hkv * p.B));
  const dim3 block(kThreads);
  const bool mask = p.mask != nullptr;
  if (p.nsplit > 1) {
    if (mask) hipLaunchKernelGGL((decode_kernel<T, D, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<T, D, false, true>), grid, block, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslice = D / (D < kMergeCols ? D : kMergeCols);
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)((int64_t)p.B * p.Hq * nslice)),
                       dim3(kMergeThreads), 0, s, p);
  } else {
    if (mask) hipLaunchKernelGGL((decode_kernel<T, D, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<T, D, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <class T>
hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_t<T, 64>(p, s);
    case 128: return launch_t<T, 128>(p, s);
    case 256: return launch_t<T, 256>(p, s);
    default: return launch_t<T, 512>(p, s);
  }
}

}  // namespace

int decode_tile_keys(int dtype, int D) {
  const bool f32 = dtype == SDPA_F32;
  return f32 ? (D >= 256 ? 16 : 4096 / D) : (D >= 256 ? 32 : 8192 / D);
}

hipError_t launch_decode(const AttnParams& p, int dtype, hipStream_t s) {
  switch (dtype) {
    case SDPA_F32: return launch_d<TF32>(p, s);
    case SDPA_F16: return launch_d<TF16>(p, s);
    default: return launch_d<TBF16>(p, s);
  }
}

}  // namespace sdpa
