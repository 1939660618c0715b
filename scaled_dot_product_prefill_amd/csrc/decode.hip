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
constexpr int kWideCUs = 256;  // MI355X compute units

// Work unit of a decode workgroup and the matrix column of one lane.  Block
// index = ((b * Hkv + hk) * nchunk + chunk) * nsplit + split.  The G query
// heads of the KV head times the Lq query rows form the columns of the 16x16
// tiles, column c = qi * G + h, 16 per chunk; lane column n is c = 16 chunk + n.
// The batch has lk real keys and lq real query rows (per-batch lengths, else
// Lk and Lq).  Query row qi < lq sees keys j < lk with j <= lk - lq + qi
// under bottom-right causal masking; rows from lq on see no key.
struct DecodeUnit {
  int split, hk, b;
  bool ok;        // lane column is a real (query row, head)
  int hq, qi;     // its query head and query row (0 for padding columns)
  int lk;         // real keys of the batch
  int last_key;   // last visible key of that row (-1: none)
  int key_end;    // one past the last key any real row of the workgroup sees
};
// Workgroup columns: chunk holds columns [16 cpw chunk, 16 cpw (chunk + 1));
// 16-column block w of them (w < cpw) belongs to wave w when cpw > 1.
__device__ inline DecodeUnit decode_unit(const AttnParams& p, int n, int cpw = 1, int w = 0) {
  DecodeUnit u;
  int chunk, r;
  if (cpw == 1 || p.nsplit > 1) {
    // decode: (split, chunk, kv head, batch), split fastest
    u.split = blockIdx.x % p.nsplit;
    r = blockIdx.x / p.nsplit;
    chunk = r % p.nchunk;
    r /= p.nchunk;
  } else {
    // one split (prefill): (kv head, batch) fastest, so that the workgroups
    // launched first are the heaviest chunks of every head under causal
    // masking (later rows see more keys), and head h stays on XCD h % 8
    // when B * Hkv is a multiple of 8
    u.split = 0;
    const int nbh = p.B * p.Hkv;
    const int ci = blockIdx.x / nbh;
    chunk = p.causal ? p.nchunk - 1 - ci : ci;
    r = blockIdx.x % nbh;
  }
  u.hk = r % p.Hkv;
  u.b = r / p.Hkv;
  const int c = 16 * (cpw * chunk + w) + n;
  u.ok = c < p.Lq * p.group;
  const int cc = u.ok ? c : 0;
  u.qi = cc / p.group;
  u.hq = u.hk * p.group + cc % p.group;
  const int lq = batch_len(p.seqlens_q, u.b, p.Lq);
  u.lk = batch_len(p.seqlens_k, u.b, p.Lk);
  u.last_key = u.qi >= lq ? -1 : (p.causal ? u.lk - lq + u.qi : u.lk);
  // the workgroup's rows run from (16 cpw chunk) / G to (16 cpw chunk + 16 cpw
  // - 1) / G; under bottom-right causal masking its last real row sees the
  // most keys
  const int qfirst = 16 * cpw * chunk / p.group;
  const int qlast = min(min(16 * cpw * (chunk + 1) - 1, p.Lq * p.group - 1) / p.group, lq - 1);
  u.key_end = qfirst >= lq ? 0 : (p.causal ? max(0, u.lk - lq + qlast + 1) : u.lk);
  return u;
}

template <class T, int D>
struct DecodeCfg {
  static constexpr int ES = T::kBytes;
  static constexpr int VEC = T::kVec;
  static constexpr int NCH = D / VEC;                  // 16-byte chunks per row
  static constexpr bool F32 = (ES == 4);
#ifndef SDPA_DECODE_TILE_BYTES
#define SDPA_DECODE_TILE_BYTES 32768  // K + V bytes per key tile (D <= 128)
#endif
#ifndef SDPA_DECODE_MAX_STAGE_BYTES
#define SDPA_DECODE_MAX_STAGE_BYTES 81920  // double-buffer LDS when 2 stages fit in this
#endif
  static constexpr int TK = F32 ? (D >= 256 ? 16 : SDPA_DECODE_TILE_BYTES / (8 * D))
                                : (D >= 256 ? 32 : SDPA_DECODE_TILE_BYTES / (4 * D));
  static constexpr int NBLK = TK / 16;                 // 16-key blocks per tile
  static constexpr int KP = D * ES + 16;               // K row pitch (bytes)
  // 16-bit: V row-major, read transposed (ds_read_b64_tr_b16); a pitch of
  // 32 (mod 256) bytes spreads the 16 rows one read touches over the banks.
  // fp32: V^T written transposed by the loading threads.
  static constexpr int VP = F32 ? TK * ES + 16 : D * 2 + 32;
  static constexpr int K_BYTES = TK * KP;
  static constexpr int V_BYTES = F32 ? D * VP : TK * VP;
  static constexpr int NS = D * ES / 64;               // Q vectors per head row / 4
  // fp32 splits the Q.K^T contraction over the waves (a full fp32 Q row
  // would not fit the registers) and sums the partial scores in LDS; 16-bit
  // waves each form the whole S^T tile.
  static constexpr int QSPLIT = F32 ? (NS < kWaves ? NS : kWaves) : 1;
  static constexpr int NSW = NS / QSPLIT;              // Q vectors per wave
  static constexpr int X_BYTES = F32 ? QSPLIT * NBLK * 64 * 16 : 0;
  static constexpr int NOB = D / 16 / kWaves;          // 16-row blocks of O^T per wave
  static constexpr int K_IT = TK * NCH / kThreads;
  static constexpr int V_IT = F32 ? (TK / 4) * NCH / kThreads : TK * NCH / kThreads;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int STAGES = 2 * STAGE <= SDPA_DECODE_MAX_STAGE_BYTES ? 2 : 1;
  static_assert(NS % QSPLIT == 0, "Q split");
  static_assert(NOB >= 1, "O split");
  static_assert(K_IT >= 1 && TK * NCH % kThreads == 0, "K tile split");
  static_assert(V_IT >= 1, "V tile split");
  static_assert(F32 ? TK % 16 == 0 : TK % 32 == 0, "tile keys");
};

template <int NCH>
__device__ constexpr int vt_row(int c, int e) { return c + NCH * e; }
template <int NCH, int VEC>
__device__ constexpr int vt_row_to_d(int rho) { return VEC * (rho % NCH) + rho / NCH; }

template <class T, int D, bool MASK, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void decode_f32_kernel(AttnParams p) {
  using C = DecodeCfg<T, D>;
  using S = typename T::storage;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::STAGES * C::STAGE + (C::X_BYTES ? C::X_BYTES : 16)];
  f32x4* Sx = (f32x4*)(smem + C::STAGES * C::STAGE);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;   // head column of the 16x16 tiles (also the K row of the A operand)
  const int g4 = lane >> 4;  // lane group

  const DecodeUnit u = decode_unit(p, n);
  const int split = u.split, hk = u.hk, b = u.b, hq = u.hq, qi = u.qi;
  const bool head_ok = u.ok;

  const int kbeg = split * p.split_len;
  const int kend = min(u.key_end, kbeg + p.split_len);
  const int ntiles = kend > kbeg ? (kend - kbeg + C::TK - 1) / C::TK : 0;

  const S* kp = (const S*)p.k + b * p.ks[0] + hk * p.ks[1];
  const S* vp = (const S*)p.v + b * p.vs[0] + hk * p.vs[1];

  // ---- Q^T operand (B of S^T = K . Q^T): vector s holds chunk 4*(s0+s) + g4
  u32x4 qreg[C::NSW];
  {
    const int s0 = wave < C::QSPLIT ? wave * C::NSW : 0;
    const S* row = (const S*)p.q + b * p.qs[0] + (int64_t)hq * p.qs[1] + (int64_t)qi * p.qs[2];
    const int nqk = p.Dqk / C::VEC;  // real chunks of a q / k row; the rest is zero
#pragma unroll
    for (int s = 0; s < C::NSW; ++s) {
      const int ch = 4 * (s0 + s) + g4;
      u32x4 v = ldg16_cached(row + min(ch, nqk - 1) * C::VEC);
      qreg[s] = head_ok && ch < nqk ? v : u32x4{0, 0, 0, 0};
    }
  }

  // mask row of this lane's head: four consecutive keys per 16-key block
  const int64_t mbase = MASK ? b * p.ms[0] + (int64_t)hq * p.ms[1] + (int64_t)qi * p.ms[2] : 0;
  const float* mrow = (const float*)p.mask + mbase;  // read as such only for fp32 masks
  const bool mask_vec = MASK && !p.mask_bool && p.ms[3] == 1 && (((uintptr_t)mrow) & 15) == 0;

  f32x4 acc[C::NOB];
#pragma unroll
  for (int i = 0; i < C::NOB; ++i) acc[i] = f32x4{};
  float m_run = kNegInf;
  float l_run = 0.f;

  // ---- tile loads (buffer resources zero-fill keys at or past kend, and
  //      chunks past the real head dims, whose offset is set to the tile's
  //      byte count)
  auto valid_bytes = [&](int j0, int64_t stride, int real_d) -> uint32_t {
    return (uint32_t)((int64_t)(min(kend - j0, C::TK) - 1) * stride * C::ES + real_d * C::ES);
  };
  u32x4 kpre[C::K_IT];
  u32x4 vpre[C::V_IT][C::F32 ? 4 : 1];
  auto prefetch = [&](int j0) {
    const uint32_t nk = valid_bytes(j0, p.ks[2], p.Dqk), nv = valid_bytes(j0, p.vs[2], p.Dv);
    const auto rk = make_rsrc(kp + (int64_t)j0 * p.ks[2], nk);
    const auto rv = make_rsrc(vp + (int64_t)j0 * p.vs[2], nv);
#pragma unroll
    for (int it = 0; it < C::K_IT; ++it) {
      const int u = tid + kThreads * it;
      const int c = u % C::NCH;
      kpre[it] = buf_load16(rk, c * C::VEC < p.Dqk ? (uint32_t)((u / C::NCH) * p.ks[2] * C::ES + c * 16) : kNoLoad);
    }
#pragma unroll
    for (int it = 0; it < C::V_IT; ++it) {
      const int u = tid + kThreads * it;
      if constexpr (C::F32) {
        const int kg = u / C::NCH, c = u % C::NCH;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vpre[it][r] =
              buf_load16(rv, c * C::VEC < p.Dv ? (uint32_t)((4 * kg + r) * p.vs[2] * C::ES + c * 16) : kNoLoad);
      } else {
        const int c = u % C::NCH;
        vpre[it][0] =
            buf_load16(rv, c * C::VEC < p.Dv ? (uint32_t)((u / C::NCH) * p.vs[2] * C::ES + c * 16) : kNoLoad);
      }
    }
  };
  auto store_tile = [&](uint8_t* st) {
    uint8_t* Ks = st;
    uint8_t* Vs = st + C::K_BYTES;
#pragma unroll
    for (int it = 0; it < C::K_IT; ++it) {
      const int u = tid + kThreads * it;
      lds_write16(Ks + (u / C::NCH) * C::KP + (u % C::NCH) * 16, kpre[it]);
    }
#pragma unroll
    for (int it = 0; it < C::V_IT; ++it) {
      const int u = tid + kThreads * it;
      if constexpr (C::F32) {
        const int kg = u / C::NCH, c = u % C::NCH;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 w = {vpre[it][0][e], vpre[it][1][e], vpre[it][2][e], vpre[it][3][e]};
          lds_write16(Vs + vt_row<C::NCH>(c, e) * C::VP + kg * 16, w);
        }
      } else {
        lds_write16(Vs + (u / C::NCH) * C::VP + (u % C::NCH) * 16, vpre[it][0]);
      }
    }
  };

  // lane part of the transposed V read (16-bit): key row 4*g4 + r/4, head-dim
  // columns 4*(r%4) of the 16-column block
  const uint32_t vtr_lane = (4 * g4 + (n >> 2)) * C::VP + 4 * (n & 3) * 2;

  auto compute = [&](const uint8_t* st, int j0) {
    const uint8_t* Ks = st;
    const uint8_t* Vs = st + C::K_BYTES;
    // ---- S^T = K . Q^T (16-bit: every wave; fp32: split over the waves)
    f32x4 sc[C::NBLK];
    if constexpr (!C::F32) {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        f32x4 s = f32x4{};
        const uint8_t* krow = Ks + (16 * blk + n) * C::KP + g4 * 16;
#pragma unroll
        for (int ss = 0; ss < C::NSW; ++ss) s = mma16(T{}, lds_read16(krow + ss * 64), qreg[ss], s);
        sc[blk] = s;
      }
    } else {
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
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        f32x4 s = Sx[blk * 64 + lane];
#pragma unroll
        for (int w = 1; w < C::QSPLIT; ++w) s += Sx[(w * C::NBLK + blk) * 64 + lane];
        sc[blk] = s;
      }
    }
    // ---- scale, mask, key tail, running max (identical in all waves)
    float mx = kNegInf;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
      const int jb = j0 + 16 * blk + 4 * g4;
      f32x4 mk = f32x4{};
      if (MASK) {
        if (mask_vec) {
          const auto rm = make_rsrc(mrow + jb, (uint32_t)max(0, kend - jb) * 4);
          mk = __builtin_bit_cast(f32x4, buf_load16(rm, 0));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            mk[r] = mask_val(p.mask, p.mask_bool, mbase + (int64_t)min(jb + r, kend - 1) * p.ms[3]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sc[blk][r] * p.scale_log2;
        if (MASK) x += kLog2e * mk[r];
        x = (jb + r < kend && jb + r <= u.last_key) ? x : kNegInf;
        sc[blk][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor16(mx));
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run)) {
      const float corr = m_new > m_run ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < C::NOB; ++i) acc[i] *= corr;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = fast_exp2(sc[blk][r] - m_use);
        sc[blk][r] = pr;
        l_run += pr;
      }

    // ---- O^T += V^T . P^T on this wave's rows
    if constexpr (C::F32) {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        const u32x4 pb = {as_uint(sc[blk][0]), as_uint(sc[blk][1]), as_uint(sc[blk][2]), as_uint(sc[blk][3])};
#pragma unroll
        for (int i = 0; i < C::NOB; ++i) {
          const int row = 16 * (wave * C::NOB + i) + n;
          acc[i] = mma16(T{}, lds_read16(Vs + row * C::VP + (16 * blk + 4 * g4) * 4), pb, acc[i]);
        }
      }
    } else {
      // k-slot 8*g4 + 4a + c <-> key 16a + 4*g4 + c of the 32-key pair pp
#pragma unroll
      for (int pp = 0; pp < C::NBLK / 2; ++pp) {
        u32x4 hi, lo;
        if constexpr (std::is_same<T, TBF16>::value) {
          // bf16 P carries 8 significant bits: feed P = hi + lo (the matrix
          // cores have ample headroom in this bandwidth-bound kernel)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t h, l;
            T::split2(sc[2 * pp + (e >> 1)][2 * (e & 1)], sc[2 * pp + (e >> 1)][2 * (e & 1) + 1], h, l);
            hi[e] = h;
            lo[e] = l;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            hi[e] = cvt_pk(T{}, sc[2 * pp + (e >> 1)][2 * (e & 1)], sc[2 * pp + (e >> 1)][2 * (e & 1) + 1]);
        }
        const uint8_t* vb = Vs + vtr_lane + 32 * pp * C::VP;
#pragma unroll
        for (int i = 0; i < C::NOB; ++i) {
          const int d0 = 16 * (wave * C::NOB + i);
          const u32x2 a0 = lds_read_tr16(vb + d0 * 2);
          const u32x2 a1 = lds_read_tr16(vb + 16 * C::VP + d0 * 2);
          const u32x4 va = {a0[0], a0[1], a1[0], a1[1]};
          acc[i] = mma16(T{}, va, hi, acc[i]);
          if constexpr (std::is_same<T, TBF16>::value) acc[i] = mma16(T{}, va, lo, acc[i]);
        }
      }
    }
  };

  if (ntiles > 0) {
    prefetch(kbeg);
    if constexpr (C::STAGES == 2) store_tile(smem);
  }
  if constexpr (C::STAGES == 2) {
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int j0 = kbeg + t * C::TK;
      if (t + 1 < ntiles) prefetch(j0 + C::TK);
      compute(smem + (t & 1) * C::STAGE, j0);
      if (t + 1 < ntiles) store_tile(smem + ((t + 1) & 1) * C::STAGE);
      __syncthreads();
    }
  } else {
    for (int t = 0; t < ntiles; ++t) {
      const int j0 = kbeg + t * C::TK;
      __syncthreads();
      store_tile(smem);
      __syncthreads();
      if (t + 1 < ntiles) prefetch(j0 + C::TK);
      compute(smem, j0);
    }
  }

  // ---- epilogue ----
  float l_tot = l_run + xor16(l_run);
  l_tot = sum_xor32(l_tot);
  const int64_t bh = ((int64_t)b * p.Hq + hq) * p.Lq + qi;  // (b, hq, query row)
  auto out_d = [&](int i, int r) {
    const int rho = 16 * (wave * C::NOB + i) + 4 * g4 + r;
    return C::F32 ? vt_row_to_d<C::NCH, C::VEC>(rho) : rho;
  };
  if constexpr (SPLIT) {
    if (head_ok) {
      float* po = p.part_o + (bh * p.nsplit + split) * D;
#pragma unroll
      for (int i = 0; i < C::NOB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) po[out_d(i, r)] = acc[i][r];
      if (wave == 0 && g4 == 0) {
        float* pml = p.part_ml + (bh * p.nsplit + split) * 2;
        pml[0] = m_run;
        pml[1] = l_tot;
      }
    }
  } else {
    float M = m_run, Ltot = l_tot;
    if (p.sinks) {
      const float sk = p.sinks[hq] * kLog2e;
      M = fmaxf(m_run, sk);
      if (M != kNegInf) Ltot = l_tot * fast_exp2(m_run - M) + fast_exp2(sk - M);
    }
    float so = 0.f, lse = kNegInf;
    if (M != kNegInf && Ltot > 0.f) {
      so = (p.sinks ? fast_exp2(m_run - M) : 1.f) / Ltot;
      lse = (M + fast_log2(Ltot)) * kLn2;
    }
    if (head_ok) {
      S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)qi * p.os[2];
#pragma unroll
      for (int i = 0; i < C::NOB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (out_d(i, r) < p.Dv) orow[out_d(i, r)] = T::from_f32(acc[i][r] * so);
      if (p.lse && wave == 0 && g4 == 0) p.lse[bh] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// 16-bit decode: K / V stream HBM -> LDS by direct (VGPR-free) buffer loads
// into a ring of NST tile stages; a wave waits only for its own loads of the
// tile it is about to use, so NST - 2 further tiles stay in flight while one
// is consumed.  Rows are stored unpadded (the direct loads fill 1 KiB lines)
// with 16-byte chunks XOR-swizzled by row, which keeps both the Q.K^T operand
// reads (16 rows, one chunk) and the transposed V reads (16 rows, two chunks)
// free of bank conflicts.
// ---------------------------------------------------------------------------
#ifndef SDPA_DECODE16_TK128
#define SDPA_DECODE16_TK128 64  // keys per tile at D <= 128
#endif
#ifndef SDPA_DECODE16_STAGES
#define SDPA_DECODE16_STAGES 2  // ring stages at D <= 128
#endif
#ifndef SDPA_DECODE16_STAGES_LARGE
#define SDPA_DECODE16_STAGES_LARGE 2  // ring stages at D >= 256 (32 KiB stages)
#endif
template <int D, int TKO = 0, int NWV = kWaves, int NSTO = 0>
struct Dec16 {
  static constexpr int RB = D * 2;                 // row bytes
  static constexpr int NCH = D / 8;                // 16-byte chunks per row
  static constexpr int TK = TKO ? TKO : (D >= 512 ? 16 : (D >= 256 ? 32 : SDPA_DECODE16_TK128 * 128 / D));
  static constexpr int TILE = TK * RB;             // bytes of the K (or V) tile
  static constexpr int NST = NSTO ? NSTO : (D >= 256 ? SDPA_DECODE16_STAGES_LARGE : SDPA_DECODE16_STAGES);
  static constexpr int STAGE = 2 * TILE;
  static constexpr int LINES = TILE / 1024;        // 1 KiB load lines per K (or V) tile
  static constexpr int LPW = 2 * LINES / NWV;      // load instructions per wave per tile
  static constexpr int NBLK = TK / 16;
  static constexpr int NQ = D / 32;                // Q vectors per lane
  static constexpr int NOB = D / 16 / kWaves;      // O^T row blocks per wave
  static_assert(LINES % NWV == 0 && LINES >= NWV, "tile lines");
  static_assert(NST >= 2 && (NST - 2) * LPW < 64, "ring depth");
};

// Wait until at most rem later tiles' direct loads (LPW per tile) are in
// flight: the oldest tile has landed.  R (the ring's spare depth) bounds rem.
template <int LPW, int R>
__device__ inline void wait_ring(int rem) {
  if constexpr (R > 0) {
    if (rem >= R) {
      wait_vmcnt<R * LPW>();
      return;
    }
    wait_ring<LPW, R - 1>(rem);
  } else {
    wait_vmcnt<0>();
  }
}

// chunk swizzle of a row (both K and V): low chunk bits ^= f(row)
template <int NCH>
__device__ constexpr int chunk_swz(int row) { return NCH >= 16 ? (row & 15) : ((row >> 1) & (NCH - 1)); }

// CPW 16-column blocks per workgroup, NW = max(CPW, 4) waves, WPB = NW / CPW
// waves per block.  The waves of a block each compute the block's scores and
// own 1 / WPB of its O^T rows: CPW = 1 (decode, G * Lq <= 16) shares one
// block among four waves; CPW = 2 and 4 (multi-query decode) let K / V stream
// once for up to 64 columns; CPW = 4 and 8 (prefill at head dim 512) give
// every wave its own 16 columns and all O^T rows.  With CPW > 1 the tiles are
// a multiple of 32 keys (at D = 512: 32 keys, 128 KiB of LDS) and P.V runs as
// 16x16x32 products, 32 keys per step, at the full matrix rate.
// NSTO (ring stages, 0 = default) deepens the ring where a grid of at most
// one workgroup per compute unit leaves LDS to spare.
template <class T, int D, bool MASK, bool SPLIT, int CPW = 1, int NSTO = 0>
__global__ __launch_bounds__(64 * (CPW > kWaves ? CPW : kWaves), 1) void decode16_kernel(AttnParams p) {
  constexpr int NW = CPW > kWaves ? CPW : kWaves;  // waves per workgroup
  constexpr int WPB = NW / CPW;                     // waves per 16-column block
  using C = Dec16<D, (CPW > 1 && D >= 512 ? 32 : 0), NW, NSTO>;
  using S = uint16_t;
  static_assert(CPW == 1 || C::NBLK % 2 == 0, "32-key products");
  constexpr int NOB = D / 16 / WPB;  // O^T row blocks per wave
  __shared__ __attribute__((aligned(1024))) uint8_t ring[C::NST * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int ob0 = (wave % WPB) * NOB;  // first O^T row block of this wave

  const DecodeUnit u = decode_unit(p, n, CPW, wave / WPB);
  const int split = u.split, hk = u.hk, b = u.b, hq = u.hq, qi = u.qi;
  const bool head_ok = u.ok;

  const int kbeg = split * p.split_len;
  const int kend = min(u.key_end, kbeg + p.split_len);
  const int ntiles = kend > kbeg ? (kend - kbeg + C::TK - 1) / C::TK : 0;

  const S* kp = (const S*)p.k + b * p.ks[0] + hk * p.ks[1];
  const S* vp = (const S*)p.v + b * p.vs[0] + hk * p.vs[1];

  // Q^T operand: vector s = chunk 4s + g4 of the head row
  u32x4 qreg[C::NQ];
  {
    const S* row = (const S*)p.q + b * p.qs[0] + (int64_t)hq * p.qs[1] + (int64_t)qi * p.qs[2];
    const int nqk = p.Dqk / 8;  // real chunks of a q / k row; the rest is zero
#pragma unroll
    for (int s = 0; s < C::NQ; ++s) {
      const u32x4 v = ldg16_cached(row + min(4 * s + g4, nqk - 1) * 8);
      qreg[s] = head_ok && 4 * s + g4 < nqk ? v : u32x4{0, 0, 0, 0};
    }
  }
  const int64_t mbase = MASK ? b * p.ms[0] + (int64_t)hq * p.ms[1] + (int64_t)qi * p.ms[2] : 0;
  const float* mrow = (const float*)p.mask + mbase;  // read as such only for fp32 masks

  // ---- per-lane direct-load offsets (fixed across tiles): wave w issues
  //      lines w, w + 4, ...; lines [0, LINES) are K, the rest V
  //      (a chunk past the real head dim loads nothing: kNoLoad)
  uint32_t voff[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int ln = (wave + NW * i) % C::LINES;
    const int pos = ln * 64 + lane;                 // 16-byte slot within the tile
    const int row = pos / C::NCH, pch = pos % C::NCH;
    const int lch = pch ^ chunk_swz<C::NCH>(row);
    const bool is_k = (wave + NW * i) < C::LINES;
    const int64_t stride = is_k ? p.ks[2] : p.vs[2];
    voff[i] = lch * 8 < (is_k ? p.Dqk : p.Dv) ? (uint32_t)(row * stride * 2 + lch * 16) : kNoLoad;
  }
  auto valid_bytes = [&](int j0, int64_t stride, int real_d) -> uint32_t {
    return (uint32_t)((int64_t)(min(kend - j0, C::TK) - 1) * stride * 2 + real_d * 2);
  };
  auto issue = [&](int t) {
    if (t >= ntiles) return;
    const int j0 = kbeg + t * C::TK;
    const S* tk = kp + (int64_t)j0 * p.ks[2];
    const S* tv = vp + (int64_t)j0 * p.vs[2];
    const uint32_t nk = valid_bytes(j0, p.ks[2], p.Dqk), nv = valid_bytes(j0, p.vs[2], p.Dv);
    const uint32_t st = lds_addr(ring) + (t % C::NST) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int gl = wave + NW * i;
      if (i < C::LINES / NW) dma16(tk, nk, st + gl * 1024, voff[i], 0);
      else dma16(tv, nv, st + C::TILE + (gl - C::LINES) * 1024, voff[i], 0);
    }
  };

  // (per-lane LDS read offsets: in the tile loop; K rows 16 blk + n, V rows
  // 16 blk + 4 g4 + n / 4)

  f32x4 acc[NOB];
#pragma unroll
  for (int i = 0; i < NOB; ++i) acc[i] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  // bf16 P goes in as hi + lo: always with one shared block (CPW = 1: the
  // matrix cores have ample headroom in this bandwidth-bound form); with
  // CPW > 1, where the products double per wave, only on workgroups whose rows
  // may see few keys (at most 256 in this split, or any row under a mask), as
  // in the prefill kernel
  const bool split_p = std::is_same<T, TBF16>::value && (CPW == 1 || MASK || kend - kbeg <= 256);

  // mask values for tile t, loaded one tile ahead
  auto load_mask = [&](int t, f32x4* mk) {
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
      const int jb = kbeg + t * C::TK + 16 * blk + 4 * g4;
      const float* mp = mrow + (int64_t)jb * p.ms[3];
      if (!p.mask_bool && p.ms[3] == 1 && jb + 3 < kend && (((uintptr_t)mp) & 15) == 0) {
        mk[blk] = *(const f32x4*)mp;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          mk[blk][r] = mask_val(p.mask, p.mask_bool, mbase + (int64_t)max(kbeg, min(jb + r, kend - 1)) * p.ms[3]);
      }
    }
  };
  f32x4 mk_next[C::NBLK];
  if (MASK && ntiles > 0) load_mask(0, mk_next);

#pragma unroll
  for (int t = 0; t < C::NST - 1; ++t) issue(t);

  for (int t = 0; t < ntiles; ++t) {
    // this wave's loads of tile t have landed once at most `rem` later tiles remain
    const int rem = min(C::NST - 2, ntiles - 1 - t);
    wait_ring<C::LPW, C::NST - 2>(rem);
    lds_barrier();  // ... and every wave's; tile t - 1 is no longer read
    const int j0 = kbeg + t * C::TK;
    // this tile's mask values were loaded in the previous iteration; the next
    // tile's are issued before the direct loads, so waiting for them never
    // waits for those
    f32x4 mk[C::NBLK];
    if (MASK) {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) mk[blk] = mk_next[blk];
      if (t + 1 < ntiles) load_mask(t + 1, mk_next);
    }
    issue(t + C::NST - 1);

    const uint8_t* Ks = ring + (t % C::NST) * C::STAGE;
    const uint8_t* Vs = Ks + C::TILE;
    // The wide form (CPW > 1) derives its per-lane LDS offsets from a fresh
    // copy of the lane index every tile: held across the loop they do not
    // fit its registers, and reloading them from scratch waited on the ring's
    // loads in flight (the reload's wait counts those too).
    const int lane_t = CPW > 1 ? fresh(lane) : lane;
    const int n_t = lane_t & 15, g4_t = lane_t >> 4;
    const int swk_t = chunk_swz<C::NCH>(n_t);
    const int vrow_t = 4 * g4_t + (n_t >> 2);
    const int swv_t = chunk_swz<C::NCH>(vrow_t);
    const uint32_t vlane_t = vrow_t * C::RB + (n_t & 1) * 8;
    // ---- S^T = K . Q^T
    f32x4 sc[C::NBLK];
    if constexpr (CPW > 1 && !(MASK && CPW >= 8)) {
      // key operands read two products ahead (a ring of two), a fence on
      // each side of every product: read just before its product, each
      // operand's LDS latency was waited out in full (causal GQA-8 D512 bf16
      // 772 -> 748 us, MHA-8 400 -> 382 us).  Not in the masked eight-block
      // kernel, whose loop already spills.
      auto kread = [&](int i) {  // i = blk * NQ + ss
        const uint8_t* krow = Ks + (16 * (i / C::NQ) + n_t) * C::RB;
        return lds_read16(krow + ((4 * (i % C::NQ) + g4_t) ^ swk_t) * 16);
      };
      constexpr int N = C::NBLK * C::NQ, LA = 2;
      u32x4 kr[LA];
#pragma unroll
      for (int j = 0; j < LA; ++j) kr[j] = kread(j < N ? j : 0);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int blk = i / C::NQ, ss = i % C::NQ;
        const u32x4 ka = kr[i % LA];
        if (i + LA < N) kr[i % LA] = kread(i + LA);
        __builtin_amdgcn_sched_barrier(0);
        sc[blk] = mma16(T{}, ka, qreg[ss], ss == 0 ? f32x4{} : sc[blk]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        f32x4 s = f32x4{};
        const uint8_t* krow = Ks + (16 * blk + n_t) * C::RB;
#pragma unroll
        for (int ss = 0; ss < C::NQ; ++ss) s = mma16(T{}, lds_read16(krow + ((4 * ss + g4_t) ^ swk_t) * 16), qreg[ss], s);
        sc[blk] = s;
      }
    }
    // ---- scale, mask, key tail, running max
    float mx = kNegInf;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
      const int jb = j0 + 16 * blk + 4 * g4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sc[blk][r] * p.scale_log2;
        if (MASK) x += kLog2e * mk[blk][r];
        x = (jb + r < kend && jb + r <= u.last_key) ? x : kNegInf;
        sc[blk][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor16(mx));
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run)) {
      const float corr = m_new > m_run ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < NOB; ++i) acc[i] *= corr;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    if constexpr (CPW > 1) {
      // ---- O^T += V^T . P^T, 32 keys per step: k-slot 8 g4 + e <-> key
      //      32 bp + 4 g4 + e (e < 4) or 32 bp + 16 + 4 g4 + e - 4 (e >= 4)
#pragma unroll
      for (int bp = 0; bp < C::NBLK / 2; ++bp) {
        float pr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          pr[r] = fast_exp2(sc[2 * bp + r / 4][r % 4] - m_use);
          l_run += pr[r];
        }
        u32x4 hi, lo = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) hi[e] = cvt_pk(T{}, pr[2 * e], pr[2 * e + 1]);
        const uint8_t* vb = Vs + 32 * bp * C::RB + vlane_t;
        if constexpr (CPW >= 8) {
          // Eight 16-column waves sit at the register limit: the two-loop
          // form below spilled inside the loop here (causal GQA-8 D512 bf16
          // 0.9 -> 4.4 ms), so the split choice stays beside each product,
          // and each value operand is read one block ahead instead, in the
          // block before its product's (bf16 897 -> 770 us, fp16 735 ->
          // 712 us).
          if constexpr (std::is_same<T, TBF16>::value) {
            if (split_p) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                uint32_t h, l;
                T::split2(pr[2 * e], pr[2 * e + 1], h, l);
                hi[e] = h;
                lo[e] = l;
              }
            }
          }
          auto vread = [&](int i) {
            const int lch = 2 * (ob0 + i) + ((n_t >> 1) & 1);
            const u32x2 v0 = lds_read_tr16(vb + ((lch ^ swv_t) * 16));
            const u32x2 v1 = lds_read_tr16(vb + 16 * C::RB + ((lch ^ swv_t) * 16));
            return u32x4{v0[0], v0[1], v1[0], v1[1]};
          };
          u32x4 va = vread(0);
#pragma unroll
          for (int i = 0; i < NOB; ++i) {
            u32x4 vn = va;
            if (i + 1 < NOB) vn = vread(i + 1);
            acc[i] = mma16(T{}, va, hi, acc[i]);
            if (split_p) acc[i] = mma16(T{}, va, lo, acc[i]);
            if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            va = vn;
          }
        } else {
          // The split (P = hi + lo, lo the rounding hi left) and unsplit
          // forms as separate loops under one branch: a runtime choice beside
          // every product put a branch around each one, and nothing was
          // scheduled across them (causal MHA-8 D512 bf16 484 -> 400 us).
          auto pv_step = [&](auto split_tag) {
#pragma unroll
            for (int i = 0; i < NOB; ++i) {
              const int lch = 2 * (ob0 + i) + ((n_t >> 1) & 1);
              const u32x2 v0 = lds_read_tr16(vb + ((lch ^ swv_t) * 16));
              const u32x2 v1 = lds_read_tr16(vb + 16 * C::RB + ((lch ^ swv_t) * 16));
              const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
              acc[i] = mma16(T{}, va, hi, acc[i]);
              if constexpr (decltype(split_tag)::value) acc[i] = mma16(T{}, va, lo, acc[i]);
              if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
          };
          if (std::is_same<T, TBF16>::value && split_p) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              lo[e] = T::pack2(pr[2 * e] - T::to_f32((uint16_t)(hi[e] & 0xffffu)),
                               pr[2 * e + 1] - T::to_f32((uint16_t)(hi[e] >> 16)));
            pv_step(std::true_type{});
          } else {
            pv_step(std::false_type{});
          }
        }
      }
    } else {
    // ---- O^T += V^T . P^T, 16 keys per step (k-slot 4 g4 + e <-> key 4 g4 + e)
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = fast_exp2(sc[blk][r] - m_use);
        l_run += pr[r];
      }
      u32x2 hi = u32x2{cvt_pk(T{}, pr[0], pr[1]), cvt_pk(T{}, pr[2], pr[3])}, lo = u32x2{0, 0};
      if constexpr (std::is_same<T, TBF16>::value) {
        if (split_p) {
          // bf16 P carries 8 significant bits: P = hi + lo
          uint32_t h0, l0, h1, l1;
          T::split2(pr[0], pr[1], h0, l0);
          T::split2(pr[2], pr[3], h1, l1);
          hi = u32x2{h0, h1};
          lo = u32x2{l0, l1};
        }
      }
      const uint8_t* vb = Vs + 16 * blk * C::RB + vlane_t;
#pragma unroll
      for (int i = 0; i < NOB; ++i) {
        const int lch = 2 * (ob0 + i) + ((n_t >> 1) & 1);  // chunk of columns d0 + 4(n%4)
        const u32x2 va = lds_read_tr16(vb + ((lch ^ swv_t) * 16));
        acc[i] = mma16k16(T{}, va, hi, acc[i]);
        if (split_p) acc[i] = mma16k16(T{}, va, lo, acc[i]);
      }
    }
    }
  }

  // ---- epilogue (identical in every wave; each writes its rows of O)
  float l_tot = l_run + xor16(l_run);
  l_tot = sum_xor32(l_tot);
  const int64_t bh = ((int64_t)b * p.Hq + hq) * p.Lq + qi;  // (b, hq, query row)
  if constexpr (SPLIT) {
    if (head_ok) {
      float* po = p.part_o + (bh * p.nsplit + split) * D;
#pragma unroll
      for (int i = 0; i < NOB; ++i)
        *(f32x4*)(po + 16 * (ob0 + i) + 4 * g4) = acc[i];
      if (wave % WPB == 0 && g4 == 0) {
        float* pml = p.part_ml + (bh * p.nsplit + split) * 2;
        pml[0] = m_run;
        pml[1] = l_tot;
      }
    }
  } else {
    float M = m_run, Ltot = l_tot;
    if (p.sinks) {
      const float sk = p.sinks[hq] * kLog2e;
      M = fmaxf(m_run, sk);
      if (M != kNegInf) Ltot = l_tot * fast_exp2(m_run - M) + fast_exp2(sk - M);
    }
    float so = 0.f, lse = kNegInf;
    if (M != kNegInf && Ltot > 0.f) {
      so = (p.sinks ? fast_exp2(m_run - M) : 1.f) / Ltot;
      lse = (M + fast_log2(Ltot)) * kLn2;
    }
    if (head_ok) {
      S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)qi * p.os[2];
#pragma unroll
      for (int i = 0; i < NOB; ++i) {
        const f32x4 o = acc[i] * so;
        if (16 * (ob0 + i) + 4 * g4 < p.Dv)
          *(u32x2*)(orow + 16 * (ob0 + i) + 4 * g4) = u32x2{cvt_pk(T{}, o[0], o[1]), cvt_pk(T{}, o[2], o[3])};
      }
      if (p.lse && wave % WPB == 0 && g4 == 0) p.lse[bh] = lse;
    }
  }
}

// Merge pass.  Workgroup (b, hq, 64-element slice of the head dim); thread
// (split group sg, element quad dq) takes splits sg, sg + NSG, ...  A thread
// fetches the (m_s, l_s, O~_s) of several splits at once (no load waits on a
// reduction, so the partials cost one memory round trip) and folds them into
// its own (m, l, O~) by the same rescaling as the online softmax; the NSG
// split groups are then combined in LDS with the sink:
//   M = max(max_g m_g, sink),  L = sum_g l_g 2^(m_g - M) + 2^(sink - M),
//   O = sum_g O~_g 2^(m_g - M) / L.  Splits with m_s = -inf weigh 0.
constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 64;  // head-dim elements per workgroup
constexpr int kMergeUnroll = 4; // splits a thread fetches together

template <class T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnParams p) {
  using S = typename T::storage;
  constexpr int NDQ = (D < kMergeCols ? D : kMergeCols) / 4;  // float4 columns per workgroup
  constexpr int NSG = kMergeThreads / NDQ;                      // split groups
  __shared__ f32x4 part[NSG][NDQ];
  __shared__ float gm[NSG], gl[NSG];
  const int tid = threadIdx.x;
  const int nslice = D / (NDQ * 4);
  const int64_t bh = blockIdx.x / nslice;  // ((b * Hq + hq) * Lq + qi)
  const int d0 = (blockIdx.x % nslice) * NDQ * 4;
  const int qi = (int)(bh % p.Lq);
  const int hq = (int)(bh / p.Lq % p.Hq);
  const int b = (int)(bh / p.Lq / p.Hq);
  const float* pml = p.part_ml + bh * p.nsplit * 2;
  const float* po = p.part_o + bh * p.nsplit * D;
  const int dq = tid % NDQ, sg = tid / NDQ;

  float m = kNegInf, l = 0.f;
  f32x4 o = f32x4{};
  for (int s0 = sg; s0 < p.nsplit; s0 += kMergeUnroll * NSG) {
    float ms[kMergeUnroll], ls[kMergeUnroll];
    f32x4 os[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int sp = s0 + u * NSG;
      const bool in = sp < p.nsplit;
      ms[u] = in ? pml[2 * sp] : kNegInf;
      ls[u] = in ? pml[2 * sp + 1] : 0.f;
      os[u] = in ? *(const f32x4*)(po + (int64_t)sp * D + d0 + 4 * dq) : f32x4{};
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      if (ms[u] == kNegInf) continue;
      const float mn = fmaxf(m, ms[u]);
      const float a = fast_exp2(m - mn), w = fast_exp2(ms[u] - mn);  // m = -inf: a = 0
      l = l * a + ls[u] * w;
      o = o * a + os[u] * w;
      m = mn;
    }
  }
  part[sg][dq] = o;
  if (dq == 0) {
    gm[sg] = m;
    gl[sg] = l;
  }
  __syncthreads();
  if (sg == 0) {
    const float sk = p.sinks ? p.sinks[hq] * kLog2e : kNegInf;
    float M = sk;
    for (int g = 0; g < NSG; ++g) M = fmaxf(M, gm[g]);
    float L = 0.f;
    f32x4 acc = f32x4{};
    if (M != kNegInf) {
      for (int g = 0; g < NSG; ++g) {
        if (gm[g] == kNegInf) continue;
        const float w = fast_exp2(gm[g] - M);
        L += gl[g] * w;
        acc += part[g][dq] * w;
      }
      if (p.sinks) L += fast_exp2(sk - M);
    }
    const bool live = M != kNegInf && L > 0.f;
    const float inv = live ? 1.f / L : 0.f;
    S* orow = (S*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)qi * p.os[2] + d0 + 4 * dq;
    if (d0 + 4 * dq < p.Dv)
#pragma unroll
      for (int e = 0; e < 4; ++e) orow[e] = T::from_f32(acc[e] * inv);
    if (p.lse && blockIdx.x % nslice == 0 && dq == 0)
      p.lse[bh] = live ? (M + fast_log2(L)) * kLn2 : kNegInf;
  }
}

#ifndef SDPA_DECODE_DEEP_RING_MAX_WG
#define SDPA_DECODE_DEEP_RING_MAX_WG 256
#endif
#ifndef SDPA_DECODE_DEEP_STAGES
#define SDPA_DECODE_DEEP_STAGES 4
#endif
constexpr int kDeepStages = SDPA_DECODE_DEEP_STAGES;
template <class T, int D, bool SPLIT>
void launch16(const AttnParams& p, int cpw, bool mask, dim3 grid, hipStream_t s) {
  const dim3 block(kThreads);  // four waves for CPW <= 4
  // At D >= 256 a stage holds 32 KiB of K and V.  A grid that fits one
  // workgroup per compute unit keeps only the one workgroup's loads in
  // flight per CU, so it gets a four-stage ring (128 KiB: three tiles in
  // flight); larger grids keep two stages and two workgroups per CU.
  constexpr bool kDeep = D >= 256;
  const bool deep = kDeep && grid.x <= (unsigned)SDPA_DECODE_DEEP_RING_MAX_WG;
  switch (cpw) {
    case 1:
      if constexpr (kDeep) {
        if (deep) {
          if (mask) hipLaunchKernelGGL((decode16_kernel<T, D, true, SPLIT, 1, kDeepStages>), grid, block, 0, s, p);
          else hipLaunchKernelGGL((decode16_kernel<T, D, false, SPLIT, 1, kDeepStages>), grid, block, 0, s, p);
          break;
        }
      }
      if (mask) hipLaunchKernelGGL((decode16_kernel<T, D, true, SPLIT, 1>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((decode16_kernel<T, D, false, SPLIT, 1>), grid, block, 0, s, p);
      break;
    case 2:
      if (mask) hipLaunchKernelGGL((decode16_kernel<T, D, true, SPLIT, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((decode16_kernel<T, D, false, SPLIT, 2>), grid, block, 0, s, p);
      break;
    default:
      if (mask) hipLaunchKernelGGL((decode16_kernel<T, D, true, SPLIT, 4>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((decode16_kernel<T, D, false, SPLIT, 4>), grid, block, 0, s, p);
  }
}

template <class T, int D>
hipError_t launch_t(const AttnParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.nsplit * p.nchunk * p.Hkv * p.B));
  const dim3 block(kThreads);
  const bool mask = p.mask != nullptr;
  constexpr bool F32 = std::is_same<T, TF32>::value;
  const int cpw = decode_cpw(F32 ? SDPA_F32 : SDPA_F16, (int64_t)p.Lq * p.group);
  if (p.nsplit > 1) {
    if constexpr (F32) {
      if (mask) hipLaunchKernelGGL((decode_f32_kernel<T, D, true, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((decode_f32_kernel<T, D, false, true>), grid, block, 0, s, p);
    } else {
      launch16<T, D, true>(p, cpw, mask, grid, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslice = D / (D < kMergeCols ? D : kMergeCols);
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)((int64_t)p.B * p.Hq * p.Lq * nslice)),
                       dim3(kMergeThreads), 0, s, p);
  } else {
    if constexpr (F32) {
      if (mask) hipLaunchKernelGGL((decode_f32_kernel<T, D, true, false>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((decode_f32_kernel<T, D, false, false>), grid, block, 0, s, p);
    } else {
      launch16<T, D, false>(p, cpw, mask, grid, s);
    }
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

// Prefill at head dim 512 (16-bit): W waves of 16 columns each per workgroup,
// one pass.  Eight waves (two per SIMD, 128 columns) hide more latency but
// quarter-fill fewer compute units; they are used when that still leaves at
// least four workgroups per compute unit (measured: causal GQA-8 over 4096
// rows 11 % faster with eight; causal MHA with 8 heads 1.6x slower, its 256
// workgroups of 1 to 32 units of work then run as one unbalanced round).
template <class T, int W>
hipError_t launch_wide_w(AttnParams p, hipStream_t s) {
  p.nchunk = (int)(((int64_t)p.Lq * p.group + 16 * W - 1) / (16 * W));
  const dim3 grid((unsigned)((int64_t)p.nchunk * p.Hkv * p.B));
  if (p.mask) hipLaunchKernelGGL((decode16_kernel<T, 512, true, false, W>), grid, dim3(64 * W), 0, s, p);
  else hipLaunchKernelGGL((decode16_kernel<T, 512, false, false, W>), grid, dim3(64 * W), 0, s, p);
  return hipGetLastError();
}
template <class T>
hipError_t launch_wide(const AttnParams& p, hipStream_t s) {
  const int64_t wg8 = ((int64_t)p.Lq * p.group + 127) / 128 * p.Hkv * p.B;
  return wg8 >= 4 * kWideCUs ? launch_wide_w<T, 8>(p, s) : launch_wide_w<T, 4>(p, s);
}

}  // namespace

hipError_t launch_prefill_wide(const AttnParams& p, int dtype, hipStream_t s) {
  return dtype == SDPA_F16 ? launch_wide<TF16>(p, s) : launch_wide<TBF16>(p, s);
}

int decode_tile_keys(int dtype, int D, int cpw) {
  if (dtype == SDPA_F32) return D >= 256 ? 16 : SDPA_DECODE_TILE_BYTES / (8 * D);
  switch (D) {
    case 64: return Dec16<64>::TK;
    case 128: return Dec16<128>::TK;
    case 256: return Dec16<256>::TK;
    default: return cpw > 1 ? Dec16<512, 32>::TK : Dec16<512>::TK;
  }
}

hipError_t launch_decode(const AttnParams& p, int dtype, hipStream_t s) {
  switch (dtype) {
    case SDPA_F32: return launch_d<TF32>(p, s);
    case SDPA_F16: return launch_d<TF16>(p, s);
    default: return launch_d<TBF16>(p, s);
  }
}

}  // namespace sdpa
