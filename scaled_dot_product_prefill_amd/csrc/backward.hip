// Gradients of the prefill attention (fp32 / fp16 / bf16 inputs; head dims D of q, k
// and Dv of v, o, any multiples of 8 up to 128, run at kernel dim 64 or 128
// with the chunks past the real dims loaded as zero and never stored).
//
// The structure follows the two backward kernels of the rustytorch
// "flash_attention.metal" page: one kernel per query block computes dQ
// ("Flash Attention backward kernel for dQ"), one per key block computes dK
// and dV ("... for dK and dV"); both recompute P = exp(S - LSE) from the
// forward's log-sum-exp instead of storing it, and use D_i = dO_i . O_i:
//
//     dS = P * (dO V^T - D),   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
//
// The inputs are those of build_sdpa_backward_graph on the "mlx 0.30.7 --
// backend/cuda/scaled_dot_product_attention.cpp" page (q, k, v, o, dO and the
// statistics, with scale, bottom-right causal mask, additive bias and sink
// token).  A sink only enters the denominator, so it changes dQ, dK, dV only
// through the LSE; its own gradient is -sum_i exp(sink - LSE_i) D_i.
//
// For rows that see few keys (at most 256, or any row under a mask) D_i is
// formed as sum_j P_ij dP_ij, which equals dO_i . O_i, instead of from the
// stored O: a 16-bit O carries its rounding (and the forward's P rounding)
// into every dS of the row, which showed as errors of a few 1e-3 in bf16 dQ
// for such rows.  Rows that see more keys read O (one pass over the keys
// fewer in the dQ kernel).
//
// Kernels, in launch order:
//   bwd_dq_kernel     workgroup = 128 query rows of one (batch, query head);
//                     each wave owns 32 rows, key tiles stream through LDS:
//                     for rows that see few keys twice, S^T = K Q^T and
//                     dP^T = V dO^T (lanes own queries) giving D_i on the
//                     first pass, otherwise D_i = dO_i . O_i; D_i goes to the
//                     workspace, then dQ^T += K^T dS^T on the (last) pass;
//   bwd_dkv_kernel    workgroup = 256 keys of one (batch, KV head), 8 waves
//                     (two per SIMD: K rows in registers, V rows in LDS, so
//                     a wave fits half the register file); each wave
//                     owns 32 keys and walks the query tiles of every query
//                     head of the group: S = Q K^T and dP = dO V^T (lanes own
//                     keys), then dV^T += dO^T P and dK^T += Q^T dS, so the
//                     group's heads add up in registers (no atomics);
//   bwd_dsink_kernel  the sink gradient, one workgroup per query head.
// The matrix products are 32x32x16 MFMAs with fp32 accumulation; P and dS
// enter the second products rounded to the input type.  bf16 P (8
// significant bits) goes into dV as hi + lo pairs on tiles whose rows may see
// few keys (at most 256, or any row under a mask): there single probabilities
// are large and their rounding shows in dV, as in the forward's P.V.  (With D
// formed from P and dP, bf16 dS fed as hi + lo measured no more accurate than
// one bf16 product: the outputs' own bf16 rounding dominates.)
#include <type_traits>

#include "sdpa_device.hpp"
#include "sdpa_internal.hpp"

namespace sdpa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;

// dK / dV workgroups: 8 waves (two per SIMD), 32 keys each.
constexpr int kDkvWaves = 8;
constexpr int kDkvThreads = 64 * kDkvWaves;
constexpr int kDkvKeys = 32 * kDkvWaves;
static_assert(kDkvKeys == kBwdKeyBlock, "the host plans the head split with this key block");

// A 64-row tile of a [rows, D] 16-bit matrix in LDS: unpadded rows whose
// 16-byte chunks are XOR-swizzled by the row (period 16 rows), filled by
// direct buffer -> LDS loads of NW waves: wave w writes 1 KiB lines w, w + NW, ...
// The LDS serves 64 four-byte banks, 16 lanes of a 16-byte read or 32 lanes
// of an 8-byte read per pass.  A row read (tile_rows) takes one chunk from
// each of 16 rows of an aligned block, a transposed read (tile_cols) 4
// consecutive chunks from each of 4 consecutive rows.  The dQ kernel's tiles
// (4 waves) swap the two 2-bit halves of row % 16, which keeps both patterns
// free of conflicts (measured: transposed reads take 0.39x the time of the
// plain row % 16 swizzle, row reads the same).  The dK / dV kernel's tiles (8
// waves) at D = 64 keep row % 16, whose transposed reads conflict 4 ways (the
// swapped form's extra address registers raised that kernel's spills).  At
// D = 128 they are padded instead (PAD): rows of 320 bytes, so each row
// starts 4 chunks further round the banks, with chunks swizzled by
// (row / 4) % 4 in their low two bits.  A transposed read then covers all 16
// bank groups (rows by the padding, chunks by themselves), and so does a row
// read (low bits by the swizzle, high bits by the padding), while a chunk's
// offset stays additive in the column block: no extra address registers.
template <int D, int NW = kBwdWaves>
struct Tile64 {
  static constexpr bool PAD = NW == kDkvWaves && D == 128;
  static constexpr int ROWS = 64;
  static constexpr int NCH = D / 8;                     // 16-byte chunks per row
  static constexpr int RB = D * 2 + (PAD ? 64 : 0);     // row bytes
  static constexpr int BYTES = ROWS * RB;
  static constexpr int LINES = BYTES / 1024;
  // unpadded: wave w fills lines w, w + NW, ... (LPW of them, STEP_ROWS rows
  // apart); padded: a 1 KiB line holds 3.2 rows, so the lines' patterns
  // repeat every 5 lines (16 rows), and waves 0..4 fill lines w, w + 5, w + 10
  // and w + 15
  static constexpr int LPW = PAD ? 4 : LINES / NW;      // lines per loading wave
  static constexpr int STEP_ROWS = PAD ? 16 : NW * 64 / NCH;
  static_assert(PAD ? LINES == 20 : (LINES % NW == 0 && STEP_ROWS % 16 == 0), "tile lines");
  __device__ static constexpr int swz(int row) {
    if constexpr (PAD) return (row >> 2) & 3;
    else if constexpr (NW == kDkvWaves) return NCH >= 16 ? (row & 15) : ((row >> 1) & 7);
    else return NCH >= 16 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
};

struct BwdParams {
  AttnParams f;          // the forward's arguments (o and lse are inputs here)
  const void* dout;
  int64_t dos[3];
  void* dq;
  int64_t dqs[3];
  void* dk;
  int64_t dks[3];
  void* dv;
  int64_t dvs[3];
  float* dsinks;
  float scale;
  float* ws_d;           // [B*Hq*Lq] D_i
  float* ws_l;           // [B*Hq*Lq] LSE_i * log2(e), +inf for rows without a key
  int hsplit;            // query-head groups per dK / dV key block (16-bit)
  float* ws_part;        // hsplit > 1: [hsplit][B][Hkv][Lk][2 D] fp32 dK (scaled), dV
};

// Per-lane source offset of the direct loads of a Tile64: the 16 bytes that
// land in LDS row r, chunk c come from logical chunk c ^ swz(r) of row r; a
// chunk past the matrix's real head dim loads nothing (kNoLoad: beyond every
// tile's byte count, so the range check returns zero).
template <int D, int NW = kBwdWaves>
__device__ inline uint32_t tile_lane_off(int wave, int lane, int64_t row_stride_elems, int real_d) {
  using L = Tile64<D, NW>;
  if constexpr (L::PAD) {
    // 20 slots per row, the last 4 padding (they load nothing)
    const int pos = wave * 64 + lane;
    const int row = pos / 20, pch = pos % 20;
    const int lch = pch ^ L::swz(row);
    return wave < 5 && pch < 16 && lch * 8 < real_d ? (uint32_t)(row * row_stride_elems * 2 + lch * 16) : kNoLoad;
  } else {
    const int pos = wave * 64 + lane;
    const int row = pos / L::NCH, pch = pos % L::NCH;
    const int lch = pch ^ L::swz(row);
    return lch * 8 < real_d ? (uint32_t)(row * row_stride_elems * 2 + lch * 16) : kNoLoad;
  }
}

// Issue this wave's direct loads of rows [r0, r0 + 64) of a matrix (rows >=
// nrows read as zero) into the Tile64 whose LDS byte address is `lds`.  The
// byte count ends at the real length (real_d elements) of the last real row.
template <int D, int NW = kBwdWaves>
__device__ inline void tile_issue(const uint16_t* base, int64_t rs, int r0, int nrows, uint32_t off,
                                  uint32_t lds, int wave, int real_d) {
  using L = Tile64<D, NW>;
  const uint16_t* tb = base + (int64_t)r0 * rs;
  const int rows = min(nrows - r0, L::ROWS);
  const uint32_t rowb = (uint32_t)(rs * 2);
  // no rows: a zero range, so that even the kNoLoad lanes read nothing
  const uint32_t nb = rows > 0 ? (uint32_t)(rows - 1) * rowb + (uint32_t)real_d * 2 : 0u;
  if constexpr (L::PAD) {
    if (wave < 5) {
#pragma unroll
      for (int i = 0; i < L::LPW; ++i) dma16(tb, nb, lds + (wave + 5 * i) * 1024, off, i * L::STEP_ROWS * rowb);
    }
  } else {
#pragma unroll
    for (int i = 0; i < L::LPW; ++i)
      dma16(tb, nb, lds + (wave + NW * i) * 1024, off, i * L::STEP_ROWS * rowb);
  }
}

// Matrix-core A operand from a Tile64, row-major: A[m = row rb + lane%32][k =
// 16 s + 8 (lane/32) + e].  rb is a multiple of 16.
template <int D, int NW = kBwdWaves>
__device__ inline u32x4 tile_rows(const uint8_t* t, int rb, int s, int l32, int g) {
  using L = Tile64<D, NW>;
  const int row = rb + l32;
  if constexpr (L::PAD) {
    // swz(row) = (l32 >> 2) & 3 = 2 h + w: chunk (2 s + g) ^ (2 h + w) is
    // 2 (s ^ h) + (g ^ w), and s ^ h = s + h for even s, s - h for odd s, so
    // the offset is a per-lane term (one for each parity of s) plus a
    // constant that the read's immediate offset carries
    const int h = (l32 >> 3) & 1, w = (l32 >> 2) & 1;
    const int lane_off = l32 * L::RB + 16 * (g ^ w) + ((s & 1) ? -32 * h : 32 * h);
    return lds_read16(t + lane_off + rb * L::RB + 32 * s);
  } else {
    return lds_read16(t + row * L::RB + (((2 * s + g) ^ L::swz(row)) * 16));
  }
}

// Matrix-core A operand from a Tile64, transposed: A[m = column 32 mb + lane%32]
// [k = kappa] = X[rb + 8 (kappa/4 % 2) + 4 (lane/32) + kappa % 4][column], the
// row order in which a 32x32 accumulator's registers 8u..8u+7 are packed as
// the B operand (u = k-step, rb = 32 * block + 16 * u).
template <int D, int NW = kBwdWaves>
__device__ inline u32x4 tile_cols(const uint8_t* t, int rb, int mb, int lane) {
  using L = Tile64<D, NW>;
  const int r16 = lane & 15, g = lane >> 5, dh = (lane >> 4) & 1;
  const int vr = rb + 4 * g + (r16 >> 2);
  if constexpr (L::PAD) {
    // rb is a multiple of 16, so swz(vr) = g and swz(vr + 8) = g ^ 2: both
    // touch only the low two chunk bits, and 4 mb passes through the XOR
    const int lo = 2 * dh + ((r16 >> 1) & 1);
    const int base = (4 * g + (r16 >> 2)) * L::RB + (r16 & 1) * 8;
    const int off0 = base + 16 * (lo ^ g), off1 = base + 8 * L::RB + 16 * (lo ^ g ^ 2);
    const u32x2 a0 = lds_read_tr16(t + off0 + rb * L::RB + 64 * mb);
    const u32x2 a1 = lds_read_tr16(t + off1 + rb * L::RB + 64 * mb);
    return u32x4{a0[0], a0[1], a1[0], a1[1]};
  } else {
    const int ch = 4 * mb + 2 * dh + ((r16 >> 1) & 1);
    const uint8_t* p0 = t + vr * L::RB + ((ch ^ L::swz(vr)) * 16) + (r16 & 1) * 8;
    const uint8_t* p1 = t + (vr + 8) * L::RB + ((ch ^ L::swz(vr + 8)) * 16) + (r16 & 1) * 8;
    const u32x2 a0 = lds_read_tr16(p0), a1 = lds_read_tr16(p1);
    return u32x4{a0[0], a0[1], a1[0], a1[1]};
  }
}

// registers 8u .. 8u+7 as bf16 hi + lo pairs (about 16 significant bits)
__device__ inline void pack_b_split(const f32x16& x, int u, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t h, l;
    TBF16::split2(x[8 * u + 2 * e], x[8 * u + 2 * e + 1], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

// registers 8u .. 8u+7 of an accumulator as a packed B operand
template <class T>
__device__ inline u32x4 pack_b(const f32x16& x, int u) {
  return u32x4{cvt_pk(T{}, x[8 * u + 0], x[8 * u + 1]), cvt_pk(T{}, x[8 * u + 2], x[8 * u + 3]),
               cvt_pk(T{}, x[8 * u + 4], x[8 * u + 5]), cvt_pk(T{}, x[8 * u + 6], x[8 * u + 7])};
}

// ---- the LSE in log2 units ------------------------------------------------
// Row my_i of (b, hq): LSE_i * log2(e), +inf for a row without a key or past
// the batch's length (ok false).  The dQ kernels, which run first and cover
// every row once, also store it (lanes of the first half) in the workspace
// for the dK/dV and sink-gradient kernels.
__device__ inline float lse_log2(const BwdParams& bp, int b, int hq, int my_i, bool ok) {
  const AttnParams& p = bp.f;
  const int64_t row = ((int64_t)b * p.Hq + hq) * p.Lq + my_i;
  const float lse = ok ? p.lse[row] : kNegInf;
  const float l2 = lse == kNegInf ? __builtin_inff() : lse * kLog2e;
  if (my_i < p.Lq && (threadIdx.x & 32) == 0) bp.ws_l[row] = l2;
  return l2;
}

// ---- dQ ---------------------------------------------------------------------
template <class T, int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kBwdThreads, MASK ? 1 : 2) void bwd_dq_kernel(BwdParams bp) {
  const AttnParams& p = bp.f;
  using L = Tile64<D>;
  constexpr int NQ = D / 16, NMB = D / 32, NKB = 2;
  using S = uint16_t;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * L::BYTES];  // (K, V) x 2 stages

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int nqt = (p.Lq + 127) / 128;
  int qt, bh;
  prefill_tile((int)blockIdx.x, (int)gridDim.x, nqt, p.B * p.Hq, CAUSAL, qt, bh);
  const int b = bh / p.Hq, hq = bh % p.Hq, hk = hq / p.group;
  const int lq = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_q, b, p.Lq));
  const int lk = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_k, b, p.Lk));
  const int coff = lk - lq;
  const int i0 = qt * 128;
  const int my_i = i0 + 32 * wave + l32;
  const bool ok = my_i < lq;
  const float c = p.scale_log2;

  // this lane's query row: Q and dO as B operands, its LSE and D
  u32x4 qreg[NQ], doreg[NQ];
  {
    const int ii = ok ? my_i : 0;
    const S* qr = (const S*)p.q + b * p.qs[0] + hq * p.qs[1] + (int64_t)ii * p.qs[2];
    const S* dr = (const S*)bp.dout + b * bp.dos[0] + hq * bp.dos[1] + (int64_t)ii * bp.dos[2];
    const int nq = p.Dqk / 8, nd = p.Dv / 8;  // real 16-byte chunks; the rest is zero
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int ch = 2 * s + g;
      const u32x4 a = ldg16_cached(qr + min(ch, nq - 1) * 8), d = ldg16_cached(dr + min(ch, nd - 1) * 8);
      qreg[s] = ok && ch < nq ? a : u32x4{0, 0, 0, 0};
      doreg[s] = ok && ch < nd ? d : u32x4{0, 0, 0, 0};
    }
  }
  const float lse2 = lse_log2(bp, b, hq, my_i, ok);

  int kend = i0 < lq ? lk : 0;
  if (CAUSAL) kend = min(kend, min(i0 + 128, lq) + coff);
  const int ntiles = kend > 0 ? (kend + 63) / 64 : 0;
  int n_int = 0;  // tiles whose every key every row of the workgroup sees
  if (!MASK) {
    int full = lk;
    if (CAUSAL) full = min(full, i0 + 1 + coff);
    n_int = full > 0 ? min(ntiles, full / 64) : 0;
  }

  const S* kbase = (const S*)p.k + b * p.ks[0] + hk * p.ks[1];
  const S* vbase = (const S*)p.v + b * p.vs[0] + hk * p.vs[1];
  const uint32_t koff = tile_lane_off<D>(wave, lane, p.ks[2], p.Dqk);
  const uint32_t voff = tile_lane_off<D>(wave, lane, p.vs[2], p.Dv);
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int t) {
    const uint32_t st = lds0 + (t & 1) * 2 * L::BYTES;
    tile_issue<D>(kbase, p.ks[2], 64 * t, lk, koff, st, wave, p.Dqk);
    tile_issue<D>(vbase, p.vs[2], 64 * t, lk, voff, st + L::BYTES, wave, p.Dv);
  };

  // S^T and dP^T of key block kb of tile t (stage Ks / Vs), and P^T
  auto scores = [&](const uint8_t* Ks, const uint8_t* Vs, int t, int kb, bool edge, f32x16& pr, f32x16& dpt) {
    f32x16 st = f32x16{};
    dpt = f32x16{};
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      st = mma32(T{}, tile_rows<D>(Ks, 32 * kb, s, l32, g), qreg[s], st);
      dpt = mma32(T{}, tile_rows<D>(Vs, 32 * kb, s, l32, g), doreg[s], dpt);
    }
    // the visibility test only on edge tiles, as separate code under a
    // wave-uniform branch (one form with a runtime test issues the test's
    // exec-masked code on every tile)
    auto probs = [&](auto edge_tag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = st[r] * c;
        if constexpr (decltype(edge_tag)::value) {
          const int j = 64 * t + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          if (MASK) {
            const int ii = ok ? my_i : 0, jj = j < lk ? j : lk - 1;
            x += kLog2e * mask_val(p.mask, p.mask_bool,
                                   b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] + (int64_t)jj * p.ms[3]);
          }
          const bool vis = (j < lk) & (!CAUSAL | (j <= my_i + coff));
          x = vis ? x : kNegInf;
        }
        pr[r] = fast_exp2(x - lse2);
      }
    };
    if (edge) probs(std::true_type{});
    else probs(std::false_type{});
  };

  // D_i.  Where every row of the workgroup sees more than 256 keys (and no
  // mask can hide them), D_i = dO_i . O_i from the forward's output: the
  // 16-bit rounding of O then shifts dS_ij = P_ij (dP_ij - D_i) by the same
  // tiny amount across many keys, and dQ_i = scale sum_j dS_ij K_j averages
  // it away.  Rows that see fewer keys form D_i = sum_j P_ij dP_ij in a first
  // pass over the keys (pass 1), free of that rounding.
  const int first_keys = i0 < lq ? (CAUSAL ? min(lk, i0 + 1 + coff) : lk) : 0;
  const bool d_from_o = !MASK && first_keys > 256;
  float dsum = 0.f;
  if (d_from_o) {
    if (ok) {
      const S* orow = (const S*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)my_i * p.os[2];
      const int nd = p.Dv / 8;
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        const int ch = 2 * s + g;  // the chunk of dO this lane holds
        if (ch < nd) {
          const u32x4 ov = ldg16_cached(orow + ch * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dsum = fmaf(T::to_f32((uint16_t)(ov[e] & 0xffffu)), T::to_f32((uint16_t)(doreg[s][e] & 0xffffu)), dsum);
            dsum = fmaf(T::to_f32((uint16_t)(ov[e] >> 16)), T::to_f32((uint16_t)(doreg[s][e] >> 16)), dsum);
          }
        }
      }
    }
  }
  // pass 1: D_i = sum_j P_ij dP_ij
  if (!d_from_o && ntiles > 0) issue(0);
  for (int t = 0; t < (d_from_o ? 0 : ntiles); ++t) {
    wait_vmcnt<0>();
    lds_barrier();  // tile t landed for every wave; tile t-1 is no longer read
    if (t + 1 < ntiles) issue(t + 1);
    const uint8_t* Ks = smem + (t & 1) * 2 * L::BYTES;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 pr, dpt;
      scores(Ks, Ks + L::BYTES, t, kb, t >= n_int, pr, dpt);
#pragma unroll
      for (int r = 0; r < 16; ++r) dsum = fmaf(pr[r], dpt[r], dsum);
    }
  }
  const float dval = ok ? sum_xor32(dsum) : 0.f;
  if (my_i < p.Lq && g == 0) bp.ws_d[((int64_t)b * p.Hq + hq) * p.Lq + my_i] = dval;

  // pass 2: dS = P (dP - D),  dQ^T += K^T dS^T
  f32x16 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x16{};
  if (ntiles > 0) {
    lds_barrier();  // every wave is done with the last tile of pass 1
    issue(0);
  }
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();
    lds_barrier();  // tile t landed for every wave; tile t-1 is no longer read
    if (t + 1 < ntiles) issue(t + 1);
    const uint8_t* Ks = smem + (t & 1) * 2 * L::BYTES;
    u32x4 dsp[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 pr, dpt, ds;
      scores(Ks, Ks + L::BYTES, t, kb, t >= n_int, pr, dpt);
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = pr[r] * (dpt[r] - dval);
      dsp[kb][0] = pack_b<T>(ds, 0);
      dsp[kb][1] = pack_b<T>(ds, 1);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[mb] = mma32(T{}, tile_cols<D>(Ks, 32 * kb + 16 * u, mb, lane), dsp[kb][u], acc[mb]);
  }

  if (my_i < p.Lq) {
    S* orow = (S*)bp.dq + b * bp.dqs[0] + hq * bp.dqs[1] + (int64_t)my_i * bp.dqs[2];
    const float sc = bp.scale;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 w = {cvt_pk(T{}, acc[mb][4 * q4] * sc, acc[mb][4 * q4 + 1] * sc),
                         cvt_pk(T{}, acc[mb][4 * q4 + 2] * sc, acc[mb][4 * q4 + 3] * sc)};
        if (32 * mb + 8 * q4 + 4 * g < p.Dqk) *(u32x2*)(orow + 32 * mb + 8 * q4 + 4 * g) = w;
      }
  }
}

// ---- dK, dV -------------------------------------------------------------------
template <class T, int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kDkvThreads, 1) void bwd_dkv_kernel(BwdParams bp) {
  const AttnParams& p = bp.f;
  using L = Tile64<D, kDkvWaves>;
  constexpr int NQ = D / 16, NMB = D / 32;
  constexpr int STAGE = 2 * L::BYTES + 2048;  // Q, dO, LSE line, D line
  // the workgroup's value rows (each lane reads back only its own row; 16
  // rows per pass).  D = 128: rows padded by one chunk (272 bytes, 68 dwords:
  // 16 rows at one chunk fall on 16 distinct 4-bank groups), so a lane's
  // reads are one base plus immediate offsets; D = 64: unpadded, chunks
  // swizzled as in an unpadded tile.
  constexpr int VRB = D >= 128 ? D * 2 + 16 : D * 2;
  auto vswz = [](int row) { return D >= 128 ? 0 : ((row >> 1) & 7); };
  constexpr int VBYTES = kDkvKeys * VRB;
  using S = uint16_t;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE + VBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // key blocks in increasing order: under causal masking the first key
  // blocks are seen by the most query rows, so the heaviest go first
  // workgroup = (key block kt, batch, KV head, query-head group hsi): the
  // group's gsub query heads hq0 .. hq0 + gsub - 1
  const int nbh = p.B * p.Hkv;
  const int hsi = (int)blockIdx.x % bp.hsplit, unit = (int)blockIdx.x / bp.hsplit;
  const int kt = unit / nbh, bhk = unit % nbh;
  const int b = bhk / p.Hkv, hk = bhk % p.Hkv;
  const int gsub = p.group / bp.hsplit;
  const int hq0 = hk * p.group + hsi * gsub;
  const int lq = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_q, b, p.Lq));
  const int lk = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_k, b, p.Lk));
  const int coff = lk - lq;
  const int k0 = kt * kDkvKeys;
  const int kw0 = k0 + 32 * wave;
  const int my_j = kw0 + l32;
  const bool kok = my_j < lk;
  const float c = p.scale_log2;

  // this lane's key row as B operands in registers and its value row, in the
  // same operand order, in this wave's own LDS rows (each lane reads back only
  // what it wrote); both zero past the batch's keys
  u32x4 kreg[NQ];
  uint8_t* const Vw = smem + 2 * STAGE + 32 * wave * VRB;
  {
    const int jj = kok ? my_j : 0;
    const S* kr = (const S*)p.k + b * p.ks[0] + hk * p.ks[1] + (int64_t)jj * p.ks[2];
    const S* vr = (const S*)p.v + b * p.vs[0] + hk * p.vs[1] + (int64_t)jj * p.vs[2];
    const int nk = p.Dqk / 8, nv = p.Dv / 8;  // real 16-byte chunks; the rest is zero
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int ch = 2 * s + g;
      const u32x4 a = ldg16_cached(kr + min(ch, nk - 1) * 8), d = ldg16_cached(vr + min(ch, nv - 1) * 8);
      kreg[s] = kok && ch < nk ? a : u32x4{0, 0, 0, 0};
      lds_write16(Vw + l32 * VRB + ((ch ^ vswz(l32)) * 16), kok && ch < nv ? d : u32x4{0, 0, 0, 0});
    }
  }

  // query tiles [qt0, nqt) of each of the group's heads
  const int ibeg = CAUSAL ? max(0, k0 - coff) : 0;
  const int qt0 = ibeg / 64;
  const int nqt = k0 < lk ? (lq + 63) / 64 : 0;
  const int per_head = max(0, nqt - qt0);
  const int ntiles = per_head * gsub;

  const uint32_t qoff = tile_lane_off<D, kDkvWaves>(wave, lane, p.qs[2], p.Dqk);
  const uint32_t dooff = tile_lane_off<D, kDkvWaves>(wave, lane, bp.dos[2], p.Dv);
  const uint32_t lds0 = lds_addr(smem);
  // tile t = (query tile qt0 + t / gsub, query head hq0 + t % gsub)
  auto issue = [&](int t) {
    const int hq = hq0 + t % gsub;
    const int q0 = 64 * (qt0 + t / gsub);
    const uint32_t st = lds0 + (t & 1) * STAGE;
    const S* qb = (const S*)p.q + b * p.qs[0] + hq * p.qs[1];
    const S* db = (const S*)bp.dout + b * bp.dos[0] + hq * bp.dos[1];
    tile_issue<D, kDkvWaves>(qb, p.qs[2], q0, lq, qoff, st, wave, p.Dqk);
    tile_issue<D, kDkvWaves>(db, bp.dos[2], q0, lq, dooff, st + L::BYTES, wave, p.Dv);
    if (wave == (L::PAD ? 5 : 0)) {  // (padded tiles: a wave that loads no tile lines)
      const int64_t r0 = ((int64_t)b * p.Hq + hq) * p.Lq + q0;
      const uint32_t nb = (uint32_t)min(64, p.Lq - q0) * 4;
      dma16(bp.ws_l + r0, nb, st + 2 * L::BYTES, lane * 16, 0);
      dma16(bp.ws_d + r0, nb, st + 2 * L::BYTES + 1024, lane * 16, 0);
    }
  };

  f32x16 dk[NMB], dv[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) dk[mb] = dv[mb] = f32x16{};

  // bf16 P (8 significant bits) goes into dV as hi + lo pairs on tiles whose
  // rows may see few keys (at most 256, or any row under a mask): there single
  // probabilities are large and their rounding shows in dV, as in the
  // forward's P.V.  Under causal masking rows see more keys the later the
  // tile, so those tiles are a prefix of the loop and run in a loop of their
  // own (one instantiation each keeps the common loop's registers unchanged).
  int n_split = 0;
  if (std::is_same<T, TBF16>::value) {
    if (MASK) {
      n_split = ntiles;
    } else {
      // query tiles qt0 .. qs - 1 hold a row that sees at most 256 keys
      const int qs = CAUSAL ? (lk <= 256 ? nqt : min(nqt, max(qt0, (256 - coff) / 64 + 1))) : (lk <= 256 ? nqt : qt0);
      // a key block past this batch's keys has nqt = 0 < qt0: no tiles at all
      n_split = max(0, qs - qt0) * gsub;
    }
  }
  auto run = [&](int t_begin, int t_end, auto split_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    for (int t = t_begin; t < t_end; ++t) {
      wait_vmcnt<0>();
      lds_barrier();  // tile t landed for every wave; tile t-1 is no longer read
      if (t + 1 < ntiles) issue(t + 1);
      const int hq = hq0 + t % gsub;
      const int q0 = 64 * (qt0 + t / gsub);
      // nothing of this wave's keys is visible to the tile's rows
      if (kw0 >= lk || (CAUSAL && kw0 > q0 + 63 + coff)) continue;
      const bool edge = MASK || q0 + 64 > lq || kw0 + 32 > lk || (CAUSAL && kw0 + 31 > q0 + coff);
      const uint8_t* Qs = smem + (t & 1) * STAGE;
      const uint8_t* Ds = Qs + L::BYTES;
      const float* Ls = (const float*)(Qs + 2 * L::BYTES);
      const float* Dv = Ls + 256;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 s_ = f32x16{}, dp = f32x16{};
        // At D = 128 the per-lane LDS offsets of each phase are derived from
        // a fresh copy of the lane index.  Held across the loop they do not
        // fit the registers: they were reloaded from scratch on every tile,
        // and each reload's wait also waited for the next tile's loads in
        // flight (measured: causal bf16 8 % faster, GQA-4 15 %).  At D = 64
        // they fit, and recomputing them cost 4 %.
        const int lane_a = D >= 128 ? fresh_lane(lane) : lane, l32_a = lane_a & 31, g_a = lane_a >> 5;
        // the operands of k-step s + 1 are read before the products of step
        // s are issued (one fence per step): each read has a step of this
        // wave's products to land, in two sets of operand registers
        auto vrow = [&](int s) { return lds_read16(Vw + l32_a * VRB + (((2 * s + g_a) ^ vswz(l32_a)) * 16)); };
        u32x4 qo = tile_rows<D, kDkvWaves>(Qs, 32 * qb, 0, l32_a, g_a);
        u32x4 doo = tile_rows<D, kDkvWaves>(Ds, 32 * qb, 0, l32_a, g_a);
        u32x4 vo = vrow(0);
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
          u32x4 qn = qo, dn = doo, vn = vo;
          if (s + 1 < NQ) {
            qn = tile_rows<D, kDkvWaves>(Qs, 32 * qb, s + 1, l32_a, g_a);
            dn = tile_rows<D, kDkvWaves>(Ds, 32 * qb, s + 1, l32_a, g_a);
            vn = vrow(s + 1);
          }
          s_ = mma32(T{}, qo, kreg[s], s_);
          dp = mma32(T{}, doo, vo, dp);
          __builtin_amdgcn_sched_barrier(0);
          qo = qn;
          doo = dn;
          vo = vn;
        }
        f32x16 pr, ds;
        // P and dS of the block; the visibility test only on edge tiles.  The
        // two forms are separate code under a wave-uniform branch: written as
        // one, the test's short-circuit on the lane's own key became per-score
        // exec-masked code that every tile issued.
        auto probs = [&](auto edge_tag) {
#pragma unroll
          for (int rh = 0; rh < 4; ++rh) {
            // rows 32 qb + 8 rh + 4 g + (0..3) of the tile
            const int ib = 32 * qb + 8 * rh + 4 * g;
            const f32x4 l4 = *(const f32x4*)(Ls + ib);
            const f32x4 d4 = *(const f32x4*)(Dv + ib);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * rh + e;
              float x = s_[r] * c;
              if constexpr (decltype(edge_tag)::value) {
                const int i = q0 + ib + e;
                if (MASK) {
                  const int ii = i < lq ? i : lq - 1, jj = kok ? my_j : lk - 1;
                  x += kLog2e * mask_val(p.mask, p.mask_bool,
                                         b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] + (int64_t)jj * p.ms[3]);
                }
                const bool vis = kok & (i < lq) & (!CAUSAL | (my_j <= i + coff));
                x = vis ? x : kNegInf;
              }
              const float pv = fast_exp2(x - l4[e]);
              pr[r] = pv;
              ds[r] = pv * (dp[r] - d4[e]);
            }
          }
        };
        if (edge) probs(std::true_type{});
        else probs(std::false_type{});
        const int lane_b = D >= 128 ? fresh_lane(lane) : lane;
        u32x4 pb[2], pl[2], db[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          db[u] = pack_b<T>(ds, u);
          if constexpr (SPLIT) pack_b_split(pr, u, pb[u], pl[u]);
          else pb[u] = pack_b<T>(pr, u);
        }
        // step i = (u, mb): the transposed dO and Q columns of step i + 1 are
        // read before the products of step i are issued
        u32x4 da = tile_cols<D, kDkvWaves>(Ds, 32 * qb, 0, lane_b);
        u32x4 qa = tile_cols<D, kDkvWaves>(Qs, 32 * qb, 0, lane_b);
#pragma unroll
        for (int i = 0; i < 2 * NMB; ++i) {
          const int u = i / NMB, mb = i % NMB;
          u32x4 dn = da, qn = qa;
          if (i + 1 < 2 * NMB) {
            const int u1 = (i + 1) / NMB, mb1 = (i + 1) % NMB;
            dn = tile_cols<D, kDkvWaves>(Ds, 32 * qb + 16 * u1, mb1, lane_b);
            qn = tile_cols<D, kDkvWaves>(Qs, 32 * qb + 16 * u1, mb1, lane_b);
          }
          dv[mb] = mma32(T{}, da, pb[u], dv[mb]);
          if constexpr (SPLIT) dv[mb] = mma32(T{}, da, pl[u], dv[mb]);
          dk[mb] = mma32(T{}, qa, db[u], dk[mb]);
          __builtin_amdgcn_sched_barrier(0);
          da = dn;
          qa = qn;
        }
      }
    }
  };
  if (ntiles > 0) issue(0);
  if constexpr (std::is_same<T, TBF16>::value) run(0, n_split, std::true_type{});
  run(n_split, ntiles, std::false_type{});

  if (bp.hsplit > 1) {
    // this head group's share, in fp32, for bwd_dkv_reduce_kernel
    if (my_j < p.Lk) {
      float* pr = bp.ws_part + ((((int64_t)hsi * p.B + b) * p.Hkv + hk) * p.Lk + my_j) * (2 * D);
      const float sc = bp.scale;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * mb + 8 * q4 + 4 * g;
          *(f32x4*)(pr + d0) = f32x4{dk[mb][4 * q4] * sc, dk[mb][4 * q4 + 1] * sc, dk[mb][4 * q4 + 2] * sc,
                                     dk[mb][4 * q4 + 3] * sc};
          *(f32x4*)(pr + D + d0) = f32x4{dv[mb][4 * q4], dv[mb][4 * q4 + 1], dv[mb][4 * q4 + 2], dv[mb][4 * q4 + 3]};
        }
    }
    return;
  }
  if (my_j < p.Lk) {
    S* kr = (S*)bp.dk + b * bp.dks[0] + hk * bp.dks[1] + (int64_t)my_j * bp.dks[2];
    S* vr = (S*)bp.dv + b * bp.dvs[0] + hk * bp.dvs[1] + (int64_t)my_j * bp.dvs[2];
    const float sc = bp.scale;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 wk = {cvt_pk(T{}, dk[mb][4 * q4] * sc, dk[mb][4 * q4 + 1] * sc),
                          cvt_pk(T{}, dk[mb][4 * q4 + 2] * sc, dk[mb][4 * q4 + 3] * sc)};
        const u32x2 wv = {cvt_pk(T{}, dv[mb][4 * q4], dv[mb][4 * q4 + 1]),
                          cvt_pk(T{}, dv[mb][4 * q4 + 2], dv[mb][4 * q4 + 3])};
        if (32 * mb + 8 * q4 + 4 * g < p.Dqk) *(u32x2*)(kr + 32 * mb + 8 * q4 + 4 * g) = wk;
        if (32 * mb + 8 * q4 + 4 * g < p.Dv) *(u32x2*)(vr + 32 * mb + 8 * q4 + 4 * g) = wv;
      }
  }
}

// ---- head groups of a split dK / dV: sum the hsplit fp32 shares of each key
// row and write dK, dV in the input type.  Thread = 4 consecutive elements of
// one row's [dK | dV] (2 D floats).
template <class T, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkv_reduce_kernel(BwdParams bp) {
  using S = uint16_t;
  const AttnParams& p = bp.f;
  constexpr int TPR = 2 * D / 4;               // threads per row
  constexpr int RPB = kBwdThreads / TPR;       // rows per workgroup
  const int64_t nrows = (int64_t)p.B * p.Hkv * p.Lk;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= nrows) return;
  const int c = (threadIdx.x % TPR) * 4;       // element within [dK | dV]
  f32x4 acc = f32x4{};
  for (int h = 0; h < bp.hsplit; ++h) acc += *(const f32x4*)(bp.ws_part + ((int64_t)h * nrows + row) * (2 * D) + c);
  const int j = (int)(row % p.Lk);
  const int bh = (int)(row / p.Lk), b = bh / p.Hkv, hk = bh % p.Hkv;
  const u32x2 w = {cvt_pk(T{}, acc[0], acc[1]), cvt_pk(T{}, acc[2], acc[3])};
  if (c < D) {
    if (c < p.Dqk) *(u32x2*)((S*)bp.dk + b * bp.dks[0] + hk * bp.dks[1] + (int64_t)j * bp.dks[2] + c) = w;
  } else if (c - D < p.Dv) {
    *(u32x2*)((S*)bp.dv + b * bp.dvs[0] + hk * bp.dvs[1] + (int64_t)j * bp.dvs[2] + (c - D)) = w;
  }
}

// ---- sink gradient: -sum over batches and rows of exp(sink - LSE_i) D_i ------
__global__ __launch_bounds__(kBwdThreads) void bwd_dsink_kernel(BwdParams bp) {
  const AttnParams& p = bp.f;
  __shared__ float red[kBwdWaves];
  const int hq = blockIdx.x;
  const float sk = p.sinks[hq] * kLog2e;
  float acc = 0.f;
  for (int b = 0; b < p.B; ++b) {
    const int64_t r0 = ((int64_t)b * p.Hq + hq) * p.Lq;
    for (int i = threadIdx.x; i < p.Lq; i += kBwdThreads)
      acc -= fast_exp2(sk - bp.ws_l[r0 + i]) * bp.ws_d[r0 + i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) bp.dsinks[hq] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ---- fp32 inputs ---------------------------------------------------------------
// fp32 matrix cores (32x32x2; one 16-byte operand vector holds four k-steps,
// see mma32(TF32)).  Tiles of 32 rows are staged through registers into LDS,
// single-buffered; the transposed copies the second products read are
// written by the loading threads (no transposing LDS read exists for 32-bit
// data).  D_i = dO_i . O_i from the fp32 O.  Layouts as in the 16-bit
// kernels: in dQ lanes own queries (S^T = K Q^T), in dK / dV lanes own keys
// (S = Q K^T); an accumulator's registers 4u .. 4u+3 (rows 8u + 4g + t) are
// the B operand of k-group u, matched by transposed rows read at 8u + 4g.
template <int D>
struct F32T {
  static constexpr int NCH = D / 4;        // 16-byte chunks per row
  static constexpr int RP = D * 4 + 16;    // row-major pitch (bytes)
  static constexpr int TP = 32 * 4 + 16;   // transposed pitch: 32 rows + pad
  static constexpr int RBYTES = 32 * RP;
  static constexpr int TBYTES = D * TP;
  static constexpr int IT = 32 * NCH / kBwdThreads;  // 16-byte chunks per thread
  static constexpr int NQ = NCH / 2;       // operand vectors per lane (chunk 2s + g)
  static constexpr int NMB = D / 32;       // 32-row blocks of a transposed product
  static_assert(IT >= 1 && 32 * NCH % kBwdThreads == 0, "tile split");
};

// Rows [r0, r0 + 32) of a [rows, D] fp32 matrix (rows >= nrows and columns >=
// real_d as zero) into row-major and / or transposed LDS copies.
template <int D>
__device__ inline void f32_tile_load(const float* base, int64_t rs, int r0, int nrows, int real_d, uint8_t* dst_r,
                                     uint8_t* dst_t, int tid) {
  using L = F32T<D>;
  u32x4 v[L::IT];
#pragma unroll
  for (int it = 0; it < L::IT; ++it) {
    const int u = tid + kBwdThreads * it, row = u / L::NCH, c = u % L::NCH, r = r0 + row;
    v[it] = r < nrows && 4 * c < real_d ? ldg16_cached(base + (int64_t)r * rs + 4 * c) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int it = 0; it < L::IT; ++it) {
    const int u = tid + kBwdThreads * it, row = u / L::NCH, c = u % L::NCH;
    if (dst_r) lds_write16(dst_r + row * L::RP + c * 16, v[it]);
    if (dst_t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) *(uint32_t*)(dst_t + (4 * c + e) * L::TP + row * 4) = v[it][e];
    }
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_f32_kernel(BwdParams bp) {
  const AttnParams& p = bp.f;
  using L = F32T<D>;
  constexpr int NQ = L::NQ, NMB = L::NMB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::RBYTES + L::TBYTES];  // K, V rows; K^T
  uint8_t* const Ks = smem;
  uint8_t* const Vs = smem + L::RBYTES;
  uint8_t* const Kt = smem + 2 * L::RBYTES;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int nqt = (p.Lq + 127) / 128;
  int qt, bh;
  prefill_tile((int)blockIdx.x, (int)gridDim.x, nqt, p.B * p.Hq, CAUSAL, qt, bh);
  const int b = bh / p.Hq, hq = bh % p.Hq, hk = hq / p.group;
  const int lq = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_q, b, p.Lq));
  const int lk = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_k, b, p.Lk));
  const int coff = lk - lq;
  const int i0 = qt * 128;
  const int my_i = i0 + 32 * wave + l32;
  const bool ok = my_i < lq;
  const float c = p.scale_log2;

  // this lane's query row: Q and dO as B operands; D_i = dO_i . O_i
  u32x4 qreg[NQ], doreg[NQ];
  float dsum = 0.f;
  {
    const int ii = ok ? my_i : 0;
    const float* qr = (const float*)p.q + b * p.qs[0] + hq * p.qs[1] + (int64_t)ii * p.qs[2];
    const float* dr = (const float*)bp.dout + b * bp.dos[0] + hq * bp.dos[1] + (int64_t)ii * bp.dos[2];
    const float* orow = (const float*)p.o + b * p.os[0] + hq * p.os[1] + (int64_t)ii * p.os[2];
    const int nq = p.Dqk / 4, nd = p.Dv / 4;  // real 16-byte chunks; the rest is zero
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int ch = 2 * s + g;
      const u32x4 a = ldg16_cached(qr + min(ch, nq - 1) * 4), d = ldg16_cached(dr + min(ch, nd - 1) * 4);
      const u32x4 o = ldg16_cached(orow + min(ch, nd - 1) * 4);
      qreg[s] = ok && ch < nq ? a : u32x4{0, 0, 0, 0};
      doreg[s] = ok && ch < nd ? d : u32x4{0, 0, 0, 0};
      if (ok && ch < nd) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dsum = fmaf(as_float(o[e]), as_float(d[e]), dsum);
      }
    }
  }
  const float dval = ok ? sum_xor32(dsum) : 0.f;
  const float lse2 = lse_log2(bp, b, hq, my_i, ok);
  if (my_i < p.Lq && g == 0) bp.ws_d[((int64_t)b * p.Hq + hq) * p.Lq + my_i] = dval;

  int kend = i0 < lq ? lk : 0;
  if (CAUSAL) kend = min(kend, min(i0 + 128, lq) + coff);
  const int ntiles = kend > 0 ? (kend + 31) / 32 : 0;
  const float* kbase = (const float*)p.k + b * p.ks[0] + hk * p.ks[1];
  const float* vbase = (const float*)p.v + b * p.vs[0] + hk * p.vs[1];

  f32x16 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x16{};
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = 32 * t;
    __syncthreads();  // the previous tile is no longer read
    f32_tile_load<D>(kbase, p.ks[2], j0, lk, p.Dqk, Ks, Kt, tid);
    f32_tile_load<D>(vbase, p.vs[2], j0, lk, p.Dv, Vs, nullptr, tid);
    __syncthreads();
    // S^T and dP^T (m = key j0 + lane row, n = query)
    f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      st = mma32(TF32{}, lds_read16(Ks + l32 * L::RP + (2 * s + g) * 16), qreg[s], st);
      dpt = mma32(TF32{}, lds_read16(Vs + l32 * L::RP + (2 * s + g) * 16), doreg[s], dpt);
    }
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
      float x = st[r] * c;
      if (MASK) {
        const int ii = ok ? my_i : 0, jj = j < lk ? j : lk - 1;
        x += kLog2e * mask_val(p.mask, p.mask_bool,
                               b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] + (int64_t)jj * p.ms[3]);
      }
      const bool vis = ok && j < lk && (!CAUSAL || j <= my_i + coff);
      const float pr = vis ? fast_exp2(x - lse2) : 0.f;
      ds[r] = pr * (dpt[r] - dval);
    }
    // dQ^T += K^T dS^T: k-group u holds keys 8u + 4g + (0..3)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 bv = {as_uint(ds[4 * u]), as_uint(ds[4 * u + 1]), as_uint(ds[4 * u + 2]), as_uint(ds[4 * u + 3])};
        acc[mb] = mma32(TF32{}, lds_read16(Kt + (32 * mb + l32) * L::TP + (8 * u + 4 * g) * 4), bv, acc[mb]);
      }
  }

  if (my_i < p.Lq) {
    float* orow = (float*)bp.dq + b * bp.dqs[0] + hq * bp.dqs[1] + (int64_t)my_i * bp.dqs[2];
    const float sc = bp.scale;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * mb + 8 * q4 + 4 * g;
        if (d0 < p.Dqk)
          *(f32x4*)(orow + d0) = f32x4{acc[mb][4 * q4] * sc, acc[mb][4 * q4 + 1] * sc, acc[mb][4 * q4 + 2] * sc,
                                       acc[mb][4 * q4 + 3] * sc};
      }
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkv_f32_kernel(BwdParams bp) {
  const AttnParams& p = bp.f;
  using L = F32T<D>;
  constexpr int NQ = L::NQ, NMB = L::NMB;
  // Q, dO rows; Q^T, dO^T; the tile's LSE (log2 units) and D
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::RBYTES + 2 * L::TBYTES + 256];
  uint8_t* const Qs = smem;
  uint8_t* const Ds = smem + L::RBYTES;
  uint8_t* const Qt = smem + 2 * L::RBYTES;
  uint8_t* const Dt = Qt + L::TBYTES;
  float* const Ls = (float*)(Dt + L::TBYTES);
  float* const Dd = Ls + 32;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  // key blocks in increasing order: under causal masking the first key
  // blocks are seen by the most query rows, so the heaviest go first
  const int nbh = p.B * p.Hkv;
  const int kt = (int)blockIdx.x / nbh, bhk = (int)blockIdx.x % nbh;
  const int b = bhk / p.Hkv, hk = bhk % p.Hkv;
  const int lq = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_q, b, p.Lq));
  const int lk = __builtin_amdgcn_readfirstlane(batch_len(p.seqlens_k, b, p.Lk));
  const int coff = lk - lq;
  const int k0 = kt * 128;
  const int kw0 = k0 + 32 * wave;
  const int my_j = kw0 + l32;
  const bool kok = my_j < lk;
  const float c = p.scale_log2;

  // this lane's key and value rows as B operands (zero past the real dims)
  u32x4 kreg[NQ], vreg[NQ];
  {
    const int jj = kok ? my_j : 0;
    const float* kr = (const float*)p.k + b * p.ks[0] + hk * p.ks[1] + (int64_t)jj * p.ks[2];
    const float* vr = (const float*)p.v + b * p.vs[0] + hk * p.vs[1] + (int64_t)jj * p.vs[2];
    const int nk = p.Dqk / 4, nv = p.Dv / 4;
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int ch = 2 * s + g;
      const u32x4 a = ldg16_cached(kr + min(ch, nk - 1) * 4), d = ldg16_cached(vr + min(ch, nv - 1) * 4);
      kreg[s] = kok && ch < nk ? a : u32x4{0, 0, 0, 0};
      vreg[s] = kok && ch < nv ? d : u32x4{0, 0, 0, 0};
    }
  }

  // query tiles [qt0, nqt) of 32 rows, for every query head of the group
  const int ibeg = CAUSAL ? max(0, k0 - coff) : 0;
  const int qt0 = ibeg / 32;
  const int nqt = k0 < lk ? (lq + 31) / 32 : 0;
  const int per_head = max(0, nqt - qt0);
  const int ntiles = per_head * p.group;

  f32x16 dk[NMB], dv[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) dk[mb] = dv[mb] = f32x16{};
  for (int t = 0; t < ntiles; ++t) {
    const int hq = hk * p.group + t % p.group;
    const int q0 = 32 * (qt0 + t / p.group);
    __syncthreads();  // the previous tile is no longer read
    const float* qb = (const float*)p.q + b * p.qs[0] + hq * p.qs[1];
    const float* db = (const float*)bp.dout + b * bp.dos[0] + hq * bp.dos[1];
    f32_tile_load<D>(qb, p.qs[2], q0, lq, p.Dqk, Qs, Qt, tid);
    f32_tile_load<D>(db, bp.dos[2], q0, lq, p.Dv, Ds, Dt, tid);
    if (tid < 32) {
      const int i = q0 + tid;
      const int64_t row = ((int64_t)b * p.Hq + hq) * p.Lq + (i < p.Lq ? i : 0);
      Ls[tid] = i < lq ? bp.ws_l[row] : __builtin_inff();
      Dd[tid] = i < lq ? bp.ws_d[row] : 0.f;
    }
    __syncthreads();
    // nothing of this wave's keys is visible to the tile's rows
    if (kw0 >= lk || (CAUSAL && kw0 > q0 + 31 + coff)) continue;
    // S and dP (m = query q0 + lane row, n = key)
    f32x16 s_ = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      s_ = mma32(TF32{}, lds_read16(Qs + l32 * L::RP + (2 * s + g) * 16), kreg[s], s_);
      dp = mma32(TF32{}, lds_read16(Ds + l32 * L::RP + (2 * s + g) * 16), vreg[s], dp);
    }
    f32x16 pr, ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = 8 * (r >> 2) + 4 * g + (r & 3), i = q0 + ir;
      float x = s_[r] * c;
      if (MASK) {
        const int ii = i < lq ? i : lq - 1, jj = kok ? my_j : lk - 1;
        x += kLog2e * mask_val(p.mask, p.mask_bool,
                               b * p.ms[0] + hq * p.ms[1] + (int64_t)ii * p.ms[2] + (int64_t)jj * p.ms[3]);
      }
      const bool vis = kok && i < lq && (!CAUSAL || my_j <= i + coff);
      pr[r] = vis ? fast_exp2(x - Ls[ir]) : 0.f;
      ds[r] = pr[r] * (dp[r] - Dd[ir]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS: k-group u holds rows 8u + 4g + (0..3)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 pb = {as_uint(pr[4 * u]), as_uint(pr[4 * u + 1]), as_uint(pr[4 * u + 2]), as_uint(pr[4 * u + 3])};
        const u32x4 db = {as_uint(ds[4 * u]), as_uint(ds[4 * u + 1]), as_uint(ds[4 * u + 2]), as_uint(ds[4 * u + 3])};
        const int off = (32 * mb + l32) * L::TP + (8 * u + 4 * g) * 4;
        dv[mb] = mma32(TF32{}, lds_read16(Dt + off), pb, dv[mb]);
        dk[mb] = mma32(TF32{}, lds_read16(Qt + off), db, dk[mb]);
      }
  }

  if (my_j < p.Lk) {
    float* kr = (float*)bp.dk + b * bp.dks[0] + hk * bp.dks[1] + (int64_t)my_j * bp.dks[2];
    float* vr = (float*)bp.dv + b * bp.dvs[0] + hk * bp.dvs[1] + (int64_t)my_j * bp.dvs[2];
    const float sc = bp.scale;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * mb + 8 * q4 + 4 * g;
        if (d0 < p.Dqk)
          *(f32x4*)(kr + d0) = f32x4{dk[mb][4 * q4] * sc, dk[mb][4 * q4 + 1] * sc, dk[mb][4 * q4 + 2] * sc,
                                     dk[mb][4 * q4 + 3] * sc};
        if (d0 < p.Dv)
          *(f32x4*)(vr + d0) = f32x4{dv[mb][4 * q4], dv[mb][4 * q4 + 1], dv[mb][4 * q4 + 2], dv[mb][4 * q4 + 3]};
      }
  }
}

template <class T, int D, bool CAUSAL, bool MASK>
hipError_t launch_main(const BwdParams& bp, hipStream_t s) {
  const AttnParams& p = bp.f;
  const dim3 block(kBwdThreads);
  if constexpr (std::is_same<T, TF32>::value) {
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL, MASK>), dim3((unsigned)((p.Lq + 127) / 128 * p.B * p.Hq)),
                       block, 0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkv_f32_kernel<D, CAUSAL, MASK>), dim3((unsigned)((p.Lk + 127) / 128 * p.B * p.Hkv)),
                       block, 0, s, bp);
    return hipGetLastError();
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, MASK>), dim3((unsigned)((p.Lq + 127) / 128 * p.B * p.Hq)),
                       block, 0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkv_kernel<T, D, CAUSAL, MASK>),
                       dim3((unsigned)((p.Lk + kDkvKeys - 1) / kDkvKeys * p.B * p.Hkv * bp.hsplit)), dim3(kDkvThreads),
                       0, s, bp);
    e = hipGetLastError();
    if (e != hipSuccess || bp.hsplit == 1) return e;
    constexpr int RPB = kBwdThreads / (2 * D / 4);
    const int64_t nrows = (int64_t)p.B * p.Hkv * p.Lk;
    hipLaunchKernelGGL((bwd_dkv_reduce_kernel<T, D>), dim3((unsigned)((nrows + RPB - 1) / RPB)), block, 0, s, bp);
    return hipGetLastError();
  }
}

template <class T, int D>
hipError_t launch_td(const BwdParams& bp, bool causal, hipStream_t s) {
  const AttnParams& p = bp.f;
  hipError_t e;
  const bool mask = p.mask != nullptr;
  if (causal) e = mask ? launch_main<T, D, true, true>(bp, s) : launch_main<T, D, true, false>(bp, s);
  else e = mask ? launch_main<T, D, false, true>(bp, s) : launch_main<T, D, false, false>(bp, s);
  if (e != hipSuccess) return e;
  if (bp.dsinks) {
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3((unsigned)p.Hq), dim3(kBwdThreads), 0, s, bp);
    e = hipGetLastError();
  }
  return e;
}

template <class T>
hipError_t launch_t(const BwdParams& bp, bool causal, hipStream_t s) {
  return bp.f.D == 64 ? launch_td<T, 64>(bp, causal, s) : launch_td<T, 128>(bp, causal, s);
}

}  // namespace

hipError_t launch_backward(const AttnParams& p, const sdpa_bwd_args& g, float scale, float* ws, int dtype,
                           bool causal, int head_split, hipStream_t s) {
  BwdParams bp{};
  bp.f = p;
  bp.scale = scale;
  bp.dout = g.dout;
  bp.dq = g.dq;
  bp.dk = g.dk;
  bp.dv = g.dv;
  for (int d = 0; d < 3; ++d) {
    bp.dos[d] = g.dout_stride[d];
    bp.dqs[d] = g.dq_stride[d];
    bp.dks[d] = g.dk_stride[d];
    bp.dvs[d] = g.dv_stride[d];
  }
  bp.dsinks = g.dsinks;
  const size_t nrows = (size_t)p.B * p.Hq * p.Lq;
  bp.ws_d = ws;
  bp.ws_l = ws + nrows;
  // (fp32 keeps one workgroup per key block and KV head)
  bp.hsplit = dtype == SDPA_F32 ? 1 : head_split;
  bp.ws_part = ws + (2 * nrows + 3) / 4 * 4;  // 16-byte aligned
  if (p.sinks == nullptr) bp.dsinks = nullptr;
  switch (dtype) {
    case SDPA_F32: return launch_t<TF32>(bp, causal, s);
    case SDPA_F16: return launch_t<TF16>(bp, causal, s);
    default: return launch_t<TBF16>(bp, causal, s);
  }
}

}  // namespace sdpa
