/*
 * sdpa_mi355x.h -- C ABI of the MI355X (gfx950) fused scaled-dot-product
 * attention forward library, libsdpa_mi355x.so.
 *
 * The library computes, for every batch b and query head hq,
 *
 *     O = softmax(scale * Q K^T + mask) V
 *
 * without materialising the Lq x Lk score matrix, in two forms:
 *
 *   sdpa_prefill  tiled full / causal self-attention with an online (running
 *                 max, running sum) softmax -- the forward kernel of the
 *                 rustytorch "flash_attention.metal" page ("Online softmax
 *                 update", "Write final output") and the full self-attention
 *                 kernels of the "Metal shaders for memory efficient self
 *                 attention on large sequences" page;
 *   sdpa_decode   single-query "vector" attention (Lq == 1) with a single-pass
 *                 and a two-pass split-K variant -- the two vector kernels of
 *                 the "Add D512 support to Metal vector attention" page --
 *                 extended to a few query rows (Lq <= 16: speculative or
 *                 chunked decoding, the qL4 control of that page).
 *
 * The optional inputs follow the SDPA graph attributes configured by
 * build_sdpa_graph on the "mlx 0.30.7 -- backend/cuda/
 * scaled_dot_product_attention.cpp" page: attention scale, log-sum-exp
 * statistics output, bottom-right causal mask, additive bias, sink token.
 *
 * Semantics (the same for both entry points):
 *   - query head hq reads KV head hq / (Hq / Hkv)   (Hq % Hkv must be 0);
 *   - S[i,j] = scale * (q_i . k_j) computed from the dtype inputs with fp32
 *     products and fp32 accumulation, then + mask[b,hq,i,j] (fp32), or -inf
 *     where a boolean mask is 0.  One exception: an fp16 sdpa_prefill call
 *     without mask and without lse output, with c = |scale| * log2(e) <= 1
 *     (every D >= 3 at the default scale), multiplies each q element by c once
 *     and rounds it to fp16 before the product, so that the matrix cores
 *     deliver the exponent directly.  That is one more rounding of at most
 *     2^-11 relative per q element: |error of S[i,j]| <= 2^-11 * |scale| *
 *     sum_d |q_id k_jd|, which perturbs each probability by a factor within
 *     exp(+-that bound).  Calls that return lse keep the exact fp32 scale, so
 *     O may differ in its last bits between the two kinds of call;
 *   - causal (bottom-right): key j is visible to query i iff
 *     j <= i + (Lk - Lq); for Lq == 1 every key is visible;
 *   - sinks[hq] (fp32, not multiplied by scale) adds exp(sinks[hq]) to the
 *     softmax denominator and nothing to the numerator;
 *   - lse[b,hq,i] = natural log of the full softmax denominator (including
 *     the sink term);
 *   - a row that sees no key and has no sink gets O = 0 and lse = -inf; a row
 *     that sees no key but has a sink gets O = 0 and lse = sink.
 *   - per-batch lengths (optional; the padding mask of the cuDNN graph on the
 *     mlx 0.30.7 page: set_padding_mask with set_seq_len_q / set_seq_len_kv):
 *     batch b holds seqlens_q[b] real query rows and seqlens_k[b] real keys,
 *     the leading ones of its L extents (values are clamped to [0, Lq] and
 *     [0, Lk]; a NULL array means the full extent).  Keys past seqlens_k[b]
 *     are seen by no row and never read into a result (their memory may hold
 *     anything, e.g. the unused tail of a fixed-capacity KV cache); query rows
 *     past seqlens_q[b] see no key and are written like any row that sees no
 *     key; causal alignment uses the batch's own lengths:
 *     j <= i + (seqlens_k[b] - seqlens_q[b]).
 *   - fp32 inputs are computed in full fp32 (no reduced-precision products).
 *
 * Memory, ownership, threading:
 *   - every pointer in sdpa_args is DEVICE memory owned by the caller; the
 *     library never allocates, frees, retains or synchronises.  Each call
 *     only enqueues kernels on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns; execution errors surface at the caller's next
 *     synchronisation.
 *   - q, k are 4-D [B, H, L, D] and v, o [B, H, L, Dv] tensors (Dv = D
 *     unless set; the cuDNN path on the mlx page takes D_qk and D_v
 *     separately) whose last dim is contiguous; *_stride[0..2] are ELEMENT
 *     strides of the B, H and L dims.  D and Dv are multiples of 8; the
 *     kernels run at the next of 64, 128, 256, 512 above both ("kernel head
 *     dim" below) with the extra columns zero.
 *     Base pointers must be 16-byte aligned and every stride * element size
 *     a multiple of 16 bytes (the input preparation rule of prepare_sdpa_input
 *     on the mlx 0.30.7 page: unit last-dim stride, aligned pointer).  The
 *     row (L) stride of k and v may be at most 8 MiB (SDPA_ERR_UNSUPPORTED
 *     above): key tiles are addressed with 32-bit offsets from their first
 *     row.
 *   - mask (optional) is indexed mask[b*s0 + hq*s1 + i*s2 + j*s3] with
 *     mask_stride[0..3] in elements; a stride of 0 broadcasts that dim (a
 *     [B,1,1,Lk] mask passes strides {Lk, 0, 0, 1}).  mask_kind selects
 *     additive fp32 entries (4-byte aligned) or boolean uint8 entries
 *     (nonzero = visible; a hidden key is the same as an additive -inf).
 *   - sinks (optional) is fp32 [Hq], contiguous (the cuDNN path on the mlx
 *     page converts sinks to float32 in prepare_sdpa_sinks).
 *   - lse (optional output) is fp32 [B, Hq, Lq], contiguous.
 *   - seqlens_q / seqlens_k (optional) are int32 [B] device arrays, 4-byte
 *     aligned, read by the kernels (the host never reads them).  A
 *     fixed-capacity KV cache [B, Hkv, T, D] is passed as it is, no copy:
 *     Lk = T, or any Lk <= T with the head stride still T * D, plus
 *     seqlens_k for the fill level of each batch.
 *   - o must not overlap q, k, v, mask, sinks or lse.
 *
 * Errors: every argument is checked on the host BEFORE anything is enqueued;
 * on any error nothing is written, the call returns a non-zero sdpa_status and
 * sdpa_last_error() describes it.  A request no kernel covers returns
 * SDPA_ERR_UNSUPPORTED -- there is no slower fallback path (the convention of
 * force_fused on the D512 page: an explicit error instead of a silent
 * fallback).  All functions are thread-safe; sdpa_last_error() is per thread.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDPA_MI355X_ABI_VERSION 2

#ifndef SDPA_API
#define SDPA_API __attribute__((visibility("default")))
#endif

typedef enum sdpa_dtype {
  SDPA_F32 = 0,
  SDPA_F16 = 1,
  SDPA_BF16 = 2
} sdpa_dtype;

typedef enum sdpa_status {
  SDPA_OK = 0,
  SDPA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  SDPA_ERR_SHAPE = 2,       /* sizes inconsistent (B, H, L, D < 1, Hq % Hkv, ...)  */
  SDPA_ERR_UNSUPPORTED = 3, /* valid request that no kernel covers (D, dtype, ...) */
  SDPA_ERR_ALIGN = 4,       /* pointer / stride alignment or non-unit D stride     */
  SDPA_ERR_WORKSPACE = 5,   /* decode workspace missing or too small               */
  SDPA_ERR_ARG = 6,         /* bad scalar (non-finite scale), overlap, bad splits  */
  SDPA_ERR_HIP = 7          /* the HIP runtime rejected a launch                   */
} sdpa_status;

/* How `mask` is read: additive fp32 values, or a boolean (one byte per
 * entry, nonzero = the key is visible, 0 = hidden; the boolean masks of the
 * MLX SDPA API, which the CUDA backend on the mlx 0.30.7 page reports as
 * unsupported, supports_bool_mask). */
typedef enum sdpa_mask_kind {
  SDPA_MASK_ADD_F32 = 0,
  SDPA_MASK_BOOL = 1
} sdpa_mask_kind;

typedef struct sdpa_args {
  int64_t B;        /* batch                                   */
  int64_t Hq;       /* query heads                             */
  int64_t Hkv;      /* key/value heads (Hq % Hkv == 0)         */
  int64_t Lq;       /* queries per head                        */
  int64_t Lk;       /* keys per head                           */
  int64_t D;        /* head dim of q and k (v, o: Dv below)    */
  int32_t dtype;    /* sdpa_dtype of q, k, v and o             */
  int32_t causal;   /* 0 or 1, bottom-right aligned            */
  float scale;      /* multiplies q.k; must be finite          */
  int32_t mask_kind; /* sdpa_mask_kind of mask (ignored without) */
  const void *q;    int64_t q_stride[3];   /* [B, Hq,  Lq, D] */
  const void *k;    int64_t k_stride[3];   /* [B, Hkv, Lk, D] */
  const void *v;    int64_t v_stride[3];   /* [B, Hkv, Lk, D] */
  void *o;          int64_t o_stride[3];   /* [B, Hq,  Lq, D] output, dtype */
  const float *mask; int64_t mask_stride[4]; /* optional [B, Hq, Lq, Lk] fp32 */
  const float *sinks;                        /* optional [Hq] fp32            */
  float *lse;                                /* optional [B, Hq, Lq] fp32 out */
  const int32_t *seqlens_q;                  /* optional [B] real query rows  */
  const int32_t *seqlens_k;                  /* optional [B] real keys        */
  int64_t Dv;       /* head dim of v and o; 0 means D          */
} sdpa_args;

/* Prefill / full self-attention, any Lq >= 1, Lk >= 1.
 * Supported: D, Dv multiples of 8 up to 512 (kernel head dim 64, 128, 256,
 * 512), dtypes F32, F16, BF16.  Kernel head dim 64 or 128 (any dtype) and 256
 * (F16, BF16) run on 128-row tiles; 512, and 256 in F32, run 16 columns
 * (query rows x the query heads of a KV head) per workgroup, the kernel the
 * decode path uses, in a single pass over the keys.
 * One kernel launch; no workspace. */
SDPA_API int sdpa_prefill(const sdpa_args *args, void *stream);

/* Host-only validation of a prefill request (no GPU work, no HIP calls).
 * Returns what sdpa_prefill would return before launching. */
SDPA_API int sdpa_prefill_check(const sdpa_args *args);

/* Prefill with a workspace: the same results as sdpa_prefill (up to the
 * rounding order of the merge), which it calls when
 * sdpa_prefill_workspace_bytes() is 0.  Otherwise (F16 / BF16, not causal,
 * no mask, no per-batch lengths, kernel head dim 64 or 128, and a 128-row
 * tile count that is not a multiple of 256) the tiles past the last multiple
 * of 256 (at most 128 of them) each run as two pieces of the key range, each
 * piece writing its
 * partial numerators, running max and row sum to the workspace, and a second
 * kernel merges the pieces by the rescaling of the two-pass split-K vector
 * kernel of the "Add D512 support to Metal vector attention" page (the same
 * algebra as the rustytorch "flash_attention.metal" page's "Online softmax
 * update"), sink and log-sum-exp included.  Two launches on `stream`.  The
 * workspace is device memory of at least sdpa_prefill_workspace_bytes()
 * bytes, 16-byte aligned, caller-owned; its contents need not be initialised
 * and are overwritten.
 * SDPA_ERR_WORKSPACE if it is needed and missing, too small or misaligned. */
SDPA_API int sdpa_prefill_ws(const sdpa_args *args, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Workspace bytes sdpa_prefill_ws needs for these arguments (0: none, and
 * sdpa_prefill_ws is sdpa_prefill).  Host-only; reads the sizes, dtype, the
 * causal flag and whether mask / seqlens pointers are set (no other pointer
 * or stride); 0 for invalid sizes. */
SDPA_API size_t sdpa_prefill_workspace_bytes(const sdpa_args *args);

/* Decode: single-query (Lq == 1) or multi-query (1 <= Lq <= 16) attention
 * whose keys stream once per KV head.  The Lq query rows and the Hq / Hkv
 * query heads sharing a KV head are processed together; causal is
 * bottom-right within the query block (it has no effect for Lq == 1).
 * Supported: head dims that are multiples of 8 up to 512 (kernel head dim
 * 64, 128, 256, 512); dtype F32, F16, BF16; any Hq / Hkv.
 * num_splits = 0 picks the split count automatically; 1 forces the
 * single-pass kernel; n >= 2 forces the two-pass split-K kernel pair with n
 * splits of the key range (n <= Lk).  The two-pass form needs a workspace of
 * sdpa_decode_workspace_bytes() bytes of device memory (16-byte aligned,
 * caller-owned, contents need not be initialised; it is overwritten). */
SDPA_API int sdpa_decode(const sdpa_args *args, int num_splits,
                void *workspace, size_t workspace_bytes, void *stream);

/* Host-only validation of a decode request (no GPU work, no HIP calls). */
SDPA_API int sdpa_decode_check(const sdpa_args *args, int num_splits,
                      const void *workspace, size_t workspace_bytes);

/* Decode that allocates nothing, for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels, split choice and results as sdpa_decode, but the
 * two-pass form keeps its split partials in a static device array of the
 * library instead of a caller workspace: SDPA_DECODE_SCRATCH_BYTES (16 MiB)
 * on each GPU the library runs on, held until the process ends.  A request
 * whose partials need more (sdpa_decode_workspace_bytes() above that, e.g.
 * B * Hq * Lq * splits * (kernel head dim + 2) * 4 > 16 MiB) returns
 * SDPA_ERR_WORKSPACE before anything is enqueued: pass fewer splits, or use
 * sdpa_decode with a workspace.  The array belongs to the CURRENT device and
 * `stream` must belong to it too (SDPA_ERR_ARG otherwise).  Every call on one
 * GPU shares the array and leaves its partials there, so calls that overlap
 * on one GPU (other streams, other host threads) race: the caller orders
 * them.  The first call on each device looks up the array's device address
 * (hipGetSymbolAddress); no call allocates, frees or synchronises. */
#define SDPA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
SDPA_API int sdpa_decode_noalloc(const sdpa_args *args, int num_splits, void *stream);

/* Number of key-range splits sdpa_decode will use for this request and
 * num_splits value (0 = automatic); 1 means the single-pass kernel.
 * Returns 0 when the request is invalid. */
SDPA_API int sdpa_decode_num_splits(const sdpa_args *args, int num_splits);

/* Workspace bytes sdpa_decode needs for this request and num_splits
 * (0 when the single-pass kernel is used or the request is invalid):
 * B * Hq * Lq * splits * (kernel head dim + 2) * 4. */
SDPA_API size_t sdpa_decode_workspace_bytes(const sdpa_args *args, int num_splits);

/* ---- gradients ------------------------------------------------------------
 * The backward pass of sdpa_prefill, following the two backward kernels of
 * the rustytorch "flash_attention.metal" page (one pass per query block for
 * dQ, one per key block for dK and dV, P recomputed from the log-sum-exp,
 * D_i = dO_i . O_i) with the inputs and attributes of build_sdpa_backward_graph
 * on the mlx 0.30.7 page (q, k, v, o, dO, statistics; scale, bottom-right
 * causal mask, additive bias, sink token):
 *
 *     P = exp(S - LSE),  dS = P * (dO V^T - D),
 *     dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 *     dsinks[hq] = -sum_{b,i} exp(sinks[hq] - LSE[b,hq,i]) D[b,hq,i].
 *
 * `fwd` is the argument block of the forward call whose output is being
 * differentiated: q, k, v, mask, sinks, seqlens_q / seqlens_k, scale and
 * causal as there; lse (its log-sum-exp, REQUIRED) is read, not written.
 * o (the forward's output, [B, Hq, Lq, Dv]) is read for D_i = dO_i . O_i on
 * query blocks whose every row sees more than 256 keys (no mask), where the
 * 16-bit rounding of O averages out; for the other rows D_i is formed as
 * sum_j P_ij (dO V^T)_ij (equal to dO_i . O_i), free of that rounding.
 * dK and dV of a KV head sum over the
 * Hq / Hkv query heads that read it.  The mask is a constant (no gradient).
 * Padding rows (past seqlens_q[b]) get dQ = 0, padding keys dK = dV = 0.
 * Supported: dtype F32, F16 or BF16; D (q, k, dq, dk) and Dv (v, o, dout, dv)
 * any multiples of 8 up to 128, as in the forward.  F32 runs fp32 matrix
 * cores and takes D_i = dO_i . O_i from its fp32 O for every row.  dq, dk, dv are written in
 * the input dtype with the layout rules of q, k, v (last dim contiguous,
 * 16-byte aligned pointers and strides); dsinks (optional, used only with
 * sinks) is fp32 [Hq].  The workspace (device memory, 16-byte aligned,
 * caller-owned, need not be initialised) holds
 * sdpa_prefill_backward_workspace_bytes(): 8 * B * Hq * Lq bytes (D_i and
 * the LSE per row), rounded up to 16, plus, for 16-bit GQA calls whose
 * 256-key dK / dV blocks are split over hs query-head groups (hs the largest
 * divisor of Hq / Hkv with B * Hkv * ceil(Lk / 256) * hs <= 512),
 * hs * B * Hkv * Lk * 2 * (64 or 128, the kernel head dim) * 4 bytes of
 * fp32 dK / dV shares.  Two to four kernels are enqueued on `stream` (dQ,
 * dK/dV, a reduction of the shares when split, the sink gradient when
 * asked for); nothing is allocated or synchronised.
 * The outputs must not overlap each other, the inputs or the workspace. */
typedef struct sdpa_bwd_args {
  const void *dout; int64_t dout_stride[3];  /* [B, Hq,  Lq, Dv] upstream gradient */
  void *dq;         int64_t dq_stride[3];    /* [B, Hq,  Lq, D]  output            */
  void *dk;         int64_t dk_stride[3];    /* [B, Hkv, Lk, D]  output            */
  void *dv;         int64_t dv_stride[3];    /* [B, Hkv, Lk, Dv] output            */
  float *dsinks;                             /* optional [Hq] fp32 output         */
} sdpa_bwd_args;

SDPA_API int sdpa_prefill_backward(const sdpa_args *fwd, const sdpa_bwd_args *grad,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Host-only validation of a backward request (no GPU work, no HIP calls). */
SDPA_API int sdpa_prefill_backward_check(const sdpa_args *fwd, const sdpa_bwd_args *grad,
                                         const void *workspace, size_t workspace_bytes);

/* Workspace bytes sdpa_prefill_backward needs (0 for an invalid request). */
SDPA_API size_t sdpa_prefill_backward_workspace_bytes(const sdpa_args *fwd);

/* Static description of a status code. */
SDPA_API const char *sdpa_status_string(int status);

/* Message of the last failing call on this thread ("" if none). */
SDPA_API const char *sdpa_last_error(void);

/* Library build description (arch, ABI version). */
SDPA_API const char *sdpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
