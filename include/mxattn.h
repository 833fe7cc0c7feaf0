/*
 * mxattn -- 4-bit block-scaled (MXFP4) FlashAttention forward for AMD MI355X
 * (gfx950).  C ABI of libmxattn.so.
 *
 * The operations and their sources:
 *   MXFP4 format  -- "BitDecoding-FP4: Algorithm-System Co-Design for Native
 *                    FP4 KV Cache Decoding", section "The KV Cache Bottleneck
 *                    in Long-Context LLM Serving": blocks of 32 elements share
 *                    one E8M0 scale; elements are FP4 E2M1.
 *   UOS scale     -- "MXAttention: Data-Free Optimal Scaling and
 *                    Pre-Normalization Quantization for MXFP4 Attention",
 *                    Abstract: the fixed boundary Qmax = 7.25.
 *   Smooth-QK,    -- "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4
 *   P-Reordering     NPUs for LLM Inference", Abstract.
 *   PNQ           -- MXAttention, Abstract.
 *   Hybrid decode,-- "HyQuant: Hybrid-Precision Quantization for LLM
 *   selection        Attention", method paragraphs.
 *
 * Conventions shared by every call
 *   - Every pointer is caller-owned device memory unless stated otherwise; the
 *     library allocates nothing and keeps no state between calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Results are ready when the stream is synchronised.
 *   - All argument checks run on the host before any launch.  On an error
 *     status nothing is launched and no output is touched; the text is in
 *     mxattn_last_error() (per thread).  A launch failure returns
 *     MXATTN_ERR_HIP.  Device faults surface at the caller's next
 *     synchronisation.
 *   - Inputs must be finite.  Rows of packed codes must be 16-byte aligned.
 *   - Thread-safe; calls on one stream execute in order.
 */
#ifndef MXATTN_H
#define MXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* mxattn_stream_t; /* hipStream_t */

typedef enum {
  MXATTN_OK = 0,
  MXATTN_ERR_INVALID_ARG = 1, /* null pointer, bad shape/stride/alignment */
  MXATTN_ERR_UNSUPPORTED = 2, /* valid but outside the supported set */
  MXATTN_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  MXATTN_ERR_HIP = 4          /* a HIP runtime call failed */
} mxattn_status_t;

typedef enum { MXATTN_F32 = 0, MXATTN_F16 = 1, MXATTN_BF16 = 2 } mxattn_dtype_t;

/* E8M0 scale rule of a block with maximum magnitude amax:
 *   OCP: e = floor(log2 amax) - 2          (amax / 2^e in [4, 8))
 *   UOS: smallest e with amax <= qmax*2^e  (amax / 2^e in (qmax/2, qmax]),
 *        qmax in (4, 8); MXAttention (Abstract) uses 7.25.
 * e is clamped to [-127, 127]; an all-zero block gets e = -127 (byte 0). */
typedef enum { MXATTN_SCALE_OCP = 0, MXATTN_SCALE_UOS = 1 } mxattn_scale_rule_t;

/* Where the 32-element blocks run:
 *   HD  -- along head_dim: row = one token, D/2 code bytes, D/32 scale bytes.
 *   KEY -- along the sequence: row = one channel d, ceil(S/32)*16 code bytes
 *          and ceil(S/32) scale bytes; a partial tail block is padded with
 *          +0 elements (code 0). */
typedef enum { MXATTN_LAYOUT_HD = 0, MXATTN_LAYOUT_KEY = 1 } mxattn_layout_t;

/* An MXFP4 tensor of logical shape [batch][heads][seq][dim].
 * Codes: two E2M1 codes per byte, element 2j in the low nibble, bit 3 of a
 * code is the sign.  Scales: one E8M0 byte (value 2^(byte-127)) per block.
 * Byte address of row r of (b, h):
 *   codes  + b*code_stride[0]  + h*code_stride[1]  + r*code_stride[2]
 *   scales + b*scale_stride[0] + h*scale_stride[1] + r*scale_stride[2]
 * where r is the token (HD) or the channel (KEY).
 * Every entry point rejects batch or heads above 65535 and seq above 2^26
 * with MXATTN_ERR_UNSUPPORTED. */
typedef struct {
  uint8_t* codes;
  uint8_t* scales;
  int64_t batch, heads, seq, dim;
  int32_t layout; /* mxattn_layout_t */
  int32_t reserved;
  int64_t code_stride[3];
  int64_t scale_stride[3];
} mxattn_mx_t;

/* ---------------------------------------------------------------------------
 * mxattn_quantize -- MXFP4-encode a [B][H][S][D] tensor (source: BitDecoding-
 * FP4, "The KV Cache Bottleneck ..."; the optional per-channel factor is the
 * Smooth-QK rescale of HiFA4, Abstract).
 *   x          bf16/fp16/fp32 values; element (b,h,s,d) at
 *              x + (b*x_stride[0] + h*x_stride[1] + s*x_stride[2] + d) elements;
 *              x and every row start must be 16-byte aligned.
 *   chan_scale nullable; fp32 [H][D], 16-byte aligned.  Each value is first widened to fp32 and
 *              multiplied by chan_scale[h][d] in IEEE fp32 (round to nearest
 *              even); the block maximum and codes are taken from that product.
 *   rule,qmax  the E8M0 rule (qmax is read for UOS only).
 *   flags      0, or MXATTN_QUANT_HADAMARD: after the channel multiply each
 *              head-dim row is rotated by the normalised Walsh-Hadamard
 *              transform (BitDecoding-FP4, key outliers: Hadamard rotation),
 *              computed in fp32 as butterflies (a, b) -> (a + b, a - b) on
 *              element pairs (i, i + h), i & h = 0, for h = 1, 2, ..., D/2 in
 *              that order, then one multiply by fp32(1/sqrt(D)).  Rotate Q
 *              and K alike (dot products are unchanged), never V.  HD layout
 *              only (MXATTN_ERR_UNSUPPORTED otherwise); other bits are
 *              MXATTN_ERR_INVALID_ARG.
 *   out        destination; out->{batch,heads,seq,dim} must equal the input
 *              shape, out->layout selects the block axis.
 * Codes are round-to-nearest-even onto {0,.5,1,1.5,2,3,4,6} of x/2^e, ties to
 * the even code, saturating at 6, sign kept (a negative value that rounds to
 * zero is code 8).  Supported: D in {64, 128}; any S >= 1 (HD) or S >= 1 with
 * padding (KEY).  Cost: one pass over x (HBM-bound). */
#define MXATTN_QUANT_HADAMARD 1
mxattn_status_t mxattn_quantize(const void* x, mxattn_dtype_t x_dtype, const int64_t x_stride[3],
                                const float* chan_scale, mxattn_scale_rule_t rule, float qmax, int32_t flags,
                                const mxattn_mx_t* out, mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_quantize_dual -- dual-residual MXFP4 (BitDecoding-FP4, "Dual-Residual
 * Query Quantization": the query split into two FP4 tensors).  `out`
 * receives exactly what mxattn_quantize writes for the same arguments;
 * `out_res` receives the MXFP4 encoding, same rule and blocks, of the
 * residual x' - dequant(out), where x' is x after the optional channel
 * multiply.  The residual is formed in fp32 and is exact (the dequantised
 * value is 0 or within a factor of two of x').  Pass both to mxattn_decode
 * (q and q_res): the logits then use dequant(out) + dequant(out_res).
 * Both descriptors must use the HD layout and the same shape
 * (MXATTN_ERR_UNSUPPORTED for KEY, MXATTN_ERR_INVALID_ARG for a shape
 * mismatch); the other arguments and checks are those of mxattn_quantize. */
mxattn_status_t mxattn_quantize_dual(const void* x, mxattn_dtype_t x_dtype, const int64_t x_stride[3],
                                     const float* chan_scale, mxattn_scale_rule_t rule, float qmax, int32_t flags,
                                     const mxattn_mx_t* out, const mxattn_mx_t* out_res, mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_quantize_batch -- the same encoding as mxattn_quantize for up to
 * MXATTN_MAX_QUANTIZE_JOBS tensors in one launch (for instance the Q, K and
 * V of one attention call, which are too small to fill the device one at a
 * time).  Each job carries exactly the arguments of mxattn_quantize, with
 * the same meaning and checks; the results are bit-identical to calling
 * mxattn_quantize once per job.  Jobs may differ in dtype, shape, layout and
 * rule.  The outputs of different jobs must not overlap each other or any
 * job's input (not checked; overlapping jobs give unspecified results).
 * Errors: MXATTN_ERR_INVALID_ARG for a null list or n_jobs outside
 * [1, MXATTN_MAX_QUANTIZE_JOBS]; otherwise the first failing job's error,
 * with nothing launched. */
#define MXATTN_MAX_QUANTIZE_JOBS 4
typedef struct {
  const void* x;
  mxattn_dtype_t x_dtype;
  int32_t flags;   /* as mxattn_quantize */
  int64_t x_stride[3];
  const float* chan_scale;
  mxattn_scale_rule_t rule;
  float qmax;
  const mxattn_mx_t* out;
} mxattn_quantize_job_t;
mxattn_status_t mxattn_quantize_batch(const mxattn_quantize_job_t* jobs, int32_t n_jobs, mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_smooth_calibrate -- static per-channel Smooth-QK factors from a
 * calibration slice (HiFA4, Abstract; BitDecoding-FP4, "Outlier-Aware Key
 * Quantization": static smoothing).
 *   q_cal  [Hq][T][D], k_cal [Hkv][T][D], contiguous, bf16/fp16/fp32.
 *   For KV head h and channel c, with qmax = max |q| over the T tokens and the
 *   Hq/Hkv query heads of h, and kmax = max |k| over the T tokens:
 *     s = sqrt(kmax/qmax) in IEEE double (1 if either max is 0), clamped to
 *     [2^-8, 2^8];  q_scale[g][c] = (float)s for every query head g of h,
 *     k_scale[h][c] = (float)(1/s).
 *   q_scale fp32 [Hq][D], k_scale fp32 [Hkv][D] (outputs).
 * Supported: Hq % Hkv == 0, D <= 256, T >= 1. */
mxattn_status_t mxattn_smooth_calibrate(const void* q_cal, const void* k_cal, mxattn_dtype_t dtype,
                                        int64_t hq, int64_t hkv, int64_t tokens, int64_t dim,
                                        float* q_scale, float* k_scale, mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_prefill -- MXFP4 FlashAttention forward with pre-normalisation P
 * quantisation (HiFA4, Abstract: 4-bit QK^T and PV, normaliser from the same
 * quantised P_hat that feeds PV; MXAttention, Abstract: PNQ, UOS).
 *   q  HD layout  [B][Hq][Sq][D]
 *   k  HD layout  [B][Hkv][Sk][D]
 *   v  KEY layout [B][Hkv][Sk][D]   (32-key blocks per channel)
 * For each query row and key tile of kv_tile keys, in ascending order:
 *   s = softmax_scale * (q_hat . k_hat); causal masks key t > query i;
 *   m' = max(m, max s); P~ = exp(s - m'); P_hat = MXFP4(P~) per 32 keys of the
 *   row (tile-aligned blocks, p_rule/p_qmax); l = exp(m-m') l + sum P_hat
 *   (sum P~ when l_from_quantized = 0); O = exp(m-m') O + P_hat v_hat.
 *   out = O / l, fp32/fp16/bf16 [B][Hq][Sq][D] contiguous; lse (nullable) =
 *   m + ln l, fp32 [B][Hq][Sq].  Query head g reads KV head g/(Hq/Hkv).
 * Softmax state is fp32; P_hat never leaves registers.
 * Supported: D in {64,128}; kv_tile in {64,128,256}; causal needs Sq == Sk;
 * Hq % Hkv == 0; p_qmax in (4, 8) for UOS; one (batch, KV head) of K spans
 * less than 2 GiB (Sk rounded up to 256 rows x row stride, codes and scales
 * alike) and so does one of V (D x row stride); MXATTN_ERR_UNSUPPORTED
 * otherwise. */
typedef struct {
  int32_t causal;
  float softmax_scale;      /* 0 selects 1/sqrt(D) */
  int32_t kv_tile;          /* Bc; 0 selects 128 */
  int32_t p_rule;           /* mxattn_scale_rule_t for P */
  float p_qmax;
  int32_t l_from_quantized; /* 1 = PNQ / P-Reordering, 0 = baseline */
} mxattn_prefill_params_t;

mxattn_status_t mxattn_prefill(const mxattn_mx_t* q, const mxattn_mx_t* k, const mxattn_mx_t* v,
                               const mxattn_prefill_params_t* params, void* out,
                               mxattn_dtype_t out_dtype, float* lse, mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_prefill_hybrid -- causal mxattn_prefill in which each query row keeps
 * some keys in bf16 under the same online softmax (HyQuant, prefill
 * paragraph: the 4-bit and full-precision paths share one FlashAttention
 * kernel and one softmax; vertical lines and a local window stay in full
 * precision).
 *   Query row i uses the bf16 rows for keys i - window < t <= i (its window,
 *   itself included) and for the selected keys t <= i in idx[b][h][0..n_sel)
 *   (strictly ascending; entries outside [0, S) are ignored; n_sel is
 *   clamped to [0, max_sel] on the device).  Every other key t <= i takes
 *   the MXFP4 path of mxattn_prefill.
 *   Order: the MXFP4 tiles first, exactly as mxattn_prefill on the remaining
 *   keys (the bf16 keys contribute 0 there and never raise a P block
 *   maximum), then the bf16 keys: logits softmax_scale * (q_bf16 . k_bf16),
 *   P unquantised (entering the bf16 MFMA as hi + lo parts), l += sum P.
 *   q, k, v    MXFP4 operands as for mxattn_prefill (may be rotated or
 *              smoothed; the bf16 rows are used as given).
 *   hybrid->q  bf16 [B][Hq][S][D] contiguous; hybrid->k, ->v bf16
 *              [B][Hkv][S][D] contiguous; all 16-byte aligned.
 * Supported: params->causal = 1, S <= 65536, window >= 0, max_sel >= 0 (idx
 * and n_sel may be NULL when max_sel = 0); otherwise as mxattn_prefill. */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;   /* [B][Hkv][max_sel] */
  const int32_t* n_sel; /* [B][Hkv] */
  int32_t max_sel;
  int32_t window;
} mxattn_prefill_hybrid_t;

mxattn_status_t mxattn_prefill_hybrid(const mxattn_mx_t* q, const mxattn_mx_t* k, const mxattn_mx_t* v,
                                      const mxattn_prefill_params_t* params,
                                      const mxattn_prefill_hybrid_t* hybrid, void* out,
                                      mxattn_dtype_t out_dtype, float* lse, mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_decode -- one query token per sequence against an MXFP4 KV cache,
 * dequantisation fused into the scan, optionally with a bf16 hybrid token set
 * under the same softmax (HyQuant, method paragraphs).
 *   q        HD layout [B][Hq][1][D] (MXFP4 query).  Or a descriptor with
 *            codes and scales NULL, which gives only the shape: the scan then
 *            encodes q_bf16 itself (OCP rule, no channel factors), with the
 *            codes mxattn_quantize would write, so one call does the step.
 *   q_res    nullable; HD layout, same shape: the residual part of a
 *            dual-residual query (mxattn_quantize_dual).  The 4-bit logits
 *            then use dequant(q) + dequant(q_res) (one more QK^T MFMA per
 *            chunk); the bf16 hybrid tokens keep using q_bf16.  Needs an
 *            encoded q.
 *   q_bf16   bf16 [B][Hq][D] contiguous, 16-byte aligned; read when hybrid
 *            != NULL or when q comes without codes.
 *   k_cache, v_cache  HD layout [B][Hkv][Tcap][D].
 *   ctx_len  device int32 [B]; token t of sequence b is attended iff
 *            t < ctx_len[b] (1 <= ctx_len[b] <= Tcap, checked on the device:
 *            out-of-range lengths are clamped).
 *   hybrid   nullable.  Tokens in idx[b][h][0..n_sel) (ascending, all below
 *            ctx-window) and the last `window` tokens [ctx-window, ctx) use
 *            q_bf16 and the bf16 rows k_sel/v_sel [B][Hkv][max_sel][D] and
 *            k_win/v_win [B][Hkv][window][D] (row w = token ctx-window+w);
 *            every other token uses the MXFP4 operands.  Each token counts
 *            once; one softmax covers all of them.
 *   split_len  tokens per split (multiple of 64; at most 8192 with a hybrid
 *            set); the splits (and the bf16 set, in parts of 512 rows) are
 *            merged with their log-sum-exp in a fixed order (deterministic);
 *            at most 4096 parts in total.
 *   workspace  device memory of mxattn_decode_workspace_bytes(...) bytes.
 *   out      fp32 [B][Hq][D];  lse nullable fp32 [B][Hq].
 * P is not quantised; logits and softmax state are fp32.
 * Supported: D = 128 (D = 64 also), Hq/Hkv in {1,2,4,8}; one (batch, KV
 * head) of each cache spans less than 2 GiB (Tcap x row stride). */
typedef struct {
  const int32_t* idx;   /* [B][Hkv][max_sel] */
  const int32_t* n_sel; /* [B][Hkv] */
  int32_t max_sel;
  int32_t window;
  const void* k_sel; /* bf16 [B][Hkv][max_sel][D] */
  const void* v_sel;
  const void* k_win; /* bf16 [B][Hkv][window][D] */
  const void* v_win;
} mxattn_hybrid_t;

/* Workspace of mxattn_decode: hybrid_rows = max_sel + window of the hybrid
 * set (0 without one).  Returns 0 for invalid sizes. */
size_t mxattn_decode_workspace_bytes(int64_t batch, int64_t hq, int64_t hkv, int64_t dim,
                                     int64_t tcap, int32_t split_len, int32_t hybrid_rows);

mxattn_status_t mxattn_decode(const mxattn_mx_t* q, const mxattn_mx_t* q_res, const void* q_bf16,
                              const mxattn_mx_t* k_cache,
                              const mxattn_mx_t* v_cache, const int32_t* ctx_len,
                              const mxattn_hybrid_t* hybrid, float softmax_scale,
                              int32_t split_len, void* workspace, size_t workspace_bytes,
                              float* out, float* lse, mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_decode_noalloc -- mxattn_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The partial slots
 * live in a library-owned device array of 16 MiB (MXATTN_DECODE_SCRATCH_BYTES)
 * that each GPU holds, once the library has run on it, until the process
 * ends; the call allocates and frees nothing.  Every argument and the result
 * are those of mxattn_decode (same kernels, the same bits).
 *   A problem whose mxattn_decode_workspace_bytes exceeds the scratch is
 *   refused with MXATTN_ERR_UNSUPPORTED before anything runs (a longer
 *   split_len needs fewer slots).
 *   The first call on a device looks up the array's device address
 *   (MXATTN_ERR_HIP if that fails).
 *   All calls on one GPU share its array and it keeps the last call's
 *   contents: calls that may overlap on one GPU (different streams, or
 *   several host threads) race and must be serialised by the caller. */
#define MXATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

mxattn_status_t mxattn_decode_noalloc(const mxattn_mx_t* q, const mxattn_mx_t* q_res, const void* q_bf16,
                                      const mxattn_mx_t* k_cache, const mxattn_mx_t* v_cache,
                                      const int32_t* ctx_len, const mxattn_hybrid_t* hybrid,
                                      float softmax_scale, int32_t split_len, float* out, float* lse,
                                      mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_decode_paged -- mxattn_decode over a paged MXFP4 KV cache
 * (BitDecoding-FP4, "System-Level Optimization": the cache is split into
 * fixed-size pages placed anywhere in GPU memory and found through a block
 * table, at the cost of indirect loads of codes and scale factors).
 *   k_pool, v_pool  HD layout with batch = number of pages, seq = page_size:
 *            codes [n_pages][Hkv][page_size][D/2] (any strides, as for
 *            mxattn_mx_t), one page holding page_size consecutive tokens of
 *            one sequence for every KV head.
 *   paging->block_table  device int32 [B][max_pages]: physical page of the
 *            sequence's logical page j (tokens [j*page_size, (j+1)*page_size)).
 *            Entries of pages holding tokens below ctx_len must lie in
 *            [0, n_pages); any other entry reads as zero codes (never stray
 *            memory), so it must not be reached.
 *   Capacity per sequence: Tcap = max_pages * page_size (ctx_len is clamped
 *   to it on the device; workspace from mxattn_decode_workspace_bytes with
 *   tcap = Tcap).  Every other argument, the dual-residual query and the
 *   hybrid set included, is as for mxattn_decode, and the result is the one
 *   mxattn_decode gives on the contiguous cache the pages spell out.
 * Supported: page_size a multiple of 32; split_len a multiple of page_size
 * and at most 64 pages; one page of one head below 2 GiB. */
typedef struct {
  const int32_t* block_table;
  int32_t max_pages;
} mxattn_paging_t;

mxattn_status_t mxattn_decode_paged(const mxattn_mx_t* q, const mxattn_mx_t* q_res, const void* q_bf16,
                                    const mxattn_mx_t* k_pool, const mxattn_mx_t* v_pool,
                                    const mxattn_paging_t* paging, const int32_t* ctx_len,
                                    const mxattn_hybrid_t* hybrid, float softmax_scale, int32_t split_len,
                                    void* workspace, size_t workspace_bytes, float* out, float* lse,
                                    mxattn_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxattn_select_vertical -- accumulate column mass and pick the top-rho
 * vertical-line tokens of the non-window prefix (HyQuant, method paragraphs).
 *   q_recent HD layout [B][Hq][R][D], R <= 64 recent MXFP4 queries.
 *   k_cache  HD layout [B][Hkv][Tcap][D].
 *   col_mass fp32 [B][Hkv][Tcap], in/out: for every recent query r and query
 *            head g of KV head h, col_mass[b][h][t] += softmax over t' < ctx of
 *            softmax_scale * q_hat.k_hat_t', for t < ctx.
 *   Then k = ceil((ctx-window) * rho_num / rho_den) (integer arithmetic)
 *   tokens of [0, ctx-window) with the largest mass (ties to the lower index)
 *   are written ascending to idx_out [B][Hkv][max_sel]; n_out [B][Hkv] = k;
 *   the remaining entries of idx_out are -1.  Masses are ordered by their
 *   fp32 bit patterns as unsigned integers, which is their value order when
 *   they are non-negative; exactly k indices are written whatever the bits.
 *   q_recent may be NULL (R = 0): col_mass is left unchanged and only the
 *   selection runs.
 *   workspace  device memory of mxattn_select_workspace_bytes(...) bytes.
 * Supported: D in {64,128}; R <= 64; Tcap <= 65536; max_sel must cover the
 * worst case ceil((Tcap-window) * rho_num / rho_den). */
size_t mxattn_select_workspace_bytes(int64_t batch, int64_t hq, int64_t recent, int64_t tcap);

mxattn_status_t mxattn_select_vertical(const mxattn_mx_t* q_recent, const mxattn_mx_t* k_cache,
                                       const int32_t* ctx_len, float softmax_scale,
                                       int32_t window, int32_t rho_num, int32_t rho_den,
                                       float* col_mass, int32_t* idx_out, int32_t* n_out,
                                       int32_t max_sel, void* workspace, size_t workspace_bytes,
                                       mxattn_stream_t stream);

const char* mxattn_status_string(mxattn_status_t status);
const char* mxattn_last_error(void);
const char* mxattn_version(void);

/* ---------------------------------------------------------------------------
 * mxattn_gather_rows -- the bf16 K and V rows of the selected tokens, copied
 * into the contiguous arrays the hybrid decode reads (HyQuant, method
 * paragraphs: the vertical-line tokens stay in full precision beside the
 * 4-bit cache; the page does not say where those rows come from, so the
 * caller keeps them and this call gathers them after each selection).
 *   k, v        bf16 [B][H][T][D] (shape), element strides k_stride /
 *               v_stride for the batch, head and token axes; channels
 *               contiguous; rows 16-byte aligned.
 *   idx, n_sel  device int32 [B][H][max_sel] and [B][H], as written by
 *               mxattn_select_vertical; rows 0 .. n_sel-1 of each (b, h) are
 *               copied (n_sel clamped to [0, max_sel] on the device).
 *   k_out, v_out  bf16 [B][H][max_sel][D] contiguous (caller-owned): row i
 *               holds token idx[b][h][i]; an index outside [0, T) gives a
 *               zero row; rows at or past n_sel are left untouched.
 * Supported: D in {64, 128}; B x H <= 65535.  max_sel = 0 does nothing. */
mxattn_status_t mxattn_gather_rows(const void* k, const void* v, const int64_t shape[4], const int64_t k_stride[3],
                                   const int64_t v_stride[3], const int32_t* idx, const int32_t* n_sel,
                                   int32_t max_sel, void* k_out, void* v_out, mxattn_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MXATTN_H */
