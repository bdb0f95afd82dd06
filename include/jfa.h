/*
 * jfa.h - C ABI of libjfa.so: jagged flash attention (JFA) and generalized
 * dot-product attention (GDPA), forward and backward, on AMD MI355X (gfx950).
 *
 * What is computed (sources: the pages on Meta's GEM training work):
 *  - "Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a
 *    Different Stack", section "Bottleneck move 1": attention directly on
 *    variable-length (jagged) tensors, with custom biases and asymmetric
 *    query/key-value lengths; GDPA uses GELU or SiLU in place of softmax;
 *    removing padding exposes tile scheduling and backward accumulation.
 *  - same page, FAQ "What is a jagged tensor?": values plus offsets.
 *  - "Meta Enhances GEM Training Efficiency with Advanced LLM-Scale
 *    Innovations", section "Leveraging Compute Efficiency through Customized
 *    Kernels": MXFP8 attention.
 *
 * For sample b with n = q_len, m = kv_len, query i < n, key j < m, head h:
 *   S_ij = qk_scale * <Q[qo_b+i,h,:], K[ko_b+j,h,:]> + bias_h(b,i,j)
 *   visible(i,j) = (!causal || j <= i + (m - n))     (bottom-right aligned)
 *                  && (window == 0 || |i + (m - n) - j| < window)   (sliding window)
 *   softmax: O_i = sum_j softmax_j(S_i.) V_j over visible j; LSE_i = log sum_j exp S_ij
 *   GDPA:    O_i = w * sum_{visible j} act(S_ij) V_j, w = 1/m if kv_len_normalize else 1,
 *            act = SiLU (x*sigmoid x) or GELU (erf form)
 * Rows with no visible key: O = 0, LSE = -inf.  Backward returns the
 * gradients of <O, dO> with respect to Q, K, V.
 *
 * Conventions for every entry point:
 *  - Layout: Q, O, dO, dQ are [total_q, H, d] row-major; K, V, dK, dV are
 *    [total_kv, H, d]; LSE is fp32 [H, total_q].  Offsets are int32 [B+1],
 *    off[0] = 0, non-decreasing, off[B] = total rows; q and kv offsets are
 *    independent (asymmetric lengths).
 *  - Memory: every pointer except `jfa_problem*`, `status_out` and the
 *    argument of jfa_tile_config is a DEVICE pointer allocated by the caller,
 *    16-byte aligned.  The library never allocates or frees device memory and
 *    keeps no mutable state between calls, except opt-in kernel timing.
 *  - Streams: `stream` is a hipStream_t (NULL = default stream).  All work is
 *    enqueued asynchronously; nothing blocks the host except
 *    jfa_read_device_status and jfa_kernel_timing.
 *  - Limits: one sample's rows are addressed with 32-bit byte offsets, so
 *    (len + 256) * H * d * element_size (bf16 output size for MXFP8) must stay below 2^31
 *    for every sample, and with a dense bias (q_len + 256) * (kv_len + 256) * 4 too; a sample
 *    beyond these limits is reported like malformed offsets (JFA_ERR_DEVICE_DATA).
 *  - Errors: host-checkable mistakes return an error before anything is
 *    enqueued.  Malformed offsets found on the device set the status word in
 *    the workspace; the kernels of that call then write nothing, and
 *    jfa_read_device_status reports JFA_ERR_DEVICE_DATA.
 */
#ifndef JFA_H
#define JFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JFA_OK = 0,
  JFA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misaligned pointer, bad enum */
  JFA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (e.g. d not in {64,128}) */
  JFA_ERR_WORKSPACE = -3,     /* workspace_bytes smaller than jfa_workspace_bytes() */
  JFA_ERR_LAUNCH = -4,        /* a HIP call failed */
  JFA_ERR_DEVICE_DATA = -5    /* offsets found malformed on the device */
} jfa_status;

typedef enum { JFA_MODE_SOFTMAX = 0, JFA_MODE_SILU = 1, JFA_MODE_GELU = 2 } jfa_mode;
typedef enum { JFA_F32 = 0, JFA_BF16 = 1, JFA_MXFP8_E4M3 = 2 } jfa_dtype;
typedef enum { JFA_BIAS_NONE = 0, JFA_BIAS_RELPOS = 1, JFA_BIAS_DENSE = 2 } jfa_bias_kind;

typedef struct {
  int32_t batch;            /* B >= 1 samples */
  int32_t heads;            /* H >= 1 */
  int32_t head_dim;         /* d: 64 or 128 */
  int64_t total_q;          /* rows of Q / O (equals q_offsets[B]; checked on the device) */
  int64_t total_kv;         /* rows of K / V (equals kv_offsets[B]; checked on the device) */
  int32_t mode;             /* jfa_mode */
  int32_t dtype;            /* jfa_dtype: storage type of Q, K, V (and O, dO, dQ, dK, dV
                               for F32/BF16).  MXFP8: Q, K, V (and dO) are codes + scales;
                               O, dQ, dK, dV are bf16. */
  int32_t causal;           /* 0 or 1; visible iff j <= i + (kv_len - q_len) */
  float qk_scale;           /* > 0, or 0 to select 1/sqrt(d); negative is invalid */
  int32_t kv_len_normalize; /* -1 default (on for SiLU/GELU, off for softmax), 0, 1;
                               must be 0 or -1 for softmax */
  int32_t bias_kind;        /* jfa_bias_kind */
  int32_t num_buckets;      /* RELPOS table width, 1..4096 (64 for the GEM workloads) */
  int32_t split_slots;      /* forward tail balancing: 0 = auto (the compute units of the
                               device), >0 = this many, <0 = never split a query tile */
  int32_t bwd_fuse;         /* -1 default (on where built), 0 off: single-pass backward for
                               samples with one query tile (64-row query tiles) or one key
                               tile (d = 64) */
  int32_t window;           /* sliding window ("GEM Training: How Meta Doubled the Efficiency of
                               Its LLM-Scale Ads Foundation Model", "Challenge 1": long sequences
                               with a short attention window; "Meta Enhances GEM Training
                               Efficiency ...", "Leveraging Compute Efficiency through Customized
                               Kernels": attention over windows).  0 = none; W > 0 keeps key j
                               for query i only when |i + (kv_len - q_len) - j| < W, i.e. the W
                               keys ending at the query's aligned position under causal, a band
                               of 2W - 1 keys otherwise.  GDPA's weight stays 1/kv_len.  Tiles
                               visit only the key (query) steps their rows can see.  Negative is
                               invalid. */
} jfa_problem;

/*
 * Bias layouts:
 *  RELPOS: fp32 [H][num_buckets].  bias_h(b,i,j) = table[h][bucket(|i + (m-n) - j|)],
 *          bucket(x) = x for x < 16, else min(num_buckets-1, 16 + 4(k-4) + ((x >> (k-2)) & 3))
 *          with k = floor(log2 x).
 *  DENSE:  storage dtype (fp32 for F32, bf16 otherwise); sample b's block [H][n][m] starts
 *          at element H * sum_{b'<b} n_b' * m_b'.  bias_h(b,i,j) = block[h][i][j].
 */

/* Bytes of device workspace that jfa_forward (backward = 0), jfa_backward (backward = 1) or
 * jfa_backward_dbias (backward = 2) needs for this problem; 0 if the problem is invalid.  With
 * split_slots = 0 this queries the current device. */
size_t jfa_workspace_bytes(const jfa_problem* p, int backward);

/* Forward pass.  q/k/v: [rows, H, d] of the storage dtype; for MXFP8 they are E4M3 codes
 * (uint8) and q_scale/k_scale/v_scale are E8M0 codes [rows, H, d/32] (NULL otherwise).
 * bias: NULL for JFA_BIAS_NONE.  o: [total_q, H, d] (bf16 for MXFP8).  lse: fp32 [H, total_q],
 * required for softmax, ignored (may be NULL) for GDPA. */
jfa_status jfa_forward(const jfa_problem* p, const void* q, const void* k, const void* v,
                       const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                       const int32_t* q_offsets, const int32_t* kv_offsets, const void* bias,
                       void* o, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Backward pass (F32 and BF16; MXFP8 inputs go through jfa_backward_mxfp8, and this call
 * returns JFA_ERR_UNSUPPORTED for them).  o and lse are the forward's outputs (softmax; may be
 * NULL for GDPA); dout like o.  Writes every row of dq [total_q, H, d], dk and dv
 * [total_kv, H, d].  Deterministic: repeated calls give bitwise-identical results. */
jfa_status jfa_backward(const jfa_problem* p, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        const int32_t* q_offsets, const int32_t* kv_offsets, const void* bias,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Backward pass on MXFP8 inputs ("Meta Enhances GEM Training Efficiency with Advanced LLM-Scale
 * Innovations", section "Leveraging Compute Efficiency through Customized Kernels": MXFP8
 * attention in training; "Meta GEM Training Efficiency: ...", section "Bottleneck move 2":
 * selective higher precision where the gradient is sensitive).  p->dtype = JFA_MXFP8_E4M3.
 * q, k, v, dout: E4M3 codes [rows, H, d] (uint8) with E8M0 scales q_scale, k_scale, v_scale,
 * dout_scale [rows, H, d/32], as jfa_quantize_mxfp8 writes them (dout quantised by the caller
 * like the forward's inputs); o (bf16) and lse as jfa_forward returned them.  dq, dk, dv are
 * bf16.  The four inputs are read as codes and scales (1 + 1/32 bytes per element) and
 * dequantised exactly to bf16 on the way to LDS; all five products run on bf16 MFMA with fp32
 * accumulation, and P and dS stay bf16 (never requantised).  The result is the gradient of
 * <O, dO> at the dequantised inputs.  Deterministic; bias, window and the single-pass classes
 * as jfa_backward; workspace from jfa_workspace_bytes(p, 1).  NULL scales are
 * JFA_ERR_INVALID_ARG; another dtype in p is JFA_ERR_INVALID_ARG. */
jfa_status jfa_backward_mxfp8(const jfa_problem* p, const uint8_t* q, const uint8_t* k,
                              const uint8_t* v, const uint8_t* q_scale, const uint8_t* k_scale,
                              const uint8_t* v_scale, const void* o, const float* lse,
                              const uint8_t* dout, const uint8_t* dout_scale,
                              const int32_t* q_offsets, const int32_t* kv_offsets,
                              const void* bias, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Backward pass that also returns the gradient of the additive bias ("Meta GEM Training
 * Efficiency: ...", section "Bottleneck move 1": custom biases, which a model trains).  The bias
 * enters each visible score additively, so its gradient is that pair's dS = dL/dS.  BF16 only
 * and a bias is required (JFA_ERR_UNSUPPORTED otherwise); dbias must not be NULL.
 *   JFA_BIAS_DENSE: dbias has the bias's own layout and dtype (bf16), dS per pair, 0 on pairs
 *     that are not visible.
 *   JFA_BIAS_RELPOS: dbias is fp32 [H][num_buckets], the sum of dS over the visible pairs of
 *     each bucket, summed per query row and then over rows in a fixed order.
 * Everything else as jfa_backward (dq, dk, dv identical up to the single-pass classes, which
 * this call leaves off); workspace from jfa_workspace_bytes(p, 2).  Deterministic. */
jfa_status jfa_backward_dbias(const jfa_problem* p, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dout,
                              const int32_t* q_offsets, const int32_t* kv_offsets,
                              const void* bias, void* dq, void* dk, void* dv, void* dbias,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Tile sizes the kernels use for this problem, in the order
 * {bm, bn, slots, bq_bm, bq_bn, bk_bn, bk_bm, fuse}: forward query/key tile rows, split slots
 * (<= 0: no split), query-stationary backward tile rows, key-stationary backward tile rows,
 * and the single-pass backward classes that are on (bit 0: samples with one query tile, bit 1:
 * samples with one key tile).  Host only (queries the device only when
 * split_slots = 0). */
jfa_status jfa_tile_config(const jfa_problem* p, int32_t cfg_out[8]);

/* Test hook: builds the tile lists of this problem into caller buffers (device).
 * fwd, comb, bwd_q, bwd_kv: int32 [capacity][4]; fwd_slot: int32 [capacity];
 * counts: int32 [8] = {forward, combine, q-stationary, kv-stationary records, split threshold,
 * partial slots, status, 0}.  Records follow the order of jfa_tile_config's tiles:
 * forward {b, t, kv_step_begin, kv_step_end} longest first (ties: b, t, kv_step_begin); combine
 * {b, t, first_slot, chunks} in (b, t) order; q-stationary {b, t, 0, kv_steps};
 * kv-stationary {b, u, q_step_begin, q_step_end}. */
jfa_status jfa_build_schedule(const jfa_problem* p, const int32_t* q_offsets,
                              const int32_t* kv_offsets, int32_t* fwd, int32_t* fwd_slot,
                              int32_t* comb, int32_t* bwd_q, int32_t* bwd_kv, int32_t* counts,
                              int64_t capacity, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Offsets from lengths ("Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a
 * Different Stack", FAQ "What is a jagged tensor?": values plus offsets; section "Bottleneck
 * move 1": custom biases over asymmetric query/key-value lengths).
 *   offsets[0] = 0, offsets[b+1] = offsets[b] + lengths[b]   (device int32, B+1 and B entries)
 *   bias_offsets_or_null (device int64 [B+1], may be NULL): the dense-bias block offsets,
 *     bias_offsets[0] = 0, bias_offsets[b+1] = bias_offsets[b] + lengths[b] * kv_len[b], where
 *     kv_len = kv_lengths_or_null (device int32 [B]) or, when that is NULL, lengths itself
 *     (self-attention).  Sample b's dense-bias block [H][n][m] starts at element
 *     H * bias_offsets[b]; the attention calls derive the same offsets from q/kv offsets
 *     themselves, so this output is for callers that lay out or slice a dense bias.
 * status (device int32, may be NULL) receives 0, or JFA_ERR_DEVICE_DATA for a negative length
 * (either array) or a row total above INT32_MAX; then neither offsets array is written.
 * Host errors: NULL lengths/offsets, batch < 0, misaligned pointers -> JFA_ERR_INVALID_ARG. */
jfa_status jfa_lengths_to_offsets(const int32_t* lengths, int32_t batch, int32_t* offsets,
                                  int64_t* bias_offsets_or_null,
                                  const int32_t* kv_lengths_or_null, int32_t* status,
                                  void* stream);

/* BlockAttention ("Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a Different
 * Stack", section "Bottleneck move 1": eligible long-sequence attention becomes independent
 * fixed-size blocks; "Meta Enhances GEM Training Efficiency with Advanced LLM-Scale
 * Innovations", section "Exploring the Customized Kernel Library": windows in place of full
 * attention).  Splits every sample of `offsets` (device int32 [batch+1], as for the attention
 * calls) into ceil(len / block) consecutive blocks of `block` rows, the last one shorter, and
 * writes them as the samples of a refined batch: block_offsets (device int32 [out_batch+1])
 * receives the block starts in sample order, then the total row count in every remaining
 * entry (empty samples).  out_batch = batch + total_rows / block always suffices.  Running
 * jfa_forward / jfa_backward with batch = out_batch and block_offsets as both q and kv offsets
 * is BlockAttention of a self-attention batch: every query attends to the keys of its own
 * block (causal within the block when causal = 1; relative positions are block-local, equal
 * to the sample-local distance; GDPA's 1/kv_len is 1/block length; a dense bias is laid out
 * over the refined samples).  status (device int32, may be NULL) receives 0, or
 * JFA_ERR_DEVICE_DATA for malformed offsets or more blocks than out_batch, in which case
 * block_offsets is left untouched.  block < 1 or out_batch < 0 is JFA_ERR_INVALID_ARG. */
jfa_status jfa_block_offsets(const int32_t* offsets, int32_t batch, int32_t block,
                             int32_t* block_offsets, int32_t out_batch, int32_t* status,
                             void* stream);

/* MXFP8 (OCP Microscaling, E4M3 elements): for each row of x (bf16 [rows, d], d % 32 == 0)
 * and each block of 32 consecutive elements, scale code s = floor(log2 amax) - 8 + 127
 * (clamped to [0, 254]; 127 for an all-zero block) into scales [rows, d/32], and codes
 * [rows, d] = E4M3 round-to-nearest-even of x * 2^(127 - s), saturating at +-448. */
jfa_status jfa_quantize_mxfp8(const void* x_bf16, int64_t rows, int32_t d, uint8_t* codes,
                              uint8_t* scales, void* stream);

/* jfa_quantize_mxfp8 on 1 to 4 tensors in one launch (Q, K, V and dO of an MXFP8 step):
 * "Meta GEM Training Efficiency: ...", section "Bottleneck move 2" (scale generation and
 * casting must not eat the low-precision gain).  xs_bf16[t] (bf16 [rows[t], d]), codes[t] and
 * scales[t] are device pointers as for jfa_quantize_mxfp8; the arrays themselves are HOST
 * arrays of `count` entries.  Results are bit-identical to one jfa_quantize_mxfp8 call per
 * tensor.  count outside [1, 4], d % 32 != 0, a negative row count, NULL or misaligned pointers
 * (x 16 B, codes 8 B) of a tensor with rows are JFA_ERR_INVALID_ARG. */
jfa_status jfa_quantize_mxfp8_batch(int32_t count, const void* const* xs_bf16,
                                    const int64_t* rows, int32_t d, uint8_t* const* codes,
                                    uint8_t* const* scales, void* stream);

/* RMS normalisation fused with the MXFP8 quantiser, producing MXFP8 attention inputs in one pass
 * over memory ("Meta GEM Training Efficiency: ...", section "Bottleneck move 2": quantisation
 * fused into the preceding normalisation, so that scale generation and casting cost no extra
 * pass).  x: bf16 [groups, n] (device), n in {32, 64, 128, 256, 512}: a head's d values
 * (groups = rows * H) or a token's H * d.  weight: fp32 [n] per-channel gain, or NULL for 1.
 * Each group becomes y = x / sqrt(mean(x^2) + eps) * weight (fp32), and y is quantised exactly
 * as jfa_quantize_mxfp8 does: codes [groups, n], scales [groups, n / 32].  eps >= 0.  Other
 * sizes, a negative count, NULL or misaligned pointers (x 16 B, codes 8 B, weight 16 B) are
 * JFA_ERR_INVALID_ARG. */
jfa_status jfa_rmsnorm_quantize_mxfp8(const void* x_bf16, const float* weight, int64_t groups,
                                      int32_t n, float eps, uint8_t* codes, uint8_t* scales,
                                      void* stream);

/* Size of the fixed device array that jfa_forward_noalloc uses as its workspace (64 MiB per
 * GPU, held from the library's first use of that GPU until the process ends). */
#define JFA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* jfa_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, kernels and results
 * as jfa_forward (bit for bit), without the workspace: the library's fixed per-GPU array of
 * JFA_NOALLOC_SCRATCH_BYTES serves instead.  Nothing is allocated or freed.  Problems whose
 * workspace (jfa_workspace_bytes(p, 0)) exceeds that size return JFA_ERR_WORKSPACE before
 * anything is enqueued; other errors as jfa_forward.  Every call on a GPU shares that GPU's
 * array and rewrites what it reads from it, so calls ordered on one stream are independent,
 * while calls that overlap on one GPU (several streams or threads at once) race.  The device
 * status of the last call is in the array and is not readable through
 * jfa_read_device_status; malformed offsets still make the kernels write nothing. */
jfa_status jfa_forward_noalloc(const jfa_problem* p, const void* q, const void* k,
                               const void* v, const uint8_t* q_scale, const uint8_t* k_scale,
                               const uint8_t* v_scale, const int32_t* q_offsets,
                               const int32_t* kv_offsets, const void* bias, void* o,
                               float* lse, void* stream);

/* Waits for `stream` and returns the device status word of the last call that used this
 * workspace (JFA_OK or JFA_ERR_DEVICE_DATA) in *status_out. */
jfa_status jfa_read_device_status(const void* workspace, void* stream, int32_t* status_out);

/* Human-readable name of a status code (static storage). */
const char* jfa_status_string(jfa_status s);

/* Opt-in per-kernel timing (for benchmarks): while enabled, every kernel launch is bracketed
 * by HIP events on its stream.  jfa_kernel_timing waits for those events and returns the
 * summed milliseconds and launch count of kernels whose name starts with `name_prefix`
 * ("" = all); reset clears the record.  Not for concurrent use from several threads. */
void jfa_set_kernel_timing(int enable);
jfa_status jfa_kernel_timing(const char* name_prefix, double* total_ms, int64_t* launches);
void jfa_kernel_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* JFA_H */
