/*
 * smoe.h -- C ABI of the MI355X (gfx950) SMOE routed-expert MoE FFN library.
 *
 * The library computes one MoE feed-forward layer whose routed experts are
 * stored as SMOE-Q4 or SMOE-Q2 group-64 symmetric-quantised weights in the
 * .smoe expert-blob layout, and (optionally) a stack of such layers with an
 * RMSNorm + residual around each.
 *
 * Sources the operations follow (page title, section):
 *  - ".smoe Binary Format", "Expert Blob Architecture": one blob per expert,
 *    [gate codes][gate scales][up codes][up scales][down codes][down scales]
 *    then zero padding to a 16,384-byte boundary; codes take
 *    ceil(rows*cols*bits/8) bytes, scales one value per 64 weights of the
 *    flattened [rows, cols] tensor; "Tensor Descriptor": gate and up are
 *    [ffn_dim, d_model], down is [d_model, ffn_dim] (the weights' original
 *    [out, in] shapes); "Immutable Encoding": little-endian.
 *  - "SMOE Quantisation", "Quantisation Levels", "Bit Packing", "Decoding:
 *    Metal Kernel": codes packed least-significant-bits first (2 per byte for
 *    Q4, 4 per byte for Q2); weight = (code - m) / m * scale with m = 7.5
 *    (Q4) or 1.5 (Q2).
 *  - "CMF v2 Format Specification", section 2.2 "MoE": softmax over all router
 *    logits, top-k with ties broken toward the lower expert index, optional
 *    renormalisation of the k selected probabilities, weighted sum of the
 *    selected experts' SwiGLU outputs, and an always-on shared expert added
 *    with weight 1.
 *  - "Model Agnosticism", "Expanding the Frontier": SiLU/SwiGLU experts only,
 *    at most 16 routed experts per token.
 *  - ".smoe Binary Format", "Arch Block": RMS-norm epsilon 1e-6.
 *
 * Conventions for every entry point:
 *  - Pointers named d_* are device pointers (HIP device memory on the current
 *    device). The caller allocates, owns and frees all of them; the library
 *    only borrows them for the duration of the call (or, for the blob bank
 *    given to smoe_load_blobs, until smoe_free).
 *  - hip_stream is a hipStream_t (NULL = the legacy default stream). All GPU
 *    work of a call is ordered on it; calls return without synchronising.
 *    A layer with a shared expert runs that expert on a stream of its own
 *    (default priority, created with two events by the layer's first
 *    forward on the current device, released by smoe_free), forked from
 *    hip_stream at the start of the call and joined back into it before the
 *    combine, so the call's work still completes in hip_stream's order (and
 *    is captured with it into a graph). Capture the first forward of such a
 *    layer only after one eager forward (stream creation is not capturable).
 *  - Return value: SMOE_OK (0) or a negative SMOE_E_* code. On failure a
 *    message is available from smoe_last_error() (thread-local, valid until
 *    the next call on the same thread). Argument checks happen on the host
 *    before anything is enqueued, so a failed call enqueues no GPU work
 *    unless it returns SMOE_E_HIP. No C++ exception crosses this ABI.
 *  - Device faults caused by pointers that do not satisfy the stated sizes
 *    cannot be detected by the library; they surface on the caller's next
 *    synchronisation.
 */
#ifndef SMOE_H_
#define SMOE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMOE_ABI_VERSION 1

/* Status codes. */
#define SMOE_OK 0
#define SMOE_E_ARG (-1)         /* null pointer, value out of range, bad flag     */
#define SMOE_E_LAYOUT (-2)      /* blob bank too small, misaligned, bad stride    */
#define SMOE_E_UNSUPPORTED (-3) /* valid for the format, not built in this library */
#define SMOE_E_HIP (-4)         /* a HIP runtime call failed (launch, attributes) */
#define SMOE_E_WORKSPACE (-5)   /* workspace null or smaller than required        */

/* Activation dtypes. */
#define SMOE_DTYPE_F32 0
#define SMOE_DTYPE_BF16 1

/* Scale storage dtypes. The .smoe files store fp16 scales; fp32 is accepted
 * as well (same layout, 4-byte scales). */
#define SMOE_SCALE_F32 0
#define SMOE_SCALE_F16 1

/* Limits of this build. */
#define SMOE_GROUP_SIZE 64       /* the only quantisation group size          */
#define SMOE_BLOB_ALIGN 16384    /* blob stride granularity                   */
#define SMOE_MAX_TOP_K 16        /* routing width cap                         */
#define SMOE_MAX_EXPERTS 512     /* routed experts per layer                  */
#define SMOE_MAX_TOKENS 4096     /* tokens per smoe_moe_forward call          */
/* Required alignment of the expert bank and shared-blob base pointers: the
 * 16 KB page boundary every .smoe blob starts on (".smoe Binary Format",
 * Immutable Encoding; "Model Agnosticism", Dynamic Buffer Allocation). */
#define SMOE_BANK_ALIGN 16384

/* Description of one MoE layer's expert bank. */
typedef struct smoe_layer_desc {
  uint32_t d_model;        /* hidden size; multiple of 64                       */
  uint32_t ffn_dim;        /* routed expert intermediate size; multiple of 64  */
  uint32_t num_experts;    /* routed experts E, 1..SMOE_MAX_EXPERTS            */
  uint32_t bits;           /* 4 (SMOE-Q4) or 2 (SMOE-Q2)                       */
  uint32_t group_size;     /* must be 64                                        */
  uint32_t scale_dtype;    /* SMOE_SCALE_F32 or SMOE_SCALE_F16                  */
  uint64_t blob_stride;    /* bytes from expert e's blob to e+1's; a multiple
                              of 16,384 and >= the raw blob size               */
  uint32_t shared_ffn_dim; /* 0 = no shared expert, else its ffn (multiple of 64) */
  uint32_t reserved;       /* must be 0                                         */
} smoe_layer_desc;

/* Byte layout of one tensor inside an expert blob. */
typedef struct smoe_tensor_layout {
  uint64_t codes_offset;   /* from the start of the blob */
  uint64_t codes_bytes;    /* ceil(rows*cols*bits/8)     */
  uint64_t scales_offset;
  uint64_t scales_bytes;   /* ceil(rows*cols/64) * scale size */
  uint32_t rows, cols;
} smoe_tensor_layout;

/* Byte layout of one expert blob. */
typedef struct smoe_expert_layout {
  smoe_tensor_layout gate, up, down;
  uint64_t raw_size;       /* end of the down scales                   */
  uint64_t padded_size;    /* raw_size rounded up to 16,384 bytes      */
} smoe_expert_layout;

/* Opaque handle: host-side metadata of a layer. Holds no device memory. */
typedef struct smoe_layer smoe_layer;

/* Library version (SMOE_ABI_VERSION). */
int smoe_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char* smoe_last_error(void);

/* Host-only: byte layout of one expert blob of the given shape
 * (".smoe Binary Format", Expert Blob Architecture). Fills *out.
 * Errors: SMOE_E_ARG for a null out, bits not in {2,4}, a zero or
 * non-multiple-of-64 dimension, or an unknown scale dtype. */
int smoe_expert_layout_of(uint32_t d_model, uint32_t ffn_dim, uint32_t bits,
                          uint32_t scale_dtype, smoe_expert_layout* out);

/* Register a resident expert bank (and optional shared-expert blob).
 *  desc          layer description (copied).
 *  d_blobs       device pointer to E blobs, expert e at d_blobs + e*blob_stride;
 *                SMOE_BANK_ALIGN-aligned. Borrowed until smoe_free.
 *  nbytes        size of the bank; must be >= (E-1)*blob_stride + raw_size.
 *  d_shared_blob device pointer to one blob of shape (d_model, shared_ffn_dim)
 *                in the same layout, SMOE_BANK_ALIGN-aligned, or NULL when
 *                shared_ffn_dim == 0.
 *  shared_nbytes its size (>= its raw size).
 *  out           receives the handle (NULL on failure).
 * No GPU work, no device allocation. Errors: SMOE_E_ARG (bad desc fields or
 * null pointers), SMOE_E_LAYOUT (stride, size or alignment), SMOE_E_UNSUPPORTED
 * (a tensor width this build has no kernel for, or an activation vector too
 * long for the batched stages' 64 KB LDS staging: d_model above 11392 with
 * fp32 hi/lo staging, or ffn_dim above 19072 for any shared or routed
 * expert). */
int smoe_load_blobs(const smoe_layer_desc* desc, const void* d_blobs, uint64_t nbytes,
                    const void* d_shared_blob, uint64_t shared_nbytes, smoe_layer** out);

/* Release a handle (NULL is allowed). Does not touch the borrowed memory. */
void smoe_free(smoe_layer* layer);

/* Bytes of device workspace smoe_moe_forward needs for n_tokens tokens and
 * top_k (0 on invalid arguments or a batch the grouping cannot hold). smoe_decode_step needs the same amount for
 * the largest layer it runs. Calls that share a workspace must be ordered
 * (one stream, or synchronised). */
uint64_t smoe_workspace_bytes(const smoe_layer* layer, int n_tokens, int top_k);

/* Routing only ("CMF v2 Format Specification", 2.2):
 *  d_logits  [n_tokens, n_experts] fp32, row-major.
 *  d_ids     [n_tokens, top_k] int32 out: expert ids by descending logit,
 *            equal logits in ascending id.
 *  d_weights [n_tokens, top_k] fp32 out: softmax-over-all probability of each
 *            selected expert, renormalised to sum 1 when norm_topk_prob != 0.
 * Errors: SMOE_E_ARG (nulls, n_tokens < 0 or > SMOE_MAX_TOKENS, n_experts
 * outside 1..SMOE_MAX_EXPERTS, top_k outside 1..min(16, n_experts)),
 * SMOE_E_HIP. n_tokens == 0 is a no-op. Non-finite logits give unspecified
 * (but in-bounds) ids. */
int smoe_route(const float* d_logits, int n_tokens, int n_experts, int top_k,
               int norm_topk_prob, int32_t* d_ids, float* d_weights, void* hip_stream);

/* Routing variants ("CMF v2 Format Specification", 2.2 MoE; 5. Masks
 * section). smoe_route_opts_init() sets the defaults (plain softmax routing,
 * no bias, factor 1, every expert routable, shared expert weight 1).
 *  sigmoid           0: softmax over the routable experts' logits; 1: each
 *                    expert scored by sigmoid(logit) on its own.
 *  scaling_factor    routed_scaling_factor: multiplies the routed weights
 *                    after the optional renormalisation; finite.
 *  d_expert_bias     device [num_experts] fp32, nullable: added to the
 *                    scores for the top-k selection only (the weights stay
 *                    the unbiased scores). With a bias the selection
 *                    compares float64 score + bias (the score recomputed in
 *                    float64 from the fp32 logits, the bias taken exactly),
 *                    equal keys to the lower id; without one it compares
 *                    the logits (the same order).
 *  d_shared_gate     device [n_tokens] fp32, nullable: per-token logits of
 *                    the shared-expert gate; the shared expert's output is
 *                    weighted by sigmoid(logit) instead of 1.
 *  use_mask, expert_mask
 *                    host bitfield of routable experts, bit e of word e / 32
 *                    (LSB-first, the masks section's byte order read as
 *                    little-endian words): selection runs over set bits
 *                    only and the softmax is taken over them only. Bits at
 *                    or past num_experts must be 0 and at least top_k bits
 *                    must be set (SMOE_E_ARG otherwise). Copied at the call.
 * Variant routing always takes the grouped (batch) kernels, also for one
 * token. */
typedef struct smoe_route_opts {
  int32_t sigmoid;
  float scaling_factor;
  const float* d_expert_bias;
  const float* d_shared_gate;
  int32_t use_mask;
  uint32_t expert_mask[SMOE_MAX_EXPERTS / 32];
} smoe_route_opts;

void smoe_route_opts_init(smoe_route_opts* opts);

/* smoe_route with routing variants (opts nullable = defaults). Errors as
 * smoe_route, plus SMOE_E_ARG for an invalid mask or a non-finite factor. */
int smoe_route_ex(const float* d_logits, int n_tokens, int n_experts, int top_k,
                  int norm_topk_prob, const smoe_route_opts* opts, int32_t* d_ids,
                  float* d_weights, void* hip_stream);

/* One MoE layer forward:
 *   out[t] = sum_j w[t,j] * down_e(silu(gate_e x[t]) * up_e x[t])   (e = ids[t,j])
 *            + shared(x[t])                                         (if present)
 *  d_x        [n_tokens, d_model], dtype x_dtype (SMOE_DTYPE_BF16 or _F32),
 *             16-byte aligned, row-major.
 *  d_logits   [n_tokens, num_experts] fp32 router logits.
 *  d_out      [n_tokens, d_model] fp32 out (overwritten).
 *  d_topk_ids, d_topk_w  optional [n_tokens, top_k] copies of the routing
 *             result (NULL to skip).
 *  d_workspace at least smoe_workspace_bytes(layer, n_tokens, top_k) bytes,
 *             256-byte aligned; contents are scratch and need no clearing.
 * Tokens that share an expert read its weights once per call.
 * Errors: SMOE_E_ARG, SMOE_E_WORKSPACE, SMOE_E_UNSUPPORTED (the grouping's
 * per-expert token bitmasks and counts, (num_experts * ((w | 1) +
 * (ceil(w / 8) | 1) + 3) + 1) * 4 bytes with w = ceil(n_tokens / 32), exceed
 * 160 KB: e.g. more than 2144 tokens with 512 experts), SMOE_E_HIP.
 * n_tokens == 0 is a no-op.
 * Activations must be finite with |x| < 2^100 (they are rescaled by a power
 * of two per vector before the fp16 dot products). */
int smoe_moe_forward(const smoe_layer* layer, const void* d_x, int x_dtype,
                     const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                     float* d_out, int32_t* d_topk_ids, float* d_topk_w,
                     void* d_workspace, uint64_t ws_bytes, void* hip_stream);

/* smoe_moe_forward with routing variants (opts nullable = defaults); d_out
 * gets sum_j w_j FFN_j(x) + sigmoid(shared_gate) * FFN_shared(x), d_topk_w the
 * final weights (renormalised and scaled). Errors as smoe_moe_forward and
 * smoe_route_ex. */
int smoe_moe_forward_ex(const smoe_layer* layer, const void* d_x, int x_dtype,
                        const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                        const smoe_route_opts* opts, float* d_out, int32_t* d_topk_ids,
                        float* d_topk_w, void* d_workspace, uint64_t ws_bytes,
                        void* hip_stream);

/* Device bytes of the static scratch behind smoe_moe_forward_noalloc, per
 * GPU. */
#define SMOE_NOALLOC_SCRATCH_BYTES (32ull << 20)

/* smoe_moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation and results, with two differences: the workspace is a
 * static array of SMOE_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends, and the shared expert runs on
 * hip_stream itself, before routing (no side stream or events).
 *  Arguments as smoe_moe_forward without d_workspace and ws_bytes;
 *  hip_stream (NULL: the null stream) belongs to the current device.
 * Calls no hipMalloc, hipFree or other allocating routine; the first call on
 * a device looks up that device's copy of the array (hipGetSymbolAddress).
 * Every call on one GPU uses that GPU's one array, which keeps the previous
 * call's contents (each call writes every word it reads, so nothing needs
 * clearing): calls that overlap on one GPU (several streams, or threads
 * without ordering between them) race and give wrong results.
 * Errors: those of smoe_moe_forward, SMOE_E_WORKSPACE when
 * smoe_workspace_bytes(layer, n_tokens, top_k) exceeds
 * SMOE_NOALLOC_SCRATCH_BYTES (e.g. past 186 tokens at top-8 for experts of
 * (4096, 1536), past 279 at top-6 for (2048, 1408) with a (2048, 2816) shared
 * expert), SMOE_E_HIP. n_tokens == 0 is a no-op. */
int smoe_moe_forward_noalloc(const smoe_layer* layer, const void* d_x, int x_dtype,
                             const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                             float* d_out, int32_t* d_topk_ids, float* d_topk_w,
                             void* hip_stream);

/* Stacked decode step over n_layers MoE layers (same d_model):
 *   for l in 0..n_layers-1:  h = h + MoE_l(rms_norm(h, eps))
 * with unit-gain RMSNorm n = h / sqrt(mean(h^2) + eps) per token.
 *  layers     array of n_layers handles.
 *  d_h        [n_tokens, d_model] fp32, updated in place (the residual stream).
 *  d_logits   [n_layers, n_tokens, num_experts] fp32, one routing per layer.
 *  eps        RMSNorm epsilon (the pages' kernels use 1e-6).
 *  d_workspace, ws_bytes  as for smoe_moe_forward, sized for the largest layer.
 * Errors as smoe_moe_forward, plus SMOE_E_ARG for n_layers < 1, mismatched
 * d_model, or eps <= 0. */
int smoe_decode_step(const smoe_layer* const* layers, int n_layers, float* d_h,
                     const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                     float eps, void* d_workspace, uint64_t ws_bytes, void* hip_stream);

/* Quantiser ("SMOE Quantisation", L2-MSE Scale Optimiser; Quantisation
 * Levels; Bit Packing): codes and group-64 scales of n_elements fp32 weights
 * taken in their flattened order (for a [rows, cols] tensor, row-major), the
 * same bytes a .smoe blob holds for that tensor.
 * For every group of 64 consecutive weights (the last group may be shorter):
 * absmax = max |w|; the 64 candidates frac_i * absmax, frac = the 64-point
 * linspace from 0.1 to 1.0 in double, are each rounded once to the scale
 * dtype; each candidate s encodes the group as
 * clamp(rint(w / s * m + m), 0, 2^bits - 1) (w / s read as 0 for s == 0) and
 * decodes it as (code - m) / m * s; its squared error is summed in double in
 * element order, every operation rounded on its own; the first minimum wins.
 *  d_w        device [n_elements] fp32, 4-byte aligned.
 *  d_codes    device out, ceil(n_elements * bits / 8) bytes, codes packed
 *             LSB-first (2 per byte for Q4, 4 for Q2); the unused high bits
 *             of a partial last byte are 0.
 *  d_scales   device out, ceil(n_elements / 64) values of scale_dtype
 *             (SMOE_SCALE_F32 or SMOE_SCALE_F16), element-aligned.
 *  n_elements at most SMOE_MAX_QUANT_ELEMENTS; a larger tensor is quantised
 *             in pieces split at multiples of 64 elements (codes advance by
 *             n * bits / 8 bytes, scales by n / 64 values per piece).
 * The outputs must not overlap the input. Deterministic: the result depends
 * on the weights only. Non-finite weights give unspecified codes and scales.
 * Errors: SMOE_E_ARG (bits not in {2, 4}, unknown scale dtype, n_elements too
 * large, null or misaligned pointers), SMOE_E_HIP. n_elements == 0 is a
 * no-op. */
#define SMOE_MAX_QUANT_ELEMENTS (1ull << 31)
int smoe_quantise(const float* d_w, uint64_t n_elements, int bits, int scale_dtype,
                  uint8_t* d_codes, void* d_scales, void* hip_stream);

/* Kernel timing hook (instrumentation for benchmarks; not an operation of
 * the pages). Arms a one-shot pair of HIP events: the next smoe_moe_forward
 * or smoe_decode_step call that launches the chosen kernel attaches them to
 * that launch as its start and stop events (hipExtLaunchKernel), so their
 * elapsed time is the kernel's own execution, then disarms.
 *  kernel  SMOE_KERNEL_GATE_UP: the routed experts' gate/up + SwiGLU launch
 *          (on the one-token path this launch also routes);
 *          SMOE_KERNEL_DOWN: the routed experts' down-projection launch (on
 *          the one-token path it also combines);
 *          SMOE_KERNEL_NONE: disarm.
 *  hip_event_before, hip_event_after  hipEvent_t values created and owned by
 *          the caller (timing enabled); read them with hipEventElapsedTime
 *          after synchronising.
 * The armed pair is process-wide, not per thread or stream.
 * Returns SMOE_OK when arming; when disarming, 1 if a pair was still armed
 * (no such launch happened since) and 0 otherwise.
 * Errors: SMOE_E_ARG for an unknown kernel or a null event when arming. */
#define SMOE_KERNEL_NONE 0
#define SMOE_KERNEL_GATE_UP 1
#define SMOE_KERNEL_DOWN 2
int smoe_trace_kernel(int kernel, void* hip_event_before, void* hip_event_after);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_H_ */
