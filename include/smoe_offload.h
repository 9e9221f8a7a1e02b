/*
 * smoe_offload.h -- host-offload streaming of a layer's routed experts (C ABI,
 * in libsmoe.so).
 *
 * Source (page title, section): "SMOE Quantisation", Why Quantise (the
 * experts of a large MoE model do not fit in memory, so the runtime streams
 * the selected experts' blobs per token, and the blob size sets the rate);
 * ".smoe Binary Format" (the Streamer is the reader that moves blobs from
 * storage into memory); "CMF v2 Format Specification", 2.2 MoE (per token
 * only the selected k experts are touched).
 *
 * On this GPU the experts live in pinned host memory and reach the device
 * over PCIe in one of two ways:
 *  - direct (no cache): the expert kernels read the selected experts' bytes
 *    from host memory themselves, through a per-expert address table; the
 *    call is as asynchronous as smoe_moe_forward.
 *  - cached (a device cache of n slots): the call routes on the GPU, waits
 *    for the ids, copies every selected expert that is not resident into a
 *    cache slot (least recently used first, never a slot this call uses;
 *    when a call selects more distinct experts than there are slots, the
 *    rest are read directly), points the table at the slots and enqueues the
 *    forward. Copies and forward run on hip_stream; the call returns after
 *    enqueuing them.
 * The results are those of smoe_moe_forward on the same blobs in device
 * memory, bit for bit (the same kernels read the same bytes).
 *
 * Conventions of smoe.h apply. Calls on one handle must be ordered (one
 * stream, or synchronised): the cache and the table are shared state.
 */
#ifndef SMOE_OFFLOAD_H_
#define SMOE_OFFLOAD_H_

#include <stdint.h>

#include "smoe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct smoe_offload smoe_offload;

/* Counters since creation. */
typedef struct smoe_offload_stats {
  uint64_t forwards;       /* calls that ran a forward (n_tokens > 0)           */
  uint64_t hits;           /* selected experts found in the cache               */
  uint64_t fetched;        /* selected experts copied into the cache            */
  uint64_t direct;         /* selected experts read from host memory directly
                              (cached mode; in direct mode every expert is, and
                              only forwards are counted)                        */
  uint64_t bytes_fetched;  /* bytes copied host -> device (raw blob bytes)      */
} smoe_offload_stats;

/* Register a host-resident layer.
 *  desc          as for smoe_load_blobs (blob_stride is the host bank's).
 *  h_blobs       pinned host memory (hipHostMalloc, or torch's pin_memory),
 *                expert e at h_blobs + e * blob_stride, SMOE_BANK_ALIGN
 *                aligned; nbytes as for smoe_load_blobs. Borrowed until
 *                smoe_offload_free. Memory that is not pinned host memory is
 *                refused (SMOE_E_LAYOUT).
 *  d_shared_blob device-resident shared expert (or NULL), as for
 *                smoe_load_blobs.
 *  d_cache       device memory for cache_bytes / blob_stride slots (NULL or
 *                0 bytes: direct mode); SMOE_BANK_ALIGN aligned.
 *  d_table       device memory for num_experts uint64 blob addresses, 8-byte
 *                aligned; written by the library (one synchronous copy here,
 *                then on the call's stream).
 * Allocates two small pinned host buffers of its own (the table image and
 * the routed ids). Errors: those of smoe_load_blobs, SMOE_E_ARG (null table,
 * misaligned cache or table), SMOE_E_LAYOUT (host bank not pinned),
 * SMOE_E_HIP. */
int smoe_offload_create(const smoe_layer_desc* desc, const void* h_blobs, uint64_t nbytes,
                        const void* d_shared_blob, uint64_t shared_nbytes, void* d_cache,
                        uint64_t cache_bytes, void* d_table, smoe_offload** out);

/* Release the handle (NULL is a no-op); waits for nothing. */
void smoe_offload_free(smoe_offload* off);

/* One layer forward with the experts in host memory. Arguments, results and
 * errors as smoe_moe_forward; workspace size smoe_offload_workspace_bytes.
 * In cached mode the call synchronises hip_stream once (after routing). */
int smoe_offload_forward(smoe_offload* off, const void* d_x, int x_dtype, const float* d_logits,
                         int n_tokens, int top_k, int norm_topk_prob, float* d_out,
                         int32_t* d_topk_ids, float* d_topk_w, void* d_workspace,
                         uint64_t ws_bytes, void* hip_stream);

/* Workspace bytes of smoe_offload_forward (0 on invalid arguments). */
uint64_t smoe_offload_workspace_bytes(const smoe_offload* off, int n_tokens, int top_k);

/* Cache slots (0 in direct mode). */
uint32_t smoe_offload_slots(const smoe_offload* off);

/* Copy of the counters. Errors: SMOE_E_ARG for a null handle or output. */
int smoe_offload_get_stats(const smoe_offload* off, smoe_offload_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_OFFLOAD_H_ */
