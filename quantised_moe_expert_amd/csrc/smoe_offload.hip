// Host-offload streaming of a layer's routed experts (include/smoe_offload.h).
//
// The layer is registered like a device bank, but with the device-visible
// address of a pinned host bank and an expert-pointer table: the expert
// kernels read expert e at table[e]. In direct mode every entry points into
// host memory. In cached mode a call first routes on the GPU, reads the ids
// back, brings the selected experts that are not resident into device
// cache slots with DMA copies on the call's stream, rewrites the table for
// them, and then runs the unchanged forward.

#include <hip/hip_runtime.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/smoe_offload.h"
#include "smoe_internal.hpp"

using smoe::report_error;
using smoe::report_ok;

struct smoe_offload {
  smoe_layer* layer = nullptr;   // registered with the host bank's device address
  const uint8_t* host = nullptr; // device-visible address of the host bank
  uint64_t stride = 0, raw = 0;
  uint32_t E = 0;
  uint8_t* cache = nullptr;
  uint32_t n_slots = 0;
  uint64_t* d_table = nullptr;
  uint64_t* h_table = nullptr;   // pinned image of the table
  int32_t* h_ids = nullptr;      // pinned routed ids of a call
  std::vector<int32_t> slot_expert;  // expert held by each slot, -1 free
  std::vector<int32_t> expert_slot;  // slot of each expert, -1 not resident
  std::vector<uint64_t> slot_tick;   // call that last used the slot
  std::vector<uint64_t> seen;        // call that last selected the expert
  uint64_t tick = 0;
  smoe_offload_stats st{};

  ~smoe_offload() {
    if (h_table) (void)hipHostFree(h_table);
    if (h_ids) (void)hipHostFree(h_ids);
    smoe_free(layer);
  }
};

namespace {

int hip_fail(hipError_t e, const char* what) {
  return report_error(SMOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned_to(const void* p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

int smoe_offload_create(const smoe_layer_desc* desc, const void* h_blobs, uint64_t nbytes,
                        const void* d_shared_blob, uint64_t shared_nbytes, void* d_cache,
                        uint64_t cache_bytes, void* d_table, smoe_offload** out) {
  if (!out) return report_error(SMOE_E_ARG, "null output handle pointer");
  *out = nullptr;
  if (!desc || !h_blobs) return report_error(SMOE_E_ARG, "null description or host bank");
  if (!d_table || !aligned_to(d_table, 8))
    return report_error(SMOE_E_ARG, "the expert table must be non-null and 8-byte aligned");
  if (d_cache && !aligned_to(d_cache, SMOE_BANK_ALIGN))
    return report_error(SMOE_E_ARG, "the cache must be %d-byte aligned", SMOE_BANK_ALIGN);
  // the host bank must be pinned host memory the device can address
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, h_blobs);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return report_error(SMOE_E_LAYOUT, "the host bank is not pinned host memory");
  }
  void* dev = nullptr;
  e = hipHostGetDevicePointer(&dev, const_cast<void*>(h_blobs), 0);
  if (e != hipSuccess) return hip_fail(e, "device address of the host bank");
  smoe_offload* o = new (std::nothrow) smoe_offload;
  if (!o) return report_error(SMOE_E_ARG, "out of host memory");
  int rc = smoe_load_blobs(desc, dev, nbytes, d_shared_blob, shared_nbytes, &o->layer);
  if (rc) {
    delete o;
    return rc;
  }
  smoe_expert_layout L;
  smoe_expert_layout_of(desc->d_model, desc->ffn_dim, desc->bits, desc->scale_dtype, &L);
  o->host = (const uint8_t*)dev;
  o->stride = desc->blob_stride;
  o->raw = L.raw_size;
  o->E = desc->num_experts;
  o->cache = d_cache ? (uint8_t*)d_cache : nullptr;
  o->n_slots = d_cache ? (uint32_t)(cache_bytes / o->stride) : 0;
  if (o->n_slots > o->E) o->n_slots = o->E;
  o->d_table = (uint64_t*)d_table;
  o->layer->info.table = o->d_table;
  e = hipHostMalloc((void**)&o->h_table, sizeof(uint64_t) * o->E, hipHostMallocDefault);
  if (e == hipSuccess)
    e = hipHostMalloc((void**)&o->h_ids, sizeof(int32_t) * SMOE_MAX_TOKENS * SMOE_MAX_TOP_K,
                      hipHostMallocDefault);
  if (e != hipSuccess) {
    delete o;
    return hip_fail(e, "pinned host buffers");
  }
  try {
    o->slot_expert.assign(o->n_slots, -1);
    o->slot_tick.assign(o->n_slots, 0);
    o->expert_slot.assign(o->E, -1);
    o->seen.assign(o->E, 0);
  } catch (const std::bad_alloc&) {
    delete o;
    return report_error(SMOE_E_ARG, "out of host memory");
  }
  for (uint32_t x = 0; x < o->E; ++x) o->h_table[x] = (uint64_t)(uintptr_t)(o->host + x * o->stride);
  e = hipMemcpy(o->d_table, o->h_table, sizeof(uint64_t) * o->E, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    delete o;
    return hip_fail(e, "expert table upload");
  }
  *out = o;
  return report_ok();
}

void smoe_offload_free(smoe_offload* off) { delete off; }

uint64_t smoe_offload_workspace_bytes(const smoe_offload* off, int n_tokens, int top_k) {
  return off ? smoe_workspace_bytes(off->layer, n_tokens, top_k) : 0;
}

uint32_t smoe_offload_slots(const smoe_offload* off) { return off ? off->n_slots : 0; }

int smoe_offload_get_stats(const smoe_offload* off, smoe_offload_stats* stats) {
  if (!off || !stats) return report_error(SMOE_E_ARG, "null handle or output");
  *stats = off->st;
  return report_ok();
}

int smoe_offload_forward(smoe_offload* off, const void* d_x, int x_dtype, const float* d_logits,
                         int n_tokens, int top_k, int norm_topk_prob, float* d_out,
                         int32_t* d_topk_ids, float* d_topk_w, void* d_workspace,
                         uint64_t ws_bytes, void* hip_stream) {
  if (!off) return report_error(SMOE_E_ARG, "null offload handle");
  const hipStream_t s = (hipStream_t)hip_stream;
  auto forward = [&]() {
    return smoe_moe_forward(off->layer, d_x, x_dtype, d_logits, n_tokens, top_k, norm_topk_prob,
                            d_out, d_topk_ids, d_topk_w, d_workspace, ws_bytes, hip_stream);
  };
  if (off->n_slots == 0) {
    const int rc = forward();
    if (rc == SMOE_OK && n_tokens > 0) off->st.forwards += 1;
    return rc;
  }
  // the checks smoe_moe_forward makes, before anything is enqueued
  const uint64_t need = smoe_workspace_bytes(off->layer, n_tokens, top_k);
  if (n_tokens < 0 || n_tokens > SMOE_MAX_TOKENS || top_k < 1 || top_k > SMOE_MAX_TOP_K ||
      top_k > (int)off->E)
    return report_error(SMOE_E_ARG, "n_tokens or top_k out of range");
  if (n_tokens == 0) return forward();
  if (need == 0) return forward();  // reports the grouping limit
  if (!d_workspace || ws_bytes < need || !aligned_to(d_workspace, 256))
    return forward();                // reports the workspace error
  if (!d_x || !d_logits || !d_out || !aligned_to(d_x, 16) || !aligned_to(d_logits, 4) ||
      !aligned_to(d_out, 4) || (x_dtype != SMOE_DTYPE_BF16 && x_dtype != SMOE_DTYPE_F32))
    return forward();                // reports the argument error
  // 1. route into the workspace and read the ids back
  const int pairs = n_tokens * top_k;
  int32_t* ids = (int32_t*)d_workspace;
  float* w = (float*)((uint8_t*)d_workspace + (uint64_t)pairs * 4);
  int rc = smoe_route(d_logits, n_tokens, (int)off->E, top_k, norm_topk_prob, ids, w, hip_stream);
  if (rc) return rc;
  hipError_t e = hipMemcpyAsync(off->h_ids, ids, (uint64_t)pairs * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "routed ids read-back");
  // 2. hits first, so that no slot this call needs is chosen as a victim
  const uint64_t t = ++off->tick;
  std::vector<int32_t> miss;
  for (int p = 0; p < pairs; ++p) {
    const int32_t x = off->h_ids[p];
    if (x < 0 || (uint32_t)x >= off->E)
      return report_error(SMOE_E_HIP, "routing returned expert id %d", x);
    if (off->seen[x] == t) continue;
    off->seen[x] = t;
    if (off->expert_slot[x] >= 0) {
      off->slot_tick[off->expert_slot[x]] = t;
      off->st.hits += 1;
    } else {
      miss.push_back(x);
    }
  }
  // 3. misses: least recently used slot not used by this call, else direct
  bool table_changed = false;
  for (int32_t x : miss) {
    int32_t victim = -1;
    uint64_t oldest = t;
    for (uint32_t q = 0; q < off->n_slots; ++q) {
      if (off->slot_tick[q] < oldest) {
        oldest = off->slot_tick[q];
        victim = (int32_t)q;
        if (off->slot_expert[q] < 0) break;  // a free slot
      }
    }
    if (victim < 0) {
      off->st.direct += 1;  // its table entry already points into host memory
      continue;
    }
    const int32_t old = off->slot_expert[victim];
    if (old >= 0) {
      off->expert_slot[old] = -1;
      off->h_table[old] = (uint64_t)(uintptr_t)(off->host + (uint64_t)old * off->stride);
    }
    uint8_t* dst = off->cache + (uint64_t)victim * off->stride;
    e = hipMemcpyAsync(dst, off->host + (uint64_t)x * off->stride, off->raw,
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "expert copy to the cache");
    off->slot_expert[victim] = x;
    off->slot_tick[victim] = t;
    off->expert_slot[x] = victim;
    off->h_table[x] = (uint64_t)(uintptr_t)dst;
    off->st.fetched += 1;
    off->st.bytes_fetched += off->raw;
    table_changed = true;
  }
  // 4. the table, then the forward, on the same stream
  if (table_changed) {
    e = hipMemcpyAsync(off->d_table, off->h_table, sizeof(uint64_t) * off->E,
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "expert table upload");
  }
  rc = forward();
  if (rc == SMOE_OK) off->st.forwards += 1;
  return rc;
}

}  // extern "C"
