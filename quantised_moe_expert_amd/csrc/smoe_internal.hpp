// Internal interface between the host API (smoe_api.hip) and the kernel
// launchers (smoe_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/smoe.h"

namespace smoe {

// Error reporting shared by the host translation units: sets the
// thread-local message smoe_last_error() returns and passes code through.
int report_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int report_ok();

// How one weight matrix is walked by a wavefront: each row of W = cols*bits/32
// 32-bit code words is split over LPR = 2^lpr_log2 lanes holding V words each
// (W == LPR * V); a wave therefore covers 64 / LPR rows per load.
struct MatPlan {
  uint64_t codes_off;   // byte offset of the codes inside the blob
  uint64_t scales_off;  // byte offset of the scales inside the blob
  int rows, cols;
  int words_per_row;    // W
  int v;                // words per lane
  int lpr_log2;
};

struct ExpertPlan {
  int d_model, ffn;
  MatPlan gate, up, down;
  uint64_t raw_size, padded_size;
};

// Result of planning one matrix; returns false if no kernel exists for it.
bool plan_matrix(int rows, int cols, int bits, uint64_t codes_off, uint64_t scales_off,
                 MatPlan* out);

// Whether the batched stages can stage one activation vector of this
// matrix's input width (fp32 split into hi + lo halves when split) in the
// 64 KB of LDS of a four-wave workgroup.
bool batch_fits(const MatPlan& m, bool split);

// Workspace layout of one forward (offsets in bytes from the workspace base).
struct WsLayout {
  uint64_t ids, w, meta, active, offs, pair_token, pair_of;
  uint64_t h, y, h_shared, y_shared;
  uint64_t prep, prep_bytes;  // prepared activations of the K-sliced stages (0 bytes: unused)
  uint64_t total;
};

// Whether the routed stages of a call with this many pairs over this many
// expert slots take the K-sliced matrix-core stage (and its prepared
// activations), and the bytes those need for V vectors of cols values.
bool gmk_wanted(int pairs, int slots);
uint64_t gmk_prep_bytes(uint64_t V, int cols);

struct LayerInfo {
  smoe_layer_desc desc;
  const uint8_t* blobs;
  uint64_t nbytes;
  const uint64_t* table;   // optional device [E] blob addresses (host offload)
  const uint8_t* shared;
  uint64_t shared_nbytes;
  ExpertPlan plan;
  ExpertPlan shared_plan;  // valid when desc.shared_ffn_dim > 0
  // shared expert: a stream of the layer's own (default priority) on which
  // it runs beside routing and the routed stages, and the fork / join events
  // (created by the layer's first forward that has a shared expert)
  mutable hipStream_t side;
  mutable hipEvent_t fork, join;
};

// Input description for the gate/up stage.
enum XMode : int {
  X_BF16 = 0,       // bf16 activations
  X_F32 = 1,        // fp32 activations
  X_F32_RMS = 2,    // fp32 residual stream; the stage applies unit-gain RMSNorm
};

// Grouping (T > 1) keeps in LDS a token bitmask per expert (ceil(T / 32)
// words), the token counts before every eighth word of it (ceil(T / 256)
// words), both rows padded to an odd number of words, and 3 E + 1 words of
// slot bookkeeping; at most 160 KB.
inline int64_t group_lds_bytes(int E, int T) {
  const int64_t tw = (T + 31) / 32, tw8 = (tw + 7) / 8;
  return ((int64_t)E * ((tw | 1) + (tw8 | 1) + 3) + 1) * 4;
}
inline bool group_fits(int E, int T) { return group_lds_bytes(E, T) <= 160 * 1024; }

// Routing variants, as the kernels take them (the ABI's smoe_route_opts
// after validation). Default-constructed = plain softmax routing.
struct RouteCfg {
  int sigmoid = 0;
  float scale = 1.0f;
  const float* bias = nullptr;
  const float* shared_gate = nullptr;
  int use_mask = 0;
  uint32_t mask[SMOE_MAX_EXPERTS / 32] = {};
  bool is_default() const {
    return !sigmoid && scale == 1.0f && !bias && !shared_gate && !use_mask;
  }
};

hipError_t launch_route(const float* logits, int T, int E, int k, int norm, int32_t* ids,
                        float* w, int32_t* user_ids, float* user_w, int group, int* meta,
                        int* active, int* offs, int* pair_token, int* pair_of,
                        hipStream_t stream, const RouteCfg& cfg = RouteCfg(), int nsh = 0);

// pairs: (token, expert) pairs of the launch (T for the shared expert on its
// own; routed plus nsh * T with the shared expert fused), used to size it.
// prep: workspace for prepared activations (gmk_prep_bytes of the stage), or
// null when the call has none.
// nsh > 0: the shared expert runs in the same launch as nsh slots after the
// routed ones (its ffn is nsh times the routed ffn; see GemvArgs), reading
// pairs P + v * T + t (P = routed pairs) of h and writing those rows of y.
hipError_t launch_gate_up(const LayerInfo& L, bool shared, const void* x, int xmode,
                          float rms_eps, int T, int pairs, int max_slots, const int* meta,
                          const int* active, const int* offs, const int* pair_token,
                          float* h, hipStream_t stream, void* prep, int nsh = 0);

hipError_t launch_down(const LayerInfo& L, bool shared, const float* h, int T, int pairs,
                       int max_slots,
                       const int* meta, const int* active, const int* offs, float* y,
                       hipStream_t stream, void* prep, int nsh = 0);

// Batch-1 path (two launches); sets *launched = false (and enqueues nothing)
// when the layer's shape has no instantiation.
hipError_t decode1_try(const LayerInfo& L, const void* x, bool xf32, bool rms, float eps,
                       const float* logits, int k, int norm, float* out, int accumulate,
                       int32_t* uids, float* uw, float* h, int32_t* ws_ids, float* ws_w,
                       hipStream_t stream, bool* launched);

// Small batches (1..4 tokens): routing, grouping and the gate/up stage in one
// launch, writing ids, w, meta, active, offs, pair_token, pair_of and h in the
// grouped layout the down stage and the combine read; nsh as for the grouped
// stages (the shared expert's parts after the routed pairs). Sets *launched =
// false (and enqueues nothing) when the call does not fit this path.
hipError_t small_try(const LayerInfo& L, const void* x, bool xf32, bool rms, float eps,
                     const float* logits, int T, int k, int norm, int nsh, int32_t* uids,
                     float* uw, int32_t* ids, float* w, int* meta, int* active, int* offs,
                     int* pair_token, int* pair_of, float* h, hipStream_t stream,
                     bool* launched);

// Up to 16 tokens: routing and grouping in one single-workgroup launch (the
// first part of the small-batch gate/up kernel), writing ids, w, meta,
// active, offs, pair_token and pair_of as the grouping launch does. Sets
// *launched = false, enqueuing nothing, when the shape does not fit.
hipError_t small_route_try(const LayerInfo& L, const float* logits, int T, int k, int norm,
                           int nsh, int32_t* uids, float* uw, int32_t* ids, float* w, int* meta,
                           int* active, int* offs, int* pair_token, int* pair_of,
                           hipStream_t stream, bool* launched);

// Small batches (1..16 tokens) in the grouped layout: the down stage of every
// grouped pair and the weighted combine (out = or += sum_j w[t, j] y[pair] +
// the shared expert's parts) in one launch. Sets *launched = false, enqueuing
// nothing, when the layer's shape has no instantiation.
hipError_t small_down_try(const LayerInfo& L, const float* h, int T, int k, int nsh,
                          const int* meta, const int* active, const int* offs,
                          const int* pair_token, const int* pair_of, const float* w, float* out,
                          int accumulate, hipStream_t stream, bool* launched);

// y_shared (nullable): nsh partial outputs of the shared expert, [nsh][T][d],
// summed; shared_gate (nullable, [T] logits): the shared expert's weight is
// sigmoid(shared_gate[t]) instead of 1.
hipError_t launch_combine(const float* y, const int* pair_of, const float* w,
                          const float* y_shared, int nsh, const float* shared_gate, float* out,
                          int T, int k, int d, int accumulate, hipStream_t stream);

// Group-64 squared-error scale search + encode + pack of n fp32 weights
// (flattened order; a short last group is allowed).
hipError_t launch_quantise(const float* w, int64_t n, int bits, int f16, uint8_t* codes,
                           void* scales, hipStream_t s);

}  // namespace smoe

// The opaque handle of include/smoe.h: host-side metadata of one layer.
struct smoe_layer {
  smoe::LayerInfo info;
  ~smoe_layer();
};
