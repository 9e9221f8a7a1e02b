// Host side of the C ABI declared in include/smoe.h: argument validation,
// layer handles, workspace layout and the per-call launch sequence.
//
// Nothing here allocates device memory: blobs, activations, outputs and the
// workspace all belong to the caller.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>

#include "smoe_internal.hpp"
#include "smoe_launch.hpp"


namespace smoe {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SMOE_OK;
}

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

// ".smoe Binary Format", Expert Blob Architecture: gate [ffn, d], up [ffn, d],
// down [d, ffn]; codes ceil(n*bits/8) bytes then ceil(n/64) scales each.
int layout_of(uint32_t d, uint32_t ffn, uint32_t bits, uint32_t sdt, smoe_expert_layout* L) {
  if (!L) return fail(SMOE_E_ARG, "null layout output");
  if (bits != 2 && bits != 4) return fail(SMOE_E_ARG, "bits must be 2 or 4 (got %u)", bits);
  if (d == 0 || ffn == 0 || d % 64 || ffn % 64)
    return fail(SMOE_E_ARG, "d_model (%u) and ffn_dim (%u) must be positive multiples of 64", d,
                ffn);
  if (sdt != SMOE_SCALE_F32 && sdt != SMOE_SCALE_F16)
    return fail(SMOE_E_ARG, "unknown scale dtype %u", sdt);
  const uint64_t ss = sdt == SMOE_SCALE_F32 ? 4 : 2;
  uint64_t off = 0;
  smoe_tensor_layout* t[3] = {&L->gate, &L->up, &L->down};
  const uint32_t rows[3] = {ffn, ffn, d}, cols[3] = {d, d, ffn};
  for (int i = 0; i < 3; ++i) {
    const uint64_t n = (uint64_t)rows[i] * cols[i];
    t[i]->rows = rows[i];
    t[i]->cols = cols[i];
    t[i]->codes_offset = off;
    t[i]->codes_bytes = (n * bits + 7) / 8;
    t[i]->scales_offset = off + t[i]->codes_bytes;
    t[i]->scales_bytes = (n + 63) / 64 * ss;
    off = t[i]->scales_offset + t[i]->scales_bytes;
  }
  L->raw_size = off;
  L->padded_size = align_up(off, SMOE_BLOB_ALIGN);
  return SMOE_OK;
}

int make_plan(uint32_t d, uint32_t ffn, uint32_t bits, uint32_t sdt, ExpertPlan* P,
              smoe_expert_layout* Lout) {
  smoe_expert_layout L;
  int rc = layout_of(d, ffn, bits, sdt, &L);
  if (rc) return rc;
  P->d_model = (int)d;
  P->ffn = (int)ffn;
  P->raw_size = L.raw_size;
  P->padded_size = L.padded_size;
  const smoe_tensor_layout* t[3] = {&L.gate, &L.up, &L.down};
  MatPlan* m[3] = {&P->gate, &P->up, &P->down};
  for (int i = 0; i < 3; ++i)
    if (!plan_matrix((int)t[i]->rows, (int)t[i]->cols, (int)bits, t[i]->codes_offset,
                     t[i]->scales_offset, m[i]))
      return fail(SMOE_E_UNSUPPORTED,
                  "no kernel for a [%u, %u] Q%u tensor (row of %u code words)", t[i]->rows,
                  t[i]->cols, bits, t[i]->cols * bits / 32);
  // the batched stages stage each token (x as fp32 hi + lo for the residual
  // stream) or each h row in one four-wave workgroup's 64 KB of LDS
  if (!batch_fits(P->gate, true) || !batch_fits(P->down, false))
    return fail(SMOE_E_UNSUPPORTED,
                "d_model %u / ffn_dim %u: one activation vector does not fit the batched "
                "stages' 64 KB staging", d, ffn);
  if (Lout) *Lout = L;
  return SMOE_OK;
}

// The shared expert runs inside the routed launches, as nsh = shared_ffn /
// ffn more slots over all T tokens, when its ffn is a multiple of the routed
// one (at most 16 times) and the launches take the plain matrix-core stages
// (the K-sliced prefill stages run routed slots only); then the result is
// nsh, else 0 and the shared expert has launches of its own.
int shared_parts(const LayerInfo& L, int T, int k) {
  const uint32_t sf = L.desc.shared_ffn_dim, f = L.desc.ffn_dim;
  if (!sf || sf % f || sf / f > 16) return 0;
  const int nsh = (int)(sf / f);
  const int P = T * k, E = (int)L.desc.num_experts;
  if (gmk_wanted(P + nsh * T, (P < E ? P : E) + nsh)) return 0;
  return nsh;
}

WsLayout ws_layout(const LayerInfo& L, int T, int k) {
  WsLayout W{};
  const uint64_t P = (uint64_t)T * k, E = L.desc.num_experts;
  const uint64_t nsh = (uint64_t)shared_parts(L, T, k);
  const uint64_t PT = P + nsh * T;  // pairs, the shared expert's parts included
  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  W.ids = take(P * 4);
  W.w = take(P * 4);
  W.meta = take(64);
  W.active = take(E * 4);
  W.offs = take((E + 1 + nsh) * 4);
  W.pair_token = take(PT * 4);
  W.pair_of = take(P * 4);
  W.h = take(PT * L.desc.ffn_dim * 4);
  W.y = take(PT * L.desc.d_model * 4);
  W.h_shared = take(nsh ? 0 : (uint64_t)T * L.desc.shared_ffn_dim * 4);
  W.y_shared = take(!nsh && L.desc.shared_ffn_dim ? (uint64_t)T * L.desc.d_model * 4 : 0);
  const uint64_t slots = P < E ? P : E;
  W.prep_bytes = 0;
  if (gmk_wanted((int)P, (int)slots)) {
    const uint64_t gu = gmk_prep_bytes((uint64_t)T, (int)L.desc.d_model);
    const uint64_t dn = gmk_prep_bytes(P, (int)L.desc.ffn_dim);
    W.prep_bytes = gu > dn ? gu : dn;
  }
  W.prep = take(W.prep_bytes);
  W.total = o;
  return W;
}

// armed timing events (smoe_trace_kernel); the kernel id is read without the
// lock, so a forward takes no lock while nothing is armed
std::mutex g_trace_mu;
std::atomic<int> g_trace_kernel{SMOE_KERNEL_NONE};
hipEvent_t g_trace_before = nullptr, g_trace_after = nullptr;

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SMOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return SMOE_OK;
}

// The shared expert's stream and fork / join events, created on first use
// (on the current device) so that registering a layer needs no GPU. The
// events are the layer's own: a forward holds g_side_mu from the fork until
// its stream has queued the wait on the join, so that calls from several
// threads never re-record an event between another call's record and wait.
std::mutex g_side_mu;

// g_side_mu held
hipError_t side_stream(const LayerInfo& L) {
  if (L.side) return hipSuccess;
  hipStream_t st = nullptr;
  hipEvent_t f = nullptr, j = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (j) (void)hipEventDestroy(j);
    if (f) (void)hipEventDestroy(f);
    if (st) (void)hipStreamDestroy(st);
    return e;
  }
  L.fork = f;
  L.join = j;
  L.side = st;
  return hipSuccess;
}

// One layer: route+group, gate/up+SwiGLU, down, combine (optionally into the
// residual stream with RMSNorm applied on the way in). side_ok: the shared
// expert may run on the layer's side stream (else on s, before routing).
int forward_impl(const LayerInfo& L, const void* x, int xmode, float eps, const float* logits,
                 int T, int k, int norm, float* out, int accumulate, int32_t* uids, float* uw,
                 uint8_t* ws, hipStream_t s, const RouteCfg& cfg = RouteCfg(),
                 bool side_ok = true) {
  const WsLayout W = ws_layout(L, T, k);
  int32_t* ids = (int32_t*)(ws + W.ids);
  float* w = (float*)(ws + W.w);
  int* meta = (int*)(ws + W.meta);
  int* active = (int*)(ws + W.active);
  int* offs = (int*)(ws + W.offs);
  int* pair_token = (int*)(ws + W.pair_token);
  int* pair_of = (int*)(ws + W.pair_of);
  float* h = (float*)(ws + W.h);
  float* y = (float*)(ws + W.y);
  const int E = (int)L.desc.num_experts;
  const int max_slots = T * k < E ? T * k : E;
  const int nsh = shared_parts(L, T, k);
  const int pairs = T * k + nsh * T;
  int rc;
  if (T == 1 && cfg.is_default()) {
    bool launched = false;
    if ((rc = check_hip(decode1_try(L, x, xmode != X_BF16, xmode == X_F32_RMS, eps, logits, k,
                                    norm, out, accumulate, uids, uw, h, ids, w, s, &launched),
                        "batch-1 layer")))
      return rc;
    if (launched) return SMOE_OK;
  }
  if (cfg.is_default()) {
    // a few tokens (or one token with a shared expert): routing, grouping
    // and gate/up in one launch, then the grouped down stage and the combine
    bool launched = false;
    if ((rc = check_hip(small_try(L, x, xmode != X_BF16, xmode == X_F32_RMS, eps, logits, T, k,
                                  norm, nsh, uids, uw, ids, w, meta, active, offs, pair_token,
                                  pair_of, h, s, &launched),
                        "small-batch gate/up launch")))
      return rc;
    if (launched) {
      if ((rc = check_hip(small_down_try(L, h, T, k, nsh, meta, active, offs, pair_token,
                                         pair_of, w, out, accumulate, s, &launched),
                          "small-batch down launch")))
        return rc;
      if (launched) return SMOE_OK;
      float* ysh = nsh ? y + (size_t)T * k * L.desc.d_model : nullptr;
      {
        TracedLaunch t(SMOE_KERNEL_DOWN);
        rc = check_hip(launch_down(L, false, h, T, pairs, max_slots, meta, active, offs, y, s,
                                   nullptr, nsh),
                       "down launch");
      }
      if (rc) return rc;
      return check_hip(launch_combine(y, pair_of, w, ysh, nsh ? nsh : 1, nullptr, out, T, k,
                                      (int)L.desc.d_model, accumulate, s),
                       "combine launch");
    }
  }
  // the shared expert needs only x: it runs on the layer's side stream from
  // the work enqueued so far, beside routing and the routed stages, and the
  // combine waits for it
  float* ysh = nsh ? y + (size_t)T * k * L.desc.d_model : nullptr;
  std::unique_lock<std::mutex> side_lock;
  if (L.desc.shared_ffn_dim && !nsh) {
    float* hsh = (float*)(ws + W.h_shared);
    ysh = (float*)(ws + W.y_shared);
    hipStream_t ss = s;
    if (side_ok) {
      side_lock = std::unique_lock<std::mutex>(g_side_mu);
      if ((rc = check_hip(side_stream(L), "shared-expert stream and events")) ||
          (rc = check_hip(hipEventRecord(L.fork, s), "shared-expert fork")) ||
          (rc = check_hip(hipStreamWaitEvent(L.side, L.fork, 0), "shared-expert fork")))
        return rc;
      ss = L.side;
    }
    if ((rc = check_hip(launch_gate_up(L, true, x, xmode, eps, T, T, 1, meta, active, offs,
                                       pair_token, hsh, ss, nullptr),
                        "shared gate/up launch")))
      return rc;
    if ((rc = check_hip(launch_down(L, true, hsh, T, T, 1, meta, active, offs, ysh, ss,
                                    nullptr),
                        "shared down launch")))
      return rc;
    if (side_ok && (rc = check_hip(hipEventRecord(L.join, L.side), "shared-expert join")))
      return rc;
  }
  bool routed = false;
  if (cfg.is_default() && !gmk_wanted(pairs, max_slots) &&
      (rc = check_hip(small_route_try(L, logits, T, k, norm, nsh, uids, uw, ids, w, meta, active,
                                      offs, pair_token, pair_of, s, &routed),
                      "small-batch route launch")))
    return rc;
  if (!routed &&
      (rc = check_hip(launch_route(logits, T, E, k, norm, ids, w, uids, uw, 1, meta, active,
                                   offs, pair_token, pair_of, s, cfg, nsh),
                      "route launch")))
    return rc;
  void* prep = W.prep_bytes && !nsh ? ws + W.prep : nullptr;
  {
    TracedLaunch t(SMOE_KERNEL_GATE_UP);
    rc = check_hip(launch_gate_up(L, false, x, xmode, eps, T, pairs, max_slots, meta, active, offs,
                                  pair_token, h, s, prep, nsh),
                   "gate/up launch");
  }
  if (rc) return rc;
  if (cfg.is_default() && !side_lock.owns_lock() && !gmk_wanted(pairs, max_slots)) {
    // up to 16 tokens: the down stage and the combine in one launch
    bool launched = false;
    if ((rc = check_hip(small_down_try(L, h, T, k, nsh, meta, active, offs, pair_token, pair_of,
                                       w, out, accumulate, s, &launched),
                        "small-batch down launch")))
      return rc;
    if (launched) return SMOE_OK;
  }
  {
    TracedLaunch t(SMOE_KERNEL_DOWN);
    rc = check_hip(launch_down(L, false, h, T, pairs, max_slots, meta, active, offs, y, s, prep,
                               nsh),
                   "down launch");
  }
  if (rc) return rc;
  if (side_lock.owns_lock()) {
    if ((rc = check_hip(hipStreamWaitEvent(s, L.join, 0), "shared-expert join"))) return rc;
    side_lock.unlock();
  }
  return check_hip(
      launch_combine(y, pair_of, w, ysh, nsh ? nsh : 1, cfg.shared_gate, out, T, k,
                     (int)L.desc.d_model,
                     accumulate, s),
      "combine launch");
}

}  // namespace

int report_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int report_ok() { return ok(); }

thread_local LaunchEvents t_launch_events;

bool trace_take(int kernel, hipEvent_t* start, hipEvent_t* stop) {
  if (g_trace_kernel.load(std::memory_order_acquire) != kernel) return false;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  if (g_trace_kernel.load(std::memory_order_relaxed) != kernel) return false;
  *start = g_trace_before;
  *stop = g_trace_after;
  g_trace_kernel.store(SMOE_KERNEL_NONE, std::memory_order_release);
  return true;
}

}  // namespace smoe

using namespace smoe;

extern "C" {

int smoe_version(void) { return SMOE_ABI_VERSION; }

const char* smoe_last_error(void) { return g_err; }

int smoe_expert_layout_of(uint32_t d_model, uint32_t ffn_dim, uint32_t bits,
                          uint32_t scale_dtype, smoe_expert_layout* out) {
  int rc = layout_of(d_model, ffn_dim, bits, scale_dtype, out);
  return rc ? rc : ok();
}

int smoe_load_blobs(const smoe_layer_desc* desc, const void* d_blobs, uint64_t nbytes,
                    const void* d_shared_blob, uint64_t shared_nbytes, smoe_layer** out) {
  if (!out) return fail(SMOE_E_ARG, "null output handle pointer");
  *out = nullptr;
  if (!desc) return fail(SMOE_E_ARG, "null layer description");
  if (!d_blobs) return fail(SMOE_E_ARG, "null blob bank");
  const smoe_layer_desc& D = *desc;
  if (D.group_size != SMOE_GROUP_SIZE)
    return fail(SMOE_E_ARG, "group_size must be 64 (got %u)", D.group_size);
  if (D.num_experts < 1 || D.num_experts > SMOE_MAX_EXPERTS)
    return fail(SMOE_E_ARG, "num_experts must be in [1, %d] (got %u)", SMOE_MAX_EXPERTS,
                D.num_experts);
  if (D.reserved != 0) return fail(SMOE_E_ARG, "reserved field must be 0");
  LayerInfo info{};
  info.desc = D;
  smoe_expert_layout L;
  int rc = make_plan(D.d_model, D.ffn_dim, D.bits, D.scale_dtype, &info.plan, &L);
  if (rc) return rc;
  if (D.blob_stride % SMOE_BLOB_ALIGN || D.blob_stride < L.raw_size)
    return fail(SMOE_E_LAYOUT,
                "blob_stride %llu must be a multiple of 16384 and >= the raw blob size %llu",
                (unsigned long long)D.blob_stride, (unsigned long long)L.raw_size);
  if (!aligned(d_blobs, SMOE_BANK_ALIGN))
    return fail(SMOE_E_LAYOUT, "blob bank must be %d-byte aligned", SMOE_BANK_ALIGN);
  const uint64_t need = (uint64_t)(D.num_experts - 1) * D.blob_stride + L.raw_size;
  if (nbytes < need)
    return fail(SMOE_E_LAYOUT, "blob bank holds %llu bytes, needs %llu",
                (unsigned long long)nbytes, (unsigned long long)need);
  info.blobs = (const uint8_t*)d_blobs;
  info.nbytes = nbytes;
  if (D.shared_ffn_dim) {
    if (!d_shared_blob) return fail(SMOE_E_ARG, "shared_ffn_dim set but no shared blob");
    smoe_expert_layout SL;
    rc = make_plan(D.d_model, D.shared_ffn_dim, D.bits, D.scale_dtype, &info.shared_plan, &SL);
    if (rc) return rc;
    if (!aligned(d_shared_blob, SMOE_BANK_ALIGN))
      return fail(SMOE_E_LAYOUT, "shared blob must be %d-byte aligned", SMOE_BANK_ALIGN);
    if (shared_nbytes < SL.raw_size)
      return fail(SMOE_E_LAYOUT, "shared blob holds %llu bytes, needs %llu",
                  (unsigned long long)shared_nbytes, (unsigned long long)SL.raw_size);
    info.shared = (const uint8_t*)d_shared_blob;
    info.shared_nbytes = shared_nbytes;
  } else if (d_shared_blob) {
    return fail(SMOE_E_ARG, "shared blob given but shared_ffn_dim is 0");
  }
  smoe_layer* h = new (std::nothrow) smoe_layer;
  if (!h) return fail(SMOE_E_ARG, "out of host memory");
  h->info = info;
  *out = h;
  return ok();
}

smoe_layer::~smoe_layer() {
  if (info.join) (void)hipEventDestroy(info.join);
  if (info.fork) (void)hipEventDestroy(info.fork);
  if (info.side) (void)hipStreamDestroy(info.side);
}

void smoe_free(smoe_layer* layer) { delete layer; }

uint64_t smoe_workspace_bytes(const smoe_layer* layer, int n_tokens, int top_k) {
  if (!layer || n_tokens < 0 || n_tokens > SMOE_MAX_TOKENS || top_k < 1 ||
      top_k > SMOE_MAX_TOP_K || !group_fits((int)layer->info.desc.num_experts, n_tokens))
    return 0;
  return ws_layout(layer->info, n_tokens, top_k).total;
}

// Validates opts against E and k and turns them into the kernels' form.
static int route_cfg(const smoe_route_opts* opts, int n_experts, int top_k, RouteCfg* cfg) {
  *cfg = RouteCfg();
  if (!opts) return SMOE_OK;
  if (opts->sigmoid != 0 && opts->sigmoid != 1) return fail(SMOE_E_ARG, "sigmoid must be 0 or 1");
  if (!std::isfinite(opts->scaling_factor))
    return fail(SMOE_E_ARG, "scaling_factor must be finite");
  if (opts->d_expert_bias && !aligned(opts->d_expert_bias, 4))
    return fail(SMOE_E_ARG, "expert bias must be 4-byte aligned");
  if (opts->d_shared_gate && !aligned(opts->d_shared_gate, 4))
    return fail(SMOE_E_ARG, "shared gate must be 4-byte aligned");
  cfg->sigmoid = opts->sigmoid;
  cfg->scale = opts->scaling_factor;
  cfg->bias = opts->d_expert_bias;
  cfg->shared_gate = opts->d_shared_gate;
  if (opts->use_mask) {
    int routable = 0;
    for (int wd = 0; wd < SMOE_MAX_EXPERTS / 32; ++wd) {
      uint32_t m = opts->expert_mask[wd];
      for (int b = 0; b < 32; ++b)
        if ((m >> b) & 1u) {
          if (wd * 32 + b >= n_experts)
            return fail(SMOE_E_ARG, "expert mask bit %d set past num_experts %d", wd * 32 + b,
                        n_experts);
          ++routable;
        }
      cfg->mask[wd] = m;
    }
    if (routable < top_k)
      return fail(SMOE_E_ARG, "expert mask leaves %d routable experts for top_k %d", routable,
                  top_k);
    cfg->use_mask = 1;
  }
  return SMOE_OK;
}

void smoe_route_opts_init(smoe_route_opts* opts) {
  if (!opts) return;
  std::memset(opts, 0, sizeof(*opts));
  opts->scaling_factor = 1.0f;
}

int smoe_route(const float* d_logits, int n_tokens, int n_experts, int top_k,
               int norm_topk_prob, int32_t* d_ids, float* d_weights, void* hip_stream) {
  return smoe_route_ex(d_logits, n_tokens, n_experts, top_k, norm_topk_prob, nullptr, d_ids,
                       d_weights, hip_stream);
}

int smoe_route_ex(const float* d_logits, int n_tokens, int n_experts, int top_k,
                  int norm_topk_prob, const smoe_route_opts* opts, int32_t* d_ids,
                  float* d_weights, void* hip_stream) {
  if (n_tokens < 0 || n_tokens > SMOE_MAX_TOKENS)
    return fail(SMOE_E_ARG, "n_tokens must be in [0, %d]", SMOE_MAX_TOKENS);
  if (n_experts < 1 || n_experts > SMOE_MAX_EXPERTS)
    return fail(SMOE_E_ARG, "n_experts must be in [1, %d]", SMOE_MAX_EXPERTS);
  const int kmax = n_experts < SMOE_MAX_TOP_K ? n_experts : SMOE_MAX_TOP_K;
  if (top_k < 1 || top_k > kmax) return fail(SMOE_E_ARG, "top_k must be in [1, %d]", kmax);
  RouteCfg cfg;
  int rc = route_cfg(opts, n_experts, top_k, &cfg);
  if (rc) return rc;
  if (n_tokens == 0) return ok();
  if (!d_logits || !d_ids || !d_weights) return fail(SMOE_E_ARG, "null pointer argument");
  rc = check_hip(launch_route(d_logits, n_tokens, n_experts, top_k, norm_topk_prob != 0, d_ids,
                              d_weights, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr,
                              nullptr, (hipStream_t)hip_stream, cfg),
                 "route launch");
  return rc ? rc : ok();
}

static int check_layer_args(const smoe_layer* layer, int n_tokens, int top_k) {
  if (!layer) return fail(SMOE_E_ARG, "null layer");
  if (n_tokens < 0 || n_tokens > SMOE_MAX_TOKENS)
    return fail(SMOE_E_ARG, "n_tokens must be in [0, %d] (got %d)", SMOE_MAX_TOKENS, n_tokens);
  const int E = (int)layer->info.desc.num_experts;
  const int kmax = E < SMOE_MAX_TOP_K ? E : SMOE_MAX_TOP_K;
  if (top_k < 1 || top_k > kmax)
    return fail(SMOE_E_ARG, "top_k must be in [1, %d] (got %d)", kmax, top_k);
  if (!group_fits(E, n_tokens))
    return fail(SMOE_E_UNSUPPORTED, "%d tokens over %d experts exceed the grouping's LDS", n_tokens,
                E);
  return SMOE_OK;
}

static int check_forward_args(const smoe_layer* layer, int n_tokens, int top_k,
                              const void* d_workspace, uint64_t ws_bytes) {
  const int rc = check_layer_args(layer, n_tokens, top_k);
  if (rc || n_tokens == 0) return rc;
  const uint64_t need = ws_layout(layer->info, n_tokens, top_k).total;
  if (!d_workspace || ws_bytes < need)
    return fail(SMOE_E_WORKSPACE, "workspace of %llu bytes needed (got %llu)",
                (unsigned long long)need, (unsigned long long)ws_bytes);
  if (!aligned(d_workspace, 256)) return fail(SMOE_E_WORKSPACE, "workspace must be 256-byte aligned");
  return SMOE_OK;
}

int smoe_moe_forward(const smoe_layer* layer, const void* d_x, int x_dtype,
                     const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                     float* d_out, int32_t* d_topk_ids, float* d_topk_w, void* d_workspace,
                     uint64_t ws_bytes, void* hip_stream) {
  return smoe_moe_forward_ex(layer, d_x, x_dtype, d_logits, n_tokens, top_k, norm_topk_prob,
                             nullptr, d_out, d_topk_ids, d_topk_w, d_workspace, ws_bytes,
                             hip_stream);
}

int smoe_moe_forward_ex(const smoe_layer* layer, const void* d_x, int x_dtype,
                        const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                        const smoe_route_opts* opts, float* d_out, int32_t* d_topk_ids,
                        float* d_topk_w, void* d_workspace, uint64_t ws_bytes,
                        void* hip_stream) {
  int rc = check_forward_args(layer, n_tokens, top_k, d_workspace, ws_bytes);
  if (rc) return rc;
  RouteCfg cfg;
  if ((rc = route_cfg(opts, (int)layer->info.desc.num_experts, top_k, &cfg))) return rc;
  if (x_dtype != SMOE_DTYPE_BF16 && x_dtype != SMOE_DTYPE_F32)
    return fail(SMOE_E_ARG, "x_dtype must be SMOE_DTYPE_BF16 or SMOE_DTYPE_F32");
  if (n_tokens == 0) return ok();
  if (!d_x || !d_logits || !d_out) return fail(SMOE_E_ARG, "null x, logits or out");
  if (!aligned(d_x, 16)) return fail(SMOE_E_ARG, "x must be 16-byte aligned");
  if (!aligned(d_logits, 4) || !aligned(d_out, 4))
    return fail(SMOE_E_ARG, "logits and out must be 4-byte aligned");
  rc = forward_impl(layer->info, d_x, x_dtype == SMOE_DTYPE_BF16 ? X_BF16 : X_F32, 0.f,
                    d_logits, n_tokens, top_k, norm_topk_prob != 0, d_out, 0, d_topk_ids,
                    d_topk_w, (uint8_t*)d_workspace, (hipStream_t)hip_stream, cfg);
  return rc ? rc : ok();
}

// Workspace of smoe_moe_forward_noalloc: one array per GPU, allocated with
// the library's code object when it is loaded on that GPU and held until the
// process ends. Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): the address comes from
// hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) uint8_t scratch[SMOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`.
int scratch_for_current_device(uint8_t** out) {
  int dev = -1;
  int rc = check_hip(hipGetDevice(&dev), "current device");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SMOE_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address")))
      return rc;
    if (!p || !aligned(p, 256)) return fail(SMOE_E_HIP, "scratch address %p is not usable", p);
    g_scratch_ptr[dev] = p;
  }
  *out = (uint8_t*)g_scratch_ptr[dev];
  return SMOE_OK;
}
}  // namespace

int smoe_moe_forward_noalloc(const smoe_layer* layer, const void* d_x, int x_dtype,
                             const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                             float* d_out, int32_t* d_topk_ids, float* d_topk_w,
                             void* hip_stream) {
  int rc = check_layer_args(layer, n_tokens, top_k);
  if (rc) return rc;
  if (x_dtype != SMOE_DTYPE_BF16 && x_dtype != SMOE_DTYPE_F32)
    return fail(SMOE_E_ARG, "x_dtype must be SMOE_DTYPE_BF16 or SMOE_DTYPE_F32");
  if (n_tokens == 0) return ok();
  const uint64_t need = ws_layout(layer->info, n_tokens, top_k).total;
  if (need > SMOE_NOALLOC_SCRATCH_BYTES)
    return fail(SMOE_E_WORKSPACE,
                "%d tokens at top-%d need %llu bytes of workspace; the static scratch holds "
                "%llu (use smoe_moe_forward with a workspace of that size)",
                n_tokens, top_k, (unsigned long long)need,
                (unsigned long long)SMOE_NOALLOC_SCRATCH_BYTES);
  if (!d_x || !d_logits || !d_out) return fail(SMOE_E_ARG, "null x, logits or out");
  if (!aligned(d_x, 16)) return fail(SMOE_E_ARG, "x must be 16-byte aligned");
  if (!aligned(d_logits, 4) || !aligned(d_out, 4))
    return fail(SMOE_E_ARG, "logits and out must be 4-byte aligned");
  uint8_t* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  rc = forward_impl(layer->info, d_x, x_dtype == SMOE_DTYPE_BF16 ? X_BF16 : X_F32, 0.f,
                    d_logits, n_tokens, top_k, norm_topk_prob != 0, d_out, 0, d_topk_ids,
                    d_topk_w, ws, (hipStream_t)hip_stream, RouteCfg(), /*side_ok=*/false);
  return rc ? rc : ok();
}

int smoe_decode_step(const smoe_layer* const* layers, int n_layers, float* d_h,
                     const float* d_logits, int n_tokens, int top_k, int norm_topk_prob,
                     float eps, void* d_workspace, uint64_t ws_bytes, void* hip_stream) {
  if (!layers || n_layers < 1) return fail(SMOE_E_ARG, "need at least one layer");
  if (!(eps > 0.f)) return fail(SMOE_E_ARG, "eps must be positive");
  const uint32_t d = layers[0] ? layers[0]->info.desc.d_model : 0;
  for (int l = 0; l < n_layers; ++l) {
    int rc = check_forward_args(layers[l], n_tokens, top_k, d_workspace, ws_bytes);
    if (rc) return rc;
    if (layers[l]->info.desc.d_model != d)
      return fail(SMOE_E_ARG, "layer %d has d_model %u, expected %u", l,
                  layers[l]->info.desc.d_model, d);
  }
  if (n_tokens == 0) return ok();
  if (!d_h || !d_logits) return fail(SMOE_E_ARG, "null h or logits");
  if (!aligned(d_h, 16) || !aligned(d_logits, 4))
    return fail(SMOE_E_ARG, "h must be 16-byte and logits 4-byte aligned");
  for (int l = 0; l < n_layers; ++l) {
    const LayerInfo& L = layers[l]->info;
    const float* lg = d_logits + (size_t)l * n_tokens * L.desc.num_experts;
    int rc = forward_impl(L, d_h, X_F32_RMS, eps, lg, n_tokens, top_k, norm_topk_prob != 0, d_h,
                          1, nullptr, nullptr, (uint8_t*)d_workspace, (hipStream_t)hip_stream);
    if (rc) return rc;
  }
  return ok();
}

int smoe_quantise(const float* d_w, uint64_t n_elements, int bits, int scale_dtype,
                  uint8_t* d_codes, void* d_scales, void* hip_stream) {
  if (bits != 2 && bits != 4) return fail(SMOE_E_ARG, "bits must be 2 or 4 (got %d)", bits);
  if (scale_dtype != SMOE_SCALE_F32 && scale_dtype != SMOE_SCALE_F16)
    return fail(SMOE_E_ARG, "unknown scale dtype %d", scale_dtype);
  if (n_elements > SMOE_MAX_QUANT_ELEMENTS)
    return fail(SMOE_E_ARG, "n_elements must be at most %llu (got %llu)",
                (unsigned long long)SMOE_MAX_QUANT_ELEMENTS, (unsigned long long)n_elements);
  if (n_elements == 0) return ok();
  if (!d_w || !d_codes || !d_scales) return fail(SMOE_E_ARG, "null pointer argument");
  if (!aligned(d_w, 4) || !aligned(d_scales, scale_dtype == SMOE_SCALE_F32 ? 4 : 2))
    return fail(SMOE_E_ARG, "weights must be 4-byte and scales element-aligned");
  int rc = check_hip(launch_quantise(d_w, (int64_t)n_elements, bits, scale_dtype == SMOE_SCALE_F16,
                                     d_codes, d_scales, (hipStream_t)hip_stream),
                     "quantise launch");
  return rc ? rc : ok();
}

int smoe_trace_kernel(int kernel, void* hip_event_before, void* hip_event_after) {
  if (kernel != SMOE_KERNEL_NONE && kernel != SMOE_KERNEL_GATE_UP && kernel != SMOE_KERNEL_DOWN)
    return fail(SMOE_E_ARG, "unknown kernel id %d", kernel);
  if (kernel != SMOE_KERNEL_NONE && (!hip_event_before || !hip_event_after))
    return fail(SMOE_E_ARG, "null event");
  std::lock_guard<std::mutex> lk(g_trace_mu);
  const int pending = g_trace_kernel.load(std::memory_order_relaxed) != SMOE_KERNEL_NONE ? 1 : 0;
  g_trace_before = (hipEvent_t)hip_event_before;
  g_trace_after = (hipEvent_t)hip_event_after;
  g_trace_kernel.store(kernel, std::memory_order_release);
  return kernel == SMOE_KERNEL_NONE ? pending : SMOE_OK;
}

}  // extern "C"
