// Routing/grouping and combine kernels, and the dispatch of the expert GEMV
// stages onto their (bits, scale type, words-per-lane) instantiations.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smoe_gemv_args.hpp"
#include "smoe_internal.hpp"

namespace smoe {

// ------------------------------------------------------------ route+group --
// One workgroup. Phase A: a wave per token selects the top-k (descending
// logit, ties to the lower id) and the softmax-over-all weights
// ("CMF v2 Format Specification", 2.2). Phase B (optional) groups the
// (token, slot) pairs by expert: active experts ascending, and inside an
// expert the pairs in ascending token order, so the grouping is unique.

constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_EPL = SMOE_MAX_EXPERTS / 64;  // logits per lane

struct RouteArgs {
  const float* logits;
  int T, E, k, norm, group;
  int32_t* ids;
  float* w;
  int32_t* user_ids;
  float* user_w;
  int* meta;
  int* active;
  int* offs;
  int* pair_token;
  int* pair_of;
};

__global__ __launch_bounds__(ROUTE_THREADS) void k_route(RouteArgs A) {
  extern __shared__ uint32_t lds[];
  const int TW = (A.T + 31) >> 5;
  uint32_t* sel = lds;                          // [E][TW] token bitmask per expert
  int* slot_of = (int*)(lds + A.E * TW);        // [E]
  int* cnt = slot_of + A.E;                     // [E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  if (A.group) {
    for (int i = tid; i < A.E * TW; i += blockDim.x) sel[i] = 0u;
    __syncthreads();
  }
  for (int t = wave; t < A.T; t += nwaves) {
    const float* lg = A.logits + (size_t)t * A.E;
    float v[ROUTE_EPL];
    bool valid[ROUTE_EPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < ROUTE_EPL; ++i) {
      const int e = lane + 64 * i;
      valid[i] = e < A.E;
      float x = valid[i] ? lg[e] : -INFINITY;
      if (x != x) x = -INFINITY;  // NaN never outranks a number
      v[i] = x;
      mx = fmaxf(mx, x);
    }
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < ROUTE_EPL; ++i)
      if (valid[i]) se += expf(v[i] - mx);
    for (int o = 32; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
    float wsum = 0.f;
    float wj[SMOE_MAX_TOP_K];
    int idj[SMOE_MAX_TOP_K];
    for (int j = 0; j < A.k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < ROUTE_EPL; ++i) {
        const int e = lane + 64 * i;
        if (valid[i] && (v[i] > bv || (v[i] == bv && e < bi))) {
          bv = v[i];
          bi = e;
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      // remove the winner from its owner's candidates
#pragma unroll
      for (int i = 0; i < ROUTE_EPL; ++i)
        if (lane + 64 * i == bi) valid[i] = false;
      const float p = expf(bv - mx) / se;
      wj[j] = p;
      idj[j] = bi;
      wsum += p;
    }
    if (lane == 0) {
      for (int j = 0; j < A.k; ++j) {
        const float wt = A.norm ? wj[j] / wsum : wj[j];
        const size_t o = (size_t)t * A.k + j;
        A.ids[o] = idj[j];
        A.w[o] = wt;
        if (A.user_ids) A.user_ids[o] = idj[j];
        if (A.user_w) A.user_w[o] = wt;
        if (A.group) atomicOr(&sel[idj[j] * TW + (t >> 5)], 1u << (t & 31));
      }
    }
  }
  if (!A.group) return;
  __syncthreads();
  for (int e = tid; e < A.E; e += blockDim.x) {
    int c = 0;
    for (int i = 0; i < TW; ++i) c += __popc(sel[e * TW + i]);
    cnt[e] = c;
  }
  __syncthreads();
  // ascending scan over experts by wave 0: active slots and pair offsets
  if (wave == 0) {
    int nact = 0, npairs = 0;
    for (int base = 0; base < A.E; base += 64) {
      const int e = base + lane;
      const int c = e < A.E ? cnt[e] : 0;
      const int act = c > 0;
      int ia = act, ic = c;  // inclusive scans
      for (int o = 1; o < 64; o <<= 1) {
        const int ta = __shfl_up(ia, o, 64), tc = __shfl_up(ic, o, 64);
        if (lane >= o) {
          ia += ta;
          ic += tc;
        }
      }
      if (act) {
        const int s = nact + ia - 1;
        slot_of[e] = s;
        A.active[s] = e;
        A.offs[s] = npairs + ic - c;
      }
      nact += __shfl(ia, 63, 64);
      npairs += __shfl(ic, 63, 64);
    }
    if (lane == 0) {
      A.offs[nact] = npairs;
      A.meta[0] = nact;
      A.meta[1] = npairs;
    }
  }
  __syncthreads();
  const int P = A.T * A.k;
  for (int i = tid; i < P; i += blockDim.x) {
    const int t = i / A.k;
    const int e = A.ids[i];
    const uint32_t* row = sel + e * TW;
    int rank = 0;
    for (int q = 0; q < (t >> 5); ++q) rank += __popc(row[q]);
    rank += __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
    const int pos = A.offs[slot_of[e]] + rank;
    A.pair_token[pos] = t;
    A.pair_of[i] = pos;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int norm, int32_t* ids,
                        float* w, int32_t* user_ids, float* user_w, int group, int* meta,
                        int* active, int* offs, int* pair_token, int* pair_of,
                        hipStream_t stream) {
  RouteArgs A{logits, T, E, k, norm, group, ids, w, user_ids, user_w,
              meta, active, offs, pair_token, pair_of};
  const int TW = (T + 31) / 32;
  const size_t lds = group ? (size_t)E * TW * 4 + (size_t)E * 8 : 0;
  int threads = T * 64;
  if (threads > ROUTE_THREADS) threads = ROUTE_THREADS;
  if (threads < 256 && group) threads = 256;
  hipLaunchKernelGGL(k_route, dim3(1), dim3(threads), lds, stream, A);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine --
// out[t, i] (+)= sum_j w[t, j] * y[pair_of[t, j], i] + y_shared[t, i]

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const int* __restrict__ pair_of,
                                                 const float* __restrict__ w,
                                                 const float* __restrict__ y_shared,
                                                 float* __restrict__ out, int k, int d,
                                                 int accumulate) {
  const int t = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d) return;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int o = t * k + j;
    acc = fmaf(w[o], y[(size_t)pair_of[o] * d + i], acc);
  }
  if (y_shared) acc += y_shared[(size_t)t * d + i];
  float* dst = out + (size_t)t * d + i;
  *dst = accumulate ? *dst + acc : acc;
}

hipError_t launch_combine(const float* y, const int* pair_of, const float* w,
                          const float* y_shared, float* out, int T, int k, int d,
                          int accumulate, hipStream_t stream) {
  dim3 grid((d + 255) / 256, T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, stream, y, pair_of, w, y_shared, out, k, d,
                     accumulate);
  return hipGetLastError();
}

// -------------------------------------------------------------- dispatch --


static bool v_supported(int v) {
#define SMOE_V_CASE(n) \
  if (v == n) return true;
  SMOE_V_LIST(SMOE_V_CASE)
#undef SMOE_V_CASE
  return false;
}

bool plan_matrix(int rows, int cols, int bits, uint64_t codes_off, uint64_t scales_off,
                 MatPlan* out) {
  if (cols % 64 || rows <= 0) return false;
  const int W = cols * bits / 32;
  int lg = 0;
  while (lg < 6 && (W % (2 << lg)) == 0) ++lg;
  const int v = W >> lg;
  if (!v_supported(v)) return false;
  *out = MatPlan{codes_off, scales_off, rows, cols, W, v, lg};
  return true;
}

static MatArgs mat_args(const MatPlan& m) {
  return MatArgs{m.codes_off, m.scales_off, m.rows, m.cols, m.words_per_row, m.lpr_log2};
}

template <int BITS, typename ST>
static hipError_t gate_up_dispatch(int v, bool bf16, dim3 grid, hipStream_t s, const GemvArgs& A) {
#define SMOE_GU_CASE(n) \
  if (v == n) return launch_gu<BITS, ST, n>(A, bf16, grid, s);
  SMOE_V_LIST(SMOE_GU_CASE)
#undef SMOE_GU_CASE
  return hipErrorInvalidValue;
}

template <int BITS, typename ST>
static hipError_t down_dispatch(int v, dim3 grid, hipStream_t s, const GemvArgs& A) {
#define SMOE_DN_CASE(n) \
  if (v == n) return launch_dn<BITS, ST, n>(A, grid, s);
  SMOE_V_LIST(SMOE_DN_CASE)
#undef SMOE_DN_CASE
  return hipErrorInvalidValue;
}

static int rows_per_wave_for(const MatPlan& m, int mult) {
  return (64 >> m.lpr_log2) * mult;
}

hipError_t launch_gate_up(const LayerInfo& L, bool shared, const void* x, int xmode,
                          float rms_eps, int T, int max_slots, const int* meta,
                          const int* active, const int* offs, const int* pair_token,
                          float* h, hipStream_t stream) {
  const ExpertPlan& P = shared ? L.shared_plan : L.plan;
  GemvArgs A{};
  A.blobs = shared ? L.shared : L.blobs;
  A.stride = shared ? 0 : L.desc.blob_stride;
  A.shared = shared;
  A.T = T;
  A.m0 = mat_args(P.gate);
  A.m1 = mat_args(P.up);
  A.rows_per_wave = rows_per_wave_for(P.gate, 4);
  A.x = x;
  A.x_ld = P.d_model;
  A.rms = xmode == X_F32_RMS;
  A.eps = rms_eps;
  A.meta = meta;
  A.active = active;
  A.offs = offs;
  A.pair_token = pair_token;
  A.out = h;
  const int rows_per_block = A.rows_per_wave * 4;
  dim3 grid((P.gate.rows + rows_per_block - 1) / rows_per_block, shared ? 1 : max_slots);
  const int v = P.gate.v;
  if (L.desc.bits == 4)
    return L.desc.scale_dtype == SMOE_SCALE_F32
               ? gate_up_dispatch<4, float>(v, xmode == X_BF16, grid, stream, A)
               : gate_up_dispatch<4, _Float16>(v, xmode == X_BF16, grid, stream, A);
  return L.desc.scale_dtype == SMOE_SCALE_F32
             ? gate_up_dispatch<2, float>(v, xmode == X_BF16, grid, stream, A)
             : gate_up_dispatch<2, _Float16>(v, xmode == X_BF16, grid, stream, A);
}

hipError_t launch_down(const LayerInfo& L, bool shared, const float* h, int T, int max_slots,
                       const int* meta, const int* active, const int* offs, float* y,
                       hipStream_t stream) {
  const ExpertPlan& P = shared ? L.shared_plan : L.plan;
  GemvArgs A{};
  A.blobs = shared ? L.shared : L.blobs;
  A.stride = shared ? 0 : L.desc.blob_stride;
  A.shared = shared;
  A.T = T;
  A.m0 = mat_args(P.down);
  A.m1 = A.m0;
  A.rows_per_wave = rows_per_wave_for(P.down, 16);
  A.x = h;
  A.x_ld = P.ffn;
  A.meta = meta;
  A.active = active;
  A.offs = offs;
  A.out = y;
  const int rows_per_block = A.rows_per_wave * 4;
  dim3 grid((P.down.rows + rows_per_block - 1) / rows_per_block, shared ? 1 : max_slots);
  const int v = P.down.v;
  if (L.desc.bits == 4)
    return L.desc.scale_dtype == SMOE_SCALE_F32 ? down_dispatch<4, float>(v, grid, stream, A)
                                                : down_dispatch<4, _Float16>(v, grid, stream, A);
  return L.desc.scale_dtype == SMOE_SCALE_F32 ? down_dispatch<2, float>(v, grid, stream, A)
                                              : down_dispatch<2, _Float16>(v, grid, stream, A);
}

}  // namespace smoe
