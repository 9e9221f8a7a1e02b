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
static hipError_t gate_up_dispatch(int v, int in, dim3 grid, unsigned lds, hipStream_t s,
                                   const GemvArgs& A) {
#define SMOE_GU_CASE(n) \
  if (v == n) return launch_gu<BITS, ST, n>(A, in, grid, lds, s);
  SMOE_V_LIST(SMOE_GU_CASE)
#undef SMOE_GU_CASE
  return hipErrorInvalidValue;
}

template <int BITS, typename ST>
static hipError_t down_dispatch(int v, dim3 grid, unsigned lds, hipStream_t s, const GemvArgs& A) {
#define SMOE_DN_CASE(n) \
  if (v == n) return launch_dn<BITS, ST, n>(A, grid, lds, s);
  SMOE_V_LIST(SMOE_DN_CASE)
#undef SMOE_DN_CASE
  return hipErrorInvalidValue;
}

// Launch shape of a grouped stage over `slots` expert slots: rows per wave
// (whole row groups, up to 8, fewer when that leaves under ~2048 workgroups)
// and tokens staged per chunk (as many as fit in 48 KB of LDS, at most 8).
static void grouped_shape(const MatPlan& m, bool split, int slots, GemvArgs& A, dim3& grid,
                          unsigned& lds) {
  const int RPW = 64 >> m.lpr_log2, LPR = 1 << m.lpr_log2;
  const int groups = (m.rows + RPW - 1) / RPW;
  int gpw = (int)((int64_t)groups * slots / (GV_WAVES * 2048));
  gpw = gpw < 1 ? 1 : (gpw > 8 ? 8 : gpw);
  A.rows_per_wave = gpw * RPW;
  const int rpb = A.rows_per_wave * GV_WAVES;
  grid = dim3((m.rows + rpb - 1) / rpb, slots);
  const int nk = m.v / 4 + m.v % 4;
  const int per_token = (m.cols / 2 * (split ? 2 : 1) + nk * LPR + 1 + GV_WAVES * 2) * 4;
  int tc = 49152 / per_token;
  tc = tc < 1 ? 1 : (tc > 8 ? 8 : tc);
  A.tc = tc;
  lds = (unsigned)gv_lds_layout(m.cols, LPR, nk, tc, split).total * 4;
}

// Launch shape of a matrix-core stage: 16-row tiles, one per wave, or one
// per workgroup with its groups split over the four waves when one tile per
// wave leaves under 1024 workgroups. Tokens per chunk: twice the mean pairs
// per slot (at least 8, at most 16, one MFMA's M) so that the LDS a
// workgroup holds stays small enough for several workgroups per CU, then cut
// to fit 64 KB; slots with more pairs take several chunks. The k-split
// partial-sum region (last in the layout) is allocated only when used.
// False when not even one token fits.
#ifndef SMOE_GM_TPW_MAX
#define SMOE_GM_TPW_MAX 4
#endif
#ifndef SMOE_GM_TC_MIN
#define SMOE_GM_TC_MIN 8
#endif
static bool gm_shape(const MatPlan& m, bool split, int pairs, int slots, GemvArgs& A, dim3& grid,
                     unsigned& lds) {
  const int tiles = (m.rows + 15) / 16;
  const int ks = (int64_t)(tiles + GV_WAVES - 1) / GV_WAVES * slots < 1024 ? GV_WAVES : 1;
  A.ksplit = ks;
  const int tpb = GV_WAVES / ks;
  // tiles per wave: more while the grid keeps over 1024 workgroups, so that
  // each staging of the tokens serves more rows
  int tpw = 1;
  if (ks == 1)
    while (tpw < SMOE_GM_TPW_MAX &&
           (int64_t)((tiles + tpb * 2 * tpw - 1) / (tpb * 2 * tpw)) * slots >= 1024)
      tpw *= 2;
  A.tiles_per_wave = tpw;
  grid = dim3((tiles + tpb * tpw - 1) / (tpb * tpw), slots);
  const int mean = (pairs + slots - 1) / slots;
  int tc = 2 * mean < SMOE_GM_TC_MIN ? SMOE_GM_TC_MIN : (2 * mean > 16 ? 16 : 2 * mean);
  auto bytes = [&](int t) {
    const GmLds L = gm_lds_layout(m.cols, t, split);
    return (ks > 1 ? L.total : L.part) * 4;
  };
  while (tc > 0 && bytes(tc) > 65536) --tc;
  if (tc == 0) return false;
  A.tc = tc;
  lds = (unsigned)bytes(tc);
  return true;
}

template <typename ST>
static hipError_t gm_dispatch(int bits, const GemvArgs& A, bool gate_up, int in, dim3 grid,
                              unsigned lds, hipStream_t s) {
  return bits == 4 ? launch_gm<4, ST>(A, gate_up, in, grid, lds, s)
                   : launch_gm<2, ST>(A, gate_up, in, grid, lds, s);
}

hipError_t launch_gate_up(const LayerInfo& L, bool shared, const void* x, int xmode,
                          float rms_eps, int T, int pairs, int max_slots, const int* meta,
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
  A.x = x;
  A.x_ld = P.d_model;
  A.rms = xmode == X_F32_RMS;
  A.eps = rms_eps;
  A.meta = meta;
  A.active = active;
  A.offs = offs;
  A.pair_token = pair_token;
  A.out = h;
  const int in = xmode == X_BF16 ? GV_BF16 : GV_F32_SPLIT;
  dim3 grid;
  unsigned lds;
  if (gm_shape(P.gate, in == GV_F32_SPLIT, pairs, shared ? 1 : max_slots, A,
               grid, lds))
    return L.desc.scale_dtype == SMOE_SCALE_F32
               ? gm_dispatch<float>(L.desc.bits, A, true, in, grid, lds, stream)
               : gm_dispatch<_Float16>(L.desc.bits, A, true, in, grid, lds, stream);
  grouped_shape(P.gate, in == GV_F32_SPLIT, shared ? 1 : max_slots, A, grid, lds);
  const int v = P.gate.v;
  if (L.desc.bits == 4)
    return L.desc.scale_dtype == SMOE_SCALE_F32
               ? gate_up_dispatch<4, float>(v, in, grid, lds, stream, A)
               : gate_up_dispatch<4, _Float16>(v, in, grid, lds, stream, A);
  return L.desc.scale_dtype == SMOE_SCALE_F32
             ? gate_up_dispatch<2, float>(v, in, grid, lds, stream, A)
             : gate_up_dispatch<2, _Float16>(v, in, grid, lds, stream, A);
}

hipError_t launch_down(const LayerInfo& L, bool shared, const float* h, int T, int pairs,
                       int max_slots,
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
  A.x = h;
  A.x_ld = P.ffn;
  A.meta = meta;
  A.active = active;
  A.offs = offs;
  A.out = y;
  dim3 grid;
  unsigned lds;
  if (gm_shape(P.down, false, pairs, shared ? 1 : max_slots, A, grid, lds))
    return L.desc.scale_dtype == SMOE_SCALE_F32
               ? gm_dispatch<float>(L.desc.bits, A, false, GV_F32, grid, lds, stream)
               : gm_dispatch<_Float16>(L.desc.bits, A, false, GV_F32, grid, lds, stream);
  grouped_shape(P.down, false, shared ? 1 : max_slots, A, grid, lds);
  const int v = P.down.v;
  if (L.desc.bits == 4)
    return L.desc.scale_dtype == SMOE_SCALE_F32
               ? down_dispatch<4, float>(v, grid, lds, stream, A)
               : down_dispatch<4, _Float16>(v, grid, lds, stream, A);
  return L.desc.scale_dtype == SMOE_SCALE_F32 ? down_dispatch<2, float>(v, grid, lds, stream, A)
                                              : down_dispatch<2, _Float16>(v, grid, lds, stream, A);
}

}  // namespace smoe
