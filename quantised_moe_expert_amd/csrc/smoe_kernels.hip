// Routing/grouping and combine kernels, and the dispatch of the expert GEMV
// stages onto their (bits, scale type, words-per-lane) instantiations.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smoe_device.hpp"
#include "smoe_gemv_args.hpp"
#include "smoe_internal.hpp"

namespace smoe {

// ------------------------------------------------------------ route+group --
// k_topk: a wave per token selects the top-k (descending logit, ties to the
// lower id) and the softmax-over-all weights ("CMF v2 Format Specification",
// 2.2), tokens spread over the whole grid (the k rounds are VALU work, too
// much for one CU at a few dozen tokens). k_group (optional, one workgroup)
// then groups the (token, slot) pairs by expert.

static_assert(SMOE_MAX_EXPERTS <= 512, "top-k kernels hold at most 8 logits per lane");

struct RouteArgs {
  const float* logits;
  int T, E, k, norm, group;
  RouteCfg cfg;
  int32_t* ids;
  float* w;
  int32_t* user_ids;
  float* user_w;
  int* meta;
  int* active;
  int* offs;
  int* pair_token;
  int* pair_of;
  int nsh;  // shared-expert slots appended after the routed ones (T pairs each)
};

// Selection key of expert e with logit f: unsigned order of the keys is the
// selection order (larger logit first, -0 equal to +0, equal logits in
// ascending id); every key is distinct and above 0, the padding key.
__device__ __forceinline__ uint64_t rt_key(float f, int e) {
  const int b = __builtin_bit_cast(int, f + 0.0f);
  const uint32_t o = (uint32_t)(b >= 0 ? b : b ^ 0x7FFFFFFF) ^ 0x80000000u;
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int rt_key_id(uint64_t k) {
  return (int)(0xFFFFFFFFu - (uint32_t)k);
}
__device__ __forceinline__ float rt_key_logit(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32) ^ 0x80000000u;
  const int b = (int)o >= 0 ? (int)o : (int)(o ^ 0x7FFFFFFFu);
  return __builtin_bit_cast(float, b);
}

// Wave-wide reductions through DPP row operations (the result in every lane).
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t rt_dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, RMASK, 0xF, false);
}
__device__ __forceinline__ uint64_t rt_max64_step(uint64_t v, uint32_t hi, uint32_t lo) {
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}
#define RT_STEP64(CTRL, RMASK)                                                    \
  v = rt_max64_step(v, rt_dpp<CTRL, RMASK>((uint32_t)(v >> 32)),                  \
                    rt_dpp<CTRL, RMASK>((uint32_t)v))
__device__ __forceinline__ uint64_t rt_wave_max_key(uint64_t v) {
  // keys are above 0, so the 0 that rows outside a broadcast's mask receive
  // never wins
  RT_STEP64(0xB1, 0xF);   // quad_perm [1,0,3,2]
  RT_STEP64(0x4E, 0xF);   // quad_perm [2,3,0,1]
  RT_STEP64(0x141, 0xF);  // row_half_mirror
  RT_STEP64(0x140, 0xF);  // row_mirror
  RT_STEP64(0x142, 0xA);  // row_bcast15
  RT_STEP64(0x143, 0xC);  // row_bcast31
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  return ((uint64_t)hi << 32) | lo;
}
#undef RT_STEP64
// Float max / sum over the wave: the same DPP steps; lanes outside a row
// broadcast's mask take 0, which can only spoil rows 0 and 2, never lane 63
// (whose value is returned).
template <int CTRL, int RMASK>
__device__ __forceinline__ float rt_dppf(float v) {
  return __builtin_bit_cast(float, (int)rt_dpp<CTRL, RMASK>(__builtin_bit_cast(uint32_t, v)));
}
__device__ __forceinline__ float rt_lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float rt_wave_max(float v) {
  v = fmaxf(v, rt_dppf<0xB1, 0xF>(v));
  v = fmaxf(v, rt_dppf<0x4E, 0xF>(v));
  v = fmaxf(v, rt_dppf<0x141, 0xF>(v));
  v = fmaxf(v, rt_dppf<0x140, 0xF>(v));
  v = fmaxf(v, rt_dppf<0x142, 0xA>(v));
  v = fmaxf(v, rt_dppf<0x143, 0xC>(v));
  return rt_lane63(v);
}
__device__ __forceinline__ float rt_wave_sum(float v) {
  v += rt_dppf<0xB1, 0xF>(v);
  v += rt_dppf<0x4E, 0xF>(v);
  v += rt_dppf<0x141, 0xF>(v);
  v += rt_dppf<0x140, 0xF>(v);
  v += rt_dppf<0x142, 0xA>(v);
  v += rt_dppf<0x143, 0xC>(v);
  return rt_lane63(v);
}

// Float64 sum / max over the wave. The butterfly adds in a different order
// on each lane, so the sum is lane 0's, broadcast: every lane divides by the
// same value.
__device__ __forceinline__ double rt_wave_sum64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return __shfl(v, 0, 64);
}
__device__ __forceinline__ double rt_wave_max64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// Top-k of one token per wave, over as many workgroups as tokens need:
// EPL = logits per lane (E <= 64 * EPL).
constexpr int TOPK_THREADS = 256;

// v from lane src (src wave-uniform)
__device__ __forceinline__ float rt_lane_value(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

template <int EPL>
__global__ __launch_bounds__(TOPK_THREADS) void k_topk(RouteArgs A) {
  const int lane = threadIdx.x & 63;
  const int gw = (int)(blockIdx.x * (TOPK_THREADS / 64) + (threadIdx.x >> 6));
  const int nw = (int)(gridDim.x * (TOPK_THREADS / 64));
  for (int t = gw; t < A.T; t += nw) {
    const float* lg = A.logits + (size_t)t * A.E;
    // this lane's logits as distinct selection keys (see rt_key); padding 0.
    // All loads unconditional (lanes past E re-read the last logit): a load
    // inside a branch would make the compiler wait for it at the join.
    float lv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) lv[i] = lg[min(lane + 64 * i, A.E - 1)];
    // routable: inside E and, with a mask, its bit set
    bool ok[EPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      ok[i] = e < A.E && (!A.cfg.use_mask || ((A.cfg.mask[e >> 5] >> (e & 31)) & 1u));
      if (lv[i] != lv[i]) lv[i] = -INFINITY;  // NaN never outranks a number
      if (ok[i]) mx = fmaxf(mx, lv[i]);
    }
    // scores: sigmoid per expert, or the softmax over the routable experts
    float sc[EPL];
    if (A.cfg.sigmoid) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) sc[i] = 1.0f / (1.0f + expf(-lv[i]));
    } else {
      mx = rt_wave_max(mx);
      float se = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        sc[i] = expf(lv[i] - mx);
        if (ok[i]) se += sc[i];
      }
      se = rt_wave_sum(se);
#pragma unroll
      for (int i = 0; i < EPL; ++i) sc[i] = sc[i] / se;
    }
    float wsum = 0.f;
    float wj[SMOE_MAX_TOP_K];
    int idj[SMOE_MAX_TOP_K];
    if (A.cfg.bias) {
      // with a bias: k rounds over the float64 key score + bias (the score
      // the float64 softmax over the routable logits, or the sigmoid; the
      // fp32 logits and bias taken exactly); the largest key wins, equal
      // keys go to the lowest id (ballots over the slots in id order)
      double kb[EPL];
      bool taken[EPL];
      if (!A.cfg.sigmoid) {
        double se = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          kb[i] = ok[i] ? exp((double)lv[i] - (double)mx) : 0.0;
          se += kb[i];
        }
        se = rt_wave_sum64(se);
#pragma unroll
        for (int i = 0; i < EPL; ++i) kb[i] = kb[i] / se;
      } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) kb[i] = 1.0 / (1.0 + exp(-(double)lv[i]));
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        kb[i] += (double)A.cfg.bias[min(e, A.E - 1)];
        taken[i] = !ok[i];
      }
#pragma unroll
      for (int j = 0; j < SMOE_MAX_TOP_K; ++j) {
        if (j < A.k) {
          double m = -INFINITY;
#pragma unroll
          for (int i = 0; i < EPL; ++i)
            if (!taken[i]) m = fmax(m, kb[i]);
          m = rt_wave_max64(m);
          int id = -1;
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            const uint64_t b = __ballot(!taken[i] && kb[i] == m);
            if (id < 0 && b) id = 64 * i + (int)__builtin_ctzll(b);
          }
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i == id) {
              taken[i] = true;
              p = sc[i];
            }
          p = rt_lane_value(p, id & 63);
          wj[j] = p;
          idj[j] = id;
          wsum += p;
        }
      }
    } else {
    // selection keys (see rt_key; 0 = not routable): the logit
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      key[i] = ok[i] ? rt_key(lv[i], e) : 0;
    }
    // k rounds: the largest remaining key over the wave wins, its owner
    // drops it and broadcasts the winner's score
#pragma unroll
    for (int j = 0; j < SMOE_MAX_TOP_K; ++j) {
      if (j < A.k) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
        best = rt_wave_max_key(best);
        const int id = rt_key_id(best);
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (key[i] == best) {
            key[i] = 0;
            p = sc[i];
          }
        p = rt_lane_value(p, id & 63);
        wj[j] = p;
        idj[j] = id;
        wsum += p;
      }
    }
    }
    // lane j < k writes selection j
#pragma unroll
    for (int j = 0; j < SMOE_MAX_TOP_K; ++j) {
      if (j < A.k && lane == j) {
        const float wt = (A.norm ? wj[j] / wsum : wj[j]) * A.cfg.scale;
        const size_t o = (size_t)t * A.k + j;
        A.ids[o] = idj[j];
        A.w[o] = wt;
        if (A.user_ids) A.user_ids[o] = idj[j];
        if (A.user_w) A.user_w[o] = wt;
      }
    }
  }
}

// Grouping of the T*k (token, slot) pairs by expert, one workgroup: active
// experts ascending, and inside an expert the pairs in ascending token order,
// so the grouping is unique. The selected ids are read GROUP_BATCH per thread
// at a time, all loads of a batch issued before the first is used; the first
// batch's ids stay in registers for the last pass. The lanes of a wave hold
// pairs of a few neighbouring tokens and many experts, so they touch the same
// word of different experts' rows: the rows are an odd number of words long,
// which puts those words in different LDS banks (with an even length they
// share one bank, and every such access is serialised lane by lane).
constexpr int GROUP_THREADS = 1024;
constexpr int GROUP_BATCH = 16;

__global__ __launch_bounds__(GROUP_THREADS) void k_group(RouteArgs A) {
  extern __shared__ uint32_t lds[];
  const int TW = (A.T + 31) >> 5, TW8 = (TW + 7) >> 3;
  const int TWS = TW | 1, TW8S = TW8 | 1;        // row strides (odd)
  uint32_t* sel = lds;                          // [E][TWS] token bitmask per expert
  int* pre8 = (int*)(sel + A.E * TWS);          // [E][TW8S] tokens before every 8th word
  int* slot_of = pre8 + A.E * TW8S;             // [E]
  int* cnt = slot_of + A.E;                     // [E]
  int* offs = cnt + A.E;                        // [E + 1] (slot order)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = A.T * A.k;
  constexpr int CH = GROUP_THREADS * GROUP_BATCH;  // pairs per batch
  // expert ids of pairs c + u * GROUP_THREADS + tid (-1 past the end)
  auto load_ids = [&](int c, int (&id)[GROUP_BATCH]) {
#pragma unroll
    for (int u = 0; u < GROUP_BATCH; ++u) {
      const int i = c + u * GROUP_THREADS + tid;
      id[u] = i < P ? A.ids[i] : -1;
    }
  };
  auto mark = [&](int c, const int (&id)[GROUP_BATCH]) {
#pragma unroll
    for (int u = 0; u < GROUP_BATCH; ++u) {
      if (id[u] >= 0) {
        const int t = (c + u * GROUP_THREADS + tid) / A.k;
        atomicOr(&sel[id[u] * TWS + (t >> 5)], 1u << (t & 31));
      }
    }
  };
  int id0[GROUP_BATCH];
  load_ids(0, id0);
  for (int i = tid; i < A.E * TWS; i += GROUP_THREADS) sel[i] = 0u;
  __syncthreads();
  mark(0, id0);
  for (int c = CH; c < P; c += CH) {
    int id[GROUP_BATCH];
    load_ids(c, id);
    mark(c, id);
  }
  __syncthreads();
  // per expert and block of eight words: tokens before the block (threads
  // take (expert, block) pairs; each expert's blocks are then summed up)
  for (int u = tid; u < A.E * TW8; u += GROUP_THREADS) {
    const int e = u / TW8, q8 = u - e * TW8;
    int c = 0;
    for (int q = q8 * 8; q < min(q8 * 8 + 8, TW); ++q) c += __popc(sel[e * TWS + q]);
    pre8[e * TW8S + q8] = c;
  }
  __syncthreads();
  for (int e = tid; e < A.E; e += GROUP_THREADS) {
    int c = 0;
    for (int q8 = 0; q8 < TW8; ++q8) {
      const int b = pre8[e * TW8S + q8];
      pre8[e * TW8S + q8] = c;
      c += b;
    }
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
        offs[s] = npairs + ic - c;
        A.active[s] = e;
        A.offs[s] = npairs + ic - c;
      }
      nact += __shfl(ia, 63, 64);
      npairs += __shfl(ic, 63, 64);
    }
    if (lane == 0) {
      for (int v = 0; v <= A.nsh; ++v) A.offs[nact + v] = npairs + v * A.T;
      A.meta[0] = nact;
      A.meta[1] = npairs;
    }
  }
  // the shared-expert slots: pair P + v * T + t is token t
  for (int i = tid; i < A.nsh * A.T; i += GROUP_THREADS) A.pair_token[P + i] = i % A.T;
  __syncthreads();
  // pair (t, j): its rank among the expert's tokens is the tokens before its
  // word's block, plus the words of the block before its word, plus the bits
  // below it in its word
  auto place = [&](int c, const int (&id)[GROUP_BATCH]) {
#pragma unroll
    for (int u = 0; u < GROUP_BATCH; ++u) {
      const int e = id[u];
      if (e >= 0) {
        const int i = c + u * GROUP_THREADS + tid;
        const int t = i / A.k;
        const uint32_t* row = sel + e * TWS;
        const int q = t >> 5;
        int rank = pre8[e * TW8S + (q >> 3)];
        for (int qq = q & ~7; qq < q; ++qq) rank += __popc(row[qq]);
        rank += __popc(row[q] & ((1u << (t & 31)) - 1u));
        const int pos = offs[slot_of[e]] + rank;
        A.pair_token[pos] = t;
        A.pair_of[i] = pos;
      }
    }
  };
  place(0, id0);
  for (int c = CH; c < P; c += CH) {
    int id[GROUP_BATCH];
    load_ids(c, id);
    place(c, id);
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int norm, int32_t* ids,
                        float* w, int32_t* user_ids, float* user_w, int group, int* meta,
                        int* active, int* offs, int* pair_token, int* pair_of,
                        hipStream_t stream, const RouteCfg& cfg, int nsh) {
  RouteArgs A{logits, T, E, k, norm, group, cfg, ids, w, user_ids, user_w,
              meta, active, offs, pair_token, pair_of, nsh};
  const int tpb = TOPK_THREADS / 64;
  int blocks = (T + tpb - 1) / tpb;
  blocks = blocks > 1024 ? 1024 : blocks;
  const dim3 grid(blocks), block(TOPK_THREADS);
  if (E <= 64)
    hipLaunchKernelGGL(k_topk<1>, grid, block, 0, stream, A);
  else if (E <= 128)
    hipLaunchKernelGGL(k_topk<2>, grid, block, 0, stream, A);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk<4>, grid, block, 0, stream, A);
  else
    hipLaunchKernelGGL(k_topk<8>, grid, block, 0, stream, A);
  if (!group) return hipGetLastError();
  const size_t lds = group_lds_bytes(E, T);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_group,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_group, dim3(1), dim3(GROUP_THREADS), lds, stream, A);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine --
// out[t, i] (+)= sum_j w[t, j] * y[pair_of[t, j], i] + g_t * sum_v y_shared[v * T + t, i]
// (nsh partial outputs of the shared expert, summed in v order; g_t = 1, or
// the sigmoid of the token's shared-gate logit)

constexpr int COMBINE_THREADS = 128;

// VEC consecutive outputs per thread (4: 16-byte loads and stores, when out
// is 16-byte aligned); the sum order over j is the same for both widths
template <int VEC>
__global__ __launch_bounds__(COMBINE_THREADS) void k_combine(const float* __restrict__ y,
                                                             const int* __restrict__ pair_of,
                                                             const float* __restrict__ w,
                                                             const float* __restrict__ y_shared,
                                                             const float* __restrict__ shared_gate,
                                                             float* __restrict__ out, int k, int d,
                                                             int accumulate, int nsh, int T) {
  using V = float __attribute__((ext_vector_type(VEC)));
  const int t = blockIdx.y;
  const int i = (blockIdx.x * COMBINE_THREADS + threadIdx.x) * VEC;
  if (i >= d) return;
  V acc = {};
  for (int j = 0; j < k; ++j) {
    const int o = t * k + j;
    const V yv = *(const V*)(y + (size_t)pair_of[o] * d + i);
    const float wj = w[o];
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = fmaf(wj, yv[c], acc[c]);
  }
  if (y_shared) {
    V ys = *(const V*)(y_shared + (size_t)t * d + i);
    for (int v = 1; v < nsh; ++v) {
      const V yv = *(const V*)(y_shared + ((size_t)v * T + t) * d + i);
#pragma unroll
      for (int c = 0; c < VEC; ++c) ys[c] += yv[c];
    }
    const float den = shared_gate ? 1.0f + expf(-shared_gate[t]) : 1.0f;
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] += shared_gate ? ys[c] / den : ys[c];
  }
  V* dst = (V*)(out + (size_t)t * d + i);
  if (accumulate) {
    const V o = *dst;
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = o[c] + acc[c];
  }
  *dst = acc;
}

hipError_t launch_combine(const float* y, const int* pair_of, const float* w,
                          const float* y_shared, int nsh, const float* shared_gate, float* out,
                          int T, int k, int d, int accumulate, hipStream_t stream) {
  // y and y_shared are workspace rows (256-byte aligned, d a multiple of 64)
  if (((uintptr_t)out & 15) == 0 && d % 4 == 0) {
    dim3 grid((d + 4 * COMBINE_THREADS - 1) / (4 * COMBINE_THREADS), T);
    hipLaunchKernelGGL(k_combine<4>, grid, dim3(COMBINE_THREADS), 0, stream, y, pair_of, w,
                       y_shared, shared_gate, out, k, d, accumulate, nsh, T);
  } else {
    dim3 grid((d + COMBINE_THREADS - 1) / COMBINE_THREADS, T);
    hipLaunchKernelGGL(k_combine<1>, grid, dim3(COMBINE_THREADS), 0, stream, y, pair_of, w,
                       y_shared, shared_gate, out, k, d, accumulate, nsh, T);
  }
  return hipGetLastError();
}

// -------------------------------------------------------------- dispatch --


bool plan_matrix(int rows, int cols, int bits, uint64_t codes_off, uint64_t scales_off,
                 MatPlan* out) {
  if (cols % 64 || rows <= 0) return false;
  const int W = cols * bits / 32;
  int lg = 0;
  while (lg < 6 && (W % (2 << lg)) == 0) ++lg;
  const int v = W >> lg;
  *out = MatPlan{codes_off, scales_off, rows, cols, W, v, lg};
  return true;
}

static MatArgs mat_args(const MatPlan& m) {
  return MatArgs{m.codes_off, m.scales_off, m.rows, m.cols, m.words_per_row, m.lpr_log2};
}

// Launch shape of a matrix-core stage: 16-row tiles, one per wave, or one
// per workgroup with its groups split over the four waves when one tile per
// wave leaves under 1024 workgroups. Tokens per chunk: twice the mean pairs
// per slot (at least 8, at most 16, one MFMA's M), cut to what the LDS
// holds; slots with more pairs take several chunks, each of which reads the
// weights again. Four-wave workgroups keep their LDS within 64 KB (two per
// CU); when that would cut a full 16-token chunk short (large batches, long
// rows) the workgroup has eight waves and up to 160 KB, one per CU, so the
// weights are read fewer times. The k-split partial-sum region (last in the
// layout) is allocated only when used. False when not even one token fits.
constexpr int GM_TPW_MAX = 4;  // 16-row tiles per wave, at most
constexpr int GM_TC_MIN = 8;   // tokens per chunk, at least
// (512 measured best against 256, 384, 1024 and 3000 on the 8- and 32-token
// layers: fewer, longer workgroups while two rounds still fill the GPU)
constexpr int GM_MIN_WG = 512;
static bool gm_shape(const MatPlan& m, bool split, int pairs, int slots, GemvArgs& A, dim3& grid,
                     unsigned& lds, int& nw) {
  const int tiles = (m.rows + 15) / 16;
  const int mean = (pairs + slots - 1) / slots;
  const int want = 2 * mean < GM_TC_MIN ? GM_TC_MIN : (2 * mean > 16 ? 16 : 2 * mean);
  auto bytes = [&](int t, int w, int k) {
    const GmLds L = gm_lds_layout(m.cols, t, split, w);
    return (k > 1 ? L.total : L.part) * 4;
  };
  nw = 4;
  if (mean >= 16 && bytes(want, 4, 1) > 65536 && bytes(want, 8, 1) <= 160 * 1024) nw = 8;
  const int ks = nw == 4 && (int64_t)(tiles + nw - 1) / nw * slots < 1024 ? nw : 1;
  A.ksplit = ks;
  const int tpb = nw / ks;
  // tiles per wave: more while the grid keeps over GM_MIN_WG
  // workgroups, so that each staging of the tokens serves more rows
  int tpw = 1;
  if (ks == 1)
    while (tpw < GM_TPW_MAX &&
           (int64_t)((tiles + tpb * 2 * tpw - 1) / (tpb * 2 * tpw)) * slots >= GM_MIN_WG)
      tpw *= 2;
  A.tiles_per_wave = tpw;
  grid = dim3((tiles + tpb * tpw - 1) / (tpb * tpw), slots);
  const int cap = nw == 8 ? 160 * 1024 : 65536;
  int tc = want;
  while (tc > 0 && bytes(tc, nw, ks) > cap) --tc;
  if (tc == 0) return false;
  A.tc = tc;
  lds = (unsigned)bytes(tc, nw, ks);
  return true;
}

bool batch_fits(const MatPlan& m, bool split) {
  // one token staged by a four-wave workgroup, k-split partial sums included
  return (int64_t)gm_lds_layout(m.cols, 1, split, 4).total * 4 <= 65536;
}

template <typename ST>
static hipError_t gm_dispatch(int bits, const GemvArgs& A, bool gate_up, int in, int nw,
                              dim3 grid, unsigned lds, hipStream_t s) {
  return bits == 4 ? launch_gm<4, ST>(A, gate_up, in, nw, grid, lds, s)
                   : launch_gm<2, ST>(A, gate_up, in, nw, grid, lds, s);
}

// Slots averaging this many routed pairs or more take the K-sliced stage
// (64 tokens per weight read) instead of 16-token chunks.
constexpr int GMK_MIN_MEAN = 24;

bool gmk_wanted(int pairs, int slots) {
  return slots > 0 && pairs / slots >= GMK_MIN_MEAN;
}

static uint64_t al256(uint64_t v) { return (v + 255) / 256 * 256; }

uint64_t gmk_prep_bytes(uint64_t V, int cols) {
  return al256(V * (uint64_t)cols * 2) + al256(V * (uint64_t)(cols / 64) * 4) + al256(V * 4);
}

// Activation vectors for the K-sliced stage, one workgroup per vector v: the
// power-of-two scale S that puts the largest magnitude just below 2^14, the
// fp16 pairs of every code word pre-divided by 2^p in the order of the MFMA
// operand (word cw, half hv -> quad cw * (PPW / 4) + hv of 16 bytes), the
// offset K = sum of the pairs times (1024 + m 2^p) of every scale group
// (stored as -K), and the output factor rms / (m S). The same arithmetic as
// k_gemm's staging.
template <int BITS, bool XF32>
__global__ __launch_bounds__(256) void k_gmk_prep(const void* x, int ld, int cols, int rms,
                                                  float eps, uint32_t* xq, float* xk, float* xo) {
  constexpr int WPW = QT<BITS>::WPW, PPW = QT<BITS>::PPW, NPOS = QT<BITS>::NPOS;
  constexpr int WPG = QT<BITS>::WPG, HALVES = PPW / 4;
  __shared__ float s_r[4][2];
  const int v = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const void* row = (const uint8_t*)x + (size_t)v * ld * (XF32 ? 4 : 2);
  const int Wr = cols / WPW, G = cols / 64;
  float amax = 0.f, ss = 0.f;
  for (int cw = tid; cw < Wr; cw += 256) {
    float xv[WPW];
    gv_load_word<BITS, XF32>(row, cw, xv);
#pragma unroll
    for (int j = 0; j < WPW; ++j) {
      amax = fmaxf(amax, fabsf(xv[j]));
      ss = fmaf(xv[j], xv[j], ss);
    }
  }
  amax = lane63(seg_max(amax, 6));
  ss = lane63(seg_sum(ss, 6));
  if (lane == 0) {
    s_r[wave][0] = amax;
    s_r[wave][1] = ss;
  }
  __syncthreads();
  float m = 0.f, q2 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    m = fmaxf(m, s_r[w][0]);
    q2 += s_r[w][1];
  }
  int ex = 0;
  frexpf(m, &ex);
  ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
  const float S = ldexpf(1.0f, 14 - ex);
  if (tid == 0) {
    const float rr = rms ? 1.0f / sqrtf(q2 / (float)cols + eps) : 1.0f;
    xo[v] = rr / (QT<BITS>::M * S);
  }
  // one code word per thread: its fp16 pairs leave as 16-byte stores, and
  // the group offset K is summed over the WPG consecutive lanes that hold
  // the group (Wr and 256 are multiples of WPG, so a lane segment is either
  // wholly inside the row or wholly past it)
  constexpr int LGW = WPG == 8 ? 3 : 2;
  static_assert((1 << LGW) == WPG, "words per group");
  uint32_t* q = xq + (size_t)v * (cols / 2);
  for (int c0 = 0; c0 < Wr; c0 += 256) {
    const int cw = c0 + tid;
    float kk = 0.f;
    if (cw < Wr) {
      float xv[WPW];
      gv_load_word<BITS, XF32>(row, cw, xv);
      uint32_t pr[PPW];
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        const int hs = p / NPOS, pos = p % NPOS;
        const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
        const float f = S * (1.0f / (float)(1 << (BITS * pos)));
        const _Float16 ha = (_Float16)(xv[ia] * f), hb = (_Float16)(xv[ib] * f);
        pr[p] = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
        kk = fmaf((float)ha + (float)hb, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)), kk);
      }
#pragma unroll
      for (int hq = 0; hq < HALVES; ++hq)
        *(u32x4*)(q + (cw * HALVES + hq) * 4) =
            u32x4{pr[4 * hq], pr[4 * hq + 1], pr[4 * hq + 2], pr[4 * hq + 3]};
    }
    kk = seg_sum(kk, LGW);
    // stored negated: the MFMA chains start from it
    if (cw < Wr && (cw & (WPG - 1)) == WPG - 1) xk[(size_t)v * G + cw / WPG] = -kk;
  }
}

static hipError_t gmk_dispatch(const LayerInfo& L, GemvArgs& A, bool gate_up, const void* x,
                               bool xf32, int V, int rows, int cols, int slots, void* prep,
                               hipStream_t s) {
  uint8_t* base = (uint8_t*)prep;
  uint32_t* xq = (uint32_t*)base;
  float* xk = (float*)(base + al256((uint64_t)V * cols * 2));
  float* xo = (float*)(base + al256((uint64_t)V * cols * 2) + al256((uint64_t)V * (cols / 64) * 4));
  A.prep_x = xq;
  A.prep_k = xk;
  A.prep_o = xo;
  if (V > 0) {
    const dim3 pg(V), pb(256);
    if (L.desc.bits == 4) {
      if (xf32)
        hipLaunchKernelGGL((k_gmk_prep<4, true>), pg, pb, 0, s, x, cols, cols, A.rms, A.eps, xq, xk, xo);
      else
        hipLaunchKernelGGL((k_gmk_prep<4, false>), pg, pb, 0, s, x, cols, cols, A.rms, A.eps, xq, xk, xo);
    } else {
      if (xf32)
        hipLaunchKernelGGL((k_gmk_prep<2, true>), pg, pb, 0, s, x, cols, cols, A.rms, A.eps, xq, xk, xo);
      else
        hipLaunchKernelGGL((k_gmk_prep<2, false>), pg, pb, 0, s, x, cols, cols, A.rms, A.eps, xq, xk, xo);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rpb = gmk_rows_per_block(gate_up);
  const dim3 grid((rows + rpb - 1) / rpb, slots);
  A.tc = GMK_TC;
  if (L.desc.bits == 4)
    return L.desc.scale_dtype == SMOE_SCALE_F32 ? launch_gm_ks<4, float>(A, gate_up, grid, s)
                                                : launch_gm_ks<4, _Float16>(A, gate_up, grid, s);
  return L.desc.scale_dtype == SMOE_SCALE_F32 ? launch_gm_ks<2, float>(A, gate_up, grid, s)
                                              : launch_gm_ks<2, _Float16>(A, gate_up, grid, s);
}

hipError_t launch_gate_up(const LayerInfo& L, bool shared, const void* x, int xmode,
                          float rms_eps, int T, int pairs, int max_slots, const int* meta,
                          const int* active, const int* offs, const int* pair_token,
                          float* h, hipStream_t stream, void* prep, int nsh) {
  const ExpertPlan& P = shared ? L.shared_plan : L.plan;
  GemvArgs A{};
  A.blobs = shared ? L.shared : L.blobs;
  A.stride = shared ? 0 : L.desc.blob_stride;
  A.table = shared ? nullptr : L.table;
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
  if (nsh > 0) {
    A.sh_blob = L.shared;
    A.nsh = nsh;
    A.sh_m0 = mat_args(L.shared_plan.gate);
    A.sh_m1 = mat_args(L.shared_plan.up);
  }
  const int in = xmode == X_BF16 ? GV_BF16 : GV_F32_SPLIT;
  if (prep && !shared && nsh == 0 && in == GV_BF16 && gmk_wanted(pairs, max_slots))
    return gmk_dispatch(L, A, true, x, false, T, P.gate.rows, P.d_model, max_slots, prep, stream);
  dim3 grid;
  unsigned lds;
  int nw;
  if (gm_shape(P.gate, in == GV_F32_SPLIT, pairs, shared ? 1 : max_slots + nsh, A, grid, lds, nw))
    return L.desc.scale_dtype == SMOE_SCALE_F32
               ? gm_dispatch<float>(L.desc.bits, A, true, in, nw, grid, lds, stream)
               : gm_dispatch<_Float16>(L.desc.bits, A, true, in, nw, grid, lds, stream);
  // unreachable for a registered layer (batch_fits is checked at load)
  return hipErrorInvalidValue;
}

hipError_t launch_down(const LayerInfo& L, bool shared, const float* h, int T, int pairs,
                       int max_slots,
                       const int* meta, const int* active, const int* offs, float* y,
                       hipStream_t stream, void* prep, int nsh) {
  const ExpertPlan& P = shared ? L.shared_plan : L.plan;
  GemvArgs A{};
  A.blobs = shared ? L.shared : L.blobs;
  A.stride = shared ? 0 : L.desc.blob_stride;
  A.table = shared ? nullptr : L.table;
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
  if (nsh > 0) {
    A.sh_blob = L.shared;
    A.nsh = nsh;
    A.sh_m0 = mat_args(L.shared_plan.down);
    A.sh_m1 = A.sh_m0;
  }
  if (prep && !shared && nsh == 0 && gmk_wanted(pairs, max_slots))
    return gmk_dispatch(L, A, false, h, true, pairs, P.down.rows, P.ffn, max_slots, prep, stream);
  dim3 grid;
  unsigned lds;
  int nw;
  if (gm_shape(P.down, false, pairs, shared ? 1 : max_slots + nsh, A, grid, lds, nw))
    return L.desc.scale_dtype == SMOE_SCALE_F32
               ? gm_dispatch<float>(L.desc.bits, A, false, GV_F32, nw, grid, lds, stream)
               : gm_dispatch<_Float16>(L.desc.bits, A, false, GV_F32, nw, grid, lds, stream);
  // unreachable for a registered layer (batch_fits is checked at load)
  return hipErrorInvalidValue;
}

}  // namespace smoe
