// One-token (batch-1 decode) MoE layer on gfx950 in two launches.
//
// The two launches meet at the kernel boundary, which on MI355X costs about
// as much as 1.5 us of streaming; a grid-wide barrier inside one launch cost
// several times that under full HBM load (its stores, atomics and polls queue
// behind the weight stream), so h, the SwiGLU intermediate, crosses through
// memory between the launches.
//
// K1 (k_dec_gate_up), NWG workgroups x 8 waves:
//   - every workgroup routes the token itself: each logit's rank is counted
//     against all others in parallel (larger logit first, equal logits in
//     ascending expert id), the k lowest ranks are the selected experts; the
//     weights are the softmax-over-all probabilities, renormalised on request
//     ("CMF v2 Format Specification", 2.2). Workgroup 0 publishes them;
//   - the fp16 activation pairs and their offsets K are built once per
//     workgroup in LDS (with the RMSNorm factor when the input is the residual
//     stream of a layer stack);
//   - the k*ffn (expert, gate/up row) units are split evenly over all waves;
//     a wave issues the non-temporal loads of a batch of units before it
//     computes any, then stores h[j, r] = silu(gate_r . x) * (up_r . x).
// K2 (k_dec_down), NWG workgroups x 8 waves:
//   - workgroup w owns a block of output rows for all k experts and wave j of
//     it owns expert slot j: the wave loads h_j (coalesced) and then the
//     block's down-projection rows (so the h loads retire first); a row is
//     spread over 16 lanes, four rows per wave load, so a row's partial sums
//     meet in a four-step DPP reduction; the wave rescales h_j by a power of
//     two into fp16 pairs once, into its own LDS region in lane-map order,
//     and each lane reads the pairs of its columns from there; the block then
//     sums the k weighted rows in ascending slot order and writes the output
//     (or adds it to the residual).

#pragma once

#include "smoe_decode_args.hpp"
#include "smoe_device.hpp"
#include "smoe_launch.hpp"

namespace smoe {

constexpr int DEC_WAVES = DEC_THREADS / 64;

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Routing key of expert e with logit f: unsigned order of the keys is the
// selection order (larger logit first, -0 equal to +0, equal logits in
// ascending id); every key is distinct and above 0, the padding key.
__device__ __forceinline__ uint64_t route_key(float f, int e) {
  const int b = __builtin_bit_cast(int, f + 0.0f);
  const uint32_t o = (uint32_t)(b >= 0 ? b : b ^ 0x7FFFFFFF) ^ 0x80000000u;
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Power-of-two factor that brings a vector whose largest magnitude is amax to
// just below 2^14.
__device__ __forceinline__ float pow2_prescale(float amax) {
  int ex = 0;
  frexpf(amax, &ex);
  ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
  return ldexpf(1.0f, 14 - ex);
}

// Activation i of a code word's slice of x held as raw 32-bit words (fp32
// values, or bf16 pairs with the lower-index value in the low half).
template <bool XF32, int N>
__device__ __forceinline__ float x_word_val(const uint32_t (&raw)[N], int i) {
  if constexpr (XF32) {
    return __builtin_bit_cast(float, raw[i]);
  } else {
    const uint32_t w = raw[i >> 1];
    return __builtin_bit_cast(float, (i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
}

// Block-wide sum of one float per thread (all DEC_THREADS threads call it).
__device__ __forceinline__ float block_sum(float v, float* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = lane63(seg_sum(v, 6));
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) t += s_tmp[w];
  __syncthreads();
  return t;
}

// --------------------------------------------------------------------- K1 --

// TBL: experts addressed through A.table (host offload); a template
// parameter so that the resident-bank kernels carry no trace of it.
template <int BITS, typename ST, int VG, bool XF32, bool TBL>
__global__ __launch_bounds__(DEC_THREADS, XF32 ? DEC_WAVES_PER_EU : DEC_GU_WAVES_PER_EU) void k_dec_gate_up(
    DecodeArgs A) {
  constexpr int PPW = QT<BITS>::PPW;
  constexpr int WPW = QT<BITS>::WPW;
  constexpr int NPOS = QT<BITS>::NPOS;
  constexpr bool SPLIT = XF32;
  using SPG = ScalePlan<BITS, VG>;
  // units per batch; two batches are in flight (double buffering). More
  // loads in flight per wave measured slower: the first batch then arrives
  // later and the memory queues hold more concurrent row streams.
  constexpr int UBr = (SPLIT ? 36 : 24) / (2 * (VG + SPG::NS));
  constexpr int UB = UBr < 1 ? 1 : (UBr > 4 ? 4 : UBr);
  constexpr int XP = VG * PPW * 64;
  constexpr int XRAW = XF32 ? WPW : WPW / 2;  // 32-bit words of x per code word

  __shared__ uint32_t s_xp[(SPLIT ? 2 : 1) * XP];
  __shared__ float s_K[VG * 64];
  __shared__ __attribute__((aligned(16))) uint64_t s_key[DEC_KEYS];
  __shared__ float s_lv[SMOE_MAX_EXPERTS];
  __shared__ int s_ids[SMOE_MAX_TOP_K];
  __shared__ float s_val[SMOE_MAX_TOP_K];
  __shared__ float s_tmp[DEC_WAVES];
  __shared__ float s_red[DEC_WAVES][2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = A.E, k = A.k;
  const int lgg = A.lg_g, LPRG = 1 << lgg, lrg = lane & (LPRG - 1), rsg = lane >> lgg;

  // 1. loads: one logit, then the x words this thread turns into fp16 pairs
  float lv = -INFINITY;
  const int nkeys = 2 * A.rk_cp << A.rk_lg;
  if (tid < E) {
    lv = A.logits[tid];
    if (lv != lv) lv = -INFINITY;  // NaN never outranks a number
    s_lv[tid] = lv;
    s_key[tid] = route_key(lv, tid);
  }
  for (int e = E + tid; e < nkeys; e += DEC_THREADS) s_key[e] = 0;
  const int Wg = A.d * BITS / 32;
  uint32_t xraw[DEC_XW][XRAW];
  // slot t is used when t * DEC_THREADS < Wg; the loads are unconditional
  // (threads past Wg load a valid word and ignore it), so waiting for them
  // later does not also wait for the weight loads issued after them
#pragma unroll
  for (int t = 0; t < DEC_XW; ++t) {
    const int cw = tid + t * DEC_THREADS;
    const uint32_t* src = (const uint32_t*)A.x + (size_t)(cw < Wg ? cw : Wg - 1) * XRAW;
#pragma unroll
    for (int c = 0; c < XRAW / 4; ++c) {
      const u32x4 v = *(const u32x4*)(src + 4 * c);
      xraw[t][4 * c] = v.x;
      xraw[t][4 * c + 1] = v.y;
      xraw[t][4 * c + 2] = v.z;
      xraw[t][4 * c + 3] = v.w;
    }
  }
  __syncthreads();

  // 2. routing: the rank of expert i is the number of keys above its own;
  //    2^rk_lg adjacent lanes share expert i, lane part p of them compares
  //    against key pairs p, p + 2^rk_lg, ... (distinct LDS banks per part),
  //    and the ranks below k place the expert in the selection
  {
    const int lg = A.rk_lg, lpk = 1 << lg;
    const int kl = lane >> lg, part = lane & (lpk - 1);
    const int i = wave * A.rk_kpw + kl;
    const bool mine = kl < A.rk_kpw && i < E;
    const uint64_t ki = s_key[mine ? i : 0];
    const u64x2* kp = (const u64x2*)s_key + part;
    int cnt = 0;
    for (int c = 0; c < A.rk_cp; c += 8) {
      u64x2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = kp[(c + u) << lg];
#pragma unroll
      for (int u = 0; u < 8; ++u) cnt += (int)(v[u].x > ki) + (int)(v[u].y > ki);
    }
    const int r = (int)seg_sum((float)cnt, lg);
    if (mine && part == lpk - 1 && r < k) {
      s_ids[r] = i;
      s_val[r] = s_lv[i];
    }
  }
  __syncthreads();

  // 3. this wave's gate/up units (k * ffn / RPWG of them, expert-major, split
  //    evenly over all waves); a chunk spans at most two experts
  const int RPWG = 64 >> lgg;
  const int upe = A.ffn / RPWG;
  const int units = k * upe;
  const int TW = (int)gridDim.x * DEC_WAVES, gw = (int)blockIdx.x * DEC_WAVES + wave;
  const int ub = units / TW, urem = units % TW;
  const int my_n = ub + (gw < urem ? 1 : 0);
  const int u0 = gw * ub + (gw < urem ? gw : urem);
  const int Gg = A.d / 64;
  int sgg[SPG::NS], tmg;
  scale_groups<BITS, VG>(lrg, LPRG, sgg, tmg);
  const int j0 = my_n > 0 ? u0 / upe : 0;
  const int rg0 = u0 - j0 * upe;
  const uint64_t* table = TBL ? A.table : nullptr;
  const uint8_t* blob0 = expert_blob(A.blobs, A.stride, table, s_ids[j0]);
  const uint8_t* blob1 = expert_blob(A.blobs, A.stride, table, s_ids[j0 + 1 < k ? j0 + 1 : j0]);
  struct Batch {
    uint32_t gw[UB][VG], uw[UB][VG];
    float gs[UB][SPG::NS], us[UB][SPG::NS];
  };
  // a wave with no units reads row 0 of the first expert and ignores it:
  // the first batch is requested unconditionally, so that later waits can
  // count the loads exactly
  auto issue_b = [&](Batch& B, int b0) {
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      const int ui = b0 + i < my_n ? b0 + i : my_n - 1;
      int rg = my_n > 0 ? rg0 + ui : 0;
      const bool second = rg >= upe;
      rg = second ? rg - upe : rg;
      const int row = rg * RPWG + rsg;
      const uint8_t* blob = second ? blob1 : blob0;
      load_row_words<VG, true>((const uint32_t*)(blob + A.gc) + (size_t)row * Wg, lrg, LPRG,
                               B.gw[i]);
      load_row_words<VG, true>((const uint32_t*)(blob + A.uc) + (size_t)row * Wg, lrg, LPRG,
                               B.uw[i]);
      load_row_scales<BITS, VG, ST, true>((const ST*)(blob + A.gs) + (size_t)row * Gg, sgg, Gg,
                                          B.gs[i]);
      load_row_scales<BITS, VG, ST, true>((const ST*)(blob + A.us) + (size_t)row * Gg, sgg, Gg,
                                          B.us[i]);
    }
  };
  Batch bA, bB;
  issue_b(bA, 0);

  // 4. while the first batch is in flight: the maximum and the sum of
  //    squares of x, then its fp16 activation pairs and offsets K, once per
  //    workgroup, into LDS
  {
    float amax = 0.f, ssq = 0.f;
#pragma unroll
    for (int t = 0; t < DEC_XW; ++t) {
      const int cw = tid + t * DEC_THREADS;
      if (t * DEC_THREADS < Wg) {
#pragma unroll
        for (int i = 0; i < WPW; ++i) {
          const float f = cw < Wg ? x_word_val<XF32>(xraw[t], i) : 0.f;
          amax = fmaxf(amax, fabsf(f));
          ssq = fmaf(f, f, ssq);
        }
      }
    }
    amax = lane63(seg_max(amax, 6));
    ssq = lane63(seg_sum(ssq, 6));
    if (lane == 0) {
      s_red[wave][0] = amax;
      s_red[wave][1] = ssq;
    }
  }
  __syncthreads();
  float S, xos;
  {
    float m = 0.f, q = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      m = fmaxf(m, s_red[w][0]);
      q += s_red[w][1];
    }
    S = pow2_prescale(m);
    const float r = A.rms ? 1.0f / sqrtf(q / (float)A.d + A.eps) : 1.0f;
    xos = r / (QT<BITS>::M * S);
  }
#pragma unroll
  for (int t = 0; t < DEC_XW; ++t) {
    const int cw = tid + t * DEC_THREADS;
    if (t * DEC_THREADS < Wg && cw < Wg) {
      // lane lr and slot w holding code word cw (inverse of LaneMap)
      constexpr int N4 = LaneMap<VG>::N4, RT = LaneMap<VG>::R;
      int lr, w;
      if (cw < 4 * N4 * LPRG) {
        const int c = cw / (4 * LPRG), rem = cw - c * 4 * LPRG;
        lr = rem >> 2;
        w = 4 * c + (rem & 3);
      } else {
        const int rem = cw - 4 * N4 * LPRG;
        lr = rem / (RT > 0 ? RT : 1);
        w = 4 * N4 + (rem - lr * (RT > 0 ? RT : 1));
      }
      float kk = 0.f;
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        const int hs = q / NPOS, pos = q % NPOS;
        const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
        const float f = S * (1.0f / (float)(1 << (BITS * pos)));
        const float a = x_word_val<XF32>(xraw[t], ia) * f, b = x_word_val<XF32>(xraw[t], ib) * f;
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        s_xp[(w * PPW + q) * LPRG + lr] = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
        float sumx = (float)ha + (float)hb;
        if constexpr (SPLIT) {
          const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
          s_xp[XP + (w * PPW + q) * LPRG + lr] = __builtin_bit_cast(uint32_t, f16x2{la, lb});
          sumx += (float)la + (float)lb;
        }
        kk = fmaf(sumx, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)), kk);
      }
      s_K[w * LPRG + lr] = kk;
    }
  }

  if (blockIdx.x == 0) {
    // softmax over all logits (only the publishing workgroup needs weights)
    const float mx = s_val[0];
    const float se = block_sum(tid < E ? expf(lv - mx) : 0.f, s_tmp);
    if (wave == 0) {
      const float p = lane < k ? expf(s_val[lane] - mx) / se : 0.f;
      const float psum = lane63(seg_sum(p, 6));
      if (lane < k) {
        const float w = A.norm ? p / psum : p;
        A.ws_ids[lane] = s_ids[lane];
        A.ws_w[lane] = w;
        if (A.user_ids) A.user_ids[lane] = s_ids[lane];
        if (A.user_w) A.user_w[lane] = w;
      }
    }
  }
  __syncthreads();
  XRegs<BITS, VG, SPLIT> X;
#pragma unroll
  for (int w = 0; w < VG; ++w) {
#pragma unroll
    for (int q = 0; q < PPW; ++q) {
      X.hi[w][q] = __builtin_bit_cast(f16x2, s_xp[(w * PPW + q) * LPRG + lrg]);
      if constexpr (SPLIT)
        X.lo[w][q] = __builtin_bit_cast(f16x2, s_xp[XP + (w * PPW + q) * LPRG + lrg]);
    }
    X.K[w] = s_K[w * LPRG + lrg];
  }
  X.oscale = xos;
  fold_k(X);

  // 5. gate/up dot products, SwiGLU, store h; the next batch's loads are
  //    issued before the current batch is computed
  auto compute_b = [&](const Batch& B, int b0) {
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      float ag = lane_row<BITS, VG, SPLIT>(B.gw[i], X, B.gs[i], tmg);
      float au = lane_row<BITS, VG, SPLIT>(B.uw[i], X, B.us[i], tmg);
      ag = seg_sum(ag, lgg);
      au = seg_sum(au, lgg);
      if (b0 + i < my_n && lrg == LPRG - 1) {
        int rg = rg0 + b0 + i;
        const bool second = rg >= upe;
        rg = second ? rg - upe : rg;
        const int j = second ? j0 + 1 : j0;
        const float g = ag * X.oscale, uu = au * X.oscale;
        A.h[(size_t)j * A.ffn + rg * RPWG + rsg] = g / (1.0f + expf(-g)) * uu;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int b0 = 0; b0 < my_n; b0 += 2 * UB) {
    if (b0 + UB < my_n) issue_b(bB, b0 + UB);
    compute_b(bA, b0);
    if (b0 + UB >= my_n) break;
    if (b0 + 2 * UB < my_n) issue_b(bA, b0 + 2 * UB);
    compute_b(bB, b0 + UB);
  }
}

// --------------------------------------------------------------------- K2 --

// K2 rows are spread over LPRD = 2^lg_d lanes (16 for the shapes built
// here), so one wave load covers 64 / LPRD rows and a row's partial sums
// meet in a short DPP reduction. Every lane of a row slot needs the same
// columns of h_j, so the wave turns h_j into fp16 pairs once, in LDS, in
// the lane-map order, and each lane reads its pairs from there.
template <int BITS, typename ST, int VD, bool TBL>
__global__ __launch_bounds__(DEC_THREADS, DEC_WAVES_PER_EU) void k_dec_down(DecodeArgs A) {
  constexpr int PPW = QT<BITS>::PPW;
  constexpr int WPW = QT<BITS>::WPW;
  constexpr int NPOS = QT<BITS>::NPOS;
  using SPD = ScalePlan<BITS, VD>;
  // row loads per batch, two batches in flight
  constexpr int UDr = 32 / (VD + SPD::NS);
  constexpr int UD = UDr < 1 ? 1 : (UDr > 4 ? 4 : UDr);

  __shared__ float s_part[SMOE_MAX_TOP_K * DEC_RB_MAX];
  __shared__ __attribute__((aligned(16))) uint32_t s_hp[DEC_WAVES][DEC_HP];
  __shared__ float s_hk[DEC_WAVES][DEC_HW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = A.k;
  // this workgroup's rows [r0, r0 + nrows); wave w takes expert slot w (and
  // w + 8 when k > 8) over every row of the block
  const int lgd = A.lg_d, LPRD = 1 << lgd, lrd = lane & (LPRD - 1), rsd = lane >> lgd;
  const int RPWD = 64 >> lgd;
  const int r0 = (int)blockIdx.x * A.rb;
  int nrows = A.d - r0;
  nrows = nrows < 0 ? 0 : (nrows > A.rb ? A.rb : nrows);
  const int upx = (nrows + RPWD - 1) / RPWD;  // row loads per expert
  const int Wd = A.ffn * BITS / 32, Gd = A.ffn / 64;
  int sgd[SPD::NS], tmd;
  scale_groups<BITS, VD>(lrd, LPRD, sgd, tmd);
  struct DBatch {
    uint32_t w[UD][VD];
    float s[UD][SPD::NS];
  };
  DBatch dA, dB;
  XRegs<BITS, VD, false> H;
  auto issue_d = [&](DBatch& D, int b0, const uint32_t* cbase, const ST* sbase) {
#pragma unroll
    for (int i = 0; i < UD; ++i) {
      const int ri = b0 + i < upx ? b0 + i : upx - 1;
      int row = r0 + ri * RPWD + rsd;
      row = row < A.d ? row : A.d - 1;
      load_row_words<VD, true>(cbase + (size_t)row * Wd, lrd, LPRD, D.w[i]);
      load_row_scales<BITS, VD, ST, true>(sbase + (size_t)row * Gd, sgd, Gd, D.s[i]);
    }
  };
  auto compute_d = [&](const DBatch& D, int b0, int j) {
#pragma unroll
    for (int i = 0; i < UD; ++i) {
      if (b0 + i < upx) {  // wave-uniform
        float a = lane_row<BITS, VD, false>(D.w[i], H, D.s[i], tmd);
        a = seg_sum(a, lgd);
        const int rl = (b0 + i) * RPWD + rsd;
        if (lrd == LPRD - 1 && rl < nrows) s_part[j * DEC_RB_MAX + rl] = a * H.oscale;
      }
    }
  };
  uint32_t* hp = s_hp[wave];
  float* hk = s_hk[wave];
#pragma unroll 1
  for (int j = wave; j < k && upx > 0; j += DEC_WAVES) {
    const int e = __builtin_amdgcn_readfirstlane(A.ws_ids[j]);
    const float wj = A.ws_w[j];
    // h_j, code word c = lane + 64 t of it per lane (coalesced), loaded
    // before the weights so that these loads retire first
    const float* hrow = A.h + (size_t)j * A.ffn;
    float hv[DEC_HC][WPW];
#pragma unroll
    for (int t = 0; t < DEC_HC; ++t) {
      const int c = lane + 64 * t;
      const float* src = hrow + (size_t)(c < Wd ? c : Wd - 1) * WPW;
#pragma unroll
      for (int i = 0; i < WPW / 4; ++i) {
        const f32x4 v = *(const f32x4*)(src + 4 * i);
        hv[t][4 * i] = v.x;
        hv[t][4 * i + 1] = v.y;
        hv[t][4 * i + 2] = v.z;
        hv[t][4 * i + 3] = v.w;
      }
    }
    const uint8_t* blob = expert_blob(A.blobs, A.stride, TBL ? A.table : nullptr, e);
    const uint32_t* cbase = (const uint32_t*)(blob + A.dc);
    const ST* sbase = (const ST*)(blob + A.ds);
    issue_d(dA, 0, cbase, sbase);
    if (UD < upx) issue_d(dB, UD, cbase, sbase);
    // fp16 pairs of h_j rescaled by a power of two (max over the vector),
    // stored at the lane-map slot of each code word with the word's offset
    float m = 0.f;
#pragma unroll
    for (int t = 0; t < DEC_HC; ++t)
      if (lane + 64 * t < Wd)
#pragma unroll
        for (int i = 0; i < WPW; ++i) m = fmaxf(m, fabsf(hv[t][i]));
    m = lane63(seg_max(m, 6));
    const float S = pow2_prescale(m);
    constexpr int N4 = LaneMap<VD>::N4, RT = LaneMap<VD>::R;
#pragma unroll
    for (int t = 0; t < DEC_HC; ++t) {
      const int c = lane + 64 * t;
      if (c < Wd) {
        int lr, sl;
        if (c < 4 * N4 * LPRD) {
          const int ch = c / (4 * LPRD), rem = c - ch * 4 * LPRD;
          lr = rem >> 2;
          sl = 4 * ch + (rem & 3);
        } else {
          const int rem = c - 4 * N4 * LPRD;
          lr = rem / (RT > 0 ? RT : 1);
          sl = 4 * N4 + (rem - lr * (RT > 0 ? RT : 1));
        }
        float kk = 0.f;
        uint32_t pw[PPW];
#pragma unroll
        for (int q = 0; q < PPW; ++q) {
          const int hs = q / NPOS, pos = q % NPOS;
          const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
          const float f = S * (1.0f / (float)(1 << (BITS * pos)));
          const _Float16 ha = (_Float16)(hv[t][ia] * f), hb = (_Float16)(hv[t][ib] * f);
          pw[q] = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
          kk = fmaf((float)ha + (float)hb, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)), kk);
        }
        uint32_t* dst = hp + (sl * LPRD + lr) * PPW;
#pragma unroll
        for (int q = 0; q < PPW; q += 4) *(u32x4*)(dst + q) = u32x4{pw[q], pw[q + 1], pw[q + 2], pw[q + 3]};
        hk[sl * LPRD + lr] = kk;
      }
    }
    // the wave's own LDS writes, read back by other lanes of the wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int w = 0; w < VD; ++w) {
      const uint32_t* src = hp + (w * LPRD + lrd) * PPW;
#pragma unroll
      for (int q = 0; q < PPW; q += 4) {
        const u32x4 v = *(const u32x4*)(src + q);
        // components to scalars before the bit casts (a bit cast of a
        // vector component reads the vector's first element)
        const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
        H.hi[w][q] = __builtin_bit_cast(f16x2, v0);
        H.hi[w][q + 1] = __builtin_bit_cast(f16x2, v1);
        H.hi[w][q + 2] = __builtin_bit_cast(f16x2, v2);
        H.hi[w][q + 3] = __builtin_bit_cast(f16x2, v3);
      }
      H.K[w] = hk[w * LPRD + lrd];
    }
    fold_k(H);
    H.oscale = wj / (QT<BITS>::M * S);
#pragma unroll 1
    for (int b0 = 0; b0 < upx; b0 += 2 * UD) {
      compute_d(dA, b0, j);
      if (b0 + UD >= upx) break;
      if (b0 + 2 * UD < upx) issue_d(dA, b0 + 2 * UD, cbase, sbase);
      compute_d(dB, b0 + UD, j);
      if (b0 + 3 * UD < upx) issue_d(dB, b0 + 3 * UD, cbase, sbase);
    }
    // the next expert slot of this wave rewrites the LDS pairs
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (tid < nrows) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc += s_part[j * DEC_RB_MAX + tid];
    float* dst = A.out + r0 + tid;
    *dst = A.accumulate ? *dst + acc : acc;
  }
}

template <int BITS, typename ST, int VG, bool XF32>
hipError_t launch_dec_gate_up(const DecodeArgs& A, int nwg, hipStream_t s) {
  if (A.table)
    return launch_kernel(k_dec_gate_up<BITS, ST, VG, XF32, true>, dim3(nwg), dim3(DEC_THREADS), s,
                         A);
  return launch_kernel(k_dec_gate_up<BITS, ST, VG, XF32, false>, dim3(nwg), dim3(DEC_THREADS), s,
                       A);
}

template <int BITS, typename ST, int VD>
hipError_t launch_dec_down(const DecodeArgs& A, int nwg, hipStream_t s) {
  if (A.table)
    return launch_kernel(k_dec_down<BITS, ST, VD, true>, dim3(nwg), dim3(DEC_THREADS), s, A);
  return launch_kernel(k_dec_down<BITS, ST, VD, false>, dim3(nwg), dim3(DEC_THREADS), s, A);
}

}  // namespace smoe
