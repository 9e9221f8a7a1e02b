// Small batches on gfx950, the one-token design extended to a few tokens:
// routing, grouping and the gate/up stage in one launch (2..4 tokens, or one
// token with a shared expert), and the down stage with the combine in one
// launch (up to 16 tokens).
//
// Every workgroup routes all T tokens itself ("CMF v2 Format Specification",
// 2.2 MoE: top-k of the logits, equal logits to the lower expert id,
// softmax-over-all weights, renormalised on request) by counting, for each
// (token, expert), the token's logits above its own; it then groups the
// selections by expert in LDS (a token bitmask per expert, a scan over the
// experts) in the grouped layout the down stage and the combine read: active
// experts ascending, inside an expert the tokens ascending, the shared
// expert's parts after the routed pairs (pair P + v T + t). Workgroup 0
// publishes that layout. The gate/up rows of every active expert (and of the
// shared expert's parts) are then split evenly over all waves, each row read
// once and dotted with every token that selected the expert, from fp16
// activation pairs built once per workgroup in LDS; SwiGLU is fused and h is
// stored per grouped pair.

#pragma once

#include "smoe_decode.hpp"
#include "smoe_small_args.hpp"

namespace smoe {

// Four waves per SIMD (two workgroups per CU, 128 registers) when a lane
// holds at most 16 activation pairs of a token and the input is bf16; else two.
template <int BITS, int VG, bool XF32>
constexpr bool sb_narrow() {
  return !XF32 && VG * QT<BITS>::PPW <= 16;
}

// A lane's code words as fp16 pairs (1024 + code, or 1024 + 2^(b pos) code
// at the higher positions), decoded once and dotted with several tokens.
template <int BITS, int V>
__device__ __forceinline__ void decode_words(const uint32_t (&cw)[V],
                                             uint32_t (&d)[V][QT<BITS>::PPW]) {
  constexpr int NPOS = QT<BITS>::NPOS;
#pragma unroll
  for (int w = 0; w < V; ++w)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const uint32_t v = hs ? (cw[w] >> 8) : cw[w];
#pragma unroll
      for (int pos = 0; pos < NPOS; ++pos) {
        constexpr uint32_t base = (1u << BITS) - 1u;
        const uint32_t m = (base << (BITS * pos)) | (base << (BITS * pos + 16));
        d[w][hs * NPOS + pos] = and_or(v, m, 0x64006400u);
      }
    }
}

// lane_row over decoded words: sum over the lane's words of
// scale(word) * (dot - K), for one row (K folded).
template <int BITS, int V, bool SPLIT>
__device__ __forceinline__ float lane_row_dec(const uint32_t (&d)[V][QT<BITS>::PPW],
                                              const XRegs<BITS, V, SPLIT>& X,
                                              const float (&s)[ScalePlan<BITS, V>::NS],
                                              int tmask) {
  using SP = ScalePlan<BITS, V>;
  constexpr int PPW = QT<BITS>::PPW;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < SP::N4; ++c) {
    float a = -X.K[c];
#pragma unroll
    for (int w = 4 * c; w < 4 * c + 4; ++w)
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        a = fdot2(d[w][q], X.hi[w][q], a);
        if constexpr (SPLIT) a = fdot2(d[w][q], X.lo[w][q], a);
      }
    acc = fmaf(a, s[c], acc);
  }
  if constexpr (SP::R > 0) {
    // the tail's scale(s) as opaque register values, so the per-word choice
    // stays a register select (not an indexed load from a stack copy)
    float t0 = s[SP::N4], t1 = s[SP::NS - 1];
    asm volatile("" : "+v"(t0), "+v"(t1));
#pragma unroll
    for (int t = 0; t < SP::R; ++t) {
      const int w = 4 * SP::N4 + t;
      float a = -X.K[SP::N4 + t];
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        a = fdot2(d[w][q], X.hi[w][q], a);
        if constexpr (SPLIT) a = fdot2(d[w][q], X.lo[w][q], a);
      }
      const float sc = (SP::NT == 2 && ((tmask >> t) & 1)) ? t1 : t0;
      acc = fmaf(a, sc, acc);
    }
  }
  return acc;
}

// tokens per wave when building the activation pairs (wave w takes w, w + 8, ...)
constexpr int SB_XSLOTS = (SB_TMAX + DEC_WAVES - 1) / DEC_WAVES;

template <int BITS, typename ST, int VG, bool XF32>
__global__ __launch_bounds__(DEC_THREADS, (sb_narrow<BITS, VG, XF32>() ? DEC_GU_WAVES_PER_EU
                                                                       : DEC_WAVES_PER_EU)) void
k_sb_gate_up(SmallArgs A) {
  constexpr int PPW = QT<BITS>::PPW;
  constexpr int WPW = QT<BITS>::WPW;
  constexpr int NPOS = QT<BITS>::NPOS;
  constexpr bool SPLIT = XF32;
  using SPG = ScalePlan<BITS, VG>;
  constexpr int UBr = (SPLIT ? 36 : 24) / (2 * (VG + SPG::NS));
  constexpr int UB = UBr < 1 ? 1 : (UBr > 2 ? 2 : UBr);  // row pairs per batch
  constexpr int XRAW = XF32 ? WPW : WPW / 2;             // 32-bit words of x per code word
  constexpr int XPT = VG * PPW * 64;                     // fp16-pair words of one token

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint64_t* s_key = (uint64_t*)smem;                      // [T * E]
  float* s_lv = (float*)(smem + A.lds_lv);                // [T * E]
  uint32_t* s_xp = (uint32_t*)(smem + A.lds_xp);          // [T][(SPLIT ? 2 : 1) * XPT]
  float* s_K = (float*)(smem + A.lds_k);                  // [T][VG * 64]
  float* s_os = (float*)(smem + A.lds_os);                // [T]
  __shared__ uint32_t s_mask[SMOE_MAX_EXPERTS];           // tokens that selected expert e
  __shared__ int s_slot[SMOE_MAX_EXPERTS];                // slot of expert e
  __shared__ int s_act[SMOE_MAX_EXPERTS];                 // expert of slot s
  __shared__ int s_off[SMOE_MAX_EXPERTS + 1];             // first grouped pair of slot s
  __shared__ int s_sel[SB_TSLOTS * SMOE_MAX_TOP_K];         // selection j of token t
  __shared__ float s_val[SB_TSLOTS * SMOE_MAX_TOP_K];       // its logit
  __shared__ int s_scan[DEC_WAVES];
  __shared__ int s_nact;
  __shared__ float s_hout[DEC_WAVES][64];                 // a unit's results before the store

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = A.T, E = A.E, k = A.k, nsh = A.nsh;
  const int TE = T * E, P = T * k;

  // 1. routing keys: (token, expert) -> key ordering larger logits first,
  //    equal logits by ascending expert id
  for (int i = tid; i < TE; i += DEC_THREADS) {
    float f = A.logits[i];
    if (f != f) f = -INFINITY;  // NaN never outranks a number
    s_lv[i] = f;
    s_key[i] = route_key(f, i % E);
  }
  for (int e = tid; e < E; e += DEC_THREADS) s_mask[e] = 0u;
  __syncthreads();

  // 2. rank of each (token, expert) among the token's keys; the k lowest are
  //    its selection
  for (int i = tid; i < TE; i += DEC_THREADS) {
    const int t = i / E, e = i - t * E;
    const uint64_t ki = s_key[i];
    const uint64_t* row = s_key + (size_t)t * E;
    int cnt = 0;
    for (int j = 0; j < E; ++j) cnt += (int)(row[j] > ki);
    if (cnt < k) {
      s_sel[t * k + cnt] = e;
      s_val[t * k + cnt] = s_lv[i];
      atomicOr(&s_mask[e], 1u << t);
    }
  }
  __syncthreads();

  // 3. grouping: a scan over the experts of (active, tokens) gives each
  //    active expert its slot and its first grouped pair
  {
    int na = 0, np = 0;  // running totals over earlier blocks of 512 experts
    for (int base = 0; base < E; base += DEC_THREADS) {
      const int e = base + tid;
      const uint32_t m = e < E ? s_mask[e] : 0u;
      const int v = m ? (1 << 16) + __popc(m) : 0;  // active count | pair count
      int x = v;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane == 63) s_scan[wave] = x;
      __syncthreads();
      int pre = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < DEC_WAVES; ++w) {
        const int sw = s_scan[w];
        pre += w < wave ? sw : 0;
        tot += sw;
      }
      const int excl = pre + x - v;
      if (m) {
        const int s = na + (excl >> 16);
        s_slot[e] = s;
        s_act[s] = e;
        s_off[s] = np + (excl & 0xFFFF);
      }
      na += tot >> 16;
      np += tot & 0xFFFF;
      __syncthreads();
    }
    if (tid == 0) s_nact = na;
  }
  __syncthreads();
  const int nact = s_nact;
  // the selection, the weights and the grouped layout, published by
  // workgroup 0 (wave w takes token w)
  auto publish = [&]() {
    for (int t = wave; t < T; t += DEC_WAVES) {
      const float mx = s_val[t * k];
      float se = 0.f;
      for (int e = lane; e < E; e += 64) se += expf(s_lv[t * E + e] - mx);
      se = lane63(seg_sum(se, 6));
      const float p = lane < k ? expf(s_val[t * k + (lane < k ? lane : 0)] - mx) / se : 0.f;
      const float psum = lane63(seg_sum(p, 6));
      if (lane < k) {
        const int e = s_sel[t * k + lane];
        const float wt = A.norm ? p / psum : p;
        const int o = t * k + lane;
        const int pos = s_off[s_slot[e]] + __popc(s_mask[e] & ((1u << t) - 1u));
        A.ids[o] = e;
        A.w[o] = wt;
        A.pair_of[o] = pos;
        A.pair_token[pos] = t;
        if (A.user_ids) A.user_ids[o] = e;
        if (A.user_w) A.user_w[o] = wt;
      }
    }
    for (int s = tid; s < nact; s += DEC_THREADS) {
      A.active[s] = s_act[s];
      A.offs[s] = s_off[s];
    }
    for (int v = tid; v <= nsh; v += DEC_THREADS) A.offs[nact + v] = P + v * T;
    for (int i = tid; i < nsh * T; i += DEC_THREADS) A.pair_token[P + i] = i % T;
    if (tid == 0) {
      A.meta[0] = nact;
      A.meta[1] = P;
    }
  };
  // routing and grouping only (one workgroup, ahead of the grouped stages)
  if (A.route_only) {
    publish();
    return;
  }

  // 4. this wave's units: (slot, row group) over the shared expert's parts
  //    first (all T tokens each), then the active experts, split evenly over
  //    all waves; a wave's units span at most two slots
  const int lgg = A.lg_g, LPRG = 1 << lgg, lrg = lane & (LPRG - 1), rsg = lane >> lgg;
  const int RPWG = 64 >> lgg;
  const int upe = A.ffn / RPWG;
  const int nq = nsh + nact;
  const int units = nq * upe;
  const int TW = (int)gridDim.x * DEC_WAVES, gw = (int)blockIdx.x * DEC_WAVES + wave;
  const int ub = units / TW, urem = units % TW;
  const int my_n = ub + (gw < urem ? 1 : 0);
  const int u0 = gw * ub + (gw < urem ? gw : urem);
  const int q0 = my_n > 0 ? u0 / upe : 0;
  const int rg0 = u0 - q0 * upe;
  const int Wg = A.d * BITS / 32, Gg = A.d / 64;
  int sgg[SPG::NS], tmg;
  scale_groups<BITS, VG>(lrg, LPRG, sgg, tmg);
  // unit q: its matrices' first row, its tokens and its first grouped pair
  struct Unit {
    const uint32_t *gc, *uc;
    const ST *gs, *us;
    uint32_t tm;
    int pb;
  };
  auto unit = [&](int q) {
    Unit U;
    const uint8_t* b;
    uint64_t row0;
    if (q < nsh) {
      b = A.shared;
      row0 = (uint64_t)q * A.ffn;
      U.gc = (const uint32_t*)(b + A.sgc) + row0 * Wg;
      U.uc = (const uint32_t*)(b + A.suc) + row0 * Wg;
      U.gs = (const ST*)(b + A.sgs) + row0 * Gg;
      U.us = (const ST*)(b + A.sus) + row0 * Gg;
      U.tm = T >= 32 ? 0xFFFFFFFFu : (1u << T) - 1u;
      U.pb = P + q * T;
    } else {
      const int s = q - nsh < nact ? q - nsh : 0;
      b = expert_blob(A.blobs, A.stride, A.table, s_act[s]);
      U.gc = (const uint32_t*)(b + A.gc);
      U.uc = (const uint32_t*)(b + A.uc);
      U.gs = (const ST*)(b + A.gs);
      U.us = (const ST*)(b + A.us);
      U.tm = s_mask[s_act[s]];
      U.pb = s_off[s];
    }
    return U;
  };
  const Unit U0 = unit(q0);
  const Unit U1 = unit(q0 + 1 < nq ? q0 + 1 : q0);
  struct Batch {
    uint32_t gw[UB][VG], uw[UB][VG];
    float gs[UB][SPG::NS], us[UB][SPG::NS];
  };
  // a wave with no units reads row 0 of its first unit and ignores it: the
  // first batch is requested unconditionally, so that later waits count the
  // loads exactly
  auto issue_b = [&](Batch& B, int b0) {
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      const int ui = b0 + i < my_n ? b0 + i : my_n - 1;
      int rg = my_n > 0 ? rg0 + ui : 0;
      const bool second = rg >= upe;
      rg = second ? rg - upe : rg;
      const int row = rg * RPWG + rsg;
      const Unit& Uu = second ? U1 : U0;
      load_row_words<VG, true>(Uu.gc + (size_t)row * Wg, lrg, LPRG, B.gw[i]);
      load_row_words<VG, true>(Uu.uc + (size_t)row * Wg, lrg, LPRG, B.uw[i]);
      load_row_scales<BITS, VG, ST, true>(Uu.gs + (size_t)row * Gg, sgg, Gg, B.gs[i]);
      load_row_scales<BITS, VG, ST, true>(Uu.us + (size_t)row * Gg, sgg, Gg, B.us[i]);
    }
  };
  // the x words of this wave's token (wave w takes token w), requested before the
  // weights so that they retire first; the loads are unconditional (a
  // missing token reads the last one, a missing word the row's last)
  uint32_t xr[SB_XSLOTS][VG][XRAW];
#pragma unroll
  for (int tt = 0; tt < SB_XSLOTS; ++tt) {
    const int tr = wave + tt * DEC_WAVES;
    const uint32_t* xt = (const uint32_t*)A.x + (size_t)(tr < T ? tr : T - 1) * Wg * XRAW;
#pragma unroll
    for (int i = 0; i < VG; ++i) {
      const int cw = lane + 64 * i;
      const uint32_t* src = xt + (size_t)(cw < Wg ? cw : Wg - 1) * XRAW;
#pragma unroll
      for (int c = 0; c < XRAW / 4; ++c) {
        const u32x4 v = *(const u32x4*)(src + 4 * c);
        xr[tt][i][4 * c] = v.x;
        xr[tt][i][4 * c + 1] = v.y;
        xr[tt][i][4 * c + 2] = v.z;
        xr[tt][i][4 * c + 3] = v.w;
      }
    }
  }
  Batch bA, bB;
  issue_b(bA, 0);

  // 5. workgroup 0 publishes the selection, the weights and the grouped
  //    layout
  if (blockIdx.x == 0) publish();

  // 6. fp16 activation pairs and offsets K of every token, built once per
  //    workgroup in LDS from the words loaded in step 4 (wave w takes token w)
#pragma unroll
  for (int tt = 0; tt < SB_XSLOTS; ++tt) {
    const int tr = wave + tt * DEC_WAVES;
    const int t = tr < T ? tr : T - 1;
    if (tr < T) {  // wave-uniform
      float amax = 0.f, ssq = 0.f;
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        if (lane + 64 * i < Wg) {
#pragma unroll
          for (int j = 0; j < WPW; ++j) {
            const float f = x_word_val<XF32>(xr[tt][i], j);
            amax = fmaxf(amax, fabsf(f));
            ssq = fmaf(f, f, ssq);
          }
        }
      }
      amax = lane63(seg_max(amax, 6));
      ssq = lane63(seg_sum(ssq, 6));
      const float S = pow2_prescale(amax);
      const float rr = A.rms ? 1.0f / sqrtf(ssq / (float)A.d + A.eps) : 1.0f;
      if (lane == 0) s_os[t] = rr / (QT<BITS>::M * S);
      uint32_t* xp = s_xp + (size_t)t * (SPLIT ? 2 : 1) * XPT;
      float* kt = s_K + (size_t)t * VG * 64;
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const int cw = lane + 64 * i;
        if (cw < Wg) {
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
          uint32_t ph[PPW], pl[PPW];
#pragma unroll
          for (int q = 0; q < PPW; ++q) {
            const int hs = q / NPOS, pos = q % NPOS;
            const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
            const float f = S * (1.0f / (float)(1 << (BITS * pos)));
            const float a = x_word_val<XF32>(xr[tt][i], ia) * f;
            const float b = x_word_val<XF32>(xr[tt][i], ib) * f;
            const _Float16 ha = (_Float16)a, hb = (_Float16)b;
            ph[q] = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
            float sumx = (float)ha + (float)hb;
            if constexpr (SPLIT) {
              const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
              pl[q] = __builtin_bit_cast(uint32_t, f16x2{la, lb});
              sumx += (float)la + (float)lb;
            } else {
              pl[q] = 0u;
            }
            kk = fmaf(sumx, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)), kk);
          }
          uint32_t* dst = xp + (w * LPRG + lr) * PPW;
#pragma unroll
          for (int q = 0; q < PPW; q += 4) {
            *(u32x4*)(dst + q) = u32x4{ph[q], ph[q + 1], ph[q + 2], ph[q + 3]};
            if constexpr (SPLIT)
              *(u32x4*)(dst + XPT + q) = u32x4{pl[q], pl[q + 1], pl[q + 2], pl[q + 3]};
          }
          kt[w * LPRG + lr] = kk;
        }
      }
    }
  }
  __syncthreads();

  // 7. gate/up dot products for every token of a unit, SwiGLU, h per pair;
  //    the next batch's loads are issued before the current batch is computed
  auto load_x = [&](int t, XRegs<BITS, VG, SPLIT>& X) {
    const uint32_t* xp = s_xp + (size_t)t * (SPLIT ? 2 : 1) * XPT;
#pragma unroll
    for (int w = 0; w < VG; ++w) {
#pragma unroll
      for (int q = 0; q < PPW; q += 4) {
        const u32x4 v = *(const u32x4*)(xp + (w * LPRG + lrg) * PPW + q);
        // components to scalars before the bit casts (a bit cast of a
        // vector component reads the vector's first element)
        const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
        X.hi[w][q] = __builtin_bit_cast(f16x2, v0);
        X.hi[w][q + 1] = __builtin_bit_cast(f16x2, v1);
        X.hi[w][q + 2] = __builtin_bit_cast(f16x2, v2);
        X.hi[w][q + 3] = __builtin_bit_cast(f16x2, v3);
        if constexpr (SPLIT) {
          const u32x4 l = *(const u32x4*)(xp + XPT + (w * LPRG + lrg) * PPW + q);
          const uint32_t l0 = l.x, l1 = l.y, l2 = l.z, l3 = l.w;
          X.lo[w][q] = __builtin_bit_cast(f16x2, l0);
          X.lo[w][q + 1] = __builtin_bit_cast(f16x2, l1);
          X.lo[w][q + 2] = __builtin_bit_cast(f16x2, l2);
          X.lo[w][q + 3] = __builtin_bit_cast(f16x2, l3);
        }
      }
      X.K[w] = s_K[(size_t)t * VG * 64 + w * LPRG + lrg];
    }
    X.oscale = s_os[t];
    fold_k(X);
  };
  auto compute_b = [&](const Batch& B, int b0) {
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      int rg = rg0 + b0 + i;
      const bool second = rg >= upe;
      rg = second ? rg - upe : rg;
      const Unit& Uu = second ? U1 : U0;
      uint32_t m = b0 + i < my_n ? Uu.tm : 0u;  // wave-uniform
      // the results go to LDS inside the token loop and to h in one store
      // after it: a global store inside a loop of unknown trip count would
      // make the compiler wait for every outstanding load (the next batch
      // included) before the loop
      int rank = 0;
      // the row's words decoded once for all of its tokens (with two waves
      // per SIMD; at four the registers do not hold them)
      constexpr bool DEC1 = !sb_narrow<BITS, VG, XF32>();
      uint32_t dg[DEC1 ? VG : 1][PPW], du[DEC1 ? VG : 1][PPW];
      if constexpr (DEC1) {
        decode_words<BITS, VG>(B.gw[i], dg);
        decode_words<BITS, VG>(B.uw[i], du);
      }
      while (m) {
        const int t = __builtin_ctz(m);
        m &= m - 1u;
        XRegs<BITS, VG, SPLIT> X;
        load_x(t, X);
        float ag, au;
        if constexpr (DEC1) {
          ag = lane_row_dec<BITS, VG, SPLIT>(dg, X, B.gs[i], tmg);
          au = lane_row_dec<BITS, VG, SPLIT>(du, X, B.us[i], tmg);
        } else {
          ag = lane_row<BITS, VG, SPLIT>(B.gw[i], X, B.gs[i], tmg);
          au = lane_row<BITS, VG, SPLIT>(B.uw[i], X, B.us[i], tmg);
        }
        ag = seg_sum(ag, lgg);
        au = seg_sum(au, lgg);
        if (lrg == LPRG - 1) {
          const float g = ag * X.oscale, uu = au * X.oscale;
          s_hout[wave][rank * RPWG + rsg] = g / (1.0f + expf(-g)) * uu;
        }
        ++rank;
      }
      if (lane < rank * RPWG)
        A.h[(size_t)(Uu.pb + lane / RPWG) * A.ffn + rg * RPWG + lane % RPWG] = s_hout[wave][lane];
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

// nwg: DEC_NWG_GU when the caller's LDS budget allows two workgroups per CU
// (reduced to DEC_NWG for the instantiations built for one)
template <int BITS, typename ST, int VG, bool XF32>
hipError_t launch_sb_gate_up(const SmallArgs& A, int nwg, hipStream_t s) {
  if (!sb_narrow<BITS, VG, XF32>() && !A.route_only) nwg = DEC_NWG;
  auto kernel = k_sb_gate_up<BITS, ST, VG, XF32>;
  if (A.lds_total > 65536) {  // workgroups of more than 64 KB of LDS need the limit raised
    const hipError_t e = hipFuncSetAttribute(
        (const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, A.lds_total);
    if (e != hipSuccess) return e;
  }
  return launch_kernel_lds(kernel, dim3(nwg), dim3(DEC_THREADS), (unsigned)A.lds_total, s, A);
}


// k_sb_down: the down projection of every grouped pair and the weighted
// combine of a small batch in one launch. Workgroup w owns output rows
// [w rb, (w + 1) rb) of every token. Every wave first requests the grouped
// layout and the h of its pairs (pairs j, j + 8, ... of the grouped order),
// then the rows of its first batch; it turns its pairs' h into fp16 pairs
// scaled by a power of two (as the one-token down stage does), all of them
// held in LDS. The units (the active experts, then the shared expert's
// parts: the grouped pairs in order) are split into eight contiguous ranges
// of about equal pairs plus units, one per wave; a unit's rows (16 lanes per
// row, four rows per wave load) go in batches of two loads with the next
// batch requested before the current one is computed, and weight x row is
// added into the wave's per-token accumulators for each pair of the unit.
// The accumulators of the eight waves are added in wave order and written
// (or added to the residual stream).
// one thread per grouped pair and per expert when the layout is staged
static_assert(SB_PAIRS <= DEC_THREADS && SMOE_MAX_EXPERTS <= DEC_THREADS, "k_sb_down staging");

// TBL: experts addressed through A.table (host offload), a template
// parameter so that the resident-bank kernel has no conditional load (which
// would make every wait on an earlier load wait for the row loads too).
template <int BITS, typename ST, int VD, bool TBL>
__global__ __launch_bounds__(DEC_THREADS, DEC_WAVES_PER_EU) void k_sb_down(SmallDownArgs A) {
  constexpr int PPW = QT<BITS>::PPW;
  constexpr int WPW = QT<BITS>::WPW;
  constexpr int NPOS = QT<BITS>::NPOS;
  using SPD = ScalePlan<BITS, VD>;
  constexpr int UB = VD > (BITS == 2 ? 8 : 12) ? 1 : 2;  // row loads per lane per batch
  // pairs whose h a wave requests at once (all of a wave's pairs when there
  // are at most 32 of them: their loads then go out before the rows')
  constexpr int HB = 4;
  // h code words per lane (Q2 rows of h hold at most 128 words: the LDS
  // region of one pair)
  constexpr int HC = BITS == 2 ? DEC_HC / 2 : DEC_HC;
  constexpr int N4 = LaneMap<VD>::N4, RT = LaneMap<VD>::R;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float s_acc[DEC_WAVES][SB_TSLOTS * SB_DOWN_RB];
  __shared__ float s_os[SB_PAIRS + 1];         // weight / (M S) of each grouped pair, a spare
  __shared__ int s_pt[DEC_THREADS];            // token of each grouped pair
  __shared__ int s_act[DEC_THREADS];           // expert of each active slot
  __shared__ int s_off[2 * DEC_THREADS];       // first pair of each unit, then the pair count
  uint32_t* s_hp = (uint32_t*)smem;            // [pairs][Wd * PPW] fp16 pairs, lane-map order
  float* s_hk = (float*)(smem + A.lds_hk);     // [pairs][Wd] their offsets

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = A.T, nsh = A.nsh, P = T * A.k, NP = P + nsh * T;
  const int Wd = A.ffn * BITS / 32, Gd = A.ffn / 64, HPS = Wd * PPW;
  const int lgd = A.lg_d, LPRD = 1 << lgd, lrd = lane & (LPRD - 1), rsd = lane >> lgd;
  const int RPWD = 64 >> lgd;
  // h of HB pairs, code word c = lane + 64 j per lane (coalesced)
  float hv[HB][HC][WPW];
  // (a request past the wave's pairs reads one address in every lane: it
  // keeps the count of loads in flight fixed and costs one cache line)
  auto load_h = [&](int r, int p, bool real) {
    const float* hrow = A.h + (size_t)p * A.ffn;
#pragma unroll
    for (int j = 0; j < HC; ++j) {
      const int c = real ? lane + 64 * j : 0;
      const float* src = hrow + (size_t)(c < Wd ? c : Wd - 1) * WPW;
#pragma unroll
      for (int i = 0; i < WPW / 4; ++i) {
        const f32x4 v = *(const f32x4*)(src + 4 * i);
        hv[r][j][4 * i] = v.x;
        hv[r][j][4 * i + 1] = v.y;
        hv[r][j][4 * i + 2] = v.z;
        hv[r][j][4 * i + 3] = v.w;
      }
    }
  };
  // pair p's h (in hv[r]) as fp16 pairs under a power of two, with the
  // offsets, at the lane-map slot of each code word
  // the lane-map slot (row word w, lane lr of the row) of this lane's code
  // words c = lane + 64 j of h, -1 past the row
  int hslot[HC];
#pragma unroll
  for (int j = 0; j < HC; ++j) {
    const int c = lane + 64 * j;
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
    hslot[j] = c < Wd ? sl * LPRD + lr : -1;
  }
  auto convert = [&](int r, int p) {
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < HC; ++j)
      if (lane + 64 * j < Wd)
#pragma unroll
        for (int i = 0; i < WPW; ++i) m = fmaxf(m, fabsf(hv[r][j][i]));
    m = lane63(seg_max(m, 6));
    const float S = pow2_prescale(m);
    uint32_t* hp = s_hp + (size_t)p * HPS;
    float* hk = s_hk + (size_t)p * Wd;
#pragma unroll
    for (int j = 0; j < HC; ++j) {
      if (hslot[j] >= 0) {
        float kk = 0.f;
        uint32_t pw[PPW];
#pragma unroll
        for (int qq = 0; qq < PPW; ++qq) {
          const int hs = qq / NPOS, pos = qq % NPOS;
          const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
          const float f = S * (1.0f / (float)(1 << (BITS * pos)));
          const _Float16 ha = (_Float16)(hv[r][j][ia] * f), hb = (_Float16)(hv[r][j][ib] * f);
          pw[qq] = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
          kk = fmaf((float)ha + (float)hb, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)),
                    kk);
        }
        uint32_t* dst = hp + hslot[j] * PPW;
#pragma unroll
        for (int qq = 0; qq < PPW; qq += 4)
          *(u32x4*)(dst + qq) = u32x4{pw[qq], pw[qq + 1], pw[qq + 2], pw[qq + 3]};
        hk[hslot[j]] = kk;
      }
    }
    if (lane == 0) s_os[p] = s_os[p] / (QT<BITS>::M * S);
  };

  // this wave's pairs: wave, wave + 8, ... (requests past the last one
  // repeat it, so that the number of loads in flight is the same on every
  // path and the waits count them exactly)
  const int npw = wave < NP ? (NP - wave + DEC_WAVES - 1) / DEC_WAVES : 0;
  auto pair_of_wave = [&](int i) {
    i = i < npw ? i : npw - 1;
    return i >= 0 ? wave + i * DEC_WAVES : 0;
  };
  // 1. the grouped layout (loads clamped to the buffers' sizes), then the h
  //    of the wave's first HB pairs; the layout goes to LDS once it arrives
  const int nact = A.meta[0], nq = nact + nsh;
  const int a_act = A.active[tid < A.E ? tid : A.E - 1];
  const int a_off0 = A.offs[tid <= A.E + nsh ? tid : A.E + nsh];
  const int a_off1 = A.offs[tid + DEC_THREADS <= A.E + nsh ? tid + DEC_THREADS : A.E + nsh];
  const int a_pt = A.pair_token[tid < NP ? tid : NP - 1];
  const int a_po = A.pair_of[tid < P ? tid : P - 1];
  const float a_w = A.w[tid < P ? tid : P - 1];
  if (npw <= 1) {  // wave-uniform: one pair (or none) takes one pair's loads
    load_h(0, pair_of_wave(0), true);
  } else {
#pragma unroll
    for (int r = 0; r < HB; ++r) load_h(r, pair_of_wave(r), r < npw);
  }
  // stores without conditions, so that the compiler keeps every load before
  // the h loads (a load moved under a condition would be waited for with
  // all the loads in flight); entries past the layout's are never read
  s_act[tid] = a_act;
  s_off[tid] = a_off0;
  s_off[tid + DEC_THREADS] = a_off1;
  s_pt[tid] = a_pt;
  // pair weights at the grouped position, the shared expert's parts 1
  s_os[tid < P ? a_po : (tid < NP ? tid : SB_PAIRS)] = tid < P ? a_w : 1.0f;
  for (int i = lane; i < SB_TSLOTS * SB_DOWN_RB; i += 64) s_acc[wave][i] = 0.f;
  __syncthreads();


  const int r0 = (int)blockIdx.x * A.rb;
  int nrows = A.d - r0;
  nrows = nrows < 0 ? 0 : (nrows > A.rb ? A.rb : nrows);
  const int upx = (nrows + RPWD - 1) / RPWD;  // row loads per unit, 1..sb_down_loads(VD)
  const int nb = (upx + UB - 1) / UB;         // batches per unit
  // this wave's units: a contiguous range, the units split so that each wave
  // gets about the same count of pairs plus units (unit u starts at
  // s_off[u] + u of NP + nq; wave w takes the units starting in
  // [w (NP + nq) / 8, (w + 1) (NP + nq) / 8))
  const int cost = NP + nq;
  auto first_unit = [&](int w) {  // the first unit whose start is >= w cost / 8
    int lo = 0, hi = nq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((s_off[mid] + mid) * DEC_WAVES >= w * cost) hi = mid;
      else lo = mid + 1;
    }
    return lo;
  };
  const int u0 = first_unit(wave), u1 = first_unit(wave + 1);
  const int nbt = (u1 - u0) * nb;  // this wave's batches, nb per unit
  int sgd[SPD::NS], tmd;
  scale_groups<BITS, VD>(lrd, LPRD, sgd, tmd);

  struct DB {
    uint32_t w[UB][VD];
    float s[UB][SPD::NS];
  };
  // the rows of batch b of the wave (a wave past its last batch requests the
  // last one again, so that the number of loads in flight is the same on
  // every path and the waits count them exactly)
  auto issue = [&](DB& D, int b) {
    b = b < nbt ? b : (nbt > 0 ? nbt - 1 : 0);
    int q = u0 + b / nb;
    const int i0 = (b % nb) * UB;
    q = q < nq ? q : nq - 1;
    const uint32_t* cbase;
    const ST* sbase;
    int cpitch, spitch;
    if (q >= nact) {  // part v of the shared expert: columns [v ffn, (v + 1) ffn)
      const int v = q - nact;
      cbase = (const uint32_t*)(A.shared + A.sdc) + (size_t)v * Wd;
      sbase = (const ST*)(A.shared + A.sds) + (size_t)v * Gd;
      cpitch = nsh * Wd;
      spitch = nsh * Gd;
    } else {
      const uint8_t* blob = expert_blob(A.blobs, A.stride, TBL ? A.table : nullptr, s_act[q]);
      cbase = (const uint32_t*)(blob + A.dc);
      sbase = (const ST*)(blob + A.ds);
      cpitch = Wd;
      spitch = Gd;
    }
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      const int ri = i0 + i < upx ? i0 + i : upx - 1;
      int row = r0 + ri * RPWD + rsd;
      row = row < A.d ? row : A.d - 1;
      load_row_words<VD, true>(cbase + (size_t)row * cpitch, lrd, LPRD, D.w[i]);
      load_row_scales<BITS, VD, ST, true>(sbase + (size_t)row * spitch, sgd, Gd, D.s[i]);
    }
  };
  // batch b's rows against the pairs of its unit, into the wave's accumulators
  auto compute = [&](const DB& D, int b) {
    const int q = u0 + b / nb;
    const int i0 = (b % nb) * UB;
    const int p0 = s_off[q], p1 = s_off[q + 1];
#pragma unroll 1
    for (int p = p0; p < p1; ++p) {
      XRegs<BITS, VD, false> H;
      const uint32_t* hp = s_hp + (size_t)p * HPS;
#pragma unroll
      for (int w = 0; w < VD; ++w) {
        const uint32_t* src = hp + (w * LPRD + lrd) * PPW;
#pragma unroll
        for (int qq = 0; qq < PPW; qq += 4) {
          const u32x4 v = *(const u32x4*)(src + qq);
          // components to scalars before the bit casts (a bit cast of a
          // vector component reads the vector's first element)
          const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
          H.hi[w][qq] = __builtin_bit_cast(f16x2, v0);
          H.hi[w][qq + 1] = __builtin_bit_cast(f16x2, v1);
          H.hi[w][qq + 2] = __builtin_bit_cast(f16x2, v2);
          H.hi[w][qq + 3] = __builtin_bit_cast(f16x2, v3);
        }
        H.K[w] = s_hk[(size_t)p * Wd + w * LPRD + lrd];
      }
      fold_k(H);
      const float os = s_os[p];
      float* acc = s_acc[wave] + s_pt[p] * SB_DOWN_RB;
#pragma unroll
      for (int i = 0; i < UB; ++i) {
        if (i0 + i < upx) {  // wave-uniform
          float a = lane_row<BITS, VD, false>(D.w[i], H, D.s[i], tmd);
          a = seg_sum(a, lgd);
          const int rl = (i0 + i) * RPWD + rsd;
          if (lrd == LPRD - 1 && rl < nrows) acc[rl] += a * os;
        }
      }
    }
  };

  // 2. the rows of the wave's first batch, its pairs into LDS, then the rows
  //    of its second batch
  DB dA, dB;
  issue(dA, 0);
#pragma unroll
  for (int r = 0; r < HB; ++r)
    if (r < npw) convert(r, pair_of_wave(r));
#pragma unroll 1
  for (int i = HB; i < npw; i += HB) {
#pragma unroll
    for (int r = 0; r < HB; ++r) load_h(r, pair_of_wave(i + r), i + r < npw);
#pragma unroll
    for (int r = 0; r < HB; ++r)
      if (i + r < npw) convert(r, pair_of_wave(i + r));
  }
  issue(dB, 1);
  __syncthreads();

  // 3. the wave's batches, two in flight
#pragma unroll 1
  for (int b = 0; b < nbt; b += 2) {
    compute(dA, b);
    if (b + 1 >= nbt) break;
    issue(dA, b + 2);
    compute(dB, b + 1);
    issue(dB, b + 3);
  }
  __syncthreads();
  // 4. the output rows of every token: the waves' sums in wave order
  for (int i = tid; i < T * nrows; i += DEC_THREADS) {
    const int t = i / nrows, rl = i - t * nrows;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) acc += s_acc[w][t * SB_DOWN_RB + rl];
    float* dst = A.out + (size_t)t * A.d + r0 + rl;
    *dst = A.accumulate ? *dst + acc : acc;
  }
}

template <int BITS, typename ST, int VD>
hipError_t launch_sb_down(const SmallDownArgs& A, int nwg, hipStream_t s) {
  auto kernel = A.table ? k_sb_down<BITS, ST, VD, true> : k_sb_down<BITS, ST, VD, false>;
  if (A.lds_total > 65536) {  // workgroups of more than 64 KB of LDS need the limit raised
    const hipError_t e = hipFuncSetAttribute(
        (const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, A.lds_total);
    if (e != hipSuccess) return e;
  }
  return launch_kernel_lds(kernel, dim3(nwg), dim3(DEC_THREADS), (unsigned)A.lds_total, s, A);
}

}  // namespace smoe
