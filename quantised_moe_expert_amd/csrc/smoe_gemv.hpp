// Grouped expert GEMV stages for batches (gate/up + SwiGLU, and down).
//
// Grid (row blocks, active-expert slots); a workgroup of 4 waves owns a block
// of rows of one expert and applies them to every token routed to it:
//   1. the slot's token vectors are staged in LDS, a chunk of up to TC tokens
//      at a time, as fp16 pairs in the lane order of the row layout (each
//      vector scaled by a power of two so its largest magnitude sits just
//      below 2^14; fp32 inputs of the gate/up stage as a hi + lo pair), with
//      the offset K of each lane's 4-word chunk and the token's output scale;
//   2. each wave walks its row groups (RPW rows per group, one row per LPR
//      lanes), loads a group's code words and scales once (the next group's
//      loads are issued before the current one is computed), decodes the
//      words into fp16 pairs once, and then takes one dot product per staged
//      token, reading the token's pairs from LDS.
// So an expert's bytes are read once per forward however many tokens chose
// it, and the decode work is shared by those tokens.

#pragma once

#include "smoe_device.hpp"
#include "smoe_gemv_args.hpp"
#include "smoe_launch.hpp"

namespace smoe {

// The WPW activations of code word cw of vector v (bf16 or fp32 elements).
template <int BITS, bool XF32>
__device__ __forceinline__ void gv_load_word(const void* v, int cw, float (&xv)[QT<BITS>::WPW]) {
  constexpr int WPW = QT<BITS>::WPW;
  if constexpr (XF32) {
    const float* p = (const float*)v + (size_t)cw * WPW;
#pragma unroll
    for (int i = 0; i < WPW / 4; ++i) {
      const f32x4 t = *(const f32x4*)(p + 4 * i);
      xv[4 * i] = t.x;
      xv[4 * i + 1] = t.y;
      xv[4 * i + 2] = t.z;
      xv[4 * i + 3] = t.w;
    }
  } else {
    const uint32_t* p = (const uint32_t*)v + (size_t)cw * (WPW / 2);
#pragma unroll
    for (int i = 0; i < WPW / 8; ++i) {
      const u32x4 t = *(const u32x4*)(p + 4 * i);
      const uint32_t tt[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[8 * i + 2 * j] = __builtin_bit_cast(float, tt[j] << 16);
        xv[8 * i + 2 * j + 1] = __builtin_bit_cast(float, tt[j] & 0xFFFF0000u);
      }
    }
  }
}

// Stage the input vectors of pairs [pc, pc + nt) of the slot: the gate/up
// stage reads x row pair_token[p] (row p for the shared expert, whose pairs
// are the tokens); the down stage reads h row p.
template <int BITS, int V, int IN, bool GU>
__device__ __forceinline__ void gv_stage(const GemvArgs& A, const MatArgs& M, uint32_t* lds,
                                         const GvLds& L, int pc, int nt) {
  constexpr int WPW = QT<BITS>::WPW, PPW = QT<BITS>::PPW, NPOS = QT<BITS>::NPOS;
  constexpr bool XF32 = IN != GV_BF16, SPLIT = IN == GV_F32_SPLIT;
  using LM = LaneMap<V>;
  constexpr int NK = LM::N4 + LM::R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cols = M.cols, Wr = M.words_per_row, LPR = 1 << M.lpr_log2;
  const size_t esz = XF32 ? 4 : 2;
  auto vec = [&](int i) {
    const int p = pc + i;
    const int t = (GU && !A.shared) ? A.pair_token[p] : p;
    return (const void*)((const uint8_t*)A.x + (size_t)t * A.x_ld * esz);
  };
  float* red = (float*)(lds + L.red);
  // pass 1: per-token max |x| and sum of squares
  for (int i = 0; i < nt; ++i) {
    const void* v = vec(i);
    float amax = 0.f, ss = 0.f;
    for (int cw = tid; cw < Wr; cw += GV_THREADS) {
      float xv[WPW];
      gv_load_word<BITS, XF32>(v, cw, xv);
#pragma unroll
      for (int j = 0; j < WPW; ++j) {
        amax = fmaxf(amax, fabsf(xv[j]));
        ss = fmaf(xv[j], xv[j], ss);
      }
    }
    amax = lane63(seg_max(amax, 6));
    ss = lane63(seg_sum(ss, 6));
    if (lane == 0) {
      red[(i * GV_WAVES + wave) * 2] = amax;
      red[(i * GV_WAVES + wave) * 2 + 1] = ss;
    }
  }
  __syncthreads();
  // pass 2: pairs and per-chunk offsets; unit u = (slot, lane): slot < N4 is
  // the lane's 4-word chunk, slot >= N4 one tail word
  float* Kl = (float*)(lds + L.k);
  float* osc = (float*)(lds + L.osc);
  for (int i = 0; i < nt; ++i) {
    float m = 0.f, q2 = 0.f;
#pragma unroll
    for (int w = 0; w < GV_WAVES; ++w) {
      m = fmaxf(m, red[(i * GV_WAVES + w) * 2]);
      q2 += red[(i * GV_WAVES + w) * 2 + 1];
    }
    int ex = 0;
    frexpf(m, &ex);
    ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
    const float S = ldexpf(1.0f, 14 - ex);
    if (tid == 0) {
      const float r = A.rms ? 1.0f / sqrtf(q2 / (float)cols + A.eps) : 1.0f;
      osc[i] = r / (QT<BITS>::M * S);
    }
    const void* v = vec(i);
    uint32_t* xhi = lds + L.xhi + i * (cols / 2);
    uint32_t* xlo = lds + L.xlo + i * (cols / 2);
    for (int u = tid; u < NK * LPR; u += GV_THREADS) {
      const int slot = u / LPR, lr = u - slot * LPR;
      const int nw = slot < LM::N4 ? 4 : 1;
      float kk = 0.f;
      for (int j = 0; j < nw; ++j) {
        const int w = slot < LM::N4 ? 4 * slot + j : 4 * LM::N4 + (slot - LM::N4);
        const int cw = LM::word(lr, LPR, w);
        float xv[WPW];
        gv_load_word<BITS, XF32>(v, cw, xv);
#pragma unroll
        for (int q = 0; q < PPW; ++q) {
          const int hs = q / NPOS, pos = q % NPOS;
          const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
          const float f = S * (1.0f / (float)(1 << (BITS * pos)));
          const float a = xv[ia] * f, b = xv[ib] * f;
          const _Float16 ha = (_Float16)a, hb = (_Float16)b;
          xhi[(w * LPR + lr) * PPW + q] = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
          float sumx = (float)ha + (float)hb;
          if constexpr (SPLIT) {
            const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
            xlo[(w * LPR + lr) * PPW + q] = __builtin_bit_cast(uint32_t, f16x2{la, lb});
            sumx += (float)la + (float)lb;
          }
          kk = fmaf(sumx, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)), kk);
        }
      }
      Kl[(i * NK + slot) * LPR + lr] = kk;
    }
  }
  __syncthreads();
}

// One row's code words and scales.
template <int BITS, int V>
struct GvRow {
  uint32_t w[V];
  float s[ScalePlan<BITS, V>::NS];
};

// Decoded fp16 pairs of one row: pair q of word w.
template <int BITS, int V>
struct GvPairs {
  uint32_t p[V][QT<BITS>::PPW];
};

template <int BITS, int V>
__device__ __forceinline__ void gv_decode(const GvRow<BITS, V>& R, GvPairs<BITS, V>& P) {
  constexpr int NPOS = QT<BITS>::NPOS;
#pragma unroll
  for (int w = 0; w < V; ++w)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const uint32_t v = hs ? (R.w[w] >> 8) : R.w[w];
#pragma unroll
      for (int pos = 0; pos < NPOS; ++pos) {
        constexpr uint32_t base = (1u << BITS) - 1u;
        const uint32_t m = (base << (BITS * pos)) | (base << (BITS * pos + 16));
        P.p[w][hs * NPOS + pos] = and_or(v, m, 0x64006400u);
      }
    }
}

// sum over the lane's words of scale * (pairs . x - K) for staged token i
template <int BITS, int V, bool SPLIT>
__device__ __forceinline__ float gv_dot(const GvPairs<BITS, V>& P, const GvRow<BITS, V>& R,
                                        const uint32_t* xhi, const uint32_t* xlo,
                                        const float* K, int lr, int LPR, int tmask) {
  constexpr int PPW = QT<BITS>::PPW;
  using SP = ScalePlan<BITS, V>;
  float acc = 0.f;
  auto word_dot = [&](int w, float a) {
#pragma unroll
    for (int q4 = 0; q4 < PPW / 4; ++q4) {
      // (components copied to scalars first: a bit cast applied directly
      // to a vector component reads the vector's first element)
      const u32x4 xh = *(const u32x4*)(xhi + (w * LPR + lr) * PPW + 4 * q4);
      const uint32_t h0 = xh.x, h1 = xh.y, h2 = xh.z, h3 = xh.w;
      a = fdot2(P.p[w][4 * q4], __builtin_bit_cast(f16x2, h0), a);
      a = fdot2(P.p[w][4 * q4 + 1], __builtin_bit_cast(f16x2, h1), a);
      a = fdot2(P.p[w][4 * q4 + 2], __builtin_bit_cast(f16x2, h2), a);
      a = fdot2(P.p[w][4 * q4 + 3], __builtin_bit_cast(f16x2, h3), a);
      if constexpr (SPLIT) {
        const u32x4 xl = *(const u32x4*)(xlo + (w * LPR + lr) * PPW + 4 * q4);
        const uint32_t l0 = xl.x, l1 = xl.y, l2 = xl.z, l3 = xl.w;
        a = fdot2(P.p[w][4 * q4], __builtin_bit_cast(f16x2, l0), a);
        a = fdot2(P.p[w][4 * q4 + 1], __builtin_bit_cast(f16x2, l1), a);
        a = fdot2(P.p[w][4 * q4 + 2], __builtin_bit_cast(f16x2, l2), a);
        a = fdot2(P.p[w][4 * q4 + 3], __builtin_bit_cast(f16x2, l3), a);
      }
    }
    return a;
  };
#pragma unroll
  for (int c = 0; c < SP::N4; ++c) {
    float a = -K[c * LPR + lr];
#pragma unroll
    for (int w = 4 * c; w < 4 * c + 4; ++w) a = word_dot(w, a);
    acc = fmaf(a, R.s[c], acc);
  }
  if constexpr (SP::R > 0) {
    float t0 = R.s[SP::N4], t1 = R.s[SP::NS - 1];
    asm volatile("" : "+v"(t0), "+v"(t1));
#pragma unroll
    for (int t = 0; t < SP::R; ++t) {
      const float a = word_dot(4 * SP::N4 + t, -K[(SP::N4 + t) * LPR + lr]);
      const float sc = (SP::NT == 2 && ((tmask >> t) & 1)) ? t1 : t0;
      acc = fmaf(a, sc, acc);
    }
  }
  return acc;
}

// GU: gate/up + SwiGLU, h[p, r] = silu(gate_r . x_p) * (up_r . x_p);
// otherwise down, y[p, r] = down_r . h_p.
template <int BITS, int V, typename ST, int IN, bool GU>
__global__ __launch_bounds__(GV_THREADS) void k_grouped(GemvArgs A) {
  extern __shared__ uint32_t lds[];
  constexpr bool SPLIT = IN == GV_F32_SPLIT;
  using SP = ScalePlan<BITS, V>;
  using LM = LaneMap<V>;
  constexpr int NK = LM::N4 + LM::R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e = 0, p0, p1;
  if (A.shared) {
    p0 = 0;
    p1 = A.T;
  } else {
    const int slot = blockIdx.y;
    if (slot >= A.meta[0]) return;  // workgroup-uniform
    e = A.active[slot];
    p0 = A.offs[slot];
    p1 = A.offs[slot + 1];
  }
  const MatArgs& M0 = A.m0;
  const int rows = M0.rows;
  const int lg = M0.lpr_log2, LPR = 1 << lg, lr = lane & (LPR - 1), rsub = lane >> lg;
  const int RPW = 64 >> lg;
  const int rpw = A.rows_per_wave;  // a multiple of RPW
  const int rw0 = (blockIdx.x * GV_WAVES + wave) * rpw;
  const int ngroups = rw0 < rows ? (min(rw0 + rpw, rows) - rw0 + RPW - 1) / RPW : 0;
  const int Wr = M0.words_per_row, G = M0.cols / 64;
  const uint8_t* blob = expert_blob(A.blobs, A.stride, A.table, e);
  const uint32_t* c0 = (const uint32_t*)(blob + M0.codes_off);
  const ST* s0 = (const ST*)(blob + M0.scales_off);
  const uint32_t* c1 = (const uint32_t*)(blob + A.m1.codes_off);
  const ST* s1 = (const ST*)(blob + A.m1.scales_off);
  int sg[SP::NS], tmask;
  scale_groups<BITS, V>(lr, LPR, sg, tmask);
  const GvLds L = gv_lds_layout(M0.cols, LPR, NK, A.tc, SPLIT);
  const uint32_t* xhi_all = lds + L.xhi;
  const uint32_t* xlo_all = lds + L.xlo;
  const float* K_all = (const float*)(lds + L.k);
  const float* osc = (const float*)(lds + L.osc);

  struct Group {
    GvRow<BITS, V> a, b;  // gate (or down) row, up row
  };
  auto load = [&](Group& g, int gi) {
    const int r = rw0 + gi * RPW + rsub;
    const int rc = r < rows ? r : rows - 1;
    load_row_words<V, true>(c0 + (size_t)rc * Wr, lr, LPR, g.a.w);
    load_row_scales<BITS, V, ST, true>(s0 + (size_t)rc * G, sg, G, g.a.s);
    if constexpr (GU) {
      load_row_words<V, true>(c1 + (size_t)rc * Wr, lr, LPR, g.b.w);
      load_row_scales<BITS, V, ST, true>(s1 + (size_t)rc * G, sg, G, g.b.s);
    }
  };

  for (int pc = p0; pc < p1; pc += A.tc) {
    const int nt = min(A.tc, p1 - pc);
    if (pc > p0) __syncthreads();  // the previous chunk's readers are done
    gv_stage<BITS, V, IN, GU>(A, M0, lds, L, pc, nt);
    Group gA, gB;
    if (ngroups > 0) load(gA, 0);
    auto compute = [&](const Group& g, int gi) {
      GvPairs<BITS, V> Pa, Pb;
      gv_decode<BITS, V>(g.a, Pa);
      if constexpr (GU) gv_decode<BITS, V>(g.b, Pb);
      const int r = rw0 + gi * RPW + rsub;
      for (int i = 0; i < nt; ++i) {
        const uint32_t* xh = xhi_all + i * (M0.cols / 2);
        const uint32_t* xl = xlo_all + i * (M0.cols / 2);
        const float* K = K_all + i * NK * LPR;
        float a = gv_dot<BITS, V, SPLIT>(Pa, g.a, xh, xl, K, lr, LPR, tmask);
        a = seg_sum(a, lg);
        float u = 0.f;
        if constexpr (GU) {
          u = gv_dot<BITS, V, SPLIT>(Pb, g.b, xh, xl, K, lr, LPR, tmask);
          u = seg_sum(u, lg);
        }
        if (lr == LPR - 1 && r < rows && r < rw0 + rpw) {
          const float o = osc[i];
          float val;
          if constexpr (GU) {
            const float gg = a * o, uu = u * o;
            val = gg / (1.0f + expf(-gg)) * uu;
          } else {
            val = a * o;
          }
          A.out[(size_t)(pc + i) * rows + r] = val;
        }
      }
    };
    for (int gi = 0; gi < ngroups; gi += 2) {
      if (gi + 1 < ngroups) load(gB, gi + 1);
      compute(gA, gi);
      if (gi + 1 >= ngroups) break;
      if (gi + 2 < ngroups) load(gA, gi + 2);
      compute(gB, gi + 1);
    }
  }
}

// Launchers, instantiated per (BITS, scale type, V) in smoe_gemv_inst.hip.
// in: GvIn of the activations; lds: dynamic LDS bytes (gv_lds_layout).
template <int BITS, typename ST, int V>
hipError_t launch_gu(const GemvArgs& A, int in, dim3 grid, unsigned lds, hipStream_t s) {
  if (in == GV_BF16)
    return launch_kernel_lds(k_grouped<BITS, V, ST, GV_BF16, true>, grid, dim3(GV_THREADS), lds,
                             s, A);
  return launch_kernel_lds(k_grouped<BITS, V, ST, GV_F32_SPLIT, true>, grid, dim3(GV_THREADS),
                           lds, s, A);
}

template <int BITS, typename ST, int V>
hipError_t launch_dn(const GemvArgs& A, dim3 grid, unsigned lds, hipStream_t s) {
  return launch_kernel_lds(k_grouped<BITS, V, ST, GV_F32, false>, grid, dim3(GV_THREADS), lds, s,
                           A);
}

}  // namespace smoe
