// Expert GEMV stages (gate/up + SwiGLU, and down) for gfx950.
#pragma once

#include "smoe_device.hpp"
#include "smoe_gemv_args.hpp"
#include "smoe_launch.hpp"

namespace smoe {

// gate/up + SwiGLU: h[p, r] = silu(gate_r . x) * (up_r . x)
template <int BITS, int V, typename ST, bool BF16>
__global__ __launch_bounds__(256) void k_gate_up(GemvArgs A) {
  constexpr bool SPLIT = !BF16;
  using SP = ScalePlan<BITS, V>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e = 0, p0, p1;
  if (A.shared) {
    p0 = 0;
    p1 = A.T;
  } else {
    const int slot = blockIdx.y;
    if (slot >= A.meta[0]) return;
    e = A.active[slot];
    p0 = A.offs[slot];
    p1 = A.offs[slot + 1];
  }
  const int rows = A.m0.rows;
  const int row0 = (blockIdx.x * (blockDim.x >> 6) + wave) * A.rows_per_wave;
  if (row0 >= rows) return;
  const int row1 = min(row0 + A.rows_per_wave, rows);
  const int lg = A.m0.lpr_log2, LPR = 1 << lg, lr = lane & (LPR - 1), rsub = lane >> lg,
            RPW = 64 >> lg;
  const int Wr = A.m0.words_per_row, G = A.m0.cols / 64;
  const uint8_t* blob = A.blobs + (uint64_t)e * A.stride;
  const uint32_t* gcodes = (const uint32_t*)(blob + A.m0.codes_off);
  const uint32_t* ucodes = (const uint32_t*)(blob + A.m1.codes_off);
  const ST* gsc = (const ST*)(blob + A.m0.scales_off);
  const ST* usc = (const ST*)(blob + A.m1.scales_off);
  int sg[SP::NS], tmask;
  scale_groups<BITS, V>(lr, LPR, sg, tmask);
  for (int p = p0; p < p1; ++p) {
    const int t = A.shared ? p : A.pair_token[p];
    XRegs<BITS, V, SPLIT> X;
    const void* xv = BF16 ? (const void*)((const uint16_t*)A.x + (size_t)t * A.x_ld)
                          : (const void*)((const float*)A.x + (size_t)t * A.x_ld);
    prep_x<BITS, V, SPLIT, BF16>(X, xv, lr, lg, A.rms != 0, A.eps, A.m0.cols);
    fold_k(X);
    for (int rb = row0; rb < row1; rb += RPW) {
      const int r = rb + rsub;
      const int rc = r < rows ? r : rows - 1;
      uint32_t gw[V], uw[V];
      load_row_words<V, false>(gcodes + (size_t)rc * Wr, lr, LPR, gw);
      load_row_words<V, false>(ucodes + (size_t)rc * Wr, lr, LPR, uw);
      float gs[SP::NS], us[SP::NS];
      load_row_scales<BITS, V, ST, false>(gsc + (size_t)rc * G, sg, G, gs);
      load_row_scales<BITS, V, ST, false>(usc + (size_t)rc * G, sg, G, us);
      float ag = lane_row<BITS, V, SPLIT>(gw, X, gs, tmask);
      float au = lane_row<BITS, V, SPLIT>(uw, X, us, tmask);
      ag = seg_sum(ag, lg);
      au = seg_sum(au, lg);
      if (lr == LPR - 1 && r < row1) {
        const float g = ag * X.oscale, u = au * X.oscale;
        A.out[(size_t)p * rows + r] = g / (1.0f + expf(-g)) * u;
      }
    }
  }
}

// down: y[p, r] = down_r . h[p]
template <int BITS, int V, typename ST, bool SPLIT>
__global__ __launch_bounds__(256) void k_down(GemvArgs A) {
  using SP = ScalePlan<BITS, V>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e = 0, p0, p1;
  if (A.shared) {
    p0 = 0;
    p1 = A.T;
  } else {
    const int slot = blockIdx.y;
    if (slot >= A.meta[0]) return;
    e = A.active[slot];
    p0 = A.offs[slot];
    p1 = A.offs[slot + 1];
  }
  const int rows = A.m0.rows;
  const int row0 = (blockIdx.x * (blockDim.x >> 6) + wave) * A.rows_per_wave;
  if (row0 >= rows) return;
  const int row1 = min(row0 + A.rows_per_wave, rows);
  const int lg = A.m0.lpr_log2, LPR = 1 << lg, lr = lane & (LPR - 1), rsub = lane >> lg,
            RPW = 64 >> lg;
  const int Wr = A.m0.words_per_row, G = A.m0.cols / 64;
  const uint8_t* blob = A.blobs + (uint64_t)e * A.stride;
  const uint32_t* codes = (const uint32_t*)(blob + A.m0.codes_off);
  const ST* sc = (const ST*)(blob + A.m0.scales_off);
  int sg[SP::NS], tmask;
  scale_groups<BITS, V>(lr, LPR, sg, tmask);
  for (int p = p0; p < p1; ++p) {
    XRegs<BITS, V, SPLIT> X;
    prep_x<BITS, V, SPLIT, false>(X, (const float*)A.x + (size_t)p * A.x_ld, lr, lg, false,
                                  0.f, A.m0.cols);
    fold_k(X);
    for (int rb = row0; rb < row1; rb += RPW) {
      const int r = rb + rsub;
      const int rc = r < rows ? r : rows - 1;
      uint32_t cw[V];
      load_row_words<V, false>(codes + (size_t)rc * Wr, lr, LPR, cw);
      float s[SP::NS];
      load_row_scales<BITS, V, ST, false>(sc + (size_t)rc * G, sg, G, s);
      float a = lane_row<BITS, V, SPLIT>(cw, X, s, tmask);
      a = seg_sum(a, lg);
      if (lr == LPR - 1 && r < row1) A.out[(size_t)p * rows + r] = a * X.oscale;
    }
  }
}


// Launchers, instantiated per (BITS, scale type, V) in smoe_gemv_inst.hip.
template <int BITS, typename ST, int V>
hipError_t launch_gu(const GemvArgs& A, bool bf16, dim3 grid, hipStream_t s) {
  return bf16 ? launch_kernel(k_gate_up<BITS, V, ST, true>, grid, dim3(256), s, A)
              : launch_kernel(k_gate_up<BITS, V, ST, false>, grid, dim3(256), s, A);
}

template <int BITS, typename ST, int V>
hipError_t launch_dn(const GemvArgs& A, dim3 grid, hipStream_t s) {
  return launch_kernel(k_down<BITS, V, ST, false>, grid, dim3(256), s, A);
}

}  // namespace smoe
