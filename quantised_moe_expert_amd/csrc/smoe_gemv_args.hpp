// Argument block of the batched expert stages (shared by the dispatcher and
// the kernel instantiation units).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smoe {

// Activation forms of the staged vectors.
enum GvIn { GV_BF16 = 0, GV_F32_SPLIT = 1, GV_F32 = 2 };

// LDS layout of the matrix-core stage (32-bit words) for a workgroup of nw
// waves: token pairs [TC * cols / 2] (+ the same again for the lo halves of
// split inputs), K [G][16], output scales [16], per-wave statistics
// [TC][nw][2], and the k-split partial sums [nw][64][8]. Every region starts
// 16-byte aligned.
struct GmLds {
  int x, xlo, k, osc, red, part, total;
};

__host__ __device__ inline GmLds gm_lds_layout(int cols, int tc, bool split, int nw) {
  auto al4 = [](int n) { return (n + 3) & ~3; };
  GmLds L;
  L.x = 0;
  L.xlo = al4(tc * cols / 2);
  L.k = L.xlo + (split ? al4(tc * cols / 2) : 0);
  L.osc = L.k + al4(cols / 64 * 16);
  L.red = L.osc + 16;
  L.part = L.red + al4(tc * nw * 2);
  L.total = L.part + nw * 64 * 8;
  return L;
}

// K-sliced matrix-core stage (k_gemm_ks): shape and LDS layout.
constexpr int GMK_NW = 8;   // waves per workgroup
constexpr int GMK_TPW = 2;  // 16-row tiles per wave
constexpr int GMK_KSG = 4;  // scale groups per K slice (256 weights)
constexpr int GMK_QPS = GMK_KSG * 8;  // 16-byte pair quads of one token's slice
constexpr int GMK_TC = 64;  // tokens per chunk: four MFMA token tiles
// rows of one matrix per workgroup: gate/up one tile of gate and up rows per
// wave, down two tiles per wave
__host__ __device__ constexpr int gmk_rows_per_block(bool gate_up) {
  return (gate_up ? GMK_TPW / 2 : GMK_TPW) * GMK_NW * 16;
}

// two tokens' slices in LDS (one direct-to-LDS load): 2 * GMK_QPS quads and
// two of padding, so that pair rows start two bank quads apart
constexpr int GMK_XPS = 2 * GMK_QPS + 2;  // 16-byte quads per token pair row

struct GmkLds {
  int x, k, osc, total;  // offsets and size in 32-bit words
};

__host__ __device__ inline GmkLds gmk_lds_layout(int tc) {
  GmkLds L;
  L.x = 0;                               // 2 buffers of tc / 2 token pair rows
  L.k = L.x + tc * GMK_XPS * 4;          // 2 buffers of KSG * tc negated offsets
  L.osc = L.k + 2 * GMK_KSG * tc;        // per-token output factor
  L.total = L.osc + tc;
  return L;
}

struct MatArgs {
  uint64_t codes_off, scales_off;
  int rows, cols, words_per_row, lpr_log2;
};

struct GemvArgs {
  const uint8_t* blobs;  // routed bank (or the shared blob)
  uint64_t stride;
  const uint64_t* table; // optional [E] blob addresses (routed experts only)
  int shared;            // 1: one expert (the shared one), all tokens, pair = token
  int T;
  MatArgs m0, m1;        // gate/up (m1 used by the gate/up stage only)
  int rows_per_wave;     // a multiple of the rows one wave covers per step
  int tc;                // tokens staged in LDS per chunk
  int ksplit;            // matrix-core stage: waves sharing one 16-row tile
  int tiles_per_wave;    // matrix-core stage: tiles each wave takes in turn
  const void* x;         // activations: gate/up: [T, cols]; down: h [pairs, cols]
  int x_ld;              // elements between consecutive activation vectors
  int rms;               // gate/up: apply unit-gain RMSNorm to x
  float eps;
  const int* meta;
  const int* active;
  const int* offs;
  const int* pair_token;
  float* out;            // gate/up: h [pairs, rows]; down: y [pairs, rows]
  // A shared expert whose ffn is nsh times the routed one, run in the same
  // launch as nsh more slots after the routed ones: slot (routed count) + v
  // takes rows [v * rows, (v + 1) * rows) of its gate and up matrices
  // (sh_m0, sh_m1), or columns [v * cols, (v + 1) * cols) of its down matrix
  // (sh_m0), over all T tokens. nsh = 0: routed slots only.
  const uint8_t* sh_blob;
  int nsh;
  MatArgs sh_m0, sh_m1;
  // K-sliced stage: activation vectors prepared by k_gmk_prep (fp16 pair
  // quads [V][cols / 8], group offsets [V][cols / 64], output factors [V])
  const uint32_t* prep_x;
  const float* prep_k;
  const float* prep_o;
};

// Matrix-core stage launchers (smoe_gemm.hpp, instantiated per (BITS, scale
// type) by smoe_gemm_inst.hip); in: GvIn of the activations.
template <int BITS, typename ST>
hipError_t launch_gm(const GemvArgs& A, bool gate_up, int in, int nw, dim3 grid, unsigned lds,
                     hipStream_t s);
// K-sliced matrix-core stage for slots of many tokens (A.tc = 64 per chunk,
// 8 waves); routed experts, bf16 tokens (gate/up) or fp32 h (down).
// Grid (ceil(rows / gmk_rows_per_block(gate_up)), slots).
template <int BITS, typename ST>
hipError_t launch_gm_ks(const GemvArgs& A, bool gate_up, dim3 grid, hipStream_t s);

}  // namespace smoe
