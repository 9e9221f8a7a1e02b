// Argument block of the expert GEMV stages (shared by the dispatcher and
// the kernel instantiation units).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smoe {

// Words-per-lane values with a kernel instantiation (each row of W code words
// is spread over W / V lanes, a power of two <= 64).
#define SMOE_V_LIST(X) \
  X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

struct MatArgs {
  uint64_t codes_off, scales_off;
  int rows, cols, words_per_row, lpr_log2;
};

struct GemvArgs {
  const uint8_t* blobs;  // routed bank (or the shared blob)
  uint64_t stride;
  int shared;            // 1: one expert (the shared one), all tokens, pair = token
  int T;
  MatArgs m0, m1;        // gate/up (m1 used by the gate/up stage only)
  int rows_per_wave;
  const void* x;         // activations: gate/up: [T, cols]; down: h [pairs, cols]
  int x_ld;              // elements between consecutive activation vectors
  int rms;               // gate/up: apply unit-gain RMSNorm to x
  float eps;
  const int* meta;
  const int* active;
  const int* offs;
  const int* pair_token;
  float* out;            // gate/up: h [pairs, rows]; down: y [pairs, rows]
};

// Launchers, defined in smoe_gemv.hpp and instantiated per (BITS, scale
// type, V) by the smoe_gemv_inst.hip units.
template <int BITS, typename ST, int V>
hipError_t launch_gu(const GemvArgs& A, bool bf16, dim3 grid, hipStream_t s);
template <int BITS, typename ST, int V>
hipError_t launch_dn(const GemvArgs& A, dim3 grid, hipStream_t s);

}  // namespace smoe
