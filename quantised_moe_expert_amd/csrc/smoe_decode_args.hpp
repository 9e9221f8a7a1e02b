// Argument block and launcher declarations of the two-launch batch-1 layer
// kernels (see smoe_decode.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/smoe.h"

namespace smoe {

constexpr int DEC_THREADS = 512;   // one workgroup of 8 waves per CU
constexpr int DEC_NWG = 256;       // workgroups per launch (one per CU)
constexpr int DEC_NWG_GU = 512;    // gate/up stage on bf16 inputs: two per CU (16 waves)
// waves per SIMD the kernels are built for (HIP's second launch-bounds
// argument): one 8-wave workgroup per CU
constexpr int DEC_WAVES_PER_EU = DEC_THREADS / 256;
// the gate/up stage on bf16 inputs runs two workgroups per CU: four waves per
// SIMD, so at most 128 registers (fp32 inputs need the hi + lo pairs and keep
// one workgroup per CU)
constexpr int DEC_GU_WAVES_PER_EU = 2 * DEC_THREADS / 256;
constexpr int DEC_RB_MAX = 64;     // down-projection rows per workgroup, max
constexpr int DEC_XW = 4;          // x code words per thread (d * bits / 32 <= 4 * 512)
constexpr int DEC_HJ = 2;          // h vectors staged per wave (k <= 16)
constexpr int DEC_HC = 4;          // h code words per lane when a wave converts h_j (ffn * bits / 32 <= 256)
constexpr int DEC_HW = 64 * DEC_HC;  // h code words per vector, max
constexpr int DEC_HP = DEC_HW * 4;   // fp16 pairs of one h vector in LDS, max (Q4: 4 per word)
constexpr int DEC_KEYS = 512;      // routing keys in LDS, padding included
constexpr int DEC_H_LDS = 12288;   // fp16 pairs of h held in LDS (k * ffn / 2 <= 12288)

struct DecodeArgs {
  const uint8_t* blobs;  // routed expert bank, expert e at blobs + e * stride
  uint64_t stride;
  const uint64_t* table; // optional [E] blob addresses (replaces blobs + e * stride)
  uint64_t gc, gs, uc, us, dc, ds;  // codes / scales offsets of gate, up, down
  int d, ffn, E, k, norm;
  int lg_g, lg_d;        // log2 lanes per row for the gate/up and the down rows
  const void* x;         // [d] bf16 or fp32 activation (the residual when rms)
  int rms;               // apply unit-gain RMSNorm to x
  float eps;
  const float* logits;   // [E]
  float* h;              // [k, ffn] workspace: SwiGLU output of each selected expert
  int32_t* ws_ids;       // [k] workspace: selected experts (written by K1)
  float* ws_w;           // [k] workspace: their weights
  float* out;            // [d]
  int accumulate;        // out += layer(x) instead of out = layer(x)
  int32_t* user_ids;     // optional [k]
  float* user_w;         // optional [k]
  int rb;                // down rows per workgroup
  // routing split: wave w ranks experts [w * rk_kpw, (w + 1) * rk_kpw), with
  // 2^rk_lg lanes per expert, each comparing against rk_cp key pairs
  int rk_kpw, rk_lg, rk_cp;
};

template <int BITS, typename ST, int VG, bool XF32>
hipError_t launch_dec_gate_up(const DecodeArgs& A, int nwg, hipStream_t s);

template <int BITS, typename ST, int VD>
hipError_t launch_dec_down(const DecodeArgs& A, int nwg, hipStream_t s);

// gate/up and down words-per-lane values with an instantiation
#define SMOE_DEC_Q4_VG(X) X(8) X(4) X(1)
#define SMOE_DEC_Q4_VD(X) X(12) X(11) X(8) X(6) X(4) X(2) X(1) X(16)
#define SMOE_DEC_Q2_VG(X) X(4) X(2) X(1)
#define SMOE_DEC_Q2_VD(X) X(6) X(11) X(8) X(4) X(2) X(1)

}  // namespace smoe
