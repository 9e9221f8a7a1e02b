// Launch arguments of the small-batch kernels (smoe_small.hpp).

#pragma once

#include "smoe_decode_args.hpp"

namespace smoe {

// Small batches (2..4 tokens, or one token with a shared expert): routing,
// grouping and the gate/up stage in one launch. Its vector dot products cost
// about 300 instructions per token and row pair, three times what the
// grouped matrix-core stage spends, so past four tokens the grouped stages
// win.
constexpr int SB_TMAX = 4;       // tokens per call on this path
constexpr int SB_TSLOTS = 16;    // token slots of the kernel's LDS tables
constexpr int SB_KEYS = 4096;    // routing keys (tokens x experts) held in LDS, max

struct SmallArgs {
  const uint8_t* blobs;  // routed bank, expert e at blobs + e * stride
  uint64_t stride;
  const uint64_t* table; // optional [E] blob addresses
  const uint8_t* shared; // shared expert blob (nsh > 0)
  uint64_t gc, gs, uc, us;       // routed gate / up codes and scales offsets
  uint64_t sgc, sgs, suc, sus;   // the shared expert's
  int d, ffn, E, k, T, norm, nsh;
  int lg_g;              // log2 lanes per gate/up row
  const void* x;         // [T, d] bf16 or fp32
  int rms;               // apply unit-gain RMSNorm to each token
  float eps;
  const float* logits;   // [T, E]
  float* h;              // [T * k + nsh * T, ffn] per grouped pair
  // the grouped layout (read by the grouped down stage and the combine)
  int32_t* ids;          // [T * k] selected experts
  float* w;              // [T * k] their weights
  int* meta;             // [0] active experts, [1] routed pairs
  int* active;           // [E] expert of each active slot
  int* offs;             // [active + nsh + 1] first grouped pair of each slot
  int* pair_token;       // [T * k + nsh * T] token of each grouped pair
  int* pair_of;          // [T * k] grouped position of pair (t, j)
  int32_t* user_ids;     // optional [T * k]
  float* user_w;         // optional [T * k]
  // dynamic LDS layout (bytes)
  int lds_lv, lds_xp, lds_k, lds_os, lds_total;
  int route_only;        // one workgroup: routing, grouping and the layout only
};

template <int BITS, typename ST, int VG, bool XF32>
hipError_t launch_sb_gate_up(const SmallArgs& A, int nwg, hipStream_t s);

// Small batches (up to SB_TSLOTS tokens): the down projection over the
// grouped pairs and the weighted combine in one launch.
struct SmallDownArgs {
  const uint8_t* blobs;  // routed bank, expert e at blobs + e * stride
  uint64_t stride;
  const uint64_t* table; // optional [E] blob addresses
  const uint8_t* shared; // shared expert blob (nsh > 0)
  uint64_t dc, ds;       // routed down codes / scales offsets
  uint64_t sdc, sds;     // the shared expert's
  int d, ffn, k, T, nsh;
  int lg_d;              // log2 lanes per down row
  int rb;                // output rows per workgroup
  const float* h;        // [T * k + nsh * T, ffn] per grouped pair
  const int* meta;       // [0] active experts
  const int* active;     // expert of each active slot
  const int* offs;       // first grouped pair of each slot (offs[active] = T * k)
  const int* pair_token; // token of each grouped pair
  const int* pair_of;    // [T * k] grouped position of pair (t, j)
  const float* w;        // [T * k] weights of the pairs (t, j)
  float* out;            // [T, d]
  int accumulate;        // out += layer(x)
  int E;                 // routed experts (size of active; offs holds E + nsh + 1)
  int lds_hk, lds_total; // dynamic LDS: fp16 pairs of every pair's h, then their offsets
};
constexpr int SB_DOWN_RB = 16;  // output rows per workgroup, max
constexpr int SB_PAIRS = SB_TSLOTS * SMOE_MAX_TOP_K + 16 * SB_TSLOTS;  // grouped pairs, max
// row loads a lane holds per expert in the small-batch down stage (16 rows
// at 16 lanes per row; half that at 16 code words per lane, to stay within
// the registers)
constexpr int sb_down_loads(int vd) { return vd > 12 ? 2 : 4; }

template <int BITS, typename ST, int VD>
hipError_t launch_sb_down(const SmallDownArgs& A, int nwg, hipStream_t s);

}  // namespace smoe
