// Host side of the batch-1 layer kernels: picks the instantiations for a
// layer's shape and enqueues the two launches. Returns "not launched" (so the
// caller takes the multi-kernel grouped path) when no instantiation fits.

#include <hip/hip_runtime.h>

#include "smoe_decode_args.hpp"
#include "smoe_small_args.hpp"
#include "smoe_internal.hpp"
#include "smoe_launch.hpp"

namespace smoe {
namespace {

typedef hipError_t (*GuLaunch)(const DecodeArgs&, int, hipStream_t);
typedef hipError_t (*DnLaunch)(const DecodeArgs&, int, hipStream_t);

template <int BITS, typename ST>
bool find_gu(int vg, bool xf32, GuLaunch* L) {
#define SMOE_FIND_G(v)                                                        \
  if (vg == v) {                                                             \
    *L = xf32 ? launch_dec_gate_up<BITS, ST, v, true>                        \
              : launch_dec_gate_up<BITS, ST, v, false>;                      \
    return true;                                                             \
  }
  if constexpr (BITS == 4) {
    SMOE_DEC_Q4_VG(SMOE_FIND_G)
  } else {
    SMOE_DEC_Q2_VG(SMOE_FIND_G)
  }
#undef SMOE_FIND_G
  return false;
}

template <int BITS, typename ST>
bool find_dn(int vd, DnLaunch* L) {
#define SMOE_FIND_D(v)                 \
  if (vd == v) {                       \
    *L = launch_dec_down<BITS, ST, v>; \
    return true;                       \
  }
  if constexpr (BITS == 4) {
    SMOE_DEC_Q4_VD(SMOE_FIND_D)
  } else {
    SMOE_DEC_Q2_VD(SMOE_FIND_D)
  }
#undef SMOE_FIND_D
  return false;
}

bool find_pair(int bits, int sdt, int vg, int vd, bool xf32, GuLaunch* G, DnLaunch* D) {
  if (bits == 4 && sdt == SMOE_SCALE_F32)
    return find_gu<4, float>(vg, xf32, G) && find_dn<4, float>(vd, D);
  if (bits == 4) return find_gu<4, _Float16>(vg, xf32, G) && find_dn<4, _Float16>(vd, D);
  if (sdt == SMOE_SCALE_F32) return find_gu<2, float>(vg, xf32, G) && find_dn<2, float>(vd, D);
  return find_gu<2, _Float16>(vg, xf32, G) && find_dn<2, _Float16>(vd, D);
}

typedef hipError_t (*SbLaunch)(const SmallArgs&, int, hipStream_t);

template <int BITS, typename ST>
bool find_sb(int vg, bool xf32, SbLaunch* L) {
#define SMOE_FIND_SB(v)                                                       \
  if (vg == v) {                                                             \
    *L = xf32 ? launch_sb_gate_up<BITS, ST, v, true>                         \
              : launch_sb_gate_up<BITS, ST, v, false>;                       \
    return true;                                                             \
  }
  if constexpr (BITS == 4) {
    SMOE_DEC_Q4_VG(SMOE_FIND_SB)
  } else {
    SMOE_DEC_Q2_VG(SMOE_FIND_SB)
  }
#undef SMOE_FIND_SB
  return false;
}

bool find_sb_any(int bits, int sdt, int vg, bool xf32, SbLaunch* L) {
  if (bits == 4 && sdt == SMOE_SCALE_F32) return find_sb<4, float>(vg, xf32, L);
  if (bits == 4) return find_sb<4, _Float16>(vg, xf32, L);
  if (sdt == SMOE_SCALE_F32) return find_sb<2, float>(vg, xf32, L);
  return find_sb<2, _Float16>(vg, xf32, L);
}

typedef hipError_t (*SdLaunch)(const SmallDownArgs&, int, hipStream_t);

template <int BITS, typename ST>
bool find_sd(int vd, SdLaunch* L) {
#define SMOE_FIND_SD(v)               \
  if (vd == v) {                      \
    *L = launch_sb_down<BITS, ST, v>; \
    return true;                      \
  }
  if constexpr (BITS == 4) {
    SMOE_DEC_Q4_VD(SMOE_FIND_SD)
  } else {
    SMOE_DEC_Q2_VD(SMOE_FIND_SD)
  }
#undef SMOE_FIND_SD
  return false;
}

bool find_sd_any(int bits, int sdt, int vd, SdLaunch* L) {
  if (bits == 4 && sdt == SMOE_SCALE_F32) return find_sd<4, float>(vd, L);
  if (bits == 4) return find_sd<4, _Float16>(vd, L);
  if (sdt == SMOE_SCALE_F32) return find_sd<2, float>(vd, L);
  return find_sd<2, _Float16>(vd, L);
}

uint64_t align16(uint64_t v) { return (v + 15) / 16 * 16; }

// static LDS of k_sb_gate_up: expert masks, slots, active list, offsets,
// selections (see smoe_small.hpp)
constexpr uint64_t SB_STATIC_LDS = (4ull * SMOE_MAX_EXPERTS + 1) * 4 +
                                   2ull * SB_TSLOTS * SMOE_MAX_TOP_K * 4 + 64 +
                                   (DEC_THREADS / 64) * 64 * 4;

// static LDS of k_sb_down: accumulators, pair scales and tokens, slots
constexpr uint64_t SD_STATIC_LDS = (uint64_t)DEC_THREADS / 64 * SB_TSLOTS * SB_DOWN_RB * 4 +
                                   2ull * SB_PAIRS * 4 + (SMOE_MAX_EXPERTS + 2ull * DEC_THREADS) * 4;

}  // namespace

hipError_t decode1_try(const LayerInfo& L, const void* x, bool xf32, bool rms, float eps,
                       const float* logits, int k, int norm, float* out, int accumulate,
                       int32_t* uids, float* uw, float* h, int32_t* ws_ids, float* ws_w,
                       hipStream_t stream, bool* launched) {
  *launched = false;
  if (L.desc.shared_ffn_dim) return hipSuccess;
  const ExpertPlan& P = L.plan;
  const int bits = (int)L.desc.bits;
  GuLaunch gu;
  DnLaunch dn;
  // the down rows go to at most 16 lanes each (see k_dec_down)
  const int lg_d = P.down.lpr_log2 < 4 ? P.down.lpr_log2 : 4;
  const int vd = P.down.words_per_row >> lg_d;
  if (!find_pair(bits, (int)L.desc.scale_dtype, P.gate.v, vd, xf32, &gu, &dn))
    return hipSuccess;
  const int rpwd = 64 >> lg_d;
  int rb = (P.d_model + DEC_NWG - 1) / DEC_NWG;
  rb = (rb + rpwd - 1) / rpwd * rpwd;
  // shape limits of the kernels' register and LDS staging
  if (rb > DEC_RB_MAX) return hipSuccess;
  if ((int64_t)P.d_model * bits / 32 > (int64_t)DEC_XW * DEC_THREADS) return hipSuccess;
  if ((int64_t)P.ffn * bits / 32 > 64 * (DEC_HC / (bits == 2 ? 2 : 1))) return hipSuccess;
  if ((int64_t)k * P.ffn / 2 > DEC_H_LDS) return hipSuccess;
  if (k > DEC_HJ * (DEC_THREADS / 64)) return hipSuccess;
  DecodeArgs A{};
  A.blobs = L.blobs;
  A.stride = L.desc.blob_stride;
  A.table = L.table;
  A.gc = P.gate.codes_off;
  A.gs = P.gate.scales_off;
  A.uc = P.up.codes_off;
  A.us = P.up.scales_off;
  A.dc = P.down.codes_off;
  A.ds = P.down.scales_off;
  A.d = P.d_model;
  A.ffn = P.ffn;
  A.E = (int)L.desc.num_experts;
  A.k = k;
  A.norm = norm;
  A.lg_g = P.gate.lpr_log2;
  A.lg_d = lg_d;
  A.x = x;
  A.rms = rms ? 1 : 0;
  A.eps = eps;
  A.logits = logits;
  A.h = h;
  A.ws_ids = ws_ids;
  A.ws_w = ws_w;
  A.out = out;
  A.accumulate = accumulate;
  A.user_ids = uids;
  A.user_w = uw;
  A.rb = rb;
  // routing split (see DecodeArgs): at most 32 lanes per expert, pairs per
  // lane a multiple of 8, the padded key count within the LDS table
  A.rk_kpw = (A.E + DEC_THREADS / 64 - 1) / (DEC_THREADS / 64);
  A.rk_lg = 0;
  while (A.rk_lg < 5 && (2 << A.rk_lg) * A.rk_kpw <= 64) ++A.rk_lg;
  A.rk_cp = ((A.E + 1) / 2 + (1 << A.rk_lg) - 1) >> A.rk_lg;
  A.rk_cp = (A.rk_cp + 7) / 8 * 8;
  if ((2 * A.rk_cp << A.rk_lg) > DEC_KEYS) return hipSuccess;
  hipError_t e;
  {
    TracedLaunch t(SMOE_KERNEL_GATE_UP);
    e = gu(A, xf32 ? DEC_NWG : DEC_NWG_GU, stream);
  }
  if (e != hipSuccess) return e;
  {
    TracedLaunch t(SMOE_KERNEL_DOWN);
    e = dn(A, DEC_NWG, stream);
  }
  if (e != hipSuccess) return e;
  *launched = true;
  return hipSuccess;
}

hipError_t small_try(const LayerInfo& L, const void* x, bool xf32, bool rms, float eps,
                     const float* logits, int T, int k, int norm, int nsh, int32_t* uids,
                     float* uw, int32_t* ids, float* w, int* meta, int* active, int* offs,
                     int* pair_token, int* pair_of, float* h, hipStream_t stream,
                     bool* launched) {
  *launched = false;
  const ExpertPlan& P = L.plan;
  const int E = (int)L.desc.num_experts, bits = (int)L.desc.bits;
  if (T < 1 || T > SB_TMAX || (int64_t)T * E > SB_KEYS) return hipSuccess;
  if (L.desc.shared_ffn_dim && nsh <= 0) return hipSuccess;
  // a unit's results (tokens x rows per wave load) are staged in 64 floats
  if (T * (64 >> P.gate.lpr_log2) > 64) return hipSuccess;
  SbLaunch sb;
  if (!find_sb_any(bits, (int)L.desc.scale_dtype, P.gate.v, xf32, &sb)) return hipSuccess;
  // dynamic LDS: keys, logits, fp16 pairs (hi, and lo for fp32 inputs), offsets
  const int ppw = 16 / bits;
  const uint64_t xpt = (uint64_t)P.gate.v * ppw * 64;
  SmallArgs A{};
  A.lds_lv = (int)align16((uint64_t)T * E * 8);
  A.lds_xp = (int)align16(A.lds_lv + (uint64_t)T * E * 4);
  A.lds_k = (int)align16(A.lds_xp + (uint64_t)T * (xf32 ? 2 : 1) * xpt * 4);
  A.lds_os = (int)align16(A.lds_k + (uint64_t)T * P.gate.v * 64 * 4);
  A.lds_total = (int)align16(A.lds_os + (uint64_t)T * 4);
  // two workgroups per CU when both fit the 160 KB of LDS (bf16 inputs)
  const uint64_t per_wg = A.lds_total + SB_STATIC_LDS;
  if (per_wg > 150 * 1024) return hipSuccess;
  const int nwg = !xf32 && per_wg <= 78 * 1024 ? DEC_NWG_GU : DEC_NWG;
  A.blobs = L.blobs;
  A.stride = L.desc.blob_stride;
  A.table = L.table;
  A.gc = P.gate.codes_off;
  A.gs = P.gate.scales_off;
  A.uc = P.up.codes_off;
  A.us = P.up.scales_off;
  if (nsh) {
    A.shared = L.shared;
    A.sgc = L.shared_plan.gate.codes_off;
    A.sgs = L.shared_plan.gate.scales_off;
    A.suc = L.shared_plan.up.codes_off;
    A.sus = L.shared_plan.up.scales_off;
  }
  A.d = P.d_model;
  A.ffn = P.ffn;
  A.E = E;
  A.k = k;
  A.T = T;
  A.norm = norm;
  A.nsh = nsh;
  A.lg_g = P.gate.lpr_log2;
  A.x = x;
  A.rms = rms ? 1 : 0;
  A.eps = eps;
  A.logits = logits;
  A.h = h;
  A.ids = ids;
  A.w = w;
  A.meta = meta;
  A.active = active;
  A.offs = offs;
  A.pair_token = pair_token;
  A.pair_of = pair_of;
  A.user_ids = uids;
  A.user_w = uw;
  hipError_t e;
  {
    TracedLaunch t(SMOE_KERNEL_GATE_UP);
    e = sb(A, nwg, stream);
  }
  if (e != hipSuccess) return e;
  *launched = true;
  return hipSuccess;
}

hipError_t small_route_try(const LayerInfo& L, const float* logits, int T, int k, int norm,
                           int nsh, int32_t* uids, float* uw, int32_t* ids, float* w, int* meta,
                           int* active, int* offs, int* pair_token, int* pair_of,
                           hipStream_t stream, bool* launched) {
  *launched = false;
  const ExpertPlan& P = L.plan;
  const int E = (int)L.desc.num_experts, bits = (int)L.desc.bits;
  // one workgroup ranks T x E keys: past 1024 of them the top-k and grouping
  // launches (spread over many workgroups) measured faster
  if (T < 1 || T > SB_TSLOTS || (int64_t)T * E > 1024) return hipSuccess;
  if (L.desc.shared_ffn_dim && nsh <= 0) return hipSuccess;
  SbLaunch sb;
  // any instantiation of the kernel serves (the gate/up part is not run)
  if (!find_sb_any(bits, (int)L.desc.scale_dtype, P.gate.v, false, &sb)) return hipSuccess;
  SmallArgs A{};
  A.lds_lv = (int)align16((uint64_t)T * E * 8);
  A.lds_xp = (int)align16(A.lds_lv + (uint64_t)T * E * 4);
  A.lds_k = A.lds_xp;
  A.lds_os = A.lds_xp;
  A.lds_total = A.lds_xp;
  A.route_only = 1;
  A.blobs = L.blobs;
  A.stride = L.desc.blob_stride;
  A.d = P.d_model;
  A.ffn = P.ffn;
  A.E = E;
  A.k = k;
  A.T = T;
  A.norm = norm;
  A.nsh = nsh;
  A.lg_g = P.gate.lpr_log2;
  A.logits = logits;
  A.ids = ids;
  A.w = w;
  A.meta = meta;
  A.active = active;
  A.offs = offs;
  A.pair_token = pair_token;
  A.pair_of = pair_of;
  A.user_ids = uids;
  A.user_w = uw;
  const hipError_t e = sb(A, 1, stream);
  if (e != hipSuccess) return e;
  *launched = true;
  return hipSuccess;
}

hipError_t small_down_try(const LayerInfo& L, const float* h, int T, int k, int nsh,
                          const int* meta, const int* active, const int* offs,
                          const int* pair_token, const int* pair_of, const float* w, float* out,
                          int accumulate, hipStream_t stream, bool* launched) {
  *launched = false;
  const ExpertPlan& P = L.plan;
  const int bits = (int)L.desc.bits;
  if (T < 1 || T > SB_TSLOTS || k > SMOE_MAX_TOP_K || nsh < 0 || nsh > 16) return hipSuccess;
  if (L.desc.shared_ffn_dim && nsh <= 0) return hipSuccess;
  // the down rows go to at most 16 lanes each, as in the one-token down stage
  const int lg_d = P.down.lpr_log2 < 4 ? P.down.lpr_log2 : 4;
  const int vd = P.down.words_per_row >> lg_d;
  SdLaunch sd;
  if (!find_sd_any(bits, (int)L.desc.scale_dtype, vd, &sd)) return hipSuccess;
  const int rpwd = 64 >> lg_d;
  int rb = (P.d_model + DEC_NWG - 1) / DEC_NWG;
  rb = (rb + rpwd - 1) / rpwd * rpwd;
  rb = rb < sb_down_loads(vd) * rpwd ? rb : sb_down_loads(vd) * rpwd;
  if (rb > SB_DOWN_RB) return hipSuccess;
  // one pair's h as fp16 pairs in the wave's LDS region
  if ((int64_t)P.ffn * bits / 32 > 64 * (DEC_HC / (bits == 2 ? 2 : 1))) return hipSuccess;
  SmallDownArgs A{};
  A.blobs = L.blobs;
  A.stride = L.desc.blob_stride;
  A.table = L.table;
  A.dc = P.down.codes_off;
  A.ds = P.down.scales_off;
  if (nsh) {
    A.shared = L.shared;
    A.sdc = L.shared_plan.down.codes_off;
    A.sds = L.shared_plan.down.scales_off;
  }
  A.d = P.d_model;
  A.ffn = P.ffn;
  A.k = k;
  A.T = T;
  A.nsh = nsh;
  A.lg_d = lg_d;
  A.rb = rb;
  A.h = h;
  A.meta = meta;
  A.active = active;
  A.offs = offs;
  A.pair_token = pair_token;
  A.pair_of = pair_of;
  A.w = w;
  A.out = out;
  A.accumulate = accumulate;
  // dynamic LDS: every pair's h as fp16 pairs, and their offsets
  const uint64_t np = (uint64_t)T * k + (uint64_t)nsh * T;
  if (np > SB_PAIRS) return hipSuccess;
  const uint64_t wd = (uint64_t)P.ffn * bits / 32;
  A.lds_hk = (int)align16(np * wd * (16 / bits) * 4);
  A.lds_total = (int)align16(A.lds_hk + np * wd * 4);
  if (A.lds_total + SD_STATIC_LDS > 150 * 1024) return hipSuccess;
  A.E = (int)L.desc.num_experts;
  const int nwg = (P.d_model + rb - 1) / rb;
  hipError_t e;
  {
    TracedLaunch t(SMOE_KERNEL_DOWN);
    e = sd(A, nwg, stream);
  }
  if (e != hipSuccess) return e;
  *launched = true;
  return hipSuccess;
}

}  // namespace smoe
