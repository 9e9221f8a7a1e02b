// Device helpers (gfx950) for the SMOE routed-expert MoE FFN: code-word
// decode into fp16 pairs, dot products, DPP segment reductions, loads.
//
// Weight decode ("SMOE Quantisation", Quantisation Levels / Bit Packing /
// Decoding): a weight is (code - m) / m * scale, m = 7.5 (Q4) or 1.5 (Q2),
// codes packed least-significant-bits first, one scale per 64 consecutive
// weights of a row (".smoe Binary Format", Expert Blob Architecture).
//
// Inner product. For one 32-bit code word w the kernel forms fp16 pairs
// without shifting each code down: (w & mask) | 0x6400 puts a code field that
// sits at bit position b (b < 10) into the mantissa of an fp16 whose value is
// 1024 + code * 2^b. Two such fields (one per 16-bit half) make an f16x2, and
// v_dot2_f32_f16 multiplies it by a pair of activations that were divided by
// 2^b beforehand, accumulating in fp32. Summing over a word gives
//   sum_i code_i * x_i + 1024 * sum(X) ,
// so  sum_i (code_i - m) * x_i = dot - K  with the per-lane constant
//   K = sum over the word's activation fp16 values X of X * (1024 + m * 2^b).
// K depends only on the activation vector, so it is computed once per vector
// and reused for every row and every expert. Q4 needs one shift per word (the
// fields at bits 8..15 of each half), Q2 likewise (four 2-bit fields per byte).
// The activation vector is scaled by a power of two before the fp16 rounding
// so that its largest magnitude sits just below 2^14 (exact rescaling; undone
// in the row's output factor).
//
// Work mapping. A row of W 32-bit code words is read by LPR lanes holding V
// consecutive words each (W = LPR * V, LPR a power of two <= 64), so one wave
// load covers 64 / LPR whole rows with 16/12/8/4-byte loads per lane. A lane
// always sees the same columns, so its activation pairs stay in VGPRs for all
// rows. Row partial sums are reduced across the LPR lanes with DPP.

#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace smoe {

// Blob of routed expert e: base + e * stride, or table[e] when the layer runs
// with an expert-pointer table (experts in a device cache or in host memory
// the device can read).
// A table entry is cast through the global address space so that the loads
// from the blob stay global loads (a plain pointer read from memory would be
// generic and turn every weight load into a flat load).
__device__ __forceinline__ const uint8_t* expert_blob(const uint8_t* base, uint64_t stride,
                                                      const uint64_t* table, int e) {
  typedef const __attribute__((address_space(1))) uint8_t* global_bytes;
  return table ? (const uint8_t*)(global_bytes)table[e] : base + (uint64_t)e * stride;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef u32x3 u32x3_a4 __attribute__((aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef f32x4 f32x4_a4 __attribute__((aligned(4)));

template <int BITS>
struct QT {
  static constexpr int WPW = 32 / BITS;  // codes per 32-bit word
  static constexpr int PPW = WPW / 2;    // fp16 pairs per word
  static constexpr int NPOS = 8 / BITS;  // code fields per byte
  static constexpr int WPG = 64 / WPW;   // words per 64-weight group
  static constexpr float M = BITS == 4 ? 7.5f : 1.5f;
};

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float fdot2(uint32_t a, f16x2 b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), b, c, false);
}

template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, RMASK, 0xF, false));
}

// Sum over aligned segments of 2^lg lanes. The full sum is valid in the
// segment's last lane (and in every lane of the segment when lg <= 4).
__device__ __forceinline__ float seg_sum(float v, int lg) {
  if (lg >= 1) v += dpp<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  if (lg >= 2) v += dpp<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  if (lg >= 3) v += dpp<0x141, 0xF>(v);  // row_half_mirror
  if (lg >= 4) v += dpp<0x140, 0xF>(v);  // row_mirror
  if (lg >= 5) v += dpp<0x142, 0xA>(v);  // row_bcast15 into rows 1, 3
  if (lg >= 6) v += dpp<0x143, 0xC>(v);  // row_bcast31 into rows 2, 3
  return v;
}

// Max over a segment for non-negative values (masked-off rows read 0).
__device__ __forceinline__ float seg_max(float v, int lg) {
  if (lg >= 1) v = fmaxf(v, dpp<0xB1, 0xF>(v));
  if (lg >= 2) v = fmaxf(v, dpp<0x4E, 0xF>(v));
  if (lg >= 3) v = fmaxf(v, dpp<0x141, 0xF>(v));
  if (lg >= 4) v = fmaxf(v, dpp<0x140, 0xF>(v));
  if (lg >= 5) v = fmaxf(v, dpp<0x142, 0xA>(v));
  if (lg >= 6) v = fmaxf(v, dpp<0x143, 0xC>(v));
  return v;
}

__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Lane <-> code-word map of one row of W = LPR * V 32-bit code words spread
// over LPR lanes. A lane's V words come as N4 = V / 4 chunks of four words and
// a tail of R = V % 4 words: chunk c of lane lr holds words
// c*4*LPR + 4*lr + [0, 4), the tail holds words 4*N4*LPR + R*lr + [0, R).
// Each load instruction therefore reads one contiguous span across the lanes
// of a row (16-byte chunks, then 4/8/12-byte tails). Slot s of a lane is its
// s-th word in this order.
template <int V>
struct LaneMap {
  static constexpr int N4 = V / 4;
  static constexpr int R = V % 4;
  static __device__ __forceinline__ int word(int lr, int LPR, int s) {
    return s < 4 * N4 ? (s >> 2) * 4 * LPR + 4 * lr + (s & 3)
                      : 4 * N4 * LPR + R * lr + (s - 4 * N4);
  }
};

template <int V, bool NT>
__device__ __forceinline__ void load_row_words(const uint32_t* __restrict__ row, int lr, int LPR,
                                               uint32_t (&w)[V]) {
  using LM = LaneMap<V>;
#pragma unroll
  for (int c = 0; c < LM::N4; ++c) {
    const u32x4_a4* p = (const u32x4_a4*)(row + c * 4 * LPR + 4 * lr);
    const u32x4 t = NT ? __builtin_nontemporal_load(p) : *p;
    w[4 * c + 0] = t.x;
    w[4 * c + 1] = t.y;
    w[4 * c + 2] = t.z;
    w[4 * c + 3] = t.w;
  }
  constexpr int B = 4 * LM::N4;
  const uint32_t* tail = row + B * LPR + LM::R * lr;
  if constexpr (LM::R == 3) {
    const u32x3 t = NT ? __builtin_nontemporal_load((const u32x3_a4*)tail) : *(const u32x3_a4*)tail;
    w[B] = t.x;
    w[B + 1] = t.y;
    w[B + 2] = t.z;
  } else if constexpr (LM::R == 2) {
    const u32x2 t = NT ? __builtin_nontemporal_load((const u32x2_a4*)tail) : *(const u32x2_a4*)tail;
    w[B] = t.x;
    w[B + 1] = t.y;
  } else if constexpr (LM::R == 1) {
    w[B] = NT ? __builtin_nontemporal_load(tail) : *tail;
  }
}

template <typename ST, bool NT>
__device__ __forceinline__ float load_scale(const ST* p) {
  return NT ? (float)__builtin_nontemporal_load(p) : (float)*p;
}

// (v & mask) | magic as one v_and_or_b32. A VOP3 instruction on gfx9-class
// targets takes no literal and reads at most one SGPR, so the mask comes in an
// SGPR and the magic in a VGPR; written as plain C the pair compiles to two
// VOP2 instructions with literals.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(magic));
  return r;
}

// Sum over one code word of (code_i - m) * x_i (up to the K offset, which the
// caller folds into acc): see the file comment.
template <int BITS>
__device__ __forceinline__ float dot_word(uint32_t w, const f16x2* xp, float acc) {
  constexpr int NPOS = QT<BITS>::NPOS;
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const uint32_t v = hs ? (w >> 8) : w;
#pragma unroll
    for (int pos = 0; pos < NPOS; ++pos) {
      constexpr uint32_t base = (1u << BITS) - 1u;
      const uint32_t m = (base << (BITS * pos)) | (base << (BITS * pos + 16));
      acc = fdot2(and_or(v, m, 0x64006400u), xp[hs * NPOS + pos], acc);
    }
  }
  return acc;
}

// Per-lane registers derived from one activation vector.
template <int BITS, int V, bool SPLIT>
struct XRegs {
  static constexpr int PPW = QT<BITS>::PPW;
  f16x2 hi[V][PPW];
  f16x2 lo[SPLIT ? V : 1][SPLIT ? PPW : 1];
  float K[V];
  float oscale;  // multiply a reduced row sum by this
};

// Reads the lane's V*WPW activations (the columns of its code words, see
// LaneMap) from a bf16 or fp32 vector, rescales by a power of two, optionally applies unit-gain
// RMSNorm (as a factor on the output), and builds the fp16 pairs and K.
template <int BITS, int V, bool SPLIT, bool BF16>
__device__ __forceinline__ void prep_x(XRegs<BITS, V, SPLIT>& X, const void* vec, int lr,
                                       int lg, bool rms, float eps, int n) {
  constexpr int WPW = QT<BITS>::WPW;
  constexpr int NPOS = QT<BITS>::NPOS;
  constexpr int PPW = QT<BITS>::PPW;
  const int LPR = 1 << lg;
  auto load_word_vals = [&](int w, float (&xv)[WPW]) {
    const int col0 = LaneMap<V>::word(lr, LPR, w) * WPW;
    if constexpr (BF16) {
      const uint32_t* p = (const uint32_t*)((const uint16_t*)vec + col0);
#pragma unroll
      for (int i = 0; i < WPW / 8; ++i) {
        u32x4 t = *(const u32x4_a4*)(p + 4 * i);
        uint32_t tt[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xv[8 * i + 2 * j] = __builtin_bit_cast(float, tt[j] << 16);
          xv[8 * i + 2 * j + 1] = __builtin_bit_cast(float, tt[j] & 0xFFFF0000u);
        }
      }
    } else {
      const float* p = (const float*)vec + col0;
#pragma unroll
      for (int i = 0; i < WPW / 4; ++i) {
        f32x4 t = *(const f32x4_a4*)(p + 4 * i);
        xv[4 * i + 0] = t.x;
        xv[4 * i + 1] = t.y;
        xv[4 * i + 2] = t.z;
        xv[4 * i + 3] = t.w;
      }
    }
  };
  // pass 1: max |x| and sum of squares over the vector (one segment holds it)
  float amax = 0.f, ss = 0.f;
#pragma unroll
  for (int w = 0; w < V; ++w) {
    float xv[WPW];
    load_word_vals(w, xv);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      amax = fmaxf(amax, fabsf(xv[i]));
      ss = fmaf(xv[i], xv[i], ss);
    }
  }
  amax = lane63(seg_max(amax, lg));
  int ex = 0;
  frexpf(amax, &ex);
  ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
  const float S = ldexpf(1.0f, 14 - ex);
  float r = 1.0f;
  if (rms) {
    ss = lane63(seg_sum(ss, lg));
    r = 1.0f / sqrtf(ss / (float)n + eps);
  }
  X.oscale = r / (QT<BITS>::M * S);
  // pass 2: fp16 pairs and offsets
#pragma unroll
  for (int w = 0; w < V; ++w) {
    float xv[WPW];
    load_word_vals(w, xv);
    float k = 0.f;
#pragma unroll
    for (int q = 0; q < PPW; ++q) {
      const int hs = q / NPOS, pos = q % NPOS;
      const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
      const float f = S * (1.0f / (float)(1 << (BITS * pos)));
      const float a = xv[ia] * f, b = xv[ib] * f;
      const _Float16 ha = (_Float16)a, hb = (_Float16)b;
      X.hi[w][q] = f16x2{ha, hb};
      float sumx = (float)ha + (float)hb;
      if constexpr (SPLIT) {
        const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
        X.lo[w][q] = f16x2{la, lb};
        sumx += (float)la + (float)lb;
      }
      k = fmaf(sumx, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)), k);
    }
    X.K[w] = k;
  }
}

// Scales a lane needs for one row. A 4-word chunk never straddles a scale
// group (a group is 8 words for Q4, 4 for Q2, and chunks are 4-aligned), so
// each chunk takes one scale; a 3-word tail may straddle two groups, the
// others take one.
template <int BITS, int V>
struct ScalePlan {
  static constexpr int WPG = QT<BITS>::WPG;
  static constexpr int N4 = LaneMap<V>::N4;
  static constexpr int R = LaneMap<V>::R;
  static constexpr int NT = R == 3 ? 2 : (R > 0 ? 1 : 0);
  static constexpr int NS = N4 + NT;
};

// Group index of each of the lane's scales, and (tmask) which tail words sit
// in the tail's second group.
template <int BITS, int V>
__device__ __forceinline__ void scale_groups(int lr, int LPR, int (&g)[ScalePlan<BITS, V>::NS],
                                             int& tmask) {
  using SP = ScalePlan<BITS, V>;
  using LM = LaneMap<V>;
#pragma unroll
  for (int c = 0; c < SP::N4; ++c) g[c] = LM::word(lr, LPR, 4 * c) / SP::WPG;
  tmask = 0;
  if constexpr (SP::R > 0) {
    const int gt = LM::word(lr, LPR, 4 * SP::N4) / SP::WPG;
    g[SP::N4] = gt;
    if constexpr (SP::NT == 2) g[SP::N4 + 1] = gt + 1;
#pragma unroll
    for (int t = 0; t < SP::R; ++t)
      if (LM::word(lr, LPR, 4 * SP::N4 + t) / SP::WPG != gt) tmask |= 1 << t;
  }
}

template <int BITS, int V, typename ST, bool NT>
__device__ __forceinline__ void load_row_scales(const ST* __restrict__ row_scales,
                                                const int (&g)[ScalePlan<BITS, V>::NS], int G,
                                                float (&s)[ScalePlan<BITS, V>::NS]) {
#pragma unroll
  for (int j = 0; j < ScalePlan<BITS, V>::NS; ++j)
    s[j] = load_scale<ST, NT>(row_scales + (g[j] < G ? g[j] : G - 1));
}

// Fold the per-word offsets to one per scale: K[c] = sum over chunk c's four
// words, then the tail words' own offsets. Call once after the pairs are built.
template <int BITS, int V, bool SPLIT>
__device__ __forceinline__ void fold_k(XRegs<BITS, V, SPLIT>& X) {
  using SP = ScalePlan<BITS, V>;
#pragma unroll
  for (int c = 0; c < SP::N4; ++c)
    X.K[c] = X.K[4 * c] + X.K[4 * c + 1] + X.K[4 * c + 2] + X.K[4 * c + 3];
#pragma unroll
  for (int t = 0; t < SP::R; ++t) X.K[SP::N4 + t] = X.K[4 * SP::N4 + t];
}

// Sum over the lane's words of scale(word) * (dot - K), for one row (K folded).
template <int BITS, int V, bool SPLIT>
__device__ __forceinline__ float lane_row(const uint32_t (&cw)[V], const XRegs<BITS, V, SPLIT>& X,
                                          const float (&s)[ScalePlan<BITS, V>::NS], int tmask) {
  using SP = ScalePlan<BITS, V>;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < SP::N4; ++c) {
    float a = -X.K[c];
#pragma unroll
    for (int w = 4 * c; w < 4 * c + 4; ++w) {
      a = dot_word<BITS>(cw[w], X.hi[w], a);
      if constexpr (SPLIT) a = dot_word<BITS>(cw[w], X.lo[w], a);
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
      float a = dot_word<BITS>(cw[w], X.hi[w], -X.K[SP::N4 + t]);
      if constexpr (SPLIT) a = dot_word<BITS>(cw[w], X.lo[w], a);
      const float sc = (SP::NT == 2 && ((tmask >> t) & 1)) ? t1 : t0;
      acc = fmaf(a, sc, acc);
    }
  }
  return acc;
}

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

}  // namespace smoe
