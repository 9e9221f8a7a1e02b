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

template <int V>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t (&w)[V]) {
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {
    u32x4 t = *(const u32x4_a4*)(p + 4 * i);
    w[4 * i + 0] = t.x;
    w[4 * i + 1] = t.y;
    w[4 * i + 2] = t.z;
    w[4 * i + 3] = t.w;
  }
  constexpr int B = V - V % 4;
  if constexpr (V % 4 == 3) {
    u32x3 t = *(const u32x3_a4*)(p + B);
    w[B] = t.x;
    w[B + 1] = t.y;
    w[B + 2] = t.z;
  } else if constexpr (V % 4 == 2) {
    u32x2 t = *(const u32x2_a4*)(p + B);
    w[B] = t.x;
    w[B + 1] = t.y;
  } else if constexpr (V % 4 == 1) {
    w[B] = p[B];
  }
}

template <typename ST>
__device__ __forceinline__ float load_scale(const ST* p) {
  return (float)*p;
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
      acc = fdot2((v & m) | 0x64006400u, xp[hs * NPOS + pos], acc);
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

// Reads the lane's V*WPW activations (columns [lr*V*WPW, ...)) from a bf16 or
// fp32 vector, rescales by a power of two, optionally applies unit-gain
// RMSNorm (as a factor on the output), and builds the fp16 pairs and K.
template <int BITS, int V, bool SPLIT, bool BF16>
__device__ __forceinline__ void prep_x(XRegs<BITS, V, SPLIT>& X, const void* vec, int lr,
                                       int lg, bool rms, float eps, int n) {
  constexpr int WPW = QT<BITS>::WPW;
  constexpr int NPOS = QT<BITS>::NPOS;
  constexpr int PPW = QT<BITS>::PPW;
  const int col0 = lr * V * WPW;
  auto load_word_vals = [&](int w, float (&xv)[WPW]) {
    if constexpr (BF16) {
      const uint32_t* p = (const uint32_t*)((const uint16_t*)vec + col0 + w * WPW);
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
      const float* p = (const float*)vec + col0 + w * WPW;
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

// Scales a lane needs for one row: its V words touch groups g0 .. g0+NS-1.
template <int BITS, int V>
struct ScalePlan {
  static constexpr int WPG = QT<BITS>::WPG;
  static constexpr bool ALIGNED = (V % WPG) == 0;  // lane starts a group
  static constexpr bool WITHIN = (WPG % V) == 0;   // lane inside one group
  static constexpr int NS = ALIGNED ? V / WPG : (WITHIN ? 1 : (V - 1) / WPG + 2);
};

// Sum over the lane's words of scale(word) * (dot - K), for one row.
template <int BITS, int V, bool SPLIT, typename ST>
__device__ __forceinline__ float lane_row(const uint32_t (&cw)[V], const XRegs<BITS, V, SPLIT>& X,
                                          const float (&s)[ScalePlan<BITS, V>::NS],
                                          const int (&slot)[V]) {
  using SP = ScalePlan<BITS, V>;
  float acc = 0.f;
  if constexpr (SP::ALIGNED || SP::WITHIN) {
    constexpr int WG = SP::ALIGNED ? SP::WPG : V;  // words sharing one scale
#pragma unroll
    for (int g = 0; g < SP::NS; ++g) {
      float kk = 0.f;
#pragma unroll
      for (int w = g * WG; w < (g + 1) * WG; ++w) kk += X.K[w];
      float a = -kk;
#pragma unroll
      for (int w = g * WG; w < (g + 1) * WG; ++w) {
        a = dot_word<BITS>(cw[w], X.hi[w], a);
        if constexpr (SPLIT) a = dot_word<BITS>(cw[w], X.lo[w], a);
      }
      acc = fmaf(a, s[g], acc);
    }
  } else {
#pragma unroll
    for (int w = 0; w < V; ++w) {
      float a = dot_word<BITS>(cw[w], X.hi[w], -X.K[w]);
      if constexpr (SPLIT) a = dot_word<BITS>(cw[w], X.lo[w], a);
      float sc = s[0];
#pragma unroll
      for (int j = 1; j < SP::NS; ++j) sc = slot[w] >= j ? s[j] : sc;
      acc = fmaf(a, sc, acc);
    }
  }
  return acc;
}

template <int BITS, int V, typename ST>
__device__ __forceinline__ void load_scales(const ST* __restrict__ row_scales, int g0, int G,
                                            float (&s)[ScalePlan<BITS, V>::NS]) {
#pragma unroll
  for (int j = 0; j < ScalePlan<BITS, V>::NS; ++j) {
    const int g = g0 + j < G ? g0 + j : G - 1;
    s[j] = load_scale(row_scales + g);
  }
}

}  // namespace smoe
