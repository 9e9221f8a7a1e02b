// GPU quantiser: SMOE-Q4/Q2 codes and group-64 scales of one weight tensor
// by the 64-candidate squared-error scale search ("SMOE Quantisation",
// L2-MSE Scale Optimiser; Quantisation Levels; Bit Packing).
//
// Groups run over the flattened tensor (the last one may be short). One wave
// per group, lane i scoring candidate i:
//   frac_i  = i * ((1 - 0.1) / 63) + 0.1 in double, frac_63 = 1 (the 64-point
//             linspace from 0.1 to 1.0),
//   s_i     = frac_i * absmax rounded once to the storage dtype (RNE),
//   code    = clamp(rint((w / s_i) * m + m), 0, 2^bits - 1), with w / s_i
//             taken as 0 when s_i == 0,
//   error_i = sum over the group, in element order, of
//             (w - ((code - m) / m) * s_i)^2,
// all in double with every product, quotient and sum rounded on its own (the
// compiler fuses nothing in this file); the lowest error wins, ties to the
// lower candidate. The winner's codes are packed LSB-first (element j of a
// byte at bit (j % per_byte) * bits).
//
// The result is that of the double definition bit for bit; the only shortcut
// is that a code is decided in fp32 when an error bound shows the double
// chain would decide the same (q_code_fast). The decoded level
// (code - m) / m comes from a 16-entry double table computed once per wave.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smoe_internal.hpp"

#pragma clang fp contract(off)

namespace smoe {

// double -> IEEE half, round to nearest even, as one conversion (a detour
// through float could round twice).
__device__ __forceinline__ uint16_t q_f64_to_f16(double d) {
  const uint64_t b = __builtin_bit_cast(uint64_t, d);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int exp = (int)((b >> 52) & 0x7FF);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (exp == 0x7FF) return sign | 0x7C00u | (man ? 0x200u : 0u);
  if (exp == 0) return sign;  // zero or double subnormal: far below half's range
  const int e = exp - 1023 + 15;  // biased half exponent
  uint64_t m;
  int shift;
  uint32_t base;
  if (e >= 1) {  // half normal (or overflow after rounding)
    m = man;
    shift = 42;
    base = (uint32_t)e << 10;
  } else {  // half subnormal: the implicit one joins the mantissa
    shift = 43 - e;
    if (shift > 53) return sign;  // below half the smallest subnormal
    m = man | (1ull << 52);
    base = 0;
  }
  const uint64_t q = m >> shift, rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  uint32_t h = base + (uint32_t)q;
  if (rem > half || (rem == half && (q & 1))) ++h;  // a carry moves into the exponent
  if (h >= 0x7C00u) return sign | 0x7C00u;          // overflow to infinity
  return sign | (uint16_t)h;
}

template <int BITS>
__device__ __forceinline__ double q_encode(double x, double s) {
  constexpr double M = BITS == 4 ? 7.5 : 1.5, CMAX = (double)((1 << BITS) - 1);
  const double nrm = s == 0.0 ? 0.0 : x / s;
  const double c = __builtin_rint(nrm * M + M);
  return c < 0.0 ? 0.0 : (c > CMAX ? CMAX : c);
}

// The code of x under scale s, decided in fp32 where that is provably the
// same decision: t = x * (m / s) + m by one fused fp32 operation differs from
// the double chain fl(fl(fl(x / s) * m) + m) by less than
// 2^-22 * (|t| + 8), so rint agrees unless t lies that close to a half-integer
// inside the clamp range; those elements (a small fraction, exact ties
// included) take the double chain. x == 0 gives t = m exactly.
// inv32 = m / s in fp32, +inf when that overflows (s below ~2^-125); then
// every code of the candidate takes the double chain.
template <int BITS>
__device__ __forceinline__ int q_code_fast(float x32, double x64, float inv32, double s,
                                           int c_zero) {
  constexpr float MF = BITS == 4 ? 7.5f : 1.5f, CMAXF = (float)((1 << BITS) - 1);
  const float t = __builtin_fmaf(x32, inv32, MF);
  const float r = __builtin_rintf(t);
  const float tol = 0x1p-22f * (__builtin_fabsf(t) + 8.0f);
  const bool in_range = t > -0.5f - tol && t < CMAXF + 0.5f + tol;
  const bool near_half = __builtin_fabsf(0.5f - __builtin_fabsf(t - r)) <= tol;
  const bool slow = x32 != 0.0f && (inv32 == __builtin_inff() || (in_range && near_half));
  int c = (int)__builtin_fminf(__builtin_fmaxf(r, 0.0f), CMAXF);
  c = x32 == 0.0f ? c_zero : c;
  if (slow) c = (int)q_encode<BITS>(x64, s);
  return c;
}

template <int BITS, bool F16>
__global__ __launch_bounds__(256) void k_quantise(const float* __restrict__ w, int64_t n,
                                                  uint8_t* __restrict__ codes,
                                                  void* __restrict__ scales) {
  constexpr double M = BITS == 4 ? 7.5 : 1.5;
  constexpr int NL = 1 << BITS;
  __shared__ float s_w[4][64];
  __shared__ double s_w64[4][64];
  __shared__ double s_err[4][64];
  __shared__ double s_lv[4][NL];
  __shared__ uint8_t s_code[4][64];
  const int lane = threadIdx.x & 63, wl = threadIdx.x >> 6;
  const int64_t g = (int64_t)blockIdx.x * 4 + wl;
  if (g * 64 >= n) return;  // wave-uniform; nothing below waits on the workgroup
  const int len = (int)(n - g * 64 < 64 ? n - g * 64 : 64);
  const float wv = lane < len ? w[g * 64 + lane] : 0.0f;
  s_w[wl][lane] = wv;
  s_w64[wl][lane] = (double)wv;
  if (lane < NL) s_lv[wl][lane] = ((double)lane - M) / M;  // the decoded levels
  float a = fabsf(wv);
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  const double absmax = (double)a;
  const double step = (1.0 - 0.1) / 63.0;
  const double frac = lane == 63 ? 1.0 : (double)lane * step + 0.1;
  const double prod = frac * absmax;
  double s;
  uint32_t sbits;
  if constexpr (F16) {
    const uint16_t h = q_f64_to_f16(prod);
    s = (double)__builtin_bit_cast(_Float16, h);
    sbits = h;
  } else {
    const float f = (float)prod;
    s = (double)f;
    sbits = __builtin_bit_cast(uint32_t, f);
  }
  // m / s in fp32 (s is exact in fp32 for both storage dtypes); 0 for s == 0
  // (then t = m, as the double chain reads w / s as 0)
  const float s32 = (float)s;
  const float inv32 = s == 0.0 ? 0.0f : (float)M / s32;
  const int c_zero = (int)__builtin_rint(M);
  __builtin_amdgcn_wave_barrier();
  double err = 0.0;
#pragma unroll 4
  for (int j = 0; j < len; ++j) {
    const double x = s_w64[wl][j];
    const int c = q_code_fast<BITS>(s_w[wl][j], x, inv32, s, c_zero);
    const double dec = s_lv[wl][c] * s;
    const double dd = x - dec;
    err = err + dd * dd;
  }
  s_err[wl][lane] = err;
  __builtin_amdgcn_wave_barrier();
  // first minimum (every lane scans the same values, so all agree)
  int best = 0;
  double be = s_err[wl][0];
  for (int i = 1; i < 64; ++i) {
    const double e = s_err[wl][i];
    if (e < be) {
      be = e;
      best = i;
    }
  }
  best = __builtin_amdgcn_readfirstlane(best);
  const uint64_t sb64 = __builtin_bit_cast(uint64_t, s);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sb64, best);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(sb64 >> 32), best);
  const double sw = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
  const uint32_t swb = (uint32_t)__builtin_amdgcn_readlane((int)sbits, best);
  s_code[wl][lane] = lane < len ? (uint8_t)q_encode<BITS>((double)wv, sw) : (uint8_t)0;
  __builtin_amdgcn_wave_barrier();
  // one byte per lane: PER codes, the first in the low bits
  constexpr int PER = 8 / BITS;
  const int nbytes = (len * BITS + 7) / 8;
  if (lane < nbytes) {
    uint32_t byte = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) byte |= (uint32_t)s_code[wl][lane * PER + q] << (q * BITS);
    codes[g * (64 * BITS / 8) + lane] = (uint8_t)byte;
  }
  if (lane == 0) {
    if constexpr (F16)
      ((uint16_t*)scales)[g] = (uint16_t)swb;
    else
      ((uint32_t*)scales)[g] = swb;
  }
}

hipError_t launch_quantise(const float* w, int64_t n, int bits, int f16, uint8_t* codes,
                           void* scales, hipStream_t s) {
  const int64_t groups = (n + 63) / 64;
  const dim3 grid((unsigned)((groups + 3) / 4)), block(256);
  if (bits == 4) {
    if (f16) hipLaunchKernelGGL((k_quantise<4, true>), grid, block, 0, s, w, n, codes, scales);
    else hipLaunchKernelGGL((k_quantise<4, false>), grid, block, 0, s, w, n, codes, scales);
  } else {
    if (f16) hipLaunchKernelGGL((k_quantise<2, true>), grid, block, 0, s, w, n, codes, scales);
    else hipLaunchKernelGGL((k_quantise<2, false>), grid, block, 0, s, w, n, codes, scales);
  }
  return hipGetLastError();
}

}  // namespace smoe
