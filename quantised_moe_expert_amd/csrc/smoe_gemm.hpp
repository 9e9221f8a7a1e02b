// Grouped expert stages for batches on the matrix cores (gate/up + SwiGLU,
// and down), v_mfma_f32_16x16x32_f16.
//
// Grid (row blocks, active-expert slots), 4-wave workgroups. Per MFMA the M
// dimension is up to 16 tokens of the slot, N is 16 weight rows, K is 32
// weights of one scale group; a group (64 weights) takes two MFMAs.
//   - B (weights): lane l holds row l % 16, k-block b = l / 16 of each
//     MFMA: for Q4 one word per MFMA, for Q2 one word whose low pairs feed
//     the first MFMA and high pairs the second. Lanes load 16 bytes of their
//     row (two Q4 groups or four Q2 groups per wave-wide load) and cross-
//     lane swaps hand each quarter its k-blocks. A word becomes fp16 pairs
//     1024 + code * 2^p by one v_and_or_b32 per pair.
//   - A (tokens): the slot's token vectors staged once per workgroup in LDS
//     as fp16 pairs pre-divided by 2^p (scaled per token by a power of two so
//     the largest magnitude sits just below 2^14), in the same pair order as
//     the decoded words, laid out so that the 16 token rows of one word are
//     contiguous; lanes of token rows past the chunk read stale rows whose
//     D rows are dropped.
//   - per group, with D the two MFMAs' sum: acc += scale[row][g] *
//     (D - K[g][token]), where K = sum over the group of the staged pairs
//     times (1024 + m * 2^p) removes both the 1024 offsets and the code
//     midpoint m.
// When the grid would have few workgroups (the shared expert), the four
// waves split the groups of one 16-row tile and add their partial sums in
// LDS.

#pragma once

#include <type_traits>

#include "smoe_device.hpp"
#include "smoe_gemv_args.hpp"
#include "smoe_launch.hpp"

namespace smoe {

// scale groups per weight load batch (a multiple of 4)
constexpr int GM_GB = 8;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

// Stage pairs [pc, pc + nt) of the slot for the matrix-core stage. Two
// passes over the activations: the largest magnitude and sum of squares of
// every token, then the fp16 pairs of every (token, code word) with the
// group offsets K summed across the WPG lanes that hold a group. In both,
// each thread has NB loads in flight before it uses any (under a weight
// stream a load takes microseconds, so staging costs a few round trips,
// not one or more per token).
template <int BITS, int IN, bool GU, int NW>
__device__ __forceinline__ void gm_stage(const GemvArgs& A, const MatArgs& M, uint32_t* lds,
                                         const GmLds& L, int pc, int nt) {
  constexpr int WPW = QT<BITS>::WPW, PPW = QT<BITS>::PPW, NPOS = QT<BITS>::NPOS;
  constexpr int WPG = QT<BITS>::WPG;  // words per group
  constexpr bool XF32 = IN != GV_BF16, SPLIT = IN == GV_F32_SPLIT;
  constexpr int NT = NW * 64;
  constexpr int VW = XF32 ? WPW : WPW / 2;  // registers of one loaded word
  constexpr int NB = VW >= 16 ? 1 : 16 / VW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cols = M.cols, Wr = M.words_per_row, TC = A.tc;
  const size_t esz = XF32 ? 4 : 2;
  // lane l (< nt) holds the activation row of the chunk's token l
  const int tl = pc + min(lane, nt - 1);
  const int rowl = (GU && !A.shared) ? A.pair_token[tl] : tl;
  auto vec = [&](int i) {
    const int t = __builtin_amdgcn_readlane(rowl, i);
    return (const void*)((const uint8_t*)A.x + (size_t)t * A.x_ld * esz);
  };
  float* red = (float*)(lds + L.red);
  for (int i0 = 0; i0 < nt; i0 += NB) {
    float amax[NB], ss[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) amax[q] = ss[q] = 0.f;
    for (int cw = tid; cw < Wr; cw += NT) {
      float xv[NB][WPW];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        if (i0 + q < nt) {  // uniform
          gv_load_word<BITS, XF32>(vec(i0 + q), cw, xv[q]);
        } else {
#pragma unroll
          for (int j = 0; j < WPW; ++j) xv[q][j] = 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int j = 0; j < WPW; ++j) {
          amax[q] = fmaxf(amax[q], fabsf(xv[q][j]));
          ss[q] = fmaf(xv[q][j], xv[q][j], ss[q]);
        }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const float m = lane63(seg_max(amax[q], 6)), s2 = lane63(seg_sum(ss[q], 6));
      if (lane == 0 && i0 + q < nt) {
        red[((i0 + q) * NW + wave) * 2] = m;
        red[((i0 + q) * NW + wave) * 2 + 1] = s2;
      }
    }
  }
  __syncthreads();
  float* Kl = (float*)(lds + L.k);
  float* osc = (float*)(lds + L.osc);
  uint32_t* X = lds + L.x;
  uint32_t* Xlo = lds + L.xlo;
  // per token: the power-of-two scale S (kept where its first partial was)
  // and the output factor
  if (tid < nt) {
    float m = 0.f, q2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      m = fmaxf(m, red[(tid * NW + w) * 2]);
      q2 += red[(tid * NW + w) * 2 + 1];
    }
    int ex = 0;
    frexpf(m, &ex);
    ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
    const float S = ldexpf(1.0f, 14 - ex);
    const float r = A.rms ? 1.0f / sqrtf(q2 / (float)cols + A.eps) : 1.0f;
    osc[tid] = r / (QT<BITS>::M * S);
    red[tid * NW * 2] = S;
  }
  __syncthreads();
  // unit u: code word cw = u % Wr of token i = u / Wr; its pairs go to
  // X[((cw * HALVES + hv) * TC + i) * 4 + (q % 4)] with hv = q / 4 (split
  // inputs: the hi halves there, the lo halves at the same place in Xlo).
  // Wr and NT are multiples of WPG, so the WPG lanes of a group's words are
  // consecutive and belong to one token.
  constexpr int HALVES = PPW / 4;
  constexpr int LGW = WPG == 8 ? 3 : 2;
  static_assert((1 << LGW) == WPG, "words per group");
  const int nu = nt * Wr;
  for (int u0 = 0; u0 < nu; u0 += NT * NB) {
    float xv[NB][WPW];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int u = u0 + q * NT + tid;
      const int i = min(u / Wr, nt - 1);
      const int ti = __shfl(rowl, i, 64);  // every lane takes part
      if (u < nu) {
        gv_load_word<BITS, XF32>((const uint8_t*)A.x + (size_t)ti * A.x_ld * esz, u - i * Wr, xv[q]);
      } else {
#pragma unroll
        for (int j = 0; j < WPW; ++j) xv[q][j] = 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int u = u0 + q * NT + tid;
      const bool in = u < nu;
      const int i = in ? u / Wr : 0, cw = in ? u - i * Wr : 0;
      const float S = red[i * NW * 2];
      float kk = 0.f;
#pragma unroll
      for (int qq = 0; qq < PPW; ++qq) {
        const int hs = qq / NPOS, pos = qq % NPOS;
        const int ia = hs * NPOS + pos, ib = ia + WPW / 2;
        const float f = S * (1.0f / (float)(1 << (BITS * pos)));
        const float a = xv[q][ia] * f, bb = xv[q][ib] * f;
        const _Float16 ha = (_Float16)a, hb = (_Float16)bb;
        const int xi = ((cw * HALVES + qq / 4) * TC + i) * 4 + (qq % 4);
        if (in) X[xi] = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
        float sumx = (float)ha + (float)hb;
        if constexpr (SPLIT) {
          const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(bb - (float)hb);
          if (in) Xlo[xi] = __builtin_bit_cast(uint32_t, f16x2{la, lb});
          sumx += (float)la + (float)lb;
        }
        kk = fmaf(sumx, 1024.0f + QT<BITS>::M * (float)(1 << (BITS * pos)), kk);
      }
      kk = seg_sum(kk, LGW);
      // stored negated: the MFMA chains start from it
      if (in && (cw & (WPG - 1)) == WPG - 1) Kl[(cw / WPG) * 16 + i] = -kk;
    }
  }
  // K of the token rows past the chunk (their D rows are never used)
  for (int u = tid; u < (cols / 64) * 16; u += NT)
    if ((u & 15) >= nt) Kl[u] = 0.f;
  __syncthreads();
}

// A constant in a scalar register the optimiser cannot see through.
__device__ __forceinline__ uint32_t gm_sreg(uint32_t c) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(c));
  return r;
}

// Decoded fp16 pairs 4h .. 4h + 3 of a code word, as one MFMA operand.
// (v & mask) | magic is written in C with the mask in an SGPR and the magic
// in a VGPR, so the compiler emits one v_and_or_b32 of its own: an MFMA that
// reads a VGPR written by VALU code needs wait states, and the compiler
// counts them only for instructions it generated (not for inline asm).
template <int BITS>
__device__ __forceinline__ h8 gm_operand(uint32_t w, int h, uint32_t magic) {
  constexpr int NPOS = QT<BITS>::NPOS;
  constexpr uint32_t base = (1u << BITS) - 1u;
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 4 * h + j, hs = q / NPOS, pos = q % NPOS;
    const uint32_t v = hs ? (w >> 8) : w;
    const uint32_t m = gm_sreg((base << (BITS * pos)) | (base << (BITS * pos + 16)));
    p[j] = (v & m) | magic;
  }
  const u32x4 t = {p[0], p[1], p[2], p[3]};
  return __builtin_bit_cast(h8, t);
}

// Four consecutive scales of one row starting at group q (a multiple of
// four, q + 4 <= G), as float bit patterns.
template <typename ST>
__device__ __forceinline__ u32x4 gm_scale_quad(const ST* rs, int q) {
  if constexpr (sizeof(ST) == 4) {
    return *(const u32x4_a4*)(rs + q);
  } else {
    const u32x2 t = *(const u32x2_a4*)(rs + q);
    const uint32_t lo = t.x, hi = t.y;
    const f16x2 a = __builtin_bit_cast(f16x2, lo), c = __builtin_bit_cast(f16x2, hi);
    const _Float16 a0 = a.x, a1 = a.y, c0 = c.x, c1 = c.y;
    return u32x4{__builtin_bit_cast(uint32_t, (float)a0), __builtin_bit_cast(uint32_t, (float)a1),
                 __builtin_bit_cast(uint32_t, (float)c0), __builtin_bit_cast(uint32_t, (float)c1)};
  }
}

// v_permlane32_swap: lanes 32..63 of a trade places with lanes 0..31 of c.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& c) {
  const auto t = __builtin_amdgcn_permlane32_swap(a, c, false, false);
  a = t[0];
  c = t[1];
}
// v_permlane16_swap: lanes 16..31 and 48..63 of a trade places with lanes
// 0..15 and 32..47 of c.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& c) {
  const auto t = __builtin_amdgcn_permlane16_swap(a, c, false, false);
  a = t[0];
  c = t[1];
}

// Code words of one load unit of a row: 16 bytes per lane, 2 groups for Q4
// and 4 for Q2. Lane quarter b = lane / 16 loads
//   Q4: words (b & 1) * 4 .. + 3 of group u0 + (b >> 1);
//   Q2: all four words of group u0 + b
// (groups past the row read its last group; their results are unused). A
// lane reads 16 bytes, twice the words of one k-block, so that each load
// instruction moves a full kilobyte.
template <int BITS>
__device__ __forceinline__ u32x4 gm_unit_load(const uint32_t* row_codes, int u0, int G, int b) {
  constexpr int WPG = QT<BITS>::WPG;
  const int g = min(u0 + (BITS == 4 ? (b >> 1) : b), G - 1);
  return *(const u32x4*)(row_codes + g * WPG + (BITS == 4 ? (b & 1) * 4 : 0));
}

// Swaps across lane quarters that give every quarter one k-block of each
// group of a loaded unit:
//   Q4: w[0], w[1] hold words wmap(b), wmap(b) + 1 of the unit's first
//       group (one per MFMA) and w[2], w[3] the same words of the second,
//       with wmap(b) = (b & 1) * 4 + (b >> 1) * 2;
//   Q2: a 4 x 4 transpose: w[j] holds word b of the unit's group j.
template <int BITS>
__device__ __forceinline__ void gm_unit_arrange(const u32x4& t, uint32_t w[4]) {
  w[0] = t.x;
  w[1] = t.y;
  w[2] = t.z;
  w[3] = t.w;
  swap32(w[0], w[2]);
  swap32(w[1], w[3]);
  if constexpr (BITS == 2) {
    swap16(w[0], w[1]);
    swap16(w[2], w[3]);
  }
}

// Q2 down with 4 waves: asking for 4 waves per SIMD keeps the kernel in 128
// registers (it took 132, three waves); the others are left to the compiler
template <int BITS, typename ST, int IN, bool GU, bool SV, int NW>
__global__ __launch_bounds__(NW * 64, (BITS == 2 && !GU && NW == 4) ? 4 : 1) void k_gemm(GemvArgs A) {
  extern __shared__ uint32_t lds[];
  constexpr int WPG = QT<BITS>::WPG, HALVES = QT<BITS>::PPW / 4;
  constexpr int GB = GM_GB;
  static_assert(GB % 4 == 0, "batches start at multiples of four groups");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const MatArgs& M0 = A.m0;
  const int rows = M0.rows, Wr = M0.words_per_row, G = M0.cols / 64, TC = A.tc;
  // the slot's pairs, matrices and row pitch (words, groups)
  int p0, p1, rpw = Wr, rpg = G;
  const uint8_t* blob;
  uint64_t c0off = M0.codes_off, s0off = M0.scales_off;
  uint64_t c1off = A.m1.codes_off, s1off = A.m1.scales_off;
  if (A.shared) {
    p0 = 0;
    p1 = A.T;
    blob = A.blobs;
  } else {
    // the shared expert's parts take the first rows of the grid: their
    // workgroups (every token of the batch each) are then dispatched ahead
    // of the routed slots' instead of starting last, when a grid larger than
    // the GPU holds at once leaves them to a second round
    const int y = blockIdx.y, nr = A.meta[0], nsh = A.nsh;
    const int slot = y < nsh ? nr + y : y - nsh;
    if (y >= nsh && slot >= nr) return;  // workgroup-uniform
    p0 = A.offs[slot];
    p1 = A.offs[slot + 1];
    if (slot < nr) {
      blob = expert_blob(A.blobs, A.stride, A.table, A.active[slot]);
    } else {
      // part v of the shared expert: a block of its gate/up rows, or a block
      // of its down columns (rows nsh times as long)
      const uint64_t v = (uint64_t)(slot - nr);
      blob = A.sh_blob;
      if constexpr (GU) {
        c0off = A.sh_m0.codes_off + v * rows * Wr * 4;
        s0off = A.sh_m0.scales_off + v * rows * G * sizeof(ST);
        c1off = A.sh_m1.codes_off + v * rows * Wr * 4;
        s1off = A.sh_m1.scales_off + v * rows * G * sizeof(ST);
      } else {
        c0off = A.sh_m0.codes_off + v * Wr * 4;
        s0off = A.sh_m0.scales_off + v * G * sizeof(ST);
        c1off = c0off;
        s1off = s0off;
        rpw = A.nsh * Wr;
        rpg = A.nsh * G;
      }
    }
  }
  if (p0 >= p1) return;  // workgroup-uniform
  const int ks = A.ksplit;           // waves per 16-row tile: 1 or 4 (4 only with NW = 4)
  const int tpw = A.tiles_per_wave;  // tiles a wave takes in turn (1 with the k-split)
  const int tw = wave / ks, kpart = wave - tw * ks;
  const int r = lane & 15, b = lane >> 4;
  const int gper = ((G + ks - 1) / ks + 3) & ~3;  // a multiple of four groups
  const int gb0 = min(G, kpart * gper), gb1 = min(G, gb0 + gper);
  const int nbt = (gb1 - gb0 + GB - 1) / GB;  // batches per tile (0: an empty k-part)
  const int nb = nbt * tpw;                   // batches of this wave per chunk
  const uint32_t* cm0 = (const uint32_t*)(blob + c0off);
  const ST* sm0 = (const ST*)(blob + s0off);
  const uint32_t* cm1 = (const uint32_t*)(blob + c1off);
  const ST* sm1 = (const ST*)(blob + s1off);
  constexpr bool SPLIT = IN == GV_F32_SPLIT;
  const GmLds L = gm_lds_layout(M0.cols, TC, SPLIT, NW);
  const uint32_t* X = lds + L.x;
  const uint32_t* Xlo = lds + L.xlo;
  const float* Kl = (const float*)(lds + L.k);
  const float* osc = (const float*)(lds + L.osc);
  float* part = (float*)(lds + L.part);
  // the fp16 pair 1024, 1024 in a VGPR (an operand of the decode)
  uint32_t magic;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  // first word of a group this lane feeds to the MFMAs (after the swaps)
  const int wmap = BITS == 4 ? (b & 1) * 4 + (b >> 1) * 2 : b;
  constexpr int UG = BITS == 4 ? 2 : 4;  // groups per load unit
  constexpr int NU = GB / UG;             // load units per batch
  static_assert(GB == 8, "one scale load per lane covers a batch of eight groups");

  // Batch k of the wave: tile item k / nbt (consecutive waves of a workgroup
  // take consecutive tiles), groups gb0 + (k % nbt) * GB onwards. Batches
  // past the wave's last are read from its last tile, past its groups
  // (clamped: cache hits, never used).
  struct Pos {
    int t, g0;
  };
  auto pos = [&](int k) -> Pos {
    const int t = min(k / max(nbt, 1), tpw - 1);
    return Pos{t, gb0 + (k - t * nbt) * GB};
  };
  auto row_of = [&](int t) { return ((blockIdx.x * tpw + t) * (NW / ks) + tw) * 16 + r; };

  // Scales (SV: every row holds whole quads of groups): one 16-byte load per
  // lane per batch, quarter b reading quad b & 1 of the batch, of the up
  // matrix when b >= 2 (gate/up) and a copy of quarters 0, 1 otherwise;
  // lane swaps broadcast each quad to all quarters at use. Without SV every
  // lane loads each scale it needs.
  struct Batch {
    u32x4 wa[NU], wb[NU];
    u32x4 sq;                                // SV
    float sa[SV ? 1 : GB], sb[SV ? 1 : GB];  // not SV
  };
  auto load = [&](Batch& B, int k) {
    const Pos P = pos(k);
    const int rc = min(row_of(P.t), rows - 1);
    const uint32_t* c0 = cm0 + (size_t)rc * rpw;
    const uint32_t* c1 = cm1 + (size_t)rc * rpw;
    const ST* s0 = sm0 + (size_t)rc * rpg;
    const ST* s1 = sm1 + (size_t)rc * rpg;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      B.wa[u] = gm_unit_load<BITS>(c0, P.g0 + u * UG, G, b);
      if constexpr (GU) B.wb[u] = gm_unit_load<BITS>(c1, P.g0 + u * UG, G, b);
    }
    if constexpr (SV) {
      B.sq = gm_scale_quad<ST>((GU && (b >> 1)) ? s1 : s0, min(P.g0 + 4 * (b & 1), G - 4));
    } else {
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        B.sa[j] = load_scale<ST, false>(s0 + min(P.g0 + j, G - 1));
        if constexpr (GU) B.sb[j] = load_scale<ST, false>(s1 + min(P.g0 + j, G - 1));
      }
    }
  };
  // the scales of a batch for this lane's row: sa (gate or the only
  // matrix), sb (up)
  auto scales = [&](const Batch& B, float* sa, float* sb) {
    if constexpr (SV) {
      uint32_t q[4] = {B.sq.x, B.sq.y, B.sq.z, B.sq.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = q[i], hi = q[i];
        swap16(lo, hi);  // lo: quarters' quad 0 (gate | up), hi: quad 1
        if constexpr (GU) {
          uint32_t lo2 = lo, hi2 = hi;
          swap32(lo, lo2);  // lo: gate quad 0, lo2: up quad 0
          swap32(hi, hi2);
          sa[i] = __builtin_bit_cast(float, lo);
          sb[i] = __builtin_bit_cast(float, lo2);
          sa[4 + i] = __builtin_bit_cast(float, hi);
          sb[4 + i] = __builtin_bit_cast(float, hi2);
        } else {
          sa[i] = __builtin_bit_cast(float, lo);
          sa[4 + i] = __builtin_bit_cast(float, hi);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        sa[j] = B.sa[j];
        if constexpr (GU) sb[j] = B.sb[j];
      }
    }
  };
  // the word that group j of an arranged batch feeds to MFMA h
  auto word = [&](const uint32_t (*w)[4], int j, int h) -> uint32_t {
    if constexpr (BITS == 4) return w[j / 2][(j % 2) * 2 + h];
    return w[j / 4][j % 4];
  };

  Batch bA, bB;
  for (int pc = p0; pc < p1; pc += TC) {
    const int nt = min(TC, p1 - pc);
    if (pc > p0) __syncthreads();  // the previous chunk's readers are done
    // the tokens are staged before the first weight batch is requested:
    // loads retire in order, so staging loads issued behind a weight batch
    // would wait for it
    gm_stage<BITS, IN, GU, NW>(A, M0, lds, L, pc, nt);
    load(bA, 0);
    // A row r of the MFMAs is token r; rows past the chunk read whatever the
    // LDS holds (row TC - 1 past the staged block) and their D rows are
    // never used
    const int rr = min(r, TC - 1);
    // LDS word offset of this lane's A operand for MFMA h of group g: word
    // cw of a group sits at ((cw * HALVES + hv) * TC + rr) * 4, which is
    // g * gstride (uniform) plus a per-lane part fixed for the chunk
    const int gstride = WPG * HALVES * TC * 4;
    int xoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int hv = BITS == 4 ? 0 : h;
      const int cwl = BITS == 4 ? wmap + h : wmap;
      xoff[h] = ((cwl * HALVES + hv) * TC + rr) * 4;
    }
    f32x4m acc_a = {0.f, 0.f, 0.f, 0.f}, acc_b = {0.f, 0.f, 0.f, 0.f};
    // batch k; groups at or past gb1 (the tail of the wave's range) count
    // with scale zero and read the last group's LDS
    auto compute = [&](const Batch& B, int k) {
      const int g0 = pos(k).g0;
      if (g0 == gb0) {  // a new tile
        acc_a = f32x4m{0.f, 0.f, 0.f, 0.f};
        acc_b = f32x4m{0.f, 0.f, 0.f, 0.f};
      }
      uint32_t wa[NU][4], wb[NU][4];
      float bsa[GB], bsb[GB];
      scales(B, bsa, bsb);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        gm_unit_arrange<BITS>(B.wa[u], wa[u]);
        if constexpr (GU) gm_unit_arrange<BITS>(B.wb[u], wb[u]);
      }
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        const bool own = g0 + j < gb1;  // wave-uniform
        const int g = min(g0 + j, G - 1);
        const float sa = own ? bsa[j] : 0.f;
        // both chains start from -K, so they leave D - K (the offsets of the
        // fp16 pairs and the code midpoint removed)
        const f32x4m nk = *(const f32x4m*)(Kl + g * 16 + 4 * b);
        f32x4m da = nk, db = nk;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int hv = BITS == 4 ? 0 : h;
          const int xi = g * gstride + xoff[h];
          const h8 av = __builtin_bit_cast(h8, *(const u32x4*)(X + xi));
          const h8 oa = gm_operand<BITS>(word(wa, j, BITS == 4 ? h : 0), hv, magic);
          da = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, oa, da, 0, 0, 0);
          h8 ob;
          if constexpr (GU) {
            ob = gm_operand<BITS>(word(wb, j, BITS == 4 ? h : 0), hv, magic);
            db = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, ob, db, 0, 0, 0);
          }
          if constexpr (SPLIT) {
            const h8 al = __builtin_bit_cast(h8, *(const u32x4*)(Xlo + xi));
            da = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, oa, da, 0, 0, 0);
            if constexpr (GU) db = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, ob, db, 0, 0, 0);
          }
        }
        acc_a.x = fmaf(sa, da.x, acc_a.x);
        acc_a.y = fmaf(sa, da.y, acc_a.y);
        acc_a.z = fmaf(sa, da.z, acc_a.z);
        acc_a.w = fmaf(sa, da.w, acc_a.w);
        if constexpr (GU) {
          const float sb = own ? bsb[j] : 0.f;
          acc_b.x = fmaf(sb, db.x, acc_b.x);
          acc_b.y = fmaf(sb, db.y, acc_b.y);
          acc_b.z = fmaf(sb, db.z, acc_b.z);
          acc_b.w = fmaf(sb, db.w, acc_b.w);
        }
      }
    };
    // the outputs of tile item t: tokens 4b .. 4b + 3 of row r
    auto store = [&](int t, const float* va, const float* vb) {
      const int row = row_of(t);
      if (kpart == 0 && row < rows) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = 4 * b + i;
          if (tk < nt) {
            const float o = osc[tk];
            float val;
            if constexpr (GU) {
              const float gg = va[i] * o, uu = vb[i] * o;
              val = gg / (1.0f + expf(-gg)) * uu;
            } else {
              val = va[i] * o;
            }
            A.out[(size_t)(pc + tk) * rows + row] = val;
          }
        }
      }
    };
    auto finish_tile = [&](int k) {  // after batch k, without the k-split
      if (ks == 1 && k - pos(k).t * nbt == nbt - 1) {
        const float va[4] = {acc_a.x, acc_a.y, acc_a.z, acc_a.w};
        const float vb[4] = {acc_b.x, acc_b.y, acc_b.z, acc_b.w};
        store(pos(k).t, va, vb);
      }
    };
    // Loads are unconditional (past the wave's work they re-read its last
    // groups, cache hits) so that the number in flight is the same on every
    // path and each wait covers exactly the batch about to be used.
    // Scheduling barriers keep each batch's loads ahead of the computation
    // on the other batch (the scheduler would otherwise sink them past it).
    for (int k = 0; k < nb; k += 2) {
      load(bB, k + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(bA, k);
      finish_tile(k);
      __builtin_amdgcn_sched_barrier(0);
      load(bA, k + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < nb) {
        compute(bB, k + 1);
        finish_tile(k + 1);
      }
    }
    if (ks > 1) {
      // partial sums of the k-split waves meet in LDS (one tile per wave)
      float va[4] = {acc_a.x, acc_a.y, acc_a.z, acc_a.w};
      float vb[4] = {acc_b.x, acc_b.y, acc_b.z, acc_b.w};
      if (kpart > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          part[((tw * 4 + kpart) * 64 + lane) * 8 + i] = va[i];
          part[((tw * 4 + kpart) * 64 + lane) * 8 + 4 + i] = vb[i];
        }
      }
      __syncthreads();
      if (kpart == 0) {
        for (int kp = 1; kp < ks; ++kp)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            va[i] += part[((tw * 4 + kp) * 64 + lane) * 8 + i];
            vb[i] += part[((tw * 4 + kp) * 64 + lane) * 8 + 4 + i];
          }
      }
      store(0, va, vb);
    }
  }
}

// ------------------------------------------------- K-sliced (prefill) stage
//
// For slots with many tokens (prefill-sized batches) each weight fetch
// should serve more tokens than one MFMA's 16, but a 4096-wide token vector
// takes 8 KB of LDS as fp16, so a chunk of 64 tokens does not fit whole.
// This stage takes the chunk one K slice (four scale groups, 256 weights) at
// a time into one of two LDS buffers and feeds every decoded weight operand
// to NTT = 4 MFMA token tiles, so a slot's weights are read once per chunk.
//   - The token vectors were converted beforehand (k_gmk_prep) into the
//     fp16 pairs, group offsets K and output factors of k_gemm's staging,
//     stored per vector in the order of the MFMA operand, so a slice is
//     copied global -> LDS with direct-to-LDS loads (global_load_lds_dwordx4:
//     lane i writes 16 bytes at LDS base + 16 i), no registers and no
//     conversion in this kernel. Such a load costs the CU about 48 cycles of
//     issue whatever its size, so each one moves a whole kilobyte (two
//     tokens' 512-byte slices). In LDS a pair's row is 66 quads long and the
//     odd token's quads are rotated by one, so the 16 tokens an MFMA operand
//     read touches sit on 16 different bank quads.
//   - Each wave owns two 16-row tiles: for gate/up the gate and the up rows
//     of the same 16 rows (SwiGLU is then applied in registers), for down
//     two adjacent tiles. Each token operand read from LDS feeds both tiles.
//   - Per slice: the next slice's weights (registers) and tokens (the other
//     LDS buffer) are requested before the current slice is multiplied; one
//     wait for the wave's loads and one barrier end the slice.
//   - A slot's tokens are cut into chunks of nearly equal size; token rows
//     past the chunk's end repeat its last token, and their sums are
//     dropped.
//   - Within a group the LDS operands of tile t + 1 are read while tile t is
//     multiplied, and tile t - 1's sums are scaled after tile t's MFMAs are
//     issued, so no vector instruction waits on an MFMA it just issued.

template <int BITS, typename ST, bool GU, bool SV, int NTT>
__global__ __launch_bounds__(GMK_NW * 64) void k_gemm_ks(GemvArgs A) {
  extern __shared__ uint32_t lds[];
  constexpr int WPG = QT<BITS>::WPG, HALVES = QT<BITS>::PPW / 4;
  constexpr int TC = 16 * NTT, KSG = GMK_KSG, QPS = GMK_QPS, XPS = GMK_XPS;
  static_assert(KSG * WPG * HALVES == QPS, "a slice is KSG groups of 8 pair quads");
  constexpr int XB = TC / 2 * XPS * 4, KB = KSG * TC;
  constexpr int TPW = GMK_TPW;
  constexpr int UG = BITS == 4 ? 2 : 4;  // scale groups per 16-byte unit load
  constexpr int NU = KSG / UG;
  constexpr int PPV = TC / 2 / GMK_NW;   // token pairs each wave copies per slice
  static_assert(QPS == 32, "one load moves two tokens' slices");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup L of the launch runs on XCD L % 8 (round-robin dispatch); give
  // each XCD whole slots, so the row blocks that share a slot's token slices
  // share that XCD's L2 (the slots past the last multiple of 8 keep the
  // plain order)
  int bx = blockIdx.x, slot = blockIdx.y;
  {
    const int nbx = gridDim.x, L = bx + slot * nbx;
    if (L < (int)(gridDim.y & ~7u) * nbx) {
      const int q = L >> 3;
      slot = q / nbx * 8 + (L & 7);
      bx = q % nbx;
    }
  }
  if (slot >= A.meta[0]) return;  // workgroup-uniform
  const int e = A.active[slot], p0 = A.offs[slot], p1 = A.offs[slot + 1];
  if (p0 >= p1) return;
  const int rows = A.m0.rows, Wr = A.m0.words_per_row, cols = A.m0.cols, G = cols / 64;
  const int NSL = (G + KSG - 1) / KSG;
  const int r = lane & 15, b = lane >> 4;
  const uint8_t* blob = expert_blob(A.blobs, A.stride, A.table, e);
  // the wave's tiles: gate/up: the gate (u = 0) and up (u = 1) rows of one
  // 16-row tile; down: two tiles
  int row[TPW];
  const uint32_t* cw0[TPW];
  const ST* sw0[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const MatArgs& M = (GU && (u & 1)) ? A.m1 : A.m0;
    row[u] = GU ? ((bx * GMK_NW + wave) * (TPW / 2) + u / 2) * 16 + r
                : ((bx * GMK_NW + wave) * TPW + u) * 16 + r;
    const int rc = min(row[u], rows - 1);
    cw0[u] = (const uint32_t*)(blob + M.codes_off) + (size_t)rc * Wr;
    sw0[u] = (const ST*)(blob + M.scales_off) + (size_t)rc * G;
  }
  const GmkLds L = gmk_lds_layout(TC);
  uint32_t* X = lds + L.x;
  float* Kl = (float*)(lds + L.k);
  float* osc = (float*)(lds + L.osc);
  uint32_t magic;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  const int wmap = BITS == 4 ? (b & 1) * 4 + (b >> 1) * 2 : b;
  // prepared vectors: pair quads [V][cols / 8] (16 bytes each), -K [V][G],
  // output factors [V]
  const u32x4* xq = (const u32x4*)A.prep_x;
  const float* xk = A.prep_k;
  const float* xo = A.prep_o;

  struct Batch {
    u32x4 w[TPW][NU];
    u32x4 sq[TPW];
  };
  // weights of slice sl (clamped) for this wave: units, then scales
  auto load_w = [&](Batch& B, int sl) __attribute__((always_inline)) {
    const int g0 = min(sl, NSL - 1) * KSG;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int n = 0; n < NU; ++n) B.w[u][n] = gm_unit_load<BITS>(cw0[u], g0 + n * UG, G, b);
      if constexpr (SV) {
        B.sq[u] = gm_scale_quad<ST>(sw0[u], g0);  // G % 4 == 0: g0 + 4 <= G
      } else {
        uint32_t s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s4[j] = __builtin_bit_cast(uint32_t, load_scale<ST, false>(sw0[u] + min(g0 + j, G - 1)));
        B.sq[u] = u32x4{s4[0], s4[1], s4[2], s4[3]};
      }
    }
  };
  // lane l's token of the chunk as a prepared-vector index
  int vA = 0;
  // token pair pp of the chunk of slice sl (clamped) into buffer buf with
  // one direct-to-LDS load: lanes 0-31 copy the even token's 32 quads in
  // order, lanes 32-63 the odd token's rotated by one (its quad q lands at
  // 32 + (q + 1) % 32), so that with pair rows XPS quads apart the 16
  // tokens an operand read touches fall on 16 different bank quads. A slice
  // past the row's end (G not a multiple of KSG) re-reads the row's last
  // quad, never used.
  auto stage_x = [&](int sl, int buf, int pp) __attribute__((always_inline)) {
    const int sc = min(sl, NSL - 1);
    const int ve = __builtin_amdgcn_readlane(vA, 2 * pp), vo = __builtin_amdgcn_readlane(vA, 2 * pp + 1);
    const int q = lane < 32 ? lane : (lane - 33) & 31;
    const int qc = min(sc * QPS + q, cols / 8 - 1);
    __builtin_amdgcn_global_load_lds(
        (const void*)(xq + (size_t)(lane < 32 ? ve : vo) * (cols / 8) + qc),
        (__attribute__((address_space(3))) void*)(X + buf * XB + pp * XPS * 4), 16, 0, 0);
  };
  // all of slice sl's loads of this wave: its weights, its token pairs and
  // (waves 0..KSG-1) the offsets of group wave of the slice for the chunk
  auto load_all = [&](Batch& B, int sl, int buf) __attribute__((always_inline)) {
    load_w(B, sl);
#pragma unroll
    for (int d = 0; d < PPV; ++d) stage_x(sl, buf, wave * PPV + d);
    if (wave < KSG) {
      const int g = min(min(sl, NSL - 1) * KSG + wave, G - 1);
      __builtin_amdgcn_global_load_lds((const void*)(xk + (size_t)vA * G + g),
                                       (__attribute__((address_space(3))) void*)(Kl + buf * KB +
                                                                                 wave * TC),
                                       4, 0, 0);
    }
  };

  f32x4m acc[TPW][NTT];
  // slice sl from buffer buf and batch B
  auto compute = [&](const Batch& B, int sl, int buf) __attribute__((always_inline)) {
    const int g0 = sl * KSG;
    const int glast = min(G - 1 - g0, KSG - 1);
    const uint32_t* Xb = X + buf * XB;
    const float* Kb = Kl + buf * KB;
    uint32_t wa[TPW][4];  // the current load unit's words, arranged
#pragma unroll
    for (int j = 0; j < KSG; ++j) {
      const bool own = g0 + j < G;  // wave-uniform
      const int gl = min(j, glast);
      if (j % UG == 0) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) gm_unit_arrange<BITS>(B.w[u][j / UG], wa[u]);
      }
      h8 op[2][TPW];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < TPW; ++u)
          op[h][u] = BITS == 4 ? gm_operand<BITS>(wa[u][(j % 2) * 2 + h], 0, magic)
                               : gm_operand<BITS>(wa[u][j % 4], h, magic);
      float sj[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const uint32_t sv = j == 0 ? B.sq[u].x : j == 1 ? B.sq[u].y : j == 2 ? B.sq[u].z : B.sq[u].w;
        sj[u] = own ? __builtin_bit_cast(float, sv) : 0.f;
      }
      // LDS operands of tile t: the two token quads and the negated offsets
      auto rd = [&](int t, h8* av, f32x4m& nk) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int hv = BITS == 4 ? 0 : h;
          const int qd = BITS == 4 ? (gl * WPG + wmap + h) : (gl * WPG + wmap) * HALVES + hv;
          const int pos = (r & 1) ? 32 + ((qd + 1) & 31) : qd;
          av[h] = __builtin_bit_cast(h8, *(const u32x4*)(Xb + (8 * t + (r >> 1)) * XPS * 4 + pos * 4));
        }
        nk = *(const f32x4m*)(Kb + gl * TC + 16 * t + 4 * b);
      };
      h8 av[2][2];
      f32x4m nk[2];
      f32x4m d[2][TPW];
      rd(0, av[0], nk[0]);
#pragma unroll
      for (int t = 0; t <= NTT; ++t) {
        if (t + 1 < NTT) rd(t + 1, av[(t + 1) & 1], nk[(t + 1) & 1]);
        if (t < NTT) {
          // the MFMAs start from -K, so they leave D - K (the offsets of the
          // fp16 pairs and the code midpoint removed) in one chain
#pragma unroll
          for (int u = 0; u < TPW; ++u)
            d[t & 1][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t & 1][0], op[0][u], nk[t & 1], 0, 0, 0);
#pragma unroll
          for (int u = 0; u < TPW; ++u)
            d[t & 1][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t & 1][1], op[1][u], d[t & 1][u], 0, 0, 0);
        }
        if (t >= 1) {
#pragma unroll
          for (int u = 0; u < TPW; ++u) {
            const f32x4m dv = d[(t - 1) & 1][u];
            f32x4m& a = acc[u][t - 1];
            a.x = fmaf(sj[u], dv.x, a.x);
            a.y = fmaf(sj[u], dv.y, a.y);
            a.z = fmaf(sj[u], dv.z, a.z);
            a.w = fmaf(sj[u], dv.w, a.w);
          }
        }
        // keep the pipeline as written (the scheduler would otherwise hoist
        // every tile's LDS reads)
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Batch bA, bB;
  const int n = p1 - p0;
  const int nch = (n + TC - 1) / TC, base = n / nch, extra = n % nch;
  int pc = p0;
  for (int c = 0; c < nch; ++c) {
    const int nt = base + (c < extra ? 1 : 0);
    const int na = (nt + 15) / 16;
    if (c > 0) __syncthreads();  // the previous chunk's LDS readers are done
    {
      const int pa = pc + min(lane, nt - 1);
      vA = GU ? A.pair_token[pa] : pa;
    }
    load_all(bA, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((const void*)(xo + vA),
                                       (__attribute__((address_space(3))) void*)osc, 4, 0, 0);
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int t = 0; t < NTT; ++t) acc[u][t] = f32x4m{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // slices in pairs (constant buffer indices, so the compiler can tell the
    // direct-to-LDS writes of one buffer from the reads of the other); every
    // load of the next slice is issued before the current one is multiplied
    // and complete before the barrier that ends it
    for (int sl = 0; sl < NSL; sl += 2) {
      if (sl + 1 < NSL) load_all(bB, sl + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(bA, sl, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (sl + 1 >= NSL) break;
      if (sl + 2 < NSL) load_all(bA, sl + 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(bB, sl + 1, 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    // outputs: lane (r, b) holds tokens 16t + 4b .. + 3 of its rows
    if constexpr (GU) {
#pragma unroll
      for (int v = 0; v < TPW / 2; ++v) {
        if (row[2 * v] >= rows) continue;
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
          if (t >= na) break;
          const float ga[4] = {acc[2 * v][t].x, acc[2 * v][t].y, acc[2 * v][t].z, acc[2 * v][t].w};
          const float ua[4] = {acc[2 * v + 1][t].x, acc[2 * v + 1][t].y, acc[2 * v + 1][t].z,
                               acc[2 * v + 1][t].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tkn = 16 * t + 4 * b + i;
            if (tkn < nt) {
              const float o = osc[tkn];
              const float gg = ga[i] * o, uu = ua[i] * o;
              A.out[(size_t)(pc + tkn) * rows + row[2 * v]] = gg / (1.0f + expf(-gg)) * uu;
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        if (row[u] >= rows) continue;
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
          if (t >= na) break;
          const float va[4] = {acc[u][t].x, acc[u][t].y, acc[u][t].z, acc[u][t].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tkn = 16 * t + 4 * b + i;
            if (tkn < nt) A.out[(size_t)(pc + tkn) * rows + row[u]] = va[i] * osc[tkn];
          }
        }
      }
    }
    pc += nt;
  }
}

// Launcher, instantiated per (BITS, scale type) in smoe_gemm_inst.hip.
// Workgroups of more than 64 KB of LDS need the kernel's limit raised.
template <typename K>
static hipError_t gm_allow_lds(K kernel, unsigned lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

template <int BITS, typename ST, bool SV, int NW>
static hipError_t launch_gm_nw(const GemvArgs& A, bool gate_up, int in, dim3 grid, unsigned lds,
                               hipStream_t s) {
  const dim3 block(NW * 64);
  auto go = [&](auto kernel) {
    const hipError_t e = gm_allow_lds(kernel, lds);
    return e != hipSuccess ? e : launch_kernel_lds(kernel, grid, block, lds, s, A);
  };
  if (!gate_up) return go(k_gemm<BITS, ST, GV_F32, false, SV, NW>);
  if (in == GV_BF16) return go(k_gemm<BITS, ST, GV_BF16, true, SV, NW>);
  return go(k_gemm<BITS, ST, GV_F32_SPLIT, true, SV, NW>);
}

template <int BITS, typename ST>
hipError_t launch_gm_ks(const GemvArgs& A, bool gate_up, dim3 grid, hipStream_t s) {
  if (A.tc != GMK_TC) return hipErrorInvalidValue;
  const unsigned lds = (unsigned)gmk_lds_layout(A.tc).total * 4;
  const dim3 block(GMK_NW * 64);
  const bool sv = A.m0.cols / 64 % 4 == 0;
  auto go = [&](auto kernel) {
    const hipError_t e = gm_allow_lds(kernel, lds);
    return e != hipSuccess ? e : launch_kernel_lds(kernel, grid, block, lds, s, A);
  };
  auto pick = [&](auto ntt) {
    constexpr int N = decltype(ntt)::value;
    if (gate_up)
      return sv ? go(k_gemm_ks<BITS, ST, true, true, N>) : go(k_gemm_ks<BITS, ST, true, false, N>);
    return sv ? go(k_gemm_ks<BITS, ST, false, true, N>) : go(k_gemm_ks<BITS, ST, false, false, N>);
  };
  return pick(std::integral_constant<int, GMK_TC / 16>{});
}

template <int BITS, typename ST>
hipError_t launch_gm(const GemvArgs& A, bool gate_up, int in, int nw, dim3 grid, unsigned lds,
                     hipStream_t s) {
  // vector scale loads when every row holds a whole number of scale quads
  const bool sv = A.m0.cols / 64 % 4 == 0;
  if (nw == 8)
    return sv ? launch_gm_nw<BITS, ST, true, 8>(A, gate_up, in, grid, lds, s)
              : launch_gm_nw<BITS, ST, false, 8>(A, gate_up, in, grid, lds, s);
  return sv ? launch_gm_nw<BITS, ST, true, 4>(A, gate_up, in, grid, lds, s)
            : launch_gm_nw<BITS, ST, false, 4>(A, gate_up, in, grid, lds, s);
}

}  // namespace smoe
