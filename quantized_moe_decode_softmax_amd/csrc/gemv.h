// Wave-level building blocks of the dequantising matrix-vector products
// (gfx950, wave64).
//
// Work unit: a chunk of 32 consecutive codes of one row (half a quantisation
// group of 64, so one scale/bias pair applies). A row of K codes has K/32
// chunks; `lpr` lanes (a power of two <= 64) share a row and lane `li` takes
// chunks li, li + lpr, ... (at most CPL of them). The lanes' partial sums are
// combined by a fixed butterfly, so every result is bitwise reproducible and
// independent of how many rows or tokens a launch handles.
//
// Arithmetic per chunk: with x the 32 input values and q the codes,
//   sum_j (q_j s + b) x_j = s * D + (b - 128 s) * X,
//   D = sum_j (128 + q_j) x_j,  X = sum_j x_j.
// For 2/3/4/6-bit codes, (128 + q) is exactly the bf16 whose mantissa holds q,
// so two codes become one bf16 pair with a single mask-and-or and D is a chain
// of v_dot2c_f32_bf16 (fp32 accumulation) against bf16 pairs of x. 8-bit
// codes are split into two nibble planes, q = 16 hi + lo, each decoded the
// same way: sum q x = D_lo + 16 D_hi - 2176 X. The flash-moe news page's reordered
// dequantisation ("FMA-optimised dequant kernel") folds scale and bias into
// the input; here they are applied once per half-group instead.
#pragma once

#include <climits>

#include "device_common.h"
#include "internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1, 1)
constexpr int kDense = 16;                // "bits" of a dense bf16 matrix

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Fused decode + dot of one bf16 code pair: acc += dot2(((a >> SH) & m) | mag,
// x), i.e. v_lshrrev + v_and_or_b32 + v_dot2c_f32_bf16 in one block, so the
// decoded pair lives in one temporary. m comes from an SGPR and mag from a
// VGPR: this architecture reads one scalar operand per instruction and VOP3
// takes no literal (left to itself the compiler emits an AND and an OR with
// literals, and schedules decodes far ahead of their use).
template <int SH>
__device__ __forceinline__ void dq_dot(float& acc, uint32_t a, uint32_t m, uint32_t mag, uint32_t x) {
  uint32_t t;
  if constexpr (SH == 0) {
    asm("v_and_or_b32 %1, %2, %3, %4\n\tv_dot2c_f32_bf16 %0, %1, %5"
        : "+v"(acc), "=&v"(t)
        : "v"(a), "s"(m), "v"(mag), "v"(x));
  } else {
    asm("v_lshrrev_b32 %1, %6, %2\n\tv_and_or_b32 %1, %1, %3, %4\n\tv_dot2c_f32_bf16 %0, %1, %5"
        : "+v"(acc), "=&v"(t)
        : "v"(a), "s"(m), "v"(mag), "v"(x), "i"(SH));
  }
}
// Same pair against two inputs (acc0 += p . x0, acc1 += p . x1).
template <int SH>
__device__ __forceinline__ void dq_dot2(float& acc0, float& acc1, uint32_t a, uint32_t m, uint32_t mag, uint32_t x0,
                                        uint32_t x1) {
  uint32_t t;
  if constexpr (SH == 0) {
    asm("v_and_or_b32 %2, %3, %4, %5\n\tv_dot2c_f32_bf16 %0, %2, %6\n\tv_dot2c_f32_bf16 %1, %2, %7"
        : "+v"(acc0), "+v"(acc1), "=&v"(t)
        : "v"(a), "s"(m), "v"(mag), "v"(x0), "v"(x1));
  } else {
    asm("v_lshrrev_b32 %2, %8, %3\n\tv_and_or_b32 %2, %2, %4, %5\n\tv_dot2c_f32_bf16 %0, %2, %6\n\t"
        "v_dot2c_f32_bf16 %1, %2, %7"
        : "+v"(acc0), "+v"(acc1), "=&v"(t)
        : "v"(a), "s"(m), "v"(mag), "v"(x0), "v"(x1), "i"(SH));
  }
}
// acc += dot2(p, x) as v_dot2c_f32_bf16 (the opcode of the blocks above, so
// the accumulator chain only ever feeds the same DOT opcode as its SrcC).
__device__ __forceinline__ void dot2c(float& acc, uint32_t p, uint32_t x) {
  asm("v_dot2c_f32_bf16 %0, %1, %2" : "+v"(acc) : "v"(p), "v"(x));
}
// A DOT result read by another VALU opcode (or as a DOT's A/B source) needs 3
// wait states, which the compiler cannot see through the asm blocks that
// wrote it: every accumulator chain ends in this fence before ordinary code
// reads it.
__device__ __forceinline__ void dot_fence(float& a) { asm volatile("s_nop 2" : "+v"(a)); }
__device__ __forceinline__ void dot_fence(float& a, float& b) { asm volatile("s_nop 2" : "+v"(a), "+v"(b)); }

// 6-bit split pair: low nibbles at bit SA of a, high 2 bits at bit SC of c
// (moved to bits 4-5): ((a >> SA) & 0x000F000F | mag) | ((c >> (SC - 4)) & 0x00300030).
template <int SA, int SCM4>
__device__ __forceinline__ uint32_t split6(uint32_t a, uint32_t c, uint32_t m4, uint32_t m2, uint32_t mag) {
  uint32_t t, u;
  asm("v_lshrrev_b32 %0, %5, %2\n\tv_and_or_b32 %0, %0, %3, %4\n\tv_lshrrev_b32 %1, %7, %6\n\t"
      "v_and_or_b32 %0, %1, %8, %0"
      : "=&v"(t), "=&v"(u)
      : "v"(a), "s"(m4), "v"(mag), "i"(SA), "v"(c), "i"(SCM4), "s"(m2));
  return t;
}

__host__ __device__ __forceinline__ int pow2ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
// lanes sharing one row of K codes
__host__ __device__ __forceinline__ int lanes_per_row(int k) {
  const int n = pow2ceil(k / 32);
  return n < 64 ? n : 64;
}
// chunks per lane
__host__ __device__ __forceinline__ int chunks_per_lane(int k) {
  const int lpr = lanes_per_row(k);
  return (k / 32 + lpr - 1) / lpr;
}

__device__ __forceinline__ void load64B(const void* p, uint32_t (&w)[16]) {
  // global memory (address space 1): a global_load, not a flat one
  const __attribute__((address_space(1))) u32x4* q = (const __attribute__((address_space(1))) u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = q[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// bf16 pair (element a, element b) of 32 natural-order bf16 values held as 16 words
template <int A, int B>
__device__ __forceinline__ uint32_t pair_of(const uint32_t (&n)[16]) {
  const uint32_t wa = n[A >> 1], wb = n[B >> 1];
  const uint32_t lo = (A & 1) ? (wa >> 16) : (wa & 0xFFFFu);
  const uint32_t hi = (B & 1) ? (wb & 0xFFFF0000u) : (wb << 16);
  return lo | hi;
}

// Pair order expected by the unpackers: bits 4 pair codes (8d+i, 8d+i+4),
// bits 6 pair codes (16u+j, 16u+j+8), bits 2 pair codes (16d+i, 16d+i+8),
// bits 8 pair codes (4k+i, 4k+i+2), a dense bf16 matrix uses natural order
// (3 bits: see tri_arrange).
template <int BITS>
__device__ __forceinline__ void arrange_pairs(const uint32_t (&n)[16], uint32_t (&o)[16]) {
  if constexpr (BITS == 2) {
#define MOE_P2(d, i) o[8 * d + i] = pair_of<16 * d + i, 16 * d + i + 8>(n);
    MOE_P2(0, 0) MOE_P2(0, 1) MOE_P2(0, 2) MOE_P2(0, 3) MOE_P2(0, 4) MOE_P2(0, 5) MOE_P2(0, 6) MOE_P2(0, 7)
    MOE_P2(1, 0) MOE_P2(1, 1) MOE_P2(1, 2) MOE_P2(1, 3) MOE_P2(1, 4) MOE_P2(1, 5) MOE_P2(1, 6) MOE_P2(1, 7)
#undef MOE_P2
  } else if constexpr (BITS == 6) {
#define MOE_P6(u, j) o[8 * u + j] = pair_of<16 * u + j, 16 * u + j + 8>(n);
    MOE_P6(0, 0) MOE_P6(0, 1) MOE_P6(0, 2) MOE_P6(0, 3) MOE_P6(0, 4) MOE_P6(0, 5) MOE_P6(0, 6) MOE_P6(0, 7)
    MOE_P6(1, 0) MOE_P6(1, 1) MOE_P6(1, 2) MOE_P6(1, 3) MOE_P6(1, 4) MOE_P6(1, 5) MOE_P6(1, 6) MOE_P6(1, 7)
#undef MOE_P6
  } else if constexpr (BITS == 3 || BITS == 4) {
#define MOE_P4(d, i) o[4 * d + i] = pair_of<8 * d + i, 8 * d + i + 4>(n);
    MOE_P4(0, 0) MOE_P4(0, 1) MOE_P4(0, 2) MOE_P4(0, 3) MOE_P4(1, 0) MOE_P4(1, 1) MOE_P4(1, 2) MOE_P4(1, 3)
    MOE_P4(2, 0) MOE_P4(2, 1) MOE_P4(2, 2) MOE_P4(2, 3) MOE_P4(3, 0) MOE_P4(3, 1) MOE_P4(3, 2) MOE_P4(3, 3)
#undef MOE_P4
  } else if constexpr (BITS == 8) {
#define MOE_P8(k) o[2 * k] = pair_of<4 * k, 4 * k + 2>(n); o[2 * k + 1] = pair_of<4 * k + 1, 4 * k + 3>(n);
    MOE_P8(0) MOE_P8(1) MOE_P8(2) MOE_P8(3) MOE_P8(4) MOE_P8(5) MOE_P8(6) MOE_P8(7)
#undef MOE_P8
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = n[i];
  }
}

// Sum of the N bf16 pairs of w (a chunk in natural or arranged order).
template <int N>
__device__ __forceinline__ float sum_words(const uint32_t* w) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) s = dot2(w[i], kOnes, s);
  return s;
}

// Element indices (a, b) of arranged pair word i, for the orders above
// (bits 3 excepted: see tri_arrange).
template <int BITS>
__host__ __device__ constexpr int pair_a(int i) {
  return BITS == 2 ? 16 * (i / 8) + i % 8
       : BITS == 4 ? 8 * (i / 4) + i % 4
       : BITS == 6 ? 16 * (i / 8) + i % 8
       : BITS == 8 ? 4 * (i / 2) + i % 2
       : 2 * i;
}
template <int BITS>
__host__ __device__ constexpr int pair_b(int i) {
  return BITS == 2 ? pair_a<BITS>(i) + 8
       : BITS == 4 ? pair_a<BITS>(i) + 4
       : BITS == 6 ? pair_a<BITS>(i) + 8
       : BITS == 8 ? pair_a<BITS>(i) + 2
       : 2 * i + 1;
}

// 3-bit codes are decoded in pairs (slot s, slot s+5) of each of the 5 words a
// chunk touches (25 pairs, 50 code positions); chunk c starts at position
// R = 32c mod 10 of that window, so position p holds chunk code p - R, and
// the x pair of a position outside the chunk is zero.
template <int R, int W, int S>
__device__ __forceinline__ uint32_t tri_x_pair(const uint32_t (&n)[16]) {
  constexpr int a = 10 * W + S - R, b = 10 * W + S + 5 - R;
  uint32_t lo = 0u, hi = 0u;
  if constexpr (a >= 0 && a < 32) lo = (a & 1) ? (n[a >> 1] >> 16) : (n[a >> 1] & 0xFFFFu);
  if constexpr (b >= 0 && b < 32) hi = (b & 1) ? (n[b >> 1] & 0xFFFF0000u) : (n[b >> 1] << 16);
  return lo | hi;
}
template <int R>
__device__ __forceinline__ void tri_arrange(const uint32_t (&n)[16], uint32_t* o) {
#define MOE_TX(w) o[5 * w + 0] = tri_x_pair<R, w, 0>(n); o[5 * w + 1] = tri_x_pair<R, w, 1>(n); \
  o[5 * w + 2] = tri_x_pair<R, w, 2>(n); o[5 * w + 3] = tri_x_pair<R, w, 3>(n); o[5 * w + 4] = tri_x_pair<R, w, 4>(n);
  MOE_TX(0) MOE_TX(1) MOE_TX(2) MOE_TX(3) MOE_TX(4)
#undef MOE_TX
}

template <int BITS>
struct XWords {
  static constexpr int N = BITS == 3 ? 25 : 16;
};

// Input operand of one lane: CPL chunks of arranged words, and chunk sums.
template <int BITS, int CPL>
struct XLane {
  uint32_t w[CPL][XWords<BITS>::N];
  float s[CPL];
};

// Arranged words of chunk c from its 16 natural-order words.
template <int BITS>
__device__ __forceinline__ void arrange_chunk(const uint32_t (&n)[16], int c, uint32_t* o) {
  if constexpr (BITS == 3) {
    switch ((2 * c) % 10) {
      case 0: tri_arrange<0>(n, o); break;
      case 2: tri_arrange<2>(n, o); break;
      case 4: tri_arrange<4>(n, o); break;
      case 6: tri_arrange<6>(n, o); break;
      default: tri_arrange<8>(n, o); break;
    }
  } else {
    arrange_pairs<BITS>(n, *reinterpret_cast<uint32_t(*)[16]>(o));
  }
}

// x from a bf16 vector [K] (natural order)
template <int BITS, int CPL>
__device__ __forceinline__ void prep_x(XLane<BITS, CPL>& x, const uint16_t* v, int K, int li, int lpr) {
  const int nch = K >> 5;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    // every lane loads (lanes past the row read its last chunk, then zero it,
    // which is needed only when the row ends inside this pass)
    const bool ok = c < nch;
    uint32_t n[16];
    load64B(v + 32 * (ok ? c : nch - 1), n);
    if (lpr * (m + 1) > nch) {
#pragma unroll
      for (int i = 0; i < 16; ++i) n[i] = ok ? n[i] : 0u;
    }
    if constexpr (BITS == 3) {
      switch ((2 * c) % 10) {
        case 0: tri_arrange<0>(n, x.w[m]); break;
        case 2: tri_arrange<2>(n, x.w[m]); break;
        case 4: tri_arrange<4>(n, x.w[m]); break;
        case 6: tri_arrange<6>(n, x.w[m]); break;
        default: tri_arrange<8>(n, x.w[m]); break;
      }
    } else {
      arrange_pairs<BITS>(n, x.w[m]);
    }
    x.s[m] = sum_words<XWords<BITS>::N>(x.w[m]);
  }
}

// Arranged hi and lo words of one chunk from 32 words w[e] = bf16 hi of element
// e | bf16 lo << 16: one byte permute per word (3 bits via natural words).
template <int BITS>
__device__ __forceinline__ void split_arrange(const uint32_t (&w)[32], int c, uint32_t* xh, uint32_t* xl) {
  if constexpr (BITS == 3) {
    uint32_t hn[16], ln[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      hn[i] = __builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x05040100u);
      ln[i] = __builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x07060302u);
    }
    arrange_chunk<3>(hn, c, xh);
    arrange_chunk<3>(ln, c, xl);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xh[i] = __builtin_amdgcn_perm(w[pair_b<BITS>(i)], w[pair_a<BITS>(i)], 0x05040100u);
      xl[i] = __builtin_amdgcn_perm(w[pair_b<BITS>(i)], w[pair_a<BITS>(i)], 0x07060302u);
    }
  }
}

// Sum of squares of the lane's x values (every element of its chunks once).
template <int BITS, int CPL>
__device__ __forceinline__ float sumsq(const XLane<BITS, CPL>& x) {
  float a = 0.f;
#pragma unroll
  for (int m = 0; m < CPL; ++m)
#pragma unroll
    for (int i = 0; i < XWords<BITS>::N; ++i) a = dot2(x.w[m][i], x.w[m][i], a);
  return a;
}

// ------------------------------------------------------------ code loading
// Load of a T at p in global memory. The address space is explicit so that the
// load is a global_load (tracked by vmcnt alone): a flat load also counts
// against lgkmcnt, so every later LDS wait would wait for the weights too.
template <class T>
__device__ __forceinline__ T gload(const uint8_t* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

// Raw packed words of chunk c (codes 32c .. 32c+31) of one row in global
// memory; up to 8 words.
template <int BITS>
__device__ __forceinline__ void load_chunk(const uint8_t* row, int c, int row_words, uint32_t (&q)[8]) {
  if constexpr (BITS == 2) {
    const u32x2 v = gload<u32x2>(row + 8 * c);
    q[0] = v.x;
    q[1] = v.y;
  } else if constexpr (BITS == 4) {
    const u32x4 v = gload<u32x4>(row + 16 * c);
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
    q[3] = v.w;
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x2 v = gload<u32x2>(row + 24 * c + 8 * i);
      q[2 * i] = v.x;
      q[2 * i + 1] = v.y;
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 v = gload<u32x4>(row + 32 * c + 16 * i);
      q[4 * i] = v.x;
      q[4 * i + 1] = v.y;
      q[4 * i + 2] = v.z;
      q[4 * i + 3] = v.w;
    }
  } else if constexpr (BITS == 3) {
    // codes 32c.. start in word w0 = floor(32c/10) at code offset (32c mod 10);
    // the chunk touches at most 5 words (clamped to the row)
    const int w0 = (32 * c) / 10;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int wi = w0 + i < row_words ? w0 + i : row_words - 1;
      q[i] = gload<uint32_t>(row + 4 * wi);
    }
  }
}

// Masks of the code fields in both bf16 halves
constexpr uint32_t kM2 = 0x00030003u, kM3 = 0x00070007u, kM4 = 0x000F000Fu, kM6 = 0x003F003Fu, kM6H = 0x00300030u;

// Sums over one chunk of (128 + q) x for the code pairs in the order
// arrange_pairs uses: d0 against x0, d1 against x1 (NX = 2).
template <int BITS, int NX, int SH>
__device__ __forceinline__ void pair_dot(float& d0, float& d1, uint32_t a, uint32_t m, uint32_t mag, uint32_t x0,
                                         uint32_t x1) {
  if constexpr (NX == 2) dq_dot2<SH>(d0, d1, a, m, mag, x0, x1);
  else dq_dot<SH>(d0, a, m, mag, x0);
}
template <int NX>
__device__ __forceinline__ void word_dot(float& d0, float& d1, uint32_t p, uint32_t x0, uint32_t x1) {
  dot2c(d0, p, x0);
  if constexpr (NX == 2) dot2c(d1, p, x1);
}

template <int BITS, int NX>
__device__ __forceinline__ void code_dots(const uint32_t (&q)[8], const uint32_t (&x0)[XWords<BITS>::N],
                                          const uint32_t (&x1)[XWords<BITS>::N], float& d0, float& d1) {
  const uint32_t mag = kMagic;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      pair_dot<4, NX, 0>(d0, d1, q[d], kM4, mag, x0[4 * d + 0], x1[4 * d + 0]);
      pair_dot<4, NX, 4>(d0, d1, q[d], kM4, mag, x0[4 * d + 1], x1[4 * d + 1]);
      pair_dot<4, NX, 8>(d0, d1, q[d], kM4, mag, x0[4 * d + 2], x1[4 * d + 2]);
      pair_dot<4, NX, 12>(d0, d1, q[d], kM4, mag, x0[4 * d + 3], x1[4 * d + 3]);
    }
  } else if constexpr (BITS == 6) {
    // unit u: dwords A, B, C; pair j holds codes (j, j + 8) of the unit
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t A = q[3 * u], B = q[3 * u + 1], C = q[3 * u + 2];
      const int o = 8 * u;
      pair_dot<6, NX, 0>(d0, d1, A, kM6, mag, x0[o + 0], x1[o + 0]);
      pair_dot<6, NX, 6>(d0, d1, A, kM6, mag, x0[o + 1], x1[o + 1]);
      word_dot<NX>(d0, d1, split6<12, 8>(A, C, kM4, kM6H, mag), x0[o + 2], x1[o + 2]);
      pair_dot<6, NX, 0>(d0, d1, B, kM6, mag, x0[o + 3], x1[o + 3]);
      pair_dot<6, NX, 6>(d0, d1, B, kM6, mag, x0[o + 4], x1[o + 4]);
      word_dot<NX>(d0, d1, split6<12, 10>(B, C, kM4, kM6H, mag), x0[o + 5], x1[o + 5]);
      pair_dot<6, NX, 0>(d0, d1, C, kM6, mag, x0[o + 6], x1[o + 6]);
      pair_dot<6, NX, 6>(d0, d1, C, kM6, mag, x0[o + 7], x1[o + 7]);
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      pair_dot<2, NX, 0>(d0, d1, q[d], kM2, mag, x0[8 * d + 0], x1[8 * d + 0]);
      pair_dot<2, NX, 2>(d0, d1, q[d], kM2, mag, x0[8 * d + 1], x1[8 * d + 1]);
      pair_dot<2, NX, 4>(d0, d1, q[d], kM2, mag, x0[8 * d + 2], x1[8 * d + 2]);
      pair_dot<2, NX, 6>(d0, d1, q[d], kM2, mag, x0[8 * d + 3], x1[8 * d + 3]);
      pair_dot<2, NX, 8>(d0, d1, q[d], kM2, mag, x0[8 * d + 4], x1[8 * d + 4]);
      pair_dot<2, NX, 10>(d0, d1, q[d], kM2, mag, x0[8 * d + 5], x1[8 * d + 5]);
      pair_dot<2, NX, 12>(d0, d1, q[d], kM2, mag, x0[8 * d + 6], x1[8 * d + 6]);
      pair_dot<2, NX, 14>(d0, d1, q[d], kM2, mag, x0[8 * d + 7], x1[8 * d + 7]);
    }
  } else if constexpr (BITS == 3) {
    // slot s at bit 3s, slot s + 5 at bit 16 + 3s of each word
#pragma unroll
    for (int w = 0; w < 5; ++w) {
      pair_dot<3, NX, 0>(d0, d1, q[w], kM3, mag, x0[5 * w + 0], x1[5 * w + 0]);
      pair_dot<3, NX, 3>(d0, d1, q[w], kM3, mag, x0[5 * w + 1], x1[5 * w + 1]);
      pair_dot<3, NX, 6>(d0, d1, q[w], kM3, mag, x0[5 * w + 2], x1[5 * w + 2]);
      pair_dot<3, NX, 9>(d0, d1, q[w], kM3, mag, x0[5 * w + 3], x1[5 * w + 3]);
      pair_dot<3, NX, 12>(d0, d1, q[w], kM3, mag, x0[5 * w + 4], x1[5 * w + 4]);
    }
  }
  if constexpr (NX == 2) dot_fence(d0, d1);
  else dot_fence(d0);
}

// 8-bit codes as two nibble planes, q = 16 hi + lo: low-plane pairs (128 + lo)
// into dl, high-plane pairs into dh, for codes (4k+i, 4k+i+2) of dword k.
template <int NX>
__device__ __forceinline__ void byte_dots(const uint32_t (&q)[8], const uint32_t (&x0)[16], const uint32_t (&x1)[16],
                                          float& dl, float& dh) {
  const uint32_t mag = kMagic;
  float el = 0.f, eh = 0.f;  // against x1
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    pair_dot<8, NX, 0>(dl, el, q[k], kM4, mag, x0[2 * k], x1[2 * k]);
    pair_dot<8, NX, 8>(dl, el, q[k], kM4, mag, x0[2 * k + 1], x1[2 * k + 1]);
    pair_dot<8, NX, 4>(dh, eh, q[k], kM4, mag, x0[2 * k], x1[2 * k]);
    pair_dot<8, NX, 12>(dh, eh, q[k], kM4, mag, x0[2 * k + 1], x1[2 * k + 1]);
  }
  dot_fence(dl, dh);
  if constexpr (NX == 2) dot_fence(el, eh);
  if constexpr (NX == 2) {
    dl += el;
    dh += eh;
  }
}

// Partial sum of one chunk: s*D + b_eff*X, for NX inputs (1 = single, 2 = hi/lo split).
template <int BITS, int NX>
__device__ __forceinline__ float chunk_partial(const uint32_t (&q)[8], uint32_t sbw,
                                               const uint32_t (&x0)[XWords<BITS>::N], float s0,
                                               const uint32_t (&x1)[XWords<BITS>::N], float s1) {
  const float s = bf16_lo_to_f32(sbw), b = bf16_hi_to_f32(sbw);
  const float sx = NX == 2 ? s0 + s1 : s0;
  if constexpr (BITS == 8) {
    // sum q x = D_lo + 16 D_hi - (128 + 16*128) X
    float dl = 0.f, dh = 0.f;
    byte_dots<NX>(q, x0, x1, dl, dh);
    return fmaf(s, fmaf(16.f, dh, dl), (b - 2176.f * s) * sx);
  } else {
    float d0 = 0.f, d1 = 0.f;
    code_dots<BITS, NX>(q, x0, x1, d0, d1);
    const float d = NX == 2 ? d0 + d1 : d0;
    return fmaf(s, d, (b - 128.f * s) * sx);
  }
}

// Dense bf16 row chunk: sum_j w_j x_j (natural pairs)
__device__ __forceinline__ float dense_chunk(const uint32_t (&w)[16], const uint32_t (&x)[16]) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) d = dot2(w[i], x[i], d);
  return d;
}

// Codes of R rows for one lane (CPL chunks each), loaded before any arithmetic.
template <int BITS, int CPL, int R>
struct RowsQ {
  uint32_t q[R][CPL][8];
  uint32_t sb[R][CPL];
};

// rc[r]: first byte of row r's codes (nullptr = unused slot, result 0);
// rs[r]: its scale/bias words. K columns, row_words = dwords per row.
template <int BITS, int CPL, int R>
__device__ __forceinline__ void load_rows(RowsQ<BITS, CPL, R>& Q, const uint8_t* const (&rc)[R],
                                          const uint32_t* const (&rs)[R], int K, int row_words, int li, int lpr) {
  const int nch = K >> 5;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = li + lpr * c;
      const bool ok = rc[r] != nullptr && ch < nch;
      if (ok) {
        load_chunk<BITS>(rc[r], ch, row_words, Q.q[r][c]);
        Q.sb[r][c] = gload<uint32_t>((const uint8_t*)(rs[r] + (ch >> 1)));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) Q.q[r][c][i] = 0u;
        Q.sb[r][c] = 0u;  // scale 0, bias 0: contributes exactly 0
      }
    }
}

// Marks the packed words and scale/bias words as redefined (no instruction is
// emitted): keeps the compiler from hoisting the unpacking of every row out of
// a loop over token rows, which would hold all decoded pairs live at once, and
// from hoisting the scale/bias arithmetic, which would wait for the weight
// loads before the loop issues its input loads.
template <int BITS, int CPL, int R>
__device__ __forceinline__ void opaque(RowsQ<BITS, CPL, R>& Q) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(Q.q[r][c][i]));
      asm volatile("" : "+v"(Q.sb[r][c]));
    }
}

template <int BITS, int CPL, int R, int NX>
__device__ __forceinline__ void dot_rows(RowsQ<BITS, CPL, R>& Q, const XLane<BITS, CPL>& x0,
                                         const XLane<BITS, CPL>& x1, float (&out)[R]) {
  opaque(Q);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc += chunk_partial<BITS, NX>(Q.q[r][c], Q.sb[r][c], x0.w[c], x0.s[c], x1.w[c], x1.s[c]);
    out[r] = acc;
  }
}

// 8-bit rows decoded once for several token rows: the bf16 pairs that
// byte_dots builds from each code dword (nibble planes at shifts 0, 8 for the
// low plane, 4, 12 for the high one), kept in registers, and the scale/bias
// word. dot_dec8 then adds, for one token row, exactly the products and sums
// of dot_rows<8, CPL, R, 1> in the same order, so results are bit for bit
// those of the fused decode.
template <int CPL, int R>
struct RowsDec8 {
  uint32_t p[R][CPL][32];
  uint32_t sb[R][CPL];
};
template <int CPL, int R>
__device__ __forceinline__ void decode8(const RowsQ<8, CPL, R>& Q, RowsDec8<CPL, R>& D) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t q = Q.q[r][c][k];
        D.p[r][c][4 * k + 0] = (q & kM4) | kMagic;
        D.p[r][c][4 * k + 1] = ((q >> 8) & kM4) | kMagic;
        D.p[r][c][4 * k + 2] = ((q >> 4) & kM4) | kMagic;
        D.p[r][c][4 * k + 3] = ((q >> 12) & kM4) | kMagic;
      }
      D.sb[r][c] = Q.sb[r][c];
    }
}
template <int CPL, int R>
__device__ __forceinline__ void dot_dec8(const RowsDec8<CPL, R>& D, const XLane<8, CPL>& x, float (&out)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float dl = 0.f, dh = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        dot2c(dl, D.p[r][c][4 * k + 0], x.w[c][2 * k]);
        dot2c(dl, D.p[r][c][4 * k + 1], x.w[c][2 * k + 1]);
        dot2c(dh, D.p[r][c][4 * k + 2], x.w[c][2 * k]);
        dot2c(dh, D.p[r][c][4 * k + 3], x.w[c][2 * k + 1]);
      }
      dot_fence(dl, dh);
      const float s = bf16_lo_to_f32(D.sb[r][c]), b = bf16_hi_to_f32(D.sb[r][c]);
      acc += fmaf(s, fmaf(16.f, dh, dl), (b - 2176.f * s) * x.s[c]);
    }
    out[r] = acc;
  }
}

// Dense bf16 rows (a bf16 router): 16 words per chunk.
template <int CPL, int R>
struct RowsD {
  uint32_t w[R][CPL][16];
};

template <int CPL, int R>
__device__ __forceinline__ void load_dense_rows(RowsD<CPL, R>& Q, const uint16_t* const (&rows)[R], int K, int li,
                                                int lpr) {
  const int nch = K >> 5;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = li + lpr * c;
      if (rows[r] != nullptr && ch < nch) {
        load64B(rows[r] + 32 * ch, Q.w[r][c]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) Q.w[r][c][i] = 0u;
      }
    }
}

template <int CPL, int R>
__device__ __forceinline__ void dot_dense_rows(RowsD<CPL, R>& Q, const XLane<kDense, CPL>& x, float (&out)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(Q.w[r][c][i]));
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc += dense_chunk(Q.w[r][c], x.w[c]);
    out[r] = acc;
  }
}

// ------------------------------------------------------ DPP wave reductions
// GFX9 data-parallel-primitive lane moves (no LDS round trip):
// quad_perm, row_half_mirror, row_mirror, row_bcast:15, row_bcast:31.
constexpr int kDppXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the lpr lanes of each row group (fixed tree). The group's last lane
// (li == lpr - 1) holds the sum; for lpr <= 16 every lane of the group does.
__device__ __forceinline__ float reduce_row(float v, int lpr) {
  if (lpr > 1) v += dpp_f<kDppXor1>(v, 0.f);
  if (lpr > 2) v += dpp_f<kDppXor2>(v, 0.f);
  if (lpr > 4) v += dpp_f<kDppHalfMirror>(v, 0.f);
  if (lpr > 8) v += dpp_f<kDppMirror>(v, 0.f);
  if (lpr > 16) v += dpp_f<kDppBcast15, 0xA>(v, 0.f);
  if (lpr > 32) v += dpp_f<kDppBcast31, 0xC>(v, 0.f);
  return v;
}

// Wave-wide sum, returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = reduce_row(v, 64);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave-wide maximum, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v, -INFINITY));
  v = fmaxf(v, dpp_f<kDppXor2>(v, -INFINITY));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v, -INFINITY));
  v = fmaxf(v, dpp_f<kDppMirror>(v, -INFINITY));
  v = fmaxf(v, dpp_f<kDppBcast15, 0xA>(v, -INFINITY));
  v = fmaxf(v, dpp_f<kDppBcast31, 0xC>(v, -INFINITY));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ------------------------------------------------------------------ top-k
// Order-preserving integer key of a float (larger float -> larger key).
__device__ __forceinline__ int fkey(float f) {
  const int b = __float_as_int(f + 0.0f);  // -0 -> +0
  return b >= 0 ? b : (b ^ 0x7FFFFFFF);
}
__device__ __forceinline__ float key_f(int k) { return __int_as_float(k >= 0 ? k : (k ^ 0x7FFFFFFF)); }

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i<kDppXor1>(v, INT_MIN));
  v = max(v, dpp_i<kDppXor2>(v, INT_MIN));
  v = max(v, dpp_i<kDppHalfMirror>(v, INT_MIN));
  v = max(v, dpp_i<kDppMirror>(v, INT_MIN));
  v = max(v, dpp_i<kDppBcast15, 0xA>(v, INT_MIN));
  v = max(v, dpp_i<kDppBcast31, 0xC>(v, INT_MIN));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v, INT_MAX));
  v = min(v, dpp_i<kDppXor2>(v, INT_MAX));
  v = min(v, dpp_i<kDppHalfMirror>(v, INT_MAX));
  v = min(v, dpp_i<kDppMirror>(v, INT_MAX));
  v = min(v, dpp_i<kDppBcast15, 0xA>(v, INT_MAX));
  v = min(v, dpp_i<kDppBcast31, 0xC>(v, INT_MAX));
  return __builtin_amdgcn_readlane(v, 63);
}

// Top-k of E logits (lane l holds the key of e = l + 64 m, m < M; entries
// with e >= E hold INT_MIN), ties to the lower index, descending; renormalised
// softmax weights over the k selected. Lane i < k ends with the i-th selected
// expert and its weight. E <= 64 M, k <= 16.
// Each lane first sorts its M values (key descending, index ascending); each
// round takes the wave maximum of the lanes' list heads; if several lanes hold
// that key, the lowest index among them wins; the winner pops its head.
// KF: k when known at compile time (0: k <= kMaxTopK at run time).
// on_round(i, id) runs on the whole wave as soon as round i has chosen its
// expert (id wave-uniform), so a caller can hand out each rank early.
struct NoRoundHook {
  __device__ void operator()(int, int) const {}
};
template <int M, int KF = 0, class OnRound = NoRoundHook>
__device__ __forceinline__ void topk_select(int (&key)[M], int k, int& lane_id, float& lane_w,
                                            const OnRound& on_round = OnRound()) {
  constexpr int KMAX = KF ? KF : kMaxTopK;
  const int lane = threadIdx.x & 63;
  int idx[M];
#pragma unroll
  for (int m = 0; m < M; ++m) idx[m] = lane + 64 * m;
  // sort the lane's list: key descending, index ascending (odd-even transposition)
#pragma unroll
  for (int pass = 0; pass < M; ++pass)
#pragma unroll
    for (int m = pass & 1; m + 1 < M; m += 2) {
      const bool swap = key[m + 1] > key[m] || (key[m + 1] == key[m] && idx[m + 1] < idx[m]);
      const int k0 = key[m], i0 = idx[m];
      key[m] = swap ? key[m + 1] : k0;
      idx[m] = swap ? idx[m + 1] : i0;
      key[m + 1] = swap ? k0 : key[m + 1];
      idx[m + 1] = swap ? i0 : idx[m + 1];
    }
  // k rounds of wave max; the selected logits are wave-uniform, lane i keeps
  // round i's (id, logit) so no per-lane array is ever indexed by the lane
  float my_sel = -INFINITY, top = 0.f;
  lane_id = 0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < k) {
      const int mx = wave_max_i(key[0]);
      const unsigned long long b = __ballot(key[0] == mx);
      int id;
      if (__popcll(b) == 1) {
        id = __builtin_amdgcn_readlane(idx[0], (int)__builtin_ctzll(b));
      } else {
        id = wave_min_i(key[0] == mx ? idx[0] : INT_MAX);
      }
      if (idx[0] == id) {  // the winner pops its head
#pragma unroll
        for (int m = 0; m + 1 < M; ++m) {
          key[m] = key[m + 1];
          idx[m] = idx[m + 1];
        }
        key[M - 1] = INT_MIN;
        idx[M - 1] = INT_MAX;
      }
      on_round(i, id);
      const float v = key_f(mx);
      if (i == 0) top = v;
      if (lane == i) {
        lane_id = id;
        my_sel = v;
      }
    }
  }
  // renormalised softmax over the k selected logits, the largest subtracted:
  // one exponential per lane, summed over lanes 0..k-1 (k <= 16, one row of
  // 16 lanes) in a fixed tree
  const float e = lane < k ? expf(my_sel - top) : 0.f;
  const float sum = reduce_row(e, 16);
  lane_w = lane < k ? e / sum : 0.f;
}

// Top-k of one token row on one wave: logits lam_src[0..E) scaled by
// *scale_src (the RMS factor); lane i < k receives the i-th (id, weight).
// M: logits per lane, E <= 64 M (the selection does not depend on M).
template <int M>
__device__ __forceinline__ void wave_topk(const float* lam_src, const float* scale_src, int E, int k, int& lane_id,
                                          float& lane_w, float& scale_out) {
  const int lane = threadIdx.x & 63;
  const float scale = *scale_src;
  scale_out = scale;
  int key[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = lane + 64 * m;
    key[m] = e < E ? fkey(scale * lam_src[e]) : INT_MIN;
  }
  topk_select(key, k, lane_id, lane_w);
}

}  // namespace moe
