// MoE decode kernels for gfx950 (wave64) and the moe_decode_layer /
// moe_decode_stack entry points.
//
// One layer runs as five stream-ordered kernels:
//   router_kernel        raw router dot products W_r h_t for every (t, e)
//   topk_kernel          RMS factor, shared gate, top-k, renormalised softmax
//                        weights, and the deduplicated list of experts used by
//                        any row (each expert's bytes are then read once per
//                        call, however many rows select it)
//   gateup_kernel        SwiGLU activations a = silu(r W_g h) * (r W_u h) for
//                        every (unit, row using it); run for the routed units
//                        and for the shared expert
//   down_kernel          routed down projections W_d a, per (row, rank)
//   down_combine_kernel  shared down projection, then the combine
//                        h + sum_i w_i y_i + sigmoid-gate * y_s in rank order,
//                        rounded to bf16 (nearest even)
// The RMS factor r = 1/sqrt(mean(h^2) + eps) is applied after each dot
// product: with RMSNorm weight 1, W (r h) = r (W h).
//
// Dot products: a wave's lanes run along the input dimension in chunks of 32
// codes (half a quantisation group). For 2/4/6-bit codes each pair of codes is
// turned into a bf16 pair (128 + q_a, 128 + q_b) by one mask-and-or (the codes
// land in the mantissa of 128.0) and multiplied with a bf16 pair of inputs by
// v_dot2c_f32_bf16, so a chunk gives D = sum (128 + q) x; the group-affine
// form then is s * D + (b - 128 s) * sum x. This is the flash-moe news page's
// reordering ("FMA-optimised dequant kernel": code*(scale*x) + bias*x) taken
// one step further: scale and bias are applied once per half-group instead of
// once per weight. 8-bit codes (which do not fit a bf16 mantissa above 128)
// use byte-to-float conversion and fp32 FMA. The down projections take the
// fp32 activations as two bf16 parts a = hi + lo (16 significant bits).
//
// Determinism and row-exactness: every reduction has a fixed order, no
// atomics touch data, and the arithmetic for one (row t, output) pair does not
// depend on T or on which other rows share an expert.
#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128.0, 128.0)
constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1.0, 1.0)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// bf16 pair from the same half of two words
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

__host__ __device__ __forceinline__ int pow2ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
__host__ __device__ __forceinline__ int lanes_per_row(int k) {
  int n = pow2ceil(k / 32);
  return n < 64 ? n : 64;
}

__device__ __forceinline__ void load16(const uint16_t* p, uint32_t (&w)[16]) {
  const u32x4* q = (const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 v = q[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// x operand of one 32-code chunk: natural-order bf16 words (single) or hi/lo parts (split)
template <bool SPLIT>
struct XChunk {
  uint32_t hi[16];
  uint32_t lo[SPLIT ? 16 : 1];
};

// D = sum_j (128 + q_j) x_j over a 32-code chunk, bits 2/4/6, from packed words w.
template <int BITS>
__device__ __forceinline__ float magic_dot(const uint32_t* w, const uint32_t (&x)[16], float acc) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q = ((w[d] >> (4 * i)) & 0x000F000Fu) | kMagic;
        const uint32_t a = x[4 * d + (i >> 1)], b = x[4 * d + 2 + (i >> 1)];
        acc = dot2(q, (i & 1) ? pair_hi(a, b) : pair_lo(a, b), acc);
      }
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t hw = w[3 * u + 2];
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sh = 2 * (4 * d + i) - 4;
          const uint32_t hs = sh >= 0 ? (hw >> sh) : (hw << (-sh));
          const uint32_t q = (((w[3 * u + d] >> (4 * i)) & 0x000F000Fu) | kMagic) | (hs & 0x00300030u);
          const int dd = 2 * u + d;
          const uint32_t a = x[4 * dd + (i >> 1)], b = x[4 * dd + 2 + (i >> 1)];
          acc = dot2(q, (i & 1) ? pair_hi(a, b) : pair_lo(a, b), acc);
        }
    }
  } else {  // BITS == 2
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t q = ((w[d] >> (2 * i)) & 0x00030003u) | kMagic;
        const uint32_t a = x[8 * d + (i >> 1)], b = x[8 * d + 4 + (i >> 1)];
        acc = dot2(q, (i & 1) ? pair_hi(a, b) : pair_lo(a, b), acc);
      }
  }
  return acc;
}

__device__ __forceinline__ float sum_pairs(const uint32_t (&x)[16], float acc) {
#pragma unroll
  for (int i = 0; i < 16; ++i) acc = dot2(x[i], kOnes, acc);
  return acc;
}

// sum_j q_j x_j for 8-bit codes (4 per dword, byte j%4), x from bf16 words
__device__ __forceinline__ float byte_dot(const uint32_t* w, const uint32_t (&x)[16], float acc) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t v = w[k];
    const uint32_t xa = x[2 * k], xb = x[2 * k + 1];
    acc = fmaf((float)(v & 0xFFu), bf16_lo_to_f32(xa), acc);
    acc = fmaf((float)((v >> 8) & 0xFFu), bf16_hi_to_f32(xa), acc);
    acc = fmaf((float)((v >> 16) & 0xFFu), bf16_lo_to_f32(xb), acc);
    acc = fmaf((float)(v >> 24), bf16_hi_to_f32(xb), acc);
  }
  return acc;
}

// sum_j q_j x_j for 3-bit codes (10 per dword), codes 32c .. 32c+31 of the row
__device__ __forceinline__ float tri_dot(const uint32_t* row, int c, const uint32_t (&x)[16], float acc) {
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const int j = 32 * c + i;
    const uint32_t q = (row[j / 10] >> (3 * (j % 10))) & 7u;
    const uint32_t xw = x[i >> 1];
    acc = fmaf((float)q, (i & 1) ? bf16_hi_to_f32(xw) : bf16_lo_to_f32(xw), acc);
  }
  return acc;
}

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* row, int c, uint32_t* w) {
  if constexpr (BITS == 2) {
    u32x2 v = *(const u32x2*)(row + 8 * c);
    w[0] = v.x;
    w[1] = v.y;
  } else if constexpr (BITS == 4) {
    u32x4 v = *(const u32x4*)(row + 16 * c);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  } else if constexpr (BITS == 6) {
    const u32x2* p = (const u32x2*)(row + 24 * c);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      u32x2 v = p[i];
      w[2 * i] = v.x;
      w[2 * i + 1] = v.y;
    }
  } else if constexpr (BITS == 8) {
    const u32x4* p = (const u32x4*)(row + 32 * c);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 v = p[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// Partial dot product of one lane: sum over its chunks (c = li, li + lpr, ...)
// of s*D + b_eff*sum(x). Quantised matrix with `BITS`, K columns, row `r`.
// x: bf16 [K] (SPLIT = false) or hi/lo bf16 [K] each (SPLIT = true).
template <int BITS, bool SPLIT>
__device__ float lane_partial(const uint8_t* codes, const uint32_t* sb, int64_t rb, int r, int K, const uint16_t* xhi,
                              const uint16_t* xlo, int li, int lpr) {
  float acc = 0.f;
  const int nch = K >> 5;
  const uint8_t* row = codes + (int64_t)r * rb;
  const uint32_t* sbr = sb + (int64_t)r * (K >> 6);
  for (int c = li; c < nch; c += lpr) {
    XChunk<SPLIT> xc;
    load16(xhi + 32 * c, xc.hi);
    if constexpr (SPLIT) load16(xlo + 32 * c, xc.lo);
    const uint32_t sbw = sbr[c >> 1];
    const float s = bf16_lo_to_f32(sbw), b = bf16_hi_to_f32(sbw);
    float d, sx;
    if constexpr (BITS == 2 || BITS == 4 || BITS == 6) {
      uint32_t w[6];
      load_codes<BITS>(row, c, w);
      d = magic_dot<BITS>(w, xc.hi, 0.f);
      sx = sum_pairs(xc.hi, 0.f);
      if constexpr (SPLIT) {
        d += magic_dot<BITS>(w, xc.lo, 0.f);
        sx += sum_pairs(xc.lo, 0.f);
      }
      acc += fmaf(s, d, (b - 128.f * s) * sx);
    } else {
      if constexpr (BITS == 8) {
        uint32_t w[8];
        load_codes<8>(row, c, w);
        d = byte_dot(w, xc.hi, 0.f);
        if constexpr (SPLIT) d += byte_dot(w, xc.lo, 0.f);
      } else {
        d = tri_dot((const uint32_t*)row, c, xc.hi, 0.f);
        if constexpr (SPLIT) d += tri_dot((const uint32_t*)row, c, xc.lo, 0.f);
      }
      sx = sum_pairs(xc.hi, 0.f);
      if constexpr (SPLIT) sx += sum_pairs(xc.lo, 0.f);
      acc += fmaf(s, d, b * sx);
    }
  }
  return acc;
}

// Partial dot product of one lane for a dense bf16 matrix row (router_bits 16).
__device__ float lane_partial_dense(const uint16_t* wmat, int r, int K, const uint16_t* x, int li, int lpr) {
  float acc = 0.f;
  const int nch = K >> 5;
  for (int c = li; c < nch; c += lpr) {
    uint32_t w[16], xw[16];
    load16(wmat + (int64_t)r * K + 32 * c, w);
    load16(x + 32 * c, xw);
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) d = dot2(w[i], xw[i], d);
    acc += d;
  }
  return acc;
}

__device__ __forceinline__ float reduce_lanes(float v, int lpr) {
  for (int off = 1; off < lpr; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------------ router
template <int RB>
__global__ void __launch_bounds__(kThreads) router_kernel(const uint8_t* layer, int64_t off, int E, int H, int T,
                                                          const uint16_t* h, float* raw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = lanes_per_row(H), rpw = 64 / lpr;
  const int sr = lane / lpr, li = lane % lpr;
  const int rows_per_iter = gridDim.x * kWaves * rpw;
  for (int base = (blockIdx.x * kWaves + wave) * rpw; base < E; base += rows_per_iter) {
    const int e = base + sr;
    const bool ok = e < E;
    const int er = ok ? e : 0;
    for (int t = 0; t < T; ++t) {
      float p;
      if constexpr (RB == 16) {
        p = lane_partial_dense((const uint16_t*)(layer + off), er, H, h + (int64_t)t * H, li, lpr);
      } else {
        const uint8_t* codes = layer + off;
        const uint32_t* sb = (const uint32_t*)(codes + matrix_codes_bytes(RB, E, H));
        p = lane_partial<RB, false>(codes, sb, row_bytes(RB, H), er, H, h + (int64_t)t * H, nullptr, li, lpr);
      }
      p = reduce_lanes(p, lpr);
      if (ok && li == 0) raw[(int64_t)t * E + e] = p;
    }
  }
}

// ------------------------------------------------------------------- top-k
struct Best {
  float v;
  int i;
};
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) { return av > bv || (av == bv && ai < bi); }

__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = red[0];
  for (int w = 1; w < kWaves; ++w) s += red[w];
  return s;
}

__global__ void __launch_bounds__(kThreads) topk_kernel(const uint16_t* gvec, int E, int H, int k, int T, float eps,
                                                        const uint16_t* h, const float* raw, float* rinv, float* sgate,
                                                        int* ids_ws, float* w_ws, int* units, uint32_t* masks,
                                                        int* ids_out, float* w_out) {
  __shared__ float lam[kMaxExperts];
  __shared__ uint32_t emask[kMaxExperts];
  __shared__ unsigned char taken[kMaxExperts];
  __shared__ float red[kWaves];
  __shared__ float bv[kWaves];
  __shared__ int bi[kWaves];
  __shared__ float selv[kMaxTopK];
  __shared__ int seli[kMaxTopK];
  __shared__ int wave_cnt[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kThreads) emask[e] = 0u;
  for (int t = 0; t < T; ++t) {
    const uint16_t* ht = h + (int64_t)t * H;
    float ss = 0.f, gd = 0.f;
    for (int j = tid; j < H; j += kThreads) {
      const float x = __uint_as_float((uint32_t)ht[j] << 16);
      ss = fmaf(x, x, ss);
      gd = fmaf(x, __uint_as_float((uint32_t)gvec[j] << 16), gd);
    }
    ss = block_sum(ss, red);
    gd = block_sum(gd, red);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    const float sg = 1.0f / (1.0f + expf(-(r * gd)));
    for (int e = tid; e < E; e += kThreads) {
      lam[e] = r * raw[(int64_t)t * E + e];
      taken[e] = 0;
    }
    __syncthreads();
    for (int i = 0; i < k; ++i) {
      float v = -INFINITY;
      int vi = 0x7FFFFFFF;
      for (int e = tid; e < E; e += kThreads)
        if (!taken[e] && better(lam[e], e, v, vi)) {
          v = lam[e];
          vi = e;
        }
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off, 64);
        const int oi = __shfl_xor(vi, off, 64);
        if (better(ov, oi, v, vi)) {
          v = ov;
          vi = oi;
        }
      }
      if (lane == 0) {
        bv[wave] = v;
        bi[wave] = vi;
      }
      __syncthreads();
      if (tid == 0) {
        float b = bv[0];
        int bidx = bi[0];
        for (int w = 1; w < kWaves; ++w)
          if (better(bv[w], bi[w], b, bidx)) {
            b = bv[w];
            bidx = bi[w];
          }
        selv[i] = b;
        seli[i] = bidx;
        taken[bidx] = 1;
      }
      __syncthreads();
    }
    if (tid == 0) {
      const float m = selv[0];
      float ex[kMaxTopK];
      float sum = 0.f;
      for (int i = 0; i < k; ++i) {
        ex[i] = expf(selv[i] - m);
        sum += ex[i];
      }
      for (int i = 0; i < k; ++i) {
        const float w = ex[i] / sum;
        ids_ws[t * k + i] = seli[i];
        w_ws[t * k + i] = w;
        if (ids_out) ids_out[t * k + i] = seli[i];
        if (w_out) w_out[t * k + i] = w;
        emask[seli[i]] |= 1u << t;
      }
      rinv[t] = r;
      sgate[t] = sg;
    }
    __syncthreads();
  }
  // compact the experts used by any row, in ascending id order
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += kThreads) {
    const int e = e0 + tid;
    const bool used = e < E && emask[e] != 0u;
    const unsigned long long bal = __ballot(used);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    if (used) {
      units[1 + off + before] = e;
      masks[off + before] = emask[e];
    }
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) tot += wave_cnt[w];
    base += tot;
    __syncthreads();
  }
  if (tid == 0) units[0] = base;
}

// ---------------------------------------------------------------- gate/up
// grid: (row blocks, units). shared == 1: one unit, the shared expert, used by
// every row, activations go to slot k. Otherwise unit y is the y-th entry of
// the deduplicated list (blocks beyond the count exit).
template <int BITS>
__global__ void __launch_bounds__(kThreads) gateup_kernel(const uint8_t* layer, int64_t off_e, int64_t stride,
                                                          int64_t off_up, int I, int H, int k, int T, int shared,
                                                          int rows_per_block, const uint16_t* h, const float* rinv,
                                                          const int* ids_ws, const int* units, const uint32_t* masks,
                                                          uint16_t* a_hi, uint16_t* a_lo, int imax) {
  int e = 0;
  uint32_t mask;
  if (shared) {
    mask = T >= 32 ? 0xFFFFFFFFu : ((1u << T) - 1u);
  } else {
    if ((int)blockIdx.y >= units[0]) return;
    e = units[1 + blockIdx.y];
    mask = masks[blockIdx.y];
  }
  const uint8_t* gate = layer + off_e + (int64_t)e * stride;
  const uint8_t* up = gate + off_up;
  const uint32_t* gsb = (const uint32_t*)(gate + matrix_codes_bytes(BITS, I, H));
  const uint32_t* usb = (const uint32_t*)(up + matrix_codes_bytes(BITS, I, H));
  const int64_t rb = row_bytes(BITS, H);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = lanes_per_row(H), rpw = 64 / lpr;
  const int sr = lane / lpr, li = lane % lpr;
  const int r0 = blockIdx.x * rows_per_block;
  int r1 = r0 + rows_per_block;
  if (r1 > I) r1 = I;
  for (int t = 0; t < T; ++t) {
    if (!(mask >> t & 1u)) continue;
    int slot = k;
    if (!shared)
      for (int i = 0; i < k; ++i)
        if (ids_ws[t * k + i] == e) slot = i;
    const float r = rinv[t];
    const uint16_t* ht = h + (int64_t)t * H;
    for (int base = r0 + wave * rpw; base < r1; base += kWaves * rpw) {
      const int row = base + sr;
      const bool ok = row < r1;
      const int rr = ok ? row : r0;
      float g = lane_partial<BITS, false>(gate, gsb, rb, rr, H, ht, nullptr, li, lpr);
      float v = lane_partial<BITS, false>(up, usb, rb, rr, H, ht, nullptr, li, lpr);
      g = reduce_lanes(g, lpr) * r;
      v = reduce_lanes(v, lpr) * r;
      if (ok && li == 0) {
        const float a = g / (1.0f + expf(-g)) * v;
        const uint32_t hb = __float_as_uint(a) & 0xFFFF0000u;
        const float lo = a - __uint_as_float(hb);
        const int64_t idx = ((int64_t)t * (k + 1) + slot) * imax + row;
        a_hi[idx] = (uint16_t)(hb >> 16);
        a_lo[idx] = (uint16_t)f32_to_bf16_rne(lo);
      }
    }
  }
}

// ------------------------------------------------------------------- down
// Routed down projections: dsum[t][slot][j] = (W_d,e a[t][slot])_j.
template <int BITS>
__global__ void __launch_bounds__(kThreads) down_kernel(const uint8_t* layer, int64_t off_e, int64_t stride,
                                                        int64_t off_down, int I, int H, int k, int T,
                                                        int rows_per_block, const int* ids_ws, const int* units,
                                                        const uint32_t* masks, const uint16_t* a_hi,
                                                        const uint16_t* a_lo, int imax, float* dsum) {
  if ((int)blockIdx.y >= units[0]) return;
  const int e = units[1 + blockIdx.y];
  const uint32_t mask = masks[blockIdx.y];
  const uint8_t* down = layer + off_e + (int64_t)e * stride + off_down;
  const uint32_t* dsb = (const uint32_t*)(down + matrix_codes_bytes(BITS, H, I));
  const int64_t rb = row_bytes(BITS, I);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = lanes_per_row(I), rpw = 64 / lpr;
  const int sr = lane / lpr, li = lane % lpr;
  const int r0 = blockIdx.x * rows_per_block;
  int r1 = r0 + rows_per_block;
  if (r1 > H) r1 = H;
  for (int t = 0; t < T; ++t) {
    if (!(mask >> t & 1u)) continue;
    int slot = 0;
    for (int i = 0; i < k; ++i)
      if (ids_ws[t * k + i] == e) slot = i;
    const int64_t aoff = ((int64_t)t * (k + 1) + slot) * imax;
    for (int base = r0 + wave * rpw; base < r1; base += kWaves * rpw) {
      const int row = base + sr;
      const bool ok = row < r1;
      float p = lane_partial<BITS, true>(down, dsb, rb, ok ? row : r0, I, a_hi + aoff, a_lo + aoff, li, lpr);
      p = reduce_lanes(p, lpr);
      if (ok && li == 0) dsum[((int64_t)t * k + slot) * H + row] = p;
    }
  }
}

// Shared down projection + combine + residual + bf16 output.
template <int BITS>
__global__ void __launch_bounds__(kThreads) down_combine_kernel(const uint8_t* layer, int64_t off_s, int64_t off_down,
                                                                int Is, int H, int k, int T, int rows_per_block,
                                                                const uint16_t* h, const float* wts, const float* sgate,
                                                                const uint16_t* a_hi, const uint16_t* a_lo, int imax,
                                                                const float* dsum, uint16_t* h_out) {
  const uint8_t* down = layer + off_s + off_down;
  const uint32_t* dsb = (const uint32_t*)(down + matrix_codes_bytes(BITS, H, Is));
  const int64_t rb = row_bytes(BITS, Is);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = lanes_per_row(Is), rpw = 64 / lpr;
  const int sr = lane / lpr, li = lane % lpr;
  const int r0 = blockIdx.x * rows_per_block;
  int r1 = r0 + rows_per_block;
  if (r1 > H) r1 = H;
  for (int t = 0; t < T; ++t) {
    const int64_t aoff = ((int64_t)t * (k + 1) + k) * imax;
    for (int base = r0 + wave * rpw; base < r1; base += kWaves * rpw) {
      const int row = base + sr;
      const bool ok = row < r1;
      float p = lane_partial<BITS, true>(down, dsb, rb, ok ? row : r0, Is, a_hi + aoff, a_lo + aoff, li, lpr);
      p = reduce_lanes(p, lpr);
      if (ok && li == 0) {
        float acc = 0.f;
        for (int i = 0; i < k; ++i) acc = fmaf(wts[t * k + i], dsum[((int64_t)t * k + i) * H + row], acc);
        acc = fmaf(sgate[t], p, acc);
        const float out = __uint_as_float((uint32_t)h[(int64_t)t * H + row] << 16) + acc;
        h_out[(int64_t)t * H + row] = (uint16_t)f32_to_bf16_rne(out);
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch
int blocks_for(int rows, int rows_per_block) { return (rows + rows_per_block - 1) / rows_per_block; }

int rows_per_block_for(int k_dim, int passes) { return kWaves * (64 / lanes_per_row(k_dim)) * passes; }

#define MOE_BITS_SWITCH(bits, B, ...)               \
  switch (bits) {                                   \
    case 2: { constexpr int B = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int B = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int B = 4; __VA_ARGS__; } break; \
    case 6: { constexpr int B = 6; __VA_ARGS__; } break; \
    case 8: { constexpr int B = 8; __VA_ARGS__; } break; \
    default: break;                                 \
  }

struct LayerCall {
  const moe_shape_t* s;
  moe_layer_layout_t L;
  WsMap m;
  uint8_t* ws;
  int T;
};

int32_t launch_layer(const LayerCall& c, const uint8_t* layer, const uint16_t* h_in, uint16_t* h_out, int32_t* ids_out,
                     float* w_out, hipStream_t st) {
  const moe_shape_t& s = *c.s;
  const WsMap& m = c.m;
  uint8_t* ws = c.ws;
  const int T = c.T, E = s.n_experts, H = s.hidden, k = s.top_k;
  const int max_units = T * k < E ? T * k : E;
  const int imax = s.inter > s.shared_inter ? s.inter : s.shared_inter;
  float* raw = (float*)(ws + m.raw_logits);
  float* rinv = (float*)(ws + m.rinv);
  float* sg = (float*)(ws + m.sgate);
  int* ids = (int*)(ws + m.ids);
  float* wts = (float*)(ws + m.wts);
  int* units = (int*)(ws + m.units);
  uint32_t* masks = (uint32_t*)(ws + m.masks);
  uint16_t* a_hi = (uint16_t*)(ws + m.a_hi);
  uint16_t* a_lo = (uint16_t*)(ws + m.a_lo);
  float* dsum = (float*)(ws + m.dsum);

  {  // router
    const int rpb = rows_per_block_for(H, 1);
    const int g = blocks_for(E, rpb);
    if (s.router_bits == 16) {
      router_kernel<16><<<g, kThreads, 0, st>>>(layer, c.L.router, E, H, T, h_in, raw);
    } else {
      MOE_BITS_SWITCH(s.router_bits, B, router_kernel<B><<<g, kThreads, 0, st>>>(layer, c.L.router, E, H, T, h_in, raw));
    }
  }
  topk_kernel<<<1, kThreads, 0, st>>>((const uint16_t*)(layer + c.L.gatevec), E, H, k, T, s.rms_eps, h_in, raw, rinv,
                                      sg, ids, wts, units, masks, ids_out, w_out);
  {  // gate/up, routed units then shared expert
    const int rpb = rows_per_block_for(H, 4);
    dim3 g(blocks_for(s.inter, rpb), max_units);
    MOE_BITS_SWITCH(s.expert_bits, B,
                    gateup_kernel<B><<<g, kThreads, 0, st>>>(layer, c.L.expert0, c.L.expert_stride, c.L.expert_up,
                                                             s.inter, H, k, T, 0, rpb, h_in, rinv, ids, units, masks,
                                                             a_hi, a_lo, imax));
    dim3 gs(blocks_for(s.shared_inter, rpb), 1);
    MOE_BITS_SWITCH(s.shared_bits, B,
                    gateup_kernel<B><<<gs, kThreads, 0, st>>>(layer, c.L.shared, 0, c.L.shared_up, s.shared_inter, H,
                                                              k, T, 1, rpb, h_in, rinv, ids, units, masks, a_hi, a_lo,
                                                              imax));
  }
  {  // down: routed, then shared + combine
    const int rpb = rows_per_block_for(s.inter, 4);
    dim3 g(blocks_for(H, rpb), max_units);
    MOE_BITS_SWITCH(s.expert_bits, B,
                    down_kernel<B><<<g, kThreads, 0, st>>>(layer, c.L.expert0, c.L.expert_stride, c.L.expert_down,
                                                           s.inter, H, k, T, rpb, ids, units, masks, a_hi, a_lo, imax,
                                                           dsum));
    const int rps = rows_per_block_for(s.shared_inter, 2);
    MOE_BITS_SWITCH(s.shared_bits, B,
                    down_combine_kernel<B><<<blocks_for(H, rps), kThreads, 0, st>>>(
                        layer, c.L.shared, c.L.shared_down, s.shared_inter, H, k, T, rps, h_in, wts, sg, a_hi, a_lo,
                        imax, dsum, h_out));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

int32_t check_call(const moe_shape_t* shape, int32_t T, const void* h_in, const void* h_out, const void* ws,
                   size_t ws_bytes, WsMap* m) {
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  if (!h_in || !h_out || !ws) return set_error(MOE_ERR_INVALID_ARG, "NULL h_in, h_out or workspace");
  if ((uintptr_t)h_in % 16 || (uintptr_t)h_out % 16) return set_error(MOE_ERR_ALIGNMENT, "h_in/h_out must be 16-byte aligned");
  if ((uintptr_t)ws % kAlign) return set_error(MOE_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  *m = ws_map(*shape, T);
  if ((int64_t)ws_bytes < m->total)
    return set_error(MOE_ERR_WORKSPACE, "workspace %zu bytes < %lld needed", ws_bytes, (long long)m->total);
  const int64_t hb = (int64_t)T * shape->hidden * 2;
  const char* a = (const char*)h_in;
  const char* b = (const char*)h_out;
  if (a < b + hb && b < a + hb) return set_error(MOE_ERR_INVALID_ARG, "h_in and h_out overlap");
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int32_t moe_decode_layer(const moe_shape_t* shape, const void* layer_dev, int32_t T,
                                    const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev, float* w_dev,
                                    void* ws_dev, size_t ws_bytes, moe_stream_t stream) {
  clear_error();
  WsMap m;
  int32_t rc = check_call(shape, T, h_in_dev, h_out_dev, ws_dev, ws_bytes, &m);
  if (rc) return rc;
  if (!layer_dev) return set_error(MOE_ERR_INVALID_ARG, "layer_dev is NULL");
  if ((uintptr_t)layer_dev % kAlign) return set_error(MOE_ERR_ALIGNMENT, "layer_dev must be 256-byte aligned");
  if (((uintptr_t)ids_dev % 4) || ((uintptr_t)w_dev % 4)) return set_error(MOE_ERR_ALIGNMENT, "ids/w must be 4-byte aligned");
  LayerCall c{shape, {}, m, (uint8_t*)ws_dev, T};
  layout_of(*shape, &c.L);
  return launch_layer(c, (const uint8_t*)layer_dev, h_in_dev, h_out_dev, ids_dev, w_dev, (hipStream_t)stream);
}

extern "C" int32_t moe_decode_stack(const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers,
                                    int32_t T, const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev,
                                    float* w_dev, uint16_t* h_trace_dev, void* ws_dev, size_t ws_bytes,
                                    moe_stream_t stream) {
  clear_error();
  WsMap m;
  int32_t rc = check_call(shape, T, h_in_dev, h_out_dev, ws_dev, ws_bytes, &m);
  if (rc) return rc;
  if (!layers_host || n_layers < 1 || n_layers > 4096) return set_error(MOE_ERR_INVALID_ARG, "bad layer list");
  for (int l = 0; l < n_layers; ++l) {
    if (!layers_host[l]) return set_error(MOE_ERR_INVALID_ARG, "layer %d pointer is NULL", l);
    if ((uintptr_t)layers_host[l] % kAlign) return set_error(MOE_ERR_ALIGNMENT, "layer %d not 256-byte aligned", l);
  }
  if (((uintptr_t)ids_dev % 4) || ((uintptr_t)w_dev % 4) || ((uintptr_t)h_trace_dev % 16))
    return set_error(MOE_ERR_ALIGNMENT, "ids/w must be 4-byte and h_trace 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  LayerCall c{shape, {}, m, (uint8_t*)ws_dev, T};
  layout_of(*shape, &c.L);
  const int64_t th = (int64_t)T * shape->hidden;
  const int64_t tk = (int64_t)T * shape->top_k;
  uint16_t* hb = (uint16_t*)((uint8_t*)ws_dev + m.hbuf);
  if (h_trace_dev) {
    hipError_t e = hipMemcpyAsync(h_trace_dev, h_in_dev, th * 2, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  }
  const uint16_t* cur = h_in_dev;
  for (int l = 0; l < n_layers; ++l) {
    uint16_t* nxt;
    if (h_trace_dev) nxt = h_trace_dev + (l + 1) * th;
    else if (l == n_layers - 1) nxt = h_out_dev;
    else nxt = hb + (l & 1) * th;
    rc = launch_layer(c, (const uint8_t*)layers_host[l], cur, nxt, ids_dev ? ids_dev + l * tk : nullptr,
                      w_dev ? w_dev + l * tk : nullptr, st);
    if (rc) return rc;
    cur = nxt;
  }
  if (h_trace_dev) {
    hipError_t e = hipMemcpyAsync(h_out_dev, cur, th * 2, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}
