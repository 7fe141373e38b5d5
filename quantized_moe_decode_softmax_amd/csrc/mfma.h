// Grouped dequant-GEMM on the gfx950 bf16 matrix cores, for calls with many
// token rows (T > 8): the router and the shared expert are then dense
// contractions of M = T rows, each weight reused by every row.
//
// Sources: flash-moe news page (ja.news.hada.io topic 27758), "Metal Compute
// Shaders" (per-group affine dequantisation w = q s + b fused into the
// product; SwiGLU; RMS normalisation) and PureDrive-35B-A3B-MLX model card,
// "How it works" (several token rows in one pass read each weight once).
//
// Arithmetic. For output row o, token row t and group g of 64 inputs:
//   y[t][o] = sum_g ( s[o][g] * D_g[t][o] + b[o][g] * X_g[t] ),
//   D_g[t][o] = sum_{j in g} q[o][j] x[t][j],   X_g[t] = sum_{j in g} x[t][j].
// An 8-bit code q (0..255) has at most 8 significant bits, so it is exact in
// bf16; so is the product of two bf16 values in the fp32 accumulator. D_g is
// two v_mfma_f32_16x16x32_bf16 (K = 32 each) into a fresh accumulator, X_g the
// same two with an all-ones weight operand, and the per-group scale and bias
// are applied on the vector unit. With x = h (bf16, the layer input) the RMS
// factor r_t multiplies y afterwards (RMSNorm has weight 1); the down
// projection's input a is the activation split a = hi + lo (two bf16 parts),
// each part its own product.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies, for
// A (16 x 32), row l % 16 and the 8 k-slots 8 (l / 16) .. + 7; for B (32 x 16)
// column l % 16 and the same slots; it receives D[4 (l / 16) + i][l % 16],
// i = 0..3. Token rows are A's rows (16 per tile, NT tiles), weight rows B's
// columns (16 per workgroup). A sum over k does not depend on which k sits in
// which slot as long as A and B agree, so the two products of group g give
// lane quadrant q the inputs 64 g + 16 q + 8 c .. + 7 (c = 0, 1): each lane
// loads its weight row's 16 codes of the group in one 16-byte load (a full
// 64-byte group per row and instruction).
//
// Token-row operands are read from a packed copy (mfma_pack_kernel for h, the
// shared expert's SwiGLU for a) in which the A operand of one product, tile tt,
// group g, half c, is 1 KB in lane order: element e of lane l = 16 q + r is
// x[16 tt + r][64 g + 16 q + 8 c + e]. A wave's load of it is one contiguous
// kilobyte; loaded from the row-major [T][K] array the same operand is 16
// rows of 64 bytes a whole row apart, which measured 5 to 6 us slower per
// call at T = 32 and H = 4096 (every workgroup reads all of h).
//
// Work split: one workgroup of 8 waves per 16 weight rows; the waves split
// the groups of K and their partial sums are added in wave order in LDS
// (fixed order: results are deterministic). Each wave issues the loads of up
// to NG groups before computing them.
#pragma once

namespace moe {
namespace {

constexpr int kMfmaMinT = 9;  // T at which the router and shared expert use the matrix cores
constexpr int kMfmaWaves = 8;
constexpr int kMfmaThreads = 64 * kMfmaWaves;

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ mf_f32x4 mfma_bf16(mf_u32x4 a, mf_u32x4 b, mf_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, a), __builtin_bit_cast(mf_bf16x8, b),
                                                 c, 0, 0, 0);
}

// 8 codes (bytes, in k order) -> 8 bf16 in k order: each byte converted to
// f32 exactly, the top halves packed (exact: at most 8 significant bits).
__device__ __forceinline__ uint32_t bytes01_bf16(uint32_t w) {
  const float f0 = (float)(w & 0xFFu), f1 = (float)((w >> 8) & 0xFFu);
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}
__device__ __forceinline__ uint32_t bytes23_bf16(uint32_t w) {
  const float f2 = (float)((w >> 16) & 0xFFu), f3 = (float)(w >> 24);
  return __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}
__device__ __forceinline__ mf_u32x4 codes8_bf16(mf_u32x2 q) {
  mf_u32x4 r;
  r.x = bytes01_bf16(q.x);
  r.y = bytes23_bf16(q.x);
  r.z = bytes01_bf16(q.y);
  r.w = bytes23_bf16(q.y);
  return r;
}

// Element index of x[t][k] in the packed copy of a [16 NT][K] operand
// (G = K / 64 groups): block (t / 16, k / 64, half), lane 16 q + t % 16.
__device__ __forceinline__ int64_t packed_index(int t, int k, int G) {
  const int g = k >> 6, w = k & 63, q = w >> 4, c = (w >> 3) & 1, e = w & 7;
  return ((((int64_t)(t >> 4) * G + g) * 2 + c) * 64 + 16 * q + (t & 15)) * 8 + e;
}

// Packed copy of h for the matrix-core kernels, and the per-row statistics:
// r_t = 1 / sqrt(mean(h_t^2) + eps) and the shared expert's gate
// sigmoid(r_t gvec . h_t). One workgroup per token row of 16 NT (rows t >= T
// are written as zeros); thread j takes 16 consecutive inputs per pass (one
// lane quadrant of a group: both halves), so the row is read contiguously.
// The sums are fp32 in a fixed order (thread, then wave tree, then waves).
__global__ void __launch_bounds__(256) mfma_pack_kernel(Dims d, Ptrs p_) {
  const Ptrs p = with_layer(p_);
  __shared__ float s_part[2][4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = d.H >> 6, nq = d.H >> 4;
  const bool live = t < d.T;
  const uint16_t* gvec = (const uint16_t*)(p.layer + d.off_gatevec);
  float ss = 0.f, gd = 0.f;
  for (int j = tid; j < nq; j += 256) {
    mf_u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
    if (live) {
      x0 = gload<mf_u32x4>((const uint8_t*)(p.h_in + (int64_t)t * d.H + 16 * j));
      x1 = gload<mf_u32x4>((const uint8_t*)(p.h_in + (int64_t)t * d.H + 16 * j + 8));
      const mf_u32x4 g0 = gload<mf_u32x4>((const uint8_t*)(gvec + 16 * j));
      const mf_u32x4 g1 = gload<mf_u32x4>((const uint8_t*)(gvec + 16 * j + 8));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = bf16_lo_to_f32(x0[i]), a1 = bf16_hi_to_f32(x0[i]);
        const float b0 = bf16_lo_to_f32(x1[i]), b1 = bf16_hi_to_f32(x1[i]);
        ss = fmaf(a0, a0, ss);
        ss = fmaf(a1, a1, ss);
        ss = fmaf(b0, b0, ss);
        ss = fmaf(b1, b1, ss);
        gd = fmaf(a0, bf16_lo_to_f32(g0[i]), gd);
        gd = fmaf(a1, bf16_hi_to_f32(g0[i]), gd);
        gd = fmaf(b0, bf16_lo_to_f32(g1[i]), gd);
        gd = fmaf(b1, bf16_hi_to_f32(g1[i]), gd);
      }
    }
    const int k = 16 * j;
    *(mf_u32x4*)(p.hp + packed_index(t, k, G)) = x0;
    *(mf_u32x4*)(p.hp + packed_index(t, k + 8, G)) = x1;
  }
  if (!live) return;
  ss = wave_sum(ss);
  gd = wave_sum(gd);
  if (lane == 0) {
    s_part[0][wave] = ss;
    s_part[1][wave] = gd;
  }
  __syncthreads();
  if (tid == 0) {
    const float sq = (s_part[0][0] + s_part[0][1]) + (s_part[0][2] + s_part[0][3]);
    const float g = (s_part[1][0] + s_part[1][1]) + (s_part[1][2] + s_part[1][3]);
    const float r = rms_factor(sq, d.H, d.eps);
    p.rinv[t] = r;
    p.sg[t] = 1.0f / (1.0f + expf(-(r * g)));
  }
}

// Partial sums of one wave over groups [g0, g1) of the 16 weight rows; the
// lane's weight row starts at row (codes) and sbrow (scale|bias words); a
// lane whose output column is not stored passes any valid row. x[n]: packed
// token-row operand of part n (G groups per row). acc[tt]: y of token tile tt.
// Every load is unconditional (clamped group), so the NG groups' loads are
// all in flight before the first product.
template <int NT, int NX, int NG>
__device__ __forceinline__ void mfma_groups(const uint16_t* const (&x)[NX], int G, const uint8_t* row,
                                            const uint32_t* sbrow, int g0, int g1, mf_f32x4 (&acc)[NT]) {
  const int lane = threadIdx.x & 63, q = lane >> 4;
  const mf_u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  for (int gb = g0; gb < g1; gb += NG) {
    mf_u32x4 xa[NG][NX][NT][2];
    mf_u32x4 bq[NG];
    uint32_t sbw[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = gb + j < g1 ? gb + j : g1 - 1;
      bq[j] = gload<mf_u32x4>(row + 64 * g + 16 * q);
      sbw[j] = gload<uint32_t>((const uint8_t*)(sbrow + g));
#pragma unroll
      for (int n = 0; n < NX; ++n)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            xa[j][n][tt][c] =
                gload<mf_u32x4>((const uint8_t*)(x[n] + ((((int64_t)tt * G + g) * 2 + c) * 64 + lane) * 8));
    }
    // the scheduler would otherwise sink each load to its first use, a round
    // trip per product
    __builtin_amdgcn_sched_barrier(0);
    // every group of the chunk is computed (no branch keeps the loads above
    // from being hoisted); a group past g1 is weighted by 0
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float okf = gb + j < g1 ? 1.f : 0.f;
      mf_f32x4 D[NT], X[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) D[tt] = X[tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const mf_u32x4 b = codes8_bf16(c ? mf_u32x2{bq[j].z, bq[j].w} : mf_u32x2{bq[j].x, bq[j].y});
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int n = 0; n < NX; ++n) {
            D[tt] = mfma_bf16(xa[j][n][tt][c], b, D[tt]);
            X[tt] = mfma_bf16(xa[j][n][tt][c], ones, X[tt]);
          }
      }
      const float s = okf * bf16_lo_to_f32(sbw[j]), bb = okf * bf16_hi_to_f32(sbw[j]);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tt][i] = fmaf(s, D[tt][i], fmaf(bb, X[tt][i], acc[tt][i]));
    }
  }
}

// LDS for the cross-wave sums: [wave][value][lane]
struct MfmaLds {
  float red[kMfmaWaves][2 * 4][64];
};

// Adds the waves' values v[0..nv) (per lane) in wave order; the totals land
// in wave 0's v. All threads of the workgroup call it.
template <int NV>
__device__ __forceinline__ void mfma_reduce(MfmaLds& L, float (&v)[NV]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i) L.red[wave][i][lane] = v[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float s = L.red[0][i][lane];
      for (int w = 1; w < kMfmaWaves; ++w) s += L.red[w][i][lane];
      v[i] = s;
    }
  }
}

// Router logits (before the RMS factor) and shared-expert activations of all
// T rows. Workgroups [0, n_rt): 16 router rows each; [n_rt, ..): 8 shared
// pairs each (gate rows as columns 0..7, up rows as 8..15), whose activations
// go to the packed copy the shared down projection reads (rows t >= T: 0).
// r_t comes from mfma_pack_kernel, launched before.
template <int NT, int NG>
__global__ void __launch_bounds__(kMfmaThreads) route_mfma_kernel(Dims d, Ptrs p_, int n_rt) {
  const Ptrs p = with_layer(p_);
  __shared__ MfmaLds L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tl = lane & 15;
  const int G = d.H >> 6;
  const int gpw = (G + kMfmaWaves - 1) / kMfmaWaves;
  const int g0 = wave * gpw, g1 = min(G, g0 + gpw);
  const bool router = (int)blockIdx.x < n_rt;
  const int64_t rb = d.H;  // 8-bit codes: one byte per input
  const uint8_t* row;
  const uint32_t* sbrow;
  int e = -1, i = -1;
  if (router) {
    e = blockIdx.x * 16 + tl;
    const int ec = e < d.E ? e : d.E - 1;  // a valid row for columns not stored
    const uint8_t* base = p.layer + d.off_router;
    row = base + ec * rb;
    sbrow = (const uint32_t*)(base + matrix_codes_bytes(8, d.E, d.H)) + (int64_t)ec * G;
  } else {
    i = (blockIdx.x - n_rt) * 8 + (tl & 7);
    const int ic = i < d.Is ? i : d.Is - 1;
    const uint8_t* base = p.layer + d.off_shared + (tl < 8 ? 0 : d.off_shared_up);
    row = base + ic * rb;
    sbrow = (const uint32_t*)(base + matrix_codes_bytes(8, d.Is, d.H)) + (int64_t)ic * G;
  }
  const uint16_t* const x[1] = {p.hp};
  // the RMS factors of the lane's output rows, requested before the products
  // so that the epilogue does not wait for them
  float rt[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 16 * tt + 4 * (lane >> 4) + c;
      rt[tt][c] = !router && wave == 0 && t < d.T ? p.rinv[t] : 0.f;
    }
  mf_f32x4 acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
  if (g0 < g1) mfma_groups<NT, 1, NG>(x, G, row, sbrow, g0, g1, acc);
  float v[4 * NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int c = 0; c < 4; ++c) v[4 * tt + c] = acc[tt][c];
  mfma_reduce(L, v);
  if (wave != 0) return;
  // lane holds rows t = 16 tt + 4 (lane / 16) + c of column tl
  const int Gi = d.Is >> 6;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 16 * tt + 4 * (lane >> 4) + c;
      const float y = v[4 * tt + c];
      if (router) {
        if (t < d.T && e >= 0 && e < d.E) p.raw[(int64_t)t * d.E + e] = y;
      } else {
        const float yv = y * rt[tt][c];
        const float partner = __shfl_xor(yv, 8);  // up row of the same pair
        if (tl < 8 && i < d.Is) {
          const float a = silu_mul(yv, partner);
          const uint32_t hb = __float_as_uint(a) & 0xFFFF0000u;
          const int64_t idx = packed_index(t, i, Gi);
          p.ap[idx] = (uint16_t)(hb >> 16);
          p.ap[(int64_t)16 * NT * d.Is + idx] = (uint16_t)f32_to_bf16_rne(a - __uint_as_float(hb));
        }
      }
    }
}

// Shared expert's down projection y_s[t][j] = W_d a_s[t] (fp32, before the
// gate) for 16 output rows per workgroup; a_s = hi + lo from the packed copy
// the route kernel wrote.
template <int NT, int NG>
__global__ void __launch_bounds__(kMfmaThreads) down_mfma_kernel(Dims d, Ptrs p_) {
  const Ptrs p = with_layer(p_);
  __shared__ MfmaLds L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tl = lane & 15;
  const int G = d.Is >> 6;
  const int gpw = (G + kMfmaWaves - 1) / kMfmaWaves;
  const int g0 = wave * gpw, g1 = min(G, g0 + gpw);
  const int j = blockIdx.x * 16 + tl;
  const int jc = j < d.H ? j : d.H - 1;  // a valid row for columns not stored
  const uint8_t* base = p.layer + d.off_shared + d.off_shared_down;
  const uint8_t* row = base + (int64_t)jc * d.Is;
  const uint32_t* sbrow = (const uint32_t*)(base + matrix_codes_bytes(8, d.H, d.Is)) + (int64_t)jc * G;
  const uint16_t* const x[2] = {p.ap, p.ap + (int64_t)16 * NT * d.Is};
  mf_f32x4 acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
  if (g0 < g1) mfma_groups<NT, 2, NG>(x, G, row, sbrow, g0, g1, acc);
  float v[4 * NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int c = 0; c < 4; ++c) v[4 * tt + c] = acc[tt][c];
  mfma_reduce(L, v);
  if (wave != 0) return;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 16 * tt + 4 * (lane >> 4) + c;
      if (t < d.T && j < d.H) p.ysh[(int64_t)t * d.H + j] = v[4 * tt + c];
    }
}

}  // namespace
}  // namespace moe
