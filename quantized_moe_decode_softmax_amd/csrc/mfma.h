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
// each part its own product. sum_j h^2 (for r_t) is the diagonal of the
// 16 x 16 Gram product h h^T of each token tile, also on the matrix cores.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies, for
// A (16 x 32), row l % 16 and the 8 consecutive k = 8 (l / 16) .. + 7; for
// B (32 x 16) column l % 16 and the same k; it receives D[4 (l / 16) + i]
// [l % 16], i = 0..3. Token rows are A's rows (16 per tile, NT tiles), weight
// rows B's columns (16 per workgroup), so each lane converts 8 codes per
// instruction pair and keeps one output row's scale and bias.
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

// A operand rows: NX parts (1: x = h; 2: x = hi + lo), token row t of part n
// at a[n] + t * stride (bf16 elements). Rows t >= T read row T - 1 instead:
// output row t of a product depends on A's row t only, and rows t >= T are
// never stored.
template <int NX>
struct MfA {
  const uint16_t* a[NX];
  int64_t stride;
  int T;
};

// Partial sums of one wave over groups [g0, g1) of the 16 weight rows; the
// lane's weight row starts at row (codes) and sbrow (scale|bias words); a
// lane whose output column is not stored passes any valid row. acc[tt]: y of
// token tile tt; ss[tt]: Gram product of part 0 (SS); gd[tt]: x . gvec (GD).
// Every load is unconditional (clamped addresses), so the NG groups' loads
// are all in flight before the first product.
template <int NT, int NX, int NG, bool SS, bool GD>
__device__ __forceinline__ void mfma_groups(const MfA<NX>& A, const uint8_t* row, const uint32_t* sbrow, int g0,
                                            int g1, const uint16_t* gvec, mf_f32x4 (&acc)[NT], mf_f32x4 (&ss)[NT],
                                            mf_f32x4 (&gd)[NT]) {
  const int lane = threadIdx.x & 63, tl = lane & 15, kq = 8 * (lane >> 4);
  const mf_u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const uint16_t* arow[NX][NT];
#pragma unroll
  for (int n = 0; n < NX; ++n)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int t = 16 * tt + tl;
      arow[n][tt] = A.a[n] + (t < A.T ? t : A.T - 1) * A.stride;
    }
  for (int gb = g0; gb < g1; gb += NG) {
    mf_u32x4 xa[NG][NX][NT][2];
    mf_u32x2 q[NG][2];
    mf_u32x4 gv[NG][2];
    uint32_t sbw[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = gb + j < g1 ? gb + j : g1 - 1;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k = 64 * g + 32 * ks + kq;
#pragma unroll
        for (int n = 0; n < NX; ++n)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) xa[j][n][tt][ks] = *(const mf_u32x4*)(arow[n][tt] + k);
        q[j][ks] = *(const mf_u32x2*)(row + k);
        if constexpr (GD) gv[j][ks] = *(const mf_u32x4*)(gvec + k);
      }
      sbw[j] = sbrow[g];
    }
    // every group of the chunk is computed (no branch keeps the loads above
    // from being hoisted); a group past g1 is weighted by 0
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float okf = gb + j < g1 ? 1.f : 0.f;
      mf_f32x4 D[NT], X[NT], S2[NT], G2[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) D[tt] = X[tt] = S2[tt] = G2[tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const mf_u32x4 b = codes8_bf16(q[j][ks]);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
          for (int n = 0; n < NX; ++n) {
            D[tt] = mfma_bf16(xa[j][n][tt][ks], b, D[tt]);
            X[tt] = mfma_bf16(xa[j][n][tt][ks], ones, X[tt]);
          }
          if constexpr (SS) S2[tt] = mfma_bf16(xa[j][0][tt][ks], xa[j][0][tt][ks], S2[tt]);
          if constexpr (GD) G2[tt] = mfma_bf16(xa[j][0][tt][ks], gv[j][ks], G2[tt]);
        }
      }
      const float s = okf * bf16_lo_to_f32(sbw[j]), bb = okf * bf16_hi_to_f32(sbw[j]);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[tt][i] = fmaf(s, D[tt][i], fmaf(bb, X[tt][i], acc[tt][i]));
          if constexpr (SS) ss[tt][i] = fmaf(okf, S2[tt][i], ss[tt][i]);
          if constexpr (GD) gd[tt][i] = fmaf(okf, G2[tt][i], gd[tt][i]);
        }
    }
  }
}

// LDS for the cross-wave sums: [wave][value][lane]
struct MfmaLds {
  float red[kMfmaWaves][3 * 2 * 4][64];
  float r[32];
  float gd[32];
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
// pairs each (gate rows as columns 0..7, up rows as 8..15). The first pair
// workgroup also writes r_t and the shared gate sigmoid(r_t gvec . h_t).
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
  const bool stats = (int)blockIdx.x == n_rt;
  MfA<1> A;
  A.a[0] = p.h_in;
  A.stride = d.H;
  A.T = d.T;
  mf_f32x4 acc[NT], ss[NT], gd[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = ss[tt] = gd[tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* gvec = (const uint16_t*)(p.layer + d.off_gatevec);
  if (g0 < g1) {
    if (router)
      mfma_groups<NT, 1, NG, false, false>(A, row, sbrow, g0, g1, gvec, acc, ss, gd);
    else if (stats)
      mfma_groups<NT, 1, NG, true, true>(A, row, sbrow, g0, g1, gvec, acc, ss, gd);
    else
      mfma_groups<NT, 1, NG, true, false>(A, row, sbrow, g0, g1, gvec, acc, ss, gd);
  }
  float v[3 * NT * 4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[4 * tt + c] = acc[tt][c];
      v[4 * NT + 4 * tt + c] = ss[tt][c];
      v[8 * NT + 4 * tt + c] = gd[tt][c];
    }
  mfma_reduce(L, v);
  // lane holds rows t = 16 tt + 4 (lane / 16) + c of column tl
  if (wave == 0 && !router) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int tr = 4 * (lane >> 4) + c;
        if (tr == tl) {  // Gram diagonal
          const int t = 16 * tt + tr;
          L.r[t] = rms_factor(v[4 * NT + 4 * tt + c], d.H, d.eps);
          L.gd[t] = v[8 * NT + 4 * tt + c];
        }
      }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 16 * tt + 4 * (lane >> 4) + c;
      const float y = v[4 * tt + c];
      if (router) {
        if (t < d.T && e >= 0 && e < d.E) p.raw[(int64_t)t * d.E + e] = y;
      } else {
        const float r = L.r[t];
        const float yv = y * r;
        const float partner = __shfl_xor(yv, 8);  // up row of the same pair
        if (t < d.T && tl < 8 && i < d.Is) store_a(d, p, t, d.k, i, silu_mul(yv, partner));
      }
    }
  if (stats && lane < d.T) {
    const float r = L.r[lane];
    p.rinv[lane] = r;
    p.sg[lane] = 1.0f / (1.0f + expf(-(r * L.gd[lane])));
  }
}

// Shared expert's down projection y_s[t][j] = W_d a_s[t] (fp32, before the
// gate) for 16 output rows per workgroup; a_s = hi + lo from the activation
// slot k.
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
  MfA<2> A;
  A.a[0] = p.a_hi + (int64_t)d.k * d.imax;
  A.a[1] = p.a_lo + (int64_t)d.k * d.imax;
  A.stride = (int64_t)(d.k + 1) * d.imax;
  A.T = d.T;
  mf_f32x4 acc[NT], ss[NT], gd[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = ss[tt] = gd[tt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
  if (g0 < g1) mfma_groups<NT, 2, NG, false, false>(A, row, sbrow, g0, g1, nullptr, acc, ss, gd);
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
