// Grouped-query decode attention over a bf16 K/V cache (gfx950): verify rows
// i = 0..T-1 at positions p0 + i attend causally to the cache, query head h
// to KV head h / g. moe_gqa_decode computes it in two kernels:
//
//   attn_partial_kernel  one workgroup per (chunk of kChunk positions, KV head):
//                        the chunk's keys and values are read for every query
//                        head of that KV head and (in passes of up to kQG
//                        queries) every verify row; per (row, head) it keeps
//                        the running maximum, the sum of exponentials and the
//                        weighted sum of values (online softmax), then combines
//                        its four waves in a fixed order and stores
//                        (max, sum, acc[d]) for the chunk;
//   attn_combine_kernel  per (row, head): merges the chunks the row sees, in
//                        ascending chunk order, and divides.
//
// Split points are the fixed multiples of kChunk, and every sum runs in an
// order fixed by the position alone, so a row of a T-row call equals a one-row
// call at that position bit for bit (PureDrive-35B-A3B-MLX model card, "How it
// works": K/V read once for all query heads of a KV head and all verify rows,
// split-K with split points and summation order that depend only on the row's
// position). Shapes of the card ("Beyond this checkpoint"): 16 query heads,
// 2 KV heads, head dimension 256; bf16 KV cache ("Hardware"). Scores are the
// bf16 products of q and k accumulated in fp32 by v_dot2c_f32_bf16, scaled by
// 1/sqrt(d); probabilities and the output are fp32.
#include <cmath>

#include "gemv.h"

namespace moe {
namespace {

constexpr int kAttnThreads = 256;              // 4 waves
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kSub = kAttnThreads;             // positions per pass over the workgroup (one per lane)
constexpr int kChunk = 2 * kSub;               // positions per workgroup (split size)
// queries per pass (registers: a key row, kQG scores and kQG x d / 64 sums per lane)
template <int D>
constexpr int qg_of() { return D >= 256 ? 8 : 16; }
constexpr int kMaxHeadDim = 256;

struct AttnArgs {
  int n_q, n_kv, g, S, T, p0, n_chunks, rg;    // rg: verify rows per pass (rg * g <= queries per pass)
  float scale;                                 // 1 / sqrt(d)
  const uint16_t* q;                           // bf16 [T][n_q][D]
  const uint16_t* k;                           // bf16 [n_kv][S][D]
  const uint16_t* v;
  float* o;                                    // fp32 [T][n_q][D]
  float* part;                                 // fp32 [n_chunks][T][n_q][D + 4]
};

template <int D>
__device__ __forceinline__ int pstride() { return D + 4; }

// Loads D bf16 values of position j (row of the cache) as D/2 words.
template <int D>
__device__ __forceinline__ void load_row(const uint16_t* base, uint32_t (&w)[D / 2]) {
  const u32x4* p = (const u32x4*)base;
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const u32x4 x = gload<u32x4>((const uint8_t*)(p + i));
    w[4 * i] = x.x;
    w[4 * i + 1] = x.y;
    w[4 * i + 2] = x.z;
    w[4 * i + 3] = x.w;
  }
}

// G: query heads per KV head (compile time, so that a query slot's row and
// head are constants); QG queries (RG whole rows of G heads) per pass.
template <int D, int G>
__global__ void __launch_bounds__(kAttnThreads) attn_partial_kernel(AttnArgs a) {
  constexpr int DL = D / 64;  // output elements per lane in the value pass
  constexpr int RG = qg_of<D>() / G;
  constexpr int QG = RG * G;
  __shared__ uint32_t s_q[QG][D / 2];                  // the pass's queries (bf16 pairs)
  __shared__ float s_p[kAttnWaves][64][QG];            // probabilities, by wave, position (lane), query
  __shared__ float s_ml[kAttnWaves][QG][2];            // per wave: running max, sum
  __shared__ float s_sc[kAttnWaves][QG];               // per wave: this step's rescale factor of each query
  __shared__ float s_acc[kAttnWaves - 1][QG][D];       // waves 1..3: weighted value sums
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x, kv = blockIdx.y;
  const int c0 = c * kChunk;
  if (c0 > a.p0 + a.T - 1) return;
  const uint16_t* kbase = a.k + (int64_t)kv * a.S * D;
  const uint16_t* vbase = a.v + (int64_t)kv * a.S * D;
  for (int t0 = 0; t0 < a.T; t0 += RG) {
    const int nr = min(RG, a.T - t0);
    const int lim0 = a.p0 + t0;  // row r of the pass sees positions <= lim0 + r
    if (c0 > lim0 + nr - 1) continue;  // no row of this pass sees the chunk (later rows may)
    __syncthreads();  // the previous pass is done with s_q and s_acc
    for (int i = threadIdx.x; i < nr * G * (D / 2); i += kAttnThreads) {
      const int qi = i / (D / 2), wd = i % (D / 2);
      s_q[qi][wd] = ((const uint32_t*)(a.q + ((int64_t)(t0 + qi / G) * a.n_q + kv * G + qi % G) * D))[wd];
    }
    __syncthreads();
    // lane qi (< QG) keeps query qi's running maximum and sum of this wave
    float m_lane = -INFINITY, l_lane = 0.f, acc[QG][DL];
#pragma unroll
    for (int qi = 0; qi < QG; ++qi)
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[qi][e] = 0.f;
#pragma unroll 1
    for (int sub = 0; sub < kChunk / kSub; ++sub) {
      const int pw = c0 + sub * kSub + wave * 64;  // the wave's first position
      if (pw > lim0 + nr - 1) break;               // wave-uniform: nothing visible from here on
      const int j = pw + lane;
      uint32_t kw[D / 2];
      load_row<D>(kbase + (int64_t)min(j, a.S - 1) * D, kw);
      // scores of position j: all query chains advance together; the query
      // words come from LDS (broadcast reads), four at a time, and the
      // compiler barrier keeps them from being hoisted out of the loop
      float s[QG];
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) s[qi] = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < D / 8; ++i4) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int qi = 0; qi < QG; ++qi) {
          const u32x4 q4 = *(const u32x4*)&s_q[qi][4 * i4];
          s[qi] = dot2(kw[4 * i4], q4.x, s[qi]);
          s[qi] = dot2(kw[4 * i4 + 1], q4.y, s[qi]);
          s[qi] = dot2(kw[4 * i4 + 2], q4.z, s[qi]);
          s[qi] = dot2(kw[4 * i4 + 3], q4.w, s[qi]);
        }
      }
      // online softmax over the wave's 64 positions: the masked scores go to
      // LDS ([position][query]); lane qi then runs query qi over the 64
      // positions in order (its maximum, the exponentials written back as
      // probabilities, their sum) and publishes the rescale factor of the
      // running sums. Slots of rows past the pass and masked positions get
      // probability 0.
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) {
        const int r = qi / G;
        s_p[wave][lane][qi] = (r < nr && j <= lim0 + r) ? s[qi] * a.scale : -INFINITY;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane < QG) {
        float mw = -INFINITY;
        for (int jj = 0; jj < 64; ++jj) mw = fmaxf(mw, s_p[wave][jj][lane]);
        const float mn = fmaxf(m_lane, mw);
        float sc = 1.f, sum = 0.f;
        if (mn != -INFINITY) {
          sc = m_lane == -INFINITY ? 0.f : expf(m_lane - mn);
          for (int jj = 0; jj < 64; ++jj) {
            const float v = s_p[wave][jj][lane];
            const float pj = v == -INFINITY ? 0.f : expf(v - mn);
            s_p[wave][jj][lane] = pj;
            sum += pj;
          }
        } else {
          for (int jj = 0; jj < 64; ++jj) s_p[wave][jj][lane] = 0.f;
        }
        l_lane = l_lane * sc + sum;
        m_lane = mn;
        s_sc[wave][lane] = sc;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) {
        const float sc = s_sc[wave][qi];
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[qi][e] *= sc;
      }
      // weighted values: this lane's DL elements over the wave's 64 positions,
      // in batches of kVB whose loads are all issued before the batch is
      // used. Positions past the last one a row of the pass sees have p = 0
      // and read the last seen row instead (the cache need not hold finite
      // values beyond the rows' positions).
      const int jlast = min(63, lim0 + nr - 1 - pw);  // >= 0 here
      constexpr int kVB = 8;
#pragma unroll 1
      for (int jb = 0; jb <= jlast; jb += kVB) {
        float vv[kVB][DL];
#pragma unroll
        for (int jj = 0; jj < kVB; ++jj) {
          const int pj = pw + min(jb + jj, jlast);
          const uint16_t* vr = vbase + (int64_t)pj * D + lane * DL;
          if constexpr (DL == 4) {
            const u32x2 x = gload<u32x2>((const uint8_t*)vr);
            vv[jj][0] = bf16_lo_to_f32(x.x);
            vv[jj][1] = bf16_hi_to_f32(x.x);
            vv[jj][2] = bf16_lo_to_f32(x.y);
            vv[jj][3] = bf16_hi_to_f32(x.y);
          } else if constexpr (DL == 2) {
            const uint32_t x = gload<uint32_t>((const uint8_t*)vr);
            vv[jj][0] = bf16_lo_to_f32(x);
            vv[jj][1] = bf16_hi_to_f32(x);
          } else {
            vv[jj][0] = __uint_as_float((uint32_t)gload<uint16_t>((const uint8_t*)vr) << 16);
          }
        }
#pragma unroll
        for (int jj = 0; jj < kVB; ++jj) {
          asm volatile("" ::: "memory");  // one position's probabilities live at a time
          float pq[QG];
#pragma unroll
          for (int qi = 0; qi < QG; ++qi) pq[qi] = s_p[wave][jb + jj][qi];
#pragma unroll
          for (int qi = 0; qi < QG; ++qi)
#pragma unroll
            for (int e = 0; e < DL; ++e) acc[qi][e] = fmaf(pq[qi], vv[jj][e], acc[qi][e]);
        }
      }
    }
    // combine the four waves in order 0..3
    if (lane < QG) {
      s_ml[wave][lane][0] = m_lane;
      s_ml[wave][lane][1] = l_lane;
    }
    __syncthreads();
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      if (qi / G >= nr) continue;
      float M = -INFINITY;
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_ml[w][qi][0]);
      const float mine = s_ml[wave][qi][0];
      const float sc = mine == -INFINITY ? 0.f : expf(mine - M);
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[qi][e] *= sc;
      if (wave > 0) {
#pragma unroll
        for (int e = 0; e < DL; ++e) s_acc[wave - 1][qi][lane * DL + e] = acc[qi][e];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) {
        const int r = qi / G;
        if (r >= nr || c0 > lim0 + r) continue;  // past the pass, or the row sees none of this chunk
        float M = -INFINITY;
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_ml[w][qi][0]);
        float L = 0.f;
        for (int w = 0; w < kAttnWaves; ++w) {
          const float mw = s_ml[w][qi][0];
          L += mw == -INFINITY ? 0.f : s_ml[w][qi][1] * expf(mw - M);
        }
        float* dst = a.part + (((int64_t)c * a.T + t0 + r) * a.n_q + kv * G + qi % G) * pstride<D>();
#pragma unroll
        for (int e = 0; e < DL; ++e) {
          float v = acc[qi][e];
          for (int w = 1; w < kAttnWaves; ++w) v += s_acc[w - 1][qi][lane * DL + e];
          dst[4 + lane * DL + e] = v;
        }
        if (lane == 0) {
          dst[0] = M;
          dst[1] = L;
        }
      }
    }
  }
}

template <int D>
__global__ void __launch_bounds__(64) attn_combine_kernel(AttnArgs a) {
  constexpr int DL = D / 64;
  const int lane = threadIdx.x;
  const int t = blockIdx.x / a.n_q, h = blockIdx.x % a.n_q;
  const int nc = (a.p0 + t) / kChunk + 1;
  const float* base = a.part + ((int64_t)t * a.n_q + h) * pstride<D>();
  const int64_t cs = (int64_t)a.T * a.n_q * pstride<D>();  // chunk stride
  // the maximum over the chunks: lanes take chunks lane, lane + 64, ...
  float M = -INFINITY;
  for (int c = lane; c < nc; c += 64) M = fmaxf(M, base[c * cs]);
  M = wave_max(M);
  // the weighted sums, chunk by chunk in ascending order (8 chunks' loads in flight)
  float L = 0.f, o[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) o[e] = 0.f;
  int c = 0;
  for (; c + 8 <= nc; c += 8) {
    float mc[8], lc[8], xc[8][DL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* pc = base + (c + u) * cs;
      mc[u] = pc[0];
      lc[u] = pc[1];
#pragma unroll
      for (int e = 0; e < DL; ++e) xc[u][e] = pc[4 + lane * DL + e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = expf(mc[u] - M);
      L = fmaf(lc[u], f, L);
#pragma unroll
      for (int e = 0; e < DL; ++e) o[e] = fmaf(xc[u][e], f, o[e]);
    }
  }
  for (; c < nc; ++c) {
    const float* pc = base + c * cs;
    const float f = expf(pc[0] - M);
    L = fmaf(pc[1], f, L);
#pragma unroll
    for (int e = 0; e < DL; ++e) o[e] = fmaf(pc[4 + lane * DL + e], f, o[e]);
  }
  float* dst = a.o + ((int64_t)t * a.n_q + h) * D + lane * DL;
#pragma unroll
  for (int e = 0; e < DL; ++e) dst[e] = o[e] / L;
}

int64_t attn_ws_bytes(int n_q, int D, int T, int max_seq) {
  const int64_t n_chunks = (max_seq + kChunk - 1) / kChunk;
  return align_up(n_chunks * T * n_q * (int64_t)(D + 4) * 4, kAlign);
}

int qg_of_dim(int d) { return d == 256 ? qg_of<256>() : d == 128 ? qg_of<128>() : qg_of<64>(); }

int32_t check_attn(const moe_attn_shape_t* s, int32_t T) {
  if (!s) return set_error(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (!(s->head_dim == 64 || s->head_dim == 128 || s->head_dim == 256))
    return set_error(MOE_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", s->head_dim);
  const int qg = qg_of_dim(s->head_dim);
  const int g = s->n_kv >= 1 ? s->n_q / s->n_kv : 0;
  if (s->n_kv < 1 || s->n_q < 1 || s->n_q % s->n_kv || g > qg || (g & (g - 1)) || s->n_q > 128)
    return set_error(MOE_ERR_UNSUPPORTED,
                     "n_q %d / n_kv %d: need n_q = g * n_kv with g a power of two <= %d, n_q <= 128", s->n_q,
                     s->n_kv, qg);
  if (s->max_seq < 1 || s->max_seq > (1 << 24)) return set_error(MOE_ERR_INVALID_ARG, "max_seq %d", s->max_seq);
  if (T < 1 || T > 8) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, 8]", T);
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int64_t moe_gqa_workspace_bytes(const moe_attn_shape_t* shape, int32_t T) {
  clear_error();
  int32_t rc = check_attn(shape, T);
  if (rc) return rc;
  return attn_ws_bytes(shape->n_q, shape->head_dim, T, shape->max_seq);
}

extern "C" int32_t moe_gqa_decode(const moe_attn_shape_t* shape, int32_t T, int32_t p0, const uint16_t* q_dev,
                                  const uint16_t* k_dev, const uint16_t* v_dev, float* o_dev, void* ws_dev,
                                  size_t ws_bytes, moe_stream_t stream) {
  clear_error();
  int32_t rc = check_attn(shape, T);
  if (rc) return rc;
  const moe_attn_shape_t& s = *shape;
  if (p0 < 0 || (int64_t)p0 + T > s.max_seq)
    return set_error(MOE_ERR_INVALID_ARG, "positions %d..%d beyond max_seq %d", p0, p0 + T - 1, s.max_seq);
  if (!q_dev || !k_dev || !v_dev || !o_dev || !ws_dev) return set_error(MOE_ERR_INVALID_ARG, "NULL buffer");
  if ((uintptr_t)q_dev % 16 || (uintptr_t)k_dev % 16 || (uintptr_t)v_dev % 16 || (uintptr_t)o_dev % 16)
    return set_error(MOE_ERR_ALIGNMENT, "q, k, v and o must be 16-byte aligned");
  if ((uintptr_t)ws_dev % kAlign) return set_error(MOE_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  const int64_t need = attn_ws_bytes(s.n_q, s.head_dim, T, s.max_seq);
  if ((int64_t)ws_bytes < need)
    return set_error(MOE_ERR_WORKSPACE, "workspace %zu bytes < %lld needed", ws_bytes, (long long)need);
  AttnArgs a;
  a.n_q = s.n_q;
  a.n_kv = s.n_kv;
  a.g = s.n_q / s.n_kv;
  a.S = s.max_seq;
  a.T = T;
  a.p0 = p0;
  a.n_chunks = (p0 + T - 1) / kChunk + 1;
  a.rg = qg_of_dim(s.head_dim) / a.g;  // (rows per pass; the kernels take it from their G)
  a.scale = (float)(1.0 / std::sqrt((double)s.head_dim));
  a.q = q_dev;
  a.k = k_dev;
  a.v = v_dev;
  a.o = o_dev;
  a.part = (float*)ws_dev;
  hipStream_t st = (hipStream_t)stream;
  const dim3 g1(a.n_chunks, a.n_kv);
#define MOE_ATTN_G(DD, GG)                                               \
  case GG: attn_partial_kernel<DD, GG><<<g1, kAttnThreads, 0, st>>>(a); break;
#define MOE_ATTN_D(DD)                                                   \
  switch (a.g) {                                                         \
    MOE_ATTN_G(DD, 1) MOE_ATTN_G(DD, 2) MOE_ATTN_G(DD, 4) MOE_ATTN_G(DD, 8) \
    default: attn_partial_kernel<DD, (qg_of<DD>() >= 16 ? 16 : 8)><<<g1, kAttnThreads, 0, st>>>(a); break; \
  }                                                                      \
  attn_combine_kernel<DD><<<T * a.n_q, 64, 0, st>>>(a);
  switch (s.head_dim) {
    case 64: MOE_ATTN_D(64) break;
    case 128: MOE_ATTN_D(128) break;
    default: MOE_ATTN_D(256) break;
  }
#undef MOE_ATTN_D
#undef MOE_ATTN_G
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return debug_finish(stream);
}
