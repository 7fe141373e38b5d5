// Grouped-query decode attention over a bf16 K/V cache (gfx950): verify rows
// i = 0..T-1 at positions p0 + i attend causally to the cache, query head h
// to KV head h / g. moe_gqa_decode computes it in two kernels:
//
//   partial kernel       one workgroup per (chunk of positions, KV head)
//                        keeps, per (row, head), the running maximum, the sum
//                        of exponentials and the weighted sum of values
//                        (online softmax) and stores (max, sum, acc[d]) for
//                        the chunk. Head dimension 256 (the card's shape):
//                        attn_mq_kernel, every verify row in one pass, the
//                        scores of all queries on the matrix cores, so the
//                        chunk's K and V are read once for all query heads
//                        and all verify rows. Head dimensions 64 and 128:
//                        attn_partial_kernel, passes of up to kQG queries on
//                        the vector units (a pass per group of verify rows);
//   attn_combine_kernel  per (row, head, 64 outputs): merges the chunks the
//                        row sees in a grouping fixed by their number, and
//                        divides.
//
// Split points are the fixed multiples of the chunk (chunk_of: from the
// cache's capacity and KV heads alone), and every sum runs in an
// order fixed by the position alone, so a row of a T-row call equals a one-row
// call at that position bit for bit (PureDrive-35B-A3B-MLX model card, "How it
// works": K/V read once for all query heads of a KV head and all verify rows,
// split-K with split points and summation order that depend only on the row's
// position). Shapes of the card ("Beyond this checkpoint"): 16 query heads,
// 2 KV heads, head dimension 256; bf16 KV cache ("Hardware"). Scores are the
// bf16 products of q and k accumulated in fp32 (v_dot2c_f32_bf16, or the
// matrix cores at head dimension 256), scaled by 1/sqrt(d); probabilities and
// the output are fp32 (at head dimension 256 the probabilities enter the
// weighted sum of values as two bf16 parts, exact to 2^-18 relative).
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
  int chunk;                                   // positions per workgroup (chunk_of)
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

// V batches: kVB positions of a wave, this lane's DL bf16 values of each,
// kept raw until used.
constexpr int kVB = 8;
template <int DL>
struct VRaw;
template <>
struct VRaw<4> { u32x2 w; };
template <>
struct VRaw<2> { uint32_t w; };
template <>
struct VRaw<1> { uint16_t w; };

template <int D>
__device__ __forceinline__ void load_vb(const uint16_t* vbase, int pw, int jb, int jlast, int lane,
                                        VRaw<D / 64> (&vv)[kVB]) {
  constexpr int DL = D / 64;
#pragma unroll
  for (int jj = 0; jj < kVB; ++jj) {
    const int pj = pw + min(jb + jj, jlast);
    const uint8_t* vr = (const uint8_t*)(vbase + (int64_t)pj * D + lane * DL);
    if constexpr (DL == 4) vv[jj].w = gload<u32x2>(vr);
    else if constexpr (DL == 2) vv[jj].w = gload<uint32_t>(vr);
    else vv[jj].w = gload<uint16_t>(vr);
  }
}

// acc[q][e] += p[position][q] * v[position][e] over one batch, positions in
// order; p is the batch's first row of the wave's probabilities in LDS.
template <int D, int QG>
__device__ __forceinline__ void pv_batch(const float* p, const VRaw<D / 64> (&vv)[kVB],
                                         float (&acc)[QG][D / 64]) {
  constexpr int DL = D / 64;
#pragma unroll
  for (int jj = 0; jj < kVB; ++jj) {
    float x[DL];
    if constexpr (DL == 4) {
      x[0] = bf16_lo_to_f32(vv[jj].w.x);
      x[1] = bf16_hi_to_f32(vv[jj].w.x);
      x[2] = bf16_lo_to_f32(vv[jj].w.y);
      x[3] = bf16_hi_to_f32(vv[jj].w.y);
    } else if constexpr (DL == 2) {
      x[0] = bf16_lo_to_f32(vv[jj].w);
      x[1] = bf16_hi_to_f32(vv[jj].w);
    } else {
      x[0] = __uint_as_float((uint32_t)vv[jj].w << 16);
    }
    asm volatile("" ::: "memory");  // one position's probabilities live at a time
    float pq[QG];
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) pq[qi] = p[jj * (QG + 1) + qi];
#pragma unroll
    for (int qi = 0; qi < QG; ++qi)
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[qi][e] = fmaf(pq[qi], x[e], acc[qi][e]);
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
  __shared__ float s_p[kAttnWaves][64][QG + 1];        // probabilities, by wave, position (lane), query
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
      // masked scores to LDS ([position][query], rows padded by one word)
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) {
        const int r = qi / G;
        s_p[wave][lane][qi] = (r < nr && j <= lim0 + r) ? s[qi] * a.scale : -INFINITY;
      }
      // weighted values: this lane's DL elements over the wave's 64 positions
      // in batches of kVB positions, two batches' loads in flight (the first
      // two are issued here, under the softmax). Positions past the last one
      // a row of the pass sees have p = 0 and read the last seen row instead
      // (the cache need not hold finite values beyond the rows' positions).
      const int jlast = min(63, lim0 + nr - 1 - pw);  // >= 0 here
      VRaw<DL> va[kVB], vb[kVB];
      load_vb<D>(vbase, pw, 0, jlast, lane, va);
      if (kVB <= jlast) load_vb<D>(vbase, pw, kVB, jlast, lane, vb);
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // online softmax: lane (query qi = lane % QG, group gq = lane / QG)
      // takes positions gq*QG .. gq*QG+QG-1 of query qi; maxima and sums are
      // completed by butterflies over the groups (every lane of a query ends
      // with the same values). The probabilities go back to LDS.
      {
        const int qi = lane % QG, gq = lane / QG;
        float v[QG];
        float mw = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < QG; ++jj) {
          v[jj] = s_p[wave][gq * QG + jj][qi];
          mw = fmaxf(mw, v[jj]);
        }
#pragma unroll
        for (int off = QG; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
        const float mn = fmaxf(m_lane, mw);
        float sc = 1.f, sum = 0.f;
        if (mn != -INFINITY) {
          sc = m_lane == -INFINITY ? 0.f : expf(m_lane - mn);
#pragma unroll
          for (int jj = 0; jj < QG; ++jj) {
            const float pj = v[jj] == -INFINITY ? 0.f : expf(v[jj] - mn);
            s_p[wave][gq * QG + jj][qi] = pj;
            sum += pj;
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < QG; ++jj) s_p[wave][gq * QG + jj][qi] = 0.f;
        }
#pragma unroll
        for (int off = QG; off < 64; off <<= 1) sum += __shfl_xor(sum, off);
        l_lane = l_lane * sc + sum;
        m_lane = mn;
        if (gq == 0) s_sc[wave][qi] = sc;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) {
        const float sc = s_sc[wave][qi];
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[qi][e] *= sc;
      }
#pragma unroll 1
      for (int jb = 0; jb <= jlast; jb += 2 * kVB) {
        pv_batch<D, QG>(&s_p[wave][jb][0], va, acc);
        if (jb + 2 * kVB <= jlast) load_vb<D>(vbase, pw, jb + 2 * kVB, jlast, lane, va);
        if (jb + kVB <= jlast) {
          pv_batch<D, QG>(&s_p[wave][jb + kVB][0], vb, acc);
          if (jb + 3 * kVB <= jlast) load_vb<D>(vbase, pw, jb + 3 * kVB, jlast, lane, vb);
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

// ---- head dimension 256: every verify row in one pass over the chunk.
// The scores of all T x G queries of a KV head are one small dense product
// per 16 positions, Q [queries x 256] times K^T [256 x 16 positions], on the
// matrix cores (v_mfma_f32_16x16x32_bf16: exact bf16 products, fp32 sums),
// so K and V are read once for all query heads and all verify rows (the
// card's "How it works"). Per step of 64 positions: wave w computes the
// scores of positions [16w, 16w + 16) of the step for every query tile and
// writes them, scaled and masked, to LDS; wave w then runs the online
// softmax of queries w, w + 4, ... over the 64 positions (wave-wide max and
// sum in a fixed tree) and writes their probabilities, split p = hi + lo into
// two bf16 parts (hi the nearest bf16, lo the nearest to the rest: 2^-18 of
// p at most is lost), as the A operand of a second product, and the rescale
// factors; finally wave w rescales its accumulators and adds
// P_hi V + P_lo V for output dimensions [64w, 64w + 64) on the matrix cores
// (V as the B operand, gathered with 16-bit loads two positions to a
// register; each V element read once). A query's result depends only on its
// own row's data, and each instantiation computes a row the same way: steps
// past a row's position add exactly nothing (p = 0, rescale 1), so a verify
// row equals a one-row call.
typedef __bf16 at_bf16x8 __attribute__((ext_vector_type(8)));
typedef float at_f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t at_u16x2 __attribute__((ext_vector_type(2)));
constexpr int kMqStep = 64;  // positions per step (16 per wave)

__device__ __forceinline__ at_f32x4 mfma_qk(u32x4 a, u32x4 b, at_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(at_bf16x8, a), __builtin_bit_cast(at_bf16x8, b),
                                                 c, 0, 0, 0);
}

// Workgroup barrier for LDS data only: the global loads in flight (the
// next step's keys, this step's values) are not waited for, as
// __syncthreads would.
__device__ __forceinline__ void mq_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int G, int QP>
__global__ void __launch_bounds__(kAttnThreads, 2) attn_mq_kernel(AttnArgs a) {
  constexpr int D = 256;
  constexpr int QPW = QP / kAttnWaves;       // softmax queries per wave
  constexpr int QT = (QP + 15) / 16 * 16;    // query rows of the products (whole 16-row tiles)
  constexpr int NQT = QT / 16;
  __shared__ __attribute__((aligned(16))) uint32_t s_q[QT][D / 2 + 4];  // bf16 pairs; rows padded by 16 bytes
  __shared__ float s_s[QT][kMqStep + 1];                               // scaled, masked scores [query][position]
  // probabilities as the A operand of the weighted-value product: per query
  // tile, half step kb (32 positions) and part (p = hi + lo, two bf16), 64
  // lanes x 8 bf16: lane 16 g + r holds query 16 qt + r, positions
  // 32 kb + 8 g .. + 7
  __shared__ __attribute__((aligned(16))) uint16_t s_pa[NQT][2][2][64 * 8];
  __shared__ __attribute__((aligned(16))) float s_sc[QT];              // this step's rescale factor of each query
  __shared__ float s_m[QT], s_l[QT];                                   // running maximum and sum of each query
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x, kv = blockIdx.y;
  const int c0 = c * a.chunk;
  const int jmax = min(c0 + a.chunk - 1, a.p0 + a.T - 1);  // last position any row sees
  if (c0 > jmax) return;
  const int nq = a.T * G, nqt = (nq + 15) / 16;
  const uint16_t* kbase = a.k + (int64_t)kv * a.S * D;
  const uint16_t* vbase = a.v + (int64_t)kv * a.S * D;
  // the queries of this KV head, row t's heads kv*G .. kv*G+G-1 as queries t*G ..
  for (int i = threadIdx.x; i < QT * (D / 2); i += kAttnThreads) {
    const int q = i / (D / 2), w = i % (D / 2);
    s_q[q][w] = q < nq ? ((const uint32_t*)(a.q + ((int64_t)(q / G) * a.n_q + kv * G + q % G) * D))[w] : 0u;
  }
  // rows of queries past the call's: probability 0 and rescale 1 for good
  for (int i = threadIdx.x; i < NQT * 2 * 2 * 64 * 8; i += kAttnThreads) {
    const int l = (i / 8) % 64;
    const int qt = i / (2 * 2 * 64 * 8);
    if (16 * qt + (l & 15) >= nq) (&s_pa[0][0][0][0])[i] = 0;
  }
  for (int q = threadIdx.x; q < QT; q += kAttnThreads) {
    if (q >= nq) s_sc[q] = 1.f;
    s_m[q] = -INFINITY;
    s_l[q] = 0.f;
  }
  // output accumulators: tile qt, dimension tile dt (dimensions
  // 64 wave + 16 dt ..), lane holds queries 16 qt + 4 (lane / 16) + i of
  // dimension 64 wave + 16 dt + lane % 16
  at_f32x4 o_acc[NQT][4];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o_acc[qt][dt] = at_f32x4{0.f, 0.f, 0.f, 0.f};
  const int tl = lane & 15, kq = 8 * (lane >> 4);
  // key rows of a step (B operand: position base + 16 wave + tl, dimensions
  // kq + 32 ks .. + 7), requested one step ahead
  u32x4 kb[D / 32];
  auto load_k = [&](int base) {
    const int pk = min(base + 16 * wave + tl, jmax);  // a visible row; masked below
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kb[ks] = gload<u32x4>((const uint8_t*)(kbase + (int64_t)pk * D + 32 * ks + kq));
  };
  load_k(c0);
  for (int base = c0; base <= jmax; base += kMqStep) {
    // this step's values as the B operand of the weighted-value product,
    // requested first (they arrive while the scores and the softmax are
    // computed): for dimension tile dt and half step kb, lane l holds
    // dimension 64 wave + 16 dt + l % 16 at positions 32 kb + 8 (l / 16) .. + 7,
    // two positions per register (16-bit loads into the low and high halves)
    const int jl = min(kMqStep - 1, jmax - base);
    at_u16x2 vb[4][2][4];
    auto load_v = [&](int h) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int j = min(32 * h + kq + 2 * e2 + x, jl);
            vb[dt][h][e2][x] = gload<uint16_t>((const uint8_t*)(vbase + (int64_t)(base + j) * D + 64 * wave + 16 * dt + tl));
          }
    };
    // at four query tiles the second half is requested after the scores,
    // so that the registers of both halves are not live across them
    constexpr bool V_SPLIT = NQT >= 4;
    load_v(0);
    if constexpr (!V_SPLIT) load_v(1);
    mq_barrier();  // s_q written (first step); the previous step's LDS reads done
    // (1) scores of positions base + 16 wave + tl for every query tile
    {
      at_f32x4 sc4[NQT];
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {  // every tile: rows past the queries are zeros, masked below
        sc4[qt] = at_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const u32x4 qa = *(const u32x4*)&s_q[16 * qt + tl][16 * ks + (kq >> 1)];
          sc4[qt] = mfma_qk(qa, kb[ks], sc4[qt]);
        }
      }
      if (base + kMqStep <= jmax) load_k(base + kMqStep);  // the next step's keys
      if constexpr (V_SPLIT) load_v(1);
      const int pos = base + 16 * wave + tl;
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = 16 * qt + 4 * (lane >> 4) + r;
          const bool vis = q < nq && pos <= a.p0 + q / G;
          s_s[q][16 * wave + tl] = vis ? sc4[qt][r] * a.scale : -INFINITY;
        }
      }
    }
    mq_barrier();
    // (2) online softmax of queries wave, wave + 4, ... over the step; the
    // probability of position `lane` goes to the A operand as hi + lo
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      const int q = wave + kAttnWaves * j;
      if (q < nq) {
        const float x = s_s[q][lane];
        const float m_old = s_m[q];
        const float mn = fmaxf(m_old, wave_max(x));
        float p = 0.f, sc = 1.f;
        if (mn != -INFINITY) {
          p = x == -INFINITY ? 0.f : expf(x - mn);
          sc = m_old == -INFINITY ? 0.f : expf(m_old - mn);
        }
        const float sum = wave_sum(p);
        const float l_new = s_l[q] * sc + sum;
        const uint32_t hi = f32_to_bf16_rne(p);
        const uint32_t lo = f32_to_bf16_rne(p - __uint_as_float(hi << 16));
        const int at = (16 * ((lane >> 3) & 3) + (q & 15)) * 8 + (lane & 7);
        s_pa[q >> 4][lane >> 5][0][at] = (uint16_t)hi;
        s_pa[q >> 4][lane >> 5][1][at] = (uint16_t)lo;
        if (lane == 0) {
          s_sc[q] = sc;
          s_m[q] = mn;
          s_l[q] = l_new;
        }
      }
    }
    mq_barrier();
    // (3) weighted values on the matrix cores: rescale, then
    // o += P_hi V + P_lo V over the step's 64 positions (positions past jl:
    // p = 0 and a copy of row jl's value)
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const float4 f = *(const float4*)&s_sc[16 * qt + 4 * (lane >> 4)];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        o_acc[qt][dt][0] *= f.x;
        o_acc[qt][dt][1] *= f.y;
        o_acc[qt][dt][2] *= f.z;
        o_acc[qt][dt][3] *= f.w;
      }
    }
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 ph = *(const u32x4*)&s_pa[qt][h][0][8 * lane];
        const u32x4 pl = *(const u32x4*)&s_pa[qt][h][1][8 * lane];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4 vv = __builtin_bit_cast(u32x4, vb[dt][h]);
          o_acc[qt][dt] = mfma_qk(ph, vv, o_acc[qt][dt]);
          o_acc[qt][dt] = mfma_qk(pl, vv, o_acc[qt][dt]);
        }
      }
  }
  // the chunk's partials of the rows that see it
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 16 * qt + 4 * (lane >> 4) + i;
      const int t = q / G;
      if (q < nq && c0 <= a.p0 + t) {
        float* dst = a.part + (((int64_t)c * a.T + t) * a.n_q + kv * G + q % G) * pstride<D>();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dst[4 + 64 * wave + 16 * dt + tl] = o_acc[qt][dt][i];
      }
    }
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int q = wave + kAttnWaves * j;
    if (q < nq && lane == 0 && c0 <= a.p0 + q / G) {
      float* dst = a.part + (((int64_t)c * a.T + q / G) * a.n_q + kv * G + q % G) * pstride<D>();
      dst[0] = s_m[q];  // written by this wave (lane 0)
      dst[1] = s_l[q];
    }
  }
}

// One workgroup per (row, head, 64-element segment of the output). Wave w
// takes the chunks w, w + kCombWaves, ... (kCombUnroll of them per round, all
// loads of a round in flight) with a running maximum of its own; the waves'
// sums are then rescaled to the common maximum and added in wave order. The
// grouping depends only on the number of chunks the row sees, that is on its
// position.
constexpr int kCombWaves = 16;
constexpr int kCombUnroll = 16;

template <int D>
__global__ void __launch_bounds__(64 * kCombWaves) attn_combine_kernel(AttnArgs a) {
  __shared__ float s_m[kCombWaves];
  __shared__ float s_l[kCombWaves];
  __shared__ float s_o[kCombWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x / a.n_q, h = blockIdx.x % a.n_q, e = blockIdx.y * 64 + lane;
  const int nc = (a.p0 + t) / a.chunk + 1;
  const float* base = a.part + ((int64_t)t * a.n_q + h) * pstride<D>();
  const int64_t cs = (int64_t)a.T * a.n_q * pstride<D>();  // chunk stride
  float mw = -INFINITY, L = 0.f, o = 0.f;
  for (int c0 = wave; c0 < nc; c0 += kCombUnroll * kCombWaves) {
    float mc[kCombUnroll], lc[kCombUnroll], xc[kCombUnroll];
#pragma unroll
    for (int u = 0; u < kCombUnroll; ++u) {
      const int cu = c0 + u * kCombWaves;
      const float* pc = base + (int64_t)min(cu, nc - 1) * cs;
      mc[u] = cu < nc ? pc[0] : -INFINITY;
      lc[u] = pc[1];
      xc[u] = pc[4 + e];
    }
    float mn = mw;
#pragma unroll
    for (int u = 0; u < kCombUnroll; ++u) mn = fmaxf(mn, mc[u]);
    const float sc = mw == -INFINITY ? 0.f : expf(mw - mn);
    L *= sc;
    o *= sc;
#pragma unroll
    for (int u = 0; u < kCombUnroll; ++u) {
      if (mc[u] == -INFINITY) continue;
      const float f = expf(mc[u] - mn);
      L = fmaf(lc[u], f, L);
      o = fmaf(xc[u], f, o);
    }
    mw = mn;
  }
  s_o[wave][lane] = o;
  if (lane == 0) {
    s_m[wave] = mw;
    s_l[wave] = L;
  }
  __syncthreads();
  if (wave == 0) {
    float M = s_m[0];
#pragma unroll
    for (int w = 1; w < kCombWaves; ++w) M = fmaxf(M, s_m[w]);
    float ot = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < kCombWaves; ++w) {
      if (s_m[w] == -INFINITY) continue;
      const float f = expf(s_m[w] - M);
      ot = fmaf(s_o[w][lane], f, ot);
      lt = fmaf(s_l[w], f, lt);
    }
    a.o[((int64_t)t * a.n_q + h) * D + e] = ot / lt;
  }
}

// Positions per workgroup. Head dimension 256: the largest of 512, 256, 128
// and 64 that still gives 512 workgroups (two per compute unit) over a full
// cache, else 64, so that short caches are not a few workgroups of many
// dependent steps; it depends on the cache's capacity and KV heads alone, so
// every call on one cache splits at the same points. Head dimensions 64 and
// 128: kChunk (the kernel's two passes of kSub positions).
int chunk_of(int D, int max_seq, int n_kv) {
  if (D != 256) return kChunk;
  for (int c = kChunk; c > kMqStep; c /= 2)
    if ((int64_t)((max_seq + c - 1) / c) * n_kv >= 512) return c;
  return kMqStep;
}

int64_t attn_ws_bytes(int n_q, int n_kv, int D, int T, int max_seq) {
  const int chunk = chunk_of(D, max_seq, n_kv);
  const int64_t n_chunks = (max_seq + chunk - 1) / chunk;
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
  return attn_ws_bytes(shape->n_q, shape->n_kv, shape->head_dim, T, shape->max_seq);
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
  const int64_t need = attn_ws_bytes(s.n_q, s.n_kv, s.head_dim, T, s.max_seq);
  if ((int64_t)ws_bytes < need)
    return set_error(MOE_ERR_WORKSPACE, "workspace %zu bytes < %lld needed", ws_bytes, (long long)need);
  AttnArgs a;
  a.n_q = s.n_q;
  a.n_kv = s.n_kv;
  a.g = s.n_q / s.n_kv;
  a.S = s.max_seq;
  a.T = T;
  a.p0 = p0;
  a.chunk = chunk_of(s.head_dim, s.max_seq, s.n_kv);
  a.n_chunks = (p0 + T - 1) / a.chunk + 1;
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
  attn_combine_kernel<DD><<<dim3(T * a.n_q, DD / 64), 64 * kCombWaves, 0, st>>>(a);
  switch (s.head_dim) {
    case 64: MOE_ATTN_D(64) break;
    case 128: MOE_ATTN_D(128) break;
    default:
      // the same per-query arithmetic in every instantiation: QP only
      // sizes the registers and LDS for the call's T x g queries
// queries per instantiation: the smallest of 8, 16, 24, 32, 64 that holds
// the call's T x g (at most 8 g; a 48-query instantiation measured slower
// than the 64-query one)
#define MOE_ATTN_MQ_QP(GG, QQ) \
  if (T * GG <= QQ) {          \
    attn_mq_kernel<GG, QQ><<<g1, kAttnThreads, 0, st>>>(a); \
    break;                     \
  }
      switch (a.g) {
        case 1: MOE_ATTN_MQ_QP(1, 8) break;
        case 2: MOE_ATTN_MQ_QP(2, 8) MOE_ATTN_MQ_QP(2, 16) break;
        case 4: MOE_ATTN_MQ_QP(4, 8) MOE_ATTN_MQ_QP(4, 16) MOE_ATTN_MQ_QP(4, 24) MOE_ATTN_MQ_QP(4, 32) break;
        default:
          MOE_ATTN_MQ_QP(8, 8) MOE_ATTN_MQ_QP(8, 16) MOE_ATTN_MQ_QP(8, 24) MOE_ATTN_MQ_QP(8, 32)
          MOE_ATTN_MQ_QP(8, 64) break;
      }
#undef MOE_ATTN_MQ_QP
      attn_combine_kernel<256><<<dim3(T * a.n_q, 256 / 64), 64 * kCombWaves, 0, st>>>(a);
      break;
  }
#undef MOE_ATTN_D
#undef MOE_ATTN_G
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return debug_finish(stream);
}
