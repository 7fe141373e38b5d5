// MoE decode kernels for gfx950 and the moe_decode_layer / moe_decode_stack
// entry points.
//
// One layer is four stream-ordered kernels; each boundary is one of the
// layer's all-to-all dependencies:
//   route_kernel  router dot products W_r h_t for every token row t and
//                 expert, and, independent of routing, the shared expert's
//                 SwiGLU activations (min(T, 4) waves per workgroup share the
//                 token rows); workgroup 0 also writes the RMS factor
//                 r_t = 1/sqrt(mean(h_t^2) + eps) and the shared expert's gate
//                 sigmoid(r_t gvec . h_t). For T > 8 with an 8-bit router and
//                 shared expert, mfma_pack_kernel (mfma.h) writes r_t, the
//                 gate and a packed copy of h, route_mfma_kernel does the rest
//                 on the matrix cores and down_mfma_kernel the shared down
//                 projection.
//   select_kernel one workgroup: top-k of r_t W_r h_t for every row (ties to
//                 the lower id, softmax renormalised over the k) and the
//                 ascending list of experts used by any row, with row masks.
//   expert_kernel SwiGLU activations silu(r W_g h) * (r W_u h) of the selected
//                 experts: at T = 1 by expert (each expert's rows read once for
//                 all rows using it); from T = 2 expert_rows_kernel goes one
//                 token row at a time per wave (the row's input arranged once).
//   down_kernel   each workgroup owns a slice of output rows; one wave per
//                 expert (routed and shared) computes W_d a for the rows that
//                 use it; the slice is then combined in rank order:
//                 h + sum_i w_i y_i + gate * y_shared, rounded to bf16
//                 (nearest even). down_kernel_wide: 16-row slices for T >= 16.
// RMSNorm has weight 1, so W (r h) = r (W h): h is used as stored (bf16) and
// r multiplies each dot product. The activations a are kept as two bf16 parts
// a = hi + lo (16 significant bits) so the down projections also run on
// v_dot2c_f32_bf16.
//
// Sources: PureDrive-35B-A3B-MLX model card, "Summary" (top-8 routed + shared
// expert) and "How it works" (several token rows verified in one pass reading
// the weights once; rows bit-identical to a one-row pass); flash-moe news page
// (ja.news.hada.io topic 27758), "Metal Compute Shaders" (SwiGLU, RMS
// normalisation, combine + residual + gate) and "Deferred GPU Expert Compute"
// (combine and residual on the GPU, handed to the next layer directly).
//
// Determinism and row-exactness: no atomics touch data (the select kernel's
// LDS bit-OR of row masks does not depend on order), every reduction has a
// fixed order, and on the vector-unit path the arithmetic of one (token row,
// output) pair is the same whatever T is and whichever rows share an expert.
#include <cmath>
#include <cstdlib>

#include "gemv.h"

namespace moe {
namespace {

constexpr int kMaxUnits = kMaxT * kMaxTopK;

struct Dims {
  int H, E, I, Is, k, T, imax;
  int rbits, ebits, sbits;
  float eps;
  int64_t off_router, off_gatevec, off_shared, off_shared_up, off_shared_down;
  int64_t off_e0, e_stride, off_e_up, off_e_down;
};

struct Ptrs {
  const uint8_t* layer;
  const uint16_t* h_in;
  uint16_t* h_out;
  int32_t* ids_out;
  float* w_out;
  float* raw;
  float* rinv;
  float* sg;
  int* ids;
  float* wts;
  int* units;
  uint32_t* masks;
  uint32_t* tmask;  // [T][k] rows of the call using the expert selected at (row, slot)
  uint16_t* a_hi;
  uint16_t* a_lo;
  float* ysh;  // shared expert's down projection [T][H] from the matrix-core path, or nullptr
  uint16_t* hp;  // matrix-core path: packed h (mfma.h)
  uint16_t* ap;  // matrix-core path: packed shared activations, hi then lo
  // the layer block is table[li] (descriptor table in device memory) when
  // table is set, else `layer`
  const uint8_t* const* table;
  int li;
};

// up to 64 layer pointers passed by value to the table writer
struct LayerBatch {
  static constexpr int kN = 64;
  const uint8_t* p[kN];
};

__device__ __forceinline__ Ptrs with_layer(Ptrs p) {
  if (p.table) p.layer = p.table[p.li];
  return p;
}

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + expf(-g)) * v; }

__device__ __forceinline__ float rms_factor(float sumsq, int H, float eps) { return 1.0f / sqrtf(sumsq / (float)H + eps); }

__device__ __forceinline__ void store_a(const Dims& d, const Ptrs& p, int t, int slot, int i, float a) {
  const uint32_t hb = __float_as_uint(a) & 0xFFFF0000u;
  const int64_t idx = ((int64_t)t * (d.k + 1) + slot) * d.imax + i;
  p.a_hi[idx] = (uint16_t)(hb >> 16);
  p.a_lo[idx] = (uint16_t)f32_to_bf16_rne(a - __uint_as_float(hb));
}

// Down-projection inputs: hi and lo halves of the activation vector [K] as
// arranged words, with the same words and sums as the stack kernel builds.
template <int BITS, int CPL>
__device__ __forceinline__ void prep_split(XLane<BITS, CPL>& xh, XLane<BITS, CPL>& xl, const uint16_t* hi,
                                           const uint16_t* lo, int K, int li, int lpr) {
  const int nch = K >> 5;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    // every lane loads (lanes past the row read its last chunk, then zero it,
    // which is needed only when the row ends inside this pass)
    const bool ok = c < nch;
    const int cc = ok ? c : nch - 1;
    uint32_t nh[16], nl[16];
    load64B(hi + 32 * cc, nh);
    load64B(lo + 32 * cc, nl);
    if (lpr * (m + 1) > nch) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        nh[i] = ok ? nh[i] : 0u;
        nl[i] = ok ? nl[i] : 0u;
      }
    }
    // the halves arranged separately: the same words as splitting the
    // stack kernel's (hi | lo << 16) words after arranging them
    arrange_chunk<BITS>(nh, c, xh.w[m]);
    arrange_chunk<BITS>(nl, c, xl.w[m]);
    xh.s[m] = sum_words<XWords<BITS>::N>(xh.w[m]);
    xl.s[m] = sum_words<XWords<BITS>::N>(xl.w[m]);
  }
}

// rows per lane group of one wave task, by chunks per lane
template <int CPL>
struct TaskRows {
  static constexpr int R = CPL >= 2 ? 2 : 4;  // rows loaded per lane group
};
// row pairs per lane group of one routed-expert task: two with one chunk per
// lane, so that a token row's arranged input serves several pairs and a wave
// has more weight bytes in flight per task; one from two chunks per lane on,
// where the registers of a second pair would cost a wave per SIMD
template <int CPL>
struct ExpertPairs {
  static constexpr int RP = CPL >= 2 ? 1 : 2;
};

// RMS factor and shared-expert gate of token row t (written once per call),
// from the lane's arranged x chunks: ss = sum of squares, gate = gvec . h with
// gvec arranged the same way (the stack kernel uses the same order).
template <int BITS, int CPL>
__device__ __forceinline__ void row_stats(const Dims& d, const Ptrs& p, int t, int li, int lpr, int sr,
                                          const XLane<BITS, CPL>& x) {
  const uint16_t* gv = (const uint16_t*)(p.layer + d.off_gatevec);
  const int nch = d.H >> 5;
  float gd = 0.f;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    uint32_t n[16];
    if (c < nch) {
      load64B(gv + 32 * c, n);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) n[i] = 0u;
    }
    uint32_t g[XWords<BITS>::N];
    arrange_chunk<BITS>(n, c, g);
#pragma unroll
    for (int i = 0; i < XWords<BITS>::N; ++i) gd = dot2(x.w[m][i], g[i], gd);
  }
  const float ss = reduce_row(sumsq(x), lpr);
  gd = reduce_row(gd, lpr);
  if (sr == 0 && li == lpr - 1) {
    const float r = rms_factor(ss, d.H, d.eps);
    p.rinv[t] = r;
    p.sg[t] = 1.0f / (1.0f + expf(-(r * gd)));
  }
}

}  // namespace
}  // namespace moe

#include "mfma.h"

namespace moe {
namespace {

// ----------------------------------------------------------- route kernel
// token rows t0, t0 + ts, ... of the call
template <int BITS, int CPL>
__device__ __forceinline__ void router_task(const Dims& d, const Ptrs& p, int task, int li, int lpr, int sr, int rpw,
                                            int t0, int ts) {
  constexpr int R = TaskRows<CPL>::R;
  int rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = task * R * rpw + sr + rpw * r;
    rows[r] = e < d.E ? e : -1;
  }
  float out[R];
  if constexpr (BITS == kDense) {
    XLane<kDense, CPL> x;
    const uint16_t* w = (const uint16_t*)(p.layer + d.off_router);
    const uint16_t* rp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rp[r] = rows[r] >= 0 ? w + (int64_t)rows[r] * d.H : nullptr;
    RowsD<CPL, R> Q;
    load_dense_rows<CPL, R>(Q, rp, d.H, li, lpr);
    for (int t = t0; t < d.T; t += ts) {
      prep_x<kDense, CPL>(x, p.h_in + (int64_t)t * d.H, d.H, li, lpr);
      if (task == 0) row_stats<kDense, CPL>(d, p, t, li, lpr, sr, x);
      dot_dense_rows<CPL, R>(Q, x, out);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = reduce_row(out[r], lpr);
        if (rows[r] >= 0 && li == lpr - 1) p.raw[(int64_t)t * d.E + rows[r]] = v;
      }
    }
  } else {
    const uint8_t* base = p.layer + d.off_router;
    const int64_t rb = row_bytes(BITS, d.H);
    const uint32_t* sb = (const uint32_t*)(base + matrix_codes_bytes(BITS, d.E, d.H));
    const uint8_t* rc[R];
    const uint32_t* rs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rc[r] = rows[r] >= 0 ? base + (int64_t)rows[r] * rb : nullptr;
      rs[r] = rows[r] >= 0 ? sb + (int64_t)rows[r] * (d.H >> 6) : nullptr;
    }
    RowsQ<BITS, CPL, R> Q;
    load_rows<BITS, CPL, R>(Q, rc, rs, d.H, (int)(rb >> 2), li, lpr);
    XLane<BITS, CPL> x;
    for (int t = t0; t < d.T; t += ts) {
      prep_x<BITS, CPL>(x, p.h_in + (int64_t)t * d.H, d.H, li, lpr);
      if (task == 0) row_stats<BITS, CPL>(d, p, t, li, lpr, sr, x);
      dot_rows<BITS, CPL, R, 1>(Q, x, x, out);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = reduce_row(out[r], lpr);
        if (rows[r] >= 0 && li == lpr - 1) p.raw[(int64_t)t * d.E + rows[r]] = v;
      }
    }
  }
}

// SwiGLU rows of one expert block (gate rows [0, I), up rows at +off_up):
// task covers pairs i = i0 + sr + rpw * r. rowmask: token rows using it.
template <int BITS, int CPL, int RP>
__device__ __forceinline__ void swiglu_task(const Dims& d, const Ptrs& p, const uint8_t* blk, int64_t off_up, int I, int i0,
                            uint32_t rowmask, int slot_fixed, int e, const int* s_ids, const float* rinv, int li,
                            int lpr, int sr, int rpw) {
  constexpr int R = 2 * RP;
  const int64_t rb = row_bytes(BITS, d.H);
  const int64_t cb = matrix_codes_bytes(BITS, I, d.H);
  const uint8_t* gate = blk;
  const uint8_t* up = blk + off_up;
  const uint32_t* gsb = (const uint32_t*)(gate + cb);
  const uint32_t* usb = (const uint32_t*)(up + cb);
  int pairs[RP];
  const uint8_t* rc[R];
  const uint32_t* rs[R];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int i = i0 + sr + rpw * r;
    pairs[r] = i < I ? i : -1;
    rc[r] = i < I ? gate + (int64_t)i * rb : nullptr;
    rs[r] = i < I ? gsb + (int64_t)i * (d.H >> 6) : nullptr;
    rc[RP + r] = i < I ? up + (int64_t)i * rb : nullptr;
    rs[RP + r] = i < I ? usb + (int64_t)i * (d.H >> 6) : nullptr;
  }
  RowsQ<BITS, CPL, R> Q;
  load_rows<BITS, CPL, R>(Q, rc, rs, d.H, (int)(rb >> 2), li, lpr);
  XLane<BITS, CPL> x;
  float out[R];
  for (int t = 0; t < d.T; ++t) {
    if (!(rowmask >> t & 1u)) continue;
    int slot = slot_fixed;
    if (slot < 0)
      for (int i = 0; i < d.k; ++i)
        if (s_ids[t * kMaxTopK + i] == e) slot = i;
    prep_x<BITS, CPL>(x, p.h_in + (int64_t)t * d.H, d.H, li, lpr);
    dot_rows<BITS, CPL, R, 1>(Q, x, x, out);
    // RMS factor: from the workspace, or from the same x chunks (lanes of a
    // row group cover the whole row)
    const float r = rinv ? rinv[t] : rms_factor(reduce_row(sumsq(x), lpr), d.H, d.eps);
#pragma unroll
    for (int q = 0; q < RP; ++q) {
      const float g = reduce_row(out[q], lpr) * r;
      const float v = reduce_row(out[RP + q], lpr) * r;
      if (pairs[q] >= 0 && li == lpr - 1) store_a(d, p, t, slot, pairs[q], silu_mul(g, v));
    }
  }
}

#define MOE_BITS_CASES(bits, B, ...)                   \
  switch (bits) {                                      \
    case 2: { constexpr int B = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int B = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int B = 4; __VA_ARGS__; } break; \
    case 6: { constexpr int B = 6; __VA_ARGS__; } break; \
    default: { constexpr int B = 8; __VA_ARGS__; } break; \
  }

// grid: n_router_tasks + n_shared_tasks workgroups of min(T, 4) waves; each
// wave loads the task's weight rows and takes token rows wave, wave + nw, ...
// (a row's arithmetic does not depend on which wave computes it)
template <int CPL>
__global__ void __launch_bounds__(256) route_kernel(Dims d, Ptrs p_, int n_rt) {
  const Ptrs p = with_layer(p_);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6, task = blockIdx.x;
  const int lpr = lanes_per_row(d.H), rpw = 64 / lpr, sr = lane / lpr, li = lane % lpr;
  if (task < n_rt) {
    if (d.rbits == kDense) {
      router_task<kDense, CPL>(d, p, task, li, lpr, sr, rpw, wave, nw);
    } else {
      MOE_BITS_CASES(d.rbits, B, router_task<B, CPL>(d, p, task, li, lpr, sr, rpw, wave, nw));
    }
  } else {
    constexpr int RP = TaskRows<CPL>::R / 2;
    const int i0 = (task - n_rt) * RP * rpw;
    uint32_t rows = 0u;
    for (int t = wave; t < d.T; t += nw) rows |= 1u << t;
    MOE_BITS_CASES(d.sbits, B,
                   swiglu_task<B, CPL, RP>(d, p, p.layer + d.off_shared, d.off_shared_up, d.Is, i0, rows, d.k, -1,
                                           nullptr, nullptr, li, lpr, sr, rpw));
  }
}

// Routed experts for many token rows, one token row at a time per wave:
// tasks are ordered (row t, slot, block of row pairs), a wave takes a run of
// them, arranges x_t once per row and streams the gate/up rows of the row's
// experts. With SHARE an expert used by several rows is read once: the task
// of the lowest row using it loads the block's rows and computes them for
// every row in the expert's mask (arranging the other rows' inputs as it
// goes), and the other rows' tasks for it do nothing; without it every
// (row, slot) task reads its expert itself, and the kernel carries none of
// that code. The arithmetic of a (row, pair) is the one of swiglu_task
// whichever task computes it, so rows stay exact.
template <int BITS, int CPL, int RP, bool SHARE>
__device__ __forceinline__ void swiglu_rows(const Dims& d, const Ptrs& p, int task0, int task1, int tps, int li,
                                            int lpr, int sr, int rpw) {
  constexpr int R = 2 * RP;
  const int64_t rb = row_bytes(BITS, d.H);
  const int64_t cb = matrix_codes_bytes(BITS, d.I, d.H);
  const int per_row = d.k * tps;
  XLane<BITS, CPL> x;
  int cur_t = -1;
  float r = 0.f;
  for (int task = task0; task < task1; ++task) {
    const int t = task / per_row, rem = task % per_row, slot = rem / tps, i0 = (rem % tps) * RP * rpw;
    if constexpr (CPL >= 4) {  // input first: the other order spills at 4 chunks per lane
      if (t != cur_t) {
        prep_x<BITS, CPL>(x, p.h_in + (int64_t)t * d.H, d.H, li, lpr);
        r = p.rinv[t];
        cur_t = t;
      }
    }
    const int e = p.ids[t * d.k + slot];
    const uint32_t emask = SHARE ? p.tmask[t * d.k + slot] : 1u << t;  // loaded beside the id, not after it
    if (SHARE && (int)__builtin_ctz(emask) != t) continue;  // a lower row's task computes this expert block
    const uint8_t* gate = p.layer + d.off_e0 + (int64_t)e * d.e_stride;
    const uint8_t* up = gate + d.off_e_up;
    const uint32_t* gsb = (const uint32_t*)(gate + cb);
    const uint32_t* usb = (const uint32_t*)(up + cb);
    int pairs[RP];
    const uint8_t* rc[R];
    const uint32_t* rs[R];
#pragma unroll
    for (int q = 0; q < RP; ++q) {
      const int i = i0 + sr + rpw * q;
      pairs[q] = i < d.I ? i : -1;
      rc[q] = i < d.I ? gate + (int64_t)i * rb : nullptr;
      rs[q] = i < d.I ? gsb + (int64_t)i * (d.H >> 6) : nullptr;
      rc[RP + q] = i < d.I ? up + (int64_t)i * rb : nullptr;
      rs[RP + q] = i < d.I ? usb + (int64_t)i * (d.H >> 6) : nullptr;
    }
    RowsQ<BITS, CPL, R> Q;
    load_rows<BITS, CPL, R>(Q, rc, rs, d.H, (int)(rb >> 2), li, lpr);
    // the token row's input after the weight loads are issued: both are in
    // flight together (the input's arrangement waits for its load)
    if (CPL < 4 && t != cur_t) {  // wave-uniform
      prep_x<BITS, CPL>(x, p.h_in + (int64_t)t * d.H, d.H, li, lpr);
      r = p.rinv[t];
      cur_t = t;
    }
    float out[R];
    dot_rows<BITS, CPL, R, 1>(Q, x, x, out);
#pragma unroll
    for (int q = 0; q < RP; ++q) {
      const float g = reduce_row(out[q], lpr) * r;
      const float v = reduce_row(out[RP + q], lpr) * r;
      if (pairs[q] >= 0 && li == lpr - 1) store_a(d, p, t, slot, pairs[q], silu_mul(g, v));
    }
    // the later rows using this expert, from the same loaded rows
    if constexpr (SHARE) for (uint32_t rest = emask & (emask - 1u); rest; rest &= rest - 1u) {
      const int t2 = __builtin_ctz(rest);
      int slot2 = 0;
      for (int i = 0; i < d.k; ++i)
        if (p.ids[t2 * d.k + i] == e) slot2 = i;
      prep_x<BITS, CPL>(x, p.h_in + (int64_t)t2 * d.H, d.H, li, lpr);
      const float r2 = p.rinv[t2];
      cur_t = -1;  // x no longer holds row t (a second register set would cost a wave per SIMD)
      dot_rows<BITS, CPL, R, 1>(Q, x, x, out);
#pragma unroll
      for (int q = 0; q < RP; ++q) {
        const float g = reduce_row(out[q], lpr) * r2;
        const float v = reduce_row(out[RP + q], lpr) * r2;
        if (pairs[q] >= 0 && li == lpr - 1) store_a(d, p, t2, slot2, pairs[q], silu_mul(g, v));
      }
    }
  }
}

// Largest T at which the routed gate/up kernel reads a shared expert once
// for all rows using it. Its task then arranges each further row's input in
// the registers that held its own row's, which the wave's next task (of the
// same row) must arrange again: at T = 8 (35B-A3B shape) the single read
// costs no time, at T = 32 (397B-A17B low-bit shape, 113 distinct experts of
// 128 selections per layer) it took the kernel from 171 to 259 us per layer
// against 12% fewer bytes, so there each row reads its expert itself (the
// down projections still read each distinct expert once). Calls above it
// run a kernel compiled without the sharing code (the code alone, never
// executed, made the T = 32 kernel about 8% slower).
constexpr int kShareMaxT = 8;

// ---------------------------------------------------------- select kernel
// Routing of the call, once: top-k of every token row (row t on wave t % 16),
// the renormalised weights, and the ascending list of experts used by any
// row with the mask of rows using each. One workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) select_kernel(Dims d, Ptrs p) {
  __shared__ uint32_t s_emask[kMaxExperts];
  __shared__ int s_ids[kMaxT * kMaxTopK];
  __shared__ int s_wcnt[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < d.E; e += 1024) s_emask[e] = 0u;
  __syncthreads();
  for (int t = wave; t < d.T; t += 16) {
    int my_id;
    float my_w, r;
    // as many logits per lane as the experts need (lists past E cost work)
    const float* raw = p.raw + (int64_t)t * d.E;
    if (d.E <= 64) wave_topk<1>(raw, p.rinv + t, d.E, d.k, my_id, my_w, r);
    else if (d.E <= 128) wave_topk<2>(raw, p.rinv + t, d.E, d.k, my_id, my_w, r);
    else if (d.E <= 256) wave_topk<4>(raw, p.rinv + t, d.E, d.k, my_id, my_w, r);
    else wave_topk<kMaxExperts / 64>(raw, p.rinv + t, d.E, d.k, my_id, my_w, r);
    if (lane < d.k) {  // lane i holds entry i
      const int i = t * d.k + lane;
      p.ids[i] = my_id;
      p.wts[i] = my_w;
      if (p.ids_out) p.ids_out[i] = my_id;
      if (p.w_out) p.w_out[i] = my_w;
      atomicOr(&s_emask[my_id], 1u << t);  // OR: the result does not depend on the order
      s_ids[i] = my_id;
    }
  }
  __syncthreads();
  // rows sharing the expert of (row, slot): computed by the lowest row's
  // task from one read of the expert's rows, up to kShareMaxT rows; above
  // that every (row, slot) reads its expert itself (see kShareMaxT)
  for (int i = tid; i < d.T * d.k; i += 1024)
    p.tmask[i] = d.T <= kShareMaxT ? s_emask[s_ids[i]] : 1u << (i / d.k);
  // experts used by any row, ascending (E <= 1024: one per thread)
  const bool used = tid < d.E && s_emask[tid] != 0u;
  const unsigned long long bal = __ballot(used);
  if (lane == 0) s_wcnt[wave] = __popcll(bal);
  __syncthreads();
  int off = __popcll(bal & ((1ull << lane) - 1ull));
  int n = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) off += s_wcnt[w];
    n += s_wcnt[w];
  }
  if (used) {
    p.units[1 + off] = tid;
    p.masks[off] = s_emask[tid];
  }
  if (tid == 0) p.units[0] = n;
}

// ---------------------------------------------------------- expert kernel
template <int CPL>
__global__ void __launch_bounds__(256, 2) expert_kernel(Dims d, Ptrs p_, int tasks_per_unit) {
  const Ptrs p = with_layer(p_);
  __shared__ int s_ids[kMaxT * kMaxTopK];
  __shared__ float s_r[kMaxT];
  __shared__ int s_units[kMaxUnits];
  __shared__ uint32_t s_masks[kMaxUnits];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the call's routing (select_kernel), staged once
  const int n_units = p.units[0];
  for (int i = tid; i < d.T * d.k; i += 256) s_ids[(i / d.k) * kMaxTopK + i % d.k] = p.ids[i];
  for (int t = tid; t < d.T; t += 256) s_r[t] = p.rinv[t];
  for (int u = tid; u < n_units; u += 256) {
    s_units[u] = p.units[1 + u];
    s_masks[u] = p.masks[u];
  }
  __syncthreads();
  // SwiGLU tasks: (unit, block of row pairs)
  const int lpr = lanes_per_row(d.H), rpw = 64 / lpr, sr = lane / lpr, li = lane % lpr;
  constexpr int RP = ExpertPairs<CPL>::RP;
  const int n_tasks = n_units * tasks_per_unit;
  for (int task = blockIdx.x * 4 + wave; task < n_tasks; task += gridDim.x * 4) {
    const int u = task / tasks_per_unit;
    const int i0 = (task % tasks_per_unit) * RP * rpw;
    const int e = s_units[u];
    const uint8_t* blk = p.layer + d.off_e0 + (int64_t)e * d.e_stride;
    MOE_BITS_CASES(d.ebits, B,
                   swiglu_task<B, CPL, RP>(d, p, blk, d.off_e_up, d.I, i0, s_masks[u], -1, e, s_ids, s_r, li, lpr, sr,
                                       rpw));
  }
}

// grid: waves of tpw consecutive (row, slot, block) tasks, tps blocks per slot
template <int CPL, bool SHARE>
__global__ void __launch_bounds__(256, 2) expert_rows_kernel(Dims d, Ptrs p_, int tps, int tpw) {
  const Ptrs p = with_layer(p_);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = lanes_per_row(d.H), rpw = 64 / lpr, sr = lane / lpr, li = lane % lpr;
  constexpr int RP = ExpertPairs<CPL>::RP;
  const int n_tasks = d.T * d.k * tps;
  const int task0 = (blockIdx.x * 4 + wave) * tpw;
  const int task1 = task0 + tpw < n_tasks ? task0 + tpw : n_tasks;
  MOE_BITS_CASES(d.ebits, B, swiglu_rows<B, CPL, RP, SHARE>(d, p, task0, task1, tps, li, lpr, sr, rpw));
}

// ------------------------------------------------------------ down kernel
template <int BITS, int CPL, int RD>
__device__ __forceinline__ void down_unit(const Dims& d, const Ptrs& p, const uint8_t* mat, int K, int j0, int J, uint32_t rowmask,
                          int slot_fixed, int e, const int* s_ids, float* s_D) {
  const int lane = threadIdx.x & 63;
  const int lpr = lanes_per_row(K), rpw = 64 / lpr, sr = lane / lpr, li = lane % lpr;
  const int64_t rb = row_bytes(BITS, K);
  const uint32_t* sb = (const uint32_t*)(mat + matrix_codes_bytes(BITS, d.H, K));
  int jj[RD];
  const uint8_t* rc[RD];
  const uint32_t* rs[RD];
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    const int q = sr + rpw * r;
    const bool ok = q < J && j0 + q < d.H;
    jj[r] = ok ? q : -1;
    rc[r] = ok ? mat + (int64_t)(j0 + q) * rb : nullptr;
    rs[r] = ok ? sb + (int64_t)(j0 + q) * (K >> 6) : nullptr;
  }
  RowsQ<BITS, CPL, RD> Q;
  load_rows<BITS, CPL, RD>(Q, rc, rs, K, (int)(rb >> 2), li, lpr);
  XLane<BITS, CPL> xh, xl;
  float out[RD];
  rowmask = __builtin_amdgcn_readfirstlane(rowmask);  // wave-uniform (read from LDS)
  for (int t = 0; t < d.T; ++t) {
    if (!(rowmask >> t & 1u)) continue;
    int slot = slot_fixed;
    if (slot < 0)
      for (int i = 0; i < d.k; ++i)
        if (s_ids[t * d.k + i] == e) slot = i;
    slot = __builtin_amdgcn_readfirstlane(slot);
    const int64_t aoff = ((int64_t)t * (d.k + 1) + slot) * d.imax;
    prep_split<BITS, CPL>(xh, xl, p.a_hi + aoff, p.a_lo + aoff, K, li, lpr);
    dot_rows<BITS, CPL, RD, 2>(Q, xh, xl, out);
#pragma unroll
    for (int r = 0; r < RD; ++r) {
      const float v = reduce_row(out[r], lpr);
      if (jj[r] >= 0 && li == lpr - 1) s_D[(t * (d.k + 1) + slot) * J + jj[r]] = v;
    }
  }
}

template <int CPL, int RD>
__device__ __forceinline__ void down_body(const Dims& d, const Ptrs& p, int J) {
  __shared__ float s_D[kMaxT * (kMaxTopK + 1) * 16];
  __shared__ int s_ids[kMaxT * kMaxTopK];
  __shared__ float s_w[kMaxT * kMaxTopK];
  __shared__ float s_sg[kMaxT];
  __shared__ int s_units[kMaxUnits + 1];
  __shared__ uint32_t s_masks[kMaxUnits];
  const int tid = threadIdx.x, wave = tid >> 6, nw = blockDim.x >> 6;
  const int j0 = blockIdx.x * J;
  // routing of this call, staged once (parallel loads)
  const int n_units = p.units[0];
  for (int i = tid; i < d.T * d.k; i += blockDim.x) {
    s_ids[i] = p.ids[i];
    s_w[i] = p.wts[i];
  }
  for (int i = tid; i < d.T; i += blockDim.x) s_sg[i] = p.sg[i];
  for (int i = tid; i < n_units; i += blockDim.x) {
    s_units[i] = p.units[1 + i];
    s_masks[i] = p.masks[i];
  }
  // residual inputs of this thread's first combine slot, loaded up front
  float h0 = 0.f;
  if (tid < d.T * J && j0 + tid % J < d.H) h0 = __uint_as_float((uint32_t)p.h_in[(int64_t)(tid / J) * d.H + j0 + tid % J] << 16);
  __syncthreads();
  const uint32_t all = d.T >= 32 ? 0xFFFFFFFFu : ((1u << d.T) - 1u);
  for (int u = wave; u <= n_units; u += nw) {
    if (u < n_units) {
      const int e = __builtin_amdgcn_readfirstlane(s_units[u]);
      const uint8_t* mat = p.layer + d.off_e0 + (int64_t)e * d.e_stride + d.off_e_down;
      MOE_BITS_CASES(d.ebits, B, down_unit<B, CPL, RD>(d, p, mat, d.I, j0, J, s_masks[u], -1, e, s_ids, s_D));
    } else if (!p.ysh) {
      const uint8_t* mat = p.layer + d.off_shared + d.off_shared_down;
      MOE_BITS_CASES(d.sbits, B, down_unit<B, CPL, RD>(d, p, mat, d.Is, j0, J, all, d.k, -1, s_ids, s_D));
    }
  }
  if (p.ysh)
    for (int idx = tid; idx < d.T * J; idx += blockDim.x) {
      const int t = idx / J, q = idx % J;
      if (j0 + q < d.H) s_D[(t * (d.k + 1) + d.k) * J + q] = p.ysh[(int64_t)t * d.H + j0 + q];
    }
  __syncthreads();
  for (int idx = tid; idx < d.T * J; idx += blockDim.x) {
    const int t = idx / J, q = idx % J, j = j0 + q;
    if (j >= d.H) continue;
    float acc = 0.f;
    for (int i = 0; i < d.k; ++i) acc = fmaf(s_w[t * d.k + i], s_D[(t * (d.k + 1) + i) * J + q], acc);
    acc = fmaf(s_sg[t], s_D[(t * (d.k + 1) + d.k) * J + q], acc);
    const float hv = idx == tid ? h0 : __uint_as_float((uint32_t)p.h_in[(int64_t)t * d.H + j] << 16);
    const float out = hv + acc;
    p.h_out[(int64_t)t * d.H + j] = (uint16_t)f32_to_bf16_rne(out);
  }
}

// up to 16 waves (one per unit in flight), RD * CPL <= 4
template <int CPL, int RD>
__global__ void __launch_bounds__(1024) down_kernel(Dims d, Ptrs p_, int J) {
  const Ptrs p = with_layer(p_);
  down_body<CPL, RD>(d, p, J);
}
// up to 12 waves (three per SIMD, as its registers allow) with 8 rows per
// lane group (J = 16 at K <= 1024): for many token rows, where each unit's
// activations are read once per workgroup and a wider slice halves those reads
template <int CPL, int RD>
__global__ void __launch_bounds__(768) down_kernel_wide(Dims d, Ptrs p_, int J) {
  const Ptrs p = with_layer(p_);
  down_body<CPL, RD>(d, p, J);
}

// Status word of a stack call that runs layer by layer: no wait can time out.
__global__ void clear_status_kernel(uint32_t* status) { status[threadIdx.x] = 0u; }

// ---------------------------------------------------------------- launch
// from this many token rows the routed experts run row by row (expert_rows_kernel)
constexpr int kRowsMinT = 2;

struct LayerPlan {
  Dims d;
  int cpl_h, cpl_i;
  int n_rt, n_st, tpu, g_grid;
  int rows_tpw, rows_grid;  // expert_rows_kernel (rows_grid > 0: used)
  int J, RD, d_grid, d_threads;
  bool d_wide;
  // matrix-core router and shared expert (T > 8, 8-bit router and shared)
  bool mfma;
  int m_nt, m_ng_route, m_ng_down, m_rt, m_pt, m_down;
};

int mfma_groups_per_load(int groups) {
  const int gpw = (groups + kMfmaWaves - 1) / kMfmaWaves;
  return gpw >= 8 ? 8 : gpw >= 4 ? 4 : 2;
}

// flags: MOE_PATH_NO_MFMA keeps batches on the vector-unit kernels
LayerPlan make_plan(const moe_shape_t& s, const moe_layer_layout_t& L, int T, int flags) {
  LayerPlan P;
  Dims& d = P.d;
  d.H = s.hidden;
  d.E = s.n_experts;
  d.I = s.inter;
  d.Is = s.shared_inter;
  d.k = s.top_k;
  d.T = T;
  d.imax = s.inter > s.shared_inter ? s.inter : s.shared_inter;
  d.rbits = s.router_bits;
  d.ebits = s.expert_bits;
  d.sbits = s.shared_bits;
  d.eps = s.rms_eps;
  d.off_router = L.router;
  d.off_gatevec = L.gatevec;
  d.off_shared = L.shared;
  d.off_shared_up = L.shared_up;
  d.off_shared_down = L.shared_down;
  d.off_e0 = L.expert0;
  d.e_stride = L.expert_stride;
  d.off_e_up = L.expert_up;
  d.off_e_down = L.expert_down;
  P.cpl_h = chunks_per_lane(s.hidden);
  P.cpl_i = chunks_per_lane(d.imax);
  const int rpw_h = 64 / lanes_per_row(s.hidden);
  const int R = P.cpl_h >= 2 ? 2 : 4;
  P.n_rt = (d.E + R * rpw_h - 1) / (R * rpw_h);
  P.n_st = (d.Is + (R / 2) * rpw_h - 1) / ((R / 2) * rpw_h);
  const int rpe = P.cpl_h >= 4 ? ExpertPairs<4>::RP : P.cpl_h == 2 ? ExpertPairs<2>::RP : ExpertPairs<1>::RP;
  P.tpu = (d.I + rpe * rpw_h - 1) / (rpe * rpw_h);
  const int max_units = T * d.k < d.E ? T * d.k : d.E;
  const int waves = max_units * P.tpu;
  P.g_grid = (waves + 3) / 4;
  if (P.g_grid > 2048) P.g_grid = 2048;
  // many token rows: one token row at a time per wave (about 8192 waves)
  P.rows_grid = 0;
  if (T >= kRowsMinT) {
    const int n_tasks = T * d.k * P.tpu;
    P.rows_tpw = (n_tasks + 8191) / 8192;
    P.rows_grid = (n_tasks + 4 * P.rows_tpw - 1) / (4 * P.rows_tpw);
  }
  // down: J output rows per workgroup (about 256 workgroups), RD rows per lane
  // group for the longest K, with RD * chunks <= 4 to bound registers; from
  // 16 token rows on, one chunk per lane, a wide variant with RD = 8 and at
  // most 12 waves (J up to 16)
  const int rpw_min = 64 / lanes_per_row(d.imax);  // rows per pass of the longest K
  P.d_wide = T >= 16 && P.cpl_i == 1;
  const int rd_max = P.d_wide ? 8 : 4 / P.cpl_i;
  int J = pow2ceil((s.hidden + 255) / 256);
  if (J < rpw_min) J = rpw_min;
  if (J > rpw_min * rd_max) J = rpw_min * rd_max;
  if (J > 16) J = 16;
  P.J = J;
  P.RD = (J + rpw_min - 1) / rpw_min;
  if (P.d_wide && P.RD != 8) P.d_wide = false;  // the wide variant is compiled for RD = 8 only
  if (!P.d_wide && P.RD * P.cpl_i > 4) {  // back to the narrow bound
    P.J = J = rpw_min * (4 / P.cpl_i);
    P.RD = 4 / P.cpl_i;
  }
  P.d_grid = (s.hidden + P.J - 1) / P.J;
  int nw = max_units + 1;
  if (nw > (P.d_wide ? 12 : 16)) nw = P.d_wide ? 12 : 16;
  P.d_threads = 64 * nw;
  P.mfma = T >= kMfmaMinT && s.router_bits == 8 && s.shared_bits == 8 && !(flags & MOE_PATH_NO_MFMA);
  P.m_nt = T > 16 ? 2 : 1;
  // groups in flight per wave, bounded by registers (the down projection has
  // two input parts)
  P.m_ng_route = mfma_groups_per_load(s.hidden / kGroup);
  P.m_ng_down = mfma_groups_per_load(s.shared_inter / kGroup);
  if (P.m_ng_down > 4) P.m_ng_down = 4;
  P.m_rt = (s.n_experts + 15) / 16;
  P.m_pt = (s.shared_inter + 7) / 8;
  P.m_down = (s.hidden + 15) / 16;
  return P;
}

template <int CPL>
void launch_route(const LayerPlan& P, const Ptrs& p, hipStream_t st) {
  const int nw = P.d.T < 4 ? P.d.T : 4;
  route_kernel<CPL><<<P.n_rt + P.n_st, 64 * nw, 0, st>>>(P.d, p, P.n_rt);
}
template <int CPL>
void launch_expert(const LayerPlan& P, const Ptrs& p, hipStream_t st) {
  select_kernel<<<1, 1024, 0, st>>>(P.d, p);
  if (P.rows_grid > 0)
    // at four chunks per lane the sharing code spills registers
    if (CPL < 4 && P.d.T <= kShareMaxT)
      expert_rows_kernel<CPL, CPL < 4><<<P.rows_grid, 256, 0, st>>>(P.d, p, P.tpu, P.rows_tpw);
    else
      expert_rows_kernel<CPL, false><<<P.rows_grid, 256, 0, st>>>(P.d, p, P.tpu, P.rows_tpw);
  else
    expert_kernel<CPL><<<P.g_grid, 256, 0, st>>>(P.d, p, P.tpu);
}
template <int NT>
void launch_mfma(const LayerPlan& P, const Ptrs& p, hipStream_t st) {
  mfma_pack_kernel<<<16 * NT, 256, 0, st>>>(P.d, p);
  switch (P.m_ng_route) {
    case 8: route_mfma_kernel<NT, 8><<<P.m_rt + P.m_pt, kMfmaThreads, 0, st>>>(P.d, p, P.m_rt); break;
    case 4: route_mfma_kernel<NT, 4><<<P.m_rt + P.m_pt, kMfmaThreads, 0, st>>>(P.d, p, P.m_rt); break;
    default: route_mfma_kernel<NT, 2><<<P.m_rt + P.m_pt, kMfmaThreads, 0, st>>>(P.d, p, P.m_rt); break;
  }
  switch (P.m_ng_down) {  // at most 4 groups in flight: two input parts
    case 4: down_mfma_kernel<NT, 4><<<P.m_down, kMfmaThreads, 0, st>>>(P.d, p); break;
    default: down_mfma_kernel<NT, 2><<<P.m_down, kMfmaThreads, 0, st>>>(P.d, p); break;
  }
}
template <int CPL, int RD>
void launch_down(const LayerPlan& P, const Ptrs& p, hipStream_t st) {
  down_kernel<CPL, RD><<<P.d_grid, P.d_threads, 0, st>>>(P.d, p, P.J);
}

#define MOE_CPL_CASES(cpl, C, ...)                     \
  switch (cpl) {                                       \
    case 1: { constexpr int C = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int C = 2; __VA_ARGS__; } break; \
    default: { constexpr int C = 4; __VA_ARGS__; } break; \
  }

// The layer block is `layer`, or entry li of the device table when table is set.
int32_t launch_layer(const LayerPlan& P, const WsMap& m, uint8_t* ws, const uint8_t* layer,
                     const uint8_t* const* table, int li, const uint16_t* h_in, uint16_t* h_out, int32_t* ids_out,
                     float* w_out, hipStream_t st) {
  Ptrs p;
  p.layer = layer;
  p.table = table;
  p.li = li;
  p.h_in = h_in;
  p.h_out = h_out;
  p.ids_out = ids_out;
  p.w_out = w_out;
  p.raw = (float*)(ws + m.raw_logits);
  p.rinv = (float*)(ws + m.rinv);
  p.sg = (float*)(ws + m.sgate);
  p.ids = (int*)(ws + m.ids);
  p.wts = (float*)(ws + m.wts);
  p.units = (int*)(ws + m.units);
  p.masks = (uint32_t*)(ws + m.masks);
  p.tmask = (uint32_t*)(ws + m.tmask);
  p.a_hi = (uint16_t*)(ws + m.a_hi);
  p.a_lo = (uint16_t*)(ws + m.a_lo);
  p.ysh = nullptr;
  p.hp = (uint16_t*)(ws + m.hpack);
  p.ap = (uint16_t*)(ws + m.apack);
  if (P.mfma) {
    p.ysh = (float*)(ws + m.ysh);
    if (P.m_nt == 2) launch_mfma<2>(P, p, st);
    else launch_mfma<1>(P, p, st);
  } else {
    MOE_CPL_CASES(P.cpl_h, C, launch_route<C>(P, p, st));
  }
  MOE_CPL_CASES(P.cpl_h, C, launch_expert<C>(P, p, st));
  // rows x chunks per lane <= 4 (make_plan), or the wide variant
  if (P.d_wide) {
    down_kernel_wide<1, 8><<<P.d_grid, P.d_threads, 0, st>>>(P.d, p, P.J);
  } else switch (P.cpl_i * 8 + P.RD) {
    case 8 + 1: launch_down<1, 1>(P, p, st); break;
    case 8 + 2: launch_down<1, 2>(P, p, st); break;
    case 8 + 4: launch_down<1, 4>(P, p, st); break;
    case 16 + 1: launch_down<2, 1>(P, p, st); break;
    case 16 + 2: launch_down<2, 2>(P, p, st); break;
    default: launch_down<4, 1>(P, p, st); break;
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

// After the launches of an entry point: with MOE_DEBUG_SYNC=1, wait for the
// stream and report a HIP error (and, for stack calls, a timed-out wait).
int32_t finish(hipStream_t st, const uint32_t* status_dev) {
  if (!debug_sync()) return MOE_OK;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "MOE_DEBUG_SYNC: %s", hipGetErrorString(e));
  if (status_dev) {
    uint32_t v = 0;
    e = hipMemcpy(&v, status_dev, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "MOE_DEBUG_SYNC status read: %s", hipGetErrorString(e));
    if (v) return set_error(MOE_ERR_TIMEOUT, "a cross-workgroup wait of the stack kernel timed out");
  }
  return MOE_OK;
}

}  // namespace

int32_t debug_finish(moe_stream_t st) { return finish((hipStream_t)st, nullptr); }

namespace {

__global__ void write_table_kernel(const uint8_t** table, LayerBatch b, int n) {
  if ((int)threadIdx.x < n) table[threadIdx.x] = b.p[threadIdx.x];
}

// A stack call: layer blocks from `src`, T rows, workspace map m (of this T).
int32_t run_stack(const moe_shape_t& s, const LayerSrc& src, int n_layers, int T, int flags, const uint16_t* h_in,
                  uint16_t* h_out, int32_t* ids, float* w, uint16_t* h_trace, uint8_t* ws, const WsMap& m,
                  hipStream_t st) {
  moe_layer_layout_t L;
  layout_of(s, &L);
  const LayerPlan P = make_plan(s, L, T, flags);
  const int64_t th = (int64_t)T * s.hidden;
  const int64_t tk = (int64_t)T * s.top_k;
  uint16_t* hb = (uint16_t*)(ws + m.hbuf);
  if (h_trace) {
    hipError_t e = hipMemcpyAsync(h_trace, h_in, th * 2, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  }
  // One-row calls run as one streaming kernel per up to 64 layers when the
  // shape allows it and the device holds its workgroups at once; every other
  // call runs layer by layer (measured on MI355X, the per-layer kernels beat
  // a persistent kernel for T >= 2: one select kernel routes all rows, the
  // routed experts go row by row, the route kernel spreads token rows over
  // waves). Both give the same results bit for bit.
  if (!(flags & MOE_PATH_PER_LAYER)) {
    int32_t rc = launch_stack_t1(s, L, m, ws, src, n_layers, T, h_in, h_out, ids, w, h_trace, st);
    if (rc != MOE_ERR_UNSUPPORTED) return rc ? rc : finish(st, (const uint32_t*)(ws + m.status));
    clear_error();
  }
  clear_status_kernel<<<1, 64, 0, st>>>((uint32_t*)(ws + m.status));
  const uint16_t* cur = h_in;
  for (int l = 0; l < n_layers; ++l) {
    uint16_t* nxt;
    if (h_trace) nxt = h_trace + (l + 1) * th;
    else if (l == n_layers - 1) nxt = h_out;
    else nxt = hb + (l & 1) * th;
    int32_t rc = launch_layer(P, m, ws, (const uint8_t*)src.at(l), src.table, l, cur, nxt, ids ? ids + l * tk : nullptr,
                              w ? w + l * tk : nullptr, st);
    if (rc) return rc;
    cur = nxt;
  }
  if (h_trace) {
    hipError_t e = hipMemcpyAsync(h_out, cur, th * 2, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  }
  return finish(st, (const uint32_t*)(ws + m.status));
}

int32_t check_outputs(const int32_t* ids, const float* w, const uint16_t* h_trace) {
  if (((uintptr_t)ids % 4) || ((uintptr_t)w % 4) || ((uintptr_t)h_trace % 16))
    return set_error(MOE_ERR_ALIGNMENT, "ids/w must be 4-byte and h_trace 16-byte aligned");
  return MOE_OK;
}

int32_t check_layer_list(const void* const* layers, int n_layers) {
  if (!layers || n_layers < 1 || n_layers > kMaxLayers) return set_error(MOE_ERR_INVALID_ARG, "bad layer list");
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l]) return set_error(MOE_ERR_INVALID_ARG, "layer %d pointer is NULL", l);
    if ((uintptr_t)layers[l] % kAlign) return set_error(MOE_ERR_ALIGNMENT, "layer %d not 256-byte aligned", l);
  }
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
  moe_layer_layout_t L;
  layout_of(*shape, &L);
  const LayerPlan P = make_plan(*shape, L, T, MOE_PATH_DEFAULT);
  hipStream_t st = (hipStream_t)stream;
  rc = launch_layer(P, m, (uint8_t*)ws_dev, (const uint8_t*)layer_dev, nullptr, 0, h_in_dev, h_out_dev, ids_dev, w_dev,
                    st);
  return rc ? rc : finish(st, nullptr);
}

int32_t moe::decode_stack_ws(const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers, int32_t T,
                             const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev, float* w_dev,
                             uint16_t* h_trace_dev, void* ws_dev, size_t ws_bytes, moe_stream_t stream) {
  WsMap m;
  int32_t rc = check_call(shape, T, h_in_dev, h_out_dev, ws_dev, ws_bytes, &m);
  if (rc) return rc;
  if ((rc = check_layer_list(layers_host, n_layers))) return rc;
  if ((rc = check_outputs(ids_dev, w_dev, h_trace_dev))) return rc;
  LayerSrc src{layers_host, nullptr};
  return run_stack(*shape, src, n_layers, T, MOE_PATH_DEFAULT, h_in_dev, h_out_dev, ids_dev, w_dev, h_trace_dev,
                   (uint8_t*)ws_dev, m, (hipStream_t)stream);
}

extern "C" int32_t moe_decode_stack(const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers,
                                    int32_t T, const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev,
                                    float* w_dev, uint16_t* h_trace_dev, void* ws_dev, size_t ws_bytes,
                                    moe_stream_t stream) {
  clear_error();
  return decode_stack_ws(shape, layers_host, n_layers, T, h_in_dev, h_out_dev, ids_dev, w_dev, h_trace_dev, ws_dev,
                         ws_bytes, stream);
}

extern "C" int32_t moe_stack_init(moe_stack_t* st, const moe_shape_t* shape, const void* const* layers_host,
                                  int32_t n_layers, int32_t t_max, int32_t flags, void* ws_dev, size_t ws_bytes,
                                  moe_stream_t stream) {
  clear_error();
  if (!st) return set_error(MOE_ERR_INVALID_ARG, "stack state is NULL");
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (t_max < 1 || t_max > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "t_max %d not in [1, %d]", t_max, kMaxT);
  if ((rc = check_layer_list(layers_host, n_layers))) return rc;
  if (flags & ~(MOE_PATH_PER_LAYER | MOE_PATH_NO_MFMA)) return set_error(MOE_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (!ws_dev) return set_error(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)ws_dev % kAlign) return set_error(MOE_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  const int64_t table_off = ws_map(*shape, t_max).total;
  const int64_t need = table_off + table_bytes(n_layers);
  if ((int64_t)ws_bytes < need)
    return set_error(MOE_ERR_WORKSPACE, "workspace %zu bytes < %lld needed", ws_bytes, (long long)need);
  hipStream_t s = (hipStream_t)stream;
  const uint8_t** table = (const uint8_t**)((uint8_t*)ws_dev + table_off);
  for (int l0 = 0; l0 < n_layers; l0 += LayerBatch::kN) {
    LayerBatch b;
    const int n = n_layers - l0 < LayerBatch::kN ? n_layers - l0 : LayerBatch::kN;
    for (int i = 0; i < n; ++i) b.p[i] = (const uint8_t*)layers_host[l0 + i];
    write_table_kernel<<<1, LayerBatch::kN, 0, s>>>(table + l0, b, n);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "descriptor table write failed: %s", hipGetErrorString(e));
  st->shape = *shape;
  st->n_layers = n_layers;
  st->t_max = t_max;
  st->flags = flags;
  st->magic = kStackMagic;
  st->ws_dev = ws_dev;
  st->ws_bytes = ws_bytes;
  st->table_offset = table_off;
  for (int i = 0; i < 4; ++i) st->reserved[i] = 0;
  return finish(s, nullptr);
}

extern "C" int32_t moe_stack_decode(const moe_stack_t* st, int32_t T, const uint16_t* h_in_dev, uint16_t* h_out_dev,
                                    int32_t* ids_dev, float* w_dev, uint16_t* h_trace_dev, moe_stream_t stream) {
  clear_error();
  if (!st || st->magic != kStackMagic) return set_error(MOE_ERR_INVALID_ARG, "stack state not initialised by moe_stack_init");
  if (T < 1 || T > st->t_max) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, t_max %d]", T, st->t_max);
  WsMap m;
  int32_t rc = check_call(&st->shape, T, h_in_dev, h_out_dev, st->ws_dev, st->ws_bytes, &m);
  if (rc) return rc;
  if ((rc = check_outputs(ids_dev, w_dev, h_trace_dev))) return rc;
  LayerSrc src{nullptr, (const uint8_t* const*)((const uint8_t*)st->ws_dev + st->table_offset)};
  return run_stack(st->shape, src, st->n_layers, T, st->flags, h_in_dev, h_out_dev, ids_dev, w_dev, h_trace_dev,
                   (uint8_t*)st->ws_dev, m, (hipStream_t)stream);
}

extern "C" int32_t moe_stack_status(const moe_shape_t* shape, int32_t T, const void* ws_dev, uint32_t* status_host,
                                    moe_stream_t stream) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  if (!ws_dev || !status_host) return set_error(MOE_ERR_INVALID_ARG, "NULL workspace or status");
  const WsMap m = ws_map(*shape, T);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(status_host, (const uint8_t*)ws_dev + m.status, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "status read failed: %s", hipGetErrorString(e));
  return MOE_OK;
}
