// Stack decode as one persistent kernel per launch (up to 64 layers):
// device code, included by the persist_*.hip instantiation units.
//
// The three dependencies of a layer (all router logits before the top-k, all
// activations of an expert before its down projection, the whole hidden state
// before the next router) are met without grid barriers or cache maintenance:
// every value that crosses workgroups is written as a 64-bit word
//   payload (32 bits) | epoch << 32,  epoch = layer index in the launch + 1
// with a device-scope relaxed store, and each consumer polls exactly the words
// it needs with device-scope relaxed loads until they carry the expected epoch.
// The data round trip is the synchronisation. A small clear kernel zeroes the
// exchange buffers before each launch, so no stale word can match.
//
// Why one buffer per kind is enough (no double buffering): a producer of layer
// l+1 only runs after it has seen all of h_{l+1}, which exists only after every
// workgroup finished its down phase of layer l, which comes after its last read
// of layer l's logits, activations and row statistics; h_{l+2} is written by a
// down phase of layer l+1, which needs every activation of layer l+1, hence
// every reader of h_{l+1} has finished.
//
// Per layer (workgroup = 8 waves, one workgroup per compute unit):
//   phase A  router rows (raw logits) and shared-expert SwiGLU rows; task 0
//            also publishes the RMS factor and the shared-expert gate
//   phase B  every workgroup computes the top-k and expert list itself, then
//            its waves compute routed SwiGLU rows (tasks spread over the grid)
//   phase C  the workgroup's slice of J output rows: one wave per expert,
//            combine in rank order, residual, bf16; the slice of h stays in
//            LDS as the next layer's residual and is published for the router
// Every wait is bounded; a timed-out wait sets status[0] and every later wait
// returns at once, so a failed launch still drains (results are then invalid
// and moe_stack_status reports it).
#pragma once
#include <cmath>

#include "gemv.h"

namespace moe {

constexpr int kPThreads = 512;
constexpr int kPWaves = kPThreads / 64;
constexpr uint32_t kSpinLimit = 1u << 21;

struct PArgs {
  int H, E, I, Is, k, T, imax;
  int rbits, ebits, sbits;
  float eps;
  int64_t off_router, off_gatevec, off_shared, off_shared_up, off_shared_down;
  int64_t off_e0, e_stride, off_e_up, off_e_down;
  int n_layers, nwg, J, n_rt, n_st, tpu;
  int mE;  // experts per lane in the top-k: E <= 64 mE, mE in {1, 2, 4, 8}
  const uint16_t* h_in;
  uint16_t* h_out;
  int32_t* ids_out;
  float* w_out;
  uint16_t* h_trace;  // [n_layers][T][H] (outputs of this launch's layers) or null
  uint64_t* tg_h;
  uint64_t* tg_logit;
  uint64_t* tg_rs;
  uint64_t* tg_a;
  uint32_t* status;
  const uint8_t* layers[kMaxLayersPerLaunch];
};

__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t v, uint32_t epoch) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_status(const uint32_t* s) {
  return __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the N words p[i * stride] carry `epoch`; payloads to out.
template <int N>
__device__ __forceinline__ void poll_words(const uint64_t* p, int stride, uint32_t epoch, uint32_t (&out)[N],
                                           uint32_t* status) {
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint64_t v = ld_tag(p + (int64_t)i * stride);
      out[i] = (uint32_t)v;
      ok &= (uint32_t)(v >> 32) == epoch;
    }
    if (ok) return;
    ++spins;
    if ((spins & 63) == 0) {
      if (ld_status(status)) return;
      if (spins > kSpinLimit) {
        __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + expf(-g)) * v; }
__device__ __forceinline__ float rms_factor(float ss, int H, float eps) { return 1.0f / sqrtf(ss / (float)H + eps); }

// Exchange layouts, transposed so that the lanes of a row group, which hold
// consecutive chunks of 32 elements, poll consecutive words:
//   h row: bf16 pair p (elements 2p, 2p + 1; chunk p / 16) at word
//          (p % 16) * (H / 32) + p / 16
//   a row: element i (bf16 hi | lo << 16; chunk i / 32) at word
//          (i % 32) * (imax / 32) + i / 32
__device__ __forceinline__ int h_word(int p, int H) { return (p & 15) * (H >> 5) + (p >> 4); }
__device__ __forceinline__ int a_word(int i, int imax) { return (i & 31) * (imax >> 5) + (i >> 5); }

// Natural bf16 words of chunk c of h row t: the launch input for its first
// layer, else the published state of epoch `ep`.
__device__ __forceinline__ void h_chunk(const PArgs& a, bool first, uint32_t ep, int t, int c, uint32_t (&n)[16]) {
  if (c >= (a.H >> 5)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) n[i] = 0u;
  } else if (first) {
    load64B(a.h_in + (int64_t)t * a.H + 32 * c, n);
  } else {
    poll_words<16>(a.tg_h + (int64_t)t * (a.H >> 1) + c, a.H >> 5, ep, n, a.status);
  }
}

template <int BITS, int CPL>
__device__ __forceinline__ void h_lane(const PArgs& a, bool first, uint32_t ep, int t, int li, int lpr,
                                       XLane<BITS, CPL>& x) {
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    uint32_t n[16];
    h_chunk(a, first, ep, t, c, n);
    arrange_chunk<BITS>(n, c, x.w[m]);
    x.s[m] = sum_words<XWords<BITS>::N>(x.w[m]);
  }
}

// Lane coordinates re-defined opaquely at the start of every task, so that
// the compiler does not hoist lane-dependent addressing of each phase and code
// width out of the layer loop (where it would stay live across all phases).
__device__ __forceinline__ void opaque_lane(int& li, int& sr) { asm volatile("" : "+v"(li), "+v"(sr)); }

template <int CPL>
struct PTaskRows {
  static constexpr int R = CPL >= 2 ? 2 : 4;
};

// ------------------------------------------------------------- phase A
// One router row per lane group (rows task * rpw + sr): the router is short
// (E rows), so one row per wave keeps the per-wave instruction chain short.
template <int BITS, int CPL>
__device__ __forceinline__ void router_rows(const PArgs& a, const uint8_t* layer, bool first, uint32_t ep, int task,
                                            int li, int lpr, int sr, int rpw) {
  constexpr int AB = BITS == kDense ? kDense : BITS;
  opaque_lane(li, sr);
  const int e = task * rpw + sr;
  const int row = e < a.E ? e : -1;
  float out[1];
  XLane<AB, CPL> x;
  if constexpr (BITS == kDense) {
    const uint16_t* w = (const uint16_t*)(layer + a.off_router);
    const uint16_t* rp[1] = {row >= 0 ? w + (int64_t)row * a.H : nullptr};
    RowsD<CPL, 1> Q;
    load_dense_rows<CPL, 1>(Q, rp, a.H, li, lpr);
    for (int t = 0; t < a.T; ++t) {
      h_lane<AB, CPL>(a, first, ep - 1, t, li, lpr, x);
      dot_dense_rows<CPL, 1>(Q, x, out);
      const float v = reduce_row(out[0], lpr);
      if (row >= 0 && li == lpr - 1) st_tag(a.tg_logit + (int64_t)t * a.E + row, __float_as_uint(v), ep);
    }
  } else {
    const uint8_t* base = layer + a.off_router;
    const int64_t rb = row_bytes(BITS, a.H);
    const uint32_t* sb = (const uint32_t*)(base + matrix_codes_bytes(BITS, a.E, a.H));
    const uint8_t* rc[1] = {row >= 0 ? base + (int64_t)row * rb : nullptr};
    const uint32_t* rs[1] = {row >= 0 ? sb + (int64_t)row * (a.H >> 6) : nullptr};
    RowsQ<BITS, CPL, 1> Q;
    load_rows<BITS, CPL, 1>(Q, rc, rs, a.H, (int)(rb >> 2), li, lpr);
    for (int t = 0; t < a.T; ++t) {
      h_lane<BITS, CPL>(a, first, ep - 1, t, li, lpr, x);
      dot_rows<BITS, CPL, 1, 1>(Q, x, x, out);
      const float v = reduce_row(out[0], lpr);
      if (row >= 0 && li == lpr - 1) st_tag(a.tg_logit + (int64_t)t * a.E + row, __float_as_uint(v), ep);
    }
  }
}

// RMS factor and shared-expert gate of every token row (one task), from h in
// the router's arrangement AB (the per-layer kernels use the same order):
// ss = sum of squares, gate = sigmoid(r * gvec . h).
template <int AB, int CPL>
__device__ __forceinline__ void stats_rows(const PArgs& a, const uint8_t* layer, bool first, uint32_t ep, int li,
                                           int lpr, int sr) {
  opaque_lane(li, sr);
  XLane<AB, CPL> x, g;
  const uint16_t* gv = (const uint16_t*)(layer + a.off_gatevec);
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    uint32_t n[16];
    if (c < (a.H >> 5)) {
      load64B(gv + 32 * c, n);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) n[i] = 0u;
    }
    arrange_chunk<AB>(n, c, g.w[m]);
  }
  for (int t = 0; t < a.T; ++t) {
    h_lane<AB, CPL>(a, first, ep - 1, t, li, lpr, x);
    float gd = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m)
#pragma unroll
      for (int i = 0; i < XWords<AB>::N; ++i) gd = dot2(x.w[m][i], g.w[m][i], gd);
    const float ss = reduce_row(sumsq(x), lpr);
    gd = reduce_row(gd, lpr);
    if (sr == 0 && li == lpr - 1) {
      const float rr = rms_factor(ss, a.H, a.eps);
      st_tag(a.tg_rs + 2 * t, __float_as_uint(rr), ep);
      st_tag(a.tg_rs + 2 * t + 1, __float_as_uint(1.0f / (1.0f + expf(-(rr * gd)))), ep);
    }
  }
}

// SwiGLU rows of one expert block (pairs i = i0 + sr + rpw r). s_r != null:
// RMS factors of the rows (routed experts); null: from the x chunks (shared).
template <int BITS, int CPL>
__device__ __forceinline__ void swiglu_rows(const PArgs& a, bool first, uint32_t ep, const uint8_t* blk,
                                            int64_t off_up, int I, int i0, uint32_t rowmask, int slot_fixed, int e,
                                            const int* s_ids, const float* s_r, int li, int lpr, int sr, int rpw) {
  constexpr int RP = PTaskRows<CPL>::R / 2;
  opaque_lane(li, sr);
  constexpr int R = 2 * RP;
  const int64_t rb = row_bytes(BITS, a.H);
  const int64_t cb = matrix_codes_bytes(BITS, I, a.H);
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
    rs[r] = i < I ? gsb + (int64_t)i * (a.H >> 6) : nullptr;
    rc[RP + r] = i < I ? up + (int64_t)i * rb : nullptr;
    rs[RP + r] = i < I ? usb + (int64_t)i * (a.H >> 6) : nullptr;
  }
  RowsQ<BITS, CPL, R> Q;
  load_rows<BITS, CPL, R>(Q, rc, rs, a.H, (int)(rb >> 2), li, lpr);
  XLane<BITS, CPL> x;
  float out[R];
  for (int t = 0; t < a.T; ++t) {
    if (!(rowmask >> t & 1u)) continue;
    int slot = slot_fixed;
    if (slot < 0)
      for (int i = 0; i < a.k; ++i)
        if (s_ids[t * kMaxTopK + i] == e) slot = i;
    h_lane<BITS, CPL>(a, first, ep - 1, t, li, lpr, x);
    dot_rows<BITS, CPL, R, 1>(Q, x, x, out);
    const float r = s_r ? s_r[t] : rms_factor(reduce_row(sumsq(x), lpr), a.H, a.eps);
#pragma unroll
    for (int q = 0; q < RP; ++q) {
      const float g = reduce_row(out[q], lpr) * r;
      const float v = reduce_row(out[RP + q], lpr) * r;
      if (pairs[q] >= 0 && li == lpr - 1) {
        const float av = silu_mul(g, v);
        const uint32_t hb = __float_as_uint(av) & 0xFFFF0000u;
        const uint32_t lo = f32_to_bf16_rne(av - __uint_as_float(hb));
        st_tag(a.tg_a + ((int64_t)t * (a.k + 1) + slot) * a.imax + a_word(pairs[q], a.imax), (hb >> 16) | (lo << 16),
               ep);
      }
    }
  }
}

// ------------------------------------------------------------- phase C
// Down projection rows [j0, j0 + J) of one expert for the token rows in
// rowmask; results to s_D[(t (k+1) + slot) J + jj].
template <int BITS, int CPL, int RD>
__device__ __forceinline__ void down_rows(const PArgs& a, uint32_t ep, const uint8_t* mat, int K, int j0,
                                          uint32_t rowmask, int slot_fixed, int e, const int* s_ids, float* s_D) {
  const int lpr = lanes_per_row(K), rpw = 64 / lpr;
  int li = (threadIdx.x & 63) % lpr, sr = (threadIdx.x & 63) / lpr;
  opaque_lane(li, sr);
  const int J = a.J;
  const int64_t rb = row_bytes(BITS, K);
  const uint32_t* sb = (const uint32_t*)(mat + matrix_codes_bytes(BITS, a.H, K));
  int jj[RD];
  const uint8_t* rc[RD];
  const uint32_t* rs[RD];
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    const int q = sr + rpw * r;
    const bool ok = q < J && j0 + q < a.H;
    jj[r] = ok ? q : -1;
    rc[r] = ok ? mat + (int64_t)(j0 + q) * rb : nullptr;
    rs[r] = ok ? sb + (int64_t)(j0 + q) * (K >> 6) : nullptr;
  }
  RowsQ<BITS, CPL, RD> Q;
  load_rows<BITS, CPL, RD>(Q, rc, rs, K, (int)(rb >> 2), li, lpr);
  XLane<BITS, CPL> xh, xl;
  float out[RD];
  const int nch = K >> 5;
  for (int t = 0; t < a.T; ++t) {
    if (!(rowmask >> t & 1u)) continue;
    int slot = slot_fixed;
    if (slot < 0)
      for (int i = 0; i < a.k; ++i)
        if (s_ids[t * kMaxTopK + i] == e) slot = i;
    const uint64_t* src = a.tg_a + ((int64_t)t * (a.k + 1) + slot) * a.imax;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      const int c = li + lpr * m;
      uint32_t w[32];
      if (c < nch) {
        poll_words<32>(src + c, a.imax >> 5, ep, w, a.status);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) w[i] = 0u;
      }
      split_arrange<BITS>(w, c, xh.w[m], xl.w[m]);
      xh.s[m] = sum_words<XWords<BITS>::N>(xh.w[m]);
      xl.s[m] = sum_words<XWords<BITS>::N>(xl.w[m]);
    }
    dot_rows<BITS, CPL, RD, 2>(Q, xh, xl, out);
#pragma unroll
    for (int r = 0; r < RD; ++r) {
      const float v = reduce_row(out[r], lpr);
      if (jj[r] >= 0 && li == lpr - 1) s_D[(t * (a.k + 1) + slot) * J + jj[r]] = v;
    }
  }
}

// ------------------------------------------------------------- phase B
// Routing of token row t on one wave: polls the row's E logits and RMS
// factor, selects the top-k (E <= 64 M) and records ids, weights and the
// experts' row masks in LDS.
template <int M>
__device__ __forceinline__ void route_row(const PArgs& a, int t, uint32_t ep, int* s_ids, float* s_w,
                                          uint32_t* s_emask, float* s_r, float* s_sg, int* s_units,
                                          uint32_t* s_masks) {
  const int lane = threadIdx.x & 63;
  uint32_t rv[M];
  uint32_t rr = 0u, rg = 0u;
  uint32_t spins = 0;
  while (true) {  // all logits of the row and its RMS factor, polled together
    bool ok = true;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int e = lane + 64 * m;
      rv[m] = 0u;
      if (e < a.E) {
        const uint64_t v = ld_tag(a.tg_logit + (int64_t)t * a.E + e);
        rv[m] = (uint32_t)v;
        ok &= (uint32_t)(v >> 32) == ep;
      }
    }
    const uint64_t v = ld_tag(a.tg_rs + 2 * t);
    rr = (uint32_t)v;
    ok &= (uint32_t)(v >> 32) == ep;
    const uint64_t vg = ld_tag(a.tg_rs + 2 * t + 1);
    rg = (uint32_t)vg;
    ok &= (uint32_t)(vg >> 32) == ep;
    if (__all(ok)) break;
    ++spins;
    if ((spins & 63) == 0) {
      if (ld_status(a.status)) break;
      if (spins > kSpinLimit) {
        __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
  const float r = __uint_as_float(rr);
  int key[M];
#pragma unroll
  for (int m = 0; m < M; ++m) key[m] = lane + 64 * m < a.E ? fkey(r * __uint_as_float(rv[m])) : INT_MIN;
  int my_id;
  float my_w;
  topk_select<M>(key, a.k, my_id, my_w);
  if (lane < a.k) {
    s_ids[t * kMaxTopK + lane] = my_id;
    s_w[t * kMaxTopK + lane] = my_w;
    if (a.T == 1) {  // one row: its k experts are the units, in rank order
      s_units[lane] = my_id;
      s_masks[lane] = 1u;
    } else {
      atomicOr(&s_emask[my_id], 1u << t);
    }
  }
  if (lane == 0) {
    s_r[t] = r;
    s_sg[t] = __uint_as_float(rg);
  }
}

#define MOE_PBITS(bits, B, ...)                        \
  switch (bits) {                                      \
    case 2: { constexpr int B = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int B = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int B = 4; __VA_ARGS__; } break; \
    case 6: { constexpr int B = 6; __VA_ARGS__; } break; \
    default: { constexpr int B = 8; __VA_ARGS__; } break; \
  }

template <int CPL_H, int CPL_I, int RD>
__global__ void __launch_bounds__(kPThreads) stack_kernel(PArgs a) {
  __shared__ int s_ids[kMaxT * kMaxTopK];
  __shared__ float s_w[kMaxT * kMaxTopK];
  __shared__ float s_r[kMaxT];
  __shared__ float s_sg[kMaxT];
  __shared__ uint32_t s_emask[kMaxExperts];
  __shared__ int s_units[kMaxT * kMaxTopK];
  __shared__ uint32_t s_masks[kMaxT * kMaxTopK];
  __shared__ int s_wcnt[kPWaves];
  __shared__ float s_D[kMaxT * (kMaxTopK + 1) * 16];
  __shared__ uint16_t s_h[kMaxT * 16];  // this workgroup's slice of h (next residual)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gw = wave * a.nwg + blockIdx.x;  // grid-wide wave index, consecutive ones on different CUs
  const int n_gw = kPWaves * a.nwg;
  const int J = a.J, j0 = blockIdx.x * J;
  const int lpr_h = lanes_per_row(a.H), rpw_h = 64 / lpr_h, sr_h = lane / lpr_h, li_h = lane % lpr_h;
  constexpr int RP = PTaskRows<CPL_H>::R / 2;
  const uint32_t all_rows = a.T >= 32 ? 0xFFFFFFFFu : ((1u << a.T) - 1u);
  // with fewer rows than waves, the last wave has no routing row: it takes
  // the shared expert's down rows during the top-k
  const bool sh_in_b = a.T < kPWaves;

  // residual slice of the launch input
  for (int i = tid; i < a.T * J; i += kPThreads) {
    const int t = i / J, q = i % J;
    s_h[i] = j0 + q < a.H ? a.h_in[(int64_t)t * a.H + j0 + q] : (uint16_t)0;
  }

  for (int l = 0; l < a.n_layers; ++l) {
    const uint8_t* layer = a.layers[l];
    const uint32_t ep = (uint32_t)l + 1;
    const bool first = l == 0;
    // ---------------- phase A: router rows, shared-expert SwiGLU, row stats
    for (int task = gw; task < a.n_rt + 1 + a.n_st; task += n_gw) {
      if (task < a.n_rt) {
        if (a.rbits == kDense) {
          router_rows<kDense, CPL_H>(a, layer, first, ep, task, li_h, lpr_h, sr_h, rpw_h);
        } else {
          MOE_PBITS(a.rbits, B, router_rows<B, CPL_H>(a, layer, first, ep, task, li_h, lpr_h, sr_h, rpw_h));
        }
      } else if (task == a.n_rt) {
        if (a.rbits == kDense) {
          stats_rows<kDense, CPL_H>(a, layer, first, ep, li_h, lpr_h, sr_h);
        } else {
          MOE_PBITS(a.rbits, B, stats_rows<B, CPL_H>(a, layer, first, ep, li_h, lpr_h, sr_h));
        }
      } else {
        const int i0 = (task - a.n_rt - 1) * RP * rpw_h;
        MOE_PBITS(a.sbits, B,
                  swiglu_rows<B, CPL_H>(a, first, ep, layer + a.off_shared, a.off_shared_up, a.Is, i0, all_rows, a.k,
                                        -1, nullptr, nullptr, li_h, lpr_h, sr_h, rpw_h));
      }
    }
    // ---------------- phase B: routing (every workgroup), routed SwiGLU rows
    if (a.T > 1) {
      for (int e = tid; e < a.E; e += kPThreads) s_emask[e] = 0u;
      __syncthreads();
    }
    if (sh_in_b && wave == kPWaves - 1 && j0 < a.H) {
      // shared-expert down rows on a wave that has no routing row
      const uint8_t* mat = layer + a.off_shared + a.off_shared_down;
      MOE_PBITS(a.sbits, B, down_rows<B, CPL_I, RD>(a, ep, mat, a.Is, j0, all_rows, a.k, -1, s_ids, s_D));
    }
    for (int t = wave; t < a.T; t += kPWaves) {
      switch (a.mE) {
        case 1: route_row<1>(a, t, ep, s_ids, s_w, s_emask, s_r, s_sg, s_units, s_masks); break;
        case 2: route_row<2>(a, t, ep, s_ids, s_w, s_emask, s_r, s_sg, s_units, s_masks); break;
        case 4: route_row<4>(a, t, ep, s_ids, s_w, s_emask, s_r, s_sg, s_units, s_masks); break;
        default: route_row<8>(a, t, ep, s_ids, s_w, s_emask, s_r, s_sg, s_units, s_masks); break;
      }
    }
    __syncthreads();
    int base = a.T == 1 ? a.k : 0;
    for (int e0 = 0; a.T > 1 && e0 < a.E; e0 += kPThreads) {
      const int e = e0 + tid;
      const bool used = e < a.E && s_emask[e] != 0u;
      const unsigned long long bal = __ballot(used);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) s_wcnt[wave] = __popcll(bal);
      __syncthreads();
      int off = base;
      for (int w = 0; w < wave; ++w) off += s_wcnt[w];
      if (used) {
        s_units[off + before] = e;
        s_masks[off + before] = s_emask[e];
      }
      for (int w = 0; w < kPWaves; ++w) base += s_wcnt[w];
      __syncthreads();
    }
    const int n_units = base;
    if (blockIdx.x == 0) {
      for (int i = tid; i < a.T * a.k; i += kPThreads) {
        const int t = i / a.k, j = i % a.k;
        if (a.ids_out) a.ids_out[(int64_t)l * a.T * a.k + i] = s_ids[t * kMaxTopK + j];
        if (a.w_out) a.w_out[(int64_t)l * a.T * a.k + i] = s_w[t * kMaxTopK + j];
      }
    }
    for (int task = gw; task < n_units * a.tpu; task += n_gw) {
      const int u = task / a.tpu;
      const int i0 = (task % a.tpu) * RP * rpw_h;
      const int e = s_units[u];
      const uint8_t* blk = layer + a.off_e0 + (int64_t)e * a.e_stride;
      MOE_PBITS(a.ebits, B,
                swiglu_rows<B, CPL_H>(a, first, ep, blk, a.off_e_up, a.I, i0, s_masks[u], -1, e, s_ids, s_r, li_h,
                                      lpr_h, sr_h, rpw_h));
    }
    // ---------------- phase C: down projections of this workgroup's rows, combine
    if (j0 < a.H) {
      const int n_down = n_units + (sh_in_b ? 0 : 1);
      for (int u = wave; u < n_down; u += kPWaves) {
        if (u < n_units) {
          const int e = s_units[u];
          const uint8_t* mat = layer + a.off_e0 + (int64_t)e * a.e_stride + a.off_e_down;
          MOE_PBITS(a.ebits, B, down_rows<B, CPL_I, RD>(a, ep, mat, a.I, j0, s_masks[u], -1, e, s_ids, s_D));
        } else {
          const uint8_t* mat = layer + a.off_shared + a.off_shared_down;
          MOE_PBITS(a.sbits, B, down_rows<B, CPL_I, RD>(a, ep, mat, a.Is, j0, all_rows, a.k, -1, s_ids, s_D));
        }
      }
      __syncthreads();
      // two adjacent output rows per thread (one published word)
      const int npair = J >> 1;
      for (int i = tid; i < a.T * npair; i += kPThreads) {
        const int t = i / npair, q = 2 * (i % npair);
        const float sg = s_sg[t];
        uint32_t o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float acc = 0.f;
          for (int r = 0; r < a.k; ++r) acc = fmaf(s_w[t * kMaxTopK + r], s_D[(t * (a.k + 1) + r) * J + q + h], acc);
          acc = fmaf(sg, s_D[(t * (a.k + 1) + a.k) * J + q + h], acc);
          const float out = __uint_as_float((uint32_t)s_h[t * J + q + h] << 16) + acc;
          o[h] = f32_to_bf16_rne(out);
          s_h[t * J + q + h] = (uint16_t)o[h];
        }
        const int j = j0 + q;
        if (j < a.H) {
          st_tag(a.tg_h + (int64_t)t * (a.H >> 1) + h_word(j >> 1, a.H), o[0] | (o[1] << 16), ep);
          const int64_t hi = (int64_t)t * a.H + j;
          if (a.h_trace) {
            a.h_trace[(int64_t)l * a.T * a.H + hi] = (uint16_t)o[0];
            a.h_trace[(int64_t)l * a.T * a.H + hi + 1] = (uint16_t)o[1];
          }
          if (l == a.n_layers - 1) {
            a.h_out[hi] = (uint16_t)o[0];
            a.h_out[hi + 1] = (uint16_t)o[1];
          }
        }
      }
    }
    __syncthreads();
  }
}


template <int CPL_H, int CPL_I, int RD>
hipError_t launch_stack_kernel(const PArgs& a, hipStream_t st) {
  stack_kernel<CPL_H, CPL_I, RD><<<a.nwg, kPThreads, 0, st>>>(a);
  return hipGetLastError();
}

// Instantiated in persist_<CPL_H><CPL_I>.hip (one file per pair, compiled in parallel).
#define MOE_STACK_INSTANTIATE(H, I, R) template hipError_t launch_stack_kernel<H, I, R>(const PArgs&, hipStream_t);

}  // namespace moe
