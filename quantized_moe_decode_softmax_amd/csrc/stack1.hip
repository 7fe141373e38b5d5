// One-row stack decode (T = 1) as one persistent kernel per up to 64 layers,
// with the weights streamed into LDS by direct global-to-LDS loads (except a
// wave's few routed gate/up pairs, which arrive sooner through registers).
//
// At one token row a layer is a short chain of device-wide dependencies
// (hidden state -> router logits -> top-k -> activations -> down projections
// -> hidden state), and the weight bytes of each step can only be fetched once
// the previous step has chosen them. What bounds the step is how many of those
// bytes are in flight at once: a compute unit needs on the order of 100 KB
// outstanding to keep its share of the 8 TB/s busy across the memory latency.
// Loading into registers ties that amount to the register file (and to the
// in-order completion counter: a register reload or any later load waits for
// every earlier one). Here each wave instead streams the rows of its tasks
// into a private LDS ring with gfx950's global_load_lds_dwordx4 (16 bytes per
// lane, 1 KB per instruction, no registers), two halves deep, and computes a
// batch of tasks from LDS while the next batch is in flight. A burst of only
// a few KB per wave is the exception: global loads into registers bring it in
// about half the time, so a wave's routed pairs, when it has at most two,
// take that path (with no direct LDS load of the wave in flight behind them,
// since both complete in issue order). The arithmetic of every dot product is
// the one of the per-layer kernels (gemv.h), so results are bitwise equal to
// them.
//
// Exchange between workgroups: 64-bit words, payload | epoch << 32 (epoch =
// layer in the launch + 1), device-scope relaxed stores and loads; a consumer
// polls the words it needs until they carry the expected epoch, so the data
// round trip is the synchronisation. Every buffer exists in n_copy copies; a
// writer stores all of them and workgroup w reads copy w % n_copy, so that no
// cache line is polled by every compute unit. Each poll round re-reads only
// the words whose tags were not yet current.
//
// Per layer and workgroup (8 waves, one workgroup per compute unit, as many
// workgroups as the hidden state has slices of J rows):
//   A  stream this workgroup's router rows and shared-expert row pairs; stage
//      h_l in LDS; compute raw logits and shared activations; publish them
//   R  wave 0: RMS factor and shared gate of the row, top-k of the logits,
//      renormalised weights (every workgroup routes for itself), then an LDS
//      flag releases the other waves; meanwhile the last wave loads the
//      shared expert's down rows [j0, j0 + J) and their inputs (published in
//      phase A) into LDS
//   B  load (registers, at most two per wave, else the ring) and compute
//      this workgroup's range of routed row pairs (k experts x I pairs split
//      evenly over the grid), storing each activation as it is computed;
//      each wave then polls the activation vector of the slot of its down
//      task into LDS
//   C  the shared expert's down rows (one task per wave, before the routed
//      activations are polled), the down-projection rows [j0, j0 + J) of the
//      k experts (weights streamed through the ring during B, or right after
//      it when B used registers), combine in rank order, residual, bf16,
//      publish the slice of h_{l+1}
//
// Buffer reuse: every workgroup publishes a slice of h in every layer. Logits
// and activations of layer l+1 are written only by workgroups that have
// seen all of h_{l+1}, i.e. after every workgroup finished layer l (one buffer
// each). h alternates between two buffers by layer parity: h_{l+2} is written
// after its writer saw all of h_{l+1}, which every workgroup published after
// reading h_l.
//
// Every wait is bounded; a timed-out wait sets status[0] and every later wait
// returns at once, so a failed launch still drains (results are then invalid
// and moe_stack_status reports it).
//
// Sources: PureDrive-35B-A3B-MLX model card, "Summary" (top-8 of 256 routed
// experts plus a shared expert) and "How it works"; flash-moe news page
// (ja.news.hada.io topic 27758), "FMA-optimised dequant kernel" (group-affine
// weights), "Metal Compute Shaders" (SwiGLU, RMS normalisation, combine +
// residual + gate) and "Deferred GPU Expert Compute" (the combined output
// feeds the next layer on the GPU).
#include <algorithm>
#include <atomic>
#include <cmath>

#include "gemv.h"

namespace moe {
namespace t1 {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRingBytes = 10240;  // per wave: two halves
constexpr int kHalf = kRingBytes / 2;
constexpr uint32_t kSpinLimit = 1u << 21;
constexpr int kMaxWG = 512;
constexpr int kMaxH = 4096;
constexpr int kMaxAWords = 12288;  // (k + 1) * imax
// Slots of the per-phase timestamps of a phase-trace build (wave recording it):
//  0 layer start (w0)            1 h staged in LDS (w0)        2 phase A computed (w0)
//  3 all logits seen (w0)        4 top-k done (w0)             5 routed loads issued (w0)
//  6 routed pairs computed (w0)  7 routed pairs computed (w7)  8 routed activations stored (w0)
//  9 first down slot's inputs in LDS (w0)
// 10 down rows done (w0)        11 combine done (thread 0)   12 shared down inputs fetched (w7)
// 13 down rows requested (w0)   14 down rows in LDS (w0)
constexpr int kPhases = 16;

struct Args {
  int H, E, I, Is, k, imax;
  int rbits, ebits, sbits;
  float eps;
  int64_t off_router, off_gatevec, off_shared, off_shared_up, off_shared_down;
  int64_t off_e0, e_stride, off_e_up, off_e_down;
  int n_layers, nwg, J;
  int ra, sa, pb;  // router rows, shared pairs and routed pairs per workgroup
  int mE;          // experts per lane in the top-k (E <= 64 mE)
  const uint16_t* h_in;
  uint16_t* h_out;
  int32_t* ids_out;
  float* w_out;
  uint16_t* h_trace;  // [n_layers][H] or null
  uint64_t* x_h;      // [2][n_copy] copies of [H/2], stride h_cs
  uint64_t* x_logit;  // [n_copy] copies of [E], stride l_cs
  uint64_t* x_a;      // [n_copy] copies of [k+1][imax], stride a_cs
  int64_t h_cs, l_cs, a_cs;
  int n_copy;
  uint32_t* status;
  // the launch's layer blocks: table[l0 + l] (a descriptor table in device
  // memory) when table is set, else layers[l]
  const uint8_t* const* table;
  int l0;
  uint64_t* phase_ts;  // per-phase timestamps [layer][workgroup][kPhases] (phase-trace builds), or null
  const uint8_t* layers[kMaxLayersPerLaunch];
};

// ------------------------------------------------------------ exchange words
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t v, uint32_t epoch) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// v | epoch << 32 at p in every copy
__device__ __forceinline__ void st_copies(uint64_t* p, int64_t cs, int n_copy, uint32_t v, uint32_t epoch) {
  for (int c = 0; c < n_copy; ++c) st_tag(p + c * cs, v, epoch);
}

// Bounded-wait bookkeeping: true when the caller must stop waiting (another
// wait timed out, or this one did).
__device__ __forceinline__ bool give_up(uint32_t& spins, uint32_t* status) {
  ++spins;
  if ((spins & 63) == 0) {
    if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return true;
    if (spins > kSpinLimit) {
      __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return true;
    }
  }
  __builtin_amdgcn_s_sleep(2);
  return false;
}

// Waits until the words p[off(i)] (i < N, bit i of `want` set) carry `epoch`;
// payloads to out[i] (0 for the others). All pending words are read in one
// batch per round, and a word is read again only until it has been seen.
template <int N, class Off>
__device__ __forceinline__ void poll(const uint64_t* p, const Off& off, uint32_t want, uint32_t epoch,
                                     uint32_t (&out)[N], uint32_t* status) {
  uint32_t pending = want;
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = 0u;
  uint32_t spins = 0;
  while (true) {
    uint64_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (pending >> i & 1u) ? ld_tag(p + off(i)) : 0ull;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((pending >> i & 1u) && (uint32_t)(v[i] >> 32) == epoch) {
        out[i] = (uint32_t)v[i];
        pending &= ~(1u << i);
      }
    }
    if (pending == 0u) return;
    if (give_up(spins, status)) return;
  }
}

// LDS words that one wave sets and others wait for: relaxed workgroup-scope
// atomics, which compile to plain ds_write / ds_read. (A volatile access
// through the generic pointer becomes a flat access, and the compiler then
// waits for every outstanding global load of the wave as well.)
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Workgroup barrier for LDS data only (the kernel never reads its own global
// stores through a barrier, so it does not wait for them as __syncthreads does).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------ LDS streaming
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Streams `bytes` (a multiple of 16) from global src into LDS at byte address
// dst, 16 bytes per lane and 1 KB per instruction; returns the number of
// instructions issued.
__device__ __forceinline__ int dma16(const uint8_t* src, uint32_t dst, int bytes) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int off = 0; off < bytes; off += 1024, ++n)
    if (off + 16 * lane < bytes)
      asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src + off + 16 * lane), "{m0}"(dst + off) : "memory");
  return n;
}
// The same for a multiple of 4 bytes, 4 bytes per lane (scale/bias words).
__device__ __forceinline__ int dma4(const uint8_t* src, uint32_t dst, int bytes) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int off = 0; off < bytes; off += 256, ++n)
    if (off + 4 * lane < bytes)
      asm volatile("global_load_lds_dword %0, off" ::"v"(src + off + 4 * lane), "{m0}"(dst + off) : "memory");
  return n;
}

#define MOE_VMW(n) \
  case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;
// Waits until at most n of this wave's vector memory operations are
// outstanding (they complete in issue order). n >= 63 needs no wait: the
// counter never holds more.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    MOE_VMW(0) MOE_VMW(1) MOE_VMW(2) MOE_VMW(3) MOE_VMW(4) MOE_VMW(5) MOE_VMW(6) MOE_VMW(7)
    MOE_VMW(8) MOE_VMW(9) MOE_VMW(10) MOE_VMW(11) MOE_VMW(12) MOE_VMW(13) MOE_VMW(14) MOE_VMW(15)
    MOE_VMW(16) MOE_VMW(17) MOE_VMW(18) MOE_VMW(19) MOE_VMW(20) MOE_VMW(21) MOE_VMW(22) MOE_VMW(23)
    MOE_VMW(24) MOE_VMW(25) MOE_VMW(26) MOE_VMW(27) MOE_VMW(28) MOE_VMW(29) MOE_VMW(30) MOE_VMW(31)
    MOE_VMW(32) MOE_VMW(33) MOE_VMW(34) MOE_VMW(35) MOE_VMW(36) MOE_VMW(37) MOE_VMW(38) MOE_VMW(39)
    MOE_VMW(40) MOE_VMW(41) MOE_VMW(42) MOE_VMW(43) MOE_VMW(44) MOE_VMW(45) MOE_VMW(46) MOE_VMW(47)
    MOE_VMW(48) MOE_VMW(49) MOE_VMW(50) MOE_VMW(51) MOE_VMW(52) MOE_VMW(53) MOE_VMW(54) MOE_VMW(55)
    MOE_VMW(56) MOE_VMW(57) MOE_VMW(58) MOE_VMW(59) MOE_VMW(60) MOE_VMW(61) MOE_VMW(62)
    default: break;
  }
}
#undef MOE_VMW

// Raw packed words of chunk c from a row held in LDS (same words as
// load_chunk reads from global memory; bits 2/4/6/8).
template <int BITS>
__device__ __forceinline__ void lds_chunk(const uint8_t* row, int c, uint32_t (&q)[8]) {
  if constexpr (BITS == 2) {
    const u32x2 v = *(const u32x2*)(row + 8 * c);
    q[0] = v.x;
    q[1] = v.y;
  } else if constexpr (BITS == 4) {
    const u32x4 v = *(const u32x4*)(row + 16 * c);
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
    q[3] = v.w;
  } else if constexpr (BITS == 6) {
    const u32x2* p = (const u32x2*)(row + 24 * c);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x2 v = p[i];
      q[2 * i] = v.x;
      q[2 * i + 1] = v.y;
    }
  } else {
    const u32x4* p = (const u32x4*)(row + 32 * c);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 v = p[i];
      q[4 * i] = v.x;
      q[4 * i + 1] = v.y;
      q[4 * i + 2] = v.z;
      q[4 * i + 3] = v.w;
    }
  }
}

// This lane's partial of a quantised row held in LDS (codes at `codes`,
// scale/bias words at `sb`): sum over the lane's chunks of chunk_partial, in
// the order dot_rows uses. NX = 2: against the split input x0 + x1.
template <int BITS, int CPL, int NX>
__device__ __forceinline__ float lds_row(const uint8_t* codes, const uint32_t* sb, int K, int li, int lpr,
                                         const XLane<BITS, CPL>& x0, const XLane<BITS, CPL>& x1) {
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    uint32_t q[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t sbw = 0u;
    if (c < (K >> 5)) {
      lds_chunk<BITS>(codes, c, q);
      sbw = sb[c >> 1];
    }
    acc += chunk_partial<BITS, NX>(q, sbw, x0.w[m], x0.s[m], x1.w[m], x1.s[m]);
  }
  return acc;
}

// The same for a dense bf16 row (a bf16 router).
template <int CPL>
__device__ __forceinline__ float lds_row_dense(const uint8_t* row, int K, int li, int lpr,
                                               const XLane<kDense, CPL>& x) {
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0u;
    if (c < (K >> 5)) {
      const u32x4* p = (const u32x4*)(row + 64 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = p[i];
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
      }
    }
    acc += dense_chunk(w, x.w[m]);
  }
  return acc;
}

// The lane's arranged chunks of the hidden state (LDS, bf16 pairs).
template <int BITS, int CPL>
__device__ __forceinline__ void h_lane(const uint32_t* s_h, int H, int li, int lpr, XLane<BITS, CPL>& x) {
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    uint32_t n[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) n[i] = c < (H >> 5) ? s_h[16 * c + i] : 0u;
    arrange_chunk<BITS>(n, c, x.w[m]);
    x.s[m] = sum_words<XWords<BITS>::N>(x.w[m]);
  }
}

// Split (hi, lo) arranged chunks of one activation vector (LDS words hi | lo << 16).
template <int BITS, int CPL>
__device__ __forceinline__ void a_lane(const uint32_t* va, int K, int li, int lpr, XLane<BITS, CPL>& xh,
                                       XLane<BITS, CPL>& xl) {
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = li + lpr * m;
    uint32_t w[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = c < (K >> 5) ? va[32 * c + i] : 0u;
    split_arrange<BITS>(w, c, xh.w[m], xl.w[m]);
    xh.s[m] = sum_words<XWords<BITS>::N>(xh.w[m]);
    xl.s[m] = sum_words<XWords<BITS>::N>(xl.w[m]);
  }
}

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + expf(-g)) * v; }
__device__ __forceinline__ float rms_factor(float ss, int H, float eps) { return 1.0f / sqrtf(ss / (float)H + eps); }
__device__ __forceinline__ uint32_t split_a(float av) {
  const uint32_t hb = __float_as_uint(av) & 0xFFFF0000u;
  return (hb >> 16) | (f32_to_bf16_rne(av - __uint_as_float(hb)) << 16);
}
// Exchange layout of an activation vector: element i at word
// (i % 32) * (imax / 32) + i / 32.
__device__ __forceinline__ int a_word(int i, int imax) { return (i & 31) * (imax >> 5) + (i >> 5); }

// Bytes of one packed row and of its scale/bias words; a run of n rows in
// the ring is [codes][scale/bias] rounded up to 16 bytes.
__host__ __device__ __forceinline__ int code_bytes(int bits, int K) { return bits == kDense ? 2 * K : K * bits / 8; }
__host__ __device__ __forceinline__ int sb_bytes(int bits, int K) { return bits == kDense ? 0 : K / 16; }
__host__ __device__ __forceinline__ int seg_bytes(int bits, int K, int n) {
  return (n * (code_bytes(bits, K) + sb_bytes(bits, K)) + 15) & ~15;
}

// ------------------------------------------------------------------ tasks
// A task is a contiguous run of rows of one matrix (or of a gate/up pair of
// matrices) that one wave computes, one row per row group; its bytes are
// streamed into the wave's ring as [codes][scale/bias] (twice for a pair).
enum Kind { kRouter = 0, kSharedPair = 1, kRoutedPair = 2, kDown = 3 };
struct Task {
  int kind;
  const uint8_t* mat;  // first matrix (gate for pairs)
  int64_t up;          // byte offset of the up matrix from mat (pairs)
  int rows_total;      // rows of the matrix (for the scale/bias offset)
  int K, bits;
  int r0, n;           // first row, rows
  int slot;            // pairs: routing rank (k = shared); down: activation slot
  int bytes;           // ring bytes
};

__host__ __device__ __forceinline__ int task_bytes(int bits, int K, int n, bool pair) {
  return (pair ? 2 : 1) * seg_bytes(bits, K, n);
}

// Streams one matrix's rows [r0, r0 + n) into LDS at dst; returns instructions.
__device__ __forceinline__ int dma_rows(const uint8_t* mat, int rows_total, int K, int bits, int r0, int n,
                                        uint32_t dst) {
  const int cb = code_bytes(bits, K);
  int cnt = dma16(mat + (int64_t)r0 * cb, dst, n * cb);
  if (bits != kDense) {
    const int sbb = sb_bytes(bits, K);
    const uint8_t* sb = mat + matrix_codes_bytes(bits, rows_total, K);
    cnt += dma4(sb + (int64_t)r0 * sbb, dst + n * cb, n * sbb);
  }
  return cnt;
}
__device__ __forceinline__ int dma_task(const Task& t, uint32_t dst) {
  int cnt = dma_rows(t.mat, t.rows_total, t.K, t.bits, t.r0, t.n, dst);
  if (t.kind == kSharedPair || t.kind == kRoutedPair)
    cnt += dma_rows(t.mat + t.up, t.rows_total, t.K, t.bits, t.r0, t.n, dst + t.bytes / 2);  // second segment
  return cnt;
}

// Runs the statement with `constexpr int B` = the code width: FIXED when it
// is nonzero (a kernel specialised for one shape: no other width is
// compiled into its instruction stream), else the runtime width `bits`.
#define MOE_T1_BITS(FIXED, bits, B, ...)                     \
  if constexpr ((FIXED) != 0) {                              \
    constexpr int B = (FIXED);                               \
    __VA_ARGS__;                                             \
  } else {                                                   \
    switch (bits) {                                          \
      case 2: { constexpr int B = 2; __VA_ARGS__; } break;   \
      case 4: { constexpr int B = 4; __VA_ARGS__; } break;   \
      case 6: { constexpr int B = 6; __VA_ARGS__; } break;   \
      default: { constexpr int B = 8; __VA_ARGS__; } break;  \
    }                                                        \
  }
// The same for the router, whose width may also be kDense (bf16 rows).
#define MOE_T1_RBITS(FIXED, bits, B, ...)                        \
  if constexpr ((FIXED) != 0) {                                  \
    constexpr int B = (FIXED);                                   \
    __VA_ARGS__;                                                 \
  } else if ((bits) == kDense) {                                 \
    constexpr int B = kDense;                                    \
    __VA_ARGS__;                                                 \
  } else {                                                       \
    MOE_T1_BITS(0, bits, B, __VA_ARGS__);                        \
  }

// Per-workgroup state shared by the phases (LDS).
struct Shared {
  uint32_t h[kMaxH / 2];         // h_l, bf16 pairs
  uint32_t a[kMaxAWords];        // activation vectors of the k + 1 slots, hi | lo << 16
  float D[(kMaxTopK + 1) * 16];  // down-projection outputs [slot][J]
  int ids[kMaxTopK];
  float w[kMaxTopK];
  float r, sg;
  uint32_t route_ep;  // epoch of the layer whose routing ids/w/r/sg hold
  // expert of rank i as soon as the top-k has chosen it: epoch << 16 | id
  // (S.r of the same layer is in place before the first of them)
  uint32_t rank_tag[kMaxTopK];
  uint32_t logit_ep;  // epoch of the layer whose logits wave 0 has seen (so all phase A output exists)
  uint32_t sd_ep;     // epoch of the layer whose shared down rows and inputs are in S.sd / S.a
  uint64_t layers[kMaxLayersPerLaunch];  // the launch's layer blocks
#ifdef MOE_PHASE_TRACE
  uint64_t ts[kPhases];  // this layer's phase timestamps (s_memrealtime, 100 MHz)
#endif
  __attribute__((aligned(16))) uint8_t ring[kWaves][kRingBytes];
  __attribute__((aligned(16))) uint8_t sd[kRingBytes];  // the shared expert's down rows of the slice
};

// ------------------------------------------------------------- the kernel
__shared__ Shared S;

// Phase timestamps (builds with MOE_PHASE_TRACE only): lane 0 of the calling
// wave stores the 100 MHz real-time counter in slot P of the layer's record.
// The counter is read in inline assembly, together with its own wait, so
// that the compiler adds no wait for the wave's outstanding memory operations
// (it does for the builtin), which would change the timing being recorded.
#ifdef MOE_PHASE_TRACE
#define MOE_TS(P)                                                                         \
  do {                                                                                    \
    if ((threadIdx.x & 63) == 0) {                                                        \
      uint64_t t_;                                                                        \
      asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t_)::"memory");       \
      S.ts[P] = t_;                                                                       \
    }                                                                                     \
  } while (0)
#else
#define MOE_TS(P) \
  do {            \
  } while (0)
#endif

// Per-thread constants of the current layer (values only: the kernel
// arguments are always referenced directly, never stored).
struct Ctx {
  const uint8_t* layer;
  uint32_t ep;
  int lane, wave, lpr_h, rpw_h, li_h, sr_h;
  int cp;  // this workgroup's copy of the exchange buffers
  // dimensions, code widths, layout offsets and grid split: constants in a
  // kernel specialised for one shape, else copied from the arguments
  int H, E, I, Is, k, imax, rbits, ebits, sbits, J, nwg, ra, sa, pb, mE, n_copy;
  float eps;
  int64_t off_router, off_gatevec, off_shared, off_shared_up, off_shared_down, off_e0, e_stride, off_e_up, off_e_down;
  int64_t h_cs, l_cs, a_cs;
};

// ---- phase A tasks: router row blocks, then shared pair blocks
template <int CPL_H, int CPL_I>
__device__ __forceinline__ int n_a_tasks(const Args& a, const Ctx& c) {
  const int r0 = blockIdx.x * c.ra, s0 = blockIdx.x * c.sa;
  const int nr = max(0, min(c.ra, c.E - r0)), ns = max(0, min(c.sa, c.Is - s0));
  return (nr + c.rpw_h - 1) / c.rpw_h + (ns + c.rpw_h - 1) / c.rpw_h;
}
template <int CPL_H, int CPL_I>
__device__ __forceinline__ Task a_task(const Args& a, const Ctx& c, int i) {
  const int r0 = blockIdx.x * c.ra, s0 = blockIdx.x * c.sa;
  const int nr = max(0, min(c.ra, c.E - r0)), ns = max(0, min(c.sa, c.Is - s0));
  const int tr = (nr + c.rpw_h - 1) / c.rpw_h;
  Task t;
  t.K = c.H;
  t.up = 0;
  t.slot = c.k;
  if (i < tr) {
    t.kind = kRouter;
    t.mat = c.layer + c.off_router;
    t.rows_total = c.E;
    t.bits = c.rbits;
    t.r0 = r0 + i * c.rpw_h;
    t.n = min(c.rpw_h, r0 + nr - t.r0);
    t.bytes = task_bytes(t.bits, t.K, t.n, false);
  } else {
    t.kind = kSharedPair;
    t.mat = c.layer + c.off_shared;
    t.up = c.off_shared_up;
    t.rows_total = c.Is;
    t.bits = c.sbits;
    t.r0 = s0 + (i - tr) * c.rpw_h;
    t.n = min(c.rpw_h, s0 + ns - t.r0);
    t.bytes = task_bytes(t.bits, t.K, t.n, true);
  }
  return t;
}

// ---- phase B tasks: this workgroup's pairs [f0, f1) of the k x I routed
// pairs (rank-major), in blocks of c.rpw_h pairs that stay within one expert
template <int CPL_H, int CPL_I>
__device__ __forceinline__ int n_b_tasks(const Args& a, const Ctx& c) {
  const int f0 = blockIdx.x * c.pb, f1 = min(c.k * c.I, f0 + c.pb);
  int n = 0;
  for (int f = f0; f < f1;) {
    const int end = min(f1, (f / c.I + 1) * c.I);
    n += (end - f + c.rpw_h - 1) / c.rpw_h;
    f = end;
  }
  return n;
}
// Split order (one pair per task, 2 x kWaves pairs per workgroup, k even,
// every workgroup a full share): workgroup g owns pairs [g pb/2, (g+1) pb/2)
// of the first k/2 ranks and the same range of the last k/2 ranks, so each
// wave's first pair is of an early rank and its second of a late one; the
// first is computed while the second, requested once the top-k reaches its
// rank, is still arriving.
__device__ __forceinline__ bool split_b(const Ctx& c) {
  return c.rpw_h == 1 && (c.k & 1) == 0 && c.pb == 2 * kWaves && c.nwg * c.pb == c.k * c.I && c.I <= 64 * c.pb;
}
// IdOf: the expert id of a rank (see rank_id).
template <int CPL_H, int CPL_I, class IdOf>
__device__ __forceinline__ Task b_task(const Args& a, const Ctx& c, int i, const IdOf& id_of) {
  const int f0 = blockIdx.x * c.pb, f1 = min(c.k * c.I, f0 + c.pb);
  Task t;
  t.kind = kRoutedPair;
  t.K = c.H;
  t.bits = c.ebits;
  t.rows_total = c.I;
  t.up = c.off_e_up;
  if (split_b(c)) {
    const int h = c.pb / 2;
    const int f = i < h ? blockIdx.x * h + i : c.k / 2 * c.I + blockIdx.x * h + (i - h);
    const int u = f / c.I;
    t.slot = u;
    t.mat = c.layer + c.off_e0 + (int64_t)id_of(u) * c.e_stride;
    t.r0 = f % c.I;
    t.n = 1;
    t.bytes = task_bytes(t.bits, t.K, t.n, true);
    return t;
  }
  for (int f = f0; f < f1;) {
    const int end = min(f1, (f / c.I + 1) * c.I);
    const int nt = (end - f + c.rpw_h - 1) / c.rpw_h;
    if (i < nt) {
      const int u = f / c.I;
      t.slot = u;
      t.mat = c.layer + c.off_e0 + (int64_t)id_of(u) * c.e_stride;
      t.r0 = f % c.I + i * c.rpw_h;
      t.n = min(c.rpw_h, end - (f + i * c.rpw_h));
      break;
    }
    i -= nt;
    f = end;
  }
  t.bytes = task_bytes(t.bits, t.K, t.n, true);
  return t;
}
// The expert of rank u once wave 0's top-k has chosen it (this layer's tag).
// On a time-out the stale id is still a valid expert (the status word says so).
__device__ __forceinline__ int rank_id(const Args& a, const Ctx& c, int u) {
  uint32_t spins = 0, v;
  while (((v = lds_ld(&S.rank_tag[u])) >> 16) != c.ep)
    if (give_up(spins, a.status)) break;
  return (int)(v & 0xFFFFu);
}

// ---- phase C tasks: for each slot (k routed experts in rank order, then
// the shared expert) the J rows of this workgroup, rpw rows per task
__device__ __forceinline__ int rpw_down(int K) { return 64 / lanes_per_row(K); }
// Rows of one down task: the workgroup's J rows of one expert, or as many
// whole row-group passes of them as fit in half a ring.
__host__ __device__ __forceinline__ int down_task_rows(int J, int K, int bits) {
  const int rpw = 64 / lanes_per_row(K);
  int n = J;
  while (n > rpw && seg_bytes(bits, K, n) > kHalf) n -= rpw;
  return n;
}
// C tasks: the routed experts' down rows of this workgroup's slice, slot by
// slot (the shared expert's rows are computed separately, see
// shared_down_fetch)
__device__ __forceinline__ int n_c_tasks(const Args& a, const Ctx& c) {
  const int de = down_task_rows(c.J, c.I, c.ebits);
  return c.k * ((c.J + de - 1) / de);
}
template <class IdOf>
__device__ __forceinline__ Task c_task(const Args& a, const Ctx& c, int i, const IdOf& id_of) {
  const int de = down_task_rows(c.J, c.I, c.ebits);
  const int tr = (c.J + de - 1) / de;
  const int j0 = blockIdx.x * c.J;
  Task t;
  t.kind = kDown;
  t.up = 0;
  t.rows_total = c.H;
  const int u = i / tr;
  t.slot = u;
  t.K = c.I;
  t.bits = c.ebits;
  t.mat = c.layer + c.off_e0 + (int64_t)id_of(u) * c.e_stride + c.off_e_down;
  t.r0 = j0 + (i % tr) * de;
  t.n = min(de, min(j0 + c.J, c.H) - t.r0);
  t.bytes = task_bytes(t.bits, t.K, t.n, false);
  return t;
}

// the shared expert's down rows of this workgroup's slice
// (one pass of a wave's row groups each, so that the waves share them)
__host__ __device__ __forceinline__ int s_task_rows(int J, int Is) {
  const int rpw = 64 / lanes_per_row(Is);
  return rpw < J ? rpw : J;
}
__device__ __forceinline__ int n_s_tasks(const Args& a, const Ctx& c) {
  const int ds = s_task_rows(c.J, c.Is);
  return (c.J + ds - 1) / ds;
}
__device__ __forceinline__ Task s_task(const Args& a, const Ctx& c, int i) {
  const int ds = s_task_rows(c.J, c.Is);
  const int j0 = blockIdx.x * c.J;
  Task t;
  t.kind = kDown;
  t.up = 0;
  t.rows_total = c.H;
  t.slot = c.k;
  t.K = c.Is;
  t.bits = c.sbits;
  t.mat = c.layer + c.off_shared + c.off_shared_down;
  t.r0 = j0 + i * ds;
  t.n = min(ds, min(j0 + c.J, c.H) - t.r0);
  t.bytes = task_bytes(t.bits, t.K, t.n, false);
  return t;
}

// ---- task computation (from the ring)
template <int CPL_H, int CPL_I, int BITS>
__device__ __forceinline__ void router_row(const Args& a, const Ctx& c, const Task& t, const uint8_t* buf) {
  XLane<BITS, CPL_H> x;
  h_lane<BITS, CPL_H>(S.h, c.H, c.li_h, c.lpr_h, x);
  const int cb = code_bytes(BITS, c.H);
  float p = 0.f;
  if (c.sr_h < t.n) {
    if constexpr (BITS == kDense)
      p = lds_row_dense<CPL_H>(buf + c.sr_h * cb, c.H, c.li_h, c.lpr_h, x);
    else
      p = lds_row<BITS, CPL_H, 1>(buf + c.sr_h * cb, (const uint32_t*)(buf + t.n * cb) + c.sr_h * (c.H >> 6), c.H, c.li_h,
                                  c.lpr_h, x, x);
  }
  const float v = reduce_row(p, c.lpr_h);
  if (c.sr_h < t.n && c.li_h == c.lpr_h - 1)
    st_copies(a.x_logit + t.r0 + c.sr_h, c.l_cs, c.n_copy, __float_as_uint(v), c.ep);
}

// gate/up rows of a pair block; r < 0: RMS factor from the lane's own x
// (shared expert), else the routed rows' factor
template <int CPL_H, int CPL_I, int BITS>
__device__ __forceinline__ void pair_rows(const Args& a, const Ctx& c, const Task& t, const uint8_t* buf,
                                        const XLane<BITS, CPL_H>& x, float r) {
  const int cb = code_bytes(BITS, c.H), sbw = c.H >> 6;
  const int half = t.bytes / 2;
  float pg = 0.f, pu = 0.f;
  if (c.sr_h < t.n) {
    const uint8_t* g = buf;
    const uint8_t* u = buf + half;
    pg = lds_row<BITS, CPL_H, 1>(g + c.sr_h * cb, (const uint32_t*)(g + t.n * cb) + c.sr_h * sbw, c.H, c.li_h, c.lpr_h, x,
                                 x);
    pu = lds_row<BITS, CPL_H, 1>(u + c.sr_h * cb, (const uint32_t*)(u + t.n * cb) + c.sr_h * sbw, c.H, c.li_h, c.lpr_h, x,
                                 x);
  }
  const float rr = r >= 0.f ? r : rms_factor(reduce_row(sumsq(x), c.lpr_h), c.H, c.eps);
  const float gv = reduce_row(pg, c.lpr_h) * rr;
  const float uv = reduce_row(pu, c.lpr_h) * rr;
  if (c.sr_h < t.n && c.li_h == c.lpr_h - 1) {
    // stored at once: consumers poll these words themselves
    const int slot = t.kind == kSharedPair ? c.k : t.slot;
    st_copies(a.x_a + (int64_t)slot * c.imax + a_word(t.r0 + c.sr_h, c.imax), c.a_cs, c.n_copy,
              split_a(silu_mul(gv, uv)), c.ep);
  }
}

// A routed pair task held in registers: the lane's chunks of its gate and up
// rows (row r0 + sr_h of each) and their scale/bias words.
template <int BITS, int CPL>
struct PairRegs {
  uint32_t g[CPL][8], u[CPL][8], gs[CPL], us[CPL];
};
// Requests the task's words with global loads (no wait); rows past the task
// and chunks past the row are zero.
template <int BITS, int CPL>
__device__ __forceinline__ void pair_load(const Ctx& c, const Task& t, PairRegs<BITS, CPL>& P) {
  const int cb = code_bytes(BITS, c.H), sbw = c.H >> 6;
  const int row = t.r0 + c.sr_h;
  const bool ok = c.sr_h < t.n;
  const uint8_t* g = t.mat + (int64_t)row * cb;
  const uint8_t* u = t.mat + t.up + (int64_t)row * cb;
  const int64_t sbo = matrix_codes_bytes(BITS, t.rows_total, c.H) + (int64_t)row * sbw * 4;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int ch = c.li_h + c.lpr_h * m;
    if (ok && ch < (c.H >> 5)) {
      load_chunk<BITS>(g, ch, cb >> 2, P.g[m]);
      load_chunk<BITS>(u, ch, cb >> 2, P.u[m]);
      P.gs[m] = gload<uint32_t>(t.mat + sbo + 4 * (ch >> 1));
      P.us[m] = gload<uint32_t>(t.mat + t.up + sbo + 4 * (ch >> 1));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        P.g[m][i] = 0u;
        P.u[m][i] = 0u;
      }
      P.gs[m] = 0u;
      P.us[m] = 0u;
    }
  }
}
// pair_rows on a task held in registers (the same sums in the same order),
// returning the activation word; store_pair publishes it. (Storing both
// pairs only after computing both measured slower: the stores then meet the
// down-row requests that follow them.)
template <int CPL_H, int CPL_I, int BITS>
__device__ __forceinline__ uint32_t pair_value_reg(const Ctx& c, const Task& t, const PairRegs<BITS, CPL_H>& P,
                                                   const XLane<BITS, CPL_H>& x, float r) {
  float pg = 0.f, pu = 0.f;
  if (c.sr_h < t.n) {
#pragma unroll
    for (int m = 0; m < CPL_H; ++m) pg += chunk_partial<BITS, 1>(P.g[m], P.gs[m], x.w[m], x.s[m], x.w[m], x.s[m]);
#pragma unroll
    for (int m = 0; m < CPL_H; ++m) pu += chunk_partial<BITS, 1>(P.u[m], P.us[m], x.w[m], x.s[m], x.w[m], x.s[m]);
  }
  const float gv = reduce_row(pg, c.lpr_h) * r;
  const float uv = reduce_row(pu, c.lpr_h) * r;
  return split_a(silu_mul(gv, uv));
}
__device__ __forceinline__ void store_pair(const Args& a, const Ctx& c, const Task& t, uint32_t v) {
  if (c.sr_h < t.n && c.li_h == c.lpr_h - 1)
    st_copies(a.x_a + (int64_t)t.slot * c.imax + a_word(t.r0 + c.sr_h, c.imax), c.a_cs, c.n_copy, v, c.ep);
}

// The task's rows of one expert's down projection: the activation vector is
// split and arranged once, then each row group takes rows sr, sr + rpw, ...
// KF: K when known at compile time (0: t.K).
template <int BITS, int CPL, int KF>
__device__ __forceinline__ void down_rows(const Args& a, const Ctx& c, const Task& t, const uint8_t* buf) {
  const int K = KF ? KF : t.K;
  const int lpr = lanes_per_row(K), rpw = 64 / lpr, li = c.lane % lpr, sr = c.lane / lpr;
  XLane<BITS, CPL> xh, xl;
  a_lane<BITS, CPL>(S.a + t.slot * c.imax, K, li, lpr, xh, xl);
  const int cb = code_bytes(BITS, K);
  const uint32_t* sb = (const uint32_t*)(buf + t.n * cb);
  for (int p = 0; p < t.n; p += rpw) {
    const int q = p + sr;
    float v = 0.f;
    if (q < t.n) v = lds_row<BITS, CPL, 2>(buf + q * cb, sb + q * (K >> 6), K, li, lpr, xh, xl);
    v = reduce_row(v, lpr);
    if (q < t.n && li == lpr - 1) S.D[t.slot * c.J + (t.r0 - blockIdx.x * c.J) + q] = v;
  }
}

// ---- phase A: all tasks of the wave fit in the ring (checked on the host),
// from byte `at` of the wave's ring (0, or the second half when phase A is
// requested during the previous layer)
template <int CPL_H, int CPL_I>
__device__ __forceinline__ void phase_a_issue(const Args& a, const Ctx& c, int at) {
  int off = 0;
  const uint32_t base = lds_addr(S.ring[c.wave]) + at;
  for (int i = c.wave; i < n_a_tasks<CPL_H, CPL_I>(a, c); i += kWaves) {
    const Task t = a_task<CPL_H, CPL_I>(a, c, i);
    dma_task(t, base + off);
    off += t.bytes;
  }
}
template <int CPL_H, int CPL_I>
__device__ __forceinline__ int phase_a_bytes(const Args& a, const Ctx& c) {
  int n = 0;
  for (int i = c.wave; i < n_a_tasks<CPL_H, CPL_I>(a, c); i += kWaves) n += a_task<CPL_H, CPL_I>(a, c, i).bytes;
  return n;
}
template <int CPL_H, int CPL_I, int RB, int SB>
__device__ __forceinline__ void phase_a_compute(const Args& a, const Ctx& c, int at) {
  wait_vm(0);
  int off = at;
  for (int i = c.wave; i < n_a_tasks<CPL_H, CPL_I>(a, c); i += kWaves) {
    const Task t = a_task<CPL_H, CPL_I>(a, c, i);
    const uint8_t* buf = S.ring[c.wave] + off;
    if (t.kind == kRouter) {
      MOE_T1_RBITS(RB, c.rbits, B, router_row<CPL_H, CPL_I, B>(a, c, t, buf));
    } else {
      MOE_T1_BITS(SB, c.sbits, B, {
        XLane<B, CPL_H> x;
        h_lane<B, CPL_H>(S.h, c.H, c.li_h, c.lpr_h, x);
        pair_rows<CPL_H, CPL_I, B>(a, c, t, buf, x, -1.f);
      });
    }
    off += t.bytes;
  }
}

// ---- stage h_l into LDS (all threads)
__device__ __forceinline__ void stage_h(const Args& a, const Ctx& c, int l) {
  const int n = c.H >> 1;
  const int tid = threadIdx.x;
  if (l == 0) {
    const uint32_t* h = (const uint32_t*)a.h_in;
    for (int i = tid; i < n; i += kThreads) S.h[i] = h[i];
    return;
  }
  const uint64_t* src = a.x_h + ((l & 1) * c.n_copy + c.cp) * c.h_cs;
  for (int i0 = tid; i0 < n; i0 += 4 * kThreads) {
    uint32_t v[4];
    uint32_t want = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) want |= (i0 + j * kThreads < n ? 1u : 0u) << j;
    poll<4>(src + i0, [](int j) { return (int64_t)j * kThreads; }, want, c.ep - 1, v, a.status);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i0 + j * kThreads < n) S.h[i0 + j * kThreads] = v[j];
  }
}

// ---- routing (c.wave 0): RMS factor and shared gate from h (in the router's
// arrangement, as the per-c.layer kernels compute them), top-k of the logits
// KF: k when known at compile time (0: run time).
template <int CPL_H, int AB, int M, int KF>
__device__ __forceinline__ void route(const Args& a, const Ctx& c, const uint32_t (&gvn)[CPL_H][16]) {
  XLane<AB, CPL_H> x, g;
#pragma unroll
  for (int m = 0; m < CPL_H; ++m) arrange_chunk<AB>(gvn[m], c.li_h + c.lpr_h * m, g.w[m]);
  h_lane<AB, CPL_H>(S.h, c.H, c.li_h, c.lpr_h, x);
  float gd = 0.f;
#pragma unroll
  for (int m = 0; m < CPL_H; ++m)
#pragma unroll
    for (int i = 0; i < XWords<AB>::N; ++i) gd = dot2(x.w[m][i], g.w[m][i], gd);
  const float ss = reduce_row(sumsq(x), c.lpr_h);
  gd = reduce_row(gd, c.lpr_h);
  // row group 0's last c.lane holds the sums
  const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rms_factor(ss, c.H, c.eps)), c.lpr_h - 1));
  gd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gd), c.lpr_h - 1));
  if (c.lane == 0) S.r = r;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // S.r in place before any rank tag
  uint32_t rv[M];
  uint32_t want = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) want |= (c.lane + 64 * m < c.E ? 1u : 0u) << m;
  poll<M>(a.x_logit + c.cp * c.l_cs + c.lane, [](int m) { return (int64_t)64 * m; }, want, c.ep, rv, a.status);
  lds_st(&S.logit_ep, c.ep);
  MOE_TS(3);
  int key[M];
#pragma unroll
  for (int m = 0; m < M; ++m) key[m] = c.lane + 64 * m < c.E ? fkey(r * __uint_as_float(rv[m])) : INT_MIN;
  int my_id;
  float my_w;
  const uint32_t ep = c.ep;
  topk_select<M, KF>(key, c.k, my_id, my_w, [ep](int i, int id) {
    if ((threadIdx.x & 63) == 0) lds_st(&S.rank_tag[i], ep << 16 | (uint32_t)id);
  });
  MOE_TS(4);
  if (c.lane < c.k) {
    S.ids[c.lane] = my_id;
    S.w[c.lane] = my_w;
  }
  if (c.lane == 0) S.sg = 1.0f / (1.0f + expf(-(r * gd)));
}


// ---- the activation vector of one slot into S.a (one wave): every element
// is an epoch-tagged word, stored by the workgroup that computed its pair as
// soon as it was computed; the words are read until all carry this layer's
// epoch (each round re-reads only those that did not). No workgroup-wide
// ready flag is needed, so no wave waits for the others of its workgroup
// before its down rows.
// NV >= K / 64: elements per lane.
template <int NV>
__device__ __forceinline__ void fetch_a(const Args& a, const Ctx& c, int slot) {
  const int K = slot < c.k ? c.I : c.Is;
  const uint64_t* src = a.x_a + c.cp * c.a_cs + (int64_t)slot * c.imax;
  const int imax = c.imax, lane = c.lane;
  auto off = [imax, lane](int j) { return (int64_t)a_word(lane + 64 * j, imax); };
  uint32_t want = 0u;
#pragma unroll
  for (int j = 0; j < NV; ++j) want |= (c.lane + 64 * j < K ? 1u : 0u) << j;
  uint32_t v[NV];
  poll<NV>(src, off, want, c.ep, v, a.status);
  uint32_t* dst = S.a + slot * c.imax;
#pragma unroll
  for (int j = 0; j < NV; ++j)
    if (want >> j & 1u) dst[c.lane + 64 * j] = v[j];
}

// ---- phases B and C: the wave's B tasks then its C tasks, streamed
// through the two ring halves, with the activation exchange between
// KI, KS: routed and shared intermediate sizes when known at compile time
// (0: run time); NV: activation elements per lane of a slot (>= imax / 64).
// Waits until LDS word *p holds epoch (set by another wave of the workgroup).
__device__ __forceinline__ void wait_lds_epoch(const uint32_t* p, uint32_t epoch, uint32_t* status) {
  uint32_t spins = 0;
  while (lds_ld(p) != epoch)
    if (give_up(spins, status)) break;
  asm volatile("" ::: "memory");
}

// The shared expert's down rows of this workgroup's slice. Their weights and
// inputs do not depend on the routing: the last wave streams the rows into
// S.sd right after phase A and reads the shared activations (published in
// phase A) once wave 0 has seen every logit (published after them), all
// while wave 0 routes; S.sd_ep then says they are in place. The rows are
// computed, one task per wave, after each wave's routed pairs.
template <int NV>
__device__ __forceinline__ void shared_down_fetch(const Args& a, const Ctx& c) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint32_t base = lds_addr(S.sd);
  const int tb = s_task(a, c, 0).bytes;
  for (int i = 0; i < n_s_tasks(a, c); ++i) dma_task(s_task(a, c, i), base + i * tb);
  wait_lds_epoch(&S.logit_ep, c.ep, a.status);
  fetch_a<NV>(a, c, c.k);  // its waits also complete the weight loads above
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  lds_st(&S.sd_ep, c.ep);
}
template <int CPL_I, int SB, int KS>
__device__ __forceinline__ void shared_down_part(const Args& a, const Ctx& c) {
  const int tb = s_task(a, c, 0).bytes;
  for (int i = c.wave; i < n_s_tasks(a, c); i += kWaves) {
    const Task t = s_task(a, c, i);
    MOE_T1_BITS(SB, c.sbits, B, down_rows<B, CPL_I, KS>(a, c, t, S.sd + i * tb));
  }
}

// Routed pair tasks per wave that phase B holds in registers (when every wave
// of the workgroup has at most this many)
constexpr int kRegPairs = 2;

// Whether the wave requests each next layer's phase A during the current
// layer (into ring half 1): on the register path of phase B, when the wave's
// C tasks fit in half 0 and its phase A tasks in half 1. Depends on the shape
// only, so it holds for every layer of the launch.
template <int CPL_H, int CPL_I>
__device__ __forceinline__ bool prefetch_mode(const Args& a, const Ctx& c) {
  if constexpr (CPL_H != 1) {
    return false;
  } else {
    if (n_b_tasks<CPL_H, CPL_I>(a, c) > kRegPairs * kWaves) return false;
    const int nc = n_c_tasks(a, c);
    int cb = 0;
    for (int i = c.wave; i < nc; i += kWaves) cb += c_task(a, c, i, [](int) { return 0; }).bytes;
    return cb <= kHalf && phase_a_bytes<CPL_H, CPL_I>(a, c) <= kHalf;
  }
}

// After the wave's routed pairs (whose activations it has stored): the
// shared expert's down rows of the slice, once the last wave has them and
// their inputs in LDS, and the complete routing for the C tasks.
template <int CPL_I, int SB, int KS>
__device__ __forceinline__ void after_b(const Args& a, const Ctx& c) {
  if (c.wave == 0) MOE_TS(8);
  wait_lds_epoch(&S.route_ep, c.ep, a.status);
  wait_lds_epoch(&S.sd_ep, c.ep, a.status);
  shared_down_part<CPL_I, SB, KS>(a, c);
}

// pre: phase A of the next layer (block `next_layer`, null after the launch's
// last layer) is requested into the second ring half after the wave's last
// activation poll (the C tasks then all sit in the first half, see
// prefetch_mode), so that no later wait of this layer waits for it.
template <int CPL_H, int CPL_I, int EB, int SB, int KI, int KS, int NV>
__device__ __forceinline__ void phases_bc(const Args& a, const Ctx& c, bool pre, const uint8_t* next_layer) {
  const int nb = n_b_tasks<CPL_H, CPL_I>(a, c), nc = n_c_tasks(a, c);
  // the wave's tasks: B tasks c.wave, c.wave + 8, ..., then C tasks likewise
  int mb = nb > c.wave ? (nb - c.wave + kWaves - 1) / kWaves : 0;
  const int mc = nc > c.wave ? (nc - c.wave + kWaves - 1) / kWaves : 0;
  // uniform over the workgroup; compiled for one chunk per lane only (the
  // registers of wider rows would make the kernel spill)
  const bool reg_b = CPL_H == 1 && nb <= kRegPairs * kWaves;
  // the register path needs only the ids of its own ranks (as each is
  // chosen); everything else waits for wave 0's complete routing
  if (!reg_b) wait_lds_epoch(&S.route_ep, c.ep, a.status);
  if constexpr (CPL_H == 1) if (reg_b) {
    auto id_of = [&](int u) { return rank_id(a, c, u); };
    // B from registers: the wave's routed pairs are requested at once with
    // global loads (a burst of a few KB per wave arrives about twice as soon
    // that way as through LDS) and computed; only then are the
    // down rows of phase C streamed into the ring, so that no wait for the
    // pairs also waits for them (both complete in issue order).
    MOE_T1_BITS(EB, c.ebits, B, {
      PairRegs<B, CPL_H> P0, P1;
      Task t0, t1;
      if (mb > 0) {
        t0 = b_task<CPL_H, CPL_I>(a, c, c.wave, id_of);
        pair_load<B, CPL_H>(c, t0, P0);
      }
      if (mb > 1) {
        t1 = b_task<CPL_H, CPL_I>(a, c, c.wave + kWaves, id_of);
        pair_load<B, CPL_H>(c, t1, P1);
      }
      if (c.wave == 0) MOE_TS(5);
      XLane<B, CPL_H> x;
      h_lane<B, CPL_H>(S.h, c.H, c.li_h, c.lpr_h, x);
      if (mb > 0) store_pair(a, c, t0, pair_value_reg<CPL_H, CPL_I, B>(c, t0, P0, x, S.r));
      if (mb > 1) store_pair(a, c, t1, pair_value_reg<CPL_H, CPL_I, B>(c, t1, P1, x, S.r));
      if (c.wave == 0) MOE_TS(6);
      if (c.wave == kWaves - 1) MOE_TS(7);
      // the down rows are requested only once these exchange stores have
      // completed: requested while the stores are in flight, they delay the
      // exchange that every workgroup waits for (1,767 against 1,816 tok/s)
      wait_vm(0);
    });
    mb = 0;
  }
  const int m = mb + mc;
  // experts by their rank tags: on the register path the C tasks are
  // requested before the wave knows that the routing is complete
  auto rid = [&](int u) { return rank_id(a, c, u); };
  auto task = [&](int j) {
    return j < mb ? b_task<CPL_H, CPL_I>(a, c, c.wave + kWaves * j, rid) : c_task(a, c, c.wave + kWaves * (j - mb), rid);
  };
  bool exchanged = false;
  const uint32_t base = lds_addr(S.ring[c.wave]);
  // batches of whole tasks in the two halves: tasks [bs, be), bn instructions
  int bs0 = 0, be0 = 0, bn0 = 0, bs1 = 0, be1 = 0, bn1 = 0;
  int next = 0;
  auto fill = [&](int h, int& bs, int& be, int& bn) {
    bs = next;
    bn = 0;
    int off = 0;
    while (next < m) {
      const Task t = task(next);
      if (off + t.bytes > kHalf) break;
      bn += dma_task(t, base + h * kHalf + off);
      off += t.bytes;
      ++next;
    }
    be = next;
  };
  auto prefetch_next = [&]() {
    if (pre && next_layer) {
      Ctx cn = c;
      cn.layer = next_layer;
      phase_a_issue<CPL_H, CPL_I>(a, cn, kHalf);
    }
  };
  fill(0, bs0, be0, bn0);
  fill(1, bs1, be1, bn1);
  if (c.wave == 0) MOE_TS(13);
  if (reg_b) {  // phase B is done; the down rows requested above arrive meanwhile
    after_b<CPL_I, SB, KS>(a, c);
    exchanged = true;
  }
  int fetched = -1;  // slot whose activations this wave holds in S.a
  for (int b = 0;; ++b) {
    const int h = b & 1;
    const int j0 = h ? bs1 : bs0, j1 = h ? be1 : be0;
    if (j0 == j1) break;
    wait_vm(h ? bn0 : bn1);  // the other half's batch was issued after this one
    if (c.wave == 0 && b == 0) MOE_TS(14);
    int off = 0;
    for (int j = j0; j < j1; ++j) {
      if (j == mb && !exchanged) {
        after_b<CPL_I, SB, KS>(a, c);
        exchanged = true;
      }
      const Task t = task(j);
      if (t.kind == kDown && t.slot != fetched) {
        fetch_a<NV>(a, c, t.slot);
        if (c.wave == 0 && fetched < 0) MOE_TS(9);
        fetched = t.slot;
      }
      if (j == m - 1) prefetch_next();  // the wave's last poll is done
      const uint8_t* buf = S.ring[c.wave] + h * kHalf + off;
      if (t.kind == kRoutedPair) {
        MOE_T1_BITS(EB, c.ebits, B, {
          XLane<B, CPL_H> x;
          h_lane<B, CPL_H>(S.h, c.H, c.li_h, c.lpr_h, x);
          pair_rows<CPL_H, CPL_I, B>(a, c, t, buf, x, S.r);
        });
        if (j + 1 == mb) {  // the wave's last routed pair: publish without waiting for the next batch
          after_b<CPL_I, SB, KS>(a, c);
          exchanged = true;
        }
      } else {
        MOE_T1_BITS(EB, c.ebits, B, down_rows<B, CPL_I, KI>(a, c, t, buf));
      }
      off += t.bytes;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // ring reads done before it is refilled
    if (h) fill(1, bs1, be1, bn1);
    else fill(0, bs0, be0, bn0);
  }
  if (!exchanged) after_b<CPL_I, SB, KS>(a, c);
  if (m == 0) prefetch_next();
}

// ---- combine: h_{l+1}[j] = bf16(h_l[j] + sum_i w_i y_i[j] + sg y_s[j])
__device__ __forceinline__ void combine(const Args& a, const Ctx& c, int l) {
  const int j0 = blockIdx.x * c.J;
  uint64_t* th = a.x_h + (int64_t)((l + 1) & 1) * c.n_copy * c.h_cs;
  for (int i = threadIdx.x; i < (c.J >> 1); i += kThreads) {
    const int q = 2 * i, j = j0 + q;
    if (j >= c.H) continue;
    const uint32_t hin = S.h[j >> 1];
    uint32_t o[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float acc = 0.f;
      for (int r = 0; r < c.k; ++r) acc = fmaf(S.w[r], S.D[r * c.J + q + hh], acc);
      acc = fmaf(S.sg, S.D[c.k * c.J + q + hh], acc);
      const float out = __uint_as_float(hh ? (hin & 0xFFFF0000u) : (hin << 16)) + acc;
      o[hh] = f32_to_bf16_rne(out);
    }
    st_copies(th + (j >> 1), c.h_cs, c.n_copy, o[0] | (o[1] << 16), c.ep);
    if (a.h_trace) {
      a.h_trace[(int64_t)l * c.H + j] = (uint16_t)o[0];
      a.h_trace[(int64_t)l * c.H + j + 1] = (uint16_t)o[1];
    }
    if (l == a.n_layers - 1) {
      a.h_out[j] = (uint16_t)o[0];
      a.h_out[j + 1] = (uint16_t)o[1];
    }
  }
}

// ----------------------------------------------------------- kernel shapes
// A shape class gives the chunks per lane CPL_H / CPL_I (template arguments
// of the row code), the code widths RB / EB / SB and experts per lane ME of
// the top-k (0: taken from the arguments at run time), and kFixed: whether
// every dimension, layout offset and the grid split are compile-time
// constants. A fixed shape folds all address arithmetic and bounds checks of
// the kernel into immediates, which keeps its per-layer instruction stream
// small enough to stay in the instruction cache from layer to layer; the
// host launches it only when all its values equal the call's.
template <int CH, int CI>
struct RtShape {
  static constexpr bool kFixed = false;
  static constexpr int k = 0, KI = 0, KS = 0, NV = 32;
  static constexpr int CPL_H = CH, CPL_I = CI, RB = 0, EB = 0, SB = 0, ME = 0;
};

constexpr int cx_lanes(int K) { return K / 32 >= 64 ? 64 : (K / 32 > 32 ? 64 : K / 32 > 16 ? 32 : K / 32 > 8 ? 16 : K / 32 > 4 ? 8 : K / 32 > 2 ? 4 : K / 32 > 1 ? 2 : 1); }
constexpr int cx_cpl(int K) { return (K / 32 + cx_lanes(K) - 1) / cx_lanes(K); }
constexpr int64_t cx_expert_bytes(int bits, int h, int inter) {
  return 2 * matrix_bytes(bits, inter, h) + matrix_bytes(bits, h, inter);
}

template <int H_, int E_, int I_, int Is_, int K_, int RB_, int EB_, int SB_, int NCU>
struct FixedShape {
  static constexpr bool kFixed = true;
  static constexpr int H = H_, E = E_, I = I_, Is = Is_, k = K_, RB = RB_, EB = EB_, SB = SB_;
  static constexpr int CPL_H = cx_cpl(H), CPL_I = cx_cpl(I > Is ? I : Is);
  static constexpr int ME = (E + 63) / 64 <= 1 ? 1 : (E + 63) / 64 <= 2 ? 2 : (E + 63) / 64 <= 4 ? 4 : 8;
  static constexpr int imax = I > Is ? I : Is;
  static constexpr int J0 = (H + NCU - 1) / NCU;
  static constexpr int J = J0 < 2 ? 2 : (J0 + 1) & ~1;
  static constexpr int nwg = (H + J - 1) / J;
  static constexpr int ra = (E + nwg - 1) / nwg, sa = (Is + nwg - 1) / nwg, pb = (K_ * I + nwg - 1) / nwg;
  static constexpr int n_copy = kExchangeCopies;
  static constexpr int NV = (imax + 63) / 64;
  static constexpr int KI = I, KS = Is;
  // layer layout (as moe_layer_layout)
  static constexpr int64_t off_router = 0;
  static constexpr int64_t off_gatevec =
      RB == kDense ? align_up((int64_t)E * H * 2, kAlign) : matrix_bytes(RB, E, H);
  static constexpr int64_t off_shared = off_gatevec + align_up((int64_t)H * 2, kAlign);
  static constexpr int64_t off_shared_up = matrix_bytes(SB, Is, H), off_shared_down = 2 * off_shared_up;
  static constexpr int64_t off_e0 = off_shared + cx_expert_bytes(SB, H, Is);
  static constexpr int64_t e_stride = cx_expert_bytes(EB, H, I);
  static constexpr int64_t off_e_up = matrix_bytes(EB, I, H), off_e_down = 2 * off_e_up;
  // exchange copy strides (as the workspace map)
  static constexpr int64_t h_cs = align_up(H / 2, 512), l_cs = align_up(E, 512),
                           a_cs = align_up((int64_t)(K_ + 1) * imax, 512);
};

template <class SH>
__device__ __forceinline__ void set_dims(const Args& a, Ctx& c) {
  if constexpr (SH::kFixed) {
    c.H = SH::H; c.E = SH::E; c.I = SH::I; c.Is = SH::Is; c.k = SH::k; c.imax = SH::imax;
    c.rbits = SH::RB; c.ebits = SH::EB; c.sbits = SH::SB; c.J = SH::J; c.nwg = SH::nwg;
    c.ra = SH::ra; c.sa = SH::sa; c.pb = SH::pb; c.mE = SH::ME; c.n_copy = SH::n_copy;
    c.off_router = SH::off_router; c.off_gatevec = SH::off_gatevec; c.off_shared = SH::off_shared;
    c.off_shared_up = SH::off_shared_up; c.off_shared_down = SH::off_shared_down; c.off_e0 = SH::off_e0;
    c.e_stride = SH::e_stride; c.off_e_up = SH::off_e_up; c.off_e_down = SH::off_e_down;
    c.h_cs = SH::h_cs; c.l_cs = SH::l_cs; c.a_cs = SH::a_cs;
  } else {
    c.H = a.H; c.E = a.E; c.I = a.I; c.Is = a.Is; c.k = a.k; c.imax = a.imax;
    c.rbits = a.rbits; c.ebits = a.ebits; c.sbits = a.sbits; c.J = a.J; c.nwg = a.nwg;
    c.ra = a.ra; c.sa = a.sa; c.pb = a.pb; c.mE = a.mE; c.n_copy = a.n_copy;
    c.off_router = a.off_router; c.off_gatevec = a.off_gatevec; c.off_shared = a.off_shared;
    c.off_shared_up = a.off_shared_up; c.off_shared_down = a.off_shared_down; c.off_e0 = a.off_e0;
    c.e_stride = a.e_stride; c.off_e_up = a.off_e_up; c.off_e_down = a.off_e_down;
    c.h_cs = a.h_cs; c.l_cs = a.l_cs; c.a_cs = a.a_cs;
  }
  c.eps = a.eps;
}

template <class SH>
__global__ void __launch_bounds__(kThreads) stack1_kernel(Args a) {
  constexpr int CPL_H = SH::CPL_H, CPL_I = SH::CPL_I, RB = SH::RB, EB = SH::EB, SB = SH::SB, ME = SH::ME;
  Ctx c;
  set_dims<SH>(a, c);
  c.lane = threadIdx.x & 63;
  c.wave = threadIdx.x >> 6;
  c.lpr_h = lanes_per_row(c.H);
  c.rpw_h = 64 / c.lpr_h;
  c.li_h = c.lane % c.lpr_h;
  c.sr_h = c.lane / c.lpr_h;
  c.cp = blockIdx.x % c.n_copy;
  if (threadIdx.x == 0) S.route_ep = S.logit_ep = S.sd_ep = 0u;  // ordered before their readers by the barrier below
  if (threadIdx.x < kMaxTopK) {
    S.rank_tag[threadIdx.x] = 0u;
    S.ids[threadIdx.x] = 0;
  }
  if ((int)threadIdx.x < a.n_layers)
    S.layers[threadIdx.x] = (uint64_t)(a.table ? a.table[a.l0 + threadIdx.x] : a.layers[threadIdx.x]);
  lds_barrier();
  auto layer_at = [](int l) {
    const uint64_t lp = S.layers[l];
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)lp);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(lp >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
  };
  c.layer = layer_at(0);
  const bool pre = prefetch_mode<CPL_H, CPL_I>(a, c);
  const int a_at = pre ? kHalf : 0;  // where phase A lands in the wave's ring
  for (int l = 0; l < a.n_layers; ++l) {
#ifdef MOE_PHASE_TRACE
    if (threadIdx.x < kPhases) S.ts[threadIdx.x] = 0u;  // phases a path does not pass stay 0
#endif
    if (c.wave == 0) MOE_TS(0);
    c.layer = layer_at(l);
    c.ep = (uint32_t)l + 1;
    // phase A weights stream in while h_l is polled (requested during the
    // previous layer in prefetch mode)
    if (!pre || l == 0) phase_a_issue<CPL_H, CPL_I>(a, c, a_at);
    uint32_t gvn[CPL_H][16];
    if (c.wave == 0) {
      const uint16_t* gv = (const uint16_t*)(c.layer + c.off_gatevec);
#pragma unroll
      for (int m = 0; m < CPL_H; ++m) {
        const int ch = c.li_h + c.lpr_h * m;
        if (ch < (c.H >> 5)) {
          load64B(gv + 32 * ch, gvn[m]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) gvn[m][i] = 0u;
        }
      }
    }
    stage_h(a, c, l);
    lds_barrier();
    if (c.wave == 0) MOE_TS(1);
    phase_a_compute<CPL_H, CPL_I, RB, SB>(a, c, a_at);
    if (c.wave == 0) {
      MOE_TS(2);
    if constexpr (ME != 0) {
      MOE_T1_RBITS(RB, c.rbits, B, route<CPL_H, B, ME, SH::k>(a, c, gvn));
    } else {
      switch (c.mE) {
        case 1: MOE_T1_RBITS(RB, c.rbits, B, route<CPL_H, B, 1, SH::k>(a, c, gvn)); break;
        case 2: MOE_T1_RBITS(RB, c.rbits, B, route<CPL_H, B, 2, SH::k>(a, c, gvn)); break;
        case 4: MOE_T1_RBITS(RB, c.rbits, B, route<CPL_H, B, 4, SH::k>(a, c, gvn)); break;
        default: MOE_T1_RBITS(RB, c.rbits, B, route<CPL_H, B, 8, SH::k>(a, c, gvn)); break;
      }
    }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // routing stored before its flag
      lds_st(&S.route_ep, c.ep);
    } else if (c.wave == kWaves - 1) {
      shared_down_fetch<SH::NV>(a, c);
      MOE_TS(12);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // phase A ring reads done
    if (blockIdx.x == 0 && threadIdx.x < c.k) {  // wave 0, whose routing is complete
      if (a.ids_out) a.ids_out[(int64_t)l * c.k + threadIdx.x] = S.ids[threadIdx.x];
      if (a.w_out) a.w_out[(int64_t)l * c.k + threadIdx.x] = S.w[threadIdx.x];
    }
    phases_bc<CPL_H, CPL_I, EB, SB, SH::KI, SH::KS, SH::NV>(a, c, pre, l + 1 < a.n_layers ? layer_at(l + 1) : nullptr);
    if (c.wave == 0) MOE_TS(10);
    lds_barrier();
    combine(a, c, l);
    lds_barrier();
#ifdef MOE_PHASE_TRACE
    if (a.phase_ts && threadIdx.x < kPhases) {
      uint64_t* dst = a.phase_ts + ((int64_t)l * kMaxWG + blockIdx.x) * kPhases;
      dst[threadIdx.x] = threadIdx.x == 11 ? __builtin_amdgcn_s_memrealtime() : S.ts[threadIdx.x];
    }
#endif
  }
}

__global__ void clear_words(uint64_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

}  // namespace t1

// ----------------------------------------------------------------- host side
// Compute units of the current device (cached per device id).
static int device_cus(int* dev_out) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  *dev_out = dev;
  int n = dev < kMaxDev ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  if (dev < kMaxDev) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Whether the device can hold `nwg` workgroups of kernel `fn` at once (the
// stack kernel's workgroups wait on each other). Cached per (device, kernel).
static bool co_resident(const void* fn, int slot, int dev, int n_cu, int nwg) {
  constexpr int kMaxDev = 64, kSlots = 8;
  static std::atomic<int> cache[kMaxDev][kSlots];  // blocks per CU + 1, 0 = unknown
  int per_cu = -1;
  if (dev < kMaxDev && slot < kSlots) per_cu = cache[dev][slot].load(std::memory_order_relaxed) - 1;
  if (per_cu < 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, t1::kThreads, 0) != hipSuccess) return false;
    per_cu = nb;
    if (dev < kMaxDev && slot < kSlots) cache[dev][slot].store(nb + 1, std::memory_order_relaxed);
  }
  return (int64_t)per_cu * n_cu >= nwg;
}

int32_t launch_stack_t1(const moe_shape_t& s, const moe_layer_layout_t& L, const WsMap& m, uint8_t* ws,
                        const LayerSrc& layers, int n_layers, int T, const uint16_t* h_in, uint16_t* h_out,
                        int32_t* ids_out, float* w_out, uint16_t* h_trace_out, moe_stream_t stream) {
  using namespace t1;
  if (T != 1) return MOE_ERR_UNSUPPORTED;
  auto bits_streamable = [](int b) { return b == 2 || b == 4 || b == 6 || b == 8; };
  if (!bits_streamable(s.expert_bits) || !bits_streamable(s.shared_bits) ||
      !(bits_streamable(s.router_bits) || s.router_bits == 16))
    return MOE_ERR_UNSUPPORTED;
  if (s.hidden > kMaxH) return MOE_ERR_UNSUPPORTED;
  const int imax = s.inter > s.shared_inter ? s.inter : s.shared_inter;
  if ((int64_t)(s.top_k + 1) * imax > kMaxAWords) return MOE_ERR_UNSUPPORTED;
  const int cpl_h = chunks_per_lane(s.hidden), cpl_i = chunks_per_lane(imax);
  if (cpl_h > 2 || cpl_i > 2) return MOE_ERR_UNSUPPORTED;
  int dev = 0;
  const int n_cu = device_cus(&dev);
  if (n_cu <= 0) return set_error(MOE_ERR_HIP, "cannot query the compute unit count");
  int J = (s.hidden + n_cu - 1) / n_cu;
  J = J < 2 ? 2 : (J + 1) & ~1;
  if (J > 16) return MOE_ERR_UNSUPPORTED;
  const int nwg = (s.hidden + J - 1) / J;
  if (nwg > kMaxWG) return MOE_ERR_UNSUPPORTED;
  // every task must fit in half a ring, and phase A's tasks of one wave in a ring
  const int lpr_h = lanes_per_row(s.hidden), rpw_h = 64 / lpr_h;
  const int ra = (s.n_experts + nwg - 1) / nwg, sa = (s.shared_inter + nwg - 1) / nwg;
  const int router_task = task_bytes(s.router_bits, s.hidden, std::min(rpw_h, ra), false);
  const int shared_task = task_bytes(s.shared_bits, s.hidden, std::min(rpw_h, sa), true);
  const int routed_task = task_bytes(s.expert_bits, s.hidden, rpw_h, true);
  const int down_task = std::max(
      task_bytes(s.expert_bits, s.inter, down_task_rows(J, s.inter, s.expert_bits), false),
      task_bytes(s.shared_bits, s.shared_inter, down_task_rows(J, s.shared_inter, s.shared_bits), false));
  if (std::max(std::max(router_task, shared_task), std::max(routed_task, down_task)) > kHalf)
    return MOE_ERR_UNSUPPORTED;
  const int a_tasks = (ra + rpw_h - 1) / rpw_h + (sa + rpw_h - 1) / rpw_h;
  if ((a_tasks + kWaves - 1) / kWaves * std::max(router_task, shared_task) > kRingBytes) return MOE_ERR_UNSUPPORTED;
  // the shared expert's down rows of a slice fit S.sd
  const int ds = s_task_rows(J, s.shared_inter);
  if ((J + ds - 1) / ds * task_bytes(s.shared_bits, s.shared_inter, ds, false) > kRingBytes)
    return MOE_ERR_UNSUPPORTED;
  const int pb = (s.top_k * s.inter + nwg - 1) / nwg;
  // a slot's activations: at most 32 per lane, from at most 128 workgroups
  if (imax > 32 * 64 || s.inter / pb + 2 > 128) return MOE_ERR_UNSUPPORTED;

  Args a;
  a.H = s.hidden;
  a.E = s.n_experts;
  a.I = s.inter;
  a.Is = s.shared_inter;
  a.k = s.top_k;
  a.imax = imax;
  a.rbits = s.router_bits;
  a.ebits = s.expert_bits;
  a.sbits = s.shared_bits;
  a.eps = s.rms_eps;
  a.off_router = L.router;
  a.off_gatevec = L.gatevec;
  a.off_shared = L.shared;
  a.off_shared_up = L.shared_up;
  a.off_shared_down = L.shared_down;
  a.off_e0 = L.expert0;
  a.e_stride = L.expert_stride;
  a.off_e_up = L.expert_up;
  a.off_e_down = L.expert_down;
  a.nwg = nwg;
  a.J = J;
  a.ra = ra;
  a.sa = sa;
  a.pb = pb;
  a.mE = pow2ceil((a.E + 63) / 64);
  a.x_h = (uint64_t*)(ws + m.x_h);
  a.x_logit = (uint64_t*)(ws + m.x_logit);
  a.x_a = (uint64_t*)(ws + m.x_a);
  a.h_cs = m.xh_cs;
  a.l_cs = m.xl_cs;
  a.a_cs = m.xa_cs;
  a.n_copy = m.n_copy;
  a.status = (uint32_t*)(ws + m.status);
  a.phase_ts = m.phase_ts >= 0 ? (uint64_t*)(ws + m.phase_ts) : nullptr;
  // the kernel instance: one specialised for the whole shape (35B-A3B and
  // 397B-A17B layers, the tiny bf16-router layer) when every value matches,
  // else a generic one
  void (*launch)(const Args&, hipStream_t) = nullptr;
  const void* fn = nullptr;
  int slot = 0;
  auto matches = [&](auto shape) {
    using SH = decltype(shape);
    return SH::H == a.H && SH::E == a.E && SH::I == a.I && SH::Is == a.Is && SH::k == a.k && SH::RB == a.rbits &&
           SH::EB == a.ebits && SH::SB == a.sbits && SH::J == a.J && SH::nwg == a.nwg && SH::ra == a.ra &&
           SH::sa == a.sa && SH::pb == a.pb && SH::ME == a.mE && SH::n_copy == a.n_copy && SH::imax == a.imax &&
           SH::off_router == a.off_router && SH::off_gatevec == a.off_gatevec && SH::off_shared == a.off_shared &&
           SH::off_shared_up == a.off_shared_up && SH::off_shared_down == a.off_shared_down &&
           SH::off_e0 == a.off_e0 && SH::e_stride == a.e_stride && SH::off_e_up == a.off_e_up &&
           SH::off_e_down == a.off_e_down && SH::h_cs == a.h_cs && SH::l_cs == a.l_cs && SH::a_cs == a.a_cs &&
           SH::CPL_H == cpl_h && SH::CPL_I == cpl_i;
  };
  using A3B = FixedShape<2048, 256, 512, 512, 8, 8, 6, 8, 256>;
  using A17B = FixedShape<4096, 512, 1024, 1024, 10, 8, 4, 4, 256>;
  using Tiny = FixedShape<256, 16, 128, 128, 2, 16, 4, 4, 256>;
  using R11 = RtShape<1, 1>;
  using R21 = RtShape<2, 1>;
  using R12 = RtShape<1, 2>;
  using R22 = RtShape<2, 2>;
#define MOE_T1_PICK(SHAPE, SLOT)                                                                           \
  do {                                                                                                    \
    launch = [](const Args& x, hipStream_t q) { stack1_kernel<SHAPE><<<x.nwg, kThreads, 0, q>>>(x); };   \
    fn = (const void*)stack1_kernel<SHAPE>;                                                               \
    slot = SLOT;                                                                                          \
  } while (0)
  if (matches(A3B())) {
    MOE_T1_PICK(A3B, 0);
  } else if (matches(A17B())) {
    MOE_T1_PICK(A17B, 1);
  } else if (matches(Tiny())) {
    MOE_T1_PICK(Tiny, 2);
  } else if (cpl_h == 1 && cpl_i == 1) {
    MOE_T1_PICK(R11, 3);
  } else if (cpl_h == 2 && cpl_i == 1) {
    MOE_T1_PICK(R21, 4);
  } else if (cpl_h == 1) {
    MOE_T1_PICK(R12, 5);
  } else {
    MOE_T1_PICK(R22, 6);
  }
#undef MOE_T1_PICK
  // every workgroup must be resident at once: otherwise the caller runs the
  // stack layer by layer
  if (!co_resident(fn, slot, dev, n_cu, nwg)) return MOE_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  const int64_t H = s.hidden, k = s.top_k;
  uint16_t* hb = (uint16_t*)(ws + m.hbuf);
  const uint16_t* cur = h_in;
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayersPerLaunch) {
    const int nl = n_layers - l0 < kMaxLayersPerLaunch ? n_layers - l0 : kMaxLayersPerLaunch;
    const bool last = l0 + nl == n_layers;
    a.n_layers = nl;
    a.table = layers.table;
    a.l0 = l0;
    for (int l = 0; l < nl; ++l) a.layers[l] = (const uint8_t*)layers.at(l0 + l);
    a.h_in = cur;
    a.h_out = last ? h_out : hb + ((l0 / kMaxLayersPerLaunch) & 1) * H;
    a.ids_out = ids_out ? ids_out + (int64_t)l0 * k : nullptr;
    a.w_out = w_out ? w_out + (int64_t)l0 * k : nullptr;
    a.h_trace = h_trace_out ? h_trace_out + (int64_t)(l0 + 1) * H : nullptr;
    // zero the exchange words (no stale epoch can match), and the status
    // word only before the first launch: a time-out in any launch of the
    // call stays reported (and makes the later launches' waits give up at once)
    int64_t cb, ce;
    clear_range(m, l0 == 0, &cb, &ce);
    clear_words<<<64, 256, 0, st>>>((uint64_t*)(ws + cb), (ce - cb) / 8);
    launch(a, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "stack kernel launch failed: %s", hipGetErrorString(e));
    cur = a.h_out;
  }
  return MOE_OK;
}

}  // namespace moe
