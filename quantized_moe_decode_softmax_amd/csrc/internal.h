// Internal declarations shared by the host code and the HIP sources of the
// library. Not part of the public ABI (include/moe_decode.h is).
#pragma once

#include <stdint.h>
#include <stddef.h>

#include "moe_decode.h"

// Layout arithmetic is used by host code (g++) and by kernels (hipcc).
#ifdef __HIPCC__
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

constexpr int kGroup = 64;
constexpr int kMaxT = 32;
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 512;
constexpr int kMaxDim = 8192;
constexpr int kMaxLayersPerLaunch = 64;
constexpr int kMaxLayers = 4096;
constexpr uint32_t kStackMagic = 0x4D4F4553u;  // marks a moe_stack_t filled by moe_stack_init
constexpr int64_t kAlign = 256;
// copies of each exchange buffer of the streaming stack kernel: a writer
// stores every copy, workgroup w polls copy w % kExchangeCopies. Two measured
// best at 256 workgroups (1, 2, 4, 8 and 16 were tried): fewer pollers per
// line than one copy, fewer stores per word than more.
constexpr int kExchangeCopies = 2;

MOE_HD constexpr inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// bytes of one row of codes
MOE_HD constexpr inline int64_t row_bytes(int bits, int cols) {
  if (bits == 3) return 4 * (((int64_t)cols + 9) / 10);
  return (int64_t)cols * bits / 8;
}
MOE_HD constexpr inline bool bits_ok(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 6 || bits == 8; }

// offsets inside one packed matrix block
MOE_HD constexpr inline int64_t matrix_codes_bytes(int bits, int rows, int cols) { return align_up(row_bytes(bits, cols) * rows, kAlign); }
MOE_HD constexpr inline int64_t matrix_sb_bytes(int rows, int cols) { return align_up((int64_t)rows * (cols / kGroup) * 4, kAlign); }
MOE_HD constexpr inline int64_t matrix_bytes(int bits, int rows, int cols) {
  return matrix_codes_bytes(bits, rows, cols) + matrix_sb_bytes(rows, cols);
}

// Workspace map (all offsets 256-aligned). T rows, up to U = min(T*k, E)
// unique routed experts per call.
struct WsMap {
  int64_t raw_logits;   // float [T][E]  router dot products with h (before the RMS factor)
  int64_t rinv;         // float [T]     1/sqrt(mean(h^2)+eps)
  int64_t sgate;        // float [T]     sigmoid gate of the shared expert
  int64_t ids;          // int32 [T][k]
  int64_t wts;          // float [T][k]
  int64_t units;        // int32 [1 + U] count, then expert ids of the unique units (ascending)
  int64_t masks;        // uint32 [U]   rows using each unit
  int64_t tmask;        // uint32 [T][k] rows using the expert selected at (row, slot)
  int64_t a_hi;         // bf16  [T][k+1][Imax]  SwiGLU activations, high part
  int64_t a_lo;         // bf16  [T][k+1][Imax]  low part: a = hi + lo to 16 significant bits
  int64_t hbuf;         // bf16  [2][T][H] ping-pong for stacks
  int64_t ysh;          // float [T][H]  shared expert's down projection (matrix-core path)
  int64_t hpack;        // bf16 [T16][H] packed h (matrix-core path; T16 = T rounded up to 16)
  int64_t apack;        // bf16 [2][T16][Is] packed shared activations, hi then lo (matrix-core path)
  // one-row streaming stack kernel (stack1.hip): exchange buffers of 64-bit
  // words = 32-bit payload | epoch << 32, each in n_copy copies (stride *_cs
  // words) that writers all store and workgroup w reads copy w % n_copy
  int n_copy;
  int64_t x_h;          // u64 [2][n_copy][H/2]      hidden state by layer parity
  int64_t x_logit;      // u64 [n_copy][E]           raw router dot products
  int64_t x_a;          // u64 [n_copy][k+1][Imax]   activations, bf16 hi | bf16 lo << 16
  int64_t xh_cs, xl_cs, xa_cs;
  int64_t status;       // u32 [64]           word 0: nonzero after a timed-out wait
  int64_t x_end;        // end of the region the streaming kernel clears per call
  // per-phase timestamps of the streaming kernel, u64 [64 layers][512 workgroups][16]
  // (phase-trace builds only; -1 otherwise)
  int64_t phase_ts;
  int64_t total;
};

WsMap ws_map(const moe_shape_t& s, int T);
// Byte range [begin, end) of the workspace that the streaming stack kernel's
// clear kernel zeroes before a launch: every exchange word, and the status
// word only before the first launch of a call.
MOE_HD inline void clear_range(const WsMap& m, bool first_launch, int64_t* begin, int64_t* end) {
  *begin = m.x_h;
  *end = first_launch ? m.x_end : m.status;
}
// bytes of the descriptor table of n layer pointers (placed after the map of
// the stack's largest T)
MOE_HD constexpr inline int64_t table_bytes(int n) { return align_up((int64_t)n * 8, kAlign); }

// thread-local error reporting
int32_t set_error(int32_t code, const char* fmt, ...);
void clear_error();
// MOE_DEBUG_SYNC=1 in the environment (read once): launching entry points
// wait for their stream and report HIP errors and wait time-outs
bool debug_sync();
// With MOE_DEBUG_SYNC=1: wait for the stream, MOE_ERR_HIP on a HIP error;
// else MOE_OK at once (device code files only).
int32_t debug_finish(moe_stream_t st);

int32_t check_shape(const moe_shape_t* s);

void layout_of(const moe_shape_t& s, moe_layer_layout_t* out);

// One-row stack decode with the streaming kernel (stack1.hip).
// MOE_ERR_UNSUPPORTED, with nothing launched, for calls it does not handle.
// Where a stack call finds its layer blocks: a host array of device pointers
// (moe_decode_stack) or the descriptor table in the workspace (moe_stack_init).
struct LayerSrc {
  const void* const* host;         // or nullptr
  const uint8_t* const* table;     // device, or nullptr
  const void* at(int l) const { return host ? host[l] : nullptr; }
};

// One-row stack decode with the streaming kernel (stack1.hip).
// MOE_ERR_UNSUPPORTED, with nothing launched, for calls it does not handle
// (also when the device cannot hold all of its workgroups at once).
int32_t launch_stack_t1(const moe_shape_t& s, const moe_layer_layout_t& L, const WsMap& m, uint8_t* ws,
                        const LayerSrc& layers, int n_layers, int T, const uint16_t* h_in, uint16_t* h_out,
                        int32_t* ids_out, float* w_out, uint16_t* h_trace_out, moe_stream_t st);

// moe_decode_stack after clear_error(): validation, then the launches, on the
// given workspace (also the static scratch of the allocation-free variant).
int32_t decode_stack_ws(const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers, int32_t T,
                        const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev, float* w_dev,
                        uint16_t* h_trace_dev, void* ws_dev, size_t ws_bytes, moe_stream_t stream);

}  // namespace moe

#ifdef MOE_PHASE_TRACE
// Phase-trace builds only: byte offset of the timestamp region in a workspace
// for T rows (layout [layer of the last launch][workgroup][16] u64).
extern "C" int64_t moe_phase_trace_offset(const moe_shape_t* shape, int32_t T);
#endif

// Host-only test hook (not part of the ABI): out = {clear begin, clear end,
// status offset, map total} for the shape, T and launch position.
extern "C" int32_t moe_internal_clear_range(const moe_shape_t* shape, int32_t T, int32_t first_launch, int64_t* out);
