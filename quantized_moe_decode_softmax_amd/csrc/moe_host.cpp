// Host-side part of the library: shape validation, layer layout, workspace
// sizing, matrix packing/unpacking and error reporting. Plain C++; no HIP
// call is made here, so every function in this file works without a GPU.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "internal.h"

namespace moe {

static thread_local char g_err[512] = "";

int32_t set_error(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

bool debug_sync() {
  static const bool on = [] {
    const char* v = getenv("MOE_DEBUG_SYNC");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}

static bool dim_ok(int v) { return v >= kGroup && v <= kMaxDim && v % kGroup == 0; }

int32_t check_shape(const moe_shape_t* s) {
  if (!s) return set_error(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->group != kGroup) return set_error(MOE_ERR_UNSUPPORTED, "group %d not supported (must be 64)", s->group);
  if (!dim_ok(s->hidden)) return set_error(MOE_ERR_UNSUPPORTED, "hidden %d must be a multiple of 64 in [64, %d]", s->hidden, kMaxDim);
  if (!dim_ok(s->inter)) return set_error(MOE_ERR_UNSUPPORTED, "inter %d must be a multiple of 64 in [64, %d]", s->inter, kMaxDim);
  if (!dim_ok(s->shared_inter))
    return set_error(MOE_ERR_UNSUPPORTED, "shared_inter %d must be a multiple of 64 in [64, %d]", s->shared_inter, kMaxDim);
  if (s->n_experts < 1 || s->n_experts > kMaxExperts)
    return set_error(MOE_ERR_INVALID_ARG, "n_experts %d must be in [1, %d]", s->n_experts, kMaxExperts);
  if (s->top_k < 1 || s->top_k > s->n_experts || s->top_k > kMaxTopK)
    return set_error(MOE_ERR_INVALID_ARG, "top_k %d must be in [1, min(n_experts, %d)]", s->top_k, kMaxTopK);
  if (!bits_ok(s->expert_bits)) return set_error(MOE_ERR_UNSUPPORTED, "expert_bits %d not in {2,3,4,6,8}", s->expert_bits);
  if (!bits_ok(s->shared_bits)) return set_error(MOE_ERR_UNSUPPORTED, "shared_bits %d not in {2,3,4,6,8}", s->shared_bits);
  if (!(bits_ok(s->router_bits) || s->router_bits == 16))
    return set_error(MOE_ERR_UNSUPPORTED, "router_bits %d not in {2,3,4,6,8,16}", s->router_bits);
  if (!(s->rms_eps > 0.0f) || !(s->rms_eps < 1.0f)) return set_error(MOE_ERR_INVALID_ARG, "rms_eps must be in (0, 1)");
  return MOE_OK;
}

static int64_t expert_block(int bits, int h, int inter, int64_t* up, int64_t* down) {
  int64_t g = matrix_bytes(bits, inter, h);
  *up = g;
  *down = 2 * g;
  return 2 * g + matrix_bytes(bits, h, inter);
}

void layout_of(const moe_shape_t& s, moe_layer_layout_t* o) {
  int64_t off = 0;
  o->router = off;
  off += s.router_bits == 16 ? align_up((int64_t)s.n_experts * s.hidden * 2, kAlign)
                             : matrix_bytes(s.router_bits, s.n_experts, s.hidden);
  o->gatevec = off;
  off += align_up((int64_t)s.hidden * 2, kAlign);
  o->shared = off;
  off += expert_block(s.shared_bits, s.hidden, s.shared_inter, &o->shared_up, &o->shared_down);
  o->expert0 = off;
  o->expert_stride = expert_block(s.expert_bits, s.hidden, s.inter, &o->expert_up, &o->expert_down);
  off += o->expert_stride * s.n_experts;
  o->total_bytes = off;
}

WsMap ws_map(const moe_shape_t& s, int T) {
  WsMap m;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    int64_t o = off;
    off += align_up(bytes, kAlign);
    return o;
  };
  const int k = s.top_k;
  const int64_t U = (int64_t)T * k < s.n_experts ? (int64_t)T * k : s.n_experts;
  const int64_t imax = s.inter > s.shared_inter ? s.inter : s.shared_inter;
  m.raw_logits = take((int64_t)T * s.n_experts * 4);
  m.rinv = take((int64_t)T * 4);
  m.sgate = take((int64_t)T * 4);
  m.ids = take((int64_t)T * k * 4);
  m.wts = take((int64_t)T * k * 4);
  m.units = take((1 + U) * 4);
  m.masks = take(U * 4);
  m.tmask = take((int64_t)T * k * 4);
  m.a_hi = take((int64_t)T * (k + 1) * imax * 2);
  m.a_lo = take((int64_t)T * (k + 1) * imax * 2);
  m.hbuf = take((int64_t)2 * T * s.hidden * 2);
  m.ysh = take((int64_t)T * s.hidden * 4);
  const int64_t t16 = ((int64_t)T + 15) / 16 * 16;
  m.hpack = take(t16 * s.hidden * 2);
  m.apack = take(2 * t16 * s.shared_inter * 2);
  m.n_copy = kExchangeCopies;
  m.xh_cs = align_up(s.hidden / 2, 512);
  m.xl_cs = align_up(s.n_experts, 512);
  m.xa_cs = align_up((int64_t)(k + 1) * imax, 512);
  m.x_h = take(2 * m.n_copy * m.xh_cs * 8);
  m.x_logit = take(m.n_copy * m.xl_cs * 8);
  m.x_a = take(m.n_copy * m.xa_cs * 8);
  m.status = take(64 * 4);
  m.x_end = off;
#ifdef MOE_PHASE_TRACE
  m.phase_ts = take((int64_t)kMaxLayersPerLaunch * 512 * 16 * 8);
#else
  m.phase_ts = -1;
#endif
  m.total = off;
  return m;
}

// ------------------------------------------------------------------ packing
static void put_bits(uint8_t* row, int64_t bit, uint32_t v, int nbits) {
  for (int b = 0; b < nbits; ++b, ++bit)
    if (v >> b & 1u) row[bit >> 3] |= (uint8_t)(1u << (bit & 7));
}
static uint32_t get_bits(const uint8_t* row, int64_t bit, int nbits) {
  uint32_t v = 0;
  for (int b = 0; b < nbits; ++b, ++bit) v |= (uint32_t)(row[bit >> 3] >> (bit & 7) & 1u) << b;
  return v;
}

// bit position (inside the row) of bit `b` of code j, for each layout
static int64_t code_bit(int bits, int64_t j, int b) {
  if (bits == 6) {
    // unit of 16 codes in dwords A, B, C; code c = jj + 8h sits in half h
    const int64_t u = j / 16;
    const int c = (int)(j % 16), h = c / 8, jj = c % 8;
    const int64_t base = u * 96 + 16 * h;
    int word, rel;
    switch (jj) {
      case 0: case 1: word = 0; rel = 6 * jj + b; break;
      case 3: case 4: word = 1; rel = 6 * (jj - 3) + b; break;
      case 6: case 7: word = 2; rel = 6 * (jj - 6) + b; break;
      case 2: word = b < 4 ? 0 : 2; rel = b < 4 ? 12 + b : 12 + (b - 4); break;
      default: word = b < 4 ? 1 : 2; rel = b < 4 ? 12 + b : 14 + (b - 4); break;  // jj == 5
    }
    return base + 32 * word + rel;
  }
  if (bits == 3) {  // slot l < 5 at bit 3l, slot l >= 5 at bit 16 + 3(l - 5)
    const int l = (int)(j % 10);
    return 32 * (j / 10) + (l < 5 ? 3 * l : 16 + 3 * (l - 5)) + b;
  }
  return (int64_t)bits * j + b;
}

static int32_t check_pack_args(int32_t bits, int32_t rows, int32_t cols, const void* a, const void* b, const void* c,
                               const void* d) {
  if (!bits_ok(bits)) return set_error(MOE_ERR_UNSUPPORTED, "bits %d not in {2,3,4,6,8}", bits);
  if (rows < 1 || cols < kGroup || cols % kGroup != 0)
    return set_error(MOE_ERR_INVALID_ARG, "rows %d / cols %d invalid (cols a positive multiple of 64)", rows, cols);
  if (!a || !b || !c || !d) return set_error(MOE_ERR_INVALID_ARG, "NULL buffer");
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_matrix_bytes(int32_t bits, int32_t rows, int32_t cols) {
  clear_error();
  if (!bits_ok(bits)) return set_error(MOE_ERR_UNSUPPORTED, "bits %d not in {2,3,4,6,8}", bits);
  if (rows < 1 || cols < kGroup || cols % kGroup != 0) return set_error(MOE_ERR_INVALID_ARG, "rows/cols invalid");
  return matrix_bytes(bits, rows, cols);
}

int32_t moe_validate_shape(const moe_shape_t* shape) {
  clear_error();
  return check_shape(shape);
}

int32_t moe_layer_layout(const moe_shape_t* shape, moe_layer_layout_t* out) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (!out) return set_error(MOE_ERR_INVALID_ARG, "out is NULL");
  layout_of(*shape, out);
  return MOE_OK;
}

int32_t moe_validate(const moe_shape_t* shape, int32_t T) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  return MOE_OK;
}

int64_t moe_expert_bytes(const moe_shape_t* shape) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  moe_layer_layout_t L;
  layout_of(*shape, &L);
  return L.expert_stride;
}

int64_t moe_layer_bytes(const moe_shape_t* shape) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  moe_layer_layout_t L;
  layout_of(*shape, &L);
  return L.total_bytes;
}

int64_t moe_workspace_bytes(const moe_shape_t* shape, int32_t n_layers, int32_t T) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  if (n_layers < 0 || n_layers > kMaxLayers)
    return set_error(MOE_ERR_INVALID_ARG, "n_layers %d not in [0, %d]", n_layers, kMaxLayers);
  return ws_map(*shape, T).total + table_bytes(n_layers);
}

int32_t moe_pack_matrix(int32_t bits, int32_t rows, int32_t cols, const uint8_t* codes, const uint16_t* scale,
                        const uint16_t* bias, void* dst) {
  clear_error();
  int32_t rc = check_pack_args(bits, rows, cols, codes, scale, bias, dst);
  if (rc) return rc;
  const int64_t total = matrix_bytes(bits, rows, cols);
  uint8_t* out = (uint8_t*)dst;
  memset(out, 0, (size_t)total);
  const int64_t rb = row_bytes(bits, cols);
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t* row = out + r * rb;
    for (int64_t j = 0; j < cols; ++j) {
      uint32_t c = codes[r * cols + j];
      if (c >> bits) return set_error(MOE_ERR_INVALID_ARG, "code %u at (%lld, %lld) does not fit in %d bits", c, (long long)r, (long long)j, bits);
      for (int b = 0; b < bits; ++b)
        if (c >> b & 1u) put_bits(row, code_bit(bits, j, b), 1u, 1);
    }
  }
  uint32_t* sb = (uint32_t*)(out + matrix_codes_bytes(bits, rows, cols));
  const int64_t ng = cols / kGroup;
  for (int64_t i = 0; i < (int64_t)rows * ng; ++i) sb[i] = (uint32_t)scale[i] | (uint32_t)bias[i] << 16;
  return MOE_OK;
}

int32_t moe_unpack_matrix(int32_t bits, int32_t rows, int32_t cols, const void* src, uint8_t* codes, uint16_t* scale,
                          uint16_t* bias) {
  clear_error();
  int32_t rc = check_pack_args(bits, rows, cols, src, codes, scale, bias);
  if (rc) return rc;
  const uint8_t* in = (const uint8_t*)src;
  const int64_t rb = row_bytes(bits, cols);
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* row = in + r * rb;
    for (int64_t j = 0; j < cols; ++j) {
      uint32_t c = 0;
      for (int b = 0; b < bits; ++b) c |= get_bits(row, code_bit(bits, j, b), 1) << b;
      codes[r * cols + j] = (uint8_t)c;
    }
  }
  const uint32_t* sb = (const uint32_t*)(in + matrix_codes_bytes(bits, rows, cols));
  const int64_t ng = cols / kGroup;
  for (int64_t i = 0; i < (int64_t)rows * ng; ++i) {
    scale[i] = (uint16_t)(sb[i] & 0xFFFFu);
    bias[i] = (uint16_t)(sb[i] >> 16);
  }
  return MOE_OK;
}

int32_t moe_internal_clear_range(const moe_shape_t* shape, int32_t T, int32_t first_launch, int64_t* out) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (T < 1 || T > kMaxT || !out) return set_error(MOE_ERR_INVALID_ARG, "bad T or out");
  const WsMap m = ws_map(*shape, T);
  clear_range(m, first_launch != 0, &out[0], &out[1]);
  out[2] = m.status;
  out[3] = m.total;
  return MOE_OK;
}

#ifdef MOE_PHASE_TRACE
int64_t moe_phase_trace_offset(const moe_shape_t* shape, int32_t T) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  return ws_map(*shape, T).phase_ts;
}
#endif

const char* moe_last_error(void) { return g_err; }

const char* moe_version(void) {
  return debug_sync() ? "moe-decode-gfx950 0.2 debug-sync" : "moe-decode-gfx950 0.2";
}

}  // extern "C"
