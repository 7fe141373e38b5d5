// Seeded synthetic weights and activations, written on the GPU directly in the
// packed layout of include/moe_decode.h.
//
// The generator is a stateless splitmix64 counter hash (Steele, Lea & Flood,
// OOPSLA 2014):
//   mix64(s)         = first splitmix64 output from state s
//   sub(layer, slot) = mix64(seed ^ mix64(layer * 2^20 + slot))
//                      slot: routed expert e -> e, shared expert -> E,
//                      router -> E + 1, shared gate vector -> E + 2
//   draw(i)          = mix64(sub ^ ((3 * tensor + field) * 2^48 + i))
//                      tensor: gate 0, up 1, down 2, router 3, gate vector 4,
//                      x rows 5; field: code 0, scale 1, bias 2
// Codes are the top `bits` bits of the draw at index row*cols + col.
// The scale of (row, group) is bf16(f32(U * C)), U = 0.5 + ((draw >> 40) +
// 0.5) * 2^-24 from the draw at row*(cols/64) + group, C = 1 / (2^(bits-1) *
// sqrt(cols)) computed on the host in fp64.
// The bias is bf16(f32((0.1 * s) * z - m * s)) with s the bf16 scale, m =
// (2^bits - 1) / 2 and z an Irwin-Hall(12) variate: the twelve 16-bit lanes L
// of the three draws 3i, 3i+1, 3i+2 give z = (sum L + 6 - 6 * 2^16) / 2^16.
// bf16 vectors (gate vector, a dense bf16 router, x rows) are bf16(f32(z *
// sigma)) with z from the three code-field draws 3i..3i+2 and sigma = 1 /
// sqrt(H) (host fp64), or 1 for x. x rows use the sub-seed
// mix64(seed_x ^ mix64(0x785F726F7773)).
// Every fp64 operation is an explicitly rounded one (no contraction), every
// conversion rounds to nearest even, so the result is bit-reproducible.
#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr uint64_t kXTag = 0x785F726F7773ull;
enum { kGate = 0, kUp = 1, kDown = 2, kRouter = 3, kGateVec = 4, kX = 5 };
enum { kCode = 0, kScale = 1, kBias = 2 };

__device__ __forceinline__ uint64_t sub_seed(uint64_t seed, int layer, int slot) {
  return mix64(seed ^ mix64(((uint64_t)layer << 20) + (uint64_t)slot));
}
__device__ __forceinline__ uint64_t draw(uint64_t sub, int tensor, int field, uint64_t idx) {
  return mix64(sub ^ (((uint64_t)(3 * tensor + field) << 48) + idx));
}
__device__ __forceinline__ uint32_t code_of(uint64_t sub, int tensor, uint64_t idx, int bits) {
  return (uint32_t)(draw(sub, tensor, kCode, idx) >> (64 - bits));
}
__device__ __forceinline__ double irwin_hall(uint64_t sub, int tensor, int field, uint64_t i) {
  int64_t s = 0;
  for (int j = 0; j < 3; ++j) {
    uint64_t d = draw(sub, tensor, field, 3 * i + j);
    s += (int64_t)(d & 0xFFFF) + (int64_t)(d >> 16 & 0xFFFF) + (int64_t)(d >> 32 & 0xFFFF) + (int64_t)(d >> 48);
  }
  return (double)(s + 6 - 6 * 65536) / 65536.0;  // exact: |numerator| < 2^20
}
__device__ __forceinline__ uint32_t f64_to_bf16(double v) { return f32_to_bf16_rne((float)v); }

// One thread per packed word of codes (bits 2/3/4/8: one dword; bits 6: one
// 16-code unit of 3 dwords). blockIdx.y selects the matrix (slot0 + y).
__global__ void gen_codes_kernel(uint8_t* base, int64_t mat_stride, int bits, int rows, int cols, uint64_t seed,
                                 int layer, int slot0, int tensor) {
  const int m = blockIdx.y;
  const uint64_t sub = sub_seed(seed, layer, slot0 + m);
  uint32_t* out = (uint32_t*)(base + (int64_t)m * mat_stride);
  int64_t words_per_row;
  if (bits == 6) words_per_row = cols / 16;
  else if (bits == 3) words_per_row = (cols + 9) / 10;
  else words_per_row = (int64_t)cols * bits / 32;
  const int64_t n = words_per_row * rows;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < n; w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = w / words_per_row, q = w % words_per_row;
    const uint64_t row0 = (uint64_t)r * cols;
    if (bits == 6) {
      // dwords A, B, C of the unit; code c = j + 8h goes to half h (bit 16h)
      uint32_t wa = 0, wb = 0, wc = 0;
      for (int c = 0; c < 16; ++c) {
        const uint32_t v = code_of(sub, tensor, row0 + q * 16 + c, 6);
        const int h = 16 * (c >> 3), j = c & 7;
        if (j < 2) wa |= v << (h + 6 * j);
        else if (j == 2) { wa |= (v & 15u) << (h + 12); wc |= (v >> 4) << (h + 12); }
        else if (j < 5) wb |= v << (h + 6 * (j - 3));
        else if (j == 5) { wb |= (v & 15u) << (h + 12); wc |= (v >> 4) << (h + 14); }
        else wc |= v << (h + 6 * (j - 6));
      }
      uint32_t* o = out + 3 * w;
      o[0] = wa;
      o[1] = wb;
      o[2] = wc;
    } else if (bits == 3) {
      uint32_t acc = 0;
      for (int c = 0; c < 10; ++c) {
        const int64_t j = q * 10 + c;
        if (j < cols) acc |= code_of(sub, tensor, row0 + j, 3) << (c < 5 ? 3 * c : 16 + 3 * (c - 5));
      }
      out[w] = acc;
    } else {
      const int per = 32 / bits;
      uint32_t acc = 0;
      for (int c = 0; c < per; ++c) acc |= code_of(sub, tensor, row0 + q * per + c, bits) << (bits * c);
      out[w] = acc;
    }
  }
}

// One thread per (row, group): scale | bias << 16.
__global__ void gen_sb_kernel(uint8_t* base, int64_t mat_stride, int bits, int rows, int cols, double cscale,
                              uint64_t seed, int layer, int slot0, int tensor) {
  const int m = blockIdx.y;
  const uint64_t sub = sub_seed(seed, layer, slot0 + m);
  uint32_t* out = (uint32_t*)(base + (int64_t)m * mat_stride);
  const int64_t n = (int64_t)rows * (cols / kGroup);
  const double mb = (double)((1 << bits) - 1) / 2.0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t d = draw(sub, tensor, kScale, (uint64_t)i);
    const double u = 0.5 + ((double)(d >> 40) + 0.5) * 0x1p-24;  // exact
    const uint32_t sbits = f64_to_bf16(__dmul_rn(u, cscale));
    const double s = (double)bf16_lo_to_f32(sbits);
    const double z = irwin_hall(sub, tensor, kBias, (uint64_t)i);
    double t = __dmul_rn(0.1, s);
    t = __dmul_rn(t, z);
    const double beta = __dsub_rn(t, __dmul_rn(mb, s));
    out[i] = sbits | f64_to_bf16(beta) << 16;
  }
}

// bf16 vector values z * sigma; one thread per value.
__global__ void gen_vec_kernel(uint16_t* out, int64_t n, double sigma, uint64_t sub, int tensor) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const double z = irwin_hall(sub, tensor, kCode, (uint64_t)i);
    out[i] = (uint16_t)f64_to_bf16(__dmul_rn(z, sigma));
  }
}

__global__ void gen_vec_sub_kernel(uint16_t* out, int64_t n, double sigma, uint64_t seed, int layer, int slot,
                                   int tensor) {
  const uint64_t sub = sub_seed(seed, layer, slot);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const double z = irwin_hall(sub, tensor, kCode, (uint64_t)i);
    out[i] = (uint16_t)f64_to_bf16(__dmul_rn(z, sigma));
  }
}

uint64_t host_mix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65535) g = 65535;
  if (g < 1) g = 1;
  return (int)g;
}

int32_t gen_matrix(uint8_t* base, int64_t mat_stride, int n_mats, int bits, int rows, int cols, uint64_t seed,
                   int layer, int slot0, int tensor, hipStream_t st) {
  int64_t words_per_row = bits == 6 ? cols / 16 : bits == 3 ? (cols + 9) / 10 : (int64_t)cols * bits / 32;
  dim3 g1(grid_for(words_per_row * rows, 256), n_mats);
  gen_codes_kernel<<<g1, 256, 0, st>>>(base, mat_stride, bits, rows, cols, seed, layer, slot0, tensor);
  const double cscale = 1.0 / (std::ldexp(1.0, bits - 1) * std::sqrt((double)cols));
  dim3 g2(grid_for((int64_t)rows * (cols / kGroup), 256), n_mats);
  gen_sb_kernel<<<g2, 256, 0, st>>>(base + matrix_codes_bytes(bits, rows, cols), mat_stride, bits, rows, cols, cscale,
                                    seed, layer, slot0, tensor);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "generator launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

int32_t gen_ffn(uint8_t* block, int64_t stride, int n, int bits, int h, int inter, int64_t up, int64_t down,
                uint64_t seed, int layer, int slot0, hipStream_t st) {
  int32_t rc = gen_matrix(block, stride, n, bits, inter, h, seed, layer, slot0, kGate, st);
  if (!rc) rc = gen_matrix(block + up, stride, n, bits, inter, h, seed, layer, slot0, kUp, st);
  if (!rc) rc = gen_matrix(block + down, stride, n, bits, h, inter, seed, layer, slot0, kDown, st);
  return rc;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int32_t moe_generate_layer(const moe_shape_t* shape, uint64_t seed, int32_t layer, void* layer_dev,
                                      moe_stream_t stream) {
  clear_error();
  int32_t rc = check_shape(shape);
  if (rc) return rc;
  if (!layer_dev) return set_error(MOE_ERR_INVALID_ARG, "layer_dev is NULL");
  if ((uintptr_t)layer_dev % kAlign) return set_error(MOE_ERR_ALIGNMENT, "layer_dev must be 256-byte aligned");
  if (layer < 0 || layer >= (1 << 20)) return set_error(MOE_ERR_INVALID_ARG, "layer %d out of range", layer);
  const moe_shape_t& s = *shape;
  hipStream_t st = (hipStream_t)stream;
  moe_layer_layout_t L;
  layout_of(s, &L);
  uint8_t* base = (uint8_t*)layer_dev;
  const int E = s.n_experts;
  const double sig = 1.0 / std::sqrt((double)s.hidden);
  if (s.router_bits == 16) {
    const int64_t n = (int64_t)E * s.hidden;
    gen_vec_sub_kernel<<<grid_for(n, 256), 256, 0, st>>>((uint16_t*)(base + L.router), n, sig, seed, layer, E + 1,
                                                          kRouter);
  } else {
    rc = gen_matrix(base + L.router, 0, 1, s.router_bits, E, s.hidden, seed, layer, E + 1, kRouter, st);
    if (rc) return rc;
  }
  gen_vec_sub_kernel<<<grid_for(s.hidden, 256), 256, 0, st>>>((uint16_t*)(base + L.gatevec), s.hidden, sig, seed,
                                                               layer, E + 2, kGateVec);
  rc = gen_ffn(base + L.shared, 0, 1, s.shared_bits, s.hidden, s.shared_inter, L.shared_up, L.shared_down, seed, layer,
               E, st);
  if (rc) return rc;
  rc = gen_ffn(base + L.expert0, L.expert_stride, E, s.expert_bits, s.hidden, s.inter, L.expert_up, L.expert_down, seed,
               layer, 0, st);
  if (rc) return rc;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "generator launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

extern "C" int32_t moe_generate_rows(uint64_t seed_x, int32_t T, int32_t H, uint16_t* out_dev, moe_stream_t stream) {
  clear_error();
  if (T < 1 || H < 1 || (int64_t)T * H > ((int64_t)1 << 40)) return set_error(MOE_ERR_INVALID_ARG, "bad T/H");
  if (!out_dev) return set_error(MOE_ERR_INVALID_ARG, "out_dev is NULL");
  if ((uintptr_t)out_dev % 16) return set_error(MOE_ERR_ALIGNMENT, "out_dev must be 16-byte aligned");
  const uint64_t sub = host_mix64(seed_x ^ host_mix64(kXTag));
  const int64_t n = (int64_t)T * H;
  gen_vec_kernel<<<grid_for(n, 256), 256, 0, (hipStream_t)stream>>>(out_dev, n, 1.0, sub, kX);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "generator launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

extern "C" int32_t moe_generate_matrix(int32_t bits, int32_t rows, int32_t cols, uint64_t seed, int32_t layer,
                                       int32_t tensor, void* dst_dev, moe_stream_t stream) {
  clear_error();
  if (!bits_ok(bits)) return set_error(MOE_ERR_UNSUPPORTED, "bits %d not in {2,3,4,6,8}", bits);
  if (rows < 1 || rows > (1 << 22) || cols < kGroup || cols > 65536 || cols % kGroup)
    return set_error(MOE_ERR_INVALID_ARG, "rows %d / cols %d invalid", rows, cols);
  if (tensor < 6 || tensor > 1023) return set_error(MOE_ERR_INVALID_ARG, "tensor id %d not in [6, 1023]", tensor);
  if (layer < 0 || layer >= (1 << 20)) return set_error(MOE_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (!dst_dev) return set_error(MOE_ERR_INVALID_ARG, "dst_dev is NULL");
  if ((uintptr_t)dst_dev % kAlign) return set_error(MOE_ERR_ALIGNMENT, "dst_dev must be 256-byte aligned");
  int32_t rc = gen_matrix((uint8_t*)dst_dev, 0, 1, bits, rows, cols, seed, layer, (1 << 20) - 1, tensor,
                          (hipStream_t)stream);
  return rc ? rc : debug_finish(stream);
}
