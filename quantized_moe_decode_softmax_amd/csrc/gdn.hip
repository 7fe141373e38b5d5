// Gated DeltaNet decode step (gfx950): moe_gdn_step advances the recurrent
// state of every value head by T tokens and returns each token's output,
//   S <- alpha S;  u = S k;  S <- S + beta (v - u) k^T;  o = S q,
// the gated delta rule of Yang, Kautz & Hatamizadeh (ICLR 2025) in the order
// of the BLAS calls the flash-moe news page names for its GatedDeltaNet
// recurrence ("Accelerate BLAS活用": cblas_sscal, cblas_sgemv, cblas_sger);
// the PureDrive-35B-A3B-MLX model card ("Summary") counts 30 such layers in
// the 35B-A3B model, the flash-moe page ("Model architecture") 45 in the 397B
// model.
//
// Every row i of a head's state S [d_v, d_k] evolves on its own: u_i and o_i
// need only row i, v_i and the head's k and q. A wave therefore owns kRows
// rows (lanes along d_k, d_k / 64 values each), keeps them in registers for
// all T tokens, and writes them back once: the state (fp32, 64 KB per head at
// 128 x 128) is read and written once per call, which is what bounds the
// step (HBM). u_i and o_i are wave sums in a fixed DPP tree, so the results
// are deterministic and a T-token call equals T one-token calls in order, bit
// for bit.
#include <cmath>

#include "gemv.h"

namespace moe {
namespace {

constexpr int kGdnThreads = 256;
constexpr int kGdnWaves = kGdnThreads / 64;
constexpr int kRows = 4;  // state rows per wave

struct GdnArgs {
  int n_k, n_v, dv, T, g;
  float* state;        // [n_v][dv][DK]
  const float* q;      // [T][n_k][DK]
  const float* k;
  const float* v;      // [T][n_v][dv]
  const float* alpha;  // [T][n_v]
  const float* beta;
  float* o;            // [T][n_v][dv]
};

template <int DK>
__global__ void __launch_bounds__(kGdnThreads) gdn_kernel(GdnArgs a) {
  constexpr int VL = DK / 64;  // state values per lane of a row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (blockIdx.x * kGdnWaves + wave) * kRows;  // first global row (head * dv + i)
  const int n_rows = a.n_v * a.dv;
  if (r0 >= n_rows) return;
  float s[kRows][VL];
  int head[kRows], row[kRows];
  bool ok[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int gr = r0 + r;
    ok[r] = gr < n_rows;
    head[r] = ok[r] ? gr / a.dv : 0;
    row[r] = ok[r] ? gr % a.dv : 0;
    const float* src = a.state + (int64_t)(ok[r] ? gr : 0) * DK + lane * VL;
#pragma unroll
    for (int e = 0; e < VL; ++e) s[r][e] = ok[r] ? src[e] : 0.f;
  }
  for (int t = 0; t < a.T; ++t) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      if (!ok[r]) continue;
      const int h = head[r], kh = h / a.g;
      const float* kp = a.k + ((int64_t)t * a.n_k + kh) * DK + lane * VL;
      const float* qp = a.q + ((int64_t)t * a.n_k + kh) * DK + lane * VL;
      float kv[VL], qv[VL];
#pragma unroll
      for (int e = 0; e < VL; ++e) {
        kv[e] = kp[e];
        qv[e] = qp[e];
      }
      const float al = a.alpha[(int64_t)t * a.n_v + h];
      const float be = a.beta[(int64_t)t * a.n_v + h];
      const float vi = a.v[((int64_t)t * a.n_v + h) * a.dv + row[r]];
      // S <- alpha S; u = S k
      float pu = 0.f;
#pragma unroll
      for (int e = 0; e < VL; ++e) {
        s[r][e] *= al;
        pu = fmaf(s[r][e], kv[e], pu);
      }
      const float u = wave_sum(pu);
      // S <- S + beta (v - u) k^T; o = S q
      const float dlt = be * (vi - u);
      float po = 0.f;
#pragma unroll
      for (int e = 0; e < VL; ++e) {
        s[r][e] = fmaf(dlt, kv[e], s[r][e]);
        po = fmaf(s[r][e], qv[e], po);
      }
      const float ov = wave_sum(po);
      if (lane == 0) a.o[((int64_t)t * a.n_v + h) * a.dv + row[r]] = ov;
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (!ok[r]) continue;
    float* dst = a.state + (int64_t)(r0 + r) * DK + lane * VL;
#pragma unroll
    for (int e = 0; e < VL; ++e) dst[e] = s[r][e];
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int32_t moe_gdn_step(const moe_gdn_shape_t* shape, int32_t T, float* state_dev, const float* q_dev,
                                const float* k_dev, const float* v_dev, const float* alpha_dev, const float* beta_dev,
                                float* o_dev, moe_stream_t stream) {
  clear_error();
  if (!shape) return set_error(MOE_ERR_INVALID_ARG, "shape is NULL");
  const moe_gdn_shape_t& s = *shape;
  if (!(s.d_k == 64 || s.d_k == 128 || s.d_k == 256))
    return set_error(MOE_ERR_UNSUPPORTED, "d_k %d not in {64, 128, 256}", s.d_k);
  if (s.d_v < 1 || s.d_v > 4096) return set_error(MOE_ERR_INVALID_ARG, "d_v %d not in [1, 4096]", s.d_v);
  if (s.n_k < 1 || s.n_v < 1 || s.n_v % s.n_k || s.n_v > 1024)
    return set_error(MOE_ERR_INVALID_ARG, "n_v %d must be a multiple of n_k %d and at most 1024", s.n_v, s.n_k);
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  if (!state_dev || !q_dev || !k_dev || !v_dev || !alpha_dev || !beta_dev || !o_dev)
    return set_error(MOE_ERR_INVALID_ARG, "NULL buffer");
  if ((uintptr_t)state_dev % 16 || (uintptr_t)q_dev % 16 || (uintptr_t)k_dev % 16 || (uintptr_t)v_dev % 4 ||
      (uintptr_t)alpha_dev % 4 || (uintptr_t)beta_dev % 4 || (uintptr_t)o_dev % 4)
    return set_error(MOE_ERR_ALIGNMENT, "state, q, k 16-byte aligned; v, alpha, beta, o 4-byte aligned");
  const char* sb = (const char*)state_dev;
  const int64_t sbytes = (int64_t)s.n_v * s.d_v * s.d_k * 4;
  const char* ob = (const char*)o_dev;
  const int64_t obytes = (int64_t)T * s.n_v * s.d_v * 4;
  if (sb < ob + obytes && ob < sb + sbytes) return set_error(MOE_ERR_INVALID_ARG, "o overlaps the state");
  GdnArgs a;
  a.n_k = s.n_k;
  a.n_v = s.n_v;
  a.dv = s.d_v;
  a.T = T;
  a.g = s.n_v / s.n_k;
  a.state = state_dev;
  a.q = q_dev;
  a.k = k_dev;
  a.v = v_dev;
  a.alpha = alpha_dev;
  a.beta = beta_dev;
  a.o = o_dev;
  const int64_t rows = (int64_t)s.n_v * s.d_v;
  const int grid = (int)((rows + kRows * kGdnWaves - 1) / (kRows * kGdnWaves));
  hipStream_t st = (hipStream_t)stream;
  switch (s.d_k) {
    case 64: gdn_kernel<64><<<grid, kGdnThreads, 0, st>>>(a); break;
    case 128: gdn_kernel<128><<<grid, kGdnThreads, 0, st>>>(a); break;
    default: gdn_kernel<256><<<grid, kGdnThreads, 0, st>>>(a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "gdn launch failed: %s", hipGetErrorString(e));
  return debug_finish(stream);
}
