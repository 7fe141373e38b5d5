// Dense group-affine matrix-vector products of the non-expert projections
// (gfx950): moe_gemv computes y_m = W_m x for up to four matrices that share
// one input, in one launch, reading x once per wave (the fused Q/K/V
// projection), and serves the attention output projection and lm_head as the
// one-matrix case; moe_generate_matrix writes a seeded synthetic matrix.
//
// Sources: PureDrive-35B-A3B-MLX model card, "Summary" (attention, shared
// expert, embedding and lm_head are 8-bit); Qwen3.5-397B on M5 Max news page,
// "Effective optimisations" (a fused Q/K/V projection kernel reads the input
// vector once instead of three times); flash-moe news page, "FMA-optimised
// dequant kernel" (group-affine weights).
//
// Work split: the rows of all matrices form one list; a wave task takes R
// rows per row group (lanes along the input in 32-code chunks, as in the
// expert kernels), loads their codes and scale/bias words once, then for each
// token row arranges that row's input and computes the R dot products with
// the arithmetic of gemv.h (the same per (row, output) whatever T is, so a
// T-row call equals T one-row calls bit for bit). Results are fp32, one lane
// per row storing.
#include <cmath>

#include "gemv.h"

namespace moe {
namespace {

constexpr int kGemvMax = 4;      // matrices per call
constexpr int kGemvWaves = 4;    // waves per workgroup
constexpr int kMaxCols = 8192;
constexpr int kMaxRows = 1 << 22;

struct GemvArgs {
  int n;            // matrices
  int K;            // columns (input length)
  int T;            // token rows
  int total;        // rows of all matrices
  int64_t row_bytes, codes_bytes;  // per row of codes; codes part of a matrix block (per matrix below)
  const uint8_t* w[kGemvMax];
  int rows[kGemvMax];
  int first[kGemvMax + 1];  // prefix sums of rows
  int64_t sb_off[kGemvMax]; // byte offset of the scale/bias words in each block
  float* y[kGemvMax];
  const uint16_t* x;        // bf16 [T, K]
};

// DEC (8-bit codes, several token rows): the task's codes are decoded into
// bf16 pairs once and reused for every token row (the same products and sums
// as decoding them per row), two rows per task so that the decoded pairs
// leave four waves per SIMD.
template <int BITS, int CPL, bool DEC>
__global__ void __launch_bounds__(64 * kGemvWaves) gemv_kernel(GemvArgs a) {
  constexpr int R = DEC ? 2 : CPL >= 2 ? 2 : 4;  // rows per row group (registers: R * CPL <= 4)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = lanes_per_row(a.K), rpw = 64 / lpr, sr = lane / lpr, li = lane % lpr;
  const int task = blockIdx.x * kGemvWaves + wave;
  const int r0 = task * R * rpw;
  if (r0 >= a.total) return;
  int m_of[R], loc[R];
  const uint8_t* rc[R];
  const uint32_t* rs[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int g = r0 + sr + rpw * i;
    int m = 0;
#pragma unroll
    for (int j = 1; j < kGemvMax; ++j) m += (j < a.n && g >= a.first[j]) ? 1 : 0;
    const bool ok = g < a.total;
    m_of[i] = m;
    loc[i] = ok ? g - a.first[m] : -1;
    rc[i] = ok ? a.w[m] + (int64_t)loc[i] * a.row_bytes : nullptr;
    rs[i] = ok ? (const uint32_t*)(a.w[m] + a.sb_off[m]) + (int64_t)loc[i] * (a.K >> 6) : nullptr;
  }
  RowsQ<BITS, CPL, R> Q;
  load_rows<BITS, CPL, R>(Q, rc, rs, a.K, (int)(a.row_bytes >> 2), li, lpr);
  XLane<BITS, CPL> x;
  float out[R];
  RowsDec8<CPL, DEC ? R : 1> Dq;
  if constexpr (DEC) decode8<CPL, R>(Q, Dq);
  for (int t = 0; t < a.T; ++t) {
    prep_x<BITS, CPL>(x, a.x + (int64_t)t * a.K, a.K, li, lpr);
    if constexpr (DEC)
      dot_dec8<CPL, R>(Dq, x, out);
    else
      dot_rows<BITS, CPL, R, 1>(Q, x, x, out);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float v = reduce_row(out[i], lpr);
      if (loc[i] >= 0 && li == lpr - 1) a.y[m_of[i]][(int64_t)t * a.rows[m_of[i]] + loc[i]] = v;
    }
  }
}

#define MOE_GEMV_BITS(bits, B, ...)                       \
  switch (bits) {                                         \
    case 2: { constexpr int B = 2; __VA_ARGS__; } break;  \
    case 3: { constexpr int B = 3; __VA_ARGS__; } break;  \
    case 4: { constexpr int B = 4; __VA_ARGS__; } break;  \
    case 6: { constexpr int B = 6; __VA_ARGS__; } break;  \
    default: { constexpr int B = 8; __VA_ARGS__; } break; \
  }

template <int CPL>
void launch_gemv(int bits, const GemvArgs& a, hipStream_t st) {
  constexpr int R = CPL >= 2 ? 2 : 4;
  const int rpw = 64 / lanes_per_row(a.K);
  const int tasks = (a.total + R * rpw - 1) / (R * rpw);
  const int grid = (tasks + kGemvWaves - 1) / kGemvWaves;
  if constexpr (CPL <= 2) {
    if (bits == 8 && a.T >= 2) {  // codes decoded once for all token rows
      const int tasks2 = (a.total + 2 * rpw - 1) / (2 * rpw);
      gemv_kernel<8, CPL, true><<<(tasks2 + kGemvWaves - 1) / kGemvWaves, 64 * kGemvWaves, 0, st>>>(a);
      return;
    }
  }
  MOE_GEMV_BITS(bits, B, gemv_kernel<B, CPL, false><<<grid, 64 * kGemvWaves, 0, st>>>(a));
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int32_t moe_gemv(int32_t bits, int32_t cols, int32_t T, const uint16_t* x_dev, const moe_gemv_mat_t* mats_host,
                            int32_t n_mats, moe_stream_t stream) {
  clear_error();
  if (!bits_ok(bits)) return set_error(MOE_ERR_UNSUPPORTED, "bits %d not in {2,3,4,6,8}", bits);
  if (cols < kGroup || cols > kMaxCols || cols % kGroup)
    return set_error(MOE_ERR_UNSUPPORTED, "cols %d must be a multiple of 64 in [64, %d]", cols, kMaxCols);
  if (T < 1 || T > kMaxT) return set_error(MOE_ERR_INVALID_ARG, "T %d not in [1, %d]", T, kMaxT);
  if (!mats_host || n_mats < 1 || n_mats > kGemvMax)
    return set_error(MOE_ERR_INVALID_ARG, "n_mats %d not in [1, %d]", n_mats, kGemvMax);
  if (!x_dev) return set_error(MOE_ERR_INVALID_ARG, "x is NULL");
  if ((uintptr_t)x_dev % 16) return set_error(MOE_ERR_ALIGNMENT, "x must be 16-byte aligned");
  GemvArgs a;
  a.n = n_mats;
  a.K = cols;
  a.T = T;
  a.row_bytes = row_bytes(bits, cols);
  int64_t total = 0;
  for (int m = 0; m < kGemvMax; ++m) {
    a.w[m] = nullptr;
    a.rows[m] = 0;
    a.sb_off[m] = 0;
    a.y[m] = nullptr;
  }
  for (int m = 0; m < n_mats; ++m) {
    const moe_gemv_mat_t& q = mats_host[m];
    if (!q.w_dev || !q.y_dev) return set_error(MOE_ERR_INVALID_ARG, "matrix %d: NULL weights or output", m);
    if ((uintptr_t)q.w_dev % kAlign) return set_error(MOE_ERR_ALIGNMENT, "matrix %d: weights not 256-byte aligned", m);
    if ((uintptr_t)q.y_dev % 4) return set_error(MOE_ERR_ALIGNMENT, "matrix %d: output not 4-byte aligned", m);
    if (q.rows < 1 || q.rows > kMaxRows) return set_error(MOE_ERR_INVALID_ARG, "matrix %d: rows %d", m, q.rows);
    a.w[m] = (const uint8_t*)q.w_dev;
    a.rows[m] = q.rows;
    a.sb_off[m] = matrix_codes_bytes(bits, q.rows, cols);
    a.y[m] = q.y_dev;
    a.first[m] = (int)total;
    total += q.rows;
  }
  if (total > kMaxRows) return set_error(MOE_ERR_INVALID_ARG, "%lld rows in all matrices", (long long)total);
  for (int m = n_mats; m <= kGemvMax; ++m) a.first[m] = (int)total;
  a.total = (int)total;
  // outputs must not overlap the input or each other's bytes of any matrix block
  const char* xb = (const char*)x_dev;
  const int64_t xbytes = (int64_t)T * cols * 2;
  for (int m = 0; m < n_mats; ++m) {
    const char* yb = (const char*)a.y[m];
    const int64_t ybytes = (int64_t)T * a.rows[m] * 4;
    if (yb < xb + xbytes && xb < yb + ybytes) return set_error(MOE_ERR_INVALID_ARG, "output %d overlaps x", m);
    for (int n = 0; n < m; ++n) {
      const char* zb = (const char*)a.y[n];
      const int64_t zbytes = (int64_t)T * a.rows[n] * 4;
      if (yb < zb + zbytes && zb < yb + ybytes) return set_error(MOE_ERR_INVALID_ARG, "outputs %d and %d overlap", n, m);
    }
  }
  a.x = x_dev;
  hipStream_t st = (hipStream_t)stream;
  const int cpl = chunks_per_lane(cols);
  if (cpl == 1) launch_gemv<1>(bits, a, st);
  else if (cpl == 2) launch_gemv<2>(bits, a, st);
  else launch_gemv<4>(bits, a, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "gemv launch failed: %s", hipGetErrorString(e));
  return debug_finish((hipStream_t)stream);
}
