// Host side of the persistent stack kernel: launch geometry, argument block,
// the clear kernel and the dispatch over the instantiated variants.
#include "persist.h"

namespace moe {

// the variants are compiled in persist_<CPL_H><CPL_I>.hip
#define MOE_STACK_EXTERN(H, I, R) extern template hipError_t launch_stack_kernel<H, I, R>(const PArgs&, hipStream_t);
MOE_STACK_EXTERN(1, 1, 1) MOE_STACK_EXTERN(1, 1, 2) MOE_STACK_EXTERN(1, 1, 4) MOE_STACK_EXTERN(1, 1, 8)
MOE_STACK_EXTERN(1, 2, 2)
MOE_STACK_EXTERN(2, 1, 1) MOE_STACK_EXTERN(2, 1, 2) MOE_STACK_EXTERN(2, 1, 4) MOE_STACK_EXTERN(2, 1, 8)
#undef MOE_STACK_EXTERN

namespace {

__global__ void clear_kernel(uint64_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0ull;
}

}  // namespace

// ----------------------------------------------------------------- host side
// Returns MOE_ERR_UNSUPPORTED (with no launch) when the shape is outside what
// the stack kernel handles; the caller then uses the per-layer kernels.
int32_t launch_stack_persistent(const moe_shape_t& s, const moe_layer_layout_t& L, const WsMap& m, uint8_t* ws,
                                const void* const* layers, int n_layers, int T, const uint16_t* h_in, uint16_t* h_out,
                                int32_t* ids_out, float* w_out, uint16_t* h_trace_out, moe_stream_t stream) {
  hipStream_t st = (hipStream_t)stream;
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
      return set_error(MOE_ERR_HIP, "cannot query the compute unit count");
  }
  PArgs a;
  a.H = s.hidden;
  a.E = s.n_experts;
  a.I = s.inter;
  a.Is = s.shared_inter;
  a.k = s.top_k;
  a.T = T;
  a.imax = s.inter > s.shared_inter ? s.inter : s.shared_inter;
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
  const int cpl_h = chunks_per_lane(s.hidden);
  const int cpl_i = chunks_per_lane(a.imax);
  if (cpl_h > 2 || cpl_i > 2) return MOE_ERR_UNSUPPORTED;
  // output rows per workgroup: even, one workgroup per compute unit
  int J = (s.hidden + n_cu - 1) / n_cu;
  J = J < 2 ? 2 : (J + 1) & ~1;
  if (J > 16) return MOE_ERR_UNSUPPORTED;
  a.J = J;
  a.nwg = n_cu;
  const int rpw_min = 64 / lanes_per_row(a.imax);
  int RD = (J + rpw_min - 1) / rpw_min;
  RD = pow2ceil(RD);
  // (more down rows per lane group would spill registers)
  if (RD > (cpl_i == 2 ? 2 : 8)) return MOE_ERR_UNSUPPORTED;
  const int rpw_h = 64 / lanes_per_row(s.hidden);
  const int R = cpl_h >= 2 ? 2 : 4;
  a.n_rt = (a.E + rpw_h - 1) / rpw_h;  // one router row per lane group
  a.n_st = (a.Is + (R / 2) * rpw_h - 1) / ((R / 2) * rpw_h);
  a.tpu = (a.I + (R / 2) * rpw_h - 1) / ((R / 2) * rpw_h);
  a.mE = pow2ceil((a.E + 63) / 64);
  a.tg_h = (uint64_t*)(ws + m.tg_h);
  a.tg_logit = (uint64_t*)(ws + m.tg_logit);
  a.tg_rs = (uint64_t*)(ws + m.tg_rs);
  a.tg_a = (uint64_t*)(ws + m.tg_a);
  a.status = (uint32_t*)(ws + m.status);
  const int64_t th = (int64_t)T * s.hidden;
  const int64_t tk = (int64_t)T * s.top_k;
  uint16_t* hb = (uint16_t*)(ws + m.hbuf);
  const uint16_t* cur = h_in;
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayersPerLaunch) {
    const int nl = n_layers - l0 < kMaxLayersPerLaunch ? n_layers - l0 : kMaxLayersPerLaunch;
    const bool last = l0 + nl == n_layers;
    a.n_layers = nl;
    for (int l = 0; l < nl; ++l) a.layers[l] = (const uint8_t*)layers[l0 + l];
    a.h_in = cur;
    a.h_out = last ? h_out : hb + ((l0 / kMaxLayersPerLaunch) & 1) * th;
    a.ids_out = ids_out ? ids_out + (int64_t)l0 * tk : nullptr;
    a.w_out = w_out ? w_out + (int64_t)l0 * tk : nullptr;
    a.h_trace = h_trace_out ? h_trace_out + (int64_t)(l0 + 1) * th : nullptr;
    // the clear covers the exchange words and the status word
    const int64_t nclr = (m.tg_end - m.tg_h) / 8;
    clear_kernel<<<64, 256, 0, st>>>(a.tg_h, nclr);
    hipError_t e = hipSuccess;
    switch (cpl_h * 100 + cpl_i * 10 + RD) {
#define MOE_STACK_CASE(H, I, R) \
  case H * 100 + I * 10 + R: e = launch_stack_kernel<H, I, R>(a, st); break;
      MOE_STACK_CASE(1, 1, 1) MOE_STACK_CASE(1, 1, 2) MOE_STACK_CASE(1, 1, 4) MOE_STACK_CASE(1, 1, 8)
      MOE_STACK_CASE(1, 2, 2)
      MOE_STACK_CASE(2, 1, 1) MOE_STACK_CASE(2, 1, 2) MOE_STACK_CASE(2, 1, 4) MOE_STACK_CASE(2, 1, 8)
#undef MOE_STACK_CASE
      default: return MOE_ERR_UNSUPPORTED;
    }
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "stack kernel launch failed: %s", hipGetErrorString(e));
    cur = a.h_out;
  }
  return MOE_OK;
}

}  // namespace moe
