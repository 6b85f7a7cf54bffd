// Combine of the MoM layer: the router-weighted sum of the per-memory reads,
// the always-on shared memory entering with weight 1 (jxzklqfsx.com write-up,
// hardware-efficient implementation section: summing the weighted outputs of
// the single-memory operators equals reading from the weighted mixture of
// memories; Mixture-of-Memories section: every token passes the shared memory).
//
// Pure streaming: each thread owns four consecutive floats of one token's
// [H][dv] row; shared read first, then j ascending, fixed order, no atomics.
#include "common.h"

namespace mom {

__global__ __launch_bounds__(256) void k_combine(int64_t n_tok, int K, int hdv4, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const float4* __restrict__ o_routed,
                                                 const float4* __restrict__ o_shared, float4* __restrict__ out) {
  const int64_t total = n_tok * hdv4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / hdv4;
    const int e = (int)(i - t * hdv4);
    float4 s = o_shared[i];
    for (int j = 0; j < K; ++j) {
      const int64_t r = inv ? (int64_t)inv[t * K + j] : t * K + j;
      const float g = w[t * K + j];
      const float4 o = o_routed[r * hdv4 + e];
      s.x = fmaf(g, o.x, s.x);
      s.y = fmaf(g, o.y, s.y);
      s.z = fmaf(g, o.z, s.z);
      s.w = fmaf(g, o.w, s.w);
    }
    out[i] = s;
  }
}

}  // namespace mom

extern "C" mom_status mom_combine(const mom_dims* dims, int32_t n_tok, const int32_t* inv, const float* w,
                                  const float* o_routed, const float* o_shared, float* out, void* stream) {
  using namespace mom;
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  if (n_tok < 0) return MOM_ERR_DIMS;
  MOM_CHECK_OPT_PTR(inv);
  MOM_CHECK_PTR(w);
  MOM_CHECK_PTR(o_routed);
  MOM_CHECK_PTR(o_shared);
  MOM_CHECK_PTR(out);
  if (n_tok == 0) return MOM_OK;
  const int hdv4 = dims->H * dims->dv / 4;
  const int64_t total = (int64_t)n_tok * hdv4;
  const int blocks = (int)(total / 256 + 1 < 65536 ? total / 256 + 1 : 65536);
  hipLaunchKernelGGL(k_combine, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (int64_t)n_tok, dims->topk, hdv4,
                     inv, w, (const float4*)o_routed, (const float4*)o_shared, (float4*)out);
  return launch_status();
}
