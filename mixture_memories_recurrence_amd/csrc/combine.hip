// Combine of the MoM layer: the router-weighted sum of the per-memory reads,
// the always-on shared memory entering with weight 1 (jxzklqfsx.com write-up,
// hardware-efficient implementation section: summing the weighted outputs of
// the single-memory operators equals reading from the weighted mixture of
// memories; Mixture-of-Memories section: every token passes the shared memory).
//
// Pure streaming: one wavefront per token; lane l owns the float4 pieces
// l + 64 c of the token's [H][dv] row.  The token's row indices and weights are
// wave-uniform (scalar loads); every o row is read once and out written once,
// with non-temporal accesses (nothing here is read again soon).  Shared term
// first, then j ascending, fixed order, no atomics.
#include "common.h"

namespace mom {

typedef float f4v __attribute__((ext_vector_type(4)));

template <int KM>
__global__ __launch_bounds__(256) void k_combine(int64_t n_tok, int K, int hdv4, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const f4v* __restrict__ o_routed,
                                                 const f4v* __restrict__ o_shared, f4v* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= n_tok) return;
  const int lane = threadIdx.x & 63;
  int64_t r[KM];
  float g[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < K) {
      r[j] = inv ? (int64_t)inv[t * K + j] : t * K + j;
      g[j] = w[t * K + j];
    }
  }
  for (int e = lane; e < hdv4; e += 64) {
    f4v s = __builtin_nontemporal_load(o_shared + t * hdv4 + e);
    f4v o[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < K) o[j] = __builtin_nontemporal_load(o_routed + r[j] * hdv4 + e);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < K) {
        s.x = fmaf(g[j], o[j].x, s.x);
        s.y = fmaf(g[j], o[j].y, s.y);
        s.z = fmaf(g[j], o[j].z, s.z);
        s.w = fmaf(g[j], o[j].w, s.w);
      }
    }
    __builtin_nontemporal_store(s, out + t * hdv4 + e);
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
  const unsigned blocks = (unsigned)(((int64_t)n_tok + 3) / 4);
#define MOM_COMBINE(KM)                                                                                         \
  hipLaunchKernelGGL((k_combine<KM>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, (int64_t)n_tok,          \
                     dims->topk, hdv4, inv, w, (const f4v*)o_routed, (const f4v*)o_shared, (f4v*)out)
  if (dims->topk <= 2) MOM_COMBINE(2);
  else if (dims->topk <= 4) MOM_COMBINE(4);
  else MOM_COMBINE(8);
#undef MOM_COMBINE
  return launch_status();
}
