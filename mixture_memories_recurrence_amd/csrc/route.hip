// Router of the MoM layer: one matmul, one softmax, one top-k, one
// renormalisation per token (podcast.do-not-panic.com page, "Router mechanics,
// step by step").
//
// One wavefront per token.  Lanes stride the model dimension eight elements at
// a time; every product of two stored inputs is exact in float64 and is
// accumulated in float64, then the M partial sums are reduced with the same
// butterfly for every memory, so equal router rows give bit-equal logits and
// the lower index wins a tie.  The top-k and the softmax of the selected
// logits run on lane 0 in float64; the weights are rounded to float32.
#include "common.h"

namespace mom {

template <typename XT>
struct Vec8;
template <>
struct Vec8<bf16_t> {
  __device__ static void load(const bf16_t* p, double* out) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = (double)__uint_as_float(w[i] << 16);
      out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Vec8<float> {
  __device__ static void load(const float* p, double* out) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};

template <typename XT, int MT>
__global__ __launch_bounds__(256) void k_route(int64_t NT, int D, int M, int K, const XT* __restrict__ x,
                                               const XT* __restrict__ wr, const float* __restrict__ bias,
                                               int32_t* __restrict__ idx, float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t n_waves = (int64_t)gridDim.x * blockDim.x / kWave;
  for (int64_t t = wave; t < NT; t += n_waves) {
    double acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0;
    const XT* xt = x + t * D;
    for (int d0 = lane * 8; d0 < D; d0 += kWave * 8) {
      double xv[8];
      Vec8<XT>::load(xt + d0, xv);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          double wv[8];
          Vec8<XT>::load(wr + (int64_t)m * D + d0, wv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[m] = fma(xv[i], wv[i], acc[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = wave_sum_xor(acc[m]);
    if (lane == 0) {
      double logit[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) logit[m] = acc[m] + (bias && m < M ? (double)bias[m] : 0.0);
      uint64_t taken = 0;
      int sel[8];
      for (int j = 0; j < K; ++j) {
        int best = -1;
        double bl = 0.0;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < M && !((taken >> m) & 1ull) && (best < 0 || logit[m] > bl)) {
            best = m;
            bl = logit[m];
          }
        }
        taken |= 1ull << best;
        sel[j] = best;
      }
      double top = 0.0, z = 0.0, e[8];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m == sel[0]) top = logit[m];
      for (int j = 0; j < K; ++j) {
        double lj = 0.0;
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m == sel[j]) lj = logit[m];
        e[j] = exp(lj - top);
        z += e[j];
      }
      for (int j = 0; j < K; ++j) {
        idx[t * K + j] = sel[j];
        w[t * K + j] = (float)(e[j] / z);
      }
    }
  }
}

template <typename XT>
static void launch_route(const mom_dims& d, const void* x, const void* wr, const float* bias, int32_t* idx,
                         float* w, hipStream_t st) {
  const int64_t NT = (int64_t)d.B * d.T;
  const int blocks = (int)((NT + 3) / 4 < 4096 ? (NT + 3) / 4 : 4096);
  const XT* xp = (const XT*)x;
  const XT* wp = (const XT*)wr;
#define MOM_ROUTE_CASE(MT)                                                                              \
  hipLaunchKernelGGL((k_route<XT, MT>), dim3(blocks), dim3(256), 0, st, NT, d.D, d.M, d.topk, xp, wp, bias, \
                     idx, w)
  if (d.M <= 4) MOM_ROUTE_CASE(4);
  else if (d.M <= 8) MOM_ROUTE_CASE(8);
  else if (d.M <= 16) MOM_ROUTE_CASE(16);
  else if (d.M <= 32) MOM_ROUTE_CASE(32);
  else MOM_ROUTE_CASE(64);
#undef MOM_ROUTE_CASE
}

}  // namespace mom

extern "C" mom_status mom_route(const mom_dims* dims, const void* x, const void* w_r, const float* bias,
                                int32_t* idx, float* w, void* stream) {
  using namespace mom;
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  MOM_CHECK_PTR(x);
  MOM_CHECK_PTR(w_r);
  MOM_CHECK_OPT_PTR(bias);
  MOM_CHECK_PTR(idx);
  MOM_CHECK_PTR(w);
  hipStream_t st = (hipStream_t)stream;
  if (dims->dtype == MOM_DTYPE_BF16)
    launch_route<bf16_t>(*dims, x, w_r, bias, idx, w, st);
  else
    launch_route<float>(*dims, x, w_r, bias, idx, w, st);
  return launch_status();
}
