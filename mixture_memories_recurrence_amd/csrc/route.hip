// Router of the MoM layer: one matmul, one softmax, one top-k, one
// renormalisation per token (podcast.do-not-panic.com page, "Router mechanics,
// step by step").
//
// G lanes per token (64 for small batches, else 16).  Every product of two stored inputs is exact and is
// accumulated in float64; the partial sums of every memory go through the same
// butterfly, so equal router rows give bit-equal logits and the lower index
// wins a tie.  The top-k and the softmax of the selected logits run on the
// group's first lane in float64; the weights are rounded to float32.
#include "common.h"

namespace mom {

// Products of two stored inputs, exact: for bfloat16 the float32 product is
// exact (8 + 8 significant bits), for float32 inputs the product is formed in
// float64.
template <typename XT>
struct ExactProd;
template <>
struct ExactProd<bf16_t> {
  typedef uint4 Raw;  // eight bf16
  __device__ static Raw raw(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void unpack(const Raw& u, float* out) {
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(wv[i] << 16);
      out[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
    }
  }
  __device__ static double fma(float a, float b, double c) { return c + (double)(a * b); }
};
template <>
struct ExactProd<float> {
  struct Raw {
    float4 a, b;
  };
  __device__ static Raw raw(const float* p) {
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  __device__ static void unpack(const Raw& r, float* out) {
    out[0] = r.a.x; out[1] = r.a.y; out[2] = r.a.z; out[3] = r.a.w;
    out[4] = r.b.x; out[5] = r.b.y; out[6] = r.b.z; out[7] = r.b.w;
  }
  __device__ static double fma(float a, float b, double c) { return ::fma((double)a, (double)b, c); }
};

// G lanes per token: lane s of a group handles elements 8 s + 8 G i of
// the row; the group's partial sums are combined with the same xor butterfly
// for every memory.
template <typename XT, int MT, int G>
__global__ __launch_bounds__(256) void k_route(int64_t NT, int D, int M, int K, const XT* __restrict__ x,
                                               const XT* __restrict__ wr, const float* __restrict__ bias,
                                               int32_t* __restrict__ idx, float* __restrict__ w) {
  using P = ExactProd<XT>;
  const int sub = threadIdx.x % G;
  const int64_t grp = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / G;
  const int64_t n_grp = (int64_t)gridDim.x * blockDim.x / G;
  for (int64_t t = grp; t < NT; t += n_grp) {
    double acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0;
    const XT* xt = x + t * D;
    // Memories m >= M (when M < MT) read row M - 1 and are never selected.  The
    // row is read in batches of NB steps whose loads are all issued before the
    // first product; steps past D read the last piece and are masked to zero.
    constexpr int NB = MT <= 8 ? 4 : 2;
    for (int d0 = sub * 8; d0 < D; d0 += NB * G * 8) {
      typename P::Raw xr[NB], wr_[NB][MT];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int d = min(d0 + b * G * 8, D - 8);
        xr[b] = P::raw(xt + d);
#pragma unroll
        for (int m = 0; m < MT; ++m) wr_[b][m] = P::raw(wr + (int64_t)(m < M ? m : M - 1) * D + d);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (d0 + b * G * 8 >= D) break;
        float xv[8];
        P::unpack(xr[b], xv);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float wv[8];
          P::unpack(wr_[b][m], wv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[m] = P::fma(xv[i], wv[i], acc[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) acc[m] += __shfl_xor(acc[m], o, kWave);
    if (sub == 0) {
      double logit[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) logit[m] = acc[m] + (bias && m < M ? (double)bias[m] : 0.0);
      uint64_t taken = 0;
      int sel[8];
      double ls[8];
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
        ls[j] = bl;
      }
      double z = 0.0, e[8];
      for (int j = 0; j < K; ++j) {
        e[j] = exp(ls[j] - ls[0]);
        z += e[j];
      }
      for (int j = 0; j < K; ++j) {
        idx[t * K + j] = sel[j];
        w[t * K + j] = (float)(e[j] / z);
      }
    }
  }
}

template <typename XT, int G>
static void launch_route_g(const mom_dims& d, const void* x, const void* wr, const float* bias, int32_t* idx,
                           float* w, hipStream_t st) {
  const int64_t NT = (int64_t)d.B * d.T;
  const int64_t need = (NT + 256 / G - 1) / (256 / G);
  const int blocks = (int)(need < 8192 ? need : 8192);
  const XT* xp = (const XT*)x;
  const XT* wp = (const XT*)wr;
#define MOM_ROUTE_CASE(MT)                                                                                 \
  hipLaunchKernelGGL((k_route<XT, MT, G>), dim3(blocks), dim3(256), 0, st, NT, d.D, d.M, d.topk, xp, wp, \
                     bias, idx, w)
  if (d.M <= 4) MOM_ROUTE_CASE(4);
  else if (d.M <= 8) MOM_ROUTE_CASE(8);
  else if (d.M <= 16) MOM_ROUTE_CASE(16);
  else if (d.M <= 32) MOM_ROUTE_CASE(32);
  else MOM_ROUTE_CASE(64);
#undef MOM_ROUTE_CASE
}

// Few tokens (decode): a whole wave per token, so the row is read in few steps;
// many tokens: 16 lanes per token, four tokens per wave.
template <typename XT>
static void launch_route(const mom_dims& d, const void* x, const void* wr, const float* bias, int32_t* idx,
                         float* w, hipStream_t st) {
  if ((int64_t)d.B * d.T < 8192) launch_route_g<XT, 64>(d, x, wr, bias, idx, w, st);
  else launch_route_g<XT, 16>(d, x, wr, bias, idx, w, st);
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
