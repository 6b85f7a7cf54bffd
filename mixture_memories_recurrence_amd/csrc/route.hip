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
// for every memory.  With cnt (one position per sequence: token t is sequence
// t) the kernel also writes the dispatch's counts, cnt[m][t] = 1 when token t
// selected memory m, else 0, so the dispatch needs no counting launch.
template <typename XT, int MT, int G>
__global__ __launch_bounds__(256) void k_route(int64_t NT, int D, int M, int K, const XT* __restrict__ x,
                                               const XT* __restrict__ wr, const float* __restrict__ bias,
                                               int32_t* __restrict__ idx, float* __restrict__ w,
                                               int32_t* __restrict__ cnt) {
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
      if (cnt)
        for (int m = 0; m < M; ++m) cnt[(int64_t)m * NT + t] = (int32_t)((taken >> m) & 1ull);
    }
  }
}

// Cross-lane moves of float64 values, one 32-bit half at a time.
typedef unsigned route_u2 __attribute__((ext_vector_type(2)));
// a <- [a of lanes 0..31, b of lanes 0..31], b <- [a of lanes 32..63, b of lanes 32..63]
__device__ __forceinline__ void swap_halves(double& a, double& b) {
  const route_u2 A = __builtin_bit_cast(route_u2, a), B = __builtin_bit_cast(route_u2, b);
  const auto lo = __builtin_amdgcn_permlane32_swap(A.x, B.x, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(A.y, B.y, false, false);
  a = __builtin_bit_cast(double, route_u2{lo[0], hi[0]});
  b = __builtin_bit_cast(double, route_u2{lo[1], hi[1]});
}
// With 16-lane rows r0..r3: a <- [a.r0, b.r0, a.r2, b.r2], b <- [a.r1, b.r1, a.r3, b.r3]
__device__ __forceinline__ void swap_rows(double& a, double& b) {
  const route_u2 A = __builtin_bit_cast(route_u2, a), B = __builtin_bit_cast(route_u2, b);
  const auto lo = __builtin_amdgcn_permlane16_swap(A.x, B.x, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(A.y, B.y, false, false);
  a = __builtin_bit_cast(double, route_u2{lo[0], hi[0]});
  b = __builtin_bit_cast(double, route_u2{lo[1], hi[1]});
}
// Lane l of each 16-lane row gets lane l - N's value, 0 for the first N lanes (DPP row_shr).
template <int N>
__device__ __forceinline__ double row_shr(double v) {
  const route_u2 V = __builtin_bit_cast(route_u2, v);
  const route_u2 R = {(unsigned)__builtin_amdgcn_update_dpp(0, (int)V.x, 0x110 + N, 0xF, 0xF, true),
                      (unsigned)__builtin_amdgcn_update_dpp(0, (int)V.y, 0x110 + N, 0xF, 0xF, true)};
  return __builtin_bit_cast(double, R);
}
__device__ __forceinline__ double read_lane(double v, int l) {
  const route_u2 V = __builtin_bit_cast(route_u2, v);
  const route_u2 R = {(unsigned)__builtin_amdgcn_readlane((int)V.x, l), (unsigned)__builtin_amdgcn_readlane((int)V.y, l)};
  return __builtin_bit_cast(double, R);
}

// bfloat16 rows, at most four memories: a wave takes TPW consecutive tokens and
// loads all their rows at once.  Lane l handles elements 8 l + 512 j + i
// (i < 8) of every row; its slice of the router rows (EPL = D / 64 values per
// memory) is loaded once per wave.  Each product goes into float64 by one fma
// of the two exactly converted inputs, which rounds exactly like the float32
// product (exact) added in float64.  The four sums of a token are reduced
// across the 64 lanes by halving exchanges (v_permlane32_swap, then
// v_permlane16_swap: each lane keeps fewer memories) and then a running sum
// along each 16-lane row (DPP row shifts), so every memory's total comes from
// the same tree and equal router rows give bit-equal logits.  Token i's logits
// stay in lane i, and lanes 0 .. TPW - 1 then run the top-k and the softmax
// of their tokens side by side.
template <int EPL, int TPW>
__global__ __launch_bounds__(256) void k_route_wave4(int64_t NT, int D, int M, int K, const bf16_t* __restrict__ x,
                                                     const bf16_t* __restrict__ wr, const float* __restrict__ bias,
                                                     int32_t* __restrict__ idx, float* __restrict__ w) {
  constexpr int MT = 4, NL = EPL / 8;
  using P = ExactProd<bf16_t>;
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_wave = ((int64_t)gridDim.x * blockDim.x) >> 6;
  float wf[MT][EPL];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const bf16_t* row = wr + (int64_t)(m < M ? m : M - 1) * D + 8 * lane;
#pragma unroll
    for (int j = 0; j < NL; ++j) P::unpack(P::raw(row + 512 * j), &wf[m][8 * j]);
  }
  for (int64_t t0 = wave * TPW; t0 < NT; t0 += n_wave * TPW) {
    typename P::Raw xr[TPW][NL];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int64_t t = t0 + i < NT ? t0 + i : NT - 1;  // past the end: a valid row, never written
#pragma unroll
      for (int j = 0; j < NL; ++j) xr[i][j] = P::raw(x + t * D + 8 * lane + 512 * j);
    }
    double mine[MT] = {0.0, 0.0, 0.0, 0.0};  // logits of token t0 + lane (lanes < TPW)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      double acc[MT] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        float xv[8];
        P::unpack(xr[i][j], xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double xd = (double)xv[e];
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[m] = ::fma(xd, (double)wf[m][8 * j + e], acc[m]);
        }
      }
      // lanes 0..31 collect memories 0, 1 and lanes 32..63 memories 2, 3 (pairs
      // of lanes l, l + 32 added); then row r of 16 lanes collects memory r
      // (pairs of rows added); a running sum along each row leaves the total
      // in its last lane.  Vector-ALU lane moves only (no LDS round trips).
      swap_halves(acc[0], acc[2]);
      swap_halves(acc[1], acc[3]);
      double k0 = acc[0] + acc[2], k1 = acc[1] + acc[3];
      swap_rows(k0, k1);
      double v = k0 + k1;
      v += row_shr<1>(v);
      v += row_shr<2>(v);
      v += row_shr<4>(v);
      v += row_shr<8>(v);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const double lm = read_lane(v, 16 * m + 15);
        if (lane == i) mine[m] = lm;
      }
    }
    const int64_t t = t0 + lane;
    if (lane < TPW && t < NT) {
      double logit[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) logit[m] = mine[m] + (bias && m < M ? (double)bias[m] : 0.0);
      uint32_t taken = 0;
      int sel[MT];
      double ls[MT];
      for (int j = 0; j < K; ++j) {
        int best = -1;
        double bl = 0.0;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < M && !((taken >> m) & 1u) && (best < 0 || logit[m] > bl)) {
            best = m;
            bl = logit[m];
          }
        }
        taken |= 1u << best;
        sel[j] = best;
        ls[j] = bl;
      }
      double z = 0.0, e[MT];
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

// Route and dispatch counts for whole sequences (bfloat16 rows, D = 1024 DG,
// M <= 4 MG): one block of eight waves per 64 positions of one sequence.  Wave
// (mg, dg, nh) holds in registers its lanes' slice of router rows 4 mg ..
// 4 mg + 3 over elements [1024 dg, 1024 dg + 1024) (lane l: 8 l + 512 j + i)
// and walks positions nh 64 / NH .. in groups of four, the next group's rows
// loaded while the current one is reduced.  The products, per-lane sums and
// cross-lane tree are k_route_wave4's; each tree's total (a partial logit over
// the wave's elements) goes to LDS, and the block's first wave adds the DG
// partials of each memory in order, runs the top-k and the softmax for its
// position (lane = position), and counts the selections per memory with
// ballots: the dispatch's count of these 64 positions, cnt[m][b][sub] (nsub =
// ceil(T / 64)), so the dispatch needs no counting launch and nothing is
// cleared first.  With DG = MG = 1 the logits are k_route_wave4's bit for bit.
template <int MG, int DG, int NH>
__global__ __launch_bounds__(512) void k_route_blk(int B, int T, int D, int M, int K, int nsub,
                                                   const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr,
                                                   const float* __restrict__ bias, int32_t* __restrict__ idx,
                                                   float* __restrict__ w, int32_t* __restrict__ cnt) {
  static_assert(MG * DG * NH == 8, "eight waves");
  using P = ExactProd<bf16_t>;
  constexpr int MP = 4 * MG, TPW = 4, NGR = 64 / NH / TPW;  // memories held, groups per wave
  __shared__ double part[DG][64][MP];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int mg = wv % MG, dg = (wv / MG) % DG, nh = wv / (MG * DG);
  const int sub = blockIdx.x, b = blockIdx.y;
  const int lp0 = nh * (64 / NH);  // first position of this wave inside the 64
  const int64_t tok0 = (int64_t)b * T;
  const int64_t col = 1024 * dg + 8 * lane;
  typename P::Raw xr[2][TPW][2];
  auto load = [&](int gi, int bufi) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      int p = sub * 64 + lp0 + gi * TPW + i;
      p = p < T ? p : T - 1;  // past the end: a valid row, never written
#pragma unroll
      for (int j = 0; j < 2; ++j) xr[bufi][i][j] = P::raw(x + (tok0 + p) * D + col + 512 * j);
    }
  };
  load(0, 0);
  if (NGR > 1) load(1, 1);
  float wf[4][16];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int mm = 4 * mg + m;
    const bf16_t* row = wr + (int64_t)(mm < M ? mm : M - 1) * D + col;
#pragma unroll
    for (int j = 0; j < 2; ++j) P::unpack(P::raw(row + 512 * j), &wf[m][8 * j]);
  }
#pragma unroll
  for (int gi = 0; gi < NGR; ++gi) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float xv[8];
        P::unpack(xr[gi & 1][i][j], xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double xd = (double)xv[e];
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m] = ::fma(xd, (double)wf[m][8 * j + e], acc[m]);
        }
      }
      swap_halves(acc[0], acc[2]);
      swap_halves(acc[1], acc[3]);
      double k0 = acc[0] + acc[2], k1 = acc[1] + acc[3];
      swap_rows(k0, k1);
      double v = k0 + k1;
      v += row_shr<1>(v);
      v += row_shr<2>(v);
      v += row_shr<4>(v);
      v += row_shr<8>(v);
      if ((lane & 15) == 15) part[dg][lp0 + gi * TPW + i][4 * mg + (lane >> 4)] = v;
    }
    if (gi + 2 < NGR) load(gi + 2, gi & 1);
  }
  __syncthreads();
  if (wv != 0) return;
  const int p = sub * 64 + lane;
  uint32_t taken = 0;
  if (p < T) {
    const int64_t t = tok0 + p;
    double logit[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      double l = part[0][lane][m];
#pragma unroll
      for (int g = 1; g < DG; ++g) l += part[g][lane][m];
      logit[m] = l + (bias && m < M ? (double)bias[m] : 0.0);
    }
    int sel[8];
    double ls[8];
    for (int j = 0; j < K; ++j) {
      int best = -1;
      double bl = 0.0;
#pragma unroll
      for (int m = 0; m < MP; ++m) {
        if (m < M && !((taken >> m) & 1u) && (best < 0 || logit[m] > bl)) {
          best = m;
          bl = logit[m];
        }
      }
      taken |= 1u << best;
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
  for (int m = 0; m < M; ++m) {
    const int n = __popcll(__ballot((taken >> m) & 1u));
    if (lane == 0) cnt[((int64_t)m * B + b) * nsub + sub] = n;
  }
}

template <typename XT, int G>
static void launch_route_g(const mom_dims& d, const void* x, const void* wr, const float* bias, int32_t* idx,
                           float* w, hipStream_t st, int32_t* cnt = nullptr) {
  const int64_t NT = (int64_t)d.B * d.T;
  const int64_t need = (NT + 256 / G - 1) / (256 / G);
  const int blocks = (int)(need < 8192 ? need : 8192);
  const XT* xp = (const XT*)x;
  const XT* wp = (const XT*)wr;
#define MOM_ROUTE_CASE(MT)                                                                                 \
  hipLaunchKernelGGL((k_route<XT, MT, G>), dim3(blocks), dim3(256), 0, st, NT, d.D, d.M, d.topk, xp, wp, \
                     bias, idx, w, cnt)
  if (d.M <= 4) MOM_ROUTE_CASE(4);
  else if (d.M <= 8) MOM_ROUTE_CASE(8);
  else if (d.M <= 16) MOM_ROUTE_CASE(16);
  else if (d.M <= 32) MOM_ROUTE_CASE(32);
  else MOM_ROUTE_CASE(64);
#undef MOM_ROUTE_CASE
}

// bfloat16 with at most four memories and D = 1024: k_route_wave4.
// Otherwise few tokens (decode): a whole wave per token, so the row is read in
// few steps; many tokens: 16 lanes per token, four tokens per wave.
template <typename XT>
static void launch_route(const mom_dims& d, const void* x, const void* wr, const float* bias, int32_t* idx,
                         float* w, hipStream_t st) {
  const int64_t NT = (int64_t)d.B * d.T;
  if constexpr (sizeof(XT) == 2) {
    if (d.M <= 4 && d.D == 1024) {
      // four rows of x in flight per wave; the router slice, held as float64,
      // takes 128 registers, so two waves fit per SIMD
      constexpr int TPW = 4;
      const int64_t waves = (NT + TPW - 1) / TPW;
      const int blocks = (int)(((waves < 8192 ? waves : 8192) + 3) / 4);
      hipLaunchKernelGGL((k_route_wave4<16, TPW>), dim3(blocks), dim3(256), 0, st, NT, d.D, d.M, d.topk,
                         (const bf16_t*)x, (const bf16_t*)wr, bias, idx, w);
      return;
    }
  }
  if (NT < 8192) launch_route_g<XT, 64>(d, x, wr, bias, idx, w, st);
  else launch_route_g<XT, 16>(d, x, wr, bias, idx, w, st);
}

}  // namespace mom

extern "C" mom_status mom_route_count(const mom_dims* dims, const void* x, const void* w_r, const float* bias,
                                      int32_t* idx, float* w, void* ws, size_t ws_bytes, void* stream) {
  using namespace mom;
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  MOM_CHECK_PTR(x);
  MOM_CHECK_PTR(w_r);
  MOM_CHECK_OPT_PTR(bias);
  MOM_CHECK_PTR(idx);
  MOM_CHECK_PTR(w);
  if (!ws || ws_bytes < mom_workspace_bytes(dims, MOM_WS_DISPATCH)) return MOM_ERR_WORKSPACE;
  MOM_CHECK_PTR(ws);
  hipStream_t st = (hipStream_t)stream;
  const mom_dims& d = *dims;
  if (d.T > 1) {  // cnt[m][b][sub]: counts of each 64 positions of each sequence
    int32_t* cnt = (int32_t*)ws;
    const int nsub = (d.T + kCountTile - 1) / kCountTile;
    const dim3 grid((unsigned)nsub, (unsigned)d.B);
    if (d.dtype == MOM_DTYPE_BF16 && ((d.D == 1024 && d.M <= 16) || (d.D == 2048 && d.M <= 4))) {
      const bf16_t* xp = (const bf16_t*)x;
      const bf16_t* wp = (const bf16_t*)w_r;
#define MOM_ROUTE_BLK(MG, DG, NH)                                                                                   \
  hipLaunchKernelGGL((k_route_blk<MG, DG, NH>), grid, dim3(512), 0, st, d.B, d.T, d.D, d.M, d.topk, nsub, xp, wp, \
                     bias, idx, w, cnt)
      if (d.D == 2048) MOM_ROUTE_BLK(1, 2, 4);
      else if (d.M <= 4) MOM_ROUTE_BLK(1, 1, 8);
      else if (d.M <= 8) MOM_ROUTE_BLK(2, 1, 4);
      else MOM_ROUTE_BLK(4, 1, 2);
#undef MOM_ROUTE_BLK
      return launch_status();
    }
    // other shapes: the router, then the dispatch's own counting kernel
    if (d.dtype == MOM_DTYPE_BF16) launch_route<bf16_t>(d, x, w_r, bias, idx, w, st);
    else launch_route<float>(d, x, w_r, bias, idx, w, st);
    const mom_status r = launch_status();
    if (r != MOM_OK) return r;
    return dispatch_count_only(dims, idx, cnt, st);
  }
  int32_t* cnt = (int32_t*)ws;  // the dispatch's count array [M][B][subs], one position per sequence here
  const int64_t NT = dims->B;
  if (dims->dtype == MOM_DTYPE_BF16) {
    if (NT < 8192) launch_route_g<bf16_t, 64>(*dims, x, w_r, bias, idx, w, st, cnt);
    else launch_route_g<bf16_t, 16>(*dims, x, w_r, bias, idx, w, st, cnt);
  } else {
    if (NT < 8192) launch_route_g<float, 64>(*dims, x, w_r, bias, idx, w, st, cnt);
    else launch_route_g<float, 16>(*dims, x, w_r, bias, idx, w, st, cnt);
  }
  return launch_status();
}

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
