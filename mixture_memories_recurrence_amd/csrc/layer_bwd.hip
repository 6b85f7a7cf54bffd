// Gradients of the layer's combine, router and dispatch gathers (the rest of
// the layer's backward pass beside the recurrence's, gdn_chunk_bwd).  The pages
// give no backward formulas; these are the chain rule applied to the forward
// definitions: the combine's weighted sum (jxzklqfsx.com write-up,
// hardware-efficient implementation section), the router's renormalised
// softmax over the top-k logits (podcast.do-not-panic.com page, "Router
// mechanics, step by step") with the top-k choice held fixed (no gradient
// through the selection), and the reordering gathers (the same page, "Solving
// scatter-gather without new kernels").
//
//   combine   out[t] = o_shared[t] + sum_j w[t][j] o[row(t, j)]
//             -> d_o[row(t, j)] = w[t][j] dout[t], d_shared[t] = dout[t],
//                dw[t][j] = <dout[t], o[row(t, j)]>
//   router    dl[idx_j] = w_j (dw_j - sum_j' w_j' dw_j'),
//             dx[t] = sum_j dl_j w_r[idx_j], dw_r[m] = sum_t dl[t][m] x[t],
//             dbias[m] = sum_t dl[t][m]
//   dispatch  gates back to [t][h][memory]; dq[t] = the query gradients of the
//             token's rows summed, shared row first
// Every sum has a fixed order (no atomics), so results are bit-reproducible.
#include "common.h"

namespace mom {

typedef float f4v __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ combine
// One wave per token; lane l owns the float4 pieces l + 64 c of the token's
// [H][dv] row.  dw[t][j] is the wave's sum of the lanes' partial dot products.
template <int KM>
__global__ __launch_bounds__(256) void k_combine_bwd(int64_t n_tok, int K, int hdv4, const int32_t* __restrict__ inv,
                                                     const float* __restrict__ w, const f4v* __restrict__ o_routed,
                                                     const f4v* __restrict__ dout, f4v* __restrict__ d_routed,
                                                     f4v* __restrict__ d_shared, float* __restrict__ dw) {
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= n_tok) return;
  const int lane = threadIdx.x & 63;
  int64_t r[KM];
  float g[KM], dot[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    dot[j] = 0.f;
    if (j < K) {
      r[j] = inv ? (int64_t)inv[t * K + j] : t * K + j;
      g[j] = w[t * K + j];
    }
  }
  for (int e = lane; e < hdv4; e += 64) {
    const f4v d = __builtin_nontemporal_load(dout + t * hdv4 + e);
    __builtin_nontemporal_store(d, d_shared + t * hdv4 + e);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < K) {
        const f4v o = __builtin_nontemporal_load(o_routed + r[j] * hdv4 + e);
        dot[j] = fmaf(d.x, o.x, fmaf(d.y, o.y, fmaf(d.z, o.z, fmaf(d.w, o.w, dot[j]))));
        __builtin_nontemporal_store(d * g[j], d_routed + r[j] * hdv4 + e);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < K) {
      const float s = wave_sum_xor(dot[j]);
      if (lane == 0) dw[t * K + j] = s;
    }
  }
}

// ------------------------------------------------------------------ router
// dl and dx: one wave per token; dl[t][j] (for the selected memories) also
// goes to the workspace for the weight gradient.
template <typename IT, int KM>
__global__ __launch_bounds__(256) void k_route_bwd_dx(int64_t n_tok, int D, int K, const IT* __restrict__ w_r,
                                                      const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      const float* __restrict__ dw, float* __restrict__ dl,
                                                      float* __restrict__ dx) {
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= n_tok) return;
  const int lane = threadIdx.x & 63;
  float wj[KM], dj[KM];
  int mj[KM];
  float sw = 0.f;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < K) {
      wj[j] = w[t * K + j];
      mj[j] = idx[t * K + j];
      sw = fmaf(wj[j], dw[t * K + j], sw);
    }
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < K) {
      dj[j] = wj[j] * (dw[t * K + j] - sw);
      if (lane == 0) dl[t * K + j] = dj[j];
    }
  }
  for (int d = lane; d < D; d += 64) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < K) s = fmaf(dj[j], load_as_f32(w_r + (int64_t)mj[j] * D + d), s);
    dx[t * D + d] = s;
  }
}

// Weight gradient, first pass: block (column chunk c of 256, token tile tt of
// kRouteTile) sums dl[t][m] x[t][d] over its tokens for its 256 columns, one
// column per thread, then writes the tile's partial [M][256]; in chunk 0,
// thread m < M also sums memory m's bias gradient over the tile.  The tile's selections and
// dl are staged in LDS and x is read 8 tokens at a time, so 8 loads per thread
// are in flight.  With MB > 0 (M <= MB) the sums live in registers, one per
// memory (each token adds its K terms through selects); with MB = 0 they live
// in LDS rows per memory.
constexpr int kRouteTile = 128;
template <typename IT, int MB>
__global__ __launch_bounds__(256) void k_route_bwd_dw(int64_t n_tok, int D, int M, int K, const IT* __restrict__ x,
                                                      const int32_t* __restrict__ idx, const float* __restrict__ dl,
                                                      float* __restrict__ part, float* __restrict__ part_b) {
  extern __shared__ float acc_l[];  // MB = 0: [M][256]
  __shared__ int s_idx[kRouteTile * 8];
  __shared__ float s_dl[kRouteTile * 8];
  const int nc = (D + 255) / 256;
  const int c = blockIdx.x % nc, tt = blockIdx.x / nc;
  const int tid = threadIdx.x;
  const int d = 256 * c + tid;
  const bool col = d < D;
  const int64_t t0 = (int64_t)tt * kRouteTile;
  const int nt = (int)min((int64_t)kRouteTile, n_tok - t0);
  for (int i = tid; i < nt * K; i += 256) {
    s_idx[i] = idx[t0 * K + i];
    s_dl[i] = dl[t0 * K + i];
  }
  float acc[MB > 0 ? MB : 1];
#pragma unroll
  for (int m = 0; m < (MB > 0 ? MB : 1); ++m) acc[m] = 0.f;
  if (MB == 0)
    for (int m = 0; m < M; ++m) acc_l[m * 256 + tid] = 0.f;
  __syncthreads();
  for (int tb = 0; tb < nt; tb += 8) {
    float xv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) xv[u] = (col && tb + u < nt) ? load_as_f32(x + (t0 + tb + u) * D + d) : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (tb + u >= nt) break;
      for (int j = 0; j < K; ++j) {
        const int m = s_idx[(tb + u) * K + j];
        const float g = s_dl[(tb + u) * K + j];
        if constexpr (MB > 0) {
#pragma unroll
          for (int mm = 0; mm < MB; ++mm) acc[mm] = fmaf(m == mm ? g : 0.f, xv[u], acc[mm]);
        } else {
          acc_l[m * 256 + tid] = fmaf(g, xv[u], acc_l[m * 256 + tid]);
        }
      }
    }
  }
  const int64_t tile = tt;
  if (col) {
    if constexpr (MB > 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
        if (m < M) part[(tile * M + m) * D + d] = acc[m];
    } else {
      for (int m = 0; m < M; ++m) part[(tile * M + m) * D + d] = acc_l[m * 256 + tid];
    }
  }
  if (c == 0 && tid < M) {
    float sb = 0.f;
    for (int i = 0; i < nt * K; ++i)
      if (s_idx[i] == tid) sb += s_dl[i];
    part_b[tile * M + tid] = sb;
  }
}

// The same first pass for M <= MB <= 8 with 16-byte loads: 256 threads = 32
// groups of 8 columns x 8 token lanes; thread (tl, cg) takes tokens tl, tl + 8,
// ... of the tile and columns 8 cg .. 8 cg + 7 of the chunk of 256, with its
// sums in registers [memory][column]; the 8 token lanes are then added in
// order through LDS.
template <typename IT>
__device__ __forceinline__ void load8(const IT* p, float* v);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename IT, int MB>
__global__ __launch_bounds__(256) void k_route_bwd_dw8(int64_t n_tok, int D, int M, int K, const IT* __restrict__ x,
                                                       const int32_t* __restrict__ idx, const float* __restrict__ dl,
                                                       float* __restrict__ part, float* __restrict__ part_b) {
  __shared__ int s_idx[kRouteTile * 8];
  __shared__ float s_dl[kRouteTile * 8];
  __shared__ float red[8][MB][257];
  const int nc = (D + 255) / 256;
  const int c = blockIdx.x % nc, tt = blockIdx.x / nc;
  const int tid = threadIdx.x, tl = tid >> 5, cg = tid & 31;
  const int d0 = 256 * c + 8 * cg;
  const bool col = d0 < D;  // D is a multiple of 64
  const int64_t t0 = (int64_t)tt * kRouteTile;
  const int nt = (int)min((int64_t)kRouteTile, n_tok - t0);
  for (int i = tid; i < nt * K; i += 256) {
    s_idx[i] = idx[t0 * K + i];
    s_dl[i] = dl[t0 * K + i];
  }
  float acc[MB][8];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
  __syncthreads();
  for (int tb = tl; tb < nt; tb += 16) {
    float xa[8], xb[8];
    const bool hb = tb + 8 < nt;
    if (col) {
      load8<IT>(x + (t0 + tb) * D + d0, xa);
      if (hb) load8<IT>(x + (t0 + tb + 8) * D + d0, xb);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !hb) break;
      const int t = tb + 8 * u;
      const float* xv = u ? xb : xa;
      for (int j = 0; j < K; ++j) {
        const int m = s_idx[t * K + j];
        const float g = s_dl[t * K + j];
#pragma unroll
        for (int mm = 0; mm < MB; ++mm) {
          const float gg = m == mm ? g : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[mm][e] = fmaf(gg, xv[e], acc[mm][e]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tl][m][8 * cg + e] = acc[m][e];
  __syncthreads();
  const int64_t tile = tt;
  for (int i = tid; i < M * 256; i += 256) {
    const int m = i >> 8, cc = i & 255;
    float sum = 0.f;
#pragma unroll
    for (int l = 0; l < 8; ++l) sum += red[l][m][cc];
    if (256 * c + cc < D) part[(tile * M + m) * D + 256 * c + cc] = sum;
  }
  if (c == 0 && tid < M) {
    float sb = 0.f;
    for (int i = 0; i < nt * K; ++i)
      if (s_idx[i] == tid) sb += s_dl[i];
    part_b[tile * M + tid] = sb;
  }
}

// Second pass: tiles summed in order.
__global__ __launch_bounds__(256) void k_route_bwd_sum(int n_tiles, int D, int M, const float* __restrict__ part,
                                                       const float* __restrict__ part_b, float* __restrict__ dw_r,
                                                       float* __restrict__ dbias) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t MD = (int64_t)M * D;
  if (i < MD) {
    float s = 0.f;
    int tt = 0;
    for (; tt + 8 <= n_tiles; tt += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(tt + u) * MD + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; tt < n_tiles; ++tt) s += part[(int64_t)tt * MD + i];
    dw_r[i] = s;
  }
  if (dbias && i < M) {
    float s = 0.f;
    for (int tt = 0; tt < n_tiles; ++tt) s += part_b[(int64_t)tt * M + i];
    dbias[i] = s;
  }
}

// ------------------------------------------------------------------ dispatch
// dq: one thread per float4 of a token's [H][dk] query gradient.
template <int KM>
__global__ __launch_bounds__(256) void k_dispatch_bwd_q(int64_t n_tok, int K, int hdk4, const int32_t* __restrict__ inv,
                                                        const f4v* __restrict__ dq_rows, f4v* __restrict__ dq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_tok * hdk4) return;
  const int64_t t = i / hdk4, e = i % hdk4;
  const int64_t NR = n_tok * K;
  f4v s = dq_rows[(NR + t) * hdk4 + e];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < K) s += dq_rows[(int64_t)inv[t * K + j] * hdk4 + e];
  dq[i] = s;
}

// gates: one thread per (token, head, memory).
__global__ __launch_bounds__(256) void k_dispatch_bwd_gates(int64_t n_tok, int H, int M, int K,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ inv,
                                                            const float* __restrict__ da_p,
                                                            const float* __restrict__ db_p, float* __restrict__ da,
                                                            float* __restrict__ db) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_tok * H * (M + 1)) return;
  const int m = (int)(i % (M + 1));
  const int64_t th = i / (M + 1), t = th / H, h = th % H;
  int64_t r = -1;
  if (m == M) {
    r = n_tok * K + t;
  } else {
    for (int j = 0; j < K; ++j)
      if (idx[t * K + j] == m) r = inv[t * K + j];
  }
  da[i] = r >= 0 ? da_p[r * H + h] : 0.f;
  db[i] = r >= 0 ? db_p[r * H + h] : 0.f;
}

size_t route_bwd_ws_bytes(const mom_dims& d) {
  const int64_t NT = (int64_t)d.B * d.T;
  const int64_t n_tiles = (NT + kRouteTile - 1) / kRouteTile;
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  return (size_t)(up(NT * d.topk * 4) + up(n_tiles * d.M * d.D * 4) + up(n_tiles * d.M * 4));
}

}  // namespace mom

extern "C" mom_status mom_combine_bwd(const mom_dims* dims, int32_t n_tok, const int32_t* inv, const float* w,
                                      const float* o_routed, const float* dout, float* d_o_routed,
                                      float* d_o_shared, float* dw, void* stream) {
  using namespace mom;
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  if (n_tok < 0) return MOM_ERR_DIMS;
  MOM_CHECK_OPT_PTR(inv);
  MOM_CHECK_PTR(w);
  MOM_CHECK_PTR(o_routed);
  MOM_CHECK_PTR(dout);
  MOM_CHECK_PTR(d_o_routed);
  MOM_CHECK_PTR(d_o_shared);
  MOM_CHECK_PTR(dw);
  if (n_tok == 0) return MOM_OK;
  const int hdv4 = dims->H * dims->dv / 4;
  const unsigned blocks = (unsigned)(((int64_t)n_tok + 3) / 4);
#define MOM_CBWD(KM)                                                                                           \
  hipLaunchKernelGGL((k_combine_bwd<KM>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, (int64_t)n_tok,     \
                     dims->topk, hdv4, inv, w, (const f4v*)o_routed, (const f4v*)dout, (f4v*)d_o_routed,        \
                     (f4v*)d_o_shared, dw)
  if (dims->topk <= 2) MOM_CBWD(2);
  else if (dims->topk <= 4) MOM_CBWD(4);
  else MOM_CBWD(8);
#undef MOM_CBWD
  return launch_status();
}

extern "C" mom_status mom_route_bwd(const mom_dims* dims, const void* x, const void* w_r, const int32_t* idx,
                                    const float* w, const float* dw, float* dx, float* dw_r, float* dbias, void* ws,
                                    size_t ws_bytes, void* stream) {
  using namespace mom;
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  MOM_CHECK_PTR(x);
  MOM_CHECK_PTR(w_r);
  MOM_CHECK_PTR(idx);
  MOM_CHECK_PTR(w);
  MOM_CHECK_PTR(dw);
  MOM_CHECK_PTR(dx);
  MOM_CHECK_PTR(dw_r);
  MOM_CHECK_OPT_PTR(dbias);
  const mom_dims& d = *dims;
  if (!ws || ws_bytes < route_bwd_ws_bytes(d)) return MOM_ERR_WORKSPACE;
  MOM_CHECK_PTR(ws);
  const int64_t NT = (int64_t)d.B * d.T;
  const int64_t n_tiles = (NT + kRouteTile - 1) / kRouteTile;
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  float* dl = (float*)ws;
  float* part = (float*)((char*)ws + up(NT * d.topk * 4));
  float* part_b = (float*)((char*)part + up(n_tiles * d.M * d.D * 4));
  hipStream_t st = (hipStream_t)stream;
  const unsigned tb = (unsigned)((NT + 3) / 4);
  const unsigned wb = (unsigned)(n_tiles * ((d.D + 255) / 256));
  const size_t lds = d.M > 16 ? (size_t)d.M * 256 * sizeof(float) : 0;  // M > 16: LDS sums, up to 64 KB
  if (d.M > 16) {
    static bool attr[2] = {false, false};  // the dynamic LDS limit is raised once per kernel
    const int ai = d.dtype == MOM_DTYPE_BF16 ? 0 : 1;
    if (!attr[ai]) {
      const void* f = ai == 0 ? (const void*)k_route_bwd_dw<bf16_t, 0> : (const void*)k_route_bwd_dw<float, 0>;
      if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 256 * 4) != hipSuccess)
        return MOM_ERR_LAUNCH;
      attr[ai] = true;
    }
  }
#define MOM_RBWD(IT, KM)                                                                                         \
  hipLaunchKernelGGL((k_route_bwd_dx<IT, KM>), dim3(tb), dim3(256), 0, st, NT, d.D, d.topk, (const IT*)w_r, idx, \
                     w, dw, dl, dx)
#define MOM_RBWD_DW(IT, MB)                                                                                       \
  hipLaunchKernelGGL((k_route_bwd_dw<IT, MB>), dim3(wb), dim3(256), lds, st, NT, d.D, d.M, d.topk, (const IT*)x, \
                     idx, dl, part, part_b)
#define MOM_RBWD_DW8(IT, MB)                                                                                   \
  hipLaunchKernelGGL((k_route_bwd_dw8<IT, MB>), dim3(wb), dim3(256), 0, st, NT, d.D, d.M, d.topk, (const IT*)x, \
                     idx, dl, part, part_b)
#define MOM_RBWD_ALL(IT)           \
  do {                             \
    if (d.topk <= 2) MOM_RBWD(IT, 2); \
    else if (d.topk <= 4) MOM_RBWD(IT, 4); \
    else MOM_RBWD(IT, 8);          \
    if (d.M <= 4) MOM_RBWD_DW8(IT, 4); \
    else if (d.M <= 8) MOM_RBWD_DW8(IT, 8); \
    else if (d.M <= 16) MOM_RBWD_DW(IT, 16); \
    else MOM_RBWD_DW(IT, 0);       \
  } while (0)
  if (d.dtype == MOM_DTYPE_BF16) MOM_RBWD_ALL(bf16_t);
  else MOM_RBWD_ALL(float);
#undef MOM_RBWD_ALL
#undef MOM_RBWD_DW8
#undef MOM_RBWD_DW
#undef MOM_RBWD
  hipLaunchKernelGGL(k_route_bwd_sum, dim3((unsigned)(((int64_t)d.M * d.D + 255) / 256)), dim3(256), 0, st,
                     (int)n_tiles, d.D, d.M, part, part_b, dw_r, dbias);
  return launch_status();
}

extern "C" mom_status mom_dispatch_bwd(const mom_dims* dims, const int32_t* idx, const int32_t* inv,
                                       const float* d_alpha_p, const float* d_beta_p, const float* dq_rows,
                                       float* d_alpha, float* d_beta, float* dq, void* stream) {
  using namespace mom;
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  MOM_CHECK_PTR(idx);
  MOM_CHECK_PTR(inv);
  MOM_CHECK_PTR(d_alpha_p);
  MOM_CHECK_PTR(d_beta_p);
  MOM_CHECK_PTR(dq_rows);
  MOM_CHECK_PTR(d_alpha);
  MOM_CHECK_PTR(d_beta);
  MOM_CHECK_PTR(dq);
  const mom_dims& d = *dims;
  const int64_t NT = (int64_t)d.B * d.T;
  hipStream_t st = (hipStream_t)stream;
  const int hdk4 = d.H * d.dk / 4;
  const unsigned qb = (unsigned)((NT * hdk4 + 255) / 256);
  if (d.topk <= 2)
    hipLaunchKernelGGL((k_dispatch_bwd_q<2>), dim3(qb), dim3(256), 0, st, NT, d.topk, hdk4, inv,
                       (const f4v*)dq_rows, (f4v*)dq);
  else if (d.topk <= 4)
    hipLaunchKernelGGL((k_dispatch_bwd_q<4>), dim3(qb), dim3(256), 0, st, NT, d.topk, hdk4, inv,
                       (const f4v*)dq_rows, (f4v*)dq);
  else
    hipLaunchKernelGGL((k_dispatch_bwd_q<8>), dim3(qb), dim3(256), 0, st, NT, d.topk, hdk4, inv,
                       (const f4v*)dq_rows, (f4v*)dq);
  const unsigned gb = (unsigned)((NT * d.H * (d.M + 1) + 255) / 256);
  hipLaunchKernelGGL(k_dispatch_bwd_gates, dim3(gb), dim3(256), 0, st, NT, d.H, d.M, d.topk, idx, inv, d_alpha_p,
                     d_beta_p, d_alpha, d_beta);
  return launch_status();
}
