// Chunkwise Gated DeltaNet, float32 vector-ALU version: the float32 path of
// gdn_chunk_fwd and the plain reference shape of the matrix-core kernel.
//
// Per memory, per head, the state S [dk][dv] follows
//   S_i = a_i S_{i-1} + k_i u_i^T,   u_i = c_i (v_i - a_i S_{i-1}^T k_i),
//   o_i = S_i^T q_i
// (gist.science page, "Core mechanism": forget then delta update; read after
// the write).  Inside a chunk of L rows entering with state S, with
// g_i = sum_{j<=i} log a_j:
//   A_ij = c_i e^{g_i-g_j} k_i.k_j  (j < i),  R_i = c_i (v_i - e^{g_i} S^T k_i)
//   (I + A) U = R                       (forward substitution, the UT form)
//   o_i = e^{g_i} S^T q_i + sum_{j<=i} e^{g_i-g_j} (q_i.k_j) u_j
//   S  <- e^{g_L} S + sum_j e^{g_L-g_j} k_j u_j^T
// Value columns evolve independently, so one block owns (segment, head,
// 32-column block) and the grid spreads over all of them.
// With DELTA false the memories use gated linear attention instead
// (S_i = a_i S_{i-1} + c_i k_i v_i^T): A = 0 and R = diag(c) V, so the
// substitution and the K S product drop out.
#include "common.h"

namespace mom {

constexpr int VDVB = 32;  // value columns per block

// VC: chunk rows (16, 32 or 64; the chunk form's result does not depend on it
// beyond rounding)
template <typename IT, int DK, bool DELTA, int VC>
__global__ __launch_bounds__(256) void k_gdn_chunk_valu(int H, int dv, int n_seg, const int32_t* __restrict__ seg_off,
                                                        const int32_t* __restrict__ seg_state,
                                                        const int32_t* __restrict__ row_token, const IT* __restrict__ q,
                                                        const IT* __restrict__ k, const IT* __restrict__ v,
                                                        const float* __restrict__ alpha_p,
                                                        const float* __restrict__ beta_p,
                                                        const float* __restrict__ state_in,
                                                        float* __restrict__ state_out, float* __restrict__ o) {
  __shared__ float Ks[VC][DK + 1];
  __shared__ float Qs[VC][DK + 1];
  __shared__ float Ss[DK][VDVB];
  __shared__ float As[VC][VC + 1];
  __shared__ float Ps[VC][VC + 1];
  __shared__ float Us[VC][VDVB + 1];
  __shared__ double gs[VC];  // prefix sums of log a in float64 (see log_gate_f64)
  __shared__ float bs[VC];

  const int nb = dv / VDVB;
  const int cb = blockIdx.x % nb;
  const int h = (blockIdx.x / nb) % H;
  const int s = blockIdx.x / (nb * H);
  if (s >= n_seg) return;
  const int tid = threadIdx.x;
  const int slot = seg_state ? seg_state[s] : s;
  const int64_t sbase = ((int64_t)slot * H + h) * DK * dv + cb * VDVB;
  for (int e = tid; e < DK * VDVB; e += 256) {
    const int d = e / VDVB, n = e % VDVB;
    Ss[d][n] = state_in ? state_in[sbase + (int64_t)d * dv + n] : 0.f;
  }
  const int64_t r_beg = seg_off[s], r_end = seg_off[s + 1];
  for (int64_t r0 = r_beg; r0 < r_end; r0 += VC) {
    const int L = (int)(r_end - r0 < VC ? r_end - r0 : VC);
    __syncthreads();
    for (int e = tid; e < L * DK; e += 256) {
      const int i = e / DK, d = e % DK;
      const int64_t row = r0 + i;
      const int64_t tk = row_token ? (int64_t)row_token[row] : row;
      Ks[i][d] = load_as_f32(k + (row * H + h) * DK + d);
      Qs[i][d] = load_as_f32(q + (tk * H + h) * DK + d);
    }
    if (tid == 0) {
      double g = 0.0;
      for (int i = 0; i < L; ++i) {
        g += log_gate_f64(alpha_p[(r0 + i) * H + h]);
        gs[i] = g;
        bs[i] = beta_p[(r0 + i) * H + h];
      }
    }
    __syncthreads();
    // A (strictly lower) and P (lower incl. diagonal)
    for (int e = tid; e < VC * VC; e += 256) {
      const int i = e / VC, j = e % VC;
      float a = 0.f, p = 0.f;
      if (i < L && j <= i) {
        float kk = 0.f, qk = 0.f;
        for (int d = 0; d < DK; ++d) {
          kk = fmaf(Ks[i][d], Ks[j][d], kk);
          qk = fmaf(Qs[i][d], Ks[j][d], qk);
        }
        const float dec = expf((float)(gs[i] - gs[j]));
        if (DELTA && j < i) a = bs[i] * dec * kk;
        p = dec * qk;
      }
      As[i][j] = a;
      Ps[i][j] = p;
    }
    // R = diag(c) (V - diag(e^g) K S)
    for (int e = tid; e < VC * VDVB; e += 256) {
      const int i = e / VDVB, n = e % VDVB;
      float r = 0.f;
      if (i < L) {
        const float vv = load_as_f32(v + ((r0 + i) * H + h) * dv + cb * VDVB + n);
        if (DELTA) {
          float ks = 0.f;
          for (int d = 0; d < DK; ++d) ks = fmaf(Ks[i][d], Ss[d][n], ks);
          r = bs[i] * (vv - expf((float)gs[i]) * ks);
        } else {
          r = bs[i] * vv;
        }
      }
      Us[i][n] = r;
    }
    __syncthreads();
    // (I + A) U = R, one thread per value column
    if (DELTA && tid < VDVB) {
      for (int i = 1; i < L; ++i) {
        float u = Us[i][tid];
        for (int j = 0; j < i; ++j) u = fmaf(-As[i][j], Us[j][tid], u);
        Us[i][tid] = u;
      }
    }
    __syncthreads();
    // O = diag(e^g) Q S + P U   (reads the entering state)
    for (int e = tid; e < VC * VDVB; e += 256) {
      const int i = e / VDVB, n = e % VDVB;
      if (i < L) {
        float qs = 0.f;
        for (int d = 0; d < DK; ++d) qs = fmaf(Qs[i][d], Ss[d][n], qs);
        float acc = expf((float)gs[i]) * qs;
        for (int j = 0; j <= i; ++j) acc = fmaf(Ps[i][j], Us[j][n], acc);
        o[((r0 + i) * H + h) * dv + cb * VDVB + n] = acc;
      }
    }
    __syncthreads();
    // S <- e^{g_L} S + K~^T U
    const double gL = gs[L - 1];
    for (int e = tid; e < DK * VDVB; e += 256) {
      const int d = e / VDVB, n = e % VDVB;
      float acc = expf((float)gL) * Ss[d][n];
      for (int j = 0; j < L; ++j) acc = fmaf(expf((float)(gL - gs[j])) * Ks[j][d], Us[j][n], acc);
      Ss[d][n] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < DK * VDVB; e += 256) {
    const int d = e / VDVB, n = e % VDVB;
    state_out[sbase + (int64_t)d * dv + n] = Ss[d][n];
  }
}

template <typename IT>
mom_status launch_gdn_chunk_valu(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                                 const int32_t* row_token, const void* q, const void* k, const void* v,
                                 const float* alpha_p, const float* beta_p, const float* state_in, float* state_out,
                                 float* o, bool delta, hipStream_t st) {
  const int64_t blocks = (int64_t)n_seg * d.H * (d.dv / VDVB);
  if (blocks == 0) return MOM_OK;
#define MOM_VALU_VC(DK, DELTA, VC)                                                                                \
  hipLaunchKernelGGL((k_gdn_chunk_valu<IT, DK, DELTA, VC>), dim3((unsigned)blocks), dim3(256), 0, st, d.H, d.dv, \
                     n_seg, seg_off, seg_state, row_token, (const IT*)q, (const IT*)k, (const IT*)v, alpha_p,      \
                     beta_p, state_in, state_out, o)
#define MOM_VALU_CASE(DK, DELTA)        \
  do {                                  \
    if (d.chunk == 16)                  \
      MOM_VALU_VC(DK, DELTA, 16);       \
    else if (d.chunk == 32)             \
      MOM_VALU_VC(DK, DELTA, 32);       \
    else                                \
      MOM_VALU_VC(DK, DELTA, 64);       \
  } while (0)
  if (d.dk == 64) {
    if (delta) MOM_VALU_CASE(64, true);
    else MOM_VALU_CASE(64, false);
  } else {
    if (delta) MOM_VALU_CASE(128, true);
    else MOM_VALU_CASE(128, false);
  }
#undef MOM_VALU_CASE
#undef MOM_VALU_VC
  return launch_status();
}

template mom_status launch_gdn_chunk_valu<float>(const mom_dims&, int, const int32_t*, const int32_t*,
                                                 const int32_t*, const void*, const void*, const void*,
                                                 const float*, const float*, const float*, float*, float*,
                                                 bool, hipStream_t);
template mom_status launch_gdn_chunk_valu<f16_t>(const mom_dims&, int, const int32_t*, const int32_t*,
                                                 const int32_t*, const void*, const void*, const void*,
                                                 const float*, const float*, const float*, float*, float*,
                                                 bool, hipStream_t);

}  // namespace mom
