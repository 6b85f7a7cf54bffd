// Gradients of the recurrence with float32 storage: the float32 path of
// gdn_chunk_bwd / gla_chunk_bwd (and of the training pair, which for float32
// keeps nothing between its two calls).  The pages give no backward formulas;
// these are the chain rule on the token recurrence of one memory (gist.science
// page, "Core mechanism": forget then delta update, read after the write)
//   w_i = S_{i-1}^T k_i,  u_i = c_i (v_i - a_i w_i),
//   S_i = a_i S_{i-1} + k_i u_i^T,  o_i = S_i^T q_i
// (gated linear attention: u_i = c_i v_i), evaluated row by row in float32 on
// the vector ALUs.  Going back from dS = dL/dS_i (dstate_out at the end):
//   dS += q_i do_i^T,  dq_i = S_i do_i,  du = dS^T k_i,  dv_i = c_i du
//   Gated DeltaNet, with g = -c_i du:
//     dc_i = du . (v_i - a_i w_i),  dk_i = dS u_i + a_i S_{i-1} g,
//     da_i = <S_{i-1}, dS> + w_i . g,  dS <- a_i (dS + k_i g^T)
//   gated linear attention:
//     dc_i = du . v_i,  dk_i = dS u_i,  da_i = <S_{i-1}, dS>,  dS <- a_i dS
// and dL/d(entering state) is the final dS.  The states S_{i-1} are
// recomputed: a forward pass stores the state entering every 64-row chunk;
// going back over a chunk, a forward pass from its entering state stores the
// state at every 8th row, and each row's S_{i-1} is recomputed from the
// nearest one before it (at most 7 steps).
//
// One block per (segment, head, 64 value columns), 256 threads: thread t owns
// column t / 4 of the block and rows t % 4 + 4 j of S and dS.  Sums over rows
// are four-lane shuffles; sums over columns (dq, dk and the scalars da, dc) go
// through shuffles inside a wave and then LDS across the four waves, added in
// a fixed order.  With more than one column block per head, every block
// writes partial dq, dk, da, dc, which k_bwd_valu_sum adds in column-block
// order; results do not depend on scheduling.
#include "chunk_mfma.h"

namespace mom {

constexpr int BV_COLS = 64;  // value columns per block
constexpr int BV_SUB = 8;    // rows between recomputation checkpoints

template <int DK>
struct BwdValu {
  static constexpr int RPT = DK / 4;  // state rows per thread
};

// Workspace (float32): the state entering every chunk [chunk][H][DK][dv]; per
// block the chunk's checkpoints every 8 rows [block][8][256][RPT]; with more
// than one column block, partial dq, dk [cb][n_rows][H][DK] and da, dc
// [cb][n_rows][H].
struct BwdValuWs {
  float *ckpt, *sub, *pq, *pk, *pa, *pc;
  size_t bytes;
};

inline BwdValuWs bwd_valu_ws_layout(void* base, int64_t n_seg, int64_t n_rows, int H, int dk, int dv) {
  auto a256 = [](size_t b) { return (b + 255) / 256 * 256; };
  const int64_t nch = n_rows / GC + n_seg, nb = dv / BV_COLS, n_blk = n_seg * H * nb;
  const size_t s_ckpt = a256((size_t)nch * H * dk * dv * 4), s_sub = a256((size_t)n_blk * BV_SUB * dk * BV_COLS * 4);
  const size_t s_pv = nb > 1 ? a256((size_t)nb * n_rows * H * dk * 4) : 0,
               s_ps = nb > 1 ? a256((size_t)nb * n_rows * H * 4) : 0;
  BwdValuWs w;
  char* p = (char*)base;
  w.ckpt = (float*)p;
  w.sub = (float*)(p + s_ckpt);
  w.pq = (float*)(p + s_ckpt + s_sub);
  w.pk = (float*)(p + s_ckpt + s_sub + s_pv);
  w.pa = (float*)(p + s_ckpt + s_sub + 2 * s_pv);
  w.pc = (float*)(p + s_ckpt + s_sub + 2 * s_pv + s_ps);
  w.bytes = s_ckpt + s_sub + 2 * s_pv + 2 * s_ps;
  return w;
}

size_t gdn_bwd_valu_ws_bytes(int64_t n_seg, int64_t n_rows, int H, int dk, int dv) {
  return bwd_valu_ws_layout(nullptr, n_seg, n_rows, H, dk, dv).bytes;
}

template <int DK, bool DELTA>
__global__ __launch_bounds__(256) void k_bwd_valu(
    int H, int dv, int n_seg, int n_rows, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_state,
    const int32_t* __restrict__ row_token, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ alpha_p, const float* __restrict__ beta_p,
    const float* __restrict__ state_in, const float* __restrict__ d_o, const float* __restrict__ dstate_out,
    float* __restrict__ dv_out, float* __restrict__ dstate_in, float* __restrict__ ckpt, float* __restrict__ sub,
    float* __restrict__ oq, float* __restrict__ ok, float* __restrict__ oa, float* __restrict__ oc) {
  constexpr int RPT = BwdValu<DK>::RPT;
  __shared__ float red_q[2][4][DK], red_k[2][4][DK], red_s[2][4][2];
  const int nb = dv / BV_COLS;
  const int cb = blockIdx.x % nb, h = (blockIdx.x / nb) % H, s = blockIdx.x / (nb * H);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, rg = tid & 3;
  const int col = cb * BV_COLS + (tid >> 2);  // this thread's value column
  const int slot = seg_state ? seg_state[s] : s;
  const int64_t rbeg = seg_off[s], rend = seg_off[s + 1];
  const int cbase = chunks_before(seg_off, s, lane);
  const int64_t sbase = ((int64_t)slot * H + h) * DK * dv + col;  // + d * dv
  // partial outputs of this column block (the outputs themselves when nb == 1)
  const int64_t pofs = (int64_t)cb * n_rows * H;
  float* sub_b = sub + (int64_t)blockIdx.x * BV_SUB * DK * BV_COLS + tid * RPT;

  float S[RPT], kr[RPT];
  // one forward step of row r on S (S_{r-1} -> S_r); w = S_{r-1}^T k_r of this column
  auto step = [&](int64_t r) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) kr[j] = k[(r * H + h) * DK + rg + 4 * j];
    const float a = alpha_p[r * H + h], c = beta_p[r * H + h];
    const float vv = v[(r * H + h) * dv + col];
    float u;
    if constexpr (DELTA) {
      float w = 0.f;
#pragma unroll
      for (int j = 0; j < RPT; ++j) w = fmaf(S[j], kr[j], w);
      w += __shfl_xor(w, 1, 64);
      w += __shfl_xor(w, 2, 64);
      u = c * (vv - a * w);
    } else {
      u = c * vv;
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) S[j] = fmaf(a, S[j], kr[j] * u);
  };

  // ---- forward: the state entering every chunk
#pragma unroll
  for (int j = 0; j < RPT; ++j) S[j] = state_in ? state_in[sbase + (int64_t)(rg + 4 * j) * dv] : 0.f;
  for (int64_t r = rbeg; r < rend; ++r) {
    if ((r - rbeg) % GC == 0) {
      float* cp = ckpt + ((int64_t)(cbase + (r - rbeg) / GC) * H + h) * DK * dv + col;
#pragma unroll
      for (int j = 0; j < RPT; ++j) cp[(int64_t)(rg + 4 * j) * dv] = S[j];
    }
    step(r);
  }

  // ---- backward, chunk by chunk from the last
  float dS[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) dS[j] = dstate_out ? dstate_out[sbase + (int64_t)(rg + 4 * j) * dv] : 0.f;
  int buf = 0;
  const int nch = (int)((rend - rbeg + GC - 1) / GC);
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int64_t r0 = rbeg + (int64_t)ci * GC;
    const int L = (int)min((int64_t)GC, rend - r0);
    const float* cp = ckpt + ((int64_t)(cbase + ci) * H + h) * DK * dv + col;
#pragma unroll
    for (int j = 0; j < RPT; ++j) S[j] = cp[(int64_t)(rg + 4 * j) * dv];
    for (int t = 0; t < L; ++t) {  // checkpoints every 8 rows (this thread's own values)
      if (t % BV_SUB == 0)
#pragma unroll
        for (int j = 0; j < RPT; ++j) sub_b[(t / BV_SUB) * DK * BV_COLS + j] = S[j];
      step(r0 + t);
    }
    for (int t = L - 1; t >= 0; --t) {
      const int t0 = t - t % BV_SUB;
#pragma unroll
      for (int j = 0; j < RPT; ++j) S[j] = sub_b[(t0 / BV_SUB) * DK * BV_COLS + j];
      for (int tt = t0; tt < t; ++tt) step(r0 + tt);
      // S = S_{r-1} of row r
      const int64_t r = r0 + t;
      const int64_t tk = row_token ? (int64_t)row_token[r] : r;
      float qr[RPT];
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        qr[j] = q[(tk * H + h) * DK + rg + 4 * j];
        kr[j] = k[(r * H + h) * DK + rg + 4 * j];
      }
      const float a = alpha_p[r * H + h], c = beta_p[r * H + h];
      const float vv = v[(r * H + h) * dv + col], dov = d_o[(r * H + h) * dv + col];
      float w = 0.f, u;
      if constexpr (DELTA) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) w = fmaf(S[j], kr[j], w);
        w += __shfl_xor(w, 1, 64);
        w += __shfl_xor(w, 2, 64);
        u = c * (vv - a * w);
      } else {
        u = c * vv;
      }
      float pq[RPT], pk[RPT], du = 0.f, pa = 0.f;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const float si = fmaf(a, S[j], kr[j] * u);  // S_r
        dS[j] = fmaf(qr[j], dov, dS[j]);
        pq[j] = si * dov;
        du = fmaf(dS[j], kr[j], du);
        pa = fmaf(S[j], dS[j], pa);
      }
      du += __shfl_xor(du, 1, 64);
      du += __shfl_xor(du, 2, 64);
      if (rg == 0) dv_out[(r * H + h) * dv + col] = c * du;
      float pc;
      if constexpr (DELTA) {
        const float g = -c * du;
        pc = rg == 0 ? du * (vv - a * w) : 0.f;
        if (rg == 0) pa = fmaf(w, g, pa);
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          pk[j] = fmaf(dS[j], u, a * S[j] * g);
          dS[j] = a * fmaf(kr[j], g, dS[j]);
        }
      } else {
        pc = rg == 0 ? du * vv : 0.f;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          pk[j] = dS[j] * u;
          dS[j] = a * dS[j];
        }
      }
      // sums over the block's columns: lanes of one row group inside the wave
      // (xor 4 .. 32), then the four waves through LDS in wave order
#pragma unroll
      for (int o = 4; o < 64; o <<= 1) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          pq[j] += __shfl_xor(pq[j], o, 64);
          pk[j] += __shfl_xor(pk[j], o, 64);
        }
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        pa += __shfl_xor(pa, o, 64);
        pc += __shfl_xor(pc, o, 64);
      }
      if (lane < 4)
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          red_q[buf][wv][lane + 4 * j] = pq[j];
          red_k[buf][wv][lane + 4 * j] = pk[j];
        }
      if (lane == 0) {
        red_s[buf][wv][0] = pa;
        red_s[buf][wv][1] = pc;
      }
      __syncthreads();
      if (tid < DK) {
        const int64_t o = (pofs + r * H + h) * DK + tid;
        oq[o] = ((red_q[buf][0][tid] + red_q[buf][1][tid]) + red_q[buf][2][tid]) + red_q[buf][3][tid];
        ok[o] = ((red_k[buf][0][tid] + red_k[buf][1][tid]) + red_k[buf][2][tid]) + red_k[buf][3][tid];
      } else if (tid == DK) {
        oa[pofs + r * H + h] = ((red_s[buf][0][0] + red_s[buf][1][0]) + red_s[buf][2][0]) + red_s[buf][3][0];
        oc[pofs + r * H + h] = ((red_s[buf][0][1] + red_s[buf][1][1]) + red_s[buf][2][1]) + red_s[buf][3][1];
      }
      buf ^= 1;  // the next row writes the other half; this barrier orders the reuse
    }
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) dstate_in[sbase + (int64_t)(rg + 4 * j) * dv] = dS[j];
}

// dq, dk, d_alpha, d_beta of the rows in [seg_off[0], seg_off[n_seg]) as the
// sums of the column blocks' partials, in column-block order.
__global__ __launch_bounds__(256) void k_bwd_valu_sum(int H, int dk, int nb, int n_rows, int n_seg,
                                                      const int32_t* __restrict__ seg_off,
                                                      const float* __restrict__ pq, const float* __restrict__ pk,
                                                      const float* __restrict__ pa, const float* __restrict__ pc,
                                                      float* __restrict__ dq, float* __restrict__ dk_out,
                                                      float* __restrict__ da, float* __restrict__ dc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, head, element)
  const int64_t per = (int64_t)H * (dk + 2);
  const int64_t r = i / per;
  if (r >= n_rows || r < seg_off[0] || r >= seg_off[n_seg]) return;
  const int64_t e = i % per, hh = e / (dk + 2), x = e % (dk + 2);
  const int64_t stride_v = (int64_t)n_rows * H * dk, stride_s = (int64_t)n_rows * H;
  if (x < dk) {
    const int64_t o = (r * H + hh) * dk + x;
    float sq = 0.f, sk = 0.f;
    for (int b = 0; b < nb; ++b) {
      sq += pq[b * stride_v + o];
      sk += pk[b * stride_v + o];
    }
    dq[o] = sq;
    dk_out[o] = sk;
  } else {
    const int64_t o = r * H + hh;
    const float* p = x == dk ? pa : pc;
    float sum = 0.f;
    for (int b = 0; b < nb; ++b) sum += p[b * stride_s + o];
    (x == dk ? da : dc)[o] = sum;
  }
}

mom_status launch_gdn_bwd_valu(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                               const int32_t* seg_state, const int32_t* row_token, const float* q, const float* k,
                               const float* v, const float* alpha_p, const float* beta_p, const float* state_in,
                               const float* d_o, const float* dstate_out, float* dq, float* dk, float* dv_out,
                               float* da, float* dc, float* dstate_in, void* ws, bool delta, hipStream_t st) {
  const BwdValuWs W = bwd_valu_ws_layout(ws, n_seg, n_rows, d.H, d.dk, d.dv);
  const int nb = d.dv / BV_COLS;
  float *oq = dq, *ok = dk, *oa = da, *oc = dc;
  if (nb > 1) {
    oq = W.pq;
    ok = W.pk;
    oa = W.pa;
    oc = W.pc;
  }
  const int64_t blocks = (int64_t)n_seg * d.H * nb;
#define MOM_BV(DK, DELTA)                                                                                          \
  hipLaunchKernelGGL((k_bwd_valu<DK, DELTA>), dim3((unsigned)blocks), dim3(256), 0, st, d.H, d.dv, n_seg, n_rows, \
                     seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p, state_in, d_o, dstate_out, dv_out,  \
                     dstate_in, W.ckpt, W.sub, oq, ok, oa, oc)
  if (d.dk == 64) {
    if (delta) MOM_BV(64, true);
    else MOM_BV(64, false);
  } else {
    if (delta) MOM_BV(128, true);
    else MOM_BV(128, false);
  }
#undef MOM_BV
  if (nb > 1) {
    const int64_t n = (int64_t)n_rows * d.H * (d.dk + 2);
    hipLaunchKernelGGL(k_bwd_valu_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, d.H, d.dk, nb, n_rows,
                       n_seg, seg_off, W.pq, W.pk, W.pa, W.pc, dq, dk, da, dc);
  }
  return launch_status();
}

}  // namespace mom
