// Gradients of the chunkwise recurrence (gdn_chunk_bwd, gla_chunk_bwd): the
// reverse-mode derivative of what gdn_chunk_fwd computes, for training (the
// jxzklqfsx.com write-up, introduction: training in linear time; the pages give
// no backward formulas, so these are the chain rule applied to the chunk form).
//
// Forward, per chunk of rows entering with state S (notation of the forward
// kernels: g = prefix sums of log a, gm = e^g, ek = e^{g_L - g}, A, X = (I+A)^-1,
// T = X diag(c), P):
//   R = V - diag(gm) K S          (R = V for gated linear attention)
//   U = T R,   O = diag(gm) Q S + P U,   S' = gm_L S + K^T diag(ek) U
// Reverse, given dO and dS' = dL/dS':
//   dU = P^T dO + diag(ek) K dS',   dR = T^T dU,   dV = dR
//   dS = gm_L dS' + Q^T diag(gm) dO - K^T diag(gm) dR
// and, summed over the value columns,
//   PQ = dO S^T,  PR = dR S^T,  PK = U dS'^T,  dT = lower(dU R^T),  dP = lower(dO U^T)
// from which
//   dQ = diag(gm) PQ + D K,       D = dP o e^{g_i - g_j}
//   dK = diag(ek) PK - diag(gm) PR + (B + B^T) K + D^T Q,
//        B = dA o c_i e^{g_i - g_j} (j < i),  dA = -X^T (dT diag(c)) X^T
//   dc_i = sum_r dT_ri X_ri + sum_j dA_ij e^{g_i - g_j} k_i.k_j
//   dg_i = gm_i q_i.PQ_i - gm_i k_i.PR_i - ek_i k_i.PK_i  (+ sum_j e_j and
//          gm_L <S, dS'> at the last row)  + rowsum - colsum of
//          (c_i G_ij + D_ij q_i.k_j),  G_ij = dA_ij e^{g_i - g_j} k_i.k_j,
//   d log a_i = sum_{i' >= i} dg_i',  da_i = d log a_i / a_i.
// k_i.PR_i = dR_i.(K S)_i and k_i.PK_i = U_i.(K dS')_i are formed per value
// slice from tiles the kernel has anyway.
//
// Launches:
//   k_gdn_prep         T, P, decays and X (half) per (chunk, head)
//   k_gdn_chain16 mode 1  the state entering every chunk, transposed half S^T
//   k_gdn_chain_bwd    reverse walk over each segment's chunks with dS in
//                      matrix-core accumulators; stores dS' of every chunk
//                      (transposed half) and dL/d(entering state)
//   k_gdn_grad         one block per (chunk, head): everything else
// A training step can skip the first two: gdn_chunk_fwd_train runs the forward
// pass with the prep that also writes X and a walk that also stores the
// states (k_gdn_chain16 mode 2), into this workspace, and gdn_chunk_bwd_saved
// then starts at the reverse walk.
#include "chunk_mfma.h"

namespace mom {

mom_status launch_chunk_states(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                               const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                               const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                               float* state_out, float* o, const ChunkWs& W, f16_t* Xws, f16_t* hws, bool delta,
                               bool with_output, hipStream_t st);

// ------------------------------------------------------------------ reverse chain
// One block per (segment, head, DVB = 32 NW value columns), NW waves, mapped to
// the XCDs as the forward walk.  Wave w owns value columns [32 w, 32 w + 32) of
// dS for every key row, in float32 accumulators.  The chunks are walked from
// the last to the first; the previous chunk's K, Q, T, P and decays are
// prefetched into the other half of an LDS double buffer, and its dO (float32)
// into registers.  Per chunk:
//   store dS (= dS' of this chunk)                      transposed half
//   Z  = K dS,   dU = P^T dO + diag(ek) Z
//   dR = T^T dU                                          (Gated DeltaNet)
//   dS <- gm_L dS + Q^T diag(gm) dO - K^T diag(gm) dR
template <int DK, int NW>
struct ChainBwdLds {
  static constexpr int DVB = 32 * NW;
  static constexpr int OFF_K = 0, OFF_Q = GC * DK, OFF_T = 2 * GC * DK, OFF_P = OFF_T + GC * GC,
                       OFF_E = OFF_P + GC * GC, OFF_TOK = OFF_E + 2 * 2 * GC;
  static constexpr int BUF = OFF_TOK + 2 * GC;  // halfs per buffer
  // after the two buffers: one 4 KB tile per wave for the dS' stores
  static constexpr size_t OST = (size_t)2 * BUF * sizeof(f16_t);
  static constexpr size_t BYTES = OST + (size_t)NW * 4096;
};

template <int DK, int NW, bool DELTA>
__global__ __launch_bounds__(64 * NW) void k_gdn_chain_bwd(
    int H, int dv, int n_seg, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_state,
    const f16_t* __restrict__ k, const f16_t* __restrict__ Tws, const f16_t* __restrict__ Pws,
    const float* __restrict__ Ews, const int32_t* __restrict__ row_token, const f16_t* __restrict__ q,
    const float* __restrict__ d_o, const float* __restrict__ dstate_out, float* __restrict__ dstate_in,
    f16_t* __restrict__ dhws) {
  using LY = ChainBwdLds<DK, NW>;
  constexpr int DVB = LY::DVB, ND = DK / 32, NKD = DK / 16;
  extern __shared__ __attribute__((aligned(16))) f16_t smem[];

  const int nb = dv / DVB;
  const int64_t pblk = blockIdx.x;
  const int64_t n_grp = (int64_t)n_seg * H;
  const int64_t full = (n_grp / 8) * 8;
  int64_t grp;
  int cb;
  if (pblk < full * nb) {
    const int64_t xi = pblk & 7, ii = pblk >> 3;
    grp = (ii / nb) * 8 + xi;
    cb = (int)(ii % nb);
  } else {
    const int64_t r = pblk - full * nb;
    grp = full + r / nb;
    cb = (int)(r % nb);
  }
  const int h = (int)(grp % H);
  const int s = n_seg - 1 - (int)(grp / H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g2 = lane >> 5;
  const int slot = seg_state ? seg_state[s] : s;
  const int ncol0 = cb * DVB + 32 * w;
  const int64_t sbase = ((int64_t)slot * H + h) * DK * dv + ncol0;
  const int64_t rbeg = seg_off[s], rend = seg_off[s + 1];
  const int nchunk = (int)((rend - rbeg + GC - 1) / GC);
  const int cbase = chunks_before(seg_off, s, lane);

  // Inputs of the chunk at row r0n into buffer b (as in the forward walk; rows
  // past the segment end repeat its last row, and T and P are zero there).
  // The tokens of the rows of the chunk walked after it (r0n - 64) travel in
  // the TOK area of its buffer.
  using CK = TileCopy<DK, NW>;
  using CT = TileCopy<GC, NW>;
  constexpr int NPF = 2 * CK::PER_WAVE + 2 * CT::PER_WAVE + 2;
  int64_t pf_r0 = 0, pf_chk = 0;
  int pf_L = 0;
  f16_t* pf_B = smem;
  int qtok[CK::PER_WAVE];
  auto pf_setup = [&](int64_t r0n, int b, const int32_t* tok_lds) {
    pf_r0 = r0n;
    pf_L = (int)min((int64_t)GC, rend - r0n);
    pf_chk = (int64_t)(cbase + (r0n - rbeg) / GC) * H + h;
    pf_B = smem + b * LY::BUF;
#pragma unroll
    for (int j = 0; j < CK::PER_WAVE; ++j) {
      const int r = min(CK::row(w, lane, j), pf_L - 1);
      if (tok_lds) qtok[j] = tok_lds[r];
      else qtok[j] = row_token ? row_token[r0n + r] : (int)(r0n + r);
    }
  };
  auto pf_issue = [&](int i) {
    if (i < CK::PER_WAVE) {
      CK::issue(pf_B + LY::OFF_K, w, lane, i, [&](int r, int c) {
        return k + ((pf_r0 + min(r, pf_L - 1)) * H + h) * DK + 8 * c;
      });
    } else if ((i -= CK::PER_WAVE) < CK::PER_WAVE) {
      const int64_t t = qtok[i];
      CK::issue(pf_B + LY::OFF_Q, w, lane, i, [&](int r, int c) { return q + (t * H + h) * DK + 8 * c; });
    } else if ((i -= CK::PER_WAVE) < CT::PER_WAVE) {
      CT::issue(pf_B + LY::OFF_T, w, lane, i, [&](int r, int c) { return Tws + (pf_chk * GC + r) * GC + 8 * c; });
    } else if ((i -= CT::PER_WAVE) < CT::PER_WAVE) {
      CT::issue(pf_B + LY::OFF_P, w, lane, i, [&](int r, int c) { return Pws + (pf_chk * GC + r) * GC + 8 * c; });
    } else if (i == CT::PER_WAVE) {
      if (w < 2) dma_b32(Ews + pf_chk * 2 * GC + GC * w + lane, pf_B + LY::OFF_E + 2 * GC * w);
    } else if (w == NW - 1) {  // tokens of the rows of the chunk walked next
      const int64_t rn = (pf_r0 - GC >= rbeg ? pf_r0 - GC : pf_r0) + lane;
      const int64_t rc = min(rn, rend - 1);
      if (row_token) dma_b32(row_token + rc, pf_B + LY::OFF_TOK);
      else reinterpret_cast<int32_t*>(pf_B + LY::OFF_TOK)[lane] = (int32_t)rc;
    }
  };
  constexpr int PZ = NPF / NKD, PA = (NPF - PZ * NKD + GC / 16 - 1) / (GC / 16);

  // dO of a chunk: lane holds rows 16 kb + 8 g + t (t < 8) of its column, the
  // 16-deep operand layout (k = chunk rows), zero past the segment end.
  float don[4 * 8];
  auto load_do = [&](int64_t r0n) {
    const int Ln = (int)min((int64_t)GC, rend - r0n);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = 16 * kb + 8 * g2 + t;
        don[8 * kb + t] = r < Ln ? d_o[((r0n + r) * H + h) * dv + ncol0 + c32] : 0.f;
      }
  };

  f16x16 dS[ND];
  if (dstate_out) {
#pragma unroll
    for (int a = 0; a < ND; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * a + 8 * (i / 4) + 4 * g2 + (i % 4);
        dS[a][i] = dstate_out[sbase + (int64_t)d * dv + c32];
      }
  } else {
#pragma unroll
    for (int a = 0; a < ND; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) dS[a][i] = 0.f;
  }
  const float ones[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  if (nchunk > 0) {
    const int64_t rl = rbeg + (int64_t)(nchunk - 1) * GC;
    pf_setup(rl, 0, nullptr);
#pragma unroll
    for (int i = 0; i < NPF; ++i) pf_issue(i);
    load_do(rl);
  }

  int buf = 0;
  for (int ci = nchunk - 1; ci >= 0; --ci, buf ^= 1) {
    const int64_t r0 = rbeg + (int64_t)ci * GC;
    vm_wait_all();
    lds_barrier();  // every wave's part has landed; every wave is done with the other buffer
    const f16_t* Bc = smem + buf * LY::BUF;
    const f16_t* Ks = Bc + LY::OFF_K;
    const f16_t* Qs = Bc + LY::OFF_Q;
    const f16_t* Ts = Bc + LY::OFF_T;
    const f16_t* Ps = Bc + LY::OFF_P;
    const float* Eg = reinterpret_cast<const float*>(Bc + LY::OFF_E);  // gm_i, then ek_i
    // this chunk's dO as operands: plain and scaled by gm (row)
    h8v dof[4], gdof[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      unsigned pw[4], pg[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * kb + 8 * g2 + 2 * t;
        pw[t] = pack_h2(don[8 * kb + 2 * t], don[8 * kb + 2 * t + 1]);
        pg[t] = pack_h2(don[8 * kb + 2 * t] * Eg[r], don[8 * kb + 2 * t + 1] * Eg[r + 1]);
      }
      dof[kb] = __builtin_bit_cast(h8v, *reinterpret_cast<const __attribute__((ext_vector_type(4))) unsigned*>(pw));
      gdof[kb] = __builtin_bit_cast(h8v, *reinterpret_cast<const __attribute__((ext_vector_type(4))) unsigned*>(pg));
    }
    const int64_t rnext = ci > 0 ? r0 - GC : r0;
    pf_setup(rnext, buf ^ 1, reinterpret_cast<const int32_t*>(Bc + LY::OFF_TOK));
    if (ci > 0) load_do(rnext);
    // dS' of this chunk, transposed, through the wave's tile
    store_state_t<DK>(dhws + ((int64_t)(cbase + ci) * H + h) * dv * DK + (int64_t)ncol0 * DK, dS,
                      reinterpret_cast<f16_t*>(reinterpret_cast<char*>(smem) + LY::OST) + 2048 * w, lane);

    // ---- Z = K dS (two 32-row tiles)
    f16x16 Z[2], dU[2];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Z[bt][i] = 0.f;
        dU[bt][i] = 0.f;
      }
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
#pragma unroll
      for (int i = PZ * kb; i < PZ * (kb + 1); ++i) pf_issue(i);
      const h8v sb = acc_to_b(dS[kb / 2], kb % 2, ones);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) Z[bt] = mfma32(row_frag<DK>(Ks, 32 * bt + c32, kb, g2), sb, Z[bt]);
    }
    CHAIN_PHASE();
    // ---- dU = P^T dO + diag(ek) Z
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb) {
#pragma unroll
      for (int i = PZ * NKD + PA * kb; i < PZ * NKD + PA * (kb + 1); ++i)
        if (i < NPF) pf_issue(i);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) dU[bt] = mfma32(col_frag<GC>(Ps, kb, 32 * bt, lane), dof[kb], dU[bt]);
    }
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dU[bt][i] += Eg[GC + 32 * bt + 8 * (i / 4) + 4 * g2 + (i % 4)] * Z[bt][i];
    CHAIN_PHASE();
    // ---- dR = T^T dU, as the operand -diag(gm) dR (k = chunk rows)
    h8v rb[GC / 16];
    if constexpr (DELTA) {
      f16x16 dR[2];
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dR[bt][i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb) {
        const h8v ub = acc_to_b(dU[kb / 2], kb % 2, ones);
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) dR[bt] = mfma32(col_frag<GC>(Ts, kb, 32 * bt, lane), ub, dR[bt]);
      }
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float sc[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            sc[t] = -Eg[32 * bt + 16 * p + 4 * g2 + t];
            sc[4 + t] = -Eg[32 * bt + 16 * p + 8 + 4 * g2 + t];
          }
          rb[2 * bt + p] = acc_to_b(dR[bt], p, sc);
        }
    }
    CHAIN_PHASE();
    // ---- dS <- gm_L dS + Q^T diag(gm) dO - K^T diag(gm) dR
    const float eL = Eg[GC - 1];
#pragma unroll
    for (int a = 0; a < ND; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) dS[a][i] *= eL;
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb)
#pragma unroll
      for (int a = 0; a < ND; ++a) {
        dS[a] = mfma32(col_frag<DK>(Qs, kb, 32 * a, lane), gdof[kb], dS[a]);
        if (DELTA) dS[a] = mfma32(col_frag<DK>(Ks, kb, 32 * a, lane), rb[kb], dS[a]);
      }
  }
  vm_wait_all();  // the last (repeated) prefetch has landed before the block ends
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * a + 8 * (i / 4) + 4 * g2 + (i % 4);
      dstate_in[sbase + (int64_t)d * dv + c32] = dS[a][i];
    }
}

// ------------------------------------------------------------------ per-chunk gradients
// One block of 8 waves per (chunk, head).  The value columns are taken 64 at a
// time (a slice); per slice, with S^T and dS'^T of the slice (from the walks),
// V and dO of the slice, and K, T, P of the chunk in LDS (products of two
// transposed factors give the transposed tiles, so that a lane holds one chunk
// row and 4 consecutive columns and writes 8-byte row pieces):
//   stage 1  waves 0-3: Y^T = S^T K^T (tile t = w), R = V - diag(gm) Y to LDS
//            waves 4-7: Z^T = dS'^T K^T, dU = P^T dO + diag(ek) Z to LDS
//   stage 2  waves 0-3: dR^T = dU^T T; dV = dR out; -diag(gm) dR to LDS;
//                       row sums of dR o Y (= k_i.PR_i) kept per lane
//            waves 4-7: U^T = R^T T^T; U and diag(ek) U to LDS; row sums of U o Z
//   stage 3  every wave: its tile of PQ += dO S^T and of
//            PK' += diag(ek) U dS'^T - diag(gm) dR S^T  (64 x DK), and of
//            dT += dU R^T (waves 0-3) or dP += dO U^T (waves 4-7)  (64 x 64)
// The next slice's inputs are loaded into registers during the current one.
// Then, all products on the matrix cores and every row / column sum taken in
// registers by the wave that holds the tile:
//   waves 0-3  dc's share sum_r dT_ri X_ri; (dT diag(c)) to LDS; then
//              X^T (dT diag(c)); then dA = -(that) X^T and K K^T, giving G, B
//   waves 4-7  D = dP o e^{g_i - g_j}, then Q K^T and the sums of D o QK
// and finally dQ, dK (matrix cores), dg and da (reverse prefix sum).
typedef _Float16 h4v __attribute__((ext_vector_type(4)));

template <int DK>
struct GradLds {
  // bytes; the slice phase and the final phase share the region after K
  static constexpr int KT = GC * DK * 2, HT = GC * GC * 2;
  static constexpr int OFF_K = 0, OFF_T = KT, OFF_P = OFF_T + HT, OFF_ST = OFF_P + HT, OFF_DST = OFF_ST + KT,
                       OFF_V = OFF_DST + KT, OFF_DO = OFF_V + HT, OFF_R = OFF_DO + HT, OFF_DU = OFF_R + HT,
                       OFF_U = OFF_DU + HT, OFF_EU = OFF_U + HT, OFF_GR = OFF_EU + HT, END1 = OFF_GR + HT;
  static constexpr int OFF_Q = KT, OFF_X = OFF_Q + KT, OFF_DTC = OFF_X + HT, OFF_XTD = OFF_DTC + HT,
                       OFF_DM = OFF_XTD + HT, OFF_BS = OFF_DM + HT, END2 = OFF_BS + HT;
  static constexpr size_t BYTES = END1 > END2 ? END1 : END2;
};

template <int RH>
__device__ __forceinline__ f16_t* tile_piece(f16_t* X, int r, int c) {
  return X + r * RH + 8 * swz<RH>(r, c);
}
template <int RH>
__device__ __forceinline__ int tile_elem(int r, int col) {
  return r * RH + 8 * swz<RH>(r, col >> 3) + (col & 7);
}
// Cross-lane sums: DPP within rows of 16 lanes (quad swaps, then the 8- and
// 16-lane mirrors), then one lane exchange between the rows.  (The swap
// instructions that exchange rows are not used here: the compiler takes both
// of their results to be equal when they are added.)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// sum over the 32 lanes of this lane's half wave, in every lane
__device__ __forceinline__ float half_wave_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x + __shfl_xor(x, 16, 64);
}
// x(lane) + x(lane ^ 32)
__device__ __forceinline__ float halves_sum(float x) { return x + __shfl_xor(x, 32, 64); }

template <int DK, bool DELTA>
__global__ __launch_bounds__(512) void k_gdn_grad(
    int H, int dv, int n_seg, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ row_token,
    const f16_t* __restrict__ q, const f16_t* __restrict__ k, const f16_t* __restrict__ v,
    const float* __restrict__ alpha_p, const float* __restrict__ beta_p, const f16_t* __restrict__ Tws,
    const f16_t* __restrict__ Pws, const f16_t* __restrict__ Xws, const f16_t* __restrict__ hws,
    const f16_t* __restrict__ dhws, const float* __restrict__ d_o, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dvo, float* __restrict__ da, float* __restrict__ dc) {
  using LY = GradLds<DK>;
  constexpr int NKD = DK / 16, NDT = DK / 32;  // k-steps over DK, 32-column tiles of DK
  constexpr int NS = DK / 64;                  // 16-byte pieces of S^T (or Q) per thread and slice
  extern __shared__ __attribute__((aligned(16))) char gsm[];
  __shared__ float g_s[GC], gm_s[GC], ek_s[GC], c_s[GC], a_s[GC];
  // per-row (or per-column) partial sums, [32-wide tile][row or column]
  __shared__ float rdy_s[2][GC], ruz_s[2][GC], rpq_s[NDT][GC], red_s[8];
  __shared__ float dct_s[2][GC], rsg_s[2][GC], csg_s[2][GC], rse_s[2][GC], cse_s[2][GC];
  f16_t* Kt = reinterpret_cast<f16_t*>(gsm + LY::OFF_K);
  f16_t* Tt = reinterpret_cast<f16_t*>(gsm + LY::OFF_T);
  f16_t* Pt = reinterpret_cast<f16_t*>(gsm + LY::OFF_P);
  f16_t* StT = reinterpret_cast<f16_t*>(gsm + LY::OFF_ST);
  f16_t* dStT = reinterpret_cast<f16_t*>(gsm + LY::OFF_DST);
  f16_t* Vt = reinterpret_cast<f16_t*>(gsm + LY::OFF_V);
  f16_t* dOt = reinterpret_cast<f16_t*>(gsm + LY::OFF_DO);
  f16_t* Rt = DELTA ? reinterpret_cast<f16_t*>(gsm + LY::OFF_R) : Vt;
  f16_t* dUt = reinterpret_cast<f16_t*>(gsm + LY::OFF_DU);
  f16_t* Ut = reinterpret_cast<f16_t*>(gsm + LY::OFF_U);
  f16_t* eUt = reinterpret_cast<f16_t*>(gsm + LY::OFF_EU);
  f16_t* gRt = reinterpret_cast<f16_t*>(gsm + LY::OFF_GR);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g2 = lane >> 5;
  const int64_t ch = blockIdx.x;  // chunk * H + head
  const int c = (int)(ch / H), h = (int)(ch % H);
  int seg, cb0;
  if (!locate_chunk(seg_off, n_seg, c, lane, seg, cb0)) return;  // the same in every wave
  const int64_t r0 = seg_off[seg] + (int64_t)(c - cb0) * GC;
  const int L = (int)min((int64_t)GC, (int64_t)seg_off[seg + 1] - r0);

  // Q (gathered by token; zero past L) and X of the chunk, needed only at the
  // end, are loaded first and kept in registers.
  h8v rq[NS], rx;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int p = tid + 512 * j, r = p / (DK / 8), cc = p % (DK / 8);
    const h8v z = {};
    rq[j] = z;
    if (r < L) {
      const int64_t tk = row_token ? (int64_t)row_token[r0 + r] : r0 + r;
      rq[j] = *reinterpret_cast<const h8v*>(q + (tk * H + h) * DK + 8 * cc);
    }
  }
  const int vr = tid >> 3, vc = tid & 7;  // a 64 x 64 half tile: row, 8-column piece of this thread
  if constexpr (DELTA) rx = *reinterpret_cast<const h8v*>(Xws + (ch * GC + vr) * GC + 8 * vc);
  // gates (as the prep kernel computes them): g prefix of log a (0 past L)
  if (w == 0) {
    float g = 0.f, aa = 1.f, bb = 0.f;
    if (lane < L) {
      aa = alpha_p[(r0 + lane) * H + h];
      bb = beta_p[(r0 + lane) * H + h];
      g = log_gate(aa);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float u = __shfl_up(g, off, 64);
      if (lane >= off) g += u;
    }
    const float gL = __shfl(g, GC - 1, 64);
    g_s[lane] = g;
    gm_s[lane] = expf(g);
    ek_s[lane] = expf(gL - g);
    c_s[lane] = bb;
    a_s[lane] = aa;
  }
  // K (rows; zero past L), T, P of the chunk
  for (int p = tid; p < GC * DK / 8; p += 512) {
    const int r = p / (DK / 8), cc = p % (DK / 8);
    h8v val = {};
    if (r < L) val = *reinterpret_cast<const h8v*>(k + ((r0 + r) * H + h) * DK + 8 * cc);
    *reinterpret_cast<h8v*>(tile_piece<DK>(Kt, r, cc)) = val;
  }
  *reinterpret_cast<h8v*>(tile_piece<GC>(Tt, vr, vc)) = *reinterpret_cast<const h8v*>(Tws + (ch * GC + vr) * GC + 8 * vc);
  *reinterpret_cast<h8v*>(tile_piece<GC>(Pt, vr, vc)) = *reinterpret_cast<const h8v*>(Pws + (ch * GC + vr) * GC + 8 * vc);

  // slice inputs in registers: S^T and dS'^T pieces (rows = value columns),
  // one V piece, one dO piece (8 floats)
  const f16_t* hc = hws + ch * (int64_t)dv * DK;
  const f16_t* dhc = dhws + ch * (int64_t)dv * DK;
  h8v rs[NS], rds[NS], rv;
  float4 ro0, ro1;
  auto load_slice = [&](int cs) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int p = tid + 512 * j, r = p / (DK / 8), cc = p % (DK / 8);
      rs[j] = *reinterpret_cast<const h8v*>(hc + (int64_t)(64 * cs + r) * DK + 8 * cc);
      rds[j] = *reinterpret_cast<const h8v*>(dhc + (int64_t)(64 * cs + r) * DK + 8 * cc);
    }
    const h8v z = {};
    rv = z;
    ro0 = make_float4(0.f, 0.f, 0.f, 0.f);
    ro1 = ro0;
    if (vr < L) {
      rv = *reinterpret_cast<const h8v*>(v + ((r0 + vr) * H + h) * dv + 64 * cs + 8 * vc);
      const float* op = d_o + ((r0 + vr) * H + h) * dv + 64 * cs + 8 * vc;
      ro0 = *reinterpret_cast<const float4*>(op);
      ro1 = *reinterpret_cast<const float4*>(op + 4);
    }
  };
  float sds = 0.f;  // <S, dS'> over this thread's pieces
  auto store_slice = [&]() {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int p = tid + 512 * j, r = p / (DK / 8), cc = p % (DK / 8);
      *reinterpret_cast<h8v*>(tile_piece<DK>(StT, r, cc)) = rs[j];
      *reinterpret_cast<h8v*>(tile_piece<DK>(dStT, r, cc)) = rds[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) sds = fmaf((float)rs[j][e], (float)rds[j][e], sds);
    }
    *reinterpret_cast<h8v*>(tile_piece<GC>(Vt, vr, vc)) = rv;
    const unsigned pw[4] = {pack_h2(ro0.x, ro0.y), pack_h2(ro0.z, ro0.w), pack_h2(ro1.x, ro1.y),
                            pack_h2(ro1.z, ro1.w)};
    *reinterpret_cast<h8v*>(tile_piece<GC>(dOt, vr, vc)) =
        __builtin_bit_cast(h8v, *reinterpret_cast<const __attribute__((ext_vector_type(4))) unsigned*>(pw));
  };

  // accumulators: this wave's tiles of PQ and PK' (64 x DK) and of dT or dP
  // (64 x 64).  With DK = 64 the 64 x DK matrices have 4 tiles: waves 0-3
  // hold PQ, waves 4-7 PK'.
  const int t4 = w & 3, bt = t4 >> 1, ct = t4 & 1;  // 64 x 64 tile of waves w and w + 4
  const int bq = NDT == 4 ? (w >> 2) : (t4 >> 1), dq_t = NDT == 4 ? (w & 3) : (t4 & 1);  // 64 x DK tile
  const bool has_pq = NDT == 4 || w < 4, has_pk = NDT == 4 || w >= 4;
  f16x16 PQ, PK, DTP;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    PQ[i] = 0.f;
    PK[i] = 0.f;
    DTP[i] = 0.f;
  }
  float prow = 0.f;  // row 32 bt + lane % 32: partial sum of dR o Y (waves 0-3) or U o Z (waves 4-7)
  auto rowof = [&](int tb, int i) { return 32 * tb + 8 * (i / 4) + 4 * g2 + (i % 4); };

  const int nsl = dv / 64;
  load_slice(0);
  for (int cs = 0; cs < nsl; ++cs) {
    __syncthreads();  // the previous slice is done with the buffers (and K, T, P, gates are in)
    store_slice();
    if (cs + 1 < nsl) load_slice(cs + 1);
    __syncthreads();
    // Lane-derived offsets are recomputed in every slice rather than kept
    // live across the loop (there are too many of them).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int l32 = ln & 31, lg = ln >> 5;
    const int i = 32 * bt + l32;  // this lane's chunk row in the transposed tiles below
    // ---- stage 1 (transposed tiles: lane holds row i, columns 32 ct + 8 qq + 4 g + 0..3)
    f16x16 A, Bv;  // Y^T or Z^T; then dR^T or U^T
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      A[e] = 0.f;
      Bv[e] = 0.f;
    }
    if (w < 4) {
      if constexpr (DELTA) {
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb)
          A = mfma32(row_frag<DK>(StT, 32 * ct + l32, kb, lg), row_frag<DK>(Kt, i, kb, lg), A);
        const float gi = gm_s[i];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int e = tile_elem<GC>(i, 32 * ct + 8 * qq + 4 * lg);
          const h4v vv = *reinterpret_cast<const h4v*>(Vt + e);
          const u2v rr = {pack_h2((float)vv[0] - gi * A[4 * qq], (float)vv[1] - gi * A[4 * qq + 1]),
                          pack_h2((float)vv[2] - gi * A[4 * qq + 2], (float)vv[3] - gi * A[4 * qq + 3])};
          *reinterpret_cast<u2v*>(Rt + e) = rr;
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
        A = mfma32(row_frag<DK>(dStT, 32 * ct + l32, kb, lg), row_frag<DK>(Kt, i, kb, lg), A);
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
        Bv = mfma32(col_frag<GC>(dOt, kb, 32 * ct, ln), col_frag<GC>(Pt, kb, 32 * bt, ln), Bv);
      const float eki = ek_s[i];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const u2v uu = {pack_h2(Bv[4 * qq] + eki * A[4 * qq], Bv[4 * qq + 1] + eki * A[4 * qq + 1]),
                        pack_h2(Bv[4 * qq + 2] + eki * A[4 * qq + 2], Bv[4 * qq + 3] + eki * A[4 * qq + 3])};
        *reinterpret_cast<u2v*>(dUt + tile_elem<GC>(i, 32 * ct + 8 * qq + 4 * lg)) = uu;
      }
    }
    __syncthreads();
    // ---- stage 2
#pragma unroll
    for (int e = 0; e < 16; ++e) Bv[e] = 0.f;
    if (w < 4) {
      // dR^T = dU^T T
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
        Bv = mfma32(col_frag<GC>(dUt, kb, 32 * ct, ln), col_frag<GC>(Tt, kb, 32 * bt, ln), Bv);
      if (i < L) {
        float* dp = dvo + ((r0 + i) * H + h) * dv + 64 * cs + 32 * ct + 4 * lg;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *reinterpret_cast<float4*>(dp + 8 * qq) =
              make_float4(Bv[4 * qq], Bv[4 * qq + 1], Bv[4 * qq + 2], Bv[4 * qq + 3]);
      }
      if constexpr (DELTA) {
        const float gi = gm_s[i];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
          for (int t = 0; t < 4; ++t) prow = fmaf(Bv[4 * qq + t], A[4 * qq + t], prow);
          const u2v rr = {pack_h2(-gi * Bv[4 * qq], -gi * Bv[4 * qq + 1]),
                          pack_h2(-gi * Bv[4 * qq + 2], -gi * Bv[4 * qq + 3])};
          *reinterpret_cast<u2v*>(gRt + tile_elem<GC>(i, 32 * ct + 8 * qq + 4 * lg)) = rr;
        }
      }
    } else {
      // U^T = R^T T^T
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
        Bv = mfma32(col_frag<GC>(Rt, kb, 32 * ct, ln), row_frag<GC>(Tt, i, kb, lg), Bv);
      const float eki = ek_s[i];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
        for (int t = 0; t < 4; ++t) prow = fmaf(Bv[4 * qq + t], A[4 * qq + t], prow);
        const int e = tile_elem<GC>(i, 32 * ct + 8 * qq + 4 * lg);
        const u2v uu = {pack_h2(Bv[4 * qq], Bv[4 * qq + 1]), pack_h2(Bv[4 * qq + 2], Bv[4 * qq + 3])};
        const u2v eu = {pack_h2(eki * Bv[4 * qq], eki * Bv[4 * qq + 1]),
                        pack_h2(eki * Bv[4 * qq + 2], eki * Bv[4 * qq + 3])};
        *reinterpret_cast<u2v*>(Ut + e) = uu;
        *reinterpret_cast<u2v*>(eUt + e) = eu;
      }
    }
    __syncthreads();
    // ---- stage 3
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb) {
      if (has_pq) PQ = mfma32(row_frag<GC>(dOt, 32 * bq + l32, kb, lg), col_frag<DK>(StT, kb, 32 * dq_t, ln), PQ);
      if (has_pk) {
        PK = mfma32(row_frag<GC>(eUt, 32 * bq + l32, kb, lg), col_frag<DK>(dStT, kb, 32 * dq_t, ln), PK);
        if (DELTA) PK = mfma32(row_frag<GC>(gRt, 32 * bq + l32, kb, lg), col_frag<DK>(StT, kb, 32 * dq_t, ln), PK);
      }
      if (w < 4) DTP = mfma32(row_frag<GC>(dUt, i, kb, lg), row_frag<GC>(Rt, 32 * ct + l32, kb, lg), DTP);
      else DTP = mfma32(row_frag<GC>(dOt, i, kb, lg), row_frag<GC>(Ut, 32 * ct + l32, kb, lg), DTP);
    }
  }
  __syncthreads();  // the slice buffers are free: the final phase reuses them

  // ---- final phase
  f16_t* Qt = reinterpret_cast<f16_t*>(gsm + LY::OFF_Q);
  f16_t* Xt = reinterpret_cast<f16_t*>(gsm + LY::OFF_X);
  f16_t* dTc = reinterpret_cast<f16_t*>(gsm + LY::OFF_DTC);  // dT diag(c)
  f16_t* XtD = reinterpret_cast<f16_t*>(gsm + LY::OFF_XTD);  // X^T dT diag(c)
  f16_t* Dm = reinterpret_cast<f16_t*>(gsm + LY::OFF_DM);
  f16_t* Bs = reinterpret_cast<f16_t*>(gsm + LY::OFF_BS);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int p = tid + 512 * j, r = p / (DK / 8), cc = p % (DK / 8);
    *reinterpret_cast<h8v*>(tile_piece<DK>(Qt, r, cc)) = rq[j];
  }
  if constexpr (DELTA) *reinterpret_cast<h8v*>(tile_piece<GC>(Xt, vr, vc)) = rx;
  {  // row sums of dR o Y / U o Z over this wave's 32 columns (two lane halves)
    const float x = halves_sum(prow);
    if (g2 == 0) (w < 4 ? rdy_s : ruz_s)[ct][32 * bt + c32] = x;
  }
  {
    const float x = halves_sum(half_wave_sum(sds));
    if (lane == 0) red_s[w] = x;
  }
  __syncthreads();
  // entries (r, j) of this wave's 64 x 64 tile: r = rowof(bt, e), j = 32 ct + c32
  const int j = 32 * ct + c32;
  float Dv[16];  // waves 4-7: D = dP o e^{g_r - g_j} (j <= r)
  if (w < 4) {
    // dc's share from T: sum_r dT_rj X_rj (X = I for gated linear attention);
    // dT diag(c) to LDS
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rowof(bt, e);
      const float t = j <= r ? DTP[e] : 0.f;
      if constexpr (DELTA) {
        x = fmaf(t, (float)Xt[tile_elem<GC>(r, j)], x);
        dTc[tile_elem<GC>(r, j)] = (f16_t)(t * c_s[j]);
      } else {
        x += r == j ? t : 0.f;
      }
    }
    x = halves_sum(x);
    if (g2 == 0) dct_s[bt][j] = x;
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rowof(bt, e);
      Dv[e] = j <= r ? DTP[e] * __expf(g_s[r] - g_s[j]) : 0.f;
      Dm[tile_elem<GC>(r, j)] = (f16_t)Dv[e];
    }
  }
  // q_i.PQ_i: this wave's PQ tile against Q
  if (has_pq) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rowof(bq, e);
      const float x = half_wave_sum(PQ[e] * (float)Qt[tile_elem<DK>(r, 32 * dq_t + c32)]);
      if (c32 == 0) rpq_s[dq_t][r] = x;
    }
  }
  __syncthreads();
  f16x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  if (w < 4) {
    if constexpr (DELTA) {
      // X^T (dT diag(c)), tile (bt, ct)
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
        acc = mfma32(col_frag<GC>(Xt, kb, 32 * bt, lane), col_frag<GC>(dTc, kb, 32 * ct, lane), acc);
#pragma unroll
      for (int e = 0; e < 16; ++e) XtD[tile_elem<GC>(rowof(bt, e), j)] = (f16_t)acc[e];
    }
  } else {
    // Q K^T, tile (bt, ct); E = D o QK, its row and column sums
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb)
      acc = mfma32(row_frag<DK>(Qt, 32 * bt + c32, kb, g2), row_frag<DK>(Kt, 32 * ct + c32, kb, g2), acc);
    float cs_ = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float em = Dv[e] * acc[e];
      cs_ += em;
      const float rsum = half_wave_sum(em);
      if (c32 == 0) rse_s[ct][rowof(bt, e)] = rsum;
    }
    cs_ = halves_sum(cs_);
    if (g2 == 0) cse_s[bt][j] = cs_;
  }
  __syncthreads();
  if (DELTA && w < 4) {
    // dA = -(X^T dT diag(c)) X^T (j < r), K K^T; G = dA o e^{g_r - g_j} o KK,
    // B = dA o c_r e^{g_r - g_j} (both halves of B + B^T)
    f16x16 dA, kk;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dA[e] = 0.f;
      kk[e] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb)
      dA = mfma32(row_frag<GC>(XtD, 32 * bt + c32, kb, g2), row_frag<GC>(Xt, j, kb, g2), dA);
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb)
      kk = mfma32(row_frag<DK>(Kt, 32 * bt + c32, kb, g2), row_frag<DK>(Kt, j, kb, g2), kk);
    float csg = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rowof(bt, e);
      const float eg = j < r ? __expf(g_s[r] - g_s[j]) : 0.f;  // e^{g_r - g_j} may overflow above the diagonal
      const float a_ = -dA[e] * eg;
      const float gg = a_ * kk[e];
      csg = fmaf(c_s[r], gg, csg);
      const float rsum = half_wave_sum(gg);
      if (c32 == 0) rsg_s[ct][r] = rsum;
      if (j <= r) {
        const f16_t bm = (f16_t)(a_ * c_s[r]);
        Bs[tile_elem<GC>(r, j)] = bm;
        Bs[tile_elem<GC>(j, r)] = bm;
      }
    }
    csg = halves_sum(csg);
    if (g2 == 0) csg_s[bt][j] = csg;
  }
  __syncthreads();
  // dg per row, then d log a by a reverse prefix sum, da and dc out
  if (w == 0) {
    const int i = lane;
    float dcr = dct_s[0][i] + dct_s[1][i];
    float dg = rse_s[0][i] + rse_s[1][i] - cse_s[0][i] - cse_s[1][i];
    if constexpr (DELTA) {
      const float rg = rsg_s[0][i] + rsg_s[1][i];
      dcr += rg;
      dg += c_s[i] * rg - csg_s[0][i] - csg_s[1][i];
      dg -= gm_s[i] * (rdy_s[0][i] + rdy_s[1][i]);
    }
    float pq = 0.f;
#pragma unroll
    for (int t = 0; t < NDT; ++t) pq += rpq_s[t][i];
    dg += gm_s[i] * pq;
    const float e = i < L ? ek_s[i] * (ruz_s[0][i] + ruz_s[1][i]) : 0.f;
    dg -= e;
    float esum = e;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) esum += __shfl_xor(esum, o, 64);
    float sdsum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) sdsum += red_s[t];
    if (i == L - 1) dg += esum + gm_s[i] * sdsum;
    if (i >= L) dg = 0.f;
    // d log a_i = sum_{i' >= i} dg_i'
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float u = __shfl_down(dg, off, 64);
      if (i + off < 64) dg += u;
    }
    if (i < L) {
      da[(r0 + i) * H + h] = dg / a_s[i];
      dc[(r0 + i) * H + h] = dcr;
    }
  }
  // dQ = diag(gm) PQ + D K and dK = PK' + (B + B^T) K + D^T Q, this wave's tiles
  if (has_pq) {
#pragma unroll
    for (int e = 0; e < 16; ++e) PQ[e] *= gm_s[rowof(bq, e)];
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb)
      PQ = mfma32(row_frag<GC>(Dm, 32 * bq + c32, kb, g2), col_frag<DK>(Kt, kb, 32 * dq_t, lane), PQ);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rowof(bq, e);
      if (r < L) dq[((r0 + r) * H + h) * DK + 32 * dq_t + c32] = PQ[e];
    }
  }
  if (has_pk) {
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb) {
      if (DELTA) PK = mfma32(row_frag<GC>(Bs, 32 * bq + c32, kb, g2), col_frag<DK>(Kt, kb, 32 * dq_t, lane), PK);
      PK = mfma32(col_frag<GC>(Dm, kb, 32 * bq, lane), col_frag<DK>(Qt, kb, 32 * dq_t, lane), PK);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rowof(bq, e);
      if (r < L) dk[((r0 + r) * H + h) * DK + 32 * dq_t + c32] = PK[e];
    }
  }
}

// ------------------------------------------------------------------ workspace + launch
// After the forward workspace (T, P, decays): X (half 64 x 64), and the
// transposed states S^T and dS'^T entering / leaving every chunk (half dv x dk),
// all per (chunk, head).
struct ChunkBwdWs {
  ChunkWs fw;
  f16_t* X;
  f16_t* h;
  f16_t* dh;
  size_t bytes;
};

inline ChunkBwdWs chunk_bwd_ws_layout(void* base, int64_t n_seg, int64_t n_rows, int H, int dk, int dv) {
  ChunkBwdWs w;
  w.fw = chunk_ws_layout(base, n_seg, n_rows, H, dk);
  const int64_t nch = n_rows / GC + n_seg;
  size_t off = w.fw.bytes;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += (b + 255) / 256 * 256;
    return o;
  };
  const size_t o_x = take((size_t)nch * H * GC * GC * 2);
  const size_t o_h = take((size_t)nch * H * dk * dv * 2);
  const size_t o_dh = take((size_t)nch * H * dk * dv * 2);
  char* b = (char*)base;
  w.X = (f16_t*)(b + o_x);
  w.h = (f16_t*)(b + o_h);
  w.dh = (f16_t*)(b + o_dh);
  w.bytes = off;
  return w;
}

template <int DK, int NW, bool DELTA>
static mom_status launch_chain_bwd(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                                   const ChunkBwdWs& W, const int32_t* row_token, const void* q, const void* k,
                                   const float* d_o, const float* dstate_out, float* dstate_in, hipStream_t st) {
  using LY = ChainBwdLds<DK, NW>;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void*)k_gdn_chain_bwd<DK, NW, DELTA>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::BYTES) != hipSuccess)
      return MOM_ERR_LAUNCH;
    attr = true;
  }
  const int64_t blocks = (int64_t)n_seg * d.H * (d.dv / LY::DVB);
  if (blocks > 0)
    hipLaunchKernelGGL((k_gdn_chain_bwd<DK, NW, DELTA>), dim3((unsigned)blocks), dim3(64 * NW), LY::BYTES, st, d.H,
                       d.dv, n_seg, seg_off, seg_state, (const f16_t*)k, W.fw.T, W.fw.P, W.fw.E, row_token,
                       (const f16_t*)q, d_o, dstate_out, dstate_in, W.dh);
  return MOM_OK;
}

template <int DK, bool DELTA>
static mom_status launch_bwd(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                             const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                             const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                             const float* d_o, const float* dstate_out, float* dq, float* dk, float* dv, float* da,
                             float* dc, float* dstate_in, void* ws, bool saved, hipStream_t st) {
  const ChunkBwdWs W = chunk_bwd_ws_layout(ws, n_seg, n_rows, d.H, d.dk, d.dv);
  mom_status r = MOM_OK;
  if (!saved) {  // otherwise the workspace holds the forward's factors and states
    r = launch_chunk_states(d, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p, state_in,
                            nullptr, nullptr, W.fw, W.X, W.h, DELTA, false, st);
    if (r != MOM_OK) return r;
  }
  r = d.dv % 128 == 0
          ? launch_chain_bwd<DK, 4, DELTA>(d, n_seg, seg_off, seg_state, W, row_token, q, k, d_o, dstate_out,
                                           dstate_in, st)
          : launch_chain_bwd<DK, 2, DELTA>(d, n_seg, seg_off, seg_state, W, row_token, q, k, d_o, dstate_out,
                                           dstate_in, st);
  if (r != MOM_OK) return r;
  using LY = GradLds<DK>;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void*)k_gdn_grad<DK, DELTA>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)LY::BYTES) != hipSuccess)
      return MOM_ERR_LAUNCH;
    attr = true;
  }
  const int64_t nch = (int64_t)n_rows / GC + n_seg;
  if (nch * d.H > 0)
    hipLaunchKernelGGL((k_gdn_grad<DK, DELTA>), dim3((unsigned)(nch * d.H)), dim3(512), LY::BYTES, st, d.H, d.dv,
                       n_seg, seg_off, row_token, (const f16_t*)q, (const f16_t*)k, (const f16_t*)v, alpha_p, beta_p,
                       W.fw.T, W.fw.P, W.X, W.h, W.dh, d_o, dq, dk, dv, da, dc);
  return launch_status();
}

// gdn_bwd_valu.hip: the float32 path
size_t gdn_bwd_valu_ws_bytes(int64_t n_seg, int64_t n_rows, int H, int dk, int dv);
mom_status launch_gdn_bwd_valu(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                               const int32_t* seg_state, const int32_t* row_token, const float* q, const float* k,
                               const float* v, const float* alpha_p, const float* beta_p, const float* state_in,
                               const float* d_o, const float* dstate_out, float* dq, float* dk, float* dv_out,
                               float* da, float* dc, float* dstate_in, void* ws, bool delta, hipStream_t st);
template <typename IT>
mom_status launch_gdn_chunk_valu(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                                 const int32_t* row_token, const void* q, const void* k, const void* v,
                                 const float* alpha_p, const float* beta_p, const float* state_in, float* state_out,
                                 float* o, bool delta, hipStream_t st);

static size_t chunk_bwd_ws_bytes(const mom_dims* dims, int32_t n_seg, int32_t n_rows) {
  if (check_dims(dims) != MOM_OK || n_seg < 0 || n_rows < 0) return 0;
  if (dims->dtype != MOM_DTYPE_BF16) return gdn_bwd_valu_ws_bytes(n_seg, n_rows, dims->H, dims->dk, dims->dv);
  return chunk_bwd_ws_layout(nullptr, n_seg, n_rows, dims->H, dims->dk, dims->dv).bytes;
}

static mom_status chunk_bwd(bool delta, bool saved, const mom_dims* dims, int32_t n_seg, int32_t n_rows,
                            int32_t n_tok, int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                            const int32_t* row_token, const void* q, const void* k, const void* v,
                            const float* alpha_p, const float* beta_p, const float* state_in, const float* d_o,
                            const float* dstate_out, float* dq, float* dk, float* dv, float* da, float* dc,
                            float* dstate_in, void* ws, size_t ws_bytes, void* stream) {
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  if (n_seg < 0 || n_rows < 0 || n_tok < 0 || n_state < 0) return MOM_ERR_DIMS;
  if (!seg_state && n_state < n_seg) return MOM_ERR_DIMS;
  MOM_CHECK_PTR(seg_off);
  MOM_CHECK_OPT_PTR(seg_state);
  MOM_CHECK_OPT_PTR(row_token);
  MOM_CHECK_OPT_PTR(state_in);
  MOM_CHECK_OPT_PTR(dstate_out);
  MOM_CHECK_PTR(dstate_in);
  if (n_rows > 0) {
    MOM_CHECK_PTR(q);
    MOM_CHECK_PTR(k);
    MOM_CHECK_PTR(v);
    MOM_CHECK_PTR(alpha_p);
    MOM_CHECK_PTR(beta_p);
    MOM_CHECK_PTR(d_o);
    MOM_CHECK_PTR(dq);
    MOM_CHECK_PTR(dk);
    MOM_CHECK_PTR(dv);
    MOM_CHECK_PTR(da);
    MOM_CHECK_PTR(dc);
  }
  const size_t need = chunk_bwd_ws_bytes(dims, n_seg, n_rows);
  if (!ws || ws_bytes < need) return MOM_ERR_WORKSPACE;
  MOM_CHECK_PTR(ws);
  if (n_seg == 0) return MOM_OK;
  hipStream_t st = (hipStream_t)stream;
  if (dims->dtype != MOM_DTYPE_BF16)  // float32: the row-by-row reverse sweep (nothing is kept between calls)
    return launch_gdn_bwd_valu(*dims, n_seg, n_rows, seg_off, seg_state, row_token, (const float*)q,
                               (const float*)k, (const float*)v, alpha_p, beta_p, state_in, d_o, dstate_out, dq, dk,
                               dv, da, dc, dstate_in, ws, delta, st);
#define MOM_BWD(DK, DELTA)                                                                                       \
  launch_bwd<DK, DELTA>(*dims, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p, state_in, \
                        d_o, dstate_out, dq, dk, dv, da, dc, dstate_in, ws, saved, st)
  if (dims->dk == 64) return delta ? MOM_BWD(64, true) : MOM_BWD(64, false);
  return delta ? MOM_BWD(128, true) : MOM_BWD(128, false);
#undef MOM_BWD
}

// The forward pass of a training step: as gdn_chunk_fwd, and the gradient
// workspace keeps T, P, the decays, X and the chunk-entry states.
static mom_status chunk_fwd_train(bool delta, const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                                  int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                                  const int32_t* row_token, const void* q, const void* k, const void* v,
                                  const float* alpha_p, const float* beta_p, const float* state_in, float* state_out,
                                  float* o, void* ws, size_t ws_bytes, void* stream) {
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  if (n_seg < 0 || n_rows < 0 || n_tok < 0 || n_state < 0) return MOM_ERR_DIMS;
  if (!seg_state && n_state < n_seg) return MOM_ERR_DIMS;
  MOM_CHECK_PTR(seg_off);
  MOM_CHECK_OPT_PTR(seg_state);
  MOM_CHECK_OPT_PTR(row_token);
  MOM_CHECK_OPT_PTR(state_in);
  MOM_CHECK_PTR(state_out);
  if (n_rows > 0) {
    MOM_CHECK_PTR(q);
    MOM_CHECK_PTR(k);
    MOM_CHECK_PTR(v);
    MOM_CHECK_PTR(alpha_p);
    MOM_CHECK_PTR(beta_p);
    MOM_CHECK_PTR(o);
  }
  if (!ws || ws_bytes < chunk_bwd_ws_bytes(dims, n_seg, n_rows)) return MOM_ERR_WORKSPACE;
  MOM_CHECK_PTR(ws);
  if (n_seg == 0) return MOM_OK;
  const mom_dims& d = *dims;
  if (d.dtype != MOM_DTYPE_BF16)  // float32: the forward pass; its backward recomputes what it needs
    return launch_gdn_chunk_valu<float>(d, n_seg, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p, state_in,
                                        state_out, o, delta, (hipStream_t)stream);
  const ChunkBwdWs W = chunk_bwd_ws_layout(ws, n_seg, n_rows, d.H, d.dk, d.dv);
  return launch_chunk_states(d, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p, state_in,
                             state_out, o, W.fw, W.X, W.h, delta, true, (hipStream_t)stream);
}

}  // namespace mom

extern "C" size_t gdn_chunk_bwd_workspace_bytes(const mom_dims* dims, int32_t n_seg, int32_t n_rows) {
  return mom::chunk_bwd_ws_bytes(dims, n_seg, n_rows);
}

extern "C" mom_status gdn_chunk_bwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                                    int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                                    const int32_t* row_token, const void* q, const void* k, const void* v,
                                    const float* alpha_p, const float* beta_p, const float* state_in,
                                    const float* d_o, const float* dstate_out, float* dq, float* dk, float* dv,
                                    float* d_alpha, float* d_beta, float* dstate_in, void* ws, size_t ws_bytes,
                                    void* stream) {
  return mom::chunk_bwd(true, false, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
                        alpha_p, beta_p, state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws,
                        ws_bytes, stream);
}

extern "C" mom_status gla_chunk_bwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                                    int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                                    const int32_t* row_token, const void* q, const void* k, const void* v,
                                    const float* alpha_p, const float* beta_p, const float* state_in,
                                    const float* d_o, const float* dstate_out, float* dq, float* dk, float* dv,
                                    float* d_alpha, float* d_beta, float* dstate_in, void* ws, size_t ws_bytes,
                                    void* stream) {
  return mom::chunk_bwd(false, false, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
                        alpha_p, beta_p, state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws,
                        ws_bytes, stream);
}

#define MOM_FWD_TRAIN_ARGS                                                                                        \
  const mom_dims *dims, int32_t n_seg, int32_t n_rows, int32_t n_tok, int32_t n_state, const int32_t *seg_off,   \
      const int32_t *seg_state, const int32_t *row_token, const void *q, const void *k, const void *v,           \
      const float *alpha_p, const float *beta_p, const float *state_in, float *state_out, float *o, void *ws,     \
      size_t ws_bytes, void *stream
extern "C" mom_status gdn_chunk_fwd_train(MOM_FWD_TRAIN_ARGS) {
  return mom::chunk_fwd_train(true, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
                              alpha_p, beta_p, state_in, state_out, o, ws, ws_bytes, stream);
}
extern "C" mom_status gla_chunk_fwd_train(MOM_FWD_TRAIN_ARGS) {
  return mom::chunk_fwd_train(false, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
                              alpha_p, beta_p, state_in, state_out, o, ws, ws_bytes, stream);
}
#undef MOM_FWD_TRAIN_ARGS

#define MOM_BWD_ARGS                                                                                              \
  const mom_dims *dims, int32_t n_seg, int32_t n_rows, int32_t n_tok, int32_t n_state, const int32_t *seg_off,   \
      const int32_t *seg_state, const int32_t *row_token, const void *q, const void *k, const void *v,           \
      const float *alpha_p, const float *beta_p, const float *state_in, const float *d_o,                        \
      const float *dstate_out, float *dq, float *dk, float *dv, float *d_alpha, float *d_beta, float *dstate_in,  \
      void *ws, size_t ws_bytes, void *stream
extern "C" mom_status gdn_chunk_bwd_saved(MOM_BWD_ARGS) {
  return mom::chunk_bwd(true, true, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
                        alpha_p, beta_p, state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws,
                        ws_bytes, stream);
}
extern "C" mom_status gla_chunk_bwd_saved(MOM_BWD_ARGS) {
  return mom::chunk_bwd(false, true, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
                        alpha_p, beta_p, state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws,
                        ws_bytes, stream);
}
#undef MOM_BWD_ARGS
