// Chunkwise Gated DeltaNet on the gfx950 matrix cores (half operands, float32
// accumulation, float32 state).  This is the bfloat16-input path of
// gdn_chunk_fwd.
//
// The recurrence of one memory (gist.science page, "Core mechanism": forget
// then delta update, read after the write) is, per head,
//   S_i = a_i S_{i-1} + k_i u_i^T,  u_i = c_i (v_i - a_i S_{i-1}^T k_i),  o_i = S_i^T q_i.
// For a chunk of rows entering with state S, g_i = sum_{j<=i} log a_j and
// gamma_i = e^{g_i}, unrolling gives the WY / UT form
//   A_ij = c_i e^{g_i-g_j} k_i.k_j (j<i),   T = (I + A)^{-1} diag(c)
//   W = T diag(gamma) K,   U~ = T V,   U = U~ - W S
//   O = diag(gamma) Q S + P U,          P_ij = e^{g_i-g_j} q_i.k_j (j<=i)
//   S <- gamma_L S + (diag(gamma_L / gamma) K)^T U
// Only U, O and the new S depend on the entering state, so the work splits in
// two launches.  The same two kernels, with DELTA false, run memories that use
// gated linear attention instead (S_i = a_i S_{i-1} + c_i k_i v_i^T): there
// A = 0, so T = diag(c), W is not needed and U = T V.
//   k_gdn_prep   fully parallel over (chunk, head): g, A and P from
//                v_mfma_f32_32x32x16_f16 products, then T by a blocked solve
//                (16x16 diagonal blocks by forward substitution, off-diagonal
//                blocks by block products), all in float32.  It stores T and P
//                as half and gamma, gamma_L / gamma as float32.
//   k_gdn_chain  one block per (segment, head, 64 or 128 value columns); it
//                walks the segment's chunks in order with the state in float32
//                matrix-core accumulators (see the comment at the kernel).
#include "chunk_mfma.h"

namespace mom {

// ------------------------------------------------------------------ chain
// One block per (segment, head, DVB = 32 NW value columns), NW waves.  Value
// columns of the state evolve independently, so wave w owns columns
// [32w, 32w + 32) of its block for every key row: its part of S stays in the
// float32 accumulators of v_mfma_f32_32x32x16_f16 for the whole segment.
// Per chunk (rows i, j; K, V, Q, T, P and gamma from LDS):
//   Y   = K S                           (depends on the entering state)
//   U   = T V - T diag(gamma) Y         (= T V - W S with W = T diag(gamma) K)
//   O^T = S^T Q^T diag(gamma) + U^T P^T
//   S  <- gamma_L S + K^T diag(gamma_L / gamma) U
// Every product reads its state-side operand from registers: accumulator rows
// 8q + 4g + t (lane group g = lane / 32) become the 16-deep operand of the next
// product after a v_permlane32_swap between lanes l and l + 32.  Nothing is
// exchanged between waves, so the only block barrier per chunk publishes the
// next chunk's inputs, which every wave prefetches into the idle half of a
// double buffer with asynchronous global -> LDS copies.
// MODE 0 is the forward pass.  For the gradients, MODE 1 only walks the
// states: it stores the state entering every chunk (transposed, half:
// hws[chunk][head][dv][DK]) and skips the read-out (no Q, P or O; state_out may
// then be null); MODE 2 does both, the forward pass of a training step that
// keeps the states for the backward pass.
template <int DK, int NW>
struct ChainLds {
  static constexpr int DVB = 32 * NW;
  static constexpr int OFF_K = 0, OFF_Q = GC * DK, OFF_V = 2 * GC * DK, OFF_T = OFF_V + GC * DVB,
                       OFF_P = OFF_T + GC * GC, OFF_E = OFF_P + GC * GC, OFF_TOK = OFF_E + 2 * 2 * GC;
  static constexpr int BUF = OFF_TOK + 2 * GC;  // halfs per buffer (E: 2 x 64 float32, TOK: 64 int32)
  // after the two buffers: one 32 x 32 float32 output tile per wave
  static constexpr size_t OST = (size_t)2 * BUF * sizeof(f16_t);
  static constexpr size_t BYTES = OST + (size_t)NW * 32 * 32 * sizeof(float);
};

template <int DK, int NW, bool DELTA, int MODE>
__global__ __launch_bounds__(64 * NW) void k_gdn_chain(
    int H, int dv, int n_seg, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_state,
    const f16_t* __restrict__ k, const f16_t* __restrict__ v,
    const f16_t* __restrict__ Tws, const f16_t* __restrict__ Pws, const float* __restrict__ Ews,
    const int32_t* __restrict__ row_token, const f16_t* __restrict__ q, const float* __restrict__ state_in,
    float* __restrict__ state_out, float* __restrict__ o, f16_t* __restrict__ hws) {
  using LY = ChainLds<DK, NW>;
  constexpr int DVB = LY::DVB, ND = DK / 32, NKD = DK / 16;
  constexpr bool SAVE = MODE == 1;            // states only
  constexpr bool STORE_H = MODE != 0;         // the chunk-entry states are stored
  extern __shared__ __attribute__((aligned(16))) f16_t smem[];

  // Blocks of a (segment, head) group are dealt round-robin over the 8 XCDs
  // (block p runs on XCD p % 8), longest segments (highest s) first.
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
  const int cbase = chunks_before(seg_off, s, lane);

  // Inputs of the chunk at row r0n into buffer b, as NPF copy instructions
  // per wave (pf_issue(i), i = 0 .. NPF - 1) that can be spread over the
  // previous chunk's products.  Rows past the segment end repeat its last row;
  // T is zero in those rows and columns, so they contribute nothing to the
  // state, and their outputs are not stored.  Query rows are gathered by token
  // (row_token; the packed row itself when it is null).  The tokens of a
  // chunk's rows travel one chunk ahead, in the TOK area of the previous
  // chunk's buffer, so that no copy waits for an index load (without
  // row_token the area holds the row numbers).
  using CK = TileCopy<DK, NW>;
  using CV = TileCopy<DVB, NW>;
  using CT = TileCopy<GC, NW>;
  constexpr int NPF = 2 * CK::PER_WAVE + CV::PER_WAVE + 2 * CT::PER_WAVE + 2;
  int64_t pf_r0 = 0, pf_chk = 0;
  int pf_L = 0;
  f16_t* pf_B = smem;
  int qtok[CK::PER_WAVE];  // token of this lane's row in each query copy
  // tok_lds: the tokens of the chunk's rows in LDS, or null to read them here
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
      if (SAVE) return;  // no read-out: Q is not needed
      const int64_t t = qtok[i];
      CK::issue(pf_B + LY::OFF_Q, w, lane, i, [&](int r, int c) { return q + (t * H + h) * DK + 8 * c; });
    } else if ((i -= CK::PER_WAVE) < CV::PER_WAVE) {
      CV::issue(pf_B + LY::OFF_V, w, lane, i, [&](int r, int c) {
        return v + ((pf_r0 + min(r, pf_L - 1)) * H + h) * dv + cb * DVB + 8 * c;
      });
    } else if ((i -= CV::PER_WAVE) < CT::PER_WAVE) {
      CT::issue(pf_B + LY::OFF_T, w, lane, i, [&](int r, int c) { return Tws + (pf_chk * GC + r) * GC + 8 * c; });
    } else if ((i -= CT::PER_WAVE) < CT::PER_WAVE) {
      if (SAVE) return;
      CT::issue(pf_B + LY::OFF_P, w, lane, i, [&](int r, int c) { return Pws + (pf_chk * GC + r) * GC + 8 * c; });
    } else if (i == CT::PER_WAVE) {
      if (w < 2) dma_b32(Ews + pf_chk * 2 * GC + GC * w + lane, pf_B + LY::OFF_E + 2 * GC * w);
    } else if (w == NW - 1) {  // tokens of the following chunk's rows
      const int64_t rn = min(pf_r0 + GC + lane, rend - 1);
      if (row_token) dma_b32(row_token + rn, pf_B + LY::OFF_TOK);
      else reinterpret_cast<int32_t*>(pf_B + LY::OFF_TOK)[lane] = (int32_t)rn;
    }
  };
  // copies issued per step of the Y / O loop, the rest during the U loop
  constexpr int PY = NPF / NKD, PU = (NPF - PY * NKD + GC / 16 - 1) / (GC / 16);

  f16x16 S[ND];
  if (state_in) {
#pragma unroll
    for (int a = 0; a < ND; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * a + 8 * (i / 4) + 4 * g2 + (i % 4);
        S[a][i] = state_in[sbase + (int64_t)d * dv + c32];
      }
  } else {
#pragma unroll
    for (int a = 0; a < ND; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[a][i] = 0.f;
  }
  const float ones[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  float* ost = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + LY::OST) + 32 * 32 * w;
  if (rbeg < rend) {
    pf_setup(rbeg, 0, nullptr);
#pragma unroll
    for (int i = 0; i < NPF; ++i) pf_issue(i);
  }

  int buf = 0;
  for (int64_t r0 = rbeg; r0 < rend; r0 += GC, buf ^= 1) {
    const int L = (int)min((int64_t)GC, rend - r0);
    // This wave's part of the chunk's inputs has landed.  Vector memory
    // operations complete in issue order; the only ones issued after the
    // prefetch are the previous chunk's 8 output stores, which need not wait.
    if (r0 == rbeg || SAVE) vm_wait_all();
    else vm_wait_8();
    lds_barrier();  // every wave's part has landed; every wave is done with the other buffer
    pf_setup(r0 + GC < rend ? r0 + GC : r0, buf ^ 1,
             reinterpret_cast<const int32_t*>(smem + buf * LY::BUF + LY::OFF_TOK));

    const f16_t* Bc = smem + buf * LY::BUF;
    const f16_t* Ks = Bc + LY::OFF_K;
    const f16_t* Qs = Bc + LY::OFF_Q;
    const f16_t* Vs = Bc + LY::OFF_V;
    const f16_t* Ts = Bc + LY::OFF_T;
    const f16_t* Ps = Bc + LY::OFF_P;
    const float* Eg = reinterpret_cast<const float*>(Bc + LY::OFF_E);  // gamma_i, then gamma_L / gamma_i
    if constexpr (STORE_H)  // the entering state, transposed, through the wave's output tile
      store_state_t<DK>(hws + ((int64_t)(cbase + (r0 - rbeg) / GC) * H + h) * dv * DK + (int64_t)ncol0 * DK, S,
                        reinterpret_cast<f16_t*>(ost), lane);

    // ---- Y = K S and O^T = S^T Q^T, two 32-row tiles each (four chains); the
    // state becomes an operand (k = key rows) one 16-row block at a time
    f16x16 Y[2], O[2];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Y[bt][i] = 0.f;
        O[bt][i] = 0.f;
      }
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
#pragma unroll
      for (int i = PY * kb; i < PY * (kb + 1); ++i) pf_issue(i);
      const h8v sb = acc_to_b(S[kb / 2], kb % 2, ones);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        Y[bt] = mfma32(row_frag<DK>(Ks, 32 * bt + c32, kb, g2), sb, Y[bt]);
        if (!SAVE) O[bt] = mfma32(sb, row_frag<DK>(Qs, 32 * bt + c32, kb, g2), O[bt]);
      }
    }
    CHAIN_PHASE();
    // ---- U = T V - T diag(gamma) Y
    f16x16 U[2];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int i = 0; i < 16; ++i) U[bt][i] = 0.f;
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb) {
#pragma unroll
      for (int i = PY * NKD + PU * kb; i < PY * NKD + PU * (kb + 1); ++i)
        if (i < NPF) pf_issue(i);
      const h8v vb = col_frag<DVB>(Vs, kb, 32 * w, lane);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) U[bt] = mfma32(row_frag<GC>(Ts, 32 * bt + c32, kb, g2), vb, U[bt]);
    }
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (!DELTA) continue;  // gated linear attention: U = T V (T = diag(c)); Y is then unused
        float sc[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sc[t] = -Eg[32 * bt + 16 * p + 4 * g2 + t];
          sc[4 + t] = -Eg[32 * bt + 16 * p + 8 + 4 * g2 + t];
        }
        const h8v yb = acc_to_b(Y[bt], p, sc);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) U[bi] = mfma32(row_frag<GC>(Ts, 32 * bi + c32, 2 * bt + p, g2), yb, U[bi]);
      }
    CHAIN_PHASE();
    // ---- U and diag(gamma_L / gamma) U as operands (k = chunk rows)
    h8v ub[GC / 16], u2b[GC / 16];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float sc[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sc[t] = Eg[GC + 32 * bt + 16 * p + 4 * g2 + t];
          sc[4 + t] = Eg[GC + 32 * bt + 16 * p + 8 + 4 * g2 + t];
        }
        ub[2 * bt + p] = acc_to_b(U[bt], p, ones);
        u2b[2 * bt + p] = acc_to_b(U[bt], p, sc);
      }
    if constexpr (!SAVE) {
      // ---- O^T += U^T P^T, after S^T Q^T is scaled to S^T Q'^T (column i by gamma_i)
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        const float gm = Eg[32 * bt + c32];
#pragma unroll
        for (int i = 0; i < 16; ++i) O[bt][i] *= gm;
      }
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) O[bt] = mfma32(ub[kb], row_frag<GC>(Ps, 32 * bt + c32, kb, g2), O[bt]);
      // O out through this wave's LDS tile, so that each store writes 8 whole
      // 128-byte rows (lane l: row 8 j + l / 8, columns 4 (l % 8) .. + 3) rather
      // than 32-byte pieces of 32 rows.  Piece c of tile row r sits at position
      // c ^ (r & 7).  8 stores (all lanes active unless this is the last chunk).
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *reinterpret_cast<float4*>(ost + 32 * c32 + 4 * ((2 * qq + g2) ^ (c32 & 7))) =
              make_float4(O[bt][4 * qq], O[bt][4 * qq + 1], O[bt][4 * qq + 2], O[bt][4 * qq + 3]);
        wave_lds_fence();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 8 * j + (lane >> 3), pc = lane & 7;
          const float4 val = *reinterpret_cast<const float4*>(ost + 32 * rr + 4 * (pc ^ (rr & 7)));
          if (32 * bt + rr < L) *reinterpret_cast<float4*>(o + ((r0 + 32 * bt + rr) * H + h) * dv + ncol0 + 4 * pc) = val;
        }
        wave_lds_fence();  // the tile is read before the next half overwrites it
      }
    }
    // ---- S <- gamma_L S + K^T U', U' = diag(gamma_L / gamma) U
    const float eL = Eg[GC - 1];
#pragma unroll
    for (int a = 0; a < ND; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[a][i] *= eL;
#pragma unroll
    for (int kb = 0; kb < GC / 16; ++kb)
#pragma unroll
      for (int a = 0; a < ND; ++a) S[a] = mfma32(col_frag<DK>(Ks, kb, 32 * a, lane), u2b[kb], S[a]);
  }
  vm_wait_all();  // the last (repeated) prefetch has landed before the block ends
  if (SAVE && !state_out) return;
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * a + 8 * (i / 4) + 4 * g2 + (i % 4);
      state_out[sbase + (int64_t)d * dv + c32] = S[a][i];
    }
}

// ------------------------------------------------------------------ prep
// One wave per (chunk, head), four per block; waves share nothing.
//   g, gamma = e^g and gamma_L / gamma from a wave prefix sum of log alpha;
//   K K^T and Q K^T (lower 32x32 tiles) on v_mfma_f32_32x32x16_f16, with both
//   operands loaded straight from global memory as row pieces (lane l holds
//   row 32 t + l % 32, halfs 16 kb + 8 (l / 32) .. + 7, for either side);
//   A_ij = c_i e^{g_i - g_j} k_i.k_j (j < i) to LDS as float32, P_ij =
//   e^{g_i - g_j} q_i.k_j (j <= i) to global as half;
//   X = (I + A)^{-1} by blocked substitution in float32 (below), T = X diag(c)
//   as half, and X itself as half when Xws is given (for the gradients).
// Rows at or past the chunk length L are zero in K, Q, A and P; T is then zero
// in those rows and columns (c = 0 there).
constexpr int PREP_ALD = GC + 4;  // float row stride of A in LDS
// Keeps the scheduler from hoisting the next phase's loads, which would hold
// every operand of the kernel in registers at once.
#define PREP_PHASE() __builtin_amdgcn_sched_barrier(0)

template <int DK, bool DELTA>
__global__ __launch_bounds__(256) void k_gdn_prep(int H, int n_seg, const int32_t* __restrict__ seg_off,
                                                  const int32_t* __restrict__ row_token, const f16_t* __restrict__ q,
                                                  const f16_t* __restrict__ k, const float* __restrict__ alpha_p,
                                                  const float* __restrict__ beta_p, f16_t* __restrict__ Tws,
                                                  f16_t* __restrict__ Pws, float* __restrict__ Ews,
                                                  f16_t* __restrict__ Xws) {
  constexpr int NKD = DK / 16;
  __shared__ __attribute__((aligned(16))) float As_all[4][GC * PREP_ALD];
  __shared__ float gs_all[4][GC];
  __shared__ __attribute__((aligned(16))) float cs_all[4][GC];
  __shared__ __attribute__((aligned(16))) float ys_all[4][16 * 17];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c32 = lane & 31, g2 = lane >> 5;
  const int64_t ch = (int64_t)blockIdx.x * 4 + w;  // chunk * H + head
  const int c = (int)(ch / H), h = (int)(ch % H);
  int lo, cb0;
  if (!locate_chunk(seg_off, n_seg, c, lane, lo, cb0)) return;  // whole wave; no block barrier below
  const int64_t r0 = seg_off[lo] + (int64_t)(c - cb0) * GC;
  const int L = (int)min((int64_t)GC, (int64_t)seg_off[lo + 1] - r0);
  float* As = As_all[w];
  float* gs = gs_all[w];
  float* cs = cs_all[w];
  float* ys = ys_all[w];

  // gates: lane i holds g_i (inclusive prefix of log alpha; 0 past L) and c_i
  float g = 0.f, bb = 0.f;
  if (lane < L) {
    g = logf(alpha_p[(r0 + lane) * H + h]);
    bb = beta_p[(r0 + lane) * H + h];
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float u = __shfl_up(g, off, 64);
    if (lane >= off) g += u;
  }
  const float gL = __shfl(g, GC - 1, 64);
  Ews[ch * 2 * GC + lane] = expf(g);
  Ews[ch * 2 * GC + GC + lane] = expf(gL - g);
  gs[lane] = g;
  cs[lane] = bb;
  wave_lds_fence();  // gs, cs visible to the whole wave
  // K row pieces (zero past L)
  h8v kf[2][NKD];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 32 * t + c32;
    const bool ok = row < L;
    const f16_t* kp = k + ((r0 + (ok ? row : 0)) * H + h) * DK + 8 * g2;
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      const h8v z = {}, kv = *reinterpret_cast<const h8v*>(kp + 16 * kb);
      kf[t][kb] = ok ? kv : z;
    }
  }
  // A' = e^{g_i - g_j} k_i.k_j (j < i), lower tiles (ti, tj) = (0,0), (1,0), (1,1)
#pragma unroll
  for (int x = 0; x < (DELTA ? 3 : 0); ++x) {
    const int ti = x == 0 ? 0 : 1, tj = x == 2 ? 1 : 0;
    f16x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) acc = mfma32(kf[ti][kb], kf[tj][kb], acc);
    const int j = 32 * tj + c32;
    const float gj = gs[j];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 32 * ti + 8 * (e / 4) + 4 * g2 + (e % 4);
      As[i * PREP_ALD + j] = j < i ? __expf(gs[i] - gj) * acc[e] : 0.f;
    }
  }
  PREP_PHASE();
  // Q row pieces and P = (e^{g_i - g_j} q_i.k_j) for j <= i
  f16_t* Pout = Pws + ch * GC * GC;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int row = 32 * ti + c32;
    const bool ok = row < L;
    const int64_t rr = r0 + (ok ? row : 0);
    const int64_t tk = row_token ? (int64_t)row_token[rr] : rr;
    const f16_t* qp = q + (tk * H + h) * DK + 8 * g2;
    h8v qf[NKD];
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      const h8v z = {}, qv = *reinterpret_cast<const h8v*>(qp + 16 * kb);
      qf[kb] = ok ? qv : z;
    }
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      const int j = 32 * tj + c32;
      if (tj > ti) {  // upper tile: zero
#pragma unroll
        for (int e = 0; e < 16; ++e) Pout[(32 * ti + 8 * (e / 4) + 4 * g2 + (e % 4)) * GC + j] = (f16_t)0.f;
        continue;
      }
      f16x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) acc = mfma32(qf[kb], kf[tj][kb], acc);
      const float gj = gs[j];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = 32 * ti + 8 * (e / 4) + 4 * g2 + (e % 4);
        Pout[i * GC + j] = (f16_t)(j <= i ? __expf(gs[i] - gj) * acc[e] : 0.f);
      }
    }
    PREP_PHASE();
  }
  wave_lds_fence();
  if constexpr (!DELTA) {
    // gated linear attention: T = diag(c), row i = lane (zero past L: c = 0 there)
    f16_t* trow = Tws + (ch * GC + lane) * GC;
#pragma unroll
    for (int m = 0; m < GC / 8; ++m) {
      half8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = (f16_t)(8 * m + e == lane ? cs[lane] : 0.f);
      *reinterpret_cast<half8*>(trow + 8 * m) = hv;
    }
    return;
  }
  // X = (I + A)^{-1}, A = diag(c) A' (A' above carries k_i.k_j e^{g_i - g_j}),
  // in 16 x 16 blocks X_ij (block rows i, columns j):
  //   X_bb = (I + A_bb)^{-1}       forward substitution, lane 16 b + cc owns
  //                                column cc of X_bb (float32 VALU)
  //   X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj   (i > j)   v_mfma_f32_16x16x4_f32
  // X_bb overwrites A'_bb in place (no longer needed); X_ij for i > j is kept in
  // the unused upper block (j, i) of the same array, row r at (16 j + r) * ld.
  {
    const int b = lane >> 4, cc = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* arow = As + (16 * b + r) * PREP_ALD + 16 * b;
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < (r & ~3); t += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(arow + t);
        acc = fmaf(a4.x, x[t], acc);
        acc = fmaf(a4.y, x[t + 1], acc);
        acc = fmaf(a4.z, x[t + 2], acc);
        acc = fmaf(a4.w, x[t + 3], acc);
      }
#pragma unroll
      for (int t = r & ~3; t < r; ++t) acc = fmaf(arow[t], x[t], acc);
      x[r] = (r == cc ? 1.f : 0.f) - cs[16 * b + r] * acc;
    }
    wave_lds_fence();  // every lane's reads of A'_bb are done
#pragma unroll
    for (int r = 0; r < 16; ++r) As[(16 * b + r) * PREP_ALD + 16 * b + cc] = x[r];
    wave_lds_fence();
  }
  {
    const int l16 = lane & 15, lg = lane >> 4;
    // X_kj as the B operand (rows 4 kb + lg, column l16)
    auto xblk = [&](int k, int j, int kb) {
      const int r = 4 * kb + lg;
      return k == j ? As[(16 * j + r) * PREP_ALD + 16 * j + l16] : As[(16 * j + r) * PREP_ALD + 16 * k + l16];
    };
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const float ci = cs[16 * i + l16];  // row factor of the A operand rows
#pragma unroll
      for (int j = i - 1; j >= 0; --j) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = j; k < i; ++k)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const float a = ci * As[(16 * i + l16) * PREP_ALD + 16 * k + 4 * kb + lg];
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, xblk(k, j, kb), y, 0, 0, 0);
          }
#pragma unroll
        for (int e = 0; e < 4; ++e) ys[(4 * lg + e) * 17 + l16] = y[e];
        wave_lds_fence();
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float a = As[(16 * i + l16) * PREP_ALD + 16 * i + 4 * kb + lg];  // X_ii
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(a, ys[(4 * kb + lg) * 17 + l16], z, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) As[(16 * j + 4 * lg + e) * PREP_ALD + 16 * i + l16] = -z[e];
        wave_lds_fence();
      }
    }
  }
  // T = X diag(c), row i = lane, eight 16-byte pieces (zero above the diagonal)
  {
    const int i = lane, ib = i >> 4;
    f16_t* trow = Tws + (ch * GC + i) * GC;
    f16_t* xrow = Xws ? Xws + (ch * GC + i) * GC : nullptr;
#pragma unroll
    for (int m = 0; m < GC / 8; ++m) {
      const int jb = m >> 1;
      half8 hv;
      if (jb > ib) {
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (f16_t)0.f;
        if (xrow) *reinterpret_cast<half8*>(xrow + 8 * m) = hv;
      } else {
        const float* src = jb == ib ? As + i * PREP_ALD + 8 * m
                                    : As + (16 * jb + (i & 15)) * PREP_ALD + 16 * ib + 8 * (m & 1);
        const float4 v0 = *reinterpret_cast<const float4*>(src);
        const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
        const float4 c0 = *reinterpret_cast<const float4*>(cs + 8 * m);
        const float4 c1 = *reinterpret_cast<const float4*>(cs + 8 * m + 4);
        const float xv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (f16_t)((jb == ib && 8 * m + e > i) ? 0.f : xv[e] * cv[e]);
        if (xrow) {
          half8 xh;
#pragma unroll
          for (int e = 0; e < 8; ++e) xh[e] = (f16_t)((jb == ib && 8 * m + e > i) ? 0.f : xv[e]);
          *reinterpret_cast<half8*>(xrow + 8 * m) = xh;
        }
      }
      *reinterpret_cast<half8*>(trow + 8 * m) = hv;
    }
  }
}

// ------------------------------------------------------------------ workspace + launch
size_t gdn_chunk_ws_bytes(int64_t n_seg, int64_t n_rows, int H, int dk) {
  return chunk_ws_layout(nullptr, n_seg, n_rows, H, dk).bytes;
}

template <int DK, int NW, bool DELTA, int MODE>
static mom_status launch_chain(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                               const ChunkWs& W, const int32_t* row_token, const void* q, const void* k,
                               const void* v, const float* state_in, float* state_out, float* o, f16_t* hws,
                               hipStream_t st) {
  using LY = ChainLds<DK, NW>;
  static bool attr = false;  // the dynamic LDS limit is raised once per kernel
  if (!attr) {
    if (hipFuncSetAttribute((const void*)k_gdn_chain<DK, NW, DELTA, MODE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)LY::BYTES) != hipSuccess)
      return MOM_ERR_LAUNCH;
    attr = true;
  }
  const int64_t blocks = (int64_t)n_seg * d.H * (d.dv / LY::DVB);
  if (blocks > 0)
    hipLaunchKernelGGL((k_gdn_chain<DK, NW, DELTA, MODE>), dim3((unsigned)blocks), dim3(64 * NW), LY::BYTES, st,
                       d.H, d.dv, n_seg, seg_off, seg_state, (const f16_t*)k, (const f16_t*)v, W.T, W.P, W.E,
                       row_token, (const f16_t*)q, state_in, state_out, o, hws);
  return MOM_OK;
}

template <int DK, bool DELTA>
static mom_status launch_chunk(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                               const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                               const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                               float* state_out, float* o, void* ws, hipStream_t st) {
  const ChunkWs W = chunk_ws_layout(ws, n_seg, n_rows, d.H, d.dk);
  const int64_t nch = (int64_t)n_rows / GC + n_seg;
  const int64_t prep_blocks = (nch * d.H + 3) / 4;  // one wave per (chunk, head)
  if (prep_blocks > 0)
    hipLaunchKernelGGL((k_gdn_prep<DK, DELTA>), dim3((unsigned)prep_blocks), dim3(256), 0, st, d.H, n_seg,
                       seg_off, row_token, (const f16_t*)q, (const f16_t*)k, alpha_p, beta_p, W.T, W.P, W.E,
                       nullptr);
  const mom_status r =
      d.dv % 128 == 0
          ? launch_chain<DK, 4, DELTA, 0>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v, state_in,
                                          state_out, o, nullptr, st)
          : launch_chain<DK, 2, DELTA, 0>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v, state_in,
                                          state_out, o, nullptr, st);
  if (r != MOM_OK) return r;
  return launch_status();
}

// delta: Gated DeltaNet memories; otherwise gated linear attention (T = diag(c)
// and no W S term).
mom_status launch_gdn_chunk_mfma(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                                 const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                                 const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                                 float* state_out, float* o, void* ws, bool delta, hipStream_t st) {
  if (d.dk == 64)
    return delta ? launch_chunk<64, true>(d, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                                          state_in, state_out, o, ws, st)
                 : launch_chunk<64, false>(d, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p,
                                           beta_p, state_in, state_out, o, ws, st);
  return delta ? launch_chunk<128, true>(d, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                                         state_in, state_out, o, ws, st)
               : launch_chunk<128, false>(d, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                                          state_in, state_out, o, ws, st);
}


// For the gradients: prep (also writing X = (I + A)^{-1}, solved in float32 and
// stored as half, for Gated DeltaNet) and the walk that stores the state
// entering every chunk (transposed, half) in hws: without the read-out (MODE 1)
// or with it, o and state_out written as in the forward pass (MODE 2).
template <int DK, bool DELTA, int MODE>
static mom_status launch_states(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                                const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                                const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                                float* state_out, float* o, const ChunkWs& W, f16_t* Xws, f16_t* hws,
                                hipStream_t st) {
  const int64_t nch = (int64_t)n_rows / GC + n_seg;
  const int64_t prep_blocks = (nch * d.H + 3) / 4;
  if (prep_blocks > 0)
    hipLaunchKernelGGL((k_gdn_prep<DK, DELTA>), dim3((unsigned)prep_blocks), dim3(256), 0, st, d.H, n_seg,
                       seg_off, row_token, (const f16_t*)q, (const f16_t*)k, alpha_p, beta_p, W.T, W.P, W.E,
                       DELTA ? Xws : nullptr);
  const mom_status r =
      d.dv % 128 == 0 ? launch_chain<DK, 4, DELTA, MODE>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v, state_in,
                                                         state_out, o, hws, st)
                      : launch_chain<DK, 2, DELTA, MODE>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v, state_in,
                                                         state_out, o, hws, st);
  return r != MOM_OK ? r : launch_status();
}

// with_output: also the forward's read-out and final states (a training
// step's forward pass); otherwise the states only (recomputed for the
// gradients).
mom_status launch_chunk_states(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                               const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                               const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                               float* state_out, float* o, const ChunkWs& W, f16_t* Xws, f16_t* hws, bool delta,
                               bool with_output, hipStream_t st) {
#define MOM_STATES(DK, DELTA, MODE)                                                                                 \
  launch_states<DK, DELTA, MODE>(d, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,       \
                                 state_in, state_out, o, W, Xws, hws, st)
  if (with_output) {
    if (d.dk == 64) return delta ? MOM_STATES(64, true, 2) : MOM_STATES(64, false, 2);
    return delta ? MOM_STATES(128, true, 2) : MOM_STATES(128, false, 2);
  }
  if (d.dk == 64) return delta ? MOM_STATES(64, true, 1) : MOM_STATES(64, false, 1);
  return delta ? MOM_STATES(128, true, 1) : MOM_STATES(128, false, 1);
#undef MOM_STATES
}

}  // namespace mom
