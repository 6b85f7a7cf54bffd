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
//   k_gdn_chain16  the walk: one block per (segment, head, 128 value
//                columns; 64 when dv = 64) of eight (four) waves with 16 columns
//                each, walking the segment's chunks in order with the state in
//                float32 matrix-core accumulators (see the comment at the
//                kernel), and the modes that store each chunk's entering state
//                for the gradients.
#include "chunk_mfma.h"

namespace mom {

// ------------------------------------------------------------------ chain, 16-column waves
// The walk with NW waves of 16 value columns each (DVB = 16 NW columns per
// block: 128 with eight waves, 64 with four), on v_mfma_f32_16x16x32_f16.
// Value columns of the state evolve independently, so a wave's part of S
// stays in its float32 accumulators for the whole segment; the kernel fits
// two waves per SIMD, and each SIMD switches to the other wave while one
// waits on LDS reads or on its products.  A block's inputs per chunk (K, Q,
// V, T, P, gamma) sit in a double-buffered LDS image that every wave fills in
// part with asynchronous global -> LDS copies of the next chunk while the
// current one is processed (rows past the segment end repeat its last row; T
// is zero in those rows and columns), with one block barrier per chunk.  Per
// chunk:
//   Y   = K S                         (4 row tiles, dk-deep)
//   O^T = S^T Q^T                     (4 row tiles of the chunk, dk-deep)
//   U   = T V - T diag(gamma) Y       (chunk-deep)
//   O^T = O^T diag(gamma) + U^T P^T
//   S  <- gamma_L S + K^T diag(gamma_L / gamma) U
// The state S (DK x 16, float32) is held as DK / 16 accumulator tiles; its
// 32-row blocks become the dk-deep operand of Y and of O^T (the same
// registers serve as B of K S and as A of S^T Q^T) through acc16_to_op, and so
// do the 32-row blocks of Y and U for the chunk-deep products.  Lane 16 G + c
// ends with the read of chunk row 16 t + c at value columns 4G .. 4G+3 of its
// wave in O[t], which it stores as one 16-byte piece (a row's 16 columns are
// four lanes' contiguous 64 bytes).
//
// MAP: the first phase of the long-segment scan (see launch_chunk_scan below).
// The segments are then the groups of chunks the scan cuts, and each block
// walks its group without read-out (no Q, P or O) from a zero state over the
// real values (ident = 0) or from the identity over zero values (ident = 1, a
// width of dk columns), giving the group's affine state map; groups that end
// their segment are skipped (grp_seg[g + 1] != grp_seg[g]).  The state is
// stored with row width sw at column col_base + the block's columns.
//
// MODE 0 is the forward pass.  For the gradients, MODE 1 only walks the
// states: it stores the state entering every chunk (transposed, half:
// hws[chunk][head][dv][DK], lane 16 G + c writing rows 4G .. 4G+3 of each
// 16-row block of its column) and skips the read-out (no Q, P or O; state_out
// may then be null); MODE 2 does both, the forward pass of a training step,
// whose o and states equal MODE 0's bit for bit.
// Rows of the entering state staged per round in the training modes: as many
// as NW waves' 16 columns fit in one buffer's Q area (GC x DK), at most DK.
template <int DK, int NW>
constexpr int chain16_state_rows() {
  return GC * DK / (NW * 16) < DK ? GC * DK / (NW * 16) : DK;
}

template <int DK, int NW, bool DELTA, bool MAP, int MODE = 0>
__global__ __launch_bounds__(64 * NW) void k_gdn_chain16(
    int H, int dv, int width, int col_base, int sw, int ident, int n_seg, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_state, const int32_t* __restrict__ grp_seg,
    const f16_t* __restrict__ k, const f16_t* __restrict__ v, const f16_t* __restrict__ Tws,
    const f16_t* __restrict__ Pws, const float* __restrict__ Ews, const int32_t* __restrict__ row_token,
    const f16_t* __restrict__ q, const float* __restrict__ state_in, float* __restrict__ state_out,
    float* __restrict__ o, f16_t* __restrict__ hws) {
  static_assert(!MAP || MODE == 0, "the scan's map walk is a forward walk");
  constexpr bool READ = !MAP && MODE != 1;  // the read-out (Q, P, O)
  constexpr int DVB = 16 * NW, ND = DK / 16, NKD = DK / 32;
  constexpr int OFF_K = 0, OFF_Q = GC * DK, OFF_V = 2 * GC * DK, OFF_T = OFF_V + GC * DVB, OFF_P = OFF_T + GC * GC,
                OFF_E = OFF_P + GC * GC, OFF_TOK = OFF_E + 2 * 2 * GC, BUF = OFF_TOK + 2 * GC;
  extern __shared__ __attribute__((aligned(16))) f16_t smem[];

  // blocks of a (segment, head) to one XCD, longest segments (highest s) first
  const int nb = width / DVB;
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
  if (MAP && (grp_seg[s] < 0 || grp_seg[s + 1] != grp_seg[s])) return;  // whole block: no map needed
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, G = lane >> 4;
  const int slot = seg_state ? seg_state[s] : s;
  const int ncol0 = cb * DVB + 16 * w;  // this wave's first column of the launch's width
  const int64_t sbase = ((int64_t)slot * H + h) * DK * sw + col_base + ncol0;
  const bool zero_v = MAP && ident;
  const int64_t rbeg = seg_off[s], rend = seg_off[s + 1];
  const int cbase = chunks_before(seg_off, s, lane);

  // prefetch of the chunk at row r0n into buffer b, NPF copy instructions per
  // wave; rows past the segment end repeat its last row (T is zero there).
  // Each lane's tile row and swizzled 16-byte piece of every copy are fixed for
  // the whole walk; per chunk only wave-uniform bases change, so a copy's
  // address is one base plus a 32-bit element offset.
  using CK = TileCopy<DK, NW>;
  using CV = TileCopy<DVB, NW>;
  using CT = TileCopy<GC, NW>;
  constexpr int NPF = 2 * CK::PER_WAVE + CV::PER_WAVE + 2 * CT::PER_WAVE + 2;
  int k_row[CK::PER_WAVE], k_pc[CK::PER_WAVE], v_row[CV::PER_WAVE], v_pc[CV::PER_WAVE];
  unsigned t_off[CT::PER_WAVE];
#pragma unroll
  for (int j = 0; j < CK::PER_WAVE; ++j) {
    k_row[j] = CK::row(w, lane, j);
    k_pc[j] = 8 * swz<DK>(k_row[j], lane % CK::CPR);
  }
#pragma unroll
  for (int j = 0; j < CV::PER_WAVE; ++j) {
    v_row[j] = CV::row(w, lane, j);
    v_pc[j] = 8 * swz<DVB>(v_row[j], lane % CV::CPR);
  }
#pragma unroll
  for (int j = 0; j < CT::PER_WAVE; ++j) {
    const int r = CT::row(w, lane, j);
    t_off[j] = (unsigned)(r * GC + 8 * swz<GC>(r, lane % CT::CPR));
  }
  const unsigned lds0 = lds_offset(smem);  // LDS byte address of the buffers
  const int64_t hstride = (int64_t)H;
  const f16_t* pf_k = k;
  const f16_t* pf_v = v;
  const f16_t* pf_t = Tws;
  const f16_t* pf_p = Pws;
  int pf_L = 0;
  int64_t pf_r0 = 0, pf_chk = 0;
  unsigned pf_lds = lds0;
  int qtok[CK::PER_WAVE];
  auto pf_setup = [&](int64_t r0n, int b, const int32_t* tok_lds) {
    pf_r0 = r0n;
    pf_L = (int)min((int64_t)GC, rend - r0n);
    pf_chk = (int64_t)(cbase + (r0n - rbeg) / GC) * H + h;
    pf_lds = lds0 + (unsigned)(b * BUF * (int)sizeof(f16_t));
    pf_k = k + (r0n * hstride + h) * DK;
    pf_v = v + (r0n * hstride + h) * dv + cb * DVB;
    pf_t = Tws + pf_chk * GC * GC;
    pf_p = Pws + pf_chk * GC * GC;
#pragma unroll
    for (int j = 0; j < CK::PER_WAVE; ++j) {
      const int r = min(k_row[j], pf_L - 1);
      if (tok_lds) qtok[j] = tok_lds[r];
      else qtok[j] = row_token ? row_token[r0n + r] : (int)(r0n + r);
    }
  };
  // LDS byte address of copy instruction j (tile row RPI (w + NW j)) of a tile at element offset off
  auto lds_at = [&](int off, int rpi, int rh, int j) {
    return pf_lds + (unsigned)((off + rpi * (w + NW * j) * rh) * (int)sizeof(f16_t));
  };
  auto pf_issue = [&](int i) {
    if (i < CK::PER_WAVE) {
      const unsigned e = (unsigned)(min(k_row[i], pf_L - 1) * H * DK + k_pc[i]);
      dma_b128_at(pf_k + e, lds_at(OFF_K, CK::RPI, DK, i));
    } else if ((i -= CK::PER_WAVE) < CK::PER_WAVE) {
      if (!READ) return;  // no read-out: Q is not needed
      dma_b128_at(q + ((int64_t)qtok[i] * H + h) * DK + k_pc[i], lds_at(OFF_Q, CK::RPI, DK, i));
    } else if ((i -= CK::PER_WAVE) < CV::PER_WAVE) {
      if (zero_v) return;
      const unsigned e = (unsigned)(min(v_row[i], pf_L - 1) * H * dv + v_pc[i]);
      dma_b128_at(pf_v + e, lds_at(OFF_V, CV::RPI, DVB, i));
    } else if ((i -= CV::PER_WAVE) < CT::PER_WAVE) {
      dma_b128_at(pf_t + t_off[i], lds_at(OFF_T, CT::RPI, GC, i));
    } else if ((i -= CT::PER_WAVE) < CT::PER_WAVE) {
      if (!READ) return;
      dma_b128_at(pf_p + t_off[i], lds_at(OFF_P, CT::RPI, GC, i));
    } else if (i == CT::PER_WAVE) {
      if (w < 2) dma_b32_at(Ews + pf_chk * 2 * GC + GC * w + lane, pf_lds + (unsigned)((OFF_E + 2 * GC * w) * 2));
    } else if (w == NW - 1) {  // tokens of the following chunk's rows
      const int64_t rn = min(pf_r0 + GC + lane, rend - 1);
      if (row_token) dma_b32_at(row_token + rn, pf_lds + (unsigned)(OFF_TOK * 2));
      else reinterpret_cast<int32_t*>(smem + (pf_lds - lds0) / 2 + OFF_TOK)[lane] = (int32_t)rn;
    }
  };
  constexpr int PY = (NPF + NKD - 1) / NKD;  // copies issued per step of the Y / O loop

  f4v S[ND];
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 16 * a + 4 * G + e;
      if (zero_v) S[a][e] = d == ncol0 + c16 ? 1.f : 0.f;  // identity start
      else S[a][e] = (!MAP && state_in) ? state_in[sbase + (int64_t)d * sw + c16] : 0.f;
    }
  const float ones[4] = {1.f, 1.f, 1.f, 1.f};
  if (rbeg < rend) {
    pf_setup(rbeg, 0, nullptr);
#pragma unroll
    for (int i = 0; i < NPF; ++i) pf_issue(i);
  }

  int buf = 0;
  for (int64_t r0 = rbeg; r0 < rend; r0 += GC, buf ^= 1) {
    const int L = (int)min((int64_t)GC, rend - r0);
    // this wave's copies have landed (only the previous chunk's stores were
    // issued after them: 4 output pieces, and in the training modes DK / 32
    // of the entering state); then every wave's
    if (r0 == rbeg || MAP) vm_wait_all();
    else if (MODE == 1) vm_wait_n<DK / 32>();
    else if (MODE == 2) vm_wait_n<DK / 32 + 4>();
    else vm_wait_4();
    lds_barrier();
    pf_setup(r0 + GC < rend ? r0 + GC : r0, buf ^ 1, reinterpret_cast<const int32_t*>(smem + buf * BUF + OFF_TOK));

    const f16_t* Bc = smem + buf * BUF;
    const f16_t* Ks = Bc + OFF_K;
    const f16_t* Qs = Bc + OFF_Q;
    const f16_t* Vs = Bc + OFF_V;
    const f16_t* Ts = Bc + OFF_T;
    const f16_t* Ps = Bc + OFF_P;
    const float* Eg = reinterpret_cast<const float*>(Bc + OFF_E);  // gamma_i, then gamma_L / gamma_i

    // ---- Y = K S and O^T = S^T Q^T; the state's 32-row blocks as operands
    f4v Y[4], O[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Y[t][e] = 0.f;
        O[t][e] = 0.f;
      }
    // operand reads one k-block ahead of the products that use them
    h8v kf[2][4], qf[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kf[0][t] = row_frag16<DK>(Ks, 16 * t + c16, 0, G);
      if (READ) qf[0][t] = row_frag16<DK>(Qs, 16 * t + c16, 0, G);
    }
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      if (kb + 1 < NKD) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          kf[(kb + 1) & 1][t] = row_frag16<DK>(Ks, 16 * t + c16, kb + 1, G);
          if (READ) qf[(kb + 1) & 1][t] = row_frag16<DK>(Qs, 16 * t + c16, kb + 1, G);
        }
      }
#pragma unroll
      for (int i = PY * kb; i < PY * (kb + 1); ++i)
        if (i < NPF) pf_issue(i);
      const h8v sop = acc16_to_op(S[2 * kb], S[2 * kb + 1], ones, ones);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        Y[t] = mfma16(kf[kb & 1][t], sop, Y[t]);
        if (READ) O[t] = mfma16(sop, qf[kb & 1][t], O[t]);
      }
    }
    // The entering state (S is updated only at the end of the chunk),
    // transposed, as half, issued after the next chunk's copies so that
    // waiting for those does not wait for these stores.  The wave's columns
    // pass through LDS, RR rows at a time (8-byte pieces in, 16-byte pieces
    // out, the 16-byte chunks of each column XOR-swizzled by column), so that
    // every store writes runs of RR / 8 whole 16-byte pieces of a column: in
    // mode 1 through the Q area of the current buffer (no read-out, so never
    // loaded), in mode 2 through an area of its own after the two buffers.
    if constexpr (MODE != 0) {
      f16_t* hw = hws + ((int64_t)(cbase + (r0 - rbeg) / GC) * H + h) * sw * DK + (int64_t)ncol0 * DK;
      constexpr int RR = chain16_state_rows<DK, NW>();  // rows per round
      constexpr int CPC = RR / 8;                       // 16-byte chunks per column
      f16_t* st = (MODE == 1 ? smem + buf * BUF + OFF_Q : smem + 2 * BUF) + w * 16 * RR;
#pragma unroll
      for (int r = 0; r < DK / RR; ++r) {
#pragma unroll
        for (int a = 0; a < RR / 16; ++a) {
          const int ch = 2 * a + G / 2;  // chunk of rows 16 a + 4 G ..
          const int aa = r * (RR / 16) + a;
          const half4 hv = {(f16_t)S[aa][0], (f16_t)S[aa][1], (f16_t)S[aa][2], (f16_t)S[aa][3]};
          *reinterpret_cast<half4*>(st + c16 * RR + 8 * (ch ^ (c16 & (CPC - 1))) + 4 * (G & 1)) = hv;
        }
        wave_lds_fence();
#pragma unroll
        for (int p0 = 0; p0 < 16 * CPC; p0 += 64) {
          const int p = p0 + lane, col = p / CPC, ch = p % CPC;
          const h8v x = *reinterpret_cast<const h8v*>(st + col * RR + 8 * (ch ^ (col & (CPC - 1))));
          *reinterpret_cast<h8v*>(hw + (int64_t)col * DK + r * RR + 8 * ch) = x;
        }
        wave_lds_fence();
      }
    }
    CHAIN_PHASE();
    // ---- U = T V - T diag(gamma) Y
    f4v U[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) U[t][e] = 0.f;
#pragma unroll
    for (int kb = 0; kb < GC / 32; ++kb) {
      h8v vb = {};
      if (!zero_v) vb = col_frag16<DVB>(Vs, kb, 16 * w, lane);
      h8v yb;
      if constexpr (DELTA) {
        float s0[4], s1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s0[e] = -Eg[32 * kb + 4 * G + e];
          s1[e] = -Eg[32 * kb + 16 + 4 * G + e];
        }
        yb = acc16_to_op(Y[2 * kb], Y[2 * kb + 1], s0, s1);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const h8v tf = row_frag16<GC>(Ts, 16 * t + c16, kb, G);
        if (!zero_v) U[t] = mfma16(tf, vb, U[t]);
        if constexpr (DELTA) U[t] = mfma16(tf, yb, U[t]);
      }
    }
    CHAIN_PHASE();
    // ---- U and diag(gamma_L / gamma) U as chunk-deep operands
    h8v ub[GC / 32], u2b[GC / 32];
#pragma unroll
    for (int kb = 0; kb < GC / 32; ++kb) {
      float s0[4], s1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s0[e] = Eg[GC + 32 * kb + 4 * G + e];
        s1[e] = Eg[GC + 32 * kb + 16 + 4 * G + e];
      }
      ub[kb] = acc16_to_op(U[2 * kb], U[2 * kb + 1], ones, ones);
      u2b[kb] = acc16_to_op(U[2 * kb], U[2 * kb + 1], s0, s1);
    }
    // ---- S <- gamma_L S + K^T U' (issued before the read-out, which the next
    // chunk does not need, so that the read-out runs while these products do)
    const float eL = Eg[GC - 1];
#pragma unroll
    for (int a = 0; a < ND; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[a][e] *= eL;
#pragma unroll
    for (int kb = 0; kb < GC / 32; ++kb)
#pragma unroll
      for (int a = 0; a < ND; ++a) S[a] = mfma16(col_frag16<DK>(Ks, kb, 16 * a, lane), u2b[kb], S[a]);
    CHAIN_PHASE();
    // ---- O^T = O^T diag(gamma) + U^T P^T, stored as 16-byte row pieces
#pragma unroll
    for (int t = 0; t < (READ ? 4 : 0); ++t) {
      const float gm = Eg[16 * t + c16];
#pragma unroll
      for (int e = 0; e < 4; ++e) O[t][e] *= gm;
#pragma unroll
      for (int kb = 0; kb < GC / 32; ++kb) O[t] = mfma16(ub[kb], row_frag16<GC>(Ps, 16 * t + c16, kb, G), O[t]);
    }
#pragma unroll
    for (int t = 0; t < (READ ? 4 : 0); ++t)
      if (16 * t + c16 < L)
        *reinterpret_cast<float4*>(o + ((r0 + 16 * t + c16) * H + h) * dv + ncol0 + 4 * G) =
            make_float4(O[t][0], O[t][1], O[t][2], O[t][3]);
  }
  vm_wait_all();  // the last (repeated) prefetch has landed before the block ends
  if (MODE == 1 && !state_out) return;
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) state_out[sbase + (int64_t)(16 * a + 4 * G + e) * sw + c16] = S[a][e];
}

template <int DK, int NW>
constexpr size_t chain16_lds_bytes(int mode = 0) {
  // two buffers, and in mode 2 the entering state's staging area (NW x 16 columns x RR rows)
  return (size_t)2 * (2 * GC * DK + GC * 16 * NW + 2 * GC * GC + 4 * GC + 2 * GC) * sizeof(f16_t) +
         (mode == 2 ? (size_t)NW * 16 * chain16_state_rows<DK, NW>() * sizeof(f16_t) : 0);
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
    g = log_gate(alpha_p[(r0 + lane) * H + h]);
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
size_t gdn_chunk_ws_bytes(int64_t n_seg, int64_t n_rows, int H, int dk, int dv) {
  const size_t chunk = chunk_ws_layout(nullptr, n_seg, n_rows, H, dk).bytes;
  const ScanPlan plan = scan_plan(n_seg, n_rows, H, dv);
  return chunk + (plan.on ? scan_ws_layout(nullptr, n_seg, plan.n_groups, H, dk, dv).bytes : 0);
}

// ------------------------------------------------------------------ long-segment scan
// The state map of a run of chunks is affine: S_out = A S_in + B, B the state
// the run reaches from a zero state, A (dk x dk) the map the run applies to the
// entering state (the state it reaches from the identity with zero values).
// For segments much longer than the grid is wide, gdn_chunk_fwd cuts every
// segment into groups of lg chunks (group boundaries on chunk boundaries, so
// the chunk numbering of the prep's factors is unchanged) and
//   1. walks every group except each segment's last in MAP mode: its B over
//      the dv value columns and its A over dk identity columns, in parallel;
//   2. k_scan_states chains them in order per (segment, head, 32 columns):
//      S_{g+1} = A_g S_g + B_g from the segment's entering state, float32,
//      storing every group's entering state;
//   3. walks every group with read-out from its entering state, in parallel;
//   4. copies each segment's last group's final state to state_out.
// The serial part is the short step 2 instead of the segment's whole walk.

// Groups of lg chunks per segment (one group for an empty segment): grp_off
// [n_groups + 1], grp_seg [n_groups + 1] (-1 past the last group, the
// sentinel), seg_grp0 [n_seg + 1].  lg = max(kScanMinGroup, chunks / target)
// over the segments' actual chunks, or the longest segment's chunk count (no
// segment split) when it is below kScanMinSeg.  One block.
__global__ __launch_bounds__(256) void k_make_groups(int n_seg, const int32_t* __restrict__ seg_off, int target,
                                                     int n_groups, int32_t* __restrict__ grp_off,
                                                     int32_t* __restrict__ grp_seg, int32_t* __restrict__ seg_grp0) {
  __shared__ int32_t wsum[4];
  __shared__ int32_t carry;
  __shared__ int64_t tot_s[4];
  __shared__ int32_t max_s[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t tot = 0;
  int mx = 0;
  for (int s = tid; s < n_seg; s += 256) {
    const int c = seg_chunks(seg_off, s);
    tot += c;
    mx = max(mx, c);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    tot += __shfl_xor(tot, o, 64);
    mx = max(mx, __shfl_xor(mx, o, 64));
  }
  if (lane == 0) {
    tot_s[wv] = tot;
    max_s[wv] = mx;
  }
  if (tid == 0) carry = 0;
  __syncthreads();
  tot = tot_s[0] + tot_s[1] + tot_s[2] + tot_s[3];
  mx = max(max(max_s[0], max_s[1]), max(max_s[2], max_s[3]));
  int lg = (int)((tot + target - 1) / target);
  if (lg < kScanMinGroup) lg = kScanMinGroup;
  if (mx < kScanMinSeg) lg = max(mx, 1);
  const int rows_g = lg * GC;
  for (int base = 0; base < n_seg; base += 256) {
    const int s = base + tid;
    int ng = 0;
    if (s < n_seg) {
      const int len = seg_off[s + 1] - seg_off[s];
      ng = len > 0 ? (len + rows_g - 1) / rows_g : 1;
    }
    int x = ng;  // inclusive scan of the group counts
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(x, o, 64);
      if (lane >= o) x += u;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int pre = carry;
    for (int w2 = 0; w2 < wv; ++w2) pre += wsum[w2];
    const int first = pre + x - ng;
    if (s < n_seg) {
      seg_grp0[s] = first;
      for (int j = 0; j < ng; ++j) {
        grp_off[first + j] = seg_off[s] + j * rows_g;
        grp_seg[first + j] = s;
      }
    }
    __syncthreads();
    if (tid == 255) carry = pre + x;
    __syncthreads();
  }
  const int total = carry;  // <= n_groups (the host's bound)
  if (tid == 0) seg_grp0[n_seg] = total;
  const int32_t end = seg_off[n_seg];
  for (int g = total + tid; g <= n_groups; g += 256) {
    grp_off[g] = end;
    grp_seg[g] = -1;
  }
}

// Step 2: one block per (segment, head, 32 value columns); the state block
// (dk x 32) in LDS, each thread one row and 16 columns of the product.
__global__ __launch_bounds__(256) void k_scan_states(int H, int dk, int dv, int n_seg,
                                                     const int32_t* __restrict__ seg_state,
                                                     const int32_t* __restrict__ seg_grp0,
                                                     const float* __restrict__ maps,
                                                     const float* __restrict__ state_in, float* __restrict__ sg) {
  __shared__ float Sx[128][33];
  const int nb = dv / 32;
  const int cb = blockIdx.x % nb, h = (blockIdx.x / nb) % H, s = blockIdx.x / (nb * H);
  const int slot = seg_state ? seg_state[s] : s;
  const int sw = dv + dk, tid = threadIdx.x;
  for (int e = tid; e < dk * 32; e += 256) {
    const int d = e >> 5, c = e & 31;
    Sx[d][c] = state_in ? state_in[(((int64_t)slot * H + h) * dk + d) * dv + 32 * cb + c] : 0.f;
  }
  __syncthreads();
  const int g0 = seg_grp0[s], g1 = seg_grp0[s + 1];
  const int d = min(tid >> 1, dk - 1), c0 = 16 * (tid & 1);  // threads past dk rows repeat the last one
  // this thread's row of A_g (dk floats) and 16 entries of B_g, loaded one
  // group ahead so the loads run under the previous group's products
  float4 ar[32];
  float br[16];
  auto load = [&](int g) {
    const float* mrow = maps + ((((int64_t)g * H + h) * dk) + d) * sw;
#pragma unroll
    for (int c = 0; c < 16; ++c) br[c] = mrow[32 * cb + c0 + c];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (4 * i < dk) ar[i] = *reinterpret_cast<const float4*>(mrow + dv + 4 * i);
  };
  if (g0 + 1 < g1) load(g0);
  for (int g = g0; g < g1; ++g) {
    float* out = sg + (((int64_t)g * H + h) * dk) * dv + 32 * cb;
    for (int e = tid; e < dk * 32; e += 256) out[(int64_t)(e >> 5) * dv + (e & 31)] = Sx[e >> 5][e & 31];
    if (g + 1 == g1) break;
    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = br[c];  // B_g
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (4 * i >= dk) break;
      const float av[4] = {ar[i].x, ar[i].y, ar[i].z, ar[i].w};  // A_g[d][4i .. 4i + 3]
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[c] = fmaf(av[u], Sx[4 * i + u][c0 + c], acc[c]);
    }
    if (g + 2 < g1) load(g + 1);
    __syncthreads();  // every thread has read the block
    if ((tid >> 1) < dk)
#pragma unroll
      for (int c = 0; c < 16; ++c) Sx[d][c0 + c] = acc[c];
    __syncthreads();
  }
}

// Step 4: each segment's last group's final state to its slot.
__global__ __launch_bounds__(256) void k_scan_final(int H, int dk, int dv, const int32_t* __restrict__ seg_state,
                                                    const int32_t* __restrict__ seg_grp0, const float* __restrict__ sg,
                                                    float* __restrict__ state_out) {
  const int h = blockIdx.x % H, s = blockIdx.x / H;
  const int slot = seg_state ? seg_state[s] : s;
  const int g = seg_grp0[s + 1] - 1;
  const float4* src = reinterpret_cast<const float4*>(sg + ((int64_t)g * H + h) * dk * dv);
  float4* dst = reinterpret_cast<float4*>(state_out + ((int64_t)slot * H + h) * dk * dv);
  for (int e = threadIdx.x; e < dk * dv / 4; e += 256) dst[e] = src[e];
}

// The walk over n_seg segments (or, with MAP, groups): width columns of the
// state from col_base, state rows sw wide (width = sw = dv for the forward).
template <int DK, int NW, bool DELTA, bool MAP, int MODE = 0>
static mom_status launch_chain16(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                                 const ChunkWs& W, const int32_t* row_token, const void* q, const void* k,
                                 const void* v, const float* state_in, float* state_out, float* o, hipStream_t st,
                                 int width, int col_base, int sw, int ident, const int32_t* grp_seg,
                                 f16_t* hws = nullptr) {
  constexpr size_t lds = chain16_lds_bytes<DK, NW>(MODE);
  static bool attr = false;  // the dynamic LDS limit is raised once per kernel
  if (!attr) {
    if (hipFuncSetAttribute((const void*)k_gdn_chain16<DK, NW, DELTA, MAP, MODE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return MOM_ERR_LAUNCH;
    attr = true;
  }
  const int64_t blocks = (int64_t)n_seg * d.H * (width / (16 * NW));
  if (blocks > 0)
    hipLaunchKernelGGL((k_gdn_chain16<DK, NW, DELTA, MAP, MODE>), dim3((unsigned)blocks), dim3(64 * NW), lds, st,
                       d.H, d.dv, width, col_base, sw, ident, n_seg, seg_off, seg_state, grp_seg, (const f16_t*)k,
                       (const f16_t*)v, W.T, W.P, W.E, row_token, (const f16_t*)q, state_in, state_out, o, hws);
  return MOM_OK;
}

template <int DK, bool DELTA>
static mom_status walk(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                       const ChunkWs& W, const int32_t* row_token, const void* q, const void* k, const void* v,
                       const float* state_in, float* state_out, float* o, hipStream_t st) {
  return d.dv % 128 == 0 ? launch_chain16<DK, 8, DELTA, false>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v,
                                                               state_in, state_out, o, st, d.dv, 0, d.dv, 0, nullptr)
                         : launch_chain16<DK, 4, DELTA, false>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v,
                                                               state_in, state_out, o, st, d.dv, 0, d.dv, 0, nullptr);
}

template <int DK, bool DELTA>
static mom_status launch_chunk_scan(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                                    const ChunkWs& W, const ScanWs& X, const ScanPlan& plan, const int32_t* row_token,
                                    const void* q, const void* k, const void* v, const float* state_in,
                                    float* state_out, float* o, hipStream_t st) {
  const int G = (int)plan.n_groups, sw = d.dv + DK;
  hipLaunchKernelGGL(k_make_groups, dim3(1), dim3(256), 0, st, n_seg, seg_off, plan.target, G, X.grp_off, X.grp_seg,
                     X.seg_grp0);
  // 1. the groups' maps: B over the values, A over identity columns
  mom_status r =
      d.dv % 128 == 0
          ? launch_chain16<DK, 8, DELTA, true>(d, G, X.grp_off, nullptr, W, row_token, q, k, v, nullptr, X.maps,
                                               nullptr, st, d.dv, 0, sw, 0, X.grp_seg)
          : launch_chain16<DK, 4, DELTA, true>(d, G, X.grp_off, nullptr, W, row_token, q, k, v, nullptr, X.maps,
                                               nullptr, st, d.dv, 0, sw, 0, X.grp_seg);
  if (r != MOM_OK) return r;
  r = launch_chain16<DK, DK / 16, DELTA, true>(d, G, X.grp_off, nullptr, W, row_token, q, k, v, nullptr, X.maps,
                                               nullptr, st, DK, d.dv, sw, 1, X.grp_seg);
  if (r != MOM_OK) return r;
  // 2. entering state of every group
  hipLaunchKernelGGL(k_scan_states, dim3((unsigned)((int64_t)n_seg * d.H * (d.dv / 32))), dim3(256), 0, st, d.H, DK,
                     d.dv, n_seg, seg_state, X.seg_grp0, X.maps, state_in, X.sg);
  // 3. every group's walk with read-out, from its entering state (in place)
  r = walk<DK, DELTA>(d, G, X.grp_off, nullptr, W, row_token, q, k, v, X.sg, X.sg, o, st);
  if (r != MOM_OK) return r;
  // 4. final states
  hipLaunchKernelGGL(k_scan_final, dim3((unsigned)((int64_t)n_seg * d.H)), dim3(256), 0, st, d.H, DK, d.dv, seg_state,
                     X.seg_grp0, X.sg, state_out);
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
  const ScanPlan plan = scan_plan(n_seg, n_rows, d.H, d.dv);
  const mom_status r =
      plan.on ? launch_chunk_scan<DK, DELTA>(d, n_seg, seg_off, seg_state, W,
                                             scan_ws_layout((char*)ws + W.bytes, n_seg, plan.n_groups, d.H, DK, d.dv),
                                             plan, row_token, q, k, v, state_in, state_out, o, st)
              : walk<DK, DELTA>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v, state_in, state_out, o, st);
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
      d.dv % 128 == 0
          ? launch_chain16<DK, 8, DELTA, false, MODE>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v, state_in,
                                                      state_out, o, st, d.dv, 0, d.dv, 0, nullptr, hws)
          : launch_chain16<DK, 4, DELTA, false, MODE>(d, n_seg, seg_off, seg_state, W, row_token, q, k, v, state_in,
                                                      state_out, o, st, d.dv, 0, d.dv, 0, nullptr, hws);
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
