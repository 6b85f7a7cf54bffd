// Projections of the MoM layer: the shared query projection over every token
// and, per memory, its own key/value projections over the rows routed to it
// (research.elamur.ai summary, "Summary": each memory has its own key/value
// projections).  Keys are L2-normalised per head.
//
// bfloat16 path: one grouped "TN" GEMM on the matrix cores
// (v_mfma_f32_32x32x16_bf16), both operands K-contiguous:
//   C[r][c] = sum_d A[r][d] * W[c][d],  A rows gathered through perm.
// Logical tiles: first the query tiles (rows = tokens), then for every memory
// m = 0..M the tiles of its packed rows, whose columns run over [W_k[m]; W_v[m]]
// (see k_project_bf16 for the tile shapes).
// The blockIdx -> tile map is XCD-aware: every XCD receives one contiguous
// range of logical tiles, so the column tiles that share a row tile run on the
// same XCD and reuse its L2 copy of the gathered rows.
// The epilogue normalises each key row over its head, converts to half and
// writes through an LDS-staged tile with 16-byte stores.
//
// float32 path: a plain 64 x 64 VALU tiled GEMM with the same tile order, then
// a row-normalisation kernel for the keys.
#include "common.h"

namespace mom {

// ------------------------------------------------------------------ tile map
struct TileJob {
  int kind;        // 0 = query, 1 = key, 2 = value, -1 = none
  int m;           // memory (key/value)
  bool direct;     // rows are tokens in order (queries, the shared memory): no perm read
  int64_t row0;    // first row of the group (packed row for k/v, token for q)
  int64_t rows;    // rows in the group
  int64_t trow;    // first row of this tile inside the group
  int col0;        // first output column inside the k or v matrix
};

// Parts of the tile map: 0 = everything; 1 = the queries and the shared
// memory's keys and values (rows NR .. NR + NT, which are the tokens in order:
// neither seg_off nor perm is read); 2 = the routed memories' keys and values.
template <int BM, int BN>
__device__ TileJob decode_tile(int64_t L, int64_t NT, int64_t NR, int M, int B, int HK, int HV,
                               const int32_t* __restrict__ seg_off, int part) {
  TileJob j;
  j.kind = -1;
  const int qcols = HK / BN;
  const int64_t qtiles = part == 2 ? 0 : (int64_t)((NT + BM - 1) / BM) * qcols;
  if (L < qtiles) {
    j.kind = 0;
    j.m = 0;
    j.direct = true;
    j.row0 = 0;
    j.rows = NT;
    j.trow = (L / qcols) * BM;
    j.col0 = (int)(L % qcols) * BN;
    return j;
  }
  L -= qtiles;
  const int kvcols = (HK + HV) / BN;
  for (int m = part == 1 ? M : 0; m <= (part == 2 ? M - 1 : M); ++m) {
    const int64_t r0 = m == M ? NR : seg_off[m * B];
    const int64_t r1 = m == M ? NR + NT : seg_off[(m + 1) * B];
    const int64_t nt = ((r1 - r0 + BM - 1) / BM) * kvcols;
    if (L < nt) {
      const int ct = (int)(L % kvcols);
      j.m = m;
      j.direct = m == M;
      j.row0 = r0;
      j.rows = r1 - r0;
      j.trow = (L / kvcols) * BM;
      if (ct * BN < HK) {
        j.kind = 1;
        j.col0 = ct * BN;
      } else {
        j.kind = 2;
        j.col0 = ct * BN - HK;
      }
      return j;
    }
    L -= nt;
  }
  return j;
}


inline int64_t n_tiles_bound(const mom_dims& d, int BM, int BN, int part = 0) {
  const Sizes s = sizes_of(d);
  const int64_t kvc = (d.H * d.dk + d.H * d.dv) / BN;
  const int64_t qt = ((s.NT + BM - 1) / BM) * (d.H * d.dk / BN);
  const int64_t shared = ((s.NT + BM - 1) / BM) * kvc;
  const int64_t routed = ((s.NR + BM - 1) / BM + d.M) * kvc;
  return part == 1 ? qt + shared : part == 2 ? routed : qt + shared + routed;
}

// ------------------------------------------------------------------ bf16 MFMA GEMM
// Tiles of BM tokens x BN output features, 2 x NWN waves; wave tile (32 IT)
// tokens x (32 JF) features = IT x JF tiles of v_mfma_f32_32x32x16_bf16 with the
// weights as the A operand, so each lane's accumulators hold four consecutive
// output features.  K-steps of BK through an NS-stage LDS ring filled by direct
// global->LDS loads (global_load_lds_dwordx4: lane l's 16 bytes land at
// base + 16 l), so the gathered rows never pass through registers.  A stage
// holds the BM token rows then the BN weight rows, 2 BK bytes each, with the
// 16-byte pieces of each row permuted (ProjCfg::swz) so that the 32-row operand
// reads are conflict-free.  The wave tile sets the LDS traffic per MFMA; a
// 128 x 128 wave tile (4 waves on 256 x 256) reads a third fewer bytes per
// product than 128 x 64, but needs one wave per SIMD for its 256 accumulators,
// hides less latency than two waves of 128 x 64 and measured slower.  A 64-deep
// K step with two stages halves the barriers per MFMA of a 32-deep step with
// four stages in the same LDS and measured 2% faster.
//   ProjCfg<4, 2, 4, 64, 2>: 256 x 256, 8 waves, wave tile 128 x 64 (large batches)
//   ProjCfg<2, 2, 1, 64, 2>: 64 x 128, 4 waves, wave tile 32 x 64 (small batches
//                     such as decode steps, where a few hundred tiles each walk
//                     the whole K = D: many short tiles and two 64-deep stages
//                     in 48 KB of LDS measured 28 us for the 256-sequence
//                     decode projections against 41 us for 128 x 128 tiles with
//                     four 32-deep stages)

__device__ __forceinline__ void lds_dma16(const void* g, bf16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int NWN_, int JF_, int IT_, int BK_ = 32, int NS_ = 4>
struct ProjCfg {
  static constexpr int NWN = NWN_, JF = JF_, IT = IT_, BK = BK_, NS = NS_;
  static constexpr int NW = 2 * NWN, THREADS = 64 * NW;
  static constexpr int BM = 2 * 32 * IT, BN = NWN * 32 * JF;
  static constexpr int CPR = BK / 8;          // 16-byte pieces per stage row
  static constexpr int RPI = 64 / CPR;        // stage rows per load instruction
  static constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per ring stage
  static constexpr int LPW = (BM + BN) / (RPI * NW);  // loads per wave per stage
  static constexpr size_t LDS = (size_t)NS * STAGE * sizeof(bf16_t);
  static_assert((BM + BN) % (RPI * NW) == 0, "stage rows must split evenly over the waves");
  static_assert(BM % RPI == 0, "a load never straddles the token and weight rows");
  static_assert(BK == 32 || BK == 64, "stage rows of 64 or 128 bytes");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  // position of 16-byte piece c of stage row r: 32-row operand reads conflict-free
  __device__ static int swz(int r, int c) { return BK == 32 ? c ^ ((r >> 2) & 3) : c ^ ((r >> 1) & 7); }
};

// One tile (rows job.trow .. + CF::BM of the job's group, columns job.col0 ..
// + CF::BN) with the CF wave layout; smem_l is the block's dynamic LDS.
template <class CF>
__device__ __forceinline__ void project_tile(const TileJob& job, bf16_t* smem_l, int D, int H, int dk, int dv,
                                             const bf16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                             const bf16_t* __restrict__ wq, const bf16_t* __restrict__ wk,
                                             const bf16_t* __restrict__ wv, f16_t* __restrict__ q,
                                             f16_t* __restrict__ k, f16_t* __restrict__ v) {
  constexpr int BM = CF::BM, BN = CF::BN, IT = CF::IT, JF = CF::JF, NWN = CF::NWN, LPW = CF::LPW;
  constexpr int BK = CF::BK, NS = CF::NS, CPR = CF::CPR, RPI = CF::RPI;
  constexpr int RPW = RPI * LPW;  // stage rows copied by one wave
  const int HK = H * dk, HV = H * dv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / NWN, wn = w % NWN;

  const bf16_t* W;
  if (job.kind == 0) W = wq + (int64_t)job.col0 * D;
  else if (job.kind == 1) W = wk + ((int64_t)job.m * HK + job.col0) * D;
  else W = wv + ((int64_t)job.m * HV + job.col0) * D;

  // loads: wave w, instruction j covers stage rows RPW w + RPI j + lane / CPR
  // (token rows first, then weight rows), LDS position lane % CPR holding the
  // global piece swz(row, lane % CPR)
  const bf16_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int R = RPW * w + RPI * j + lane / CPR;
    const int c = CF::swz(R, lane % CPR);
    if (R < BM) {
      int64_t gr = job.trow + R;
      if (gr >= job.rows) gr = job.rows - 1;  // rows past the end reuse the last row; never stored
      const int64_t tok = job.direct ? gr : (int64_t)perm[job.row0 + gr];
      src[j] = x + tok * D + 8 * c;
    } else {
      src[j] = W + (int64_t)(R - BM) * D + 8 * c;
    }
  }
  auto issue = [&](int kt) {
    bf16_t* st = smem_l + (kt % NS) * CF::STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(src[j] + kt * BK, st + (RPW * w + RPI * j) * BK);
  };

  // acc[jf][it]: element e holds feature (32 JF) wn + 32 jf + 8 (e / 4) + 4 g + (e % 4)
  // of token (BM / 2) wm + 32 it + l32 (g = lane / 32, l32 = lane % 32)
  f32x16 acc[JF][IT];
#pragma unroll
  for (int jf = 0; jf < JF; ++jf)
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[jf][it][e] = 0.f;
  const int l32 = lane & 31, g = lane >> 5;

  // Operand pieces of one 16-deep k block of stage kt (ring slot kt % NS).
  auto read_frags = [&](int kt, int kb, bfv8* wf, bfv8* xf) {
    const bf16_t* As = smem_l + (kt % NS) * CF::STAGE;
    const bf16_t* Bs = As + BM * BK;
    const int ch = 2 * kb + g;  // 16-byte piece of the stage row
#pragma unroll
    for (int jf = 0; jf < JF; ++jf) {
      const int r = 32 * JF * wn + 32 * jf + l32;
      wf[jf] = *reinterpret_cast<const bfv8*>(Bs + r * BK + 8 * CF::swz(r, ch));
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (BM / 2) * wm + 32 * it + l32;
      xf[it] = *reinterpret_cast<const bfv8*>(As + r * BK + 8 * CF::swz(r, ch));
    }
  };
  auto mfmas = [&](const bfv8* wf, const bfv8* xf) {
#pragma unroll
    for (int jf = 0; jf < JF; ++jf)
#pragma unroll
      for (int it = 0; it < IT; ++it)
        acc[jf][it] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[jf], xf[it], acc[jf][it], 0, 0, 0);
  };
  // Stage kt has landed once at most the loads of the stages issued after it
  // (LPW per stage per wave) are outstanding.
  auto wait_stage = [&](int later) {
    if (NS >= 4 && later >= 2) wait_vm<2 * LPW>();
    else if (NS >= 3 && later >= 1) wait_vm<LPW>();
    else wait_vm<0>();
  };

  // Software pipeline over the BK / 16 sub-blocks of each stage: the MFMAs of
  // one sub-block run while the operand reads of the next are in flight; the
  // barrier that publishes stage kt + 1 sits before the last sub-block of kt.
  constexpr int KB = BK / 16;
  const int nk = D / BK;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st);
  wait_stage(min(NS - 2, nk - 1));
  lds_sync();
  if (NS - 1 < nk) issue(NS - 1);
  bfv8 wfr[2][JF], xfr[2][IT];
  read_frags(0, 0, wfr[0], xfr[0]);
  for (int kt = 0; kt + 1 < nk; ++kt) {
#pragma unroll
    for (int kb = 0; kb + 1 < KB; ++kb) {
      read_frags(kt, kb + 1, wfr[(kb + 1) & 1], xfr[(kb + 1) & 1]);
      mfmas(wfr[kb & 1], xfr[kb & 1]);
    }
    wait_stage(min(NS - 2, nk - 2 - kt));
    lds_sync();  // stage kt + 1 visible; every wave is done reading stage kt
    if (kt + NS < nk) issue(kt + NS);
    read_frags(kt + 1, 0, wfr[KB & 1], xfr[KB & 1]);
    mfmas(wfr[(KB - 1) & 1], xfr[(KB - 1) & 1]);
  }
#pragma unroll
  for (int kb = 0; kb + 1 < KB; ++kb) {
    read_frags(nk - 1, kb + 1, wfr[(kb + 1) & 1], xfr[(kb + 1) & 1]);
    mfmas(wfr[kb & 1], xfr[kb & 1]);
  }
  mfmas(wfr[(KB - 1) & 1], xfr[(KB - 1) & 1]);
  lds_sync();  // every wave done with the ring: LDS is free for the epilogue

  // ---- key rows normalised per head: scl[it][jf] = 1 / |k| of the head that
  // feature block jf belongs to (1 for queries and values), applied while the
  // accumulators are converted below
  float scl[IT][JF];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int jf = 0; jf < JF; ++jf) scl[it][jf] = 1.f;
  if (job.kind == 1) {
    constexpr int FW = 32 * JF;  // features per wave
    if (dk >= FW) {              // a head spans dk / FW waves: partial sums through LDS
      float* red = reinterpret_cast<float*>(smem_l);  // [NWN][BM tokens]
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        float s = 0.f;
#pragma unroll
        for (int jf = 0; jf < JF; ++jf)
#pragma unroll
          for (int e = 0; e < 16; ++e) s = fmaf(acc[jf][it][e], acc[jf][it][e], s);
        s += __shfl_xor(s, 32, 64);  // sum over this wave's features
        if (g == 0) red[wn * BM + (BM / 2) * wm + 32 * it + l32] = s;
      }
      lds_sync();
      const int per_head = dk / FW;
      const int w0h = (wn / per_head) * per_head;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int tt = (BM / 2) * wm + 32 * it + l32;
        float s = 0.f;
        for (int u = 0; u < per_head; ++u) s += red[(w0h + u) * BM + tt];
        const float inv_n = 1.0f / sqrtf(s);
#pragma unroll
        for (int jf = 0; jf < JF; ++jf) scl[it][jf] = inv_n;
      }
      lds_sync();
    } else {  // a wave holds FW / dk whole heads of dk / 32 feature blocks each
      const int jph = dk / 32;
#pragma unroll
      for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int h0 = 0; h0 < JF; ++h0) {
          if (h0 % jph) continue;
          float s = 0.f;
#pragma unroll
          for (int jf = 0; jf < JF; ++jf)
            if (jf >= h0 && jf < h0 + jph)
#pragma unroll
              for (int e = 0; e < 16; ++e) s = fmaf(acc[jf][it][e], acc[jf][it][e], s);
          s += __shfl_xor(s, 32, 64);
          const float inv_n = 1.0f / sqrtf(s);
#pragma unroll
          for (int jf = 0; jf < JF; ++jf)
            if (jf >= h0 && jf < h0 + jph) scl[it][jf] = inv_n;
        }
    }
  }
  // ---- output through LDS, BM / 2 tokens (one wm half) at a time, 16-byte stores
  f16_t* out;
  int ld;
  int64_t orow0;
  if (job.kind == 0) {
    out = q;
    ld = HK;
    orow0 = job.trow;
  } else if (job.kind == 1) {
    out = k;
    ld = HK;
    orow0 = job.row0 + job.trow;
  } else {
    out = v;
    ld = HV;
    orow0 = job.row0 + job.trow;
  }
  const int64_t nrows = job.rows - job.trow < BM ? job.rows - job.trow : BM;
  constexpr int CLD = BN + 8;
  constexpr int HR = BM / 2;  // tokens per half
  static_assert((size_t)HR * CLD * sizeof(f16_t) <= CF::LDS, "output staging fits the ring");
  static_assert((HR * BN / 8) % CF::THREADS == 0, "output pieces split evenly");
  f16_t* Cs = reinterpret_cast<f16_t*>(smem_l);  // [HR tokens][CLD]
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int jf = 0; jf < JF; ++jf)
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float sc = scl[it][jf];
            const half4 hv = {(f16_t)(acc[jf][it][4 * qq] * sc), (f16_t)(acc[jf][it][4 * qq + 1] * sc),
                              (f16_t)(acc[jf][it][4 * qq + 2] * sc), (f16_t)(acc[jf][it][4 * qq + 3] * sc)};
            *reinterpret_cast<half4*>(Cs + (32 * it + l32) * CLD + 32 * JF * wn + 32 * jf + 8 * qq + 4 * g) = hv;
          }
    }
    lds_sync();
#pragma unroll
    for (int p = 0; p < (HR * BN / 8) / CF::THREADS; ++p) {
      const int c = tid + CF::THREADS * p;
      const int r = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
      const int64_t row = HR * half + r;
      if (row < nrows)
        *reinterpret_cast<uint4*>(out + (orow0 + row) * ld + job.col0 + c8) =
            *reinterpret_cast<const uint4*>(Cs + r * CLD + c8);
    }
    lds_sync();
  }
}

// Tiles of CF (the first n_main tiles of the tile map) then, when the last
// round of tiles would leave most compute units idle, the remaining tiles cut
// into CF::BM / CFT::BM sub-tiles of CFT::BM rows each (same columns), so the
// last round is a fraction of a tile long.  Block p < n_main takes tile
// xcd_remap(p); block n_main + s takes sub-tile s % SPLIT of tile
// n_main + s / SPLIT.
template <class CF, class CFT>
__global__ __launch_bounds__(CF::THREADS) void k_project_bf16(
    int64_t n_main, int64_t NT, int64_t NR, int part, int D, int H, int dk, int dv, int M, int B,
    const bf16_t* __restrict__ x,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ seg_off, const bf16_t* __restrict__ wq,
    const bf16_t* __restrict__ wk, const bf16_t* __restrict__ wv, f16_t* __restrict__ q, f16_t* __restrict__ k,
    f16_t* __restrict__ v) {
  static_assert(CF::THREADS == CFT::THREADS && CF::BN == CFT::BN && CF::BM % CFT::BM == 0, "sub-tiles of CF");
  constexpr int SPLIT = CF::BM / CFT::BM;
  extern __shared__ __attribute__((aligned(16))) bf16_t smem_l[];
  const int HK = H * dk, HV = H * dv;
  const int64_t p = blockIdx.x;
  if (p < n_main) {
    const TileJob job = decode_tile<CF::BM, CF::BN>(xcd_remap(p, n_main), NT, NR, M, B, HK, HV, seg_off, part);
    if (job.kind < 0) return;
    project_tile<CF>(job, smem_l, D, H, dk, dv, x, perm, wq, wk, wv, q, k, v);
  } else {
    const int64_t t = p - n_main;
    TileJob job = decode_tile<CF::BM, CF::BN>(n_main + t / SPLIT, NT, NR, M, B, HK, HV, seg_off, part);
    if (job.kind < 0) return;
    job.trow += (t % SPLIT) * CFT::BM;
    if (job.trow >= job.rows) return;  // a sub-tile past the end of the group
    project_tile<CFT>(job, smem_l, D, H, dk, dv, x, perm, wq, wk, wv, q, k, v);
  }
}

template <class CF, class CFT>
static mom_status launch_project_bf16(const mom_dims& d, const Sizes& z, const void* x, const int32_t* perm,
                                      const int32_t* seg_off, const void* w_q, const void* w_k, const void* w_v,
                                      void* q, void* k, void* v, int part, hipStream_t st) {
  // blocks that fit on the device at once, found once per device
  static int slots_dev = -1, slots = 0;  // benign if two threads race
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOM_ERR_LAUNCH;
  if (dev != slots_dev) {
    if (hipFuncSetAttribute((const void*)k_project_bf16<CF, CFT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)CF::LDS) != hipSuccess)
      return MOM_ERR_LAUNCH;
    int n_cu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_project_bf16<CF, CFT>, CF::THREADS,
                                                     CF::LDS) != hipSuccess)
      return MOM_ERR_LAUNCH;
    slots = n_cu * (per_cu > 0 ? per_cu : 1);
    slots_dev = dev;
  }
  // The tile map's tile count is a bound (the exact count depends on seg_off,
  // which stays on the device); a last round of at most half the slots is cut
  // into sub-tiles.
  constexpr int SPLIT = CF::BM / CFT::BM;
  const int64_t n_tiles = n_tiles_bound(d, CF::BM, CF::BN, part);
  const int64_t rem = slots > 0 ? n_tiles % slots : 0;
  const int64_t n_main = (rem > 0 && 2 * rem <= slots) ? n_tiles - rem : n_tiles;
  const int64_t G = n_main + (n_tiles - n_main) * SPLIT;
  static_assert(CF::LDS >= CFT::LDS, "one LDS size serves both tile shapes");
  hipLaunchKernelGGL((k_project_bf16<CF, CFT>), dim3((unsigned)G), dim3(CF::THREADS), CF::LDS, st, n_main, z.NT,
                     z.NR, part, d.D, d.H, d.dk, d.dv, d.M, d.B, (const bf16_t*)x, perm, seg_off, (const bf16_t*)w_q,
                     (const bf16_t*)w_k, (const bf16_t*)w_v, (f16_t*)q, (f16_t*)k, (f16_t*)v);
  return MOM_OK;
}

// ------------------------------------------------------------------ fp32 VALU GEMM
constexpr int PF_M = 64, PF_N = 64, PF_K = 16;

__global__ __launch_bounds__(256) void k_project_f32(int64_t NT, int64_t NR, int part, int D, int H, int dk, int dv,
                                                     int M, int B,
                                                     const float* __restrict__ x, const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ seg_off, const float* __restrict__ wq,
                                                     const float* __restrict__ wk, const float* __restrict__ wv,
                                                     float* __restrict__ q, float* __restrict__ k, float* __restrict__ v) {
  __shared__ float As[PF_K][PF_M + 4];
  __shared__ float Bs[PF_K][PF_N + 4];
  const int HK = H * dk, HV = H * dv;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const TileJob job = decode_tile<PF_M, PF_N>(L, NT, NR, M, B, HK, HV, seg_off, part);
  if (job.kind < 0) return;
  const float* W;
  if (job.kind == 0) W = wq + (int64_t)job.col0 * D;
  else if (job.kind == 1) W = wk + ((int64_t)job.m * HK + job.col0) * D;
  else W = wv + ((int64_t)job.m * HV + job.col0) * D;
  const int tid = threadIdx.x;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  int64_t gr = job.trow + lr;
  if (gr >= job.rows) gr = job.rows - 1;
  const int64_t tok = job.direct ? gr : (int64_t)perm[job.row0 + gr];
  const float* a_src = x + tok * D + lk;
  const float* b_src = W + (int64_t)lr * D + lk;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < D; k0 += PF_K) {
    const float4 a = *reinterpret_cast<const float4*>(a_src + k0);
    const float4 b = *reinterpret_cast<const float4*>(b_src + k0);
    As[lk + 0][lr] = a.x; As[lk + 1][lr] = a.y; As[lk + 2][lr] = a.z; As[lk + 3][lr] = a.w;
    Bs[lk + 0][lr] = b.x; Bs[lk + 1][lr] = b.y; Bs[lk + 2][lr] = b.z; Bs[lk + 3][lr] = b.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < PF_K; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* out;
  int ld;
  int64_t orow0;
  if (job.kind == 0) {
    out = q;
    ld = HK;
    orow0 = job.trow;
  } else if (job.kind == 1) {
    out = k;
    ld = HK;
    orow0 = job.row0 + job.trow;
  } else {
    out = v;
    ld = HV;
    orow0 = job.row0 + job.trow;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (job.trow + r < job.rows) {
      float4 o = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      *reinterpret_cast<float4*>(out + (orow0 + r) * ld + job.col0 + tx * 4) = o;
    }
  }
}

// Normalise rows of length n (<= 128) in place: one wave per row.
__global__ __launch_bounds__(256) void k_l2norm_rows_f32(int64_t rows, int n, float* __restrict__ a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  if (r >= rows) return;
  float* p = a + r * n;
  const float v0 = lane < n ? p[lane] : 0.f;
  const float v1 = lane + 64 < n ? p[lane + 64] : 0.f;
  float s = wave_sum_xor(fmaf(v0, v0, v1 * v1));
  const float inv_n = 1.0f / sqrtf(s);
  if (lane < n) p[lane] = v0 * inv_n;
  if (lane + 64 < n) p[lane + 64] = v1 * inv_n;
}

}  // namespace mom

namespace mom {
static mom_status project(const mom_dims* dims, const void* x, const int32_t* perm, const int32_t* seg_off,
                          const void* w_q, const void* w_k, const void* w_v, void* q, void* k, void* v, int part,
                          void* stream) {
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  if (part < 0 || part > 2) return MOM_ERR_DIMS;
  MOM_CHECK_PTR(x);
  if (part != 1) {  // the queries and the shared memory's rows read neither
    MOM_CHECK_PTR(perm);
    MOM_CHECK_PTR(seg_off);
  }
  MOM_CHECK_PTR(w_q);
  MOM_CHECK_PTR(w_k);
  MOM_CHECK_PTR(w_v);
  MOM_CHECK_PTR(q);
  MOM_CHECK_PTR(k);
  MOM_CHECK_PTR(v);
  const mom_dims& d = *dims;
  const Sizes z = sizes_of(d);
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == MOM_DTYPE_BF16) {
    if ((d.H * d.dk) % 128 || (d.H * d.dv) % 128) return MOM_ERR_UNSUPPORTED;
    mom_status r;
    if ((d.H * d.dk) % 256 == 0 && (d.H * d.dv) % 256 == 0 && z.NT >= 4096)
      r = launch_project_bf16<ProjCfg<4, 2, 4, 64, 2>, ProjCfg<4, 2, 1, 64, 2>>(d, z, x, perm, seg_off, w_q, w_k,
                                                                               w_v, q, k, v, part, st);
    else
      r = launch_project_bf16<ProjCfg<2, 2, 1, 64, 2>, ProjCfg<2, 2, 1, 64, 2>>(d, z, x, perm, seg_off, w_q, w_k,
                                                                               w_v, q, k, v, part, st);
    if (r != MOM_OK) return r;
  } else {
    const int64_t G = n_tiles_bound(d, PF_M, PF_N, part);
    hipLaunchKernelGGL(k_project_f32, dim3((unsigned)G), dim3(256), 0, st, z.NT, z.NR, part, d.D, d.H, d.dk, d.dv,
                       d.M, d.B, (const float*)x, perm, seg_off, (const float*)w_q, (const float*)w_k,
                       (const float*)w_v, (float*)q, (float*)k, (float*)v);
    // keys of the part's rows: routed rows [0, NR), shared rows [NR, N)
    const int64_t r0 = part == 1 ? z.NR : 0, r1 = part == 2 ? z.NR : z.N;
    const int64_t rows = (r1 - r0) * d.H;
    hipLaunchKernelGGL(k_l2norm_rows_f32, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, rows, d.dk,
                       (float*)k + r0 * d.H * d.dk);
  }
  return launch_status();
}
}  // namespace mom

extern "C" mom_status mom_project(const mom_dims* dims, const void* x, const int32_t* perm, const int32_t* seg_off,
                                  const void* w_q, const void* w_k, const void* w_v, void* q, void* k, void* v,
                                  void* stream) {
  return mom::project(dims, x, perm, seg_off, w_q, w_k, w_v, q, k, v, 0, stream);
}

extern "C" mom_status mom_project_part(const mom_dims* dims, const void* x, const int32_t* perm,
                                       const int32_t* seg_off, const void* w_q, const void* w_k, const void* w_v,
                                       void* q, void* k, void* v, int32_t part, void* stream) {
  return mom::project(dims, x, perm, seg_off, w_q, w_k, w_v, q, k, v, part, stream);
}
