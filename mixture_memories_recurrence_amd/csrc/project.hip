// Projections of the MoM layer: the shared query projection over every token
// and, per memory, its own key/value projections over the rows routed to it
// (research.elamur.ai summary, "Summary": each memory has its own key/value
// projections).  Keys are L2-normalised per head.
//
// bfloat16 path: one grouped "TN" GEMM on the matrix cores
// (v_mfma_f32_16x16x32_bf16), both operands K-contiguous:
//   C[r][c] = sum_d A[r][d] * W[c][d],  A rows gathered through perm.
// Logical tiles: first the query tiles (rows = tokens), then for every memory
// m = 0..M the tiles of its packed rows, whose columns run over [W_k[m]; W_v[m]].
// A tile is 128 x 128 with K-steps of 64, staged through LDS with a register
// double buffer; four waves each own a 64 x 64 quadrant (4 x 4 MFMA tiles).
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
  int64_t row0;    // first row of the group (packed row for k/v, token for q)
  int64_t rows;    // rows in the group
  int64_t trow;    // first row of this tile inside the group
  int col0;        // first output column inside the k or v matrix
};

template <int BM, int BN>
__device__ TileJob decode_tile(int64_t L, int64_t NT, int M, int B, int HK, int HV,
                               const int32_t* __restrict__ seg_off) {
  TileJob j;
  j.kind = -1;
  const int qcols = HK / BN;
  const int64_t qtiles = (int64_t)((NT + BM - 1) / BM) * qcols;
  if (L < qtiles) {
    j.kind = 0;
    j.m = 0;
    j.row0 = 0;
    j.rows = NT;
    j.trow = (L / qcols) * BM;
    j.col0 = (int)(L % qcols) * BN;
    return j;
  }
  L -= qtiles;
  const int kvcols = (HK + HV) / BN;
  for (int m = 0; m <= M; ++m) {
    const int64_t r0 = seg_off[m * B];
    const int64_t r1 = seg_off[(m + 1) * B];
    const int64_t nt = ((r1 - r0 + BM - 1) / BM) * kvcols;
    if (L < nt) {
      const int ct = (int)(L % kvcols);
      j.m = m;
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


inline int64_t n_tiles_bound(const mom_dims& d, int BM, int BN) {
  const Sizes s = sizes_of(d);
  const int64_t qt = ((s.NT + BM - 1) / BM) * (d.H * d.dk / BN);
  const int64_t kvt = ((s.N + BM - 1) / BM + d.M + 1) * ((d.H * d.dk + d.H * d.dv) / BN);
  return qt + kvt;
}

// ------------------------------------------------------------------ bf16 MFMA GEMM
constexpr int PB_M = 128, PB_N = 128, PB_K = 64, PB_LD = PB_K + 8;  // LDS row stride (bf16)
constexpr int PB_CLD = PB_N + 8;                                    // LDS stride of the C tile (half)

__global__ __launch_bounds__(256, 2) void k_project_bf16(int64_t NT, int D, int H, int dk, int dv, int M, int B,
                                                         const bf16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ seg_off,
                                                         const bf16_t* __restrict__ wq, const bf16_t* __restrict__ wk,
                                                         const bf16_t* __restrict__ wv, f16_t* __restrict__ q,
                                                         f16_t* __restrict__ k, f16_t* __restrict__ v) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * 2 * PB_M * PB_LD];
  bf16_t* As = smem;                      // [2][128][72]
  bf16_t* Bs = smem + 2 * PB_M * PB_LD;   // [2][128][72]
  __shared__ float red[2][PB_M];

  const int HK = H * dk, HV = H * dv;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const TileJob job = decode_tile<PB_M, PB_N>(L, NT, M, B, HK, HV, seg_off);
  if (job.kind < 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wv_id = tid >> 6;
  const int wm = wv_id >> 1, wn = wv_id & 1;

  // weight rows of this tile: W[col][d]
  const bf16_t* W;
  if (job.kind == 0) W = wq + (int64_t)job.col0 * D;
  else if (job.kind == 1) W = wk + ((int64_t)job.m * HK + job.col0) * D;
  else W = wv + ((int64_t)job.m * HV + job.col0) * D;

  // per-thread source rows for the 4 A chunks and 4 B chunks it loads
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;
  const bf16_t* a_src[4];
  const bf16_t* b_src[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = lrow + 32 * p;
    int64_t gr = job.trow + r;
    if (gr >= job.rows) gr = job.rows - 1;  // rows past the end reuse the last row; never stored
    const int64_t tok = (job.kind == 0) ? gr : (int64_t)perm[job.row0 + gr];
    a_src[p] = x + tok * D + lcol;
    b_src[p] = W + (int64_t)r * D + lcol;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      ra[p] = *reinterpret_cast<const uint4*>(a_src[p] + k0);
      rb[p] = *reinterpret_cast<const uint4*>(b_src[p] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      *reinterpret_cast<uint4*>(As + (buf * PB_M + lrow + 32 * p) * PB_LD + lcol) = ra[p];
      *reinterpret_cast<uint4*>(Bs + (buf * PB_M + lrow + 32 * p) * PB_LD + lcol) = rb[p];
    }
  };

  const int nk = D / PB_K;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * PB_K);
#pragma unroll
    for (int ks = 0; ks < PB_K / 32; ++ks) {
      bfv8 af[4], bfr[4];
      const int kof = ks * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bfv8*>(As + (cur * PB_M + wm * 64 + 16 * i + (lane & 15)) * PB_LD + kof);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bfv8*>(Bs + (cur * PB_M + wn * 64 + 16 * j + (lane & 15)) * PB_LD + kof);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: key rows normalised per head
  if (job.kind == 1) {
    float ss[4][4];  // [i][r] partial sum of squares over this lane's 4 columns
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) s = fmaf(acc[i][j][r], acc[i][j][r], s);
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        s += __shfl_xor(s, 8, 64);
        ss[i][r] = s;  // sum over this wave's 64 columns
      }
    if (dk == 128) {
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[wn][wm * 64 + 16 * i + 4 * (lane >> 4) + r] = ss[i][r];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = wm * 64 + 16 * i + 4 * (lane >> 4) + r;
          ss[i][r] = red[0][rr] + red[1][rr];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float inv_n = 1.0f / sqrtf(ss[i][r]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j][r] *= inv_n;
      }
  }
  // ---- stage the half tile in LDS (the operand buffers are free now)
  f16_t* Cs = reinterpret_cast<f16_t*>(smem);  // [128][136]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(wm * 64 + 16 * i + 4 * (lane >> 4) + r) * PB_CLD + wn * 64 + 16 * j + (lane & 15)] = (f16_t)acc[i][j][r];
  __syncthreads();
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
  const int64_t nrows = job.rows - job.trow < PB_M ? job.rows - job.trow : PB_M;
#pragma unroll
  for (int p = 0; p < (PB_M * PB_N / 8) / 256; ++p) {
    const int c = tid + 256 * p;
    const int r = c >> 4, c8 = (c & 15) * 8;
    if (r < nrows)
      *reinterpret_cast<uint4*>(out + (orow0 + r) * ld + job.col0 + c8) =
          *reinterpret_cast<const uint4*>(Cs + r * PB_CLD + c8);
  }
}

// ------------------------------------------------------------------ bf16 MFMA GEMM, large tiles
// 256 x 256 tiles, 8 waves (wave tile 128 x 64 = 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16), K-steps of
// 32 through a 4-stage LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at base + 16 l), so the
// gathered rows never pass through registers.  Each 64-byte row of a stage
// holds 4 16-byte chunks; chunk c of row r sits at position c ^ ((r >> 2) & 3),
// which keeps the 16-row fragment reads of one MFMA operand conflict-free.
constexpr int PL_M = 256, PL_N = 256, PL_K = 32, PL_NS = 4;
constexpr int PL_STAGE = (PL_M + PL_N) * PL_K;  // bf16 elements per stage
constexpr int PL_THREADS = 512;

__device__ __forceinline__ void lds_dma16(const void* g, bf16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(PL_THREADS) void k_project_bf16_l(int64_t NT, int D, int H, int dk, int dv, int M,
                                                              int B, const bf16_t* __restrict__ x,
                                                              const int32_t* __restrict__ perm,
                                                              const int32_t* __restrict__ seg_off,
                                                              const bf16_t* __restrict__ wq,
                                                              const bf16_t* __restrict__ wk,
                                                              const bf16_t* __restrict__ wv, f16_t* __restrict__ q,
                                                              f16_t* __restrict__ k, f16_t* __restrict__ v) {
  extern __shared__ __attribute__((aligned(16))) bf16_t smem_l[];
  const int HK = H * dk, HV = H * dv;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const TileJob job = decode_tile<PL_M, PL_N>(L, NT, M, B, HK, HV, seg_off);
  if (job.kind < 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;

  const bf16_t* W;
  if (job.kind == 0) W = wq + (int64_t)job.col0 * D;
  else if (job.kind == 1) W = wk + ((int64_t)job.m * HK + job.col0) * D;
  else W = wv + ((int64_t)job.m * HV + job.col0) * D;

  // loads: wave w, instruction j in {0,1} covers stage rows 32w + 16j + lane/4,
  // LDS position lane%4 holding global chunk (lane%4) ^ ((row >> 2) & 3)
  const bf16_t* a_src[2];
  const bf16_t* b_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * w + 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    int64_t gr = job.trow + r;
    if (gr >= job.rows) gr = job.rows - 1;  // rows past the end reuse the last row; never stored
    const int64_t tok = (job.kind == 0) ? gr : (int64_t)perm[job.row0 + gr];
    a_src[j] = x + tok * D + 8 * c;
    b_src[j] = W + (int64_t)r * D + 8 * c;
  }
  auto issue = [&](int kt) {
    bf16_t* st = smem_l + (kt % PL_NS) * PL_STAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lds_dma16(a_src[j] + kt * PL_K, st + (32 * w + 16 * j) * PL_K);
      lds_dma16(b_src[j] + kt * PL_K, st + PL_M * PL_K + (32 * w + 16 * j) * PL_K);
    }
  };

  // acc[jf][it]: v_mfma_f32_32x32x16_bf16 tiles, weights as the A operand:
  // element e holds feature 64 wn + 32 jf + 8 (e / 4) + 4 g + (e % 4) of token
  // 128 wm + 32 it + l32 (g = lane / 32, l32 = lane % 32)
  f32x16 acc[2][4];
#pragma unroll
  for (int jf = 0; jf < 2; ++jf)
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[jf][it][e] = 0.f;
  const int l32 = lane & 31, g = lane >> 5;

  const int nk = D / PL_K;
#pragma unroll
  for (int s = 0; s < PL_NS - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // tile kt has landed once at most the loads of the later issued tiles are outstanding
    const int later = min(PL_NS - 2, nk - 1 - kt);
    if (later >= 2) wait_vm<8>();
    else if (later == 1) wait_vm<4>();
    else wait_vm<0>();
    lds_sync();
    if (kt + PL_NS - 1 < nk) issue(kt + PL_NS - 1);
    const bf16_t* As = smem_l + (kt % PL_NS) * PL_STAGE;
    const bf16_t* Bs = As + PL_M * PL_K;
#pragma unroll
    for (int kb = 0; kb < PL_K / 16; ++kb) {
      const int ch = 2 * kb + g;  // 16-byte piece of the 64-byte row
      bfv8 wf[2], xf[4];
#pragma unroll
      for (int jf = 0; jf < 2; ++jf) {
        const int r = 64 * wn + 32 * jf + l32;
        wf[jf] = *reinterpret_cast<const bfv8*>(Bs + r * PL_K + 8 * (ch ^ ((r >> 2) & 3)));
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = 128 * wm + 32 * it + l32;
        xf[it] = *reinterpret_cast<const bfv8*>(As + r * PL_K + 8 * (ch ^ ((r >> 2) & 3)));
      }
#pragma unroll
      for (int jf = 0; jf < 2; ++jf)
#pragma unroll
        for (int it = 0; it < 4; ++it)
          acc[jf][it] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[jf], xf[it], acc[jf][it], 0, 0, 0);
    }
  }
  lds_sync();  // every wave done with the ring: LDS is free for the epilogue

  // ---- key rows normalised per head (head = dk features)
  if (job.kind == 1) {
    float* red = reinterpret_cast<float*>(smem_l);  // [4 wn][256 tokens]
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float s = 0.f;
#pragma unroll
      for (int jf = 0; jf < 2; ++jf)
#pragma unroll
        for (int e = 0; e < 16; ++e) s = fmaf(acc[jf][it][e], acc[jf][it][e], s);
      s += __shfl_xor(s, 32, 64);  // sum over this wave's 64 features
      if (g == 0) red[wn * 256 + 128 * wm + 32 * it + l32] = s;
    }
    lds_sync();
    const int per_head = dk / 64;  // waves per head
    const int w0 = (wn / per_head) * per_head;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int tt = 128 * wm + 32 * it + l32;
      float s = 0.f;
      for (int u = 0; u < per_head; ++u) s += red[(w0 + u) * 256 + tt];
      const float inv_n = 1.0f / sqrtf(s);
#pragma unroll
      for (int jf = 0; jf < 2; ++jf)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[jf][it][e] *= inv_n;
    }
    lds_sync();
  }
  // ---- output through LDS, 128 tokens (one wm half) at a time, 16-byte stores
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
  const int64_t nrows = job.rows - job.trow < PL_M ? job.rows - job.trow : PL_M;
  constexpr int CLD = PL_N + 8;
  f16_t* Cs = reinterpret_cast<f16_t*>(smem_l);  // [128 tokens][264]
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int jf = 0; jf < 2; ++jf)
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const half4 hv = {(f16_t)acc[jf][it][4 * qq], (f16_t)acc[jf][it][4 * qq + 1],
                              (f16_t)acc[jf][it][4 * qq + 2], (f16_t)acc[jf][it][4 * qq + 3]};
            *reinterpret_cast<half4*>(Cs + (32 * it + l32) * CLD + 64 * wn + 32 * jf + 8 * qq + 4 * g) = hv;
          }
    }
    lds_sync();
#pragma unroll
    for (int p = 0; p < (128 * PL_N / 8) / PL_THREADS; ++p) {
      const int c = tid + PL_THREADS * p;
      const int r = c >> 5, c8 = (c & 31) * 8;
      const int64_t row = 128 * half + r;
      if (row < nrows)
        *reinterpret_cast<uint4*>(out + (orow0 + row) * ld + job.col0 + c8) =
            *reinterpret_cast<const uint4*>(Cs + r * CLD + c8);
    }
    lds_sync();
  }
}

// ------------------------------------------------------------------ fp32 VALU GEMM
constexpr int PF_M = 64, PF_N = 64, PF_K = 16;

__global__ __launch_bounds__(256) void k_project_f32(int64_t NT, int D, int H, int dk, int dv, int M, int B,
                                                     const float* __restrict__ x, const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ seg_off, const float* __restrict__ wq,
                                                     const float* __restrict__ wk, const float* __restrict__ wv,
                                                     float* __restrict__ q, float* __restrict__ k, float* __restrict__ v) {
  __shared__ float As[PF_K][PF_M + 4];
  __shared__ float Bs[PF_K][PF_N + 4];
  const int HK = H * dk, HV = H * dv;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const TileJob job = decode_tile<PF_M, PF_N>(L, NT, M, B, HK, HV, seg_off);
  if (job.kind < 0) return;
  const float* W;
  if (job.kind == 0) W = wq + (int64_t)job.col0 * D;
  else if (job.kind == 1) W = wk + ((int64_t)job.m * HK + job.col0) * D;
  else W = wv + ((int64_t)job.m * HV + job.col0) * D;
  const int tid = threadIdx.x;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  int64_t gr = job.trow + lr;
  if (gr >= job.rows) gr = job.rows - 1;
  const int64_t tok = (job.kind == 0) ? gr : (int64_t)perm[job.row0 + gr];
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

extern "C" mom_status mom_project(const mom_dims* dims, const void* x, const int32_t* perm, const int32_t* seg_off,
                                  const void* w_q, const void* w_k, const void* w_v, void* q, void* k, void* v,
                                  void* stream) {
  using namespace mom;
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  MOM_CHECK_PTR(x);
  MOM_CHECK_PTR(perm);
  MOM_CHECK_PTR(seg_off);
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
    if ((d.H * d.dk) % PB_N || (d.H * d.dv) % PB_N) return MOM_ERR_UNSUPPORTED;
    if ((d.H * d.dk) % PL_N == 0 && (d.H * d.dv) % PL_N == 0 && z.NT >= 4096) {
      const int64_t G = n_tiles_bound(d, PL_M, PL_N);
      const size_t lds = (size_t)PL_NS * PL_STAGE * sizeof(bf16_t);
      static bool attr_set = false;  // idempotent; benign if two threads race
      if (!attr_set) {
        if (hipFuncSetAttribute((const void*)k_project_bf16_l, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
          return MOM_ERR_LAUNCH;
        attr_set = true;
      }
      hipLaunchKernelGGL(k_project_bf16_l, dim3((unsigned)G), dim3(PL_THREADS), lds, st, z.NT, d.D, d.H, d.dk, d.dv,
                         d.M, d.B, (const bf16_t*)x, perm, seg_off, (const bf16_t*)w_q, (const bf16_t*)w_k,
                         (const bf16_t*)w_v, (f16_t*)q, (f16_t*)k, (f16_t*)v);
      return launch_status();
    }
    const int64_t G = n_tiles_bound(d, PB_M, PB_N);
    hipLaunchKernelGGL(k_project_bf16, dim3((unsigned)G), dim3(256), 0, st, z.NT, d.D, d.H, d.dk, d.dv, d.M, d.B,
                       (const bf16_t*)x, perm, seg_off, (const bf16_t*)w_q, (const bf16_t*)w_k, (const bf16_t*)w_v,
                       (f16_t*)q, (f16_t*)k, (f16_t*)v);
  } else {
    const int64_t G = n_tiles_bound(d, PF_M, PF_N);
    hipLaunchKernelGGL(k_project_f32, dim3((unsigned)G), dim3(256), 0, st, z.NT, d.D, d.H, d.dk, d.dv, d.M, d.B,
                       (const float*)x, perm, seg_off, (const float*)w_q, (const float*)w_k, (const float*)w_v,
                       (float*)q, (float*)k, (float*)v);
    const int64_t rows = z.N * d.H;
    hipLaunchKernelGGL(k_l2norm_rows_f32, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, rows, d.dk, (float*)k);
  }
  return launch_status();
}
