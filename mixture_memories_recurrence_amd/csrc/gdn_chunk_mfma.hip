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
// two launches:
//   k_gdn_prep   fully parallel over (chunk, head): g, A and P from two MFMA
//                products, then T by a blocked solve (16x16 diagonal blocks by
//                forward substitution, off-diagonal blocks by block products),
//                all in float32; T and P are stored as half, g as float32.
//   k_gdn_chain  one block per (segment, head, 64 value columns); value
//                columns of the state evolve independently.  It walks the
//                segment's chunks in order with the state in MFMA accumulators
//                (float32) and a half copy of S^T in LDS as the operand.
// Every product is v_mfma_f32_16x16x32_f16 with both operands staged in LDS
// with the contraction index contiguous.
#include "common.h"

namespace mom {

constexpr int GC = 64;     // chunk rows
constexpr int GDVB = 64;   // value columns per chain block
constexpr int GLD = 72;    // LDS row stride (halfs) of 64-wide tiles

__device__ __forceinline__ f32x4 mfma16(const half8& a, const half8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 lds8(const f16_t* p) { return *reinterpret_cast<const half8*>(p); }

// ------------------------------------------------------------------ chunk numbering
// chunk_base[s] = number of chunks in segments before s; chunk_base[n_seg] = total.
__global__ __launch_bounds__(1024) void k_chunk_base(int n_seg, const int32_t* __restrict__ seg_off,
                                                     int32_t* __restrict__ chunk_base) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n_seg; base += 1024) {
    const int i = base + threadIdx.x;
    const int32_t v = i < n_seg ? (seg_off[i + 1] - seg_off[i] + GC - 1) / GC : 0;
    int32_t s = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t u = __shfl_up(s, o, 64);
      if (lane >= o) s += u;
    }
    if (lane == 63) wsum[wv] = s;
    __syncthreads();
    int32_t pre = carry_s;
    for (int w2 = 0; w2 < wv; ++w2) pre += wsum[w2];
    if (i < n_seg) chunk_base[i] = pre + s - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry_s = pre + s;
    __syncthreads();
  }
  if (threadIdx.x == 0) chunk_base[n_seg] = carry_s;
}

// ------------------------------------------------------------------ prep
template <int DK>
__global__ __launch_bounds__(256) void k_gdn_prep(int H, int n_seg, const int32_t* __restrict__ seg_off,
                                                  const int32_t* __restrict__ chunk_base,
                                                  const int32_t* __restrict__ row_token, const f16_t* __restrict__ q,
                                                  const f16_t* __restrict__ k, const float* __restrict__ alpha_p,
                                                  const float* __restrict__ beta_p, f16_t* __restrict__ Tws,
                                                  f16_t* __restrict__ Pws, float* __restrict__ Gws,
                                                  f16_t* __restrict__ Qws) {
  constexpr int KLD = DK + 8;
  __shared__ __attribute__((aligned(16))) f16_t Ks[GC * KLD];
  __shared__ __attribute__((aligned(16))) f16_t Qs[GC * KLD];
  __shared__ float As[GC][GC + 1];
  __shared__ float Xs[GC][GC + 1];
  __shared__ float Ys[3][16][17];
  __shared__ float gs[GC], bs[GC];

  const int h = blockIdx.x % H;
  const int c = blockIdx.x / H;
  const int total = chunk_base[n_seg];
  if (c >= total) return;
  // segment of chunk c: the last s with chunk_base[s] <= c
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_base[mid] <= c) lo = mid;
    else hi = mid - 1;
  }
  const int s = lo;
  const int64_t r0 = seg_off[s] + (int64_t)(c - chunk_base[s]) * GC;
  const int L = (int)min((int64_t)GC, (int64_t)seg_off[s + 1] - r0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // K and Q rows of the chunk (zero past L)
  constexpr int CPR = DK / 8;  // 16-byte pieces per row
  for (int e = tid; e < GC * CPR; e += 256) {
    const int i = e / CPR, p = (e % CPR) * 8;
    uint4 kv = {0, 0, 0, 0}, qv = {0, 0, 0, 0};
    if (i < L) {
      const int64_t row = r0 + i;
      const int64_t tk = row_token ? (int64_t)row_token[row] : row;
      kv = *reinterpret_cast<const uint4*>(k + (row * H + h) * DK + p);
      qv = *reinterpret_cast<const uint4*>(q + (tk * H + h) * DK + p);
    }
    *reinterpret_cast<uint4*>(Ks + i * KLD + p) = kv;
    *reinterpret_cast<uint4*>(Qs + i * KLD + p) = qv;
  }
  if (w == 0) {
    float la = 0.f, bb = 0.f;
    if (lane < L) {
      la = logf(alpha_p[(r0 + lane) * H + h]);
      bb = beta_p[(r0 + lane) * H + h];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(la, o, 64);
      if (lane >= o) la += u;
    }
    gs[lane] = la;
    bs[lane] = bb;
  }
  __syncthreads();

  // wave w: row block w of K K^T and Q K^T (column blocks jb <= w)
  const int64_t ch = (int64_t)c * H + h;
  f16_t* Pout = Pws + ch * GC * GC;
  for (int jb = 0; jb < 4; ++jb) {
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
    if (jb <= w) {
#pragma unroll
      for (int d0 = 0; d0 < DK; d0 += 32) {
        const int off = d0 + 8 * (lane >> 4);
        const half8 ka = lds8(Ks + (16 * w + (lane & 15)) * KLD + off);
        const half8 qa = lds8(Qs + (16 * w + (lane & 15)) * KLD + off);
        const half8 kb = lds8(Ks + (16 * jb + (lane & 15)) * KLD + off);
        kk = mfma16(ka, kb, kk);
        qk = mfma16(qa, kb, qk);
      }
    }
    const int j = 16 * jb + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * w + 4 * (lane >> 4) + r;
      float a = 0.f, p = 0.f;
      if (j <= i) {
        const float dec = expf(gs[i] - gs[j]);
        if (j < i) a = bs[i] * dec * kk[r];
        p = dec * qk[r];
      }
      As[i][j] = a;
      Pout[i * GC + j] = (f16_t)p;
    }
  }
  __syncthreads();

  // X = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution, one lane
  // per (block, column)
  if (tid < 64) {
    const int bb = tid >> 4, cc = tid & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < r; ++t) v = fmaf(-As[16 * bb + r][16 * bb + t], x[t], v);
      x[r] = v;
      Xs[16 * bb + r][16 * bb + cc] = v;
    }
  }
  __syncthreads();
  // off-diagonal blocks, one block-diagonal at a time:
  //   X_ij = -X_ii * sum_{t=j}^{i-1} A_it X_tj
  for (int dist = 1; dist < 4; ++dist) {
    const int nblk = 4 - dist;
    const int r = tid >> 4, cc = tid & 15;
    for (int bI = 0; bI < nblk; ++bI) {
      const int ib = bI + dist, jb = bI;
      float acc = 0.f;
      for (int t = 16 * jb; t < 16 * ib; ++t) acc = fmaf(As[16 * ib + r][t], Xs[t][16 * jb + cc], acc);
      Ys[bI][r][cc] = acc;
    }
    __syncthreads();
    for (int bI = 0; bI < nblk; ++bI) {
      const int ib = bI + dist, jb = bI;
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) acc = fmaf(Xs[16 * ib + r][16 * ib + u], Ys[bI][u][cc], acc);
      Xs[16 * ib + r][16 * jb + cc] = -acc;
    }
    __syncthreads();
  }
  // T = X diag(beta), lower block triangle; zero above
  f16_t* Tout = Tws + ch * GC * GC;
  for (int e = tid; e < GC * GC; e += 256) {
    const int i = e / GC, j = e % GC;
    const bool lower = (j >> 4) < (i >> 4) || ((j >> 4) == (i >> 4) && j <= i);
    Tout[e] = (f16_t)(lower ? Xs[i][j] * bs[j] : 0.f);
  }
  if (tid < GC) Gws[ch * GC + tid] = gs[tid];
  // the chunk's (gathered, zero-padded) queries, contiguous for the chain kernel
  for (int e = tid; e < GC * CPR; e += 256) {
    const int i = e / CPR, p = (e % CPR) * 8;
    *reinterpret_cast<uint4*>(Qws + ch * GC * DK + i * DK + p) = *reinterpret_cast<const uint4*>(Qs + i * KLD + p);
  }
}

// ------------------------------------------------------------------ chain
// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not for
// its global loads, so prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wave-local LDS hand-off: rows written by this wave are read back by this wave.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint4 zero_if(bool z, uint4 v) {
  return z ? uint4{0u, 0u, 0u, 0u} : v;
}

constexpr int CHAIN_THREADS = 512;  // 8 waves: wave w owns row block w & 3 and column half w >> 2

template <int DK, bool GATHER>
__global__ __launch_bounds__(CHAIN_THREADS) void k_gdn_chain(
    int H, int dv, int n_seg, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_state,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ row_token, const f16_t* __restrict__ q,
    const f16_t* __restrict__ k, const f16_t* __restrict__ v, const f16_t* __restrict__ Tws,
    const f16_t* __restrict__ Pws, const float* __restrict__ Gws, const float* __restrict__ state_in,
    float* __restrict__ state_out, float* __restrict__ o) {
  constexpr int NT = CHAIN_THREADS;
  constexpr int KLD = DK + 8;
  constexpr int NDB = DK / 16;          // 16-row blocks of the state / 16-column blocks of W
  constexpr int SDB = NDB / 4;          // state row blocks per wave
  constexpr int WDB = NDB / 2;          // W column blocks per wave
  constexpr int QPR = DK / 8;           // 16-byte pieces per Q row
  constexpr int QIT = GC * QPR / NT;    // Q pieces per thread
  constexpr int ND = DK / 32;           // contraction steps over d
  __shared__ __attribute__((aligned(16))) f16_t KT[DK * GLD];     // K^T  [d][j]
  __shared__ __attribute__((aligned(16))) f16_t Qh[GC * KLD];     // Q    [i][d]
  __shared__ __attribute__((aligned(16))) f16_t VT[GDVB * GLD];   // V^T  [n][j]
  __shared__ __attribute__((aligned(16))) f16_t Th[GC * GLD];     // T    [i][j]
  __shared__ __attribute__((aligned(16))) f16_t Ph[GC * GLD];     // P    [i][j]
  __shared__ __attribute__((aligned(16))) f16_t ST[GDVB * KLD];   // S^T  [n][d]
  __shared__ __attribute__((aligned(16))) f16_t Wh[GC * KLD];     // W    [i][d]
  __shared__ __attribute__((aligned(16))) f16_t UT[GDVB * GLD];   // U^T  [n][j]
  __shared__ __attribute__((aligned(16))) f16_t UT2[GDVB * GLD];  // (diag(gamma_L/gamma) U)^T
  __shared__ __attribute__((aligned(16))) float eg[GC];           // gamma_i
  __shared__ float egl[GC];                                       // gamma_L / gamma_i

  // Work items are (segment, head) groups of nb column blocks.  Block p runs on
  // XCD p % 8.  The first 8*floor(groups/8) groups are dealt round-robin over
  // the XCDs, each group's nb blocks on one XCD one after another (they read
  // the same K, Q, T, P through that XCD's L2); the remaining groups follow in
  // plain order.  Groups are numbered from the last segment (the shared
  // memory's, the longest) backwards, so long chains start first everywhere.
  const int nb = dv / GDVB;
  const int64_t p = blockIdx.x;
  const int64_t n_grp = (int64_t)n_seg * H;
  const int64_t full = (n_grp / 8) * 8;
  int64_t grp;
  int cb;
  if (p < full * nb) {
    const int64_t xi = p & 7, ii = p >> 3;
    grp = (ii / nb) * 8 + xi;
    cb = (int)(ii % nb);
  } else {
    const int64_t r = p - full * nb;
    grp = full + r / nb;
    cb = (int)(r % nb);
  }
  const int h = (int)(grp % H);
  const int s = n_seg - 1 - (int)(grp / H);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rb = w & 3, chh = w >> 2;   // row block, column half
  const int l16 = lane & 15, lg = lane >> 4;
  const int ip = tid & 31, pg = tid >> 5;  // row pair and 8-column group of the transposed loads (pg < 16)
  const int slot = seg_state ? seg_state[s] : s;
  const int64_t sbase = ((int64_t)slot * H + h) * DK * dv + cb * GDVB;
  const int64_t rbeg = seg_off[s], rend = seg_off[s + 1];
  const int cbase = chunk_base[s];
  const int qi0 = tid / QPR, qp = (tid % QPR) * 8;  // Q piece: row qi0 + (NT/QPR)*it

  // ---- registers of the next chunk's inputs (loaded during the current chunk)
  constexpr int KPI = (DK / 8 + 15) / 16;  // K column groups per thread
  uint4 rk0[KPI], rk1[KPI], rq[QIT], rv0, rv1, rt, rp;
  int32_t rtok[QIT];
  float rg = 0.f;
  auto prefetch_a = [&](int64_t r0) {  // everything but the gathered queries
    const int L = (int)min((int64_t)GC, rend - r0);
    const int64_t chk = (int64_t)(cbase + (r0 - rbeg) / GC) * H + h;
    const int64_t ra = r0 + min(2 * ip, L - 1), rbr = r0 + min(2 * ip + 1, L - 1);
#pragma unroll
    for (int it = 0; it < KPI; ++it) {
      const int p = 8 * (pg + 16 * it);
      if (p < DK) {
        rk0[it] = *reinterpret_cast<const uint4*>(k + (ra * H + h) * DK + p);
        rk1[it] = *reinterpret_cast<const uint4*>(k + (rbr * H + h) * DK + p);
      }
    }
    if (pg < GDVB / 8) {
      rv0 = *reinterpret_cast<const uint4*>(v + (ra * H + h) * dv + cb * GDVB + 8 * pg);
      rv1 = *reinterpret_cast<const uint4*>(v + (rbr * H + h) * dv + cb * GDVB + 8 * pg);
    }
    rt = reinterpret_cast<const uint4*>(Tws + chk * GC * GC)[tid];
    rp = reinterpret_cast<const uint4*>(Pws + chk * GC * GC)[tid];
    rg = Gws[chk * GC + (tid & (GC - 1))];
  };
  // Row tokens run two chunks ahead of the gathered query loads, so a query
  // load never waits on the token load it depends on.
  auto load_tokens = [&](int64_t r0) {
    const int L = (int)min((int64_t)GC, rend - r0);
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int64_t row = r0 + min(qi0 + (NT / QPR) * it, L - 1);
      rtok[it] = GATHER ? row_token[row] : (int32_t)row;
    }
  };
  auto prefetch_b = [&]() {  // gathered queries of the chunk whose tokens are in rtok
#pragma unroll
    for (int it = 0; it < QIT; ++it)
      rq[it] = *reinterpret_cast<const uint4*>(q + ((int64_t)rtok[it] * H + h) * DK + qp);
  };
  auto stage = [&](int L) {
    const bool z0 = 2 * ip >= L, z1 = 2 * ip + 1 >= L;
#pragma unroll
    for (int it = 0; it < KPI; ++it) {
      const int p = 8 * (pg + 16 * it);
      if (p < DK) {
        const uint4 a4 = zero_if(z0, rk0[it]), b4 = zero_if(z1, rk1[it]);
        const f16_t* a = reinterpret_cast<const f16_t*>(&a4);
        const f16_t* b = reinterpret_cast<const f16_t*>(&b4);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          __attribute__((ext_vector_type(2))) _Float16 pr = {a[t], b[t]};
          *reinterpret_cast<decltype(pr)*>(KT + (p + t) * GLD + 2 * ip) = pr;
        }
      }
    }
    if (pg < GDVB / 8) {
      const uint4 a4 = zero_if(z0, rv0), b4 = zero_if(z1, rv1);
      const f16_t* a = reinterpret_cast<const f16_t*>(&a4);
      const f16_t* b = reinterpret_cast<const f16_t*>(&b4);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        __attribute__((ext_vector_type(2))) _Float16 pr = {a[t], b[t]};
        *reinterpret_cast<decltype(pr)*>(VT + (8 * pg + t) * GLD + 2 * ip) = pr;
      }
    }
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int i = qi0 + (NT / QPR) * it;
      *reinterpret_cast<uint4*>(Qh + i * KLD + qp) = zero_if(i >= L, rq[it]);
    }
    {
      const int i = tid >> 3, p = (tid & 7) * 8;
      *reinterpret_cast<uint4*>(Th + i * GLD + p) = rt;
      *reinterpret_cast<uint4*>(Ph + i * GLD + p) = rp;
    }
    if (tid < GC) {
      const float gl = __shfl(rg, GC - 1, 64);
      eg[tid] = expf(rg);
      egl[tid] = expf(gl - rg);
    }
  };

  // state accumulators: wave owns state rows [16*SDB*rb, +16*SDB) and column blocks 2*chh, 2*chh+1
  f32x4 S[SDB][2];
  if (state_in) {
#pragma unroll
    for (int a = 0; a < SDB; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 16 * (SDB * rb + a) + 4 * lg + r;
          S[a][c][r] = state_in[sbase + (int64_t)d * dv + 16 * (2 * chh + c) + l16];
        }
  } else {
#pragma unroll
    for (int a = 0; a < SDB; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) S[a][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  auto write_st = [&]() {
#pragma unroll
    for (int a = 0; a < SDB; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int d = 16 * (SDB * rb + a) + 4 * lg;
        half4 hv = {(f16_t)S[a][c][0], (f16_t)S[a][c][1], (f16_t)S[a][c][2], (f16_t)S[a][c][3]};
        *reinterpret_cast<half4*>(ST + (16 * (2 * chh + c) + l16) * KLD + d) = hv;
      }
  };
  write_st();
  if (rbeg < rend) {
    prefetch_a(rbeg);
    load_tokens(rbeg);
    prefetch_b();
    load_tokens(min(rbeg + GC, rend - 1));
  }
  // The loads for the next chunk are issued unconditionally (the last chunk
  // reloads itself), so they land straight in the registers staged next.

  const int arow = 16 * rb + l16;
  for (int64_t r0 = rbeg; r0 < rend; r0 += GC) {
    const int L = (int)min((int64_t)GC, rend - r0);
    const bool more = r0 + GC < rend;
    lds_barrier();  // previous chunk done with every LDS tile; ST written
    stage(L);
    lds_barrier();
    prefetch_a(more ? r0 + GC : r0);  // in flight during this chunk's products
    prefetch_b();                      // queries of chunk r0 + GC (tokens loaded a chunk ago)
    load_tokens(r0 + 2 * GC < rend ? r0 + 2 * GC : r0);

    // ---- W = T diag(gamma) K: row block rb, column blocks [WDB*chh, WDB*(chh+1))
    {
      half8 ta[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const half8 t8 = lds8(Th + arow * GLD + 32 * x + 8 * lg);
        const float4 g0 = *reinterpret_cast<const float4*>(eg + 32 * x + 8 * lg);
        const float4 g1 = *reinterpret_cast<const float4*>(eg + 32 * x + 8 * lg + 4);
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) ta[x][t] = (f16_t)((float)t8[t] * gg[t]);
      }
      half8 kb[WDB][2];
#pragma unroll
      for (int y = 0; y < WDB; ++y) {
        const int db = WDB * chh + y;
        kb[y][0] = lds8(KT + (16 * db + l16) * GLD + 8 * lg);
        kb[y][1] = lds8(KT + (16 * db + l16) * GLD + 32 + 8 * lg);
      }
      f32x4 acc[WDB];
#pragma unroll
      for (int y = 0; y < WDB; ++y) acc[y] = mfma16(ta[0], kb[y][0], (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int y = 0; y < WDB; ++y) acc[y] = mfma16(ta[1], kb[y][1], acc[y]);
#pragma unroll
      for (int y = 0; y < WDB; ++y)
#pragma unroll
        for (int r = 0; r < 4; ++r) Wh[(16 * rb + 4 * lg + r) * KLD + 16 * (WDB * chh + y) + l16] = (f16_t)acc[y][r];
    }
    lds_barrier();  // W rows come from two waves
    // ---- U~ = T V, Q S and W S (sharing the S^T operand), then U and U^T
    f32x4 O[2];
    {
      half8 qa[ND], wa[ND];
#pragma unroll
      for (int d0 = 0; d0 < ND; ++d0) {
        qa[d0] = lds8(Qh + arow * KLD + 32 * d0 + 8 * lg);
        wa[d0] = lds8(Wh + arow * KLD + 32 * d0 + 8 * lg);
      }
      const half8 t0 = lds8(Th + arow * GLD + 8 * lg), t1 = lds8(Th + arow * GLD + 32 + 8 * lg);
      half8 sb[2][ND], vb[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int nbk = 2 * chh + c;
#pragma unroll
        for (int d0 = 0; d0 < ND; ++d0) sb[c][d0] = lds8(ST + (16 * nbk + l16) * KLD + 32 * d0 + 8 * lg);
        vb[c][0] = lds8(VT + (16 * nbk + l16) * GLD + 8 * lg);
        vb[c][1] = lds8(VT + (16 * nbk + l16) * GLD + 32 + 8 * lg);
      }
      float gi[4], gli[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gi[r] = eg[16 * rb + 4 * lg + r];
        gli[r] = egl[16 * rb + 4 * lg + r];
      }
      f32x4 ut[2], qs[2], ws[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        ut[c] = mfma16(t0, vb[c][0], (f32x4){0.f, 0.f, 0.f, 0.f});
        qs[c] = mfma16(qa[0], sb[c][0], (f32x4){0.f, 0.f, 0.f, 0.f});
        ws[c] = mfma16(wa[0], sb[c][0], (f32x4){0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int d0 = 1; d0 < ND; ++d0)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          qs[c] = mfma16(qa[d0], sb[c][d0], qs[c]);
          ws[c] = mfma16(wa[d0], sb[c][d0], ws[c]);
        }
#pragma unroll
      for (int c = 0; c < 2; ++c) ut[c] = mfma16(t1, vb[c][1], ut[c]);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int nbk = 2 * chh + c;
        half4 u1, u2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float u = ut[c][r] - ws[c][r];
          O[c][r] = qs[c][r] * gi[r];
          u1[r] = (f16_t)u;
          u2[r] = (f16_t)(u * gli[r]);
        }
        *reinterpret_cast<half4*>(UT + (16 * nbk + l16) * GLD + 16 * rb + 4 * lg) = u1;
        *reinterpret_cast<half4*>(UT2 + (16 * nbk + l16) * GLD + 16 * rb + 4 * lg) = u2;
      }
    }
    lds_barrier();
    // ---- O += P U (store), S <- gamma_L S + K^T U'
    {
      const half8 p0 = lds8(Ph + arow * GLD + 8 * lg), p1 = lds8(Ph + arow * GLD + 32 + 8 * lg);
      half8 ub[2][2], u2b[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int nbk = 2 * chh + c;
        ub[c][0] = lds8(UT + (16 * nbk + l16) * GLD + 8 * lg);
        ub[c][1] = lds8(UT + (16 * nbk + l16) * GLD + 32 + 8 * lg);
        u2b[c][0] = lds8(UT2 + (16 * nbk + l16) * GLD + 8 * lg);
        u2b[c][1] = lds8(UT2 + (16 * nbk + l16) * GLD + 32 + 8 * lg);
      }
      half8 ka[SDB][2];
#pragma unroll
      for (int a = 0; a < SDB; ++a) {
        const int drow = 16 * (SDB * rb + a) + l16;
        ka[a][0] = lds8(KT + drow * GLD + 8 * lg);
        ka[a][1] = lds8(KT + drow * GLD + 32 + 8 * lg);
      }
      const float eL = eg[GC - 1];
#pragma unroll
      for (int c = 0; c < 2; ++c) O[c] = mfma16(p0, ub[c][0], O[c]);
#pragma unroll
      for (int a = 0; a < SDB; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int r = 0; r < 4; ++r) S[a][c][r] *= eL;
          S[a][c] = mfma16(ka[a][0], u2b[c][0], S[a][c]);
        }
#pragma unroll
      for (int c = 0; c < 2; ++c) O[c] = mfma16(p1, ub[c][1], O[c]);
#pragma unroll
      for (int a = 0; a < SDB; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) S[a][c] = mfma16(ka[a][1], u2b[c][1], S[a][c]);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * rb + 4 * lg + r;
          if (i < L) o[((r0 + i) * H + h) * dv + cb * GDVB + 16 * (2 * chh + c) + l16] = O[c][r];
        }
    }
    write_st();  // ST is no longer read in this chunk
  }
#pragma unroll
  for (int a = 0; a < SDB; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * (SDB * rb + a) + 4 * lg + r;
        state_out[sbase + (int64_t)d * dv + 16 * (2 * chh + c) + l16] = S[a][c][r];
      }
}

// ------------------------------------------------------------------ chain, column-owner form
// One block per (segment, head, DVB value columns), DVB/32 waves; wave w owns
// value columns [32w, 32w+32) of the block for every key row, so its part of
// the state lives in float32 accumulators of v_mfma_f32_32x32x16_f16 and never
// leaves the wave.  Accumulator rows of a 32x32 tile (8q + 4g + t for lane
// group g = lane / 32) become the 16-deep B operand of the next product after a
// v_permlane32_swap between lanes l and l+32, so S and U feed W S, Q S, P U and
// K~^T U' straight from registers.  Per chunk, the inputs are staged in LDS
// (K and V transposed) and W = T diag(gamma) K is formed once per block; the
// rest runs per wave without block barriers.
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f16x16 __attribute__((ext_vector_type(16)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x16 mfma32(const h8v& a, const h8v& b, const f16x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ unsigned pack_h2(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (unsigned)__builtin_bit_cast(unsigned short, x) | ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}
// Rows [16p, 16p+16) of a 32x32 accumulator tile as the B operand (k = row) of
// a 32x32x16 product; rows are scaled by sc[0..7] = the scales of rows 8q+4g+t
// for q = 2p, 2p+1 (t = 0..3), or by 1.
__device__ __forceinline__ h8v acc_to_b(const f16x16& d, int p, const float* sc) {
  const unsigned X0 = pack_h2(d[8 * p + 0] * sc[0], d[8 * p + 1] * sc[1]);
  const unsigned X1 = pack_h2(d[8 * p + 2] * sc[2], d[8 * p + 3] * sc[3]);
  const unsigned Y0 = pack_h2(d[8 * p + 4] * sc[4], d[8 * p + 5] * sc[5]);
  const unsigned Y1 = pack_h2(d[8 * p + 6] * sc[6], d[8 * p + 7] * sc[7]);
  const u2v s0 = __builtin_amdgcn_permlane32_swap(X0, Y0, false, false);
  const u2v s1 = __builtin_amdgcn_permlane32_swap(X1, Y1, false, false);
  const unsigned w4[4] = {s0.x, s1.x, s0.y, s1.y};
  return __builtin_bit_cast(h8v, *reinterpret_cast<const __attribute__((ext_vector_type(4))) unsigned*>(w4));
}

__device__ __forceinline__ void chunk_dma16(const void* g, f16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void chunk_wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing LDS read (ds_read_b64_tr_b16): inside each 16-lane group, lane i
// receives element i % 4 of the 8-byte values addressed by lanes i / 4,
// 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group.  Pointing lane j of a group
// at X[k0 + j / 4][n0 + 4 (j % 4)] hands lane i the column n0 + i of rows
// k0 .. k0 + 3, so a k-major MFMA operand comes straight from a row-major tile.
typedef short s4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s4v lds_tr4(const f16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)p);
}
// 32x32x16 operand fragment (k = 16 kb .. 16 kb + 15, 32 rows/columns from c0)
// out of a row-major LDS tile X[k][c] with row stride RS halfs.
template <int RS>
__device__ __forceinline__ h8v kmajor_frag(const f16_t* X, int kb, int c0, int lane) {
  const int row = 16 * kb + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const s4v a = lds_tr4(X + row * RS + col);
  const s4v b = lds_tr4(X + (row + 4) * RS + col);
  const s4v v8[2] = {a, b};
  return __builtin_bit_cast(h8v, v8);
}

template <int DK, int DVB>
__global__ __launch_bounds__(DVB * 2) void k_gdn_chain3(
    int H, int dv, int n_seg, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_state,
    const int32_t* __restrict__ chunk_base, const f16_t* __restrict__ k, const f16_t* __restrict__ v,
    const f16_t* __restrict__ Tws, const f16_t* __restrict__ Pws, const float* __restrict__ Gws,
    const f16_t* __restrict__ Qws, const float* __restrict__ state_in, float* __restrict__ state_out,
    float* __restrict__ o) {
  constexpr int NW = DVB / 32;          // waves
  constexpr int NT = 64 * NW;           // threads
  constexpr int RS = DK + 32;           // K row stride: 4 consecutive rows land on distinct banks
  constexpr int VRS = DVB + 32;         // V row stride
  constexpr int KLD = DK + 8;
  constexpr int ND = DK / 32;           // 32-row tiles of the state
  constexpr int NKD = DK / 16;          // 16-deep k blocks over d
  constexpr int WT = 2 * ND / NW;       // W^T tiles per wave
  constexpr int KC = GC * (DK / 8) / NT;
  constexpr int VC = GC * (DVB / 8) / NT;
  constexpr int TC = GC * (GC / 8) / NT;
  __shared__ __attribute__((aligned(16))) f16_t Ks[GC * RS];      // K    [j][d]
  __shared__ __attribute__((aligned(16))) f16_t Vs[GC * VRS];     // V    [j][n]
  __shared__ __attribute__((aligned(16))) f16_t Th[GC * GLD];     // T    [i][j]
  __shared__ __attribute__((aligned(16))) f16_t Ph[GC * GLD];     // P    [i][j]
  __shared__ __attribute__((aligned(16))) f16_t Qh[GC * KLD];     // Q    [i][d]
  __shared__ __attribute__((aligned(16))) f16_t Wh[GC * KLD];     // W    [i][d]
  __shared__ __attribute__((aligned(16))) float eg[GC];           // gamma_i
  __shared__ __attribute__((aligned(16))) float egl[GC];          // gamma_L / gamma_i

  // (segment, head) groups dealt round-robin over the 8 XCDs, longest first
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
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, g2 = lane >> 5;
  const int slot = seg_state ? seg_state[s] : s;
  const int ncol0 = cb * DVB + 32 * w;      // first value column of this wave
  const int64_t sbase = ((int64_t)slot * H + h) * DK * dv + ncol0;
  const int64_t rbeg = seg_off[s], rend = seg_off[s + 1];
  const int cbase = chunk_base[s];

  // ---- next-chunk registers: coalesced 16-byte pieces (row = e / (width / 8))
  uint4 rk[KC], rv[VC], rq[KC], rt[TC], rp[TC];
  float rg = 0.f;
  auto prefetch = [&](int64_t r0) {
    const int L = (int)min((int64_t)GC, rend - r0);
    const int64_t chk = (int64_t)(cbase + (r0 - rbeg) / GC) * H + h;
#pragma unroll
    for (int it = 0; it < KC; ++it) {
      const int e = tid + NT * it, i = e / (DK / 8), p = (e % (DK / 8)) * 8;
      const int64_t row = r0 + min(i, L - 1);
      rk[it] = *reinterpret_cast<const uint4*>(k + (row * H + h) * DK + p);
      rq[it] = *reinterpret_cast<const uint4*>(Qws + chk * GC * DK + i * DK + p);
    }
#pragma unroll
    for (int it = 0; it < VC; ++it) {
      const int e = tid + NT * it, i = e / (DVB / 8), p = (e % (DVB / 8)) * 8;
      const int64_t row = r0 + min(i, L - 1);
      rv[it] = *reinterpret_cast<const uint4*>(v + (row * H + h) * dv + cb * DVB + p);
    }
#pragma unroll
    for (int it = 0; it < TC; ++it) {
      rt[it] = reinterpret_cast<const uint4*>(Tws + chk * GC * GC)[tid + NT * it];
      rp[it] = reinterpret_cast<const uint4*>(Pws + chk * GC * GC)[tid + NT * it];
    }
    rg = Gws[chk * GC + (tid & (GC - 1))];
  };
  auto stage = [&](int L) {
#pragma unroll
    for (int it = 0; it < KC; ++it) {
      const int e = tid + NT * it, i = e / (DK / 8), p = (e % (DK / 8)) * 8;
      *reinterpret_cast<uint4*>(Ks + i * RS + p) = zero_if(i >= L, rk[it]);
      *reinterpret_cast<uint4*>(Qh + i * KLD + p) = rq[it];
    }
#pragma unroll
    for (int it = 0; it < VC; ++it) {
      const int e = tid + NT * it, i = e / (DVB / 8), p = (e % (DVB / 8)) * 8;
      *reinterpret_cast<uint4*>(Vs + i * VRS + p) = zero_if(i >= L, rv[it]);
    }
#pragma unroll
    for (int it = 0; it < TC; ++it) {
      const int e = tid + NT * it, i = e >> 3, p = (e & 7) * 8;
      *reinterpret_cast<uint4*>(Th + i * GLD + p) = rt[it];
      *reinterpret_cast<uint4*>(Ph + i * GLD + p) = rp[it];
    }
    if (tid < GC) {
      const float gl = __shfl(rg, GC - 1, 64);
      eg[tid] = expf(rg);
      egl[tid] = expf(gl - rg);
    }
  };

  // ---- state: ND tiles of 32 key rows x the wave's 32 value columns
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
  if (rbeg < rend) prefetch(rbeg);
  const float ones[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

  for (int64_t r0 = rbeg; r0 < rend; r0 += GC) {
    const int L = (int)min((int64_t)GC, rend - r0);
    lds_barrier();  // the previous chunk is done with every LDS tile
    stage(L);
    lds_barrier();
    prefetch(r0 + GC < rend ? r0 + GC : r0);  // lands during this chunk's products

    // ---- W^T tiles of this wave: D[d][i] = sum_j K^T[d][j] (T diag(gamma))^T[j][i] -> Wh[i][d]
#pragma unroll
    for (int x = 0; x < WT; ++x) {
      const int tix = w * WT + x;
      const int a = tix % ND, bt = tix / ND;  // d tile, i tile
      f16x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb) {
        const h8v ka = kmajor_frag<RS>(Ks, kb, 32 * a, lane);
        h8v tb = *reinterpret_cast<const h8v*>(Th + (32 * bt + c32) * GLD + 16 * kb + 8 * g2);
        const float4 e0 = *reinterpret_cast<const float4*>(eg + 16 * kb + 8 * g2);
        const float4 e1 = *reinterpret_cast<const float4*>(eg + 16 * kb + 8 * g2 + 4);
        const float es[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) tb[t] = (f16_t)((float)tb[t] * es[t]);
        acc = mfma32(ka, tb, acc);
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const half4 hv = {(f16_t)acc[4 * qq], (f16_t)acc[4 * qq + 1], (f16_t)acc[4 * qq + 2], (f16_t)acc[4 * qq + 3]};
        *reinterpret_cast<half4*>(Wh + (32 * bt + c32) * KLD + 32 * a + 8 * qq + 4 * g2) = hv;
      }
    }
    lds_barrier();  // W complete

    // ---- state as an operand (k = key rows): B of W S, A of S^T Q^T
    h8v sb[NKD];
#pragma unroll
    for (int a = 0; a < ND; ++a) {
      sb[2 * a] = acc_to_b(S[a], 0, ones);
      sb[2 * a + 1] = acc_to_b(S[a], 1, ones);
    }
    // ---- U = T V - W S for the two 32-row tiles
    f16x16 U[2];
    {
      h8v vb[GC / 16];
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb) vb[kb] = kmajor_frag<VRS>(Vs, kb, 32 * w, lane);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        f16x16 ut, ws;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          ut[i] = 0.f;
          ws[i] = 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < GC / 16; ++kb)
          ut = mfma32(*reinterpret_cast<const h8v*>(Th + (32 * bt + c32) * GLD + 16 * kb + 8 * g2), vb[kb], ut);
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb)
          ws = mfma32(*reinterpret_cast<const h8v*>(Wh + (32 * bt + c32) * KLD + 16 * kb + 8 * g2), sb[kb], ws);
#pragma unroll
        for (int i = 0; i < 16; ++i) U[bt][i] = ut[i] - ws[i];
      }
    }
    // ---- U and diag(gamma_L / gamma) U as operands (k = chunk rows)
    h8v ub[GC / 16], u2b[GC / 16];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float sc[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sc[t] = egl[32 * bt + 16 * p + 4 * g2 + t];
          sc[4 + t] = egl[32 * bt + 16 * p + 8 + 4 * g2 + t];
        }
        ub[2 * bt + p] = acc_to_b(U[bt], p, ones);
        u2b[2 * bt + p] = acc_to_b(U[bt], p, sc);
      }
    // ---- O^T = diag... : O^T[n][i] = gamma_i (S^T Q^T)[n][i] + (U^T P^T)[n][i]; float4 stores
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) {
      f16x16 ot;
#pragma unroll
      for (int i = 0; i < 16; ++i) ot[i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
        ot = mfma32(sb[kb], *reinterpret_cast<const h8v*>(Qh + (32 * bt + c32) * KLD + 16 * kb + 8 * g2), ot);
      const float gi = eg[32 * bt + c32];
#pragma unroll
      for (int i = 0; i < 16; ++i) ot[i] *= gi;
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
        ot = mfma32(ub[kb], *reinterpret_cast<const h8v*>(Ph + (32 * bt + c32) * GLD + 16 * kb + 8 * g2), ot);
      const int ri = 32 * bt + c32;
      if (ri < L) {
        float* orow = o + ((r0 + ri) * H + h) * dv + ncol0 + 4 * g2;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *reinterpret_cast<float4*>(orow + 8 * qq) = make_float4(ot[4 * qq], ot[4 * qq + 1], ot[4 * qq + 2], ot[4 * qq + 3]);
      }
    }
    // ---- S <- gamma_L S + K^T U'
    const float eL = eg[GC - 1];
#pragma unroll
    for (int a = 0; a < ND; ++a) {
#pragma unroll
      for (int i = 0; i < 16; ++i) S[a][i] *= eL;
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb) S[a] = mfma32(kmajor_frag<RS>(Ks, kb, 32 * a, lane), u2b[kb], S[a]);
    }
  }
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * a + 8 * (i / 4) + 4 * g2 + (i % 4);
      state_out[sbase + (int64_t)d * dv + c32] = S[a][i];
    }
}

// ------------------------------------------------------------------ chain, double-buffered (dk = 128, 128 columns)
// Same products as k_gdn_chain3, but every chunk input (K, V, Q, T, P) is
// prefetched straight from global memory into the idle half of a double
// buffer with global_load_lds_dwordx4 (lane l's 16 bytes land at base + 16 l),
// so no registers hold in-flight data.  Rows are unpadded; the 16-byte chunk
// c of row r is stored at position c ^ sw(r):
//   K, V (256-byte rows, read transposed 4 rows x 64 bytes): sw = 4 (r & 3)
//   Q    (256-byte rows, read 16 rows x 16 bytes):            sw = r & 15
//   T, P (128-byte rows, read 16 rows x 16 bytes):            sw = (r >> 1) & 7
// Rows past the segment end are loaded from its last row; T has zero rows and
// columns there and the prepared queries are zero, so they contribute nothing.
__device__ __forceinline__ int swz_kv(int r, int c) { return c ^ (4 * (r & 3)); }
__device__ __forceinline__ int swz_q(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_tp(int r, int c) { return c ^ ((r >> 1) & 7); }

// 32x32x16 operand (k = 16 kb ..) from a swizzled 256-byte-row tile read transposed.
__device__ __forceinline__ h8v kmajor_frag_sw(const f16_t* X, int kb, int c0, int lane) {
  const int row = 16 * kb + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // halfs
  const int ch = col >> 3, sub = col & 7;
  const s4v a = lds_tr4(X + row * 128 + 8 * swz_kv(row, ch) + sub);
  const s4v b = lds_tr4(X + (row + 4) * 128 + 8 * swz_kv(row + 4, ch) + sub);
  const s4v v8[2] = {a, b};
  return __builtin_bit_cast(h8v, v8);
}

__global__ __launch_bounds__(256) void k_gdn_chain4(
    int H, int dv, int n_seg, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_state,
    const int32_t* __restrict__ chunk_base, const f16_t* __restrict__ k, const f16_t* __restrict__ v,
    const f16_t* __restrict__ Tws, const f16_t* __restrict__ Pws, const float* __restrict__ Gws,
    const f16_t* __restrict__ Qws, const float* __restrict__ state_in, float* __restrict__ state_out,
    float* __restrict__ o) {
  constexpr int DK = 128, DVB = 128;
  constexpr int KLD = DK + 8;
  constexpr int ND = DK / 32, NKD = DK / 16, WT = 2;
  constexpr int BUF = GC * 128 * 3 + GC * 64 * 2;  // halfs per buffer: K, V, Q + T, P
  extern __shared__ __attribute__((aligned(16))) f16_t smem4[];
  f16_t* Wh = smem4 + 2 * BUF;                                        // W [i][d], padded
  float* egb = reinterpret_cast<float*>(Wh + GC * KLD);                // [2][2][64]: gamma, gamma_L/gamma

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
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, g2 = lane >> 5;
  const int slot = seg_state ? seg_state[s] : s;
  const int ncol0 = cb * DVB + 32 * w;
  const int64_t sbase = ((int64_t)slot * H + h) * DK * dv + ncol0;
  const int64_t rbeg = seg_off[s], rend = seg_off[s + 1];
  const int cbase = chunk_base[s];

  float rg = 0.f;  // log-decay prefix of the next chunk (thread tid < 64)
  auto prefetch = [&](int64_t r0, int buf) {
    const int L = (int)min((int64_t)GC, rend - r0);
    const int64_t chk = (int64_t)(cbase + (r0 - rbeg) / GC) * H + h;
    f16_t* B = smem4 + buf * BUF;
    // K, V, Q: 64 rows x 16 chunks; wave w, instruction it covers rows 4 (w + 4 it) .. +3
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rbase = 4 * (w + 4 * it);
      const int r = rbase + (lane >> 4), pos = lane & 15;
      const int64_t row = r0 + min(r, L - 1);
      chunk_dma16(k + (row * H + h) * DK + 8 * swz_kv(r, pos), B + rbase * 128);
      chunk_dma16(v + (row * H + h) * dv + cb * DVB + 8 * swz_kv(r, pos), B + GC * 128 + rbase * 128);
      chunk_dma16(Qws + chk * GC * DK + r * DK + 8 * swz_q(r, pos), B + 2 * GC * 128 + rbase * 128);
    }
    // T, P: 64 rows x 8 chunks; instruction it covers rows 8 (w + 4 it) .. +7
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int rbase = 8 * (w + 4 * it);
      const int r = rbase + (lane >> 3), pos = lane & 7;
      chunk_dma16(Tws + chk * GC * GC + r * GC + 8 * swz_tp(r, pos), B + 3 * GC * 128 + rbase * 64);
      chunk_dma16(Pws + chk * GC * GC + r * GC + 8 * swz_tp(r, pos), B + 3 * GC * 128 + GC * 64 + rbase * 64);
    }
    rg = Gws[chk * GC + (tid & (GC - 1))];
  };

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
  if (rbeg < rend) prefetch(rbeg, 0);

  int buf = 0;
  for (int64_t r0 = rbeg; r0 < rend; r0 += GC, buf ^= 1) {
    const int L = (int)min((int64_t)GC, rend - r0);
    chunk_wait_vm0();                   // this chunk's inputs (and the last chunk's stores) are done
    float* eg = egb + buf * 128;    // gamma_i
    float* egl = eg + 64;           // gamma_L / gamma_i
    if (tid < GC) {
      const float gl = __shfl(rg, GC - 1, 64);
      eg[tid] = expf(rg);
      egl[tid] = expf(gl - rg);
    }
    lds_barrier();                     // inputs visible; every wave is done with the other buffer
    prefetch(r0 + GC < rend ? r0 + GC : r0, buf ^ 1);
    const f16_t* Ks = smem4 + buf * BUF;
    const f16_t* Vs = Ks + GC * 128;
    const f16_t* Qs = Ks + 2 * GC * 128;
    const f16_t* Ts = Ks + 3 * GC * 128;
    const f16_t* Ps = Ts + GC * 64;
    auto tfrag = [&](const f16_t* X, int row, int kb) {  // 16-byte operand piece of a T/P row
      return *reinterpret_cast<const h8v*>(X + row * 64 + 8 * swz_tp(row, 2 * kb + g2));
    };
    auto qfrag = [&](int row, int kb) {
      return *reinterpret_cast<const h8v*>(Qs + row * 128 + 8 * swz_q(row, 2 * kb + g2));
    };

    // ---- W^T tiles: wave w computes (d tile w, i tiles 0 and 1) -> Wh[i][d]
    {
      f16x16 acc[WT];
#pragma unroll
      for (int x = 0; x < WT; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[x][i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb) {
        const h8v ka = kmajor_frag_sw(Ks, kb, 32 * w, lane);
        const float4 e0 = *reinterpret_cast<const float4*>(eg + 16 * kb + 8 * g2);
        const float4 e1 = *reinterpret_cast<const float4*>(eg + 16 * kb + 8 * g2 + 4);
        const float es[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int x = 0; x < WT; ++x) {
          h8v tb = tfrag(Ts, 32 * x + c32, kb);
#pragma unroll
          for (int t = 0; t < 8; ++t) tb[t] = (f16_t)((float)tb[t] * es[t]);
          acc[x] = mfma32(ka, tb, acc[x]);
        }
      }
#pragma unroll
      for (int x = 0; x < WT; ++x)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const half4 hv = {(f16_t)acc[x][4 * qq], (f16_t)acc[x][4 * qq + 1], (f16_t)acc[x][4 * qq + 2],
                            (f16_t)acc[x][4 * qq + 3]};
          *reinterpret_cast<half4*>(Wh + (32 * x + c32) * KLD + 32 * w + 8 * qq + 4 * g2) = hv;
        }
    }
    lds_barrier();  // W complete

    // ---- state as an operand (k = key rows)
    h8v sb[NKD];
#pragma unroll
    for (int a = 0; a < ND; ++a) {
      sb[2 * a] = acc_to_b(S[a], 0, ones);
      sb[2 * a + 1] = acc_to_b(S[a], 1, ones);
    }
    // ---- U = T V - W S, both 32-row tiles interleaved
    f16x16 U[2];
    {
      f16x16 ut[2], ws[2];
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          ut[bt][i] = 0.f;
          ws[bt][i] = 0.f;
        }
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb) {
        const h8v vb = kmajor_frag_sw(Vs, kb, 32 * w, lane);
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) ut[bt] = mfma32(tfrag(Ts, 32 * bt + c32, kb), vb, ut[bt]);
      }
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
          ws[bt] = mfma32(*reinterpret_cast<const h8v*>(Wh + (32 * bt + c32) * KLD + 16 * kb + 8 * g2), sb[kb], ws[bt]);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int i = 0; i < 16; ++i) U[bt][i] = ut[bt][i] - ws[bt][i];
    }
    // ---- U and diag(gamma_L / gamma) U as operands (k = chunk rows)
    h8v ub[GC / 16], u2b[GC / 16];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float sc[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sc[t] = egl[32 * bt + 16 * p + 4 * g2 + t];
          sc[4 + t] = egl[32 * bt + 16 * p + 8 + 4 * g2 + t];
        }
        ub[2 * bt + p] = acc_to_b(U[bt], p, ones);
        u2b[2 * bt + p] = acc_to_b(U[bt], p, sc);
      }
    // ---- O^T[n][i] = gamma_i (S^T Q^T)[n][i] + (U^T P^T)[n][i], both i tiles interleaved
    {
      f16x16 ot[2];
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int i = 0; i < 16; ++i) ot[bt][i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) ot[bt] = mfma32(sb[kb], qfrag(32 * bt + c32, kb), ot[bt]);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        const float gi = eg[32 * bt + c32];
#pragma unroll
        for (int i = 0; i < 16; ++i) ot[bt][i] *= gi;
      }
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) ot[bt] = mfma32(ub[kb], tfrag(Ps, 32 * bt + c32, kb), ot[bt]);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        const int ri = 32 * bt + c32;
        if (ri < L) {
          float* orow = o + ((r0 + ri) * H + h) * dv + ncol0 + 4 * g2;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            *reinterpret_cast<float4*>(orow + 8 * qq) =
                make_float4(ot[bt][4 * qq], ot[bt][4 * qq + 1], ot[bt][4 * qq + 2], ot[bt][4 * qq + 3]);
        }
      }
    }
    // ---- S <- gamma_L S + K^T U', the four state tiles interleaved
    {
      const float eL = eg[GC - 1];
#pragma unroll
      for (int a = 0; a < ND; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[a][i] *= eL;
#pragma unroll
      for (int kb = 0; kb < GC / 16; ++kb)
#pragma unroll
        for (int a = 0; a < ND; ++a) S[a] = mfma32(kmajor_frag_sw(Ks, kb, 32 * a, lane), u2b[kb], S[a]);
    }
  }
  chunk_wait_vm0();  // the dummy prefetch of the last chunk has landed before the block ends
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * a + 8 * (i / 4) + 4 * g2 + (i % 4);
      state_out[sbase + (int64_t)d * dv + c32] = S[a][i];
    }
}
constexpr size_t CHAIN4_LDS = (size_t)(2 * (GC * 128 * 3 + GC * 64 * 2) + GC * (128 + 8)) * 2 + 2 * 2 * 64 * 4;

// ------------------------------------------------------------------ workspace + launch
struct ChunkWs {
  int32_t* chunk_base;
  f16_t* T;
  f16_t* P;
  f16_t* Q;
  float* G;
  size_t bytes;
};

inline ChunkWs chunk_ws_layout(void* base, int64_t n_seg, int64_t n_rows, int H, int dk) {
  const int64_t nch = n_rows / GC + n_seg;  // bound on the number of chunks
  ChunkWs w;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += (b + 255) / 256 * 256;
    return o;
  };
  const size_t o_cb = take((size_t)(n_seg + 1) * 4);
  const size_t o_t = take((size_t)nch * H * GC * GC * 2);
  const size_t o_p = take((size_t)nch * H * GC * GC * 2);
  const size_t o_g = take((size_t)nch * H * GC * 4);
  const size_t o_q = take((size_t)nch * H * GC * dk * 2);
  char* b = (char*)base;
  w.chunk_base = (int32_t*)(b + o_cb);
  w.T = (f16_t*)(b + o_t);
  w.P = (f16_t*)(b + o_p);
  w.G = (float*)(b + o_g);
  w.Q = (f16_t*)(b + o_q);
  w.bytes = off;
  return w;
}

size_t gdn_chunk_ws_bytes(int64_t n_seg, int64_t n_rows, int H, int dk) {
  return chunk_ws_layout(nullptr, n_seg, n_rows, H, dk).bytes;
}

mom_status launch_gdn_chunk_mfma(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                                 const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                                 const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                                 float* state_out, float* o, void* ws, hipStream_t st) {
  const ChunkWs W = chunk_ws_layout(ws, n_seg, n_rows, d.H, d.dk);
  const int64_t nch = (int64_t)n_rows / GC + n_seg;
  hipLaunchKernelGGL(k_chunk_base, dim3(1), dim3(1024), 0, st, n_seg, seg_off, W.chunk_base);
  const int64_t prep_blocks = nch * d.H;
  const int64_t chain_blocks = (int64_t)n_seg * d.H * (d.dv / GDVB);
#define MOM_MFMA_CASE(DK)                                                                                          \
  do {                                                                                                             \
    if (prep_blocks > 0)                                                                                           \
      hipLaunchKernelGGL((k_gdn_prep<DK>), dim3((unsigned)prep_blocks), dim3(256), 0, st, d.H, n_seg, seg_off,     \
                         W.chunk_base, row_token, (const f16_t*)q, (const f16_t*)k, alpha_p, beta_p, W.T, W.P, W.G,  \
                         W.Q);                                                                                     \
    if (DK == 128 && d.dv % 128 == 0) {                                                                           \
      static bool attr4 = false;                                                                                   \
      if (!attr4) {                                                                                                \
        if (hipFuncSetAttribute((const void*)k_gdn_chain4, hipFuncAttributeMaxDynamicSharedMemorySize,             \
                                (int)CHAIN4_LDS) != hipSuccess)                                                    \
          return MOM_ERR_LAUNCH;                                                                                   \
        attr4 = true;                                                                                              \
      }                                                                                                            \
      hipLaunchKernelGGL(k_gdn_chain4, dim3((unsigned)((int64_t)n_seg * d.H * (d.dv / 128))), dim3(256),          \
                         CHAIN4_LDS, st, d.H, d.dv, n_seg, seg_off, seg_state, W.chunk_base, (const f16_t*)k,      \
                         (const f16_t*)v, W.T, W.P, W.G, W.Q, state_in, state_out, o);                              \
    } else if (d.dv % 128 == 0)                                                                                    \
      hipLaunchKernelGGL((k_gdn_chain3<DK, 128>), dim3((unsigned)((int64_t)n_seg * d.H * (d.dv / 128))), dim3(256), \
                         0, st, d.H, d.dv, n_seg, seg_off, seg_state, W.chunk_base, (const f16_t*)k,               \
                         (const f16_t*)v, W.T, W.P, W.G, W.Q, state_in, state_out, o);                              \
    else                                                                                                           \
      hipLaunchKernelGGL((k_gdn_chain3<DK, 64>), dim3((unsigned)chain_blocks), dim3(128), 0, st, d.H, d.dv, n_seg,  \
                         seg_off, seg_state, W.chunk_base, (const f16_t*)k, (const f16_t*)v, W.T, W.P, W.G, W.Q,   \
                         state_in, state_out, o);                                                                  \
  } while (0)
  if (d.dk == 64) MOM_MFMA_CASE(64);
  else MOM_MFMA_CASE(128);
#undef MOM_MFMA_CASE
  return launch_status();
}

}  // namespace mom
