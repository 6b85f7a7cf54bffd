// Dispatch of the MoM layer: the scatter/gather of routed tokens becomes a
// reordering of each memory's tokens into one contiguous segment per
// (memory, sequence) (podcast.do-not-panic.com page, "Solving scatter-gather
// without new kernels").
//
// A stable counting sort, all integer work, in tiles of 64 positions of one
// sequence (one wave each):
//   k_count   per-memory counts of each tile from wave ballots, written to
//             cnt[m][b][sub] (sub = position / 64; no atomics, every entry
//             written).  mom_route_count writes the same counts from the
//             router's pass, which saves this launch;
//   k_scan    one block: exclusive scan of cnt in (m, b, sub) order, which is
//             exactly the packed row order, into a second area of the
//             workspace (the counts stay as they are, so a counted dispatch
//             can run again on them); writes seg_off.  When cnt is small (at
//             most kFuseScan entries) every k_scatter block scans it in LDS
//             itself instead, which saves this launch;
//   k_scatter one block per tile again: a token's rank among the tile's tokens
//             routed to the same memory comes from wavefront ballots (popcount
//             of the lower lanes; with tiles of several waves, plus the totals
//             of the waves before it), so the order inside a segment is
//             increasing position.  The block then writes perm/inv, gathers
//             the gates of the routed memory and, if asked, the x rows.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace mom {

constexpr int kTile = kDispatchTile;
constexpr int kSub = kCountTile;
constexpr int kSubPerTile = kTile / kSub;
static_assert(kSub == kWave && kTile % kSub == 0, "one wave per count");
constexpr int kFuseScan = 1024;  // largest cnt scanned inside every k_scatter block

__global__ __launch_bounds__(kTile) void k_count(int B, int T, int M, int K, int nsub,
                                                 const int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
  const int tile = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, sub = tile * kSubPerTile + (threadIdx.x >> 6);
  if (sub >= nsub) return;  // whole wave
  const int t = sub * kSub + lane;
  const int64_t tok = (int64_t)b * T + t;
  int mem[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mem[j] = (t < T && j < K) ? idx[tok * K + j] : -1;
  for (int m = 0; m < M; ++m) {  // out-of-range entries are ignored
    bool f = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) f |= (mem[j] == m);
    const int n = __popcll(__ballot(f));
    if (lane == 0) cnt[((int64_t)m * B + b) * nsub + sub] = n;
  }
}

// Exclusive scan of n counts in place (single block of 1024 threads).
__global__ __launch_bounds__(1024) void k_scan(int B, int T, int M, int K, int nsub, int last_seg,
                                               const int32_t* __restrict__ cnt, int32_t* __restrict__ offs,
                                               int32_t* __restrict__ seg_off) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int n = M * B * nsub;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int32_t v = i < n ? cnt[i] : 0;
    // inclusive scan inside the wave
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
    if (i < n) offs[i] = pre + s - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry_s = pre + s;
    __syncthreads();
  }
  const int64_t NR = (int64_t)B * T * K;
  for (int s = threadIdx.x; s <= last_seg; s += 1024) {
    int64_t off;
    if (s < M * B) off = offs[(int64_t)s * nsub];
    else if (s < (M + 1) * B) off = NR + (int64_t)(s - M * B) * T;
    else off = NR + (int64_t)B * T;
    seg_off[s] = (int32_t)off;
  }
}

// Exclusive scan of cnt[0, n) into cs (LDS), n <= kFuseScan, by one block of
// kTile threads: contiguous runs per thread, then a scan of the run totals.
__device__ void block_exclusive_scan(const int32_t* __restrict__ cnt, int n, int32_t* cs, int32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + kTile - 1) / kTile;
  for (int i = tid; i < n; i += kTile) cs[i] = cnt[i];
  __syncthreads();
  const int i0 = tid * per, i1 = min(n, i0 + per);
  int32_t run = 0;
  for (int i = i0; i < i1; ++i) run += cs[i];
  int32_t sc = run;  // inclusive scan of the run totals inside the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t u = __shfl_up(sc, o, 64);
    if (lane >= o) sc += u;
  }
  if (lane == 63) wsum[wv] = sc;
  __syncthreads();
  int32_t pre = sc - run;
  for (int w2 = 0; w2 < wv; ++w2) pre += wsum[w2];
  for (int i = i0; i < i1; ++i) {
    const int32_t c = cs[i];
    cs[i] = pre;
    pre += c;
  }
  __syncthreads();
}

// base: the counts cnt[m][b][sub] (scanned in LDS when FUSED), else their
// exclusive scan; the tile's rows of memory m start at the scan's entry of its
// first 64 positions.
template <typename XT, bool FUSED>
__global__ __launch_bounds__(kTile) void k_scatter(int B, int T, int D, int H, int M, int K, int nsub, int last_seg,
                                                   bool shared_rows,
                                                   const int32_t* __restrict__ idx, const int32_t* __restrict__ base,
                                                   int32_t* __restrict__ seg_off,
                                                   const float* __restrict__ alpha, const float* __restrict__ beta,
                                                   int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                   float* __restrict__ alpha_p, float* __restrict__ beta_p,
                                                   const XT* __restrict__ x, XT* __restrict__ x_packed) {
  __shared__ int32_t wave_tot[64][kTile / kWave];
  __shared__ int32_t rows_s[kTile * 8];
  __shared__ int32_t cs[FUSED ? kFuseScan : 1];
  __shared__ int32_t wsum[kTile / kWave];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int64_t NR = (int64_t)B * T * K;
  if (FUSED) {
    block_exclusive_scan(base, M * B * nsub, cs, wsum);
    if (tile == 0 && b == 0)
      for (int sg = threadIdx.x; sg <= last_seg; sg += kTile) {
        int64_t off;
        if (sg < M * B) off = cs[(int64_t)sg * nsub];
        else if (sg < (M + 1) * B) off = NR + (int64_t)(sg - M * B) * T;
        else off = NR + (int64_t)B * T;
        seg_off[sg] = (int32_t)off;
      }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = tile * kTile + threadIdx.x;
  const bool valid = t < T;
  const int64_t tok = (int64_t)b * T + (valid ? t : 0);
  int mem[8], rank[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mem[j] = (valid && j < K) ? idx[tok * K + j] : -1;
    if ((unsigned)mem[j] >= (unsigned)M) mem[j] = -1;
    rank[j] = 0;
  }
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int m = 0; m < M; ++m) {
    bool f = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) f |= (mem[j] == m);
    const uint64_t bal = __ballot(f);
    const int pre = __popcll(bal & lower);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (mem[j] == m) rank[j] = pre;
    if (lane == 0) wave_tot[m][wv] = __popcll(bal);
  }
  __syncthreads();
  if (valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K && mem[j] >= 0) {
        const int m = mem[j];
        int r = rank[j];
        for (int w2 = 0; w2 < wv; ++w2) r += wave_tot[m][w2];
        const int64_t bi = ((int64_t)m * B + b) * nsub + (int64_t)tile * kSubPerTile;
        const int32_t row = (FUSED ? cs[bi] : base[bi]) + r;
        perm[row] = (int32_t)tok;
        inv[tok * K + j] = row;
        rows_s[threadIdx.x * 8 + j] = row;
        for (int h = 0; h < H; ++h) {
          const int64_t src = (tok * H + h) * (M + 1) + m;
          alpha_p[(int64_t)row * H + h] = alpha[src];
          beta_p[(int64_t)row * H + h] = beta[src];
        }
      }
    }
    if (shared_rows) {
      const int64_t srow = NR + tok;
      perm[srow] = (int32_t)tok;
      for (int h = 0; h < H; ++h) {
        const int64_t src = (tok * H + h) * (M + 1) + M;
        alpha_p[srow * H + h] = alpha[src];
        beta_p[srow * H + h] = beta[src];
      }
    }
  }
  if (x_packed == nullptr) return;
  __syncthreads();
  // gather x rows: one wave per (token, j), 16-byte lanes
  const int n_valid = min(kTile, T - tile * kTile);
  constexpr int kEl = 16 / (int)sizeof(XT);
  for (int e = wv; e < n_valid * K; e += kTile / kWave) {
    const int tt = e / K, j = e % K;
    const int64_t src_tok = (int64_t)b * T + tile * kTile + tt;
    const int32_t row = rows_s[tt * 8 + j];
    const uint4* s = reinterpret_cast<const uint4*>(x + src_tok * D);
    uint4* d = reinterpret_cast<uint4*>(x_packed + (int64_t)row * D);
    for (int c = lane; c < D / kEl; c += kWave) d[c] = s[c];
  }
}

// The shared memory's rows alone (they need no routing): row NR + t holds
// token t, its gates are alpha/beta[t][h][M]; the shared segments start at
// NR + b T.  One thread per (token, head).
__global__ __launch_bounds__(256) void k_dispatch_shared(int B, int T, int H, int M, int K,
                                                         const float* __restrict__ alpha,
                                                         const float* __restrict__ beta, int32_t* __restrict__ seg_off,
                                                         int32_t* __restrict__ perm, float* __restrict__ alpha_p,
                                                         float* __restrict__ beta_p) {
  const int64_t NT = (int64_t)B * T, NR = NT * K;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i <= B) seg_off[(int64_t)M * B + i] = (int32_t)(NR + i * T);
  if (i >= NT * H) return;
  const int64_t t = i / H, h = i % H;
  const int64_t src = (t * H + h) * (M + 1) + M;
  alpha_p[(NR + t) * H + h] = alpha[src];
  beta_p[(NR + t) * H + h] = beta[src];
  if (h == 0) perm[NR + t] = (int32_t)t;
}

}  // namespace mom

namespace mom {
// The dispatch's counts alone (cnt[m][b][sub], every entry written), for
// mom_route_count on shapes its fused kernel does not take.
mom_status dispatch_count_only(const mom_dims* dims, const int32_t* idx, int32_t* cnt, hipStream_t st) {
  const mom_dims& d = *dims;
  const int ntile = ceil_div(d.T, kTile), nsub = ceil_div(d.T, kSub);
  hipLaunchKernelGGL(k_count, dim3(ntile, d.B), dim3(kTile), 0, st, d.B, d.T, d.M, d.topk, nsub, idx, cnt);
  return launch_status();
}

// Argument checks of the dispatch entry points other than the workspace
// (part as in mom_dispatch_part).
static mom_status dispatch_check(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                                 const float* beta, const int32_t* seg_off, const int32_t* perm, const int32_t* inv,
                                 const void* x_packed, const float* alpha_p, const float* beta_p, int part) {
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  if (part < 0 || part > 2) return MOM_ERR_DIMS;
  MOM_CHECK_PTR(alpha);
  MOM_CHECK_PTR(beta);
  MOM_CHECK_PTR(seg_off);
  MOM_CHECK_PTR(perm);
  MOM_CHECK_PTR(alpha_p);
  MOM_CHECK_PTR(beta_p);
  if (part == 1) return MOM_OK;
  MOM_CHECK_PTR(idx);
  MOM_CHECK_PTR(inv);
  MOM_CHECK_OPT_PTR(x_packed);
  if (x_packed) MOM_CHECK_PTR(x);
  if ((int64_t)ceil_div(dims->T, kSub) * dims->B * dims->M > 0x7fffffff / 2) return MOM_ERR_DIMS;
  return MOM_OK;
}

// counted: ws already holds the counts (mom_route_count, one position per sequence)
static mom_status dispatch(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                           const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv, void* x_packed,
                           float* alpha_p, float* beta_p, void* ws, size_t ws_bytes, int part, void* stream,
                           bool counted = false) {
  const mom_status s = dispatch_check(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, part);
  if (s != MOM_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const mom_dims& d = *dims;
  if (part == 1) {  // the shared memory's rows: no routing needed
    const int64_t n = std::max((int64_t)d.B * d.T * d.H, (int64_t)d.B + 1);  // rows x heads, and B + 1 offsets
    hipLaunchKernelGGL(k_dispatch_shared, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, d.B, d.T, d.H, d.M,
                       d.topk, alpha, beta, seg_off, perm, alpha_p, beta_p);
    return launch_status();
  }
  const size_t need = mom_workspace_bytes(dims, MOM_WS_DISPATCH);
  if (!ws || ws_bytes < need) return MOM_ERR_WORKSPACE;
  MOM_CHECK_PTR(ws);
  const int ntile = ceil_div(d.T, kTile), nsub = ceil_div(d.T, kSub);
  // part 2 leaves the shared rows and the shared segments' offsets (past M B) to part 1
  const int last_seg = part == 2 ? d.M * d.B : (d.M + 1) * d.B;
  const bool shared_rows = part == 0;
  // counts, then (when not scanned inside the scatter) their exclusive scan
  int32_t* cnt = (int32_t*)ws;
  int32_t* offs = cnt + dispatch_offs_at(d);
  if (!counted)
    hipLaunchKernelGGL(k_count, dim3(ntile, d.B), dim3(kTile), 0, st, d.B, d.T, d.M, d.topk, nsub, idx, cnt);
  const bool fused = (int64_t)d.M * d.B * nsub <= kFuseScan;
  if (!fused)
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, d.B, d.T, d.M, d.topk, nsub, last_seg, cnt, offs,
                       seg_off);
#define MOM_SCATTER(XT, F)                                                                                         \
  hipLaunchKernelGGL((k_scatter<XT, F>), dim3(ntile, d.B), dim3(kTile), 0, st, d.B, d.T, d.D, d.H, d.M, d.topk,    \
                     nsub, last_seg, shared_rows, idx, F ? cnt : offs, seg_off, alpha, beta, perm, inv, alpha_p,  \
                     beta_p, (const XT*)x, (XT*)x_packed)
  if (d.dtype == MOM_DTYPE_BF16) {
    if (fused) MOM_SCATTER(bf16_t, true);
    else MOM_SCATTER(bf16_t, false);
  } else {
    if (fused) MOM_SCATTER(float, true);
    else MOM_SCATTER(float, false);
  }
#undef MOM_SCATTER
  return launch_status();
}
}  // namespace mom

extern "C" mom_status mom_dispatch(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                                   const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                                   void* x_packed, float* alpha_p, float* beta_p, void* ws, size_t ws_bytes,
                                   void* stream) {
  return mom::dispatch(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws, ws_bytes, 0,
                       stream);
}

extern "C" mom_status mom_dispatch_counted(const mom_dims* dims, const int32_t* idx, const void* x,
                                           const float* alpha, const float* beta, int32_t* seg_off, int32_t* perm,
                                           int32_t* inv, void* x_packed, float* alpha_p, float* beta_p, void* ws,
                                           size_t ws_bytes, void* stream) {
  return mom::dispatch(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws, ws_bytes, 0,
                       stream, true);
}

extern "C" mom_status mom_dispatch_counted_part(const mom_dims* dims, const int32_t* idx, const void* x,
                                                const float* alpha, const float* beta, int32_t* seg_off,
                                                int32_t* perm, int32_t* inv, void* x_packed, float* alpha_p,
                                                float* beta_p, void* ws, size_t ws_bytes, int32_t part,
                                                void* stream) {
  return mom::dispatch(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws, ws_bytes, part,
                       stream, true);
}

extern "C" mom_status mom_dispatch_part(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                                        const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                                        void* x_packed, float* alpha_p, float* beta_p, void* ws, size_t ws_bytes,
                                        int32_t part, void* stream) {
  return mom::dispatch(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws, ws_bytes, part,
                       stream);
}

// ------------------------------------------------------------------ allocation-free dispatch
// mom_dispatch_noalloc keeps the dispatch's workspace (the counts, int32
// [M][B][ceil(T/64)], written in full by k_count before k_scan or k_scatter
// read them, and their scan, so nothing needs clearing) in this array instead of a caller workspace.  In host code
// `scratch` only names the symbol: its device address is looked up once per
// device with hipGetSymbolAddress and kept in scratch_ptr.
namespace mom {
constexpr int64_t kNoAllocCounts = 65536;  // 256 KiB
static __device__ __align__(256) int32_t scratch[kNoAllocCounts];
namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` on device i, null until looked up

// Address of `scratch` on the current device (the stream's device), or null
// with *st set.
void* scratch_address(hipStream_t stream, mom_status* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    *st = MOM_ERR_LAUNCH;
    return nullptr;
  }
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) {
      *st = MOM_ERR_DIMS;  // the stream belongs to another device than the current one
      return nullptr;
    }
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = MOM_ERR_UNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *st = MOM_ERR_LAUNCH;
      return nullptr;
    }
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
}  // namespace
}  // namespace mom

extern "C" mom_status mom_dispatch_noalloc(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                                           const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                                           void* x_packed, float* alpha_p, float* beta_p, void* stream) {
  using namespace mom;
  mom_status s = dispatch_check(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, 0);
  if (s != MOM_OK) return s;
  const size_t need = mom_workspace_bytes(dims, MOM_WS_DISPATCH);
  if (need > (size_t)kNoAllocCounts * sizeof(int32_t)) return MOM_ERR_TOO_LARGE;
  void* ws = scratch_address((hipStream_t)stream, &s);
  if (!ws) return s;
  return dispatch(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws,
                  (size_t)kNoAllocCounts * sizeof(int32_t), 0, stream);
}
