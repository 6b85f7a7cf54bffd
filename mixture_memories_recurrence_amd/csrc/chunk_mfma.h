// Device helpers shared by the chunkwise kernels on the gfx950 matrix cores
// (forward and gradients): chunk numbering over packed segments, LDS fences,
// the 32x32x16 half product and its accumulator-to-operand move, asynchronous
// global -> LDS copies, and the swizzled LDS tile reads.
#pragma once
#include <algorithm>

#include "common.h"

namespace mom {

constexpr int GC = 64;     // chunk rows


// ------------------------------------------------------------------ chunk numbering
// The chunks of segment s are numbered from the count of chunks (ceil(len / 64)
// each) in the segments before it.  Each wave that needs the numbering scans
// the segments' chunk counts itself, 64 segments per step, so no separate
// launch computes it.
__device__ __forceinline__ int seg_chunks(const int32_t* seg_off, int i) {
  return (seg_off[i + 1] - seg_off[i] + GC - 1) / GC;
}
// Chunks in segments [0, s); the same value in every lane.
__device__ __forceinline__ int chunks_before(const int32_t* __restrict__ seg_off, int s, int lane) {
  int sum = 0;
  for (int s0 = 0; s0 < s; s0 += 64) {
    int n = s0 + lane < s ? seg_chunks(seg_off, s0 + lane) : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o, 64);
    sum += n;
  }
  return sum;
}
// Segment holding chunk c and the number of its first chunk; false when c is
// at or past the last chunk.  The same result in every lane.
__device__ __forceinline__ bool locate_chunk(const int32_t* __restrict__ seg_off, int n_seg, int c, int lane,
                                             int& seg, int& base) {
  int before = 0;
  for (int s0 = 0; s0 < n_seg; s0 += 64) {
    const int n = s0 + lane < n_seg ? seg_chunks(seg_off, s0 + lane) : 0;
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    const int first = before + incl - n;  // number of this lane's segment's first chunk
    const uint64_t hit = __ballot(n > 0 && first <= c && c < first + n);
    if (hit) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      seg = s0 + l;
      base = __shfl(first, l, 64);
      return true;
    }
    before += __shfl(incl, 63, 64);
  }
  return false;
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Program order of one wave's LDS accesses to the same addresses, for the
// compiler only: a wave's LDS operations are performed in issue order, so a
// read after a write (or a write after a read) of the same location by the
// same wave needs no wait; the compiler still waits before a read's data is
// used.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void vm_wait_4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void vm_wait_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f16x16 __attribute__((ext_vector_type(16)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));
typedef short s4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x16 mfma32(const h8v& a, const h8v& b, const f16x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));
// Two floats to a half pair (round to nearest even; one v_cvt_pk_f16_f32).
__device__ __forceinline__ unsigned pack_h2(float a, float b) {
  const f2v v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, h2v));
}
// Rows [16p, 16p+16) of a 32x32 accumulator tile as the 16-deep operand (k =
// row) of a 32x32x16 product, row 8q+4g+t scaled by sc[4 (q - 2p) + t].
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

// ------------------------------------------------------------------ 16 x 16 x 32 products
// v_mfma_f32_16x16x32_f16: lane l = 16 G + c (G = l / 16) holds
//   A[row c][k 8G .. 8G+7],  B[k 8G .. 8G+7][col c],  D[rows 4G .. 4G+3][col c].
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f4v mfma16(const h8v& a, const h8v& b, const f4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Two accumulator tiles of one 32-row block (t0: rows 0..15, t1: rows 16..31,
// lane 16 G + c holding rows 4G .. 4G+3 of column c), row r scaled by s0[r % 4]
// (t0) or s1[r % 4] (t1), as the 32-deep operand of a 16x16x32 product: lane
// 16 G + c receives rows 8G .. 8G+7 of column c.  Lane group G needs the rows
// of groups 2(G % 2) and 2(G % 2) + 1 of tile G / 2: one exchange between the
// wave's halves (v_permlane32_swap) brings t1's groups 0, 1 next to t0's groups
// 2, 3, and one between neighbouring 16-lane rows (v_permlane16_swap) pairs
// each group with the one it needs.
__device__ __forceinline__ h8v acc16_to_op(const f4v& t0, const f4v& t1, const float* s0, const float* s1) {
  const unsigned X0 = pack_h2(t0[0] * s0[0], t0[1] * s0[1]), X1 = pack_h2(t0[2] * s0[2], t0[3] * s0[3]);
  const unsigned Y0 = pack_h2(t1[0] * s1[0], t1[1] * s1[1]), Y1 = pack_h2(t1[2] * s1[2], t1[3] * s1[3]);
  const u2v a0 = __builtin_amdgcn_permlane32_swap(X0, Y0, false, false);
  const u2v a1 = __builtin_amdgcn_permlane32_swap(X1, Y1, false, false);
  const u2v b0 = __builtin_amdgcn_permlane16_swap(a0.x, a0.y, false, false);
  const u2v b1 = __builtin_amdgcn_permlane16_swap(a1.x, a1.y, false, false);
  const unsigned w4[4] = {b0.x, b1.x, b0.y, b1.y};
  return __builtin_bit_cast(h8v, *reinterpret_cast<const __attribute__((ext_vector_type(4))) unsigned*>(w4));
}

// A wave's 32 value columns of a DK x dv state (accumulator tiles S[a], rows
// 32 a + 8 (i / 4) + 4 g + i % 4 of this lane's column), stored as half,
// transposed (each column's DK key rows contiguous) at dst = the wave's first
// column.  The columns are contiguous, so the wave's piece is one DK x 64-byte
// run; it goes out through the wave's 4 KB LDS tile in rounds of 64 key rows,
// and each of a round's 4 stores writes 8 whole 128-byte lines rather than 32
// separate 16-byte pieces.  Piece c (16 bytes) of column r sits at tile
// position c ^ (r & 7), so that neither the 8-byte writes nor the 16-byte reads
// conflict.  The tile must not be in use by other code of the wave meanwhile.
template <int DK>
__device__ __forceinline__ void store_state_t(f16_t* __restrict__ dst, const f16x16* S, f16_t* tile, int lane) {
  const int c32 = lane & 31, g2 = lane >> 5;
#pragma unroll
  for (int rd = 0; rd < DK / 64; ++rd) {
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f16x16& t = S[2 * rd + a2];
        const u2v pc = {pack_h2(t[4 * qq], t[4 * qq + 1]), pack_h2(t[4 * qq + 2], t[4 * qq + 3])};
        *reinterpret_cast<u2v*>(tile + 64 * c32 + 8 * ((4 * a2 + qq) ^ (c32 & 7)) + 4 * g2) = pc;
      }
    wave_lds_order();
    h8v val[4];  // all four reads in flight before the first store
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 8 * j + (lane >> 3), pcs = lane & 7;
      val[j] = *reinterpret_cast<const h8v*>(tile + 64 * col + 8 * (pcs ^ (col & 7)));
    }
    wave_lds_order();  // read before the next round (or other code) overwrites the tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 8 * j + (lane >> 3), pcs = lane & 7;
      *reinterpret_cast<h8v*>(dst + (int64_t)col * DK + 64 * rd + 8 * pcs) = val[j];
    }
  }
}

// Asynchronous global -> LDS copies (global_load_lds_dwordx4 / _dword): lane
// l's 16 (4) bytes land at lds_base + 16 l (4 l); lds_base must be the same in
// every lane.  They are issued from inline assembly so that the compiler, which
// cannot tell the two halves of the double buffer apart, does not wait for them
// before every LDS read; the kernel waits for them itself (vm_wait_all) before
// the barrier that publishes the data.  M0 is restored after the issue.
__device__ __forceinline__ unsigned lds_offset(const void* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)(const __attribute__((address_space(3))) void*)p);
}
__device__ __forceinline__ void dma_b128(const void* g, const void* lds_base) {
  unsigned save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "s"(lds_offset(lds_base)), "v"(g)
               : "memory");
}
__device__ __forceinline__ void dma_b32(const void* g, const void* lds_base) {
  unsigned save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "s"(lds_offset(lds_base)), "v"(g)
               : "memory");
}

// The same copy with the LDS byte address given directly (wave-uniform).
__device__ __forceinline__ void dma_b128_at(const void* g, unsigned lds_addr) {
  unsigned save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "s"(lds_addr), "v"(g)
               : "memory");
}
__device__ __forceinline__ void dma_b32_at(const void* g, unsigned lds_addr) {
  unsigned save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "s"(lds_addr), "v"(g)
               : "memory");
}

// LDS tiles are stored without padding, the 16-byte piece c of row r at piece
// position c ^ swz(r), so that both access patterns below are conflict-free:
// 16 consecutive rows read at one piece (operands with k along the row), and 4
// consecutive rows read 32 bytes each (transposed operands).
//   256-byte rows: swz = 2 (r & 3) + 8 ((r >> 2) & 1) + ((r >> 3) & 1)
//   128-byte rows: swz = 2 ((r >> 1) & 3) + ((r >> 3) & 1)
template <int RH>  // halfs per row: 128 or 64
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (RH == 128) return c ^ (((r & 3) << 1) | (((r >> 2) & 1) << 3) | ((r >> 3) & 1));
  else return c ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}
// Operand with k along the row: X[row][16 kb + 8 g .. + 7] (g = lane / 32).
template <int RH>
__device__ __forceinline__ h8v row_frag(const f16_t* X, int row, int kb, int g) {
  return *reinterpret_cast<const h8v*>(X + row * RH + 8 * swz<RH>(row, 2 * kb + g));
}
// Transposing LDS read (ds_read_b64_tr_b16): inside each 16-lane group, lane i
// receives element i % 4 of the 8-byte values addressed by lanes i / 4,
// 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group.  Pointing lane j at
// X[k0 + j / 4][n0 + 4 (j % 4)] hands lane i the column n0 + i of rows
// k0 .. k0 + 3, so a k-major operand comes straight from a row-major tile.
__device__ __forceinline__ s4v lds_tr4(const f16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)p);
}
// Operand with k down the rows: X[16 kb + 8 g + t][c0 + lane % 32], t = 0..7.
template <int RH>
__device__ __forceinline__ h8v col_frag(const f16_t* X, int kb, int c0, int lane) {
  const int row = 16 * kb + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int ch = col >> 3, sub = col & 7;
  const s4v a = lds_tr4(X + row * RH + 8 * swz<RH>(row, ch) + sub);
  const s4v b = lds_tr4(X + (row + 4) * RH + 8 * swz<RH>(row + 4, ch) + sub);
  const s4v v8[2] = {a, b};
  return __builtin_bit_cast(h8v, v8);
}
// 16x16x32 operand with k along the row: X[row][8 (4 kb + G) .. + 7], G = lane / 16.
template <int RH>
__device__ __forceinline__ h8v row_frag16(const f16_t* X, int row, int kb, int G) {
  return *reinterpret_cast<const h8v*>(X + row * RH + 8 * swz<RH>(row, 4 * kb + G));
}
// 16x16x32 operand with k down the rows: X[32 kb + 8 G + t][c0 + lane % 16], t = 0..7.
template <int RH>
__device__ __forceinline__ h8v col_frag16(const f16_t* X, int kb, int c0, int lane) {
  const int row = 32 * kb + 8 * (lane >> 4) + ((lane & 15) >> 2);
  const int col = c0 + 4 * (lane & 3);
  const int ch = col >> 3, sub = col & 7;
  const s4v a = lds_tr4(X + row * RH + 8 * swz<RH>(row, ch) + sub);
  const s4v b = lds_tr4(X + (row + 4) * RH + 8 * swz<RH>(row + 4, ch) + sub);
  const s4v v8[2] = {a, b};
  return __builtin_bit_cast(h8v, v8);
}

// Copy instruction j (of GC / RPI / NW per wave) of a 64-row tile of RH-half
// rows, copied by waves [0, NW) into its swizzled LDS image; src(r, c) is the
// global address of piece c of tile row r.
template <int RH, int NW>
struct TileCopy {
  static constexpr int CPR = RH / 8, RPI = 64 / CPR, PER_WAVE = GC / RPI / NW;
  static_assert(GC % (RPI * NW) == 0, "tile rows split evenly over the waves");
  // tile row whose piece lane `lane` of wave w copies in instruction j
  __device__ static __forceinline__ int row(int w, int lane, int j) { return RPI * (w + NW * j) + lane / CPR; }
  template <class Src>
  __device__ static __forceinline__ void issue(f16_t* dst, int w, int lane, int j, Src src) {
    const int it = w + NW * j;
    const int r = RPI * it + lane / CPR;
    dma_b128(src(r, swz<RH>(r, lane % CPR)), dst + RPI * it * RH);
  }
};

// Keeps the scheduler from mixing the phases of a chunk, which would raise the
// number of live registers past the 256 architectural VGPRs.
#define CHAIN_PHASE() __builtin_amdgcn_sched_barrier(0)

// Workspace of the chunkwise path, per (chunk, head): the solved triangular
// factor T and the decayed query-key products P (half), and gamma,
// gamma_L / gamma (float32).  n_rows / 64 + n_seg bounds the chunk count.
struct ChunkWs {
  f16_t* T;
  f16_t* P;
  float* E;
  size_t bytes;
};

// Long segments: when the walk would leave most compute units idle (few
// (segment, head) pairs) and segments are long, gdn_chunk_fwd cuts them into
// groups of lg chunks and scans the groups' affine state maps (see
// launch_chunk_scan).  The plan depends only on host-known sizes, so the
// workspace size and the launch agree.
// The scan does about 2.5 times the walk's work to cut its serial length, so
// it pays only where the walk would leave the GPU nearly idle: the host takes
// it when the walk would run at most kScanMaxWalks blocks over segments of 16
// or more chunks on average (a single long sequence with few heads; none of
// the layer's configurations, whose other work fills the GPU meanwhile), and
// reserves the workspace for groups of at least kScanMinGroup chunks.
// k_make_groups then sets the group length from the segments' actual chunk
// counts (about target groups in all, at most kScanMaxGroups per segment on
// average, never shorter than kScanMinGroup chunks), and leaves every segment
// whole when none is longer than kScanMinSeg chunks.
constexpr int kScanCUs = 256;       // compute units the walk's grid is sized against
constexpr int kScanMaxWalks = 8;    // walk blocks
constexpr int kScanMinGroup = 8;    // chunks
constexpr int kScanMinSeg = 64;     // chunks
constexpr int kScanMaxGroups = 24;  // groups per segment (the chaining step is serial)
struct ScanPlan {
  bool on;
  int target;        // groups wanted: two rounds of walk blocks
  int64_t n_groups;  // bound on the number of groups
};
inline ScanPlan scan_plan(int64_t n_seg, int64_t n_rows, int H, int dv) {
  ScanPlan p{false, 0, 0};
  const int nvb = dv % 128 == 0 ? dv / 128 : 1;  // walk blocks per (segment, head)
  const int64_t walk_blocks = n_seg * H * nvb, full_chunks = n_rows / GC;
  if (n_seg == 0 || walk_blocks > kScanMaxWalks || full_chunks < 16 * n_seg) return p;
  p.on = true;
  p.target = (int)std::min<int64_t>(2 * kScanCUs / (H * nvb), kScanMaxGroups * n_seg);
  p.n_groups = n_rows / ((int64_t)kScanMinGroup * GC) + n_seg;
  return p;
}
// Scan workspace, after the chunk workspace: the groups' row offsets and
// segments (n_groups + 1 each, a -1 sentinel), each segment's first group
// (n_seg + 1), the groups' maps [group][H][dk][dv + dk] (B, then A) and
// entering states [group][H][dk][dv], float32.
struct ScanWs {
  int32_t* grp_off;
  int32_t* grp_seg;
  int32_t* seg_grp0;
  float* maps;
  float* sg;
  size_t bytes;
};
inline ScanWs scan_ws_layout(void* base, int64_t n_seg, int64_t n_groups, int H, int dk, int dv) {
  ScanWs w;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += (b + 255) / 256 * 256;
    return o;
  };
  const size_t o_go = take((size_t)(n_groups + 1) * 4), o_gs = take((size_t)(n_groups + 1) * 4);
  const size_t o_s0 = take((size_t)(n_seg + 1) * 4);
  const size_t o_m = take((size_t)n_groups * H * dk * (dv + dk) * 4), o_sg = take((size_t)n_groups * H * dk * dv * 4);
  char* b = (char*)base;
  w.grp_off = (int32_t*)(b + o_go);
  w.grp_seg = (int32_t*)(b + o_gs);
  w.seg_grp0 = (int32_t*)(b + o_s0);
  w.maps = (float*)(b + o_m);
  w.sg = (float*)(b + o_sg);
  w.bytes = off;
  return w;
}

inline ChunkWs chunk_ws_layout(void* base, int64_t n_seg, int64_t n_rows, int H, int dk) {
  const int64_t nch = n_rows / GC + n_seg;  // bound on the number of chunks
  ChunkWs w;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += (b + 255) / 256 * 256;
    return o;
  };
  const size_t o_t = take((size_t)nch * H * GC * GC * 2);
  const size_t o_p = take((size_t)nch * H * GC * GC * 2);
  const size_t o_e = take((size_t)nch * H * 2 * GC * 4);
  char* b = (char*)base;
  w.T = (f16_t*)(b + o_t);
  w.P = (f16_t*)(b + o_p);
  w.E = (float*)(b + o_e);
  w.bytes = off;
  return w;
}

}  // namespace mom
