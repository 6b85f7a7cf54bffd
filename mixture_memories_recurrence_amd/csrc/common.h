// Internal helpers shared by the gfx950 kernels of libmom (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mom.h"

namespace mom {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef _Float16 f16_t;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bfv8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kDispatchTile = 64;  // positions per dispatch tile (one scatter block of one wave)
constexpr int kCountTile = 64;     // positions per dispatch count (one wave)

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float load_as_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_as_f32(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_as_f32(const f16_t* p) { return (float)*p; }
__device__ __forceinline__ void store_from_f32(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_from_f32(f16_t* p, float v) { *p = (f16_t)v; }

// ---------------------------------------------------------------- forget gates
// The chunk form works with prefix sums of log alpha.  A gate of 0 (log = -inf)
// would turn the decay ratios e^{g_i - g_j} into NaN, so each row's log gate is
// held at or above -30: e^{-30} ~ 9e-14 is already a zero decay at float32's
// resolution of the state, and every sum stays finite.
constexpr float kLogGateFloor = -30.f;
__device__ __forceinline__ float log_gate(float a) { return fmaxf(logf(a), kLogGateFloor); }
// The same in float64, for prefix sums whose differences must keep float32's
// relative precision after a floored row (a sum near -30 loses 5 bits in float32).
__device__ __forceinline__ double log_gate_f64(float a) { return fmax(log((double)a), (double)kLogGateFloor); }

// ---------------------------------------------------------------- derived sizes
struct Sizes {
  int64_t NT, NR, N, n_seg, n_state;
};

inline Sizes sizes_of(const mom_dims& d) {
  Sizes s;
  s.NT = (int64_t)d.B * d.T;
  s.NR = s.NT * d.topk;
  s.N = s.NR + s.NT;
  s.n_seg = (int64_t)(d.M + 1) * d.B;
  s.n_state = (int64_t)d.B * (d.M + 1);
  return s;
}

// ---------------------------------------------------------------- host checks
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks common to every entry point.
inline mom_status check_dims(const mom_dims* d) {
  if (!d) return MOM_ERR_NULL;
  if (d->B < 1 || d->T < 1 || d->H < 1 || d->M < 1 || d->topk < 1) return MOM_ERR_DIMS;
  if (d->topk > d->M) return MOM_ERR_DIMS;
  if (d->M > 64 || d->topk > 8) return MOM_ERR_UNSUPPORTED;
  if (d->dk != 64 && d->dk != 128) return MOM_ERR_UNSUPPORTED;
  // 64, 128 or 256 everywhere; a multiple of 128 up to 1024 for the entry points
  // other than gdn_decode_step (which rejects it)
  if (d->dv != 64 && !(d->dv % 128 == 0 && d->dv >= 128 && d->dv <= 1024)) return MOM_ERR_UNSUPPORTED;
  // chunk rows: 64 on the matrix cores; 16, 32 or 64 with float32 storage
  if (d->chunk != 64 && !(d->dtype == MOM_DTYPE_F32 && (d->chunk == 16 || d->chunk == 32))) return MOM_ERR_UNSUPPORTED;
  if (d->dtype != MOM_DTYPE_F32 && d->dtype != MOM_DTYPE_BF16) return MOM_ERR_UNSUPPORTED;
  if (d->D < 64 || d->D > 8192 || d->D % 64 != 0) return MOM_ERR_UNSUPPORTED;
  if (d->H > 64) return MOM_ERR_UNSUPPORTED;
  if (d->B > 65535) return MOM_ERR_UNSUPPORTED;
  const Sizes s = sizes_of(*d);
  if (s.N >= (int64_t)1 << 31) return MOM_ERR_DIMS;
  if (s.N * d->H * (int64_t)d->dv >= ((int64_t)1 << 40)) return MOM_ERR_DIMS;
  return MOM_OK;
}

#define MOM_CHECK_PTR(p)                  \
  do {                                    \
    if (!(p)) return MOM_ERR_NULL;        \
    if (!aligned16(p)) return MOM_ERR_ALIGN; \
  } while (0)
#define MOM_CHECK_OPT_PTR(p)                          \
  do {                                                \
    if ((p) && !aligned16(p)) return MOM_ERR_ALIGN;   \
  } while (0)

inline mom_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOM_OK : MOM_ERR_LAUNCH;
}

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// The dispatch's workspace: the counts (int32 [M][B][ceil(T / 64)]), then,
// from this offset in int32 entries, their exclusive scan.
inline int64_t dispatch_offs_at(const mom_dims& d) {
  const int64_t n = (int64_t)d.M * d.B * ((d.T + kCountTile - 1) / kCountTile);
  return (n + 63) / 64 * 64;
}

// dispatch.hip: the dispatch's per-64-position counts of idx into cnt
mom_status dispatch_count_only(const mom_dims* dims, const int32_t* idx, int32_t* cnt, hipStream_t st);

// ---------------------------------------------------------------- wave helpers
template <typename T>
__device__ __forceinline__ T wave_sum_xor(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Workgroups are handed to the 8 XCDs round-robin (block p runs on XCD p % 8).
// Map physical block p to a logical index so that each XCD receives one
// contiguous range of logical work items: neighbours in logical order then
// share that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t p, int64_t G) {
  const int64_t x = p & 7, i = p >> 3;
  const int64_t per = G >> 3, rem = G & 7;
  return x * per + (x < rem ? x : rem) + i;
}

}  // namespace mom
