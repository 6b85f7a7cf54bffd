// One recurrent step per sequence (constant cost per token, jxzklqfsx.com
// write-up, introduction and inference-efficiency section).  For each
// (sequence, activated memory incl. the shared one, head):
//   a = S^T k, b = S^T q                 one pass over S
//   u = c (v - a_g a)                    a_g = forget gate, c = write strength
//   o = a_g b + (k.q) u                  = (a_g S + k u^T)^T q
//   S <- a_g S + k u^T                   written back in place
// (gist.science page, "Core mechanism": forget then delta update; read after
// the write.)  Every value column of the state is updated independently, so
// the reductions over key rows stay within a block that holds whole rows: one
// block per (sequence, slot, head) keeps its [dk][dv] state in registers
// between the read and the write (16 row groups, dk / 16 float4 rows per
// thread: 1024 threads for dv = 256), so each state is read once and written
// once (non-temporal: a state is not touched again within the step) and each
// row goes as one contiguous run.  Measured on the same states: whole 1 KB rows
// move 10% faster than two 512-byte column halves, and 16 row groups of 8 rows
// 5% faster than 8 of 16.
// With DELTA false the memories use gated linear attention: u = c v (no
// a = S^T k term), the rest unchanged.
#include "common.h"

namespace mom {

typedef float dv4 __attribute__((ext_vector_type(4)));

// One slot j of the decode step of sequence b, head h (slot K: the shared
// memory): the state is read and written in place, and the row-group-0
// threads get their four output columns in ov.  Returns false, before any
// barrier, when the slot's memory is out of range (nothing is done).  Every
// thread of the block takes part; the caller separates two calls by a barrier.
template <typename IT, int DK, int DV, int NT, bool DELTA>
__device__ __forceinline__ bool decode_slot(int n_seq, int H, int M, int K, int b, int h, int j,
                                            const int32_t* __restrict__ idx, const int32_t* __restrict__ inv,
                                            const IT* __restrict__ q, const IT* __restrict__ k,
                                            const IT* __restrict__ v, const float* __restrict__ alpha,
                                            const float* __restrict__ beta, float* __restrict__ states, float4& ov) {
  constexpr int CPR = DV / 4;     // threads per state row (float4 each)
  constexpr int RG = NT / CPR;    // row groups
  constexpr int RPT = DK / RG;    // rows per thread
  static_assert(RG * CPR == NT && RPT * RG == DK, "thread layout");
  __shared__ float qs[DK], ks[DK], vs[DV];
  __shared__ float4 red_a[RG][CPR], red_b[RG][CPR];
  __shared__ float kq_s;

  const int tid = threadIdx.x;
  int m;
  int64_t row;
  if (j < K) {
    m = idx[(int64_t)b * K + j];
    row = inv[(int64_t)b * K + j];
  } else {
    m = M;
    row = (int64_t)n_seq * K + b;
  }
  // a routed slot names one of the M routed memories; only the shared slot (j = K) is memory M
  if (j < K && (unsigned)m >= (unsigned)M) return false;
  const float ag = alpha[((int64_t)b * H + h) * (M + 1) + m];
  const float cg = beta[((int64_t)b * H + h) * (M + 1) + m];
  for (int e = tid; e < DK; e += NT) {
    qs[e] = load_as_f32(q + ((int64_t)b * H + h) * DK + e);
    ks[e] = load_as_f32(k + (row * H + h) * DK + e);
  }
  for (int e = tid; e < DV; e += NT) vs[e] = load_as_f32(v + (row * H + h) * DV + e);
  float4* S = reinterpret_cast<float4*>(states + ((((int64_t)b * (M + 1) + m) * H + h) * DK) * DV);
  constexpr int RS4 = DV / 4;  // float4 per full state row
  const int c4 = tid % CPR, rg = tid / CPR;
  float4 reg[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const dv4 t = __builtin_nontemporal_load(reinterpret_cast<const dv4*>(S) + (int64_t)(rg + RG * r) * RS4 + c4);
    reg[r] = make_float4(t.x, t.y, t.z, t.w);
  }
  __syncthreads();
  if (tid < 64) {
    float p = 0.f;
    for (int e = tid; e < DK; e += 64) p = fmaf(ks[e], qs[e], p);
    p = wave_sum_xor(p);
    if (tid == 0) kq_s = p;
  }
  float4 pa = {0.f, 0.f, 0.f, 0.f}, pb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const float kd = ks[rg + RG * r], qd = qs[rg + RG * r];
    pa.x = fmaf(reg[r].x, kd, pa.x); pa.y = fmaf(reg[r].y, kd, pa.y);
    pa.z = fmaf(reg[r].z, kd, pa.z); pa.w = fmaf(reg[r].w, kd, pa.w);
    pb.x = fmaf(reg[r].x, qd, pb.x); pb.y = fmaf(reg[r].y, qd, pb.y);
    pb.z = fmaf(reg[r].z, qd, pb.z); pb.w = fmaf(reg[r].w, qd, pb.w);
  }
  red_a[rg][c4] = pa;
  red_b[rg][c4] = pb;
  __syncthreads();
  // row group 0 adds the partials of its columns in order and publishes the sums
  if (rg == 0) {
    float4 ta0 = red_a[0][c4], tb0 = red_b[0][c4];
#pragma unroll
    for (int g = 1; g < RG; ++g) {
      const float4 ta = red_a[g][c4], tb = red_b[g][c4];
      ta0.x += ta.x; ta0.y += ta.y; ta0.z += ta.z; ta0.w += ta.w;
      tb0.x += tb.x; tb0.y += tb.y; tb0.z += tb.z; tb0.w += tb.w;
    }
    red_a[0][c4] = ta0;
    red_b[0][c4] = tb0;
  }
  __syncthreads();
  const float4 sa = red_a[0][c4], sb = red_b[0][c4];
  const float kq = kq_s;
  const float4 vv = reinterpret_cast<const float4*>(vs)[c4];
  float4 u;
  if (DELTA) {
    u.x = cg * (vv.x - ag * sa.x);
    u.y = cg * (vv.y - ag * sa.y);
    u.z = cg * (vv.z - ag * sa.z);
    u.w = cg * (vv.w - ag * sa.w);
  } else {
    u.x = cg * vv.x;
    u.y = cg * vv.y;
    u.z = cg * vv.z;
    u.w = cg * vv.w;
  }
  if (rg == 0) {
    ov.x = fmaf(kq, u.x, ag * sb.x);
    ov.y = fmaf(kq, u.y, ag * sb.y);
    ov.z = fmaf(kq, u.z, ag * sb.z);
    ov.w = fmaf(kq, u.w, ag * sb.w);
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const float kd = ks[rg + RG * r];
    float4 s2;
    s2.x = fmaf(kd, u.x, ag * reg[r].x);
    s2.y = fmaf(kd, u.y, ag * reg[r].y);
    s2.z = fmaf(kd, u.z, ag * reg[r].z);
    s2.w = fmaf(kd, u.w, ag * reg[r].w);
    const dv4 t2 = {s2.x, s2.y, s2.z, s2.w};
    __builtin_nontemporal_store(t2, reinterpret_cast<dv4*>(S) + (int64_t)(rg + RG * r) * RS4 + c4);
  }
  return true;
}

template <typename IT, int DK, int DV, int NT, bool DELTA>
__global__ __launch_bounds__(NT) void k_gdn_decode(int n_seq, int H, int M, int K, const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ inv, const IT* __restrict__ q,
                                                    const IT* __restrict__ k, const IT* __restrict__ v,
                                                    const float* __restrict__ alpha, const float* __restrict__ beta,
                                                    float* __restrict__ states, float* __restrict__ o) {
  const int bid = blockIdx.x;
  const int h = bid % H;
  const int j = (bid / H) % (K + 1);
  const int b = bid / (H * (K + 1));
  float4 ov = {0.f, 0.f, 0.f, 0.f};
  if (!decode_slot<IT, DK, DV, NT, DELTA>(n_seq, H, M, K, b, h, j, idx, inv, q, k, v, alpha, beta, states, ov))
    return;
  const int64_t row = j < K ? (int64_t)inv[(int64_t)b * K + j] : (int64_t)n_seq * K + b;
  if ((int)threadIdx.x < DV / 4) reinterpret_cast<float4*>(o + (row * H + h) * DV)[threadIdx.x] = ov;
}

// The decode step with the combine folded in: one block per (sequence, head)
// runs the shared memory's slot and then the routed slots in order, and adds
// their outputs as mom_combine does (the shared one, then one fma w_j o_j per
// routed slot, j ascending), writing out[b][h] directly; no per-slot outputs
// are stored.  A slot whose memory is out of range (idx not from mom_route)
// adds nothing.
template <typename IT, int DK, int DV, int NT, bool DELTA>
__global__ __launch_bounds__(NT) void k_gdn_decode_combined(int n_seq, int H, int M, int K,
                                                             const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ inv,
                                                             const float* __restrict__ w, const IT* __restrict__ q,
                                                             const IT* __restrict__ k, const IT* __restrict__ v,
                                                             const float* __restrict__ alpha,
                                                             const float* __restrict__ beta,
                                                             float* __restrict__ states, float* __restrict__ out) {
  const int h = blockIdx.x % H, b = blockIdx.x / H;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int jj = 0; jj <= K; ++jj) {  // the shared memory's slot K first, then 0 .. K - 1
    const int j = jj == 0 ? K : jj - 1;
    if (jj > 0) __syncthreads();  // the previous slot is done with the shared arrays
    float4 ov = {0.f, 0.f, 0.f, 0.f};
    if (!decode_slot<IT, DK, DV, NT, DELTA>(n_seq, H, M, K, b, h, j, idx, inv, q, k, v, alpha, beta, states, ov))
      continue;
    if (jj == 0) {
      acc = ov;
    } else {
      const float g = w[(int64_t)b * K + j];
      acc.x = fmaf(g, ov.x, acc.x);
      acc.y = fmaf(g, ov.y, acc.y);
      acc.z = fmaf(g, ov.z, acc.z);
      acc.w = fmaf(g, ov.w, acc.w);
    }
  }
  if ((int)threadIdx.x < DV / 4) reinterpret_cast<float4*>(out + ((int64_t)b * H + h) * DV)[threadIdx.x] = acc;
}

// w non-null: the combined kernel (o is then the layer's output [n_seq][H][dv]).
template <typename IT>
static void launch_decode(const mom_dims& d, int n_seq, const int32_t* idx, const int32_t* inv, const void* q,
                          const void* k, const void* v, const float* alpha, const float* beta, float* states,
                          float* o, bool delta, hipStream_t st, const float* w = nullptr) {
  const int64_t slots = (int64_t)n_seq * (d.topk + 1) * d.H;
#define MOM_DEC2(DK, DV, DELTA)                                                                                  \
  do {                                                                                                           \
    if (w)                                                                                                       \
      hipLaunchKernelGGL((k_gdn_decode_combined<IT, DK, DV, 4 * DV, DELTA>), dim3((unsigned)(n_seq * d.H)),      \
                         dim3(4 * DV), 0, st, n_seq, d.H, d.M, d.topk, idx, inv, w, (const IT*)q, (const IT*)k,  \
                         (const IT*)v, alpha, beta, states, o);                                                \
    else                                                                                                         \
      hipLaunchKernelGGL((k_gdn_decode<IT, DK, DV, 4 * DV, DELTA>), dim3((unsigned)slots), dim3(4 * DV), 0, st, \
                         n_seq, d.H, d.M, d.topk, idx, inv, (const IT*)q, (const IT*)k, (const IT*)v, alpha,     \
                         beta, states, o);                                                                     \
  } while (0)
#define MOM_DEC(DK, DV)           \
  do {                            \
    if (delta)                    \
      MOM_DEC2(DK, DV, true);     \
    else                          \
      MOM_DEC2(DK, DV, false);    \
  } while (0)
  if (d.dk == 64) {
    if (d.dv == 64) MOM_DEC(64, 64);
    else if (d.dv == 128) MOM_DEC(64, 128);
    else MOM_DEC(64, 256);
  } else {
    if (d.dv == 64) MOM_DEC(128, 64);
    else if (d.dv == 128) MOM_DEC(128, 128);
    else MOM_DEC(128, 256);
  }
#undef MOM_DEC
#undef MOM_DEC2
}

}  // namespace mom

namespace mom {
static mom_status decode_step(bool delta, const mom_dims* dims, int32_t n_seq, const int32_t* idx,
                              const int32_t* inv, const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, float* states, float* o, void* stream, bool combined = false,
                              const float* w = nullptr) {
  mom_status s = check_dims(dims);
  if (s != MOM_OK) return s;
  if (dims->dv != 64 && dims->dv != 128 && dims->dv != 256) return MOM_ERR_UNSUPPORTED;
  if (n_seq < 0) return MOM_ERR_DIMS;
  MOM_CHECK_PTR(idx);
  MOM_CHECK_PTR(inv);
  MOM_CHECK_PTR(q);
  MOM_CHECK_PTR(k);
  MOM_CHECK_PTR(v);
  MOM_CHECK_PTR(alpha);
  MOM_CHECK_PTR(beta);
  MOM_CHECK_PTR(states);
  MOM_CHECK_PTR(o);
  if (combined) MOM_CHECK_PTR(w);
  if (n_seq == 0) return MOM_OK;
  hipStream_t st = (hipStream_t)stream;
  if (dims->dtype == MOM_DTYPE_BF16)
    launch_decode<f16_t>(*dims, n_seq, idx, inv, q, k, v, alpha, beta, states, o, delta, st, w);
  else
    launch_decode<float>(*dims, n_seq, idx, inv, q, k, v, alpha, beta, states, o, delta, st, w);
  return launch_status();
}
}  // namespace mom

extern "C" mom_status gdn_decode_step(const mom_dims* dims, int32_t n_seq, const int32_t* idx, const int32_t* inv,
                                      const void* q, const void* k, const void* v, const float* alpha,
                                      const float* beta, float* states, float* o, void* stream) {
  return mom::decode_step(true, dims, n_seq, idx, inv, q, k, v, alpha, beta, states, o, stream);
}

extern "C" mom_status gla_decode_step(const mom_dims* dims, int32_t n_seq, const int32_t* idx, const int32_t* inv,
                                      const void* q, const void* k, const void* v, const float* alpha,
                                      const float* beta, float* states, float* o, void* stream) {
  return mom::decode_step(false, dims, n_seq, idx, inv, q, k, v, alpha, beta, states, o, stream);
}

extern "C" mom_status gdn_decode_step_combined(const mom_dims* dims, int32_t n_seq, const int32_t* idx,
                                               const int32_t* inv, const float* w, const void* q, const void* k,
                                               const void* v, const float* alpha, const float* beta, float* states,
                                               float* out, void* stream) {
  return mom::decode_step(true, dims, n_seq, idx, inv, q, k, v, alpha, beta, states, out, stream, true, w);
}

extern "C" mom_status gla_decode_step_combined(const mom_dims* dims, int32_t n_seq, const int32_t* idx,
                                               const int32_t* inv, const float* w, const void* q, const void* k,
                                               const void* v, const float* alpha, const float* beta, float* states,
                                               float* out, void* stream) {
  return mom::decode_step(false, dims, n_seq, idx, inv, q, k, v, alpha, beta, states, out, stream, true, w);
}
