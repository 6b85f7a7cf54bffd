// Entry points without kernels of their own: gdn_chunk_fwd's validation and
// dispatch to the kernel variant for the storage type, workspace sizes, and
// status strings.
#include "common.h"

namespace mom {
template <typename IT>
mom_status launch_gdn_chunk_valu(const mom_dims& d, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                                 const int32_t* row_token, const void* q, const void* k, const void* v,
                                 const float* alpha_p, const float* beta_p, const float* state_in, float* state_out,
                                 float* o, bool delta, hipStream_t st);
mom_status launch_gdn_chunk_mfma(const mom_dims& d, int n_seg, int n_rows, const int32_t* seg_off,
                                 const int32_t* seg_state, const int32_t* row_token, const void* q, const void* k,
                                 const void* v, const float* alpha_p, const float* beta_p, const float* state_in,
                                 float* state_out, float* o, void* ws, bool delta, hipStream_t st);
size_t gdn_chunk_ws_bytes(int64_t n_seg, int64_t n_rows, int H, int dk, int dv);
size_t route_bwd_ws_bytes(const mom_dims& d);
}  // namespace mom

extern "C" size_t gdn_chunk_workspace_bytes(const mom_dims* dims, int32_t n_seg, int32_t n_rows) {
  using namespace mom;
  if (check_dims(dims) != MOM_OK || n_seg < 0 || n_rows < 0) return 0;
  if (dims->dtype != MOM_DTYPE_BF16) return 0;
  return gdn_chunk_ws_bytes(n_seg, n_rows, dims->H, dims->dk, dims->dv);
}

namespace mom {
// Validation and dispatch shared by the two update rules.
static mom_status chunk_fwd(bool delta, const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
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
  const size_t need = gdn_chunk_workspace_bytes(dims, n_seg, n_rows);
  if (need && (!ws || ws_bytes < need)) return MOM_ERR_WORKSPACE;
  MOM_CHECK_OPT_PTR(ws);
  if (n_seg == 0) return MOM_OK;
  hipStream_t st = (hipStream_t)stream;
  if (dims->dtype == MOM_DTYPE_BF16)
    return launch_gdn_chunk_mfma(*dims, n_seg, n_rows, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                                 state_in, state_out, o, ws, delta, st);
  return launch_gdn_chunk_valu<float>(*dims, n_seg, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                                      state_in, state_out, o, delta, st);
}
}  // namespace mom

extern "C" mom_status gdn_chunk_fwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                                    int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                                    const int32_t* row_token, const void* q, const void* k, const void* v,
                                    const float* alpha_p, const float* beta_p, const float* state_in,
                                    float* state_out, float* o, void* ws, size_t ws_bytes, void* stream) {
  return mom::chunk_fwd(true, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p,
                        beta_p, state_in, state_out, o, ws, ws_bytes, stream);
}

extern "C" mom_status gla_chunk_fwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                                    int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                                    const int32_t* row_token, const void* q, const void* k, const void* v,
                                    const float* alpha_p, const float* beta_p, const float* state_in,
                                    float* state_out, float* o, void* ws, size_t ws_bytes, void* stream) {
  return mom::chunk_fwd(false, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
                        alpha_p, beta_p, state_in, state_out, o, ws, ws_bytes, stream);
}

extern "C" size_t mom_workspace_bytes(const mom_dims* dims, int32_t which) {
  using namespace mom;
  if (check_dims(dims) != MOM_OK) return 0;
  const mom_dims& d = *dims;
  if (which == MOM_WS_DISPATCH) {
    const int64_t nsub = (d.T + kCountTile - 1) / kCountTile;
    const int64_t bytes = (dispatch_offs_at(d) + (int64_t)d.M * d.B * nsub) * 4;  // counts, then their scan
    return (size_t)((bytes + 255) / 256 * 256);
  }
  if (which == MOM_WS_CHUNK) {
    const Sizes z = sizes_of(d);
    return gdn_chunk_workspace_bytes(dims, (int32_t)z.n_seg, (int32_t)z.N);
  }
  if (which == MOM_WS_ROUTE_BWD) return route_bwd_ws_bytes(d);
  return 0;
}

extern "C" const char* mom_status_string(int32_t status) {
  switch (status) {
    case MOM_OK: return "ok";
    case MOM_ERR_NULL: return "a required pointer is NULL";
    case MOM_ERR_DIMS: return "a size is out of range or inconsistent";
    case MOM_ERR_UNSUPPORTED: return "shape or dtype outside the supported set";
    case MOM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOM_ERR_WORKSPACE: return "workspace missing or too small";
    case MOM_ERR_LAUNCH: return "kernel launch failed";
    case MOM_ERR_TOO_LARGE: return "sizes exceed the fixed scratch of an allocation-free entry point";
    default: return "unknown status";
  }
}
