// Backward dispatch: picks the (head dim, mode, input format) instance of the MFMA backward
// (bwd_inst.hip, compiled once per triple) or the fp32 path.
#include "jfa_internal.h"

namespace jfa {

hipError_t launch_backward_f32(const BwdParams& p, const TileCfg& tc, int head_dim,
                               int64_t max_q_items, int64_t max_k_items, int cu_count,
                               hipStream_t s);

namespace {

hipError_t dispatch(const BwdParams& p, const TileCfg& tc, int head_dim, int64_t mq, int64_t mk,
                    int cu, hipStream_t s, bool dbias, bool fp8) {
#define JFA_BWD_CASE(D_, M_)                                                            \
  if (head_dim == D_ && p.mode == M_)                                                   \
    return fp8 ? launch_bwd_dm<D_, M_, true>(p, tc, mq, mk, cu, s, dbias)               \
               : launch_bwd_dm<D_, M_, false>(p, tc, mq, mk, cu, s, dbias);
  JFA_BWD_CASE(128, JFA_MODE_SOFTMAX)
  JFA_BWD_CASE(128, JFA_MODE_SILU)
  JFA_BWD_CASE(128, JFA_MODE_GELU)
  JFA_BWD_CASE(64, JFA_MODE_SOFTMAX)
  JFA_BWD_CASE(64, JFA_MODE_SILU)
  JFA_BWD_CASE(64, JFA_MODE_GELU)
#undef JFA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward_dbias(const BwdParams& p, const TileCfg& tc, int head_dim,
                                 int64_t max_q_items, int64_t max_k_items, int cu_count,
                                 hipStream_t s) {
  return dispatch(p, tc, head_dim, max_q_items, max_k_items, cu_count, s, true, false);
}

hipError_t launch_backward(const BwdParams& p, const TileCfg& tc, int head_dim, int dtype,
                           int64_t max_q_items, int64_t max_k_items, int cu_count, hipStream_t s) {
  if (dtype == JFA_F32)
    return launch_backward_f32(p, tc, head_dim, max_q_items, max_k_items, cu_count, s);
  if (dtype != JFA_BF16 && dtype != JFA_MXFP8_E4M3) return hipErrorInvalidValue;
  return dispatch(p, tc, head_dim, max_q_items, max_k_items, cu_count, s, false,
                  dtype == JFA_MXFP8_E4M3);
}

}  // namespace jfa
