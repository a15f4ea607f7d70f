// Q4_K (row and stream layouts) instantiation of the grouped mat-vec kernels
// (gemv_impl.h).
#include "gemv_impl.h"

namespace pesti_gemv {

int group_q4_k(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream) {
  return group_dispatch<pesti::FmtQ4_K>(n_ops, ops, batch, stream);
}

int group_q4_k_stream(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream) {
  return group_dispatch<pesti::FmtQ4_KS>(n_ops, ops, batch, stream);
}

int swiglu_q4_k(PESTI_SWIGLU_ARGS) {
  return swiglu_dispatch<pesti::FmtQ4_K>(out_features, in_features, w_gate, w_up, gate_scales, up_scales, x,
                                       h, batch, stream);
}

}  // namespace pesti_gemv
