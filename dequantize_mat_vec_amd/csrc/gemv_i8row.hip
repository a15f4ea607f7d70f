// I8ROW instantiation of the grouped mat-vec kernels (gemv_impl.h).
#include "gemv_impl.h"

namespace pesti_gemv {

int group_i8row(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream) {
  return group_dispatch<pesti::FmtI8Row>(n_ops, ops, batch, stream);
}

int swiglu_i8row(PESTI_SWIGLU_ARGS) {
  return swiglu_dispatch<pesti::FmtI8Row>(out_features, in_features, w_gate, w_up, gate_scales, up_scales, x,
                                       h, batch, stream);
}

}  // namespace pesti_gemv
