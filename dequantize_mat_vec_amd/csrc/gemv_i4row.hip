// I4ROW instantiation of the grouped mat-vec kernels (gemv_impl.h).
#include "gemv_impl.h"

namespace pesti_gemv {

int group_i4row(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream) {
  return group_dispatch<pesti::FmtI4Row>(n_ops, ops, batch, stream);
}

int swiglu_i4row(PESTI_SWIGLU_ARGS) {
  return swiglu_dispatch<pesti::FmtI4Row>(out_features, in_features, w_gate, w_up, gate_scales, up_scales, x,
                                       h, batch, stream);
}

}  // namespace pesti_gemv
