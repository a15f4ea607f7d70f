// Q8_0 instantiation of the grouped mat-vec kernels (gemv_impl.h).
#include "gemv_impl.h"

namespace pesti_gemv {

// Q8_0 rows with an even block count use the two-block unit; a group uses
// it only if every op qualifies.
int group_q8_0(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream) {
  bool pairs = true;
  for (int i = 0; i < n_ops && ops; ++i)
    if (ops[i].in_features % 64 != 0) pairs = false;
  return pairs ? group_dispatch<pesti::FmtQ8_0x2>(n_ops, ops, batch, stream)
               : group_dispatch<pesti::FmtQ8_0>(n_ops, ops, batch, stream);
}

int swiglu_q8_0(PESTI_SWIGLU_ARGS) {
  return in_features % 64 == 0
             ? swiglu_dispatch<pesti::FmtQ8_0x2>(out_features, in_features, w_gate, w_up, gate_scales,
                                                 up_scales, x, h, batch, stream)
             : swiglu_dispatch<pesti::FmtQ8_0>(out_features, in_features, w_gate, w_up, gate_scales,
                                               up_scales, x, h, batch, stream);
}

}  // namespace pesti_gemv
