// Q8_0 instantiation of the grouped mat-vec kernels (gemv_impl.h).
#include "gemv_impl.h"

namespace pesti_gemv {

// Q8_0 rows with an even block count use the two-block unit, the others the
// one-block unit.  The unit is chosen per op, never per group, so a grouped
// op gives the same bits as its own single call: a group holding both kinds
// is split into one launch per kind, after every op has been validated (an
// invalid op enqueues nothing).
int group_q8_0(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream) {
  if (n_ops < 0 || n_ops > PESTI_MAX_GROUP) return PESTI_ERR_SHAPE;
  if (n_ops > 0 && !ops) return PESTI_ERR_NULL;
  if (batch < 0 || batch > PESTI_MAX_BATCH) return PESTI_ERR_BATCH;
  pesti_gemv_op pairs[PESTI_MAX_GROUP], singles[PESTI_MAX_GROUP];
  int np = 0, ns = 0;
  for (int i = 0; i < n_ops; ++i) {
    const int st = check_op<pesti::FmtQ8_0x2>(ops[i], batch);
    if (st < 0) return st;
    if (ops[i].in_features % 64 == 0) pairs[np++] = ops[i];
    else singles[ns++] = ops[i];
  }
  if (np > 0) {
    const int st = group_dispatch<pesti::FmtQ8_0x2>(np, pairs, batch, stream);
    if (st != PESTI_OK) return st;
  }
  return ns > 0 ? group_dispatch<pesti::FmtQ8_0>(ns, singles, batch, stream) : PESTI_OK;
}

int swiglu_q8_0(PESTI_SWIGLU_ARGS) {
  return in_features % 64 == 0
             ? swiglu_dispatch<pesti::FmtQ8_0x2>(out_features, in_features, w_gate, w_up, gate_scales,
                                                 up_scales, x, h, batch, stream)
             : swiglu_dispatch<pesti::FmtQ8_0>(out_features, in_features, w_gate, w_up, gate_scales,
                                               up_scales, x, h, batch, stream);
}

}  // namespace pesti_gemv
