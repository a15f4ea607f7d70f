// C entry points of the fused dequantize + mat-vec (kernels in gemv_impl.h,
// instantiated per format in gemv_q8_0.hip, gemv_q2_k.hip, gemv_q3_k.hip,
// gemv_q4_k.hip, gemv_q5_k.hip, gemv_q6_k.hip, gemv_i8row.hip and gemv_i4row.hip).
#include "gemv_impl.h"

namespace pesti {

// Ops with in_features == 0: y = bias (or zeros), every batch column.
__global__ __launch_bounds__(kThreads) void bias_fill_kernel(GroupArgs g, int batch) {
  const GemvArgs a = g.op[blockIdx.y];
  const int64_t o = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (o >= a.out) return;
  const float v = a.bias ? a.bias[o] : 0.f;
  for (int b = 0; b < batch; ++b) a.y[b * a.out + o] = v;
}

}  // namespace pesti

namespace pesti_gemv {

int fill_bias(const GroupArgs& g, int batch, hipStream_t stream) {
  int64_t rows = 0;
  for (int i = 0; i < g.n_ops; ++i) rows = g.op[i].out > rows ? g.op[i].out : rows;
  if (rows <= 0 || batch <= 0) return PESTI_OK;
  const int64_t blocks = (rows + pesti::kThreads - 1) / pesti::kThreads;
  GroupArgs args = g;
  int nb = batch;
  void* params[] = {&args, &nb};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::bias_fill_kernel),
                                       dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(g.n_ops)),
                                       dim3(pesti::kThreads), params, 0, stream);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

}  // namespace pesti_gemv

extern "C" {

int pesti_gemv_group(int32_t format, int32_t n_ops, const pesti_gemv_op* ops, int32_t batch,
                     void* stream) {
  switch (format) {
    case PESTI_FMT_Q8_0: return pesti_gemv::group_q8_0(n_ops, ops, batch, stream);
    case PESTI_FMT_Q4_K: return pesti_gemv::group_q4_k(n_ops, ops, batch, stream);
    case PESTI_FMT_Q4_K_STREAM: return pesti_gemv::group_q4_k_stream(n_ops, ops, batch, stream);
    case PESTI_FMT_Q5_K: return pesti_gemv::group_q5_k(n_ops, ops, batch, stream);
    case PESTI_FMT_Q2_K: return pesti_gemv::group_q2_k(n_ops, ops, batch, stream);
    case PESTI_FMT_Q3_K: return pesti_gemv::group_q3_k(n_ops, ops, batch, stream);
    case PESTI_FMT_Q6_K: return pesti_gemv::group_q6_k(n_ops, ops, batch, stream);
    case PESTI_FMT_I8ROW: return pesti_gemv::group_i8row(n_ops, ops, batch, stream);
    case PESTI_FMT_I4ROW: return pesti_gemv::group_i4row(n_ops, ops, batch, stream);
    default: return PESTI_ERR_SHAPE;
  }
}

int pesti_gemv_swiglu(int32_t format, int64_t out_features, int64_t in_features, const void* w_gate,
                      const void* w_up, const float* gate_scales, const float* up_scales, const float* x,
                      float* h, int32_t batch, void* stream) {
  switch (format) {
    case PESTI_FMT_Q8_0:
      return pesti_gemv::swiglu_q8_0(out_features, in_features, w_gate, w_up, nullptr, nullptr, x, h, batch,
                                     stream);
    case PESTI_FMT_Q4_K:
      return pesti_gemv::swiglu_q4_k(out_features, in_features, w_gate, w_up, nullptr, nullptr, x, h, batch,
                                     stream);
    case PESTI_FMT_Q2_K:
      return pesti_gemv::swiglu_q2_k(out_features, in_features, w_gate, w_up, nullptr, nullptr, x, h, batch,
                                     stream);
    case PESTI_FMT_Q3_K:
      return pesti_gemv::swiglu_q3_k(out_features, in_features, w_gate, w_up, nullptr, nullptr, x, h, batch,
                                     stream);
    case PESTI_FMT_Q5_K:
      return pesti_gemv::swiglu_q5_k(out_features, in_features, w_gate, w_up, nullptr, nullptr, x, h, batch,
                                     stream);
    case PESTI_FMT_Q6_K:
      return pesti_gemv::swiglu_q6_k(out_features, in_features, w_gate, w_up, nullptr, nullptr, x, h, batch,
                                     stream);
    case PESTI_FMT_I8ROW:
      return pesti_gemv::swiglu_i8row(out_features, in_features, w_gate, w_up, gate_scales, up_scales, x, h,
                                      batch, stream);
    case PESTI_FMT_I4ROW:
      return pesti_gemv::swiglu_i4row(out_features, in_features, w_gate, w_up, gate_scales, up_scales, x, h,
                                      batch, stream);
    default: return PESTI_ERR_SHAPE;
  }
}

int pesti_gemv_q8_0(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, blocks, nullptr, x, y, bias);
  return pesti_gemv::group_q8_0(1, &o, batch, stream);
}

int pesti_gemv_q4_k(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, blocks, nullptr, x, y, bias);
  return pesti_gemv::group_q4_k(1, &o, batch, stream);
}

int pesti_gemv_q4_k_stream(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, blocks, nullptr, x, y, bias);
  return pesti_gemv::group_q4_k_stream(1, &o, batch, stream);
}

int pesti_gemv_q2_k(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, blocks, nullptr, x, y, bias);
  return pesti_gemv::group_q2_k(1, &o, batch, stream);
}

int pesti_gemv_q3_k(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, blocks, nullptr, x, y, bias);
  return pesti_gemv::group_q3_k(1, &o, batch, stream);
}

int pesti_gemv_q5_k(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, blocks, nullptr, x, y, bias);
  return pesti_gemv::group_q5_k(1, &o, batch, stream);
}

int pesti_gemv_q6_k(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, blocks, nullptr, x, y, bias);
  return pesti_gemv::group_q6_k(1, &o, batch, stream);
}

int pesti_gemv_i8row(int64_t out_features, int64_t in_features, const int8_t* codes,
                     const float* row_scales, const float* x, float* y, const float* bias,
                     int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, codes, row_scales, x, y, bias);
  return pesti_gemv::group_i8row(1, &o, batch, stream);
}

int pesti_gemv_i4row(int64_t out_features, int64_t in_features, const void* packed,
                     const float* row_scales, const float* x, float* y, const float* bias,
                     int32_t batch, void* stream) {
  const pesti_gemv_op o = pesti_gemv::make_op(out_features, in_features, packed, row_scales, x, y, bias);
  return pesti_gemv::group_i4row(1, &o, batch, stream);
}

}  // extern "C"
