// Small-M GEMMs with a caller's workspace: the split form of the K-split
// kernels ("inferno" README, "Benchmarks": the prompt-width products), for
// narrow layers with long rows, where one workgroup per output tile leaves
// most compute units idle.  The partial tiles of the splits go to the
// workspace; a second launch sums them in split order and adds the bias, so
// results do not depend on timing.  An allocation-free variant takes the
// partials to a static device array of the library instead.
#include <atomic>

#include "common.h"

namespace pesti {

// y[e] = part[0][e] + ... + part[splits-1][e] + bias[e % n], four outputs
// per thread when n is a multiple of 4 (then m * n is, and every row starts
// 16-byte aligned), else one.
template <bool V4>
__global__ __launch_bounds__(256) void split_sum_kernel(int64_t m, int64_t n, const float* part, int splits,
                                                        const float* bias, float* y) {
  const int64_t mn = m * n;
  if constexpr (V4) {
    const int64_t e = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
    if (e >= mn) return;
    float4 r = *reinterpret_cast<const float4*>(part + e);
    for (int s = 1; s < splits; ++s) {
      const float4 p = *reinterpret_cast<const float4*>(part + s * mn + e);
      r.x += p.x;
      r.y += p.y;
      r.z += p.z;
      r.w += p.w;
    }
    if (bias) {
      const int64_t c = e % n;
      r.x += bias[c];
      r.y += bias[c + 1];
      r.z += bias[c + 2];
      r.w += bias[c + 3];
    }
    *reinterpret_cast<float4*>(y + e) = r;
  } else {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= mn) return;
    float r = part[e];
    for (int s = 1; s < splits; ++s) r += part[s * mn + e];
    y[e] = r + (bias ? bias[e % n] : 0.f);
  }
}

}  // namespace pesti

int pesti_host::launch_split_sum(int64_t m, int64_t n, const float* part, int splits, const float* bias, float* y,
                                 hipStream_t st) {
  const bool v4 = n % 4 == 0;
  const int64_t threads = v4 ? m * n / 4 : m * n;
  void* params[] = {&m, &n, &part, &splits, &bias, &y};
  const void* fn = v4 ? reinterpret_cast<const void*>(&pesti::split_sum_kernel<true>)
                      : reinterpret_cast<const void*>(&pesti::split_sum_kernel<false>);
  const hipError_t e =
      hipLaunchKernel(fn, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), params, 0, st);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

// The allocation-free variant's scratch: this array per GPU, held until the
// process ends.  In host code its name is only a stand-in; kernels get the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[PESTI_GEMM_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of `scratch`, looked up once per device (every
// thread that races here stores the same address).
int scratch_on(int dev, float** out) {
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return PESTI_ERR_DEVICE;
    p = static_cast<float*>(a);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PESTI_OK;
}

bool gemm_format(int32_t format) {
  switch (format) {
    case PESTI_FMT_F16:
    case PESTI_FMT_Q8_0:
    case PESTI_FMT_Q2_K:
    case PESTI_FMT_Q3_K:
    case PESTI_FMT_Q4_K:
    case PESTI_FMT_Q5_K:
    case PESTI_FMT_Q6_K:
      return true;
    default:
      return false;
  }
}

int64_t workspace_bytes(int32_t format, int64_t m, int64_t out_features, int64_t in_features) {
  const int s = pesti_host::gemm_splits(format, m, out_features, in_features);
  return s > 1 ? static_cast<int64_t>(s) * m * out_features * static_cast<int64_t>(sizeof(float)) : 0;
}

int run(int32_t format, int64_t m, int64_t n, int64_t k, const void* w, const uint16_t* x, float* y,
        const float* bias, float* ws, hipStream_t st) {
  if (format == PESTI_FMT_F16)
    return pesti_host::gemm_f16_run(m, n, k, static_cast<const uint16_t*>(w), x, y, bias, ws, st);
  return pesti_host::gemm_quant_run(format, m, n, k, w, x, y, bias, ws, st);
}

}  // namespace

extern "C" {

int64_t pesti_gemm_workspace_bytes(int32_t format, int64_t m, int64_t out_features, int64_t in_features) {
  if (!gemm_format(format)) return PESTI_ERR_SHAPE;
  if (out_features < 0 || in_features < 0 || in_features % 32 != 0 || in_features > PESTI_MAX_IN_FEATURES)
    return PESTI_ERR_SHAPE;
  if (m < 0 || m > PESTI_MAX_GEMM_M) return PESTI_ERR_BATCH;
  return workspace_bytes(format, m, out_features, in_features);
}

int pesti_gemm_smallm_ws(int32_t format, int64_t m, int64_t out_features, int64_t in_features, const void* w,
                         const uint16_t* x, float* y, const float* bias, void* workspace, int64_t workspace_bytes_,
                         void* stream) {
  const int64_t need = pesti_gemm_workspace_bytes(format, m, out_features, in_features);
  if (need < 0) return static_cast<int>(need);
  float* ws = nullptr;
  if (need > 0) {
    if (!workspace || workspace_bytes_ < need) return PESTI_ERR_WORKSPACE;
    if (!pesti_host::aligned(workspace, 16)) return PESTI_ERR_ALIGN;
    ws = static_cast<float*>(workspace);
  }
  return run(format, m, out_features, in_features, w, x, y, bias, ws, static_cast<hipStream_t>(stream));
}

int pesti_gemm_smallm_noalloc(int32_t format, int64_t m, int64_t out_features, int64_t in_features,
                              const void* w, const uint16_t* x, float* y, const float* bias, void* stream) {
  const int64_t need = pesti_gemm_workspace_bytes(format, m, out_features, in_features);
  if (need < 0) return static_cast<int>(need);
  if (need > PESTI_GEMM_SCRATCH_BYTES) return PESTI_ERR_WORKSPACE;
  float* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    size_t lds = 0;
    int st = pesti_host::current_device(&dev, &lds);
    if (st != PESTI_OK) return st;
    st = scratch_on(dev, &ws);
    if (st != PESTI_OK) return st;
  }
  return run(format, m, out_features, in_features, w, x, y, bias, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
