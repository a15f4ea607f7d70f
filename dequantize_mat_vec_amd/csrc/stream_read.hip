// Measurement hook: a plain streaming read of a device buffer, the
// "size-matched streaming-read ceiling" a mat-vec of the same byte count is
// compared with.  Every 16-byte chunk is read once with a vector load; each
// workgroup folds what it read into one XOR written to partial[group], so
// the reads cannot be elided and the result can be checked.
#include "common.h"

namespace pesti {

constexpr int kReadGroups = PESTI_READ_GROUPS;
constexpr int kReadUnroll = 4;   // loads in flight per thread and iteration

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4a* __restrict__ p, int64_t n,
                                                               uint32_t* partial) {
  __shared__ uint32_t red[kWavesPerGroup];
  const int64_t stride = static_cast<int64_t>(kReadGroups) * kThreads;
  uint32_t acc = 0;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
    u32x4a v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += stride) {
    const u32x4a v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // XOR over the wave, then over the workgroup's waves.
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kWavesPerGroup; ++w) r ^= red[w];
    partial[blockIdx.x] = r;
  }
}

}  // namespace pesti

extern "C" int pesti_stream_read(const void* buf, int64_t bytes, uint32_t* partial, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return PESTI_ERR_SHAPE;
  if (!partial || (bytes > 0 && !buf)) return PESTI_ERR_NULL;
  if ((buf && !pesti_host::aligned(buf, 16)) || !pesti_host::aligned(partial, 4)) return PESTI_ERR_ALIGN;
  int dev = 0;
  size_t lds = 0;
  const int st = pesti_host::current_device(&dev, &lds);
  if (st != PESTI_OK) return st;
  const pesti::u32x4a* p = static_cast<const pesti::u32x4a*>(buf);
  int64_t n = bytes / 16;
  void* params[] = {&p, &n, &partial};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::stream_read_kernel),
                                       dim3(pesti::kReadGroups), dim3(pesti::kThreads), params, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}
