// Host-only part of the C ABI: device check, packed row sizes, status text.
#include <atomic>
#include <cstring>

#include "common.h"

namespace {

constexpr int kMaxDevices = 64;
// Per device: 0 = unknown, 1 = gfx950, 2 = other.  Benign races only (every
// writer stores the same value).
std::atomic<int> g_arch[kMaxDevices];
std::atomic<size_t> g_lds[kMaxDevices];

}  // namespace

namespace pesti_host {

int current_device(int* device, size_t* lds_per_group) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PESTI_ERR_DEVICE;
  int known = g_arch[dev].load(std::memory_order_relaxed);
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PESTI_ERR_DEVICE;
    known = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_lds[dev].store(prop.sharedMemPerBlock, std::memory_order_relaxed);
    g_arch[dev].store(known, std::memory_order_relaxed);
  }
  if (known != 1) return PESTI_ERR_DEVICE;
  *device = dev;
  *lds_per_group = g_lds[dev].load(std::memory_order_relaxed);
  return PESTI_OK;
}

}  // namespace pesti_host

extern "C" {

int64_t pesti_row_bytes(int32_t format, int64_t in_features) {
  if (in_features < 0 || in_features % 32 != 0) return -1;
  switch (format) {
    case PESTI_FMT_Q8_0: return (in_features / 32) * 34;
    case PESTI_FMT_Q4_K: return ((in_features + 255) / 256) * 144;
    case PESTI_FMT_Q5_K: return ((in_features + 255) / 256) * 176;
    case PESTI_FMT_Q2_K: return ((in_features + 255) / 256) * 84;
    case PESTI_FMT_Q3_K: return ((in_features + 255) / 256) * 110;
    case PESTI_FMT_Q6_K: return ((in_features + 255) / 256) * 210;
    case PESTI_FMT_I8ROW: return in_features;
    case PESTI_FMT_I4ROW: return ((in_features + 63) / 64) * 32;
    default: return -1;   // PESTI_FMT_Q4_K_STREAM rows have no fixed size
  }
}

int64_t pesti_matrix_bytes(int32_t format, int64_t rows, int64_t in_features) {
  if (rows < 0) return -1;
  if (format == PESTI_FMT_Q4_K_STREAM) {
    if (in_features < 0 || in_features % 64 != 0) return -1;
    return (rows * in_features + 255) / 256 * 144;
  }
  const int64_t rb = pesti_row_bytes(format, in_features);
  return rb < 0 ? -1 : rows * rb;
}

const char* pesti_strerror(int status) {
  switch (status) {
    case PESTI_OK: return "success";
    case PESTI_ERR_NULL: return "a required pointer is NULL";
    case PESTI_ERR_SHAPE: return "unsupported shape (negative size, in_features not a multiple of 32, or too large)";
    case PESTI_ERR_BATCH: return "batch (or GEMM m) out of range";
    case PESTI_ERR_ALIGN: return "pointer not aligned (16 bytes for data, 4 for bias/scales)";
    case PESTI_ERR_LAUNCH: return "HIP kernel launch failed";
    case PESTI_ERR_DEVICE: return "current HIP device is missing or not gfx950";
    case PESTI_ERR_WORKSPACE: return "GEMM workspace missing or smaller than pesti_gemm_workspace_bytes";
    default: return "unknown status";
  }
}

int32_t pesti_abi_version(void) { return PESTI_ABI_VERSION; }

}  // extern "C"
