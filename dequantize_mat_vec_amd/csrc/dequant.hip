// Dequantization to float32 ("PESTI - Portable Execution Substrate for
// Transformer Inference", "What This Is": the page checks its unpacking of
// the K-family formats against a reference, to the byte).  One thread
// expands one 32-weight sub-block of one row and
// writes its float32 values; the mat-vec kernels never do this, the entry
// points exist so the unpacking itself can be checked bit for bit.
//
// Exactness in float32: binary16 d has 11 significant bits, so d*q (Q8_0),
// d*sc*(q-32) (Q6_K, |sc*(q-32)| <= 4096) and the two Q4_K / Q5_K terms
// d*sc*q and dmin*m are exact; their subtraction is the single rounding, and an FMA
// of the exact product with the exact negated min rounds the same way.
#include "common.h"

namespace pesti {

struct DequantArgs {
  const uint8_t* w;
  const float* scales;
  float* out;
  int64_t rows;
  int64_t in;
  int64_t row_bytes;
};

__device__ __forceinline__ float f16_at(const uint8_t* p) {
  const uint32_t bits = static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 8);
  return f16_lo(bits);
}

__global__ __launch_bounds__(256) void dequant_q8_0_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, j = t % nsub;
  const uint8_t* blk = a.w + row * a.row_bytes + j * 34;
  const float d = f16_at(blk);
  float* o = a.out + row * a.in + j * 32;
  for (int k = 0; k < 32; ++k) o[k] = d * static_cast<float>(static_cast<int8_t>(blk[2 + k]));
}

__global__ __launch_bounds__(256) void dequant_q4_k_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, j = t % nsub;
  const uint8_t* sb = a.w + row * a.row_bytes + (j / 8) * 144;
  const int s = static_cast<int>(j % 8);   // sub-block within the super-block
  const float d = f16_at(sb), dmin = f16_at(sb + 2);
  const uint8_t* S = sb + 4;
  uint32_t sc, m;
  if (s < 4) {
    sc = S[s] & 63u;
    m = S[s + 4] & 63u;
  } else {
    sc = (S[s + 4] & 15u) | ((S[s - 4] >> 6) << 4);
    m = (S[s + 4] >> 4) | ((S[s] >> 6) << 4);
  }
  const float dsc = d * static_cast<float>(sc);
  const float dmm = dmin * static_cast<float>(m);
  // sub-block s uses code bytes 32*(s/2) .. +31, low nibble when s is even
  const uint8_t* qs = sb + 16 + 32 * (s / 2);
  const int shift = (s & 1) ? 4 : 0;
  float* o = a.out + row * a.in + j * 32;
  for (int k = 0; k < 32; ++k) {
    const float q = static_cast<float>((qs[k] >> shift) & 15u);
    o[k] = fmaf(dsc, q, -dmm);
  }
}

// Q2_K: one thread per 32 weights = two 16-weight sub-blocks s, s + 1 of
// one j (weight 128h + 32j + 16c + l: bits 2j of code byte 32h + 16c + l,
// sub-block 8h + 2j + c).  d*sc*q and dmin*m are exact.
__global__ __launch_bounds__(256) void dequant_q2_k_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, jj = t % nsub;
  const uint8_t* sb = a.w + row * a.row_bytes + (jj / 8) * 84;
  const int g = static_cast<int>(jj % 8), h = g / 4, j = g % 4;   // weights 128h + 32j + [0, 32)
  const float d = f16_at(sb + 80), dmin = f16_at(sb + 82);
  float* o = a.out + row * a.in + jj * 32;
  for (int c = 0; c < 2; ++c) {
    const uint32_t sc = sb[8 * h + 2 * j + c];
    const float dsc = d * static_cast<float>(sc & 15u), dmm = dmin * static_cast<float>(sc >> 4);
    for (int l = 0; l < 16; ++l) {
      const uint32_t q = (sb[16 + 32 * h + 16 * c + l] >> (2 * j)) & 3u;
      o[16 * c + l] = fmaf(dsc, static_cast<float>(q), -dmm);
    }
  }
}

// Q3_K: as Q2_K's arrangement, the code minus 4 where its high bit (bit
// 4h + j of high-bit byte 16c + l) is clear, 6-bit scales minus 32.
// d*(scale - 32)*q needs at most 20 bits: exact.
__global__ __launch_bounds__(256) void dequant_q3_k_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, jj = t % nsub;
  const uint8_t* sb = a.w + row * a.row_bytes + (jj / 8) * 110;
  const int g = static_cast<int>(jj % 8), h = g / 4, j = g % 4;
  const float d = f16_at(sb + 108);
  const uint8_t* S = sb + 96;
  float* o = a.out + row * a.in + jj * 32;
  for (int c = 0; c < 2; ++c) {
    const int k = 8 * h + 2 * j + c;
    const int scale = static_cast<int>(((S[k % 8] >> (4 * (k / 8))) & 15u) |
                                       (((S[8 + k % 4] >> (2 * (k / 4))) & 3u) << 4)) - 32;
    const float ds = d * static_cast<float>(scale);
    for (int l = 0; l < 16; ++l) {
      const int low = (sb[32 + 32 * h + 16 * c + l] >> (2 * j)) & 3;
      const int high = (sb[16 * c + l] >> (4 * h + j)) & 1;
      o[16 * c + l] = ds * static_cast<float>(low - 4 * (1 - high));
    }
  }
}

// Q5_K: Q4_K's header and code runs, plus a fifth bit per weight: weight
// 64r + 32c + l takes bit 2r + c of high-bit byte l (bytes 16..47); the
// low-nibble runs start at byte 48.  d*sc*q (22 bits) and dmin*m are exact.
__global__ __launch_bounds__(256) void dequant_q5_k_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, j = t % nsub;
  const uint8_t* sb = a.w + row * a.row_bytes + (j / 8) * 176;
  const int s = static_cast<int>(j % 8);   // sub-block = 2 * run + half
  const float d = f16_at(sb), dmin = f16_at(sb + 2);
  const uint8_t* S = sb + 4;
  uint32_t sc, m;
  if (s < 4) {
    sc = S[s] & 63u;
    m = S[s + 4] & 63u;
  } else {
    sc = (S[s + 4] & 15u) | ((S[s - 4] >> 6) << 4);
    m = (S[s + 4] >> 4) | ((S[s] >> 6) << 4);
  }
  const float dsc = d * static_cast<float>(sc);
  const float dmm = dmin * static_cast<float>(m);
  const uint8_t* qh = sb + 16;
  const uint8_t* qs = sb + 48 + 32 * (s / 2);
  const int shift = (s & 1) ? 4 : 0;
  float* o = a.out + row * a.in + j * 32;
  for (int k = 0; k < 32; ++k) {
    const uint32_t q = ((qs[k] >> shift) & 15u) | (((qh[k] >> s) & 1u) << 4);
    o[k] = fmaf(dsc, static_cast<float>(q), -dmm);
  }
}

__global__ __launch_bounds__(256) void dequant_q6_k_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, j = t % nsub;
  const uint8_t* sb = a.w + row * a.row_bytes + (j / 8) * 210;
  const int s32 = static_cast<int>(j % 8);      // 32-weight group within the super-block
  const int h = s32 / 4, g = s32 % 4;           // weight i = 128h + 32g + l
  const uint8_t* ql = sb + 64 * h + 32 * (g % 2);
  const uint8_t* qh = sb + 128 + 32 * h;
  const int8_t* sc = reinterpret_cast<const int8_t*>(sb + 192);
  const float d = f16_at(sb + 208);
  float* o = a.out + row * a.in + j * 32;
  for (int l = 0; l < 32; ++l) {
    const uint32_t low = (g < 2) ? (ql[l] & 15u) : (ql[l] >> 4);
    const uint32_t high = (qh[l] >> (2 * g)) & 3u;
    const int q = static_cast<int>(low | (high << 4)) - 32;
    const float dsc = d * static_cast<float>(sc[(32 * s32 + l) / 16]);
    o[l] = dsc * static_cast<float>(q);
  }
}

__global__ __launch_bounds__(256) void dequant_i8row_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, j = t % nsub;
  const int8_t* q = reinterpret_cast<const int8_t*>(a.w + row * a.in + j * 32);
  const float s = a.scales[row];
  float* o = a.out + row * a.in + j * 32;
  for (int k = 0; k < 32; ++k) o[k] = s * static_cast<float>(q[k]);
}

// i4row: weight i of a row is nibble i % 2 (low first) of byte i / 2, a
// 4-bit two's complement code; the row is 32 bytes per 64 weights.
__global__ __launch_bounds__(256) void dequant_i4row_kernel(DequantArgs a) {
  const int64_t nsub = a.in / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.rows * nsub) return;
  const int64_t row = t / nsub, j = t % nsub;
  const uint8_t* q = a.w + row * a.row_bytes + j * 16;
  const float s = a.scales[row];
  float* o = a.out + row * a.in + j * 32;
  for (int k = 0; k < 16; ++k) {
    const int lo = static_cast<int>(q[k] & 15u), hi = static_cast<int>(q[k] >> 4);
    o[2 * k] = s * static_cast<float>(lo - ((lo & 8) << 1));
    o[2 * k + 1] = s * static_cast<float>(hi - ((hi & 8) << 1));
  }
}

}  // namespace pesti

namespace {

int dequant_launch(void (*kernel)(pesti::DequantArgs), int64_t rows, int64_t in, const void* w,
                   const float* scales, float* out, void* stream, int64_t row_bytes, bool need_scales) {
  if (rows < 0 || in < 0 || in % 32 != 0 || in > PESTI_MAX_IN_FEATURES) return PESTI_ERR_SHAPE;
  if (rows == 0 || in == 0) return PESTI_OK;
  if (!w || !out || (need_scales && !scales)) return PESTI_ERR_NULL;
  if (!pesti_host::aligned(w, 16) || !pesti_host::aligned(out, 16) ||
      (scales && !pesti_host::aligned(scales, 4)))
    return PESTI_ERR_ALIGN;
  int dev = 0;
  size_t lds = 0;
  int st = pesti_host::current_device(&dev, &lds);
  if (st != PESTI_OK) return st;
  pesti::DequantArgs a{static_cast<const uint8_t*>(w), scales, out, rows, in, row_bytes};
  const int64_t threads = rows * (in / 32);
  const unsigned grid = static_cast<unsigned>((threads + 255) / 256);
  void* params[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(256), params,
                                 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int pesti_dequant_q8_0(int64_t rows, int64_t in_features, const void* blocks, float* w_out,
                       void* stream) {
  return dequant_launch(pesti::dequant_q8_0_kernel, rows, in_features, blocks, nullptr, w_out, stream,
                        (in_features / 32) * 34, false);
}

int pesti_dequant_q4_k(int64_t rows, int64_t in_features, const void* blocks, float* w_out,
                       void* stream) {
  return dequant_launch(pesti::dequant_q4_k_kernel, rows, in_features, blocks, nullptr, w_out, stream,
                        ((in_features + 255) / 256) * 144, false);
}

// The stream layout is one long Q4_K row of ceil(rows * in / 256)
// super-blocks; its first rows * in weights, in order, are w_out [rows][in].
int pesti_dequant_q4_k_stream(int64_t rows, int64_t in_features, const void* blocks, float* w_out,
                              void* stream) {
  if (rows < 0 || in_features < 0 || in_features % 64 != 0 || in_features > PESTI_MAX_IN_FEATURES)
    return PESTI_ERR_SHAPE;
  if (rows == 0 || in_features == 0) return PESTI_OK;
  if (!blocks || !w_out) return PESTI_ERR_NULL;
  if (!pesti_host::aligned(blocks, 16) || !pesti_host::aligned(w_out, 16)) return PESTI_ERR_ALIGN;
  int dev = 0;
  size_t lds = 0;
  const int st = pesti_host::current_device(&dev, &lds);
  if (st != PESTI_OK) return st;
  const int64_t n = rows * in_features;
  pesti::DequantArgs a{static_cast<const uint8_t*>(blocks), nullptr, w_out, 1, n, (n + 255) / 256 * 144};
  const int64_t threads = n / 32;
  void* params[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::dequant_q4_k_kernel),
                                       dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), params,
                                       0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

int pesti_dequant_q2_k(int64_t rows, int64_t in_features, const void* blocks, float* w_out,
                       void* stream) {
  return dequant_launch(pesti::dequant_q2_k_kernel, rows, in_features, blocks, nullptr, w_out, stream,
                        ((in_features + 255) / 256) * 84, false);
}

int pesti_dequant_q3_k(int64_t rows, int64_t in_features, const void* blocks, float* w_out,
                       void* stream) {
  return dequant_launch(pesti::dequant_q3_k_kernel, rows, in_features, blocks, nullptr, w_out, stream,
                        ((in_features + 255) / 256) * 110, false);
}

int pesti_dequant_q5_k(int64_t rows, int64_t in_features, const void* blocks, float* w_out,
                       void* stream) {
  return dequant_launch(pesti::dequant_q5_k_kernel, rows, in_features, blocks, nullptr, w_out, stream,
                        ((in_features + 255) / 256) * 176, false);
}

int pesti_dequant_q6_k(int64_t rows, int64_t in_features, const void* blocks, float* w_out,
                       void* stream) {
  return dequant_launch(pesti::dequant_q6_k_kernel, rows, in_features, blocks, nullptr, w_out, stream,
                        ((in_features + 255) / 256) * 210, false);
}

int pesti_dequant_i8row(int64_t rows, int64_t in_features, const int8_t* codes,
                        const float* row_scales, float* w_out, void* stream) {
  return dequant_launch(pesti::dequant_i8row_kernel, rows, in_features, codes, row_scales, w_out,
                        stream, in_features, true);
}

int pesti_dequant_i4row(int64_t rows, int64_t in_features, const void* packed,
                        const float* row_scales, float* w_out, void* stream) {
  return dequant_launch(pesti::dequant_i4row_kernel, rows, in_features, packed, row_scales, w_out,
                        stream, ((in_features + 63) / 64) * 32, true);
}

}  // extern "C"
