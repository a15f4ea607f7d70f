// Shared device and host helpers of the gfx950 mat-vec kernels.
//
// Execution model used by every mat-vec kernel (one wavefront per row tile):
//   * a workgroup is 4 wavefronts of 64 lanes;
//   * a row is served by a group of L lanes (L = 16, 32 or 64), so a wave
//     holds 64/L rows at once; each lane walks the row's "units" (a fixed
//     run of packed bytes and the weights it encodes) with stride L;
//   * x is staged once per workgroup in LDS; weights stream from HBM
//     straight into registers and are decoded there, never written back;
//   * per-lane float32 partial sums are combined across the L lanes with
//     DPP row operations (plus one swizzle step per doubling beyond 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pesti.h"

namespace pesti {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWave * kWavesPerGroup;

// ---------------------------------------------------------------------------
// LDS layout of x: logical float i lives at phys(i) = i + 4 * (i / 64), i.e.
// every 64-float chunk is followed by 4 padding floats.  Lanes of a row group
// read 64-float chunks 64 floats apart; the padding puts consecutive chunks
// 16 bytes apart in bank space so their 16-byte reads do not collide.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int64_t xs_phys(int64_t i) { return i + 4 * (i >> 6); }

// Floats of LDS per staged batch row when the row is padded to `pad_to`.
__host__ __device__ constexpr int64_t xs_stride(int64_t in_features, int64_t pad_to) {
  return xs_phys(((in_features + pad_to - 1) / pad_to) * pad_to);
}

// Unaligned-safe vector types: global loads of these need only 4-byte
// alignment.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(16)));
typedef float f32x4 __attribute__((ext_vector_type(4), aligned(16)));

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load_u32x4_a16(const void* p) {
  return *reinterpret_cast<const u32x4a*>(p);
}
__device__ __forceinline__ uint32_t load_u32(const void* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ uint16_t load_u16(const void* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// binary16 bit pattern (low 16 bits) -> float32, exact (subnormals kept).
__device__ __forceinline__ float f16_lo(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}
__device__ __forceinline__ float f16_hi(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits >> 16)));
}

// Signed byte k of a dword as float32 (one SDWA sign-extending convert).
template <int K>
__device__ __forceinline__ float sbyte(uint32_t v) {
  return static_cast<float>(static_cast<int8_t>(v >> (8 * K)));
}
// Unsigned byte k of a dword as float32 (v_cvt_f32_ubyte{k}).
template <int K>
__device__ __forceinline__ float ubyte(uint32_t v) {
  return static_cast<float>((v >> (8 * K)) & 0xFFu);
}

// (hi:lo) >> (8 * shift) for shift in 0..3 (v_alignbyte_b32).
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t shift) {
  return __builtin_amdgcn_alignbyte(hi, lo, shift);
}

// ---------------------------------------------------------------------------
// Cross-lane sums within groups of L lanes; every lane of the group ends with
// the group's total.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "group of 4 to 64 lanes");
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (L >= 8) v += dpp<0x141>(v);    // row_half_mirror: lane i <-> 7 - i within 8
  if constexpr (L >= 16) v += dpp<0x140>(v);   // row_mirror: lane i <-> 15 - i within 16
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Stage x [batch][in] (float32, global) into LDS in the padded layout, zero
// filling logical columns in..padded_len-1.
// ---------------------------------------------------------------------------
template <int B>
__device__ __forceinline__ void stage_x(float* xs, const float* __restrict__ x, int64_t in_features,
                                        int64_t padded_len, int64_t stride) {
  // All loads of a chunk are issued before any LDS store, so a wide x costs
  // one memory round trip per chunk of kPer * kThreads float4 per batch
  // row, not one per float4 a thread stages.
  constexpr int kPer = 8;
  const int n4 = static_cast<int>(padded_len >> 2);   // float4 slots per batch row
  const int in4 = static_cast<int>(in_features >> 2);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const f32x4* src = reinterpret_cast<const f32x4*>(x + b * in_features);
    float* dst = xs + b * stride;
    for (int base = 0; base < n4; base += kPer * kThreads) {
      f32x4 v[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int s = base + r * kThreads + static_cast<int>(threadIdx.x);
        v[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s < in4) v[r] = src[s];
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int s = base + r * kThreads + static_cast<int>(threadIdx.x);
        if (s < n4) *reinterpret_cast<f32x4*>(dst + xs_phys(4 * s)) = v[r];
      }
    }
  }
}

// The code c nearest to dm / ds, the ratio of a sub-block's min term to
// its scale, if it lies in 0..cmax, else 0.  With it a weight is
// w = ds (q - c) + (ds c - dm): the matrix cores take the small integers
// q - c, and the remainder ds c - dm, computed in float32 once per
// sub-block, is exactly 0 when every weight of the sub-block is (q = c,
// ds c = dm), where taking ds q and dm apart would leave the rounding
// errors of two large sums.  The remainder is always exact in float32: it
// is a multiple of the smaller of d's and dmin's binary16 ulps, and for
// c >= 1 (dm >= ds / 2) its magnitude, at most ds / 2, is below 2^17 of
// those; so a one-hot x still yields each weight with a single rounding.
// v_rcp_f32 is within an ulp, so an integer ratio rounds to itself; ds = 0
// or a negative ratio gives c = 0.
__device__ __forceinline__ float nearest_code(float dm, float ds, float cmax) {
  const float r = rintf(dm * __builtin_amdgcn_rcpf(ds));
  return (r >= 0.f && r <= cmax) ? r : 0.f;   // false for NaN and infinity
}

// Row tile of workgroup b of a grid of n along x.  Workgroups go to the 8
// XCDs in turn (b % 8), and each XCD has its own L2: with tile = b,
// neighbouring tiles sit on different XCDs and a 128-byte line that two
// tiles share is fetched by both L2s.  With PESTI_XCD_TILES each XCD takes
// one contiguous run of tiles instead (XCD j: [start_j, start_j +
// count_j), the first n % 8 XCDs one more than the others; a bijection for
// every n).  Measured on the decode step, it cut the Q/K/V launch's reads
// from 730 to 665 KB and gate/up's from 5.07 to 5.00 MB, and made every
// mat-vec slower (step 371 -> 397 us, the down projections 3.9 -> 4.1 and
// 4.7 -> 4.9 us): the tiles stay in launch order by default.
#ifndef PESTI_XCD_TILES
#define PESTI_XCD_TILES 0
#endif
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t n) {
  if constexpr (PESTI_XCD_TILES == 0) {
    return b;
  } else {
    const int64_t xcd = b % kXcds, slot = b / kXcds;
    const int64_t per = n / kXcds, rem = n % kXcds;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  }
}

// Read 4 consecutive logical floats starting at logical index i (i % 4 == 0).
__device__ __forceinline__ f32x4 xs4(const float* xs, int64_t i) {
  return *reinterpret_cast<const f32x4*>(xs + xs_phys(i));
}

}  // namespace pesti

// ---------------------------------------------------------------------------
// Host-side helpers shared by the entry points.
// ---------------------------------------------------------------------------
namespace pesti_host {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Checks that the current device is gfx950 and reports its per-workgroup
// LDS limit.  Returns PESTI_OK or PESTI_ERR_DEVICE.
int current_device(int* device, size_t* lds_per_group);

// Small-M GEMMs on narrow layers (under 96 16-column tiles) with long rows
// (over 128 k-steps) leave most compute units idle: a workgroup per column
// tile and row tile of X.  There the K range is split over `splits`
// workgroups per tile, each writing its partial tile to a float32 workspace
// [splits][m][n], and a second launch sums the partials in split order and
// adds the bias.  At most 4 splits, so that about 256 workgroups run; the
// binary16 GEMM splits only single row tiles of X (it measured slower at
// two), and below m = 16 it runs on the vector ALUs, unsplit.
//
// Q3_K and Q6_K, whose K-split kernels are bound by their count of small W
// loads per workgroup, take two row tiles of X per workgroup when split
// (gemm_split_row_tiles), which halves the W loads at the same workgroup
// count; the other formats measured slower that way (Q8_0 too, once it read
// its blocks in pairs).
inline int gemm_split_row_tiles(int32_t format, int64_t m) {
  const bool pairs = format == PESTI_FMT_Q3_K || format == PESTI_FMT_Q6_K;
  return pairs && m > 16 ? 2 : 1;
}
inline int gemm_splits(int32_t format, int64_t m, int64_t n, int64_t k) {
  const int64_t tiles_n = (n + 15) / 16, tiles_m = (m + 15) / 16;
  if (m <= 0 || n <= 0 || tiles_n >= 96 || k / 32 <= 128) return 1;
  if (format == PESTI_FMT_F16 && (m < 16 || tiles_m > 1)) return 1;
  const int mt = gemm_split_row_tiles(format, m);
  const int64_t s = 256 / (tiles_n * ((tiles_m + mt - 1) / mt));
  return s >= 4 ? 4 : (s >= 2 ? static_cast<int>(s) : 1);
}

// The GEMM entry points behind the C ABI.  ws: nullptr, or a device buffer
// of gemm_splits(...) * m * n floats (16-byte aligned) for the split form.
int gemm_f16_run(int64_t m, int64_t n, int64_t k, const uint16_t* w, const uint16_t* x, float* y,
                 const float* bias, float* ws, hipStream_t st);
int gemm_quant_run(int32_t format, int64_t m, int64_t n, int64_t k, const void* blocks, const uint16_t* x,
                   float* y, const float* bias, float* ws, hipStream_t st);
// y[e] = sum over s < splits of part[s][e] (in order) + bias[e % n].
int launch_split_sum(int64_t m, int64_t n, const float* part, int splits, const float* bias, float* y,
                     hipStream_t st);

// Largest batch that fits LDS when one staged row takes `bytes_per_row`.
inline int batch_per_launch(size_t lds_limit, size_t bytes_per_row, size_t fixed_bytes, int batch) {
  if (bytes_per_row == 0) return batch;
  size_t room = lds_limit > fixed_bytes ? lds_limit - fixed_bytes : 0;
  size_t fit = room / bytes_per_row;
  return fit >= static_cast<size_t>(batch) ? batch : static_cast<int>(fit);
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

// Workgroups for a grid-stride kernel over `tiles` row tiles.
inline unsigned grid_for(int64_t tiles, int64_t cap) {
  int64_t g = tiles < cap ? tiles : cap;
  return static_cast<unsigned>(g < 1 ? 1 : g);
}

}  // namespace pesti_host
