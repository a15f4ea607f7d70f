// Fused dequantize + mat-vec kernels for gfx950: y = W x + b with W in
// Q8_0, Q4_K, Q6_K or per-row int8, x and y in float32.
//
// The operation is the row-major matrix-vector product of a decode step and
// the fused dequantize + mat-vec that never expands weights to float32
// ("Project scaffold: modules, CLI, and correctness harness", file summaries
// of tensor.rs and quant.rs), over the K-family formats of "PESTI - Portable
// Execution Substrate for Transformer Inference" ("What This Is").  The
// block layouts are the GGUF ones (the pages name the formats only):
//   Q8_0  : d (binary16) | int8 q[32]                          w = d q
//   Q4_K  : d | dmin | 12 B scales/mins (6 bit) | 128 B nibbles w = d sc q - dmin m
//   Q6_K  : 128 B low nibbles | 64 B 2-bit highs | int8 sc[16] | d
//                                                             w = d sc (q - 32)
//   i8row : int8 q[out][in] + float32 scale[out]              w = s q
//
// Work decomposition (see common.h): L lanes per row, each lane walks the
// row's units with stride L.  A unit is:
//   Q8_0  one 34-byte block (32 weights);
//   Q4_K  one 64-weight run of a super-block: its 32 code bytes (low nibbles
//         = sub-block 2g, high nibbles = sub-block 2g+1) plus the 16-byte
//         super-block header;
//   Q6_K  16 consecutive positions l of one 128-weight half h, for all four
//         32-weight groups g (64 weights from 16+16 low-part bytes and 16
//         high-part bytes);
//   i8row 64 consecutive code bytes.
// Every lane keeps float32 partial sums per batch column; the sub-block
// scales are applied once per sub-block (d sc sum(q x) - dmin m sum(x) for
// Q4_K, with sum(x) per 32 staged in LDS next to x).
#include <type_traits>

#include "common.h"

namespace pesti {

struct GemvArgs {
  const uint8_t* w;       // packed rows
  const float* scales;    // i8row row scales (else null)
  const float* x;         // [batch][in]
  float* y;               // [batch][out]
  const float* bias;      // [out] or null
  int64_t out;
  int64_t in;
  int64_t row_bytes;
  int64_t units;          // units per row (loop bound)
  int64_t xpad;           // logical x length staged (zero filled past in)
  int64_t xstride;        // LDS floats per staged batch row
};

// ---------------------------------------------------------------------------
// Q8_0: one 34-byte block per unit.  Blocks start 2-byte aligned; the lane
// reads the dwords covering the block and realigns the codes in registers.
// ---------------------------------------------------------------------------
struct FmtQ8_0 {
  static constexpr bool kSums = false;
  static constexpr int kPad = 64;

  template <int B>
  __device__ __forceinline__ static void unit(const GemvArgs& a, const uint8_t* rp, int64_t u,
                                              const float* xs, const float*, int64_t, float* acc) {
    const uint8_t* p = rp + u * 34;
    const uint32_t s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);   // 0 or 2
    const uint8_t* pa = p - s;
    const u32x4 w0 = load_u32x4(pa);
    const u32x4 w1 = load_u32x4(pa + 16);
    // The ninth dword is whole only when s = 2; for s = 0 its upper half lies
    // past the block (and, for the last block, past the buffer), so only the
    // lower 16 bits are read.
    const uint32_t w8 = static_cast<uint32_t>(load_u16(pa + 32)) |
                        (s ? static_cast<uint32_t>(load_u16(pa + 34)) << 16 : 0u);
    const uint32_t w[9] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w8};
    const float d = s ? f16_hi(w[0]) : f16_lo(w[0]);
    float part[B];
#pragma unroll
    for (int b = 0; b < B; ++b) part[b] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = s ? w[j + 1] : align_bytes(w[j + 1], w[j], 2);
      const float q0 = sbyte<0>(c), q1 = sbyte<1>(c), q2 = sbyte<2>(c), q3 = sbyte<3>(c);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const f32x4 xv = xs4(xs + b * a.xstride, u * 32 + 4 * j);
        part[b] = fmaf(q0, xv.x, part[b]);
        part[b] = fmaf(q1, xv.y, part[b]);
        part[b] = fmaf(q2, xv.z, part[b]);
        part[b] = fmaf(q3, xv.w, part[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = fmaf(d, part[b], acc[b]);
  }

  __device__ static bool valid(const GemvArgs&, int64_t) { return true; }
};

// ---------------------------------------------------------------------------
// Q4_K: unit u = super-block u/4, run g = u%4.  g is fixed per lane (L is a
// multiple of 4), so the bit positions of its two scales and mins are
// computed once per lane.
// ---------------------------------------------------------------------------
struct Q4KLane {
  uint32_t lo_sc_shift0, lo_sc_shift1, lo_m_shift0, lo_m_shift1, lo_width;
  uint32_t hi_shift0, hi_shift1, hi_width;
  bool low_half;   // sub-blocks 0..3 (g < 2)
};

__device__ __forceinline__ Q4KLane q4k_lane(int g) {
  Q4KLane s;
  const int j0 = 2 * g, j1 = 2 * g + 1;
  s.low_half = g < 2;
  if (g < 2) {
    // sc[j] = S[j] & 63 and m[j] = S[j+4] & 63: byte j of dwords 1 and 2.
    s.lo_sc_shift0 = 8 * j0; s.lo_sc_shift1 = 8 * j1;
    s.lo_m_shift0 = 8 * j0;  s.lo_m_shift1 = 8 * j1;
    s.lo_width = 6; s.hi_width = 0; s.hi_shift0 = 0; s.hi_shift1 = 0;
  } else {
    // sc[j] = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
    // m[j]  = (S[j+4] >> 4) | (S[j] >> 6) << 4, with k = j - 4:
    // low parts in byte k of dword 3, high parts in bits 6-7 of byte k of
    // dwords 1 (scales) and 2 (mins).
    const int k0 = j0 - 4, k1 = j1 - 4;
    s.lo_sc_shift0 = 8 * k0; s.lo_sc_shift1 = 8 * k1;
    s.lo_m_shift0 = 8 * k0 + 4; s.lo_m_shift1 = 8 * k1 + 4;
    s.lo_width = 4; s.hi_width = 2; s.hi_shift0 = 8 * k0 + 6; s.hi_shift1 = 8 * k1 + 6;
  }
  return s;
}

struct FmtQ4_K {
  static constexpr bool kSums = true;
  static constexpr int kPad = 256;

  template <int B>
  __device__ __forceinline__ static void unit(const GemvArgs& a, const uint8_t* rp, int64_t u,
                                              const float* xs, const float* sums, int64_t nsub,
                                              float* acc, const Q4KLane& L) {
    const int64_t sb = u >> 2;
    const int g = static_cast<int>(u & 3);
    const uint8_t* sbp = rp + sb * 144;
    const u32x4 hdr = load_u32x4_a16(sbp);
    const u32x4 qa = load_u32x4_a16(sbp + 16 + 32 * g);
    const u32x4 qb = load_u32x4_a16(sbp + 32 + 32 * g);
    const float d = f16_lo(hdr.x), dmin = f16_hi(hdr.x);
    const uint32_t src_sc = L.low_half ? hdr.y : hdr.w;
    const uint32_t src_m = L.low_half ? hdr.z : hdr.w;
    const uint32_t sc0 = __builtin_amdgcn_ubfe(src_sc, L.lo_sc_shift0, L.lo_width) |
                         (__builtin_amdgcn_ubfe(hdr.y, L.hi_shift0, L.hi_width) << 4);
    const uint32_t sc1 = __builtin_amdgcn_ubfe(src_sc, L.lo_sc_shift1, L.lo_width) |
                         (__builtin_amdgcn_ubfe(hdr.y, L.hi_shift1, L.hi_width) << 4);
    const uint32_t m0 = __builtin_amdgcn_ubfe(src_m, L.lo_m_shift0, L.lo_width) |
                        (__builtin_amdgcn_ubfe(hdr.z, L.hi_shift0, L.hi_width) << 4);
    const uint32_t m1 = __builtin_amdgcn_ubfe(src_m, L.lo_m_shift1, L.lo_width) |
                        (__builtin_amdgcn_ubfe(hdr.z, L.hi_shift1, L.hi_width) << 4);
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    float p0[B], p1[B];
#pragma unroll
    for (int b = 0; b < B; ++b) { p0[b] = 0.f; p1[b] = 0.f; }
    const int64_t x0 = 64 * u;   // first weight of the run (sub-block 2g)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t lo = q[t] & 0x0F0F0F0Fu;
      const uint32_t hi = (q[t] >> 4) & 0x0F0F0F0Fu;
      const float l0 = ubyte<0>(lo), l1 = ubyte<1>(lo), l2 = ubyte<2>(lo), l3 = ubyte<3>(lo);
      const float h0 = ubyte<0>(hi), h1 = ubyte<1>(hi), h2 = ubyte<2>(hi), h3 = ubyte<3>(hi);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float* xb = xs + b * a.xstride;
        const f32x4 xl = xs4(xb, x0 + 4 * t);
        const f32x4 xh = xs4(xb, x0 + 32 + 4 * t);
        p0[b] = fmaf(l0, xl.x, p0[b]); p0[b] = fmaf(l1, xl.y, p0[b]);
        p0[b] = fmaf(l2, xl.z, p0[b]); p0[b] = fmaf(l3, xl.w, p0[b]);
        p1[b] = fmaf(h0, xh.x, p1[b]); p1[b] = fmaf(h1, xh.y, p1[b]);
        p1[b] = fmaf(h2, xh.z, p1[b]); p1[b] = fmaf(h3, xh.w, p1[b]);
      }
    }
    const float ds0 = d * static_cast<float>(sc0), ds1 = d * static_cast<float>(sc1);
    const float dm0 = dmin * static_cast<float>(m0), dm1 = dmin * static_cast<float>(m1);
    const int64_t j0 = 2 * u;    // sub-block index of the row (32 weights each)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float* sb_sums = sums + b * nsub;
      float r = ds0 * p0[b];
      r = fmaf(ds1, p1[b], r);
      r = fmaf(-dm0, sb_sums[j0], r);
      r = fmaf(-dm1, sb_sums[j0 + 1], r);
      acc[b] += r;
    }
  }
};

// ---------------------------------------------------------------------------
// Q6_K: unit u = super-block u/4, half h = (u/2)%2, column block c = u%2;
// it covers weights 128h + 32g + 16c + [0, 16) for g = 0..3.  Super-blocks
// are 210 bytes, so every other one starts 2 bytes past a dword boundary:
// the lane loads the covering dwords and realigns them.  Each code byte is
// rebuilt as the signed byte 4(q - 32) = 4*low + 64*(high - 2), exact, so
// one sign-extending convert yields it.
// ---------------------------------------------------------------------------
struct FmtQ6_K {
  static constexpr bool kSums = false;
  static constexpr int kPad = 256;

  __device__ __forceinline__ static void load16(const uint8_t* p, uint32_t s, uint32_t* out) {
    const u32x4 v = load_u32x4(p);
    const uint32_t e = load_u32(p + 16);
    out[0] = align_bytes(v.y, v.x, s);
    out[1] = align_bytes(v.z, v.y, s);
    out[2] = align_bytes(v.w, v.z, s);
    out[3] = align_bytes(e, v.w, s);
  }

  __device__ static bool valid(const GemvArgs& a, int64_t u) {
    return 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1) < a.in;
  }

  template <int B>
  __device__ __forceinline__ static void unit(const GemvArgs& a, const uint8_t* rp, int64_t u,
                                              const float* xs, const float*, int64_t, float* acc) {
    const int64_t sb = u >> 2;
    const int h = static_cast<int>((u >> 1) & 1);
    const int c = static_cast<int>(u & 1);
    const uint8_t* sbp = rp + sb * 210;
    const uint32_t s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sbp) & 3u);   // 0 or 2
    const uint8_t* base = sbp - s;
    uint32_t qla[4], qlb[4], qh[4];
    load16(base + 64 * h + 16 * c, s, qla);
    load16(base + 64 * h + 32 + 16 * c, s, qlb);
    load16(base + 128 + 32 * h + 16 * c, s, qh);
    // int8 scales sc[8h + 2g + c], g = 0..3: bytes c, c+2 of the realigned
    // dwords at offset 192 + 8h.  The third dword is only needed when s = 2;
    // for s = 0 it is re-read from in-bounds memory.
    const uint8_t* scp = base + 192 + 8 * h;
    const uint32_t s0 = load_u32(scp), s1 = load_u32(scp + 4), s2 = load_u32(scp + (s ? 8 : 4));
    const uint32_t S0 = align_bytes(s1, s0, s) >> (8 * c);
    const uint32_t S1 = align_bytes(s2, s1, s) >> (8 * c);
    const float sc[4] = {sbyte<0>(S0), sbyte<2>(S0), sbyte<0>(S1), sbyte<2>(S1)};
    const float dq = 0.25f * f16_lo(load_u16(sbp + 208));
    float p[4][B];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int b = 0; b < B; ++b) p[g][b] = 0.f;
    const int64_t xbase = 256 * sb + 128 * h + 16 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hf = qh[j] ^ 0xAAAAAAAAu;   // each 2-bit high part XOR 2
      uint32_t v[4];
      v[0] = ((qla[j] << 2) & 0x3C3C3C3Cu) | ((hf << 6) & 0xC0C0C0C0u);
      v[1] = ((qlb[j] << 2) & 0x3C3C3C3Cu) | ((hf << 4) & 0xC0C0C0C0u);
      v[2] = ((qla[j] >> 2) & 0x3C3C3C3Cu) | ((hf << 2) & 0xC0C0C0C0u);
      v[3] = ((qlb[j] >> 2) & 0x3C3C3C3Cu) | (hf & 0xC0C0C0C0u);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float q0 = sbyte<0>(v[g]), q1 = sbyte<1>(v[g]), q2 = sbyte<2>(v[g]), q3 = sbyte<3>(v[g]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const f32x4 xv = xs4(xs + b * a.xstride, xbase + 32 * g + 4 * j);
          p[g][b] = fmaf(q0, xv.x, p[g][b]);
          p[g][b] = fmaf(q1, xv.y, p[g][b]);
          p[g][b] = fmaf(q2, xv.z, p[g][b]);
          p[g][b] = fmaf(q3, xv.w, p[g][b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float r = (dq * sc[0]) * p[0][b];
      r = fmaf(dq * sc[1], p[1][b], r);
      r = fmaf(dq * sc[2], p[2][b], r);
      r = fmaf(dq * sc[3], p[3][b], r);
      acc[b] += r;
    }
  }
};

// ---------------------------------------------------------------------------
// i8row: 64 code bytes per unit; the row scale is applied after the sum.
// ---------------------------------------------------------------------------
struct FmtI8Row {
  static constexpr bool kSums = false;
  static constexpr int kPad = 64;

  __device__ static bool valid(const GemvArgs&, int64_t) { return true; }

  template <int B>
  __device__ __forceinline__ static void unit(const GemvArgs& a, const uint8_t* rp, int64_t u,
                                              const float* xs, const float*, int64_t, float* acc) {
    const uint8_t* p = rp + u * 64;
    uint32_t q[16];
    const bool full = 64 * u + 64 <= a.in;   // a 32-weight tail ends the row
    const u32x4 v0 = load_u32x4_a16(p), v1 = load_u32x4_a16(p + 16);
    u32x4 v2 = {0u, 0u, 0u, 0u}, v3 = {0u, 0u, 0u, 0u};
    if (full) { v2 = load_u32x4_a16(p + 32); v3 = load_u32x4_a16(p + 48); }
    q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
    q[4] = v1.x; q[5] = v1.y; q[6] = v1.z; q[7] = v1.w;
    q[8] = v2.x; q[9] = v2.y; q[10] = v2.z; q[11] = v2.w;
    q[12] = v3.x; q[13] = v3.y; q[14] = v3.z; q[15] = v3.w;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float q0 = sbyte<0>(q[t]), q1 = sbyte<1>(q[t]), q2 = sbyte<2>(q[t]), q3 = sbyte<3>(q[t]);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const f32x4 xv = xs4(xs + b * a.xstride, 64 * u + 4 * t);
        acc[b] = fmaf(q0, xv.x, acc[b]);
        acc[b] = fmaf(q1, xv.y, acc[b]);
        acc[b] = fmaf(q2, xv.z, acc[b]);
        acc[b] = fmaf(q3, xv.w, acc[b]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// The kernel: stage x (and Q4_K sub-block sums), then walk row tiles.
// ---------------------------------------------------------------------------
template <class F, int L, int B>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ float lds[];
  float* xs = lds;
  float* sums = lds + B * a.xstride;
  const int64_t nsub = a.xpad / 32;
  stage_x<B>(xs, a.x, a.in, a.xpad, a.xstride);
  if constexpr (F::kSums) {
    __syncthreads();
    // sum of x over each 32-weight sub-block, sequential within the block
    for (int64_t t = threadIdx.x; t < B * nsub; t += kThreads) {
      const int64_t b = t / nsub, j = t % nsub;
      const float* xb = xs + b * a.xstride;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const f32x4 v = xs4(xb, 32 * j + i);
        s += v.x; s += v.y; s += v.z; s += v.w;
      }
      sums[b * nsub + j] = s;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & (L - 1);
  const int grp = lane / L;
  constexpr int kRowsPerWave = kWave / L;
  constexpr int kRowsPerGroup = kWavesPerGroup * kRowsPerWave;

  [[maybe_unused]] Q4KLane q4l;
  if constexpr (F::kSums) q4l = q4k_lane(sub & 3);

  for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup; r0 < a.out;
       r0 += static_cast<int64_t>(gridDim.x) * kRowsPerGroup) {
    const int64_t row = r0 + wave * kRowsPerWave + grp;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    if (row < a.out) {
      const uint8_t* rp = a.w + row * a.row_bytes;
      for (int64_t u = sub; u < a.units; u += L) {
        if constexpr (F::kSums) {
          F::template unit<B>(a, rp, u, xs, sums, nsub, acc, q4l);
        } else {
          if (F::valid(a, u)) F::template unit<B>(a, rp, u, xs, sums, nsub, acc);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = group_sum<L>(acc[b]);
    if (sub == 0 && row < a.out) {
      const float bv = a.bias ? a.bias[row] : 0.f;
      const float rs = a.scales ? a.scales[row] : 1.f;
#pragma unroll
      for (int b = 0; b < B; ++b) a.y[b * a.out + row] = fmaf(acc[b], rs, bv);
    }
  }
}

}  // namespace pesti

// ---------------------------------------------------------------------------
// Host side: validation, batch chunking to fit LDS, dispatch on (L, B).
// ---------------------------------------------------------------------------
namespace {

using pesti::GemvArgs;

template <class F, int L, int B>
int launch_one(const GemvArgs& a, size_t lds_bytes, hipStream_t stream) {
  constexpr int kRowsPerGroup = pesti::kWavesPerGroup * (pesti::kWave / L);
  const int64_t tiles = (a.out + kRowsPerGroup - 1) / kRowsPerGroup;
  const unsigned grid = pesti_host::grid_for(tiles, 8192);
  GemvArgs args = a;
  void* params[] = {&args};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemv_kernel<F, L, B>),
                                 dim3(grid), dim3(pesti::kThreads), params, lds_bytes, stream);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <class F, int L>
int launch_b(const GemvArgs& a, int batch, size_t lds, hipStream_t st) {
  switch (batch) {
    case 1: return launch_one<F, L, 1>(a, lds, st);
    case 2: return launch_one<F, L, 2>(a, lds, st);
    case 3: return launch_one<F, L, 3>(a, lds, st);
    case 4: return launch_one<F, L, 4>(a, lds, st);
    case 5: return launch_one<F, L, 5>(a, lds, st);
    case 6: return launch_one<F, L, 6>(a, lds, st);
    case 7: return launch_one<F, L, 7>(a, lds, st);
    case 8: return launch_one<F, L, 8>(a, lds, st);
    default: return PESTI_ERR_BATCH;
  }
}

// Lanes per row: enough that a lane has few units, few enough that a
// workgroup covers several rows.
inline int lanes_for(int64_t units) {
  if (units <= 16) return 16;
  if (units <= 32) return 32;
  return 64;
}

template <class F>
int gemv_dispatch(int64_t out, int64_t in, const void* w, const float* scales, const float* x,
                  float* y, const float* bias, int32_t batch, void* stream, int64_t row_bytes,
                  int64_t units) {
  if (out < 0 || in < 0) return PESTI_ERR_SHAPE;
  if (batch < 0 || batch > PESTI_MAX_BATCH) return PESTI_ERR_BATCH;
  if (out == 0 || batch == 0) return PESTI_OK;
  if (in % 32 != 0 || in > PESTI_MAX_IN_FEATURES) return PESTI_ERR_SHAPE;
  if (!y || (in > 0 && (!w || !x))) return PESTI_ERR_NULL;
  if (scales == nullptr && std::is_same<F, pesti::FmtI8Row>::value && in > 0) return PESTI_ERR_NULL;
  if (!pesti_host::aligned(y, 16) || (w && !pesti_host::aligned(w, 16)) ||
      (x && !pesti_host::aligned(x, 16)) || (bias && !pesti_host::aligned(bias, 4)) ||
      (scales && !pesti_host::aligned(scales, 4)))
    return PESTI_ERR_ALIGN;
  int dev = 0;
  size_t lds_limit = 0;
  int st = pesti_host::current_device(&dev, &lds_limit);
  if (st != PESTI_OK) return st;

  GemvArgs a{};
  a.w = static_cast<const uint8_t*>(w);
  a.scales = scales;
  a.bias = bias;
  a.out = out;
  a.in = in;
  a.row_bytes = row_bytes;
  a.units = units;
  const int64_t pad = F::kPad;
  a.xpad = ((in + pad - 1) / pad) * pad;
  a.xstride = pesti::xs_stride(in, pad);
  const size_t row_lds = sizeof(float) * (a.xstride + (F::kSums ? a.xpad / 32 : 0));
  const int per_launch = pesti_host::batch_per_launch(lds_limit, row_lds, 0, batch);
  if (per_launch < 1) return PESTI_ERR_SHAPE;
  const int L = lanes_for(units);
  hipStream_t stream_h = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < batch; b0 += per_launch) {
    const int nb = batch - b0 < per_launch ? batch - b0 : per_launch;
    GemvArgs c = a;
    c.x = x ? x + static_cast<int64_t>(b0) * in : nullptr;
    c.y = y + static_cast<int64_t>(b0) * out;
    const size_t lds = row_lds * nb;
    int r;
    if (L == 16) r = launch_b<F, 16>(c, nb, lds, stream_h);
    else if (L == 32) r = launch_b<F, 32>(c, nb, lds, stream_h);
    else r = launch_b<F, 64>(c, nb, lds, stream_h);
    if (r != PESTI_OK) return r;
  }
  return PESTI_OK;
}

}  // namespace

extern "C" {

int pesti_gemv_q8_0(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const int64_t nb = in_features / 32;
  return gemv_dispatch<pesti::FmtQ8_0>(out_features, in_features, blocks, nullptr, x, y, bias, batch,
                                       stream, nb * 34, nb);
}

int pesti_gemv_q4_k(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const int64_t nsb = (in_features + 255) / 256;
  return gemv_dispatch<pesti::FmtQ4_K>(out_features, in_features, blocks, nullptr, x, y, bias, batch,
                                       stream, nsb * 144, (in_features + 63) / 64);
}

int pesti_gemv_q6_k(int64_t out_features, int64_t in_features, const void* blocks, const float* x,
                    float* y, const float* bias, int32_t batch, void* stream) {
  const int64_t nsb = (in_features + 255) / 256;
  return gemv_dispatch<pesti::FmtQ6_K>(out_features, in_features, blocks, nullptr, x, y, bias, batch,
                                       stream, nsb * 210, nsb * 4);
}

int pesti_gemv_i8row(int64_t out_features, int64_t in_features, const int8_t* codes,
                     const float* row_scales, const float* x, float* y, const float* bias,
                     int32_t batch, void* stream) {
  return gemv_dispatch<pesti::FmtI8Row>(out_features, in_features, codes, row_scales, x, y, bias,
                                        batch, stream, in_features, (in_features + 63) / 64);
}

}  // extern "C"
