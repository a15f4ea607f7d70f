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
//   Q8_0  two consecutive 34-byte blocks (68 bytes, 64 weights) when a row
//         has an even number of blocks, else one block;
//   Q4_K  one 64-weight run of a super-block: its 32 code bytes (low nibbles
//         = sub-block 2g, high nibbles = sub-block 2g+1) plus the 16-byte
//         super-block header;
//   Q6_K  16 consecutive positions l of one 128-weight half h, for all four
//         32-weight groups g (64 weights from 16+16 low-part bytes and 16
//         high-part bytes);
//   i8row 64 consecutive code bytes.
// Each unit is split into issue() - the global loads, returning raw dwords -
// and compute() - decode and FMA against x in LDS.  The kernel issues the
// loads of a lane's next unit before computing the current one, and issues
// the first unit's loads before staging x, so the weight stream overlaps
// both the x staging and the arithmetic.  Partial sums are float32 per
// batch column; sub-block scales are applied once per sub-block.
//
// One workgroup serves one tile of rows, and one launch may carry several
// independent mat-vecs of one format (a grouped launch, e.g. the Q/K/V or
// gate/up projections that read the same activations), which shortens a
// decode step's chain of dependent launches.
#pragma once

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
  int64_t units;          // units per row
  int64_t xpad;           // logical x length staged (zero filled past in)
  int64_t xstride;        // LDS floats per staged batch row
};

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four 4-bit codes (bits 0-3 of each byte of v) as float32 times 2^-9: a
// nibble in the low bits of an otherwise zero OCP e4m3 byte encodes exactly
// q * 2^-9 (subnormal for q < 8, exponent field 1 for q >= 8), and one
// v_cvt_pk_f32_fp8 converts two bytes.
__device__ __forceinline__ void nibbles_x512(uint32_t v, float& a, float& b, float& c, float& d) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v), false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v), true);
  a = lo.x; b = lo.y; c = hi.x; d = hi.y;
}

// ---------------------------------------------------------------------------
// Q8_0, two blocks per unit: the 68 bytes of blocks 2u, 2u+1 start on a
// dword boundary (rows are 34 * even bytes).  Block A = d in dword 0 low
// half, codes at bytes 2..33; block B = d in dword 8 high half, codes in
// dwords 9..16.
// ---------------------------------------------------------------------------
struct FmtQ8_0x2 {
  static constexpr bool kSums = false;
  static constexpr int kPad = 64;
  struct Raw { uint32_t w[17]; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }
  __device__ static bool valid(const GemvArgs&, int64_t) { return true; }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int64_t u, Raw& r) {
    const uint8_t* p = rp + u * 68;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = load_u32x4(p + 16 * i);
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
    r.w[16] = load_u32(p + 64);
  }

  template <int B>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw& r, int64_t u,
                                                 const float* xs, const float*, int64_t,
                                                 const Lane&, float* acc) {
    const float dA = f16_lo(r.w[0]), dB = f16_hi(r.w[8]);
    float pa[B], pb[B];
#pragma unroll
    for (int b = 0; b < B; ++b) { pa[b] = 0.f; pb[b] = 0.f; }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ca = align_bytes(r.w[j + 1], r.w[j], 2);
      const uint32_t cb = r.w[9 + j];
      const float a0 = sbyte<0>(ca), a1 = sbyte<1>(ca), a2 = sbyte<2>(ca), a3 = sbyte<3>(ca);
      const float b0 = sbyte<0>(cb), b1 = sbyte<1>(cb), b2 = sbyte<2>(cb), b3 = sbyte<3>(cb);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float* xb = xs + b * a.xstride;
        const f32x4 xa = xs4(xb, 64 * u + 4 * j);
        const f32x4 xc = xs4(xb, 64 * u + 32 + 4 * j);
        pa[b] = fmaf(a0, xa.x, pa[b]); pa[b] = fmaf(a1, xa.y, pa[b]);
        pa[b] = fmaf(a2, xa.z, pa[b]); pa[b] = fmaf(a3, xa.w, pa[b]);
        pb[b] = fmaf(b0, xc.x, pb[b]); pb[b] = fmaf(b1, xc.y, pb[b]);
        pb[b] = fmaf(b2, xc.z, pb[b]); pb[b] = fmaf(b3, xc.w, pb[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = fmaf(dB, pb[b], fmaf(dA, pa[b], acc[b]));
  }
};

// ---------------------------------------------------------------------------
// Q8_0, one block per unit (rows with an odd block count start 2 bytes off a
// dword boundary every other row): read the dwords covering the block and
// realign.  The ninth dword is whole only when the block starts 2 bytes
// past a boundary; otherwise only its lower half belongs to the block (and
// the upper half may lie past the buffer), so only 16 bits are read.
// ---------------------------------------------------------------------------
struct FmtQ8_0 {
  static constexpr bool kSums = false;
  static constexpr int kPad = 64;
  struct Raw { uint32_t w[9]; uint32_t s; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }
  __device__ static bool valid(const GemvArgs&, int64_t) { return true; }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int64_t u, Raw& r) {
    const uint8_t* p = rp + u * 34;
    const uint32_t s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);   // 0 or 2
    const uint8_t* pa = p - s;
    const u32x4 w0 = load_u32x4(pa);
    const u32x4 w1 = load_u32x4(pa + 16);
    r.w[0] = w0.x; r.w[1] = w0.y; r.w[2] = w0.z; r.w[3] = w0.w;
    r.w[4] = w1.x; r.w[5] = w1.y; r.w[6] = w1.z; r.w[7] = w1.w;
    r.w[8] = static_cast<uint32_t>(load_u16(pa + 32)) |
             (s ? static_cast<uint32_t>(load_u16(pa + 34)) << 16 : 0u);
    r.s = s;
  }

  template <int B>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw& r, int64_t u,
                                                 const float* xs, const float*, int64_t,
                                                 const Lane&, float* acc) {
    const float d = r.s ? f16_hi(r.w[0]) : f16_lo(r.w[0]);
    float part[B];
#pragma unroll
    for (int b = 0; b < B; ++b) part[b] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = r.s ? r.w[j + 1] : align_bytes(r.w[j + 1], r.w[j], 2);
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
};

// ---------------------------------------------------------------------------
// Q4_K: unit u = super-block u/4, run g = u%4.  g is fixed per lane (L is a
// multiple of 4), so the bit positions of its two scales and mins are
// computed once per lane.
// ---------------------------------------------------------------------------
struct FmtQ4_K {
  static constexpr bool kSums = true;
  static constexpr int kPad = 256;
  struct Raw { u32x4 hdr, qa, qb; };
  struct Lane {
    uint32_t lo_sc_shift0, lo_sc_shift1, lo_m_shift0, lo_m_shift1, lo_width;
    uint32_t hi_shift0, hi_shift1, hi_width;
    bool low_half;   // sub-blocks 0..3 (g < 2)
  };
  __device__ static bool valid(const GemvArgs&, int64_t) { return true; }

  __device__ static Lane lane_state(int sub) {
    const int g = sub & 3;
    Lane s;
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

  __device__ __forceinline__ static void issue(const uint8_t* rp, int64_t u, Raw& r) {
    const uint8_t* sbp = rp + (u >> 2) * 144;
    const int g = static_cast<int>(u & 3);
    r.hdr = load_u32x4_a16(sbp);
    r.qa = load_u32x4_a16(sbp + 16 + 32 * g);
    r.qb = load_u32x4_a16(sbp + 32 + 32 * g);
  }

  template <int B>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw& r, int64_t u,
                                                 const float* xs, const float* sums, int64_t nsub,
                                                 const Lane& L, float* acc) {
    const u32x4 hdr = r.hdr;
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
    const uint32_t q[8] = {r.qa.x, r.qa.y, r.qa.z, r.qa.w, r.qb.x, r.qb.y, r.qb.z, r.qb.w};
    float p0[B], p1[B];
#pragma unroll
    for (int b = 0; b < B; ++b) { p0[b] = 0.f; p1[b] = 0.f; }
    const int64_t x0 = 64 * u;   // first weight of the run (sub-block 2g)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float l0, l1, l2, l3, h0, h1, h2, h3;
      nibbles_x512(q[t] & 0x0F0F0F0Fu, l0, l1, l2, l3);
      nibbles_x512((q[t] >> 4) & 0x0F0F0F0Fu, h0, h1, h2, h3);
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
    // p0, p1 carry a factor 2^-9 from the code conversion: scale d by 2^9.
    const float d512 = d * 512.0f;
    const float ds0 = d512 * static_cast<float>(sc0), ds1 = d512 * static_cast<float>(sc1);
    const float dm0 = dmin * static_cast<float>(m0), dm1 = dmin * static_cast<float>(m1);
    const int64_t j0 = 2 * u;    // sub-block index of the row (32 weights each)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float* sb_sums = sums + b * nsub;
      float v = ds0 * p0[b];
      v = fmaf(ds1, p1[b], v);
      v = fmaf(-dm0, sb_sums[j0], v);
      v = fmaf(-dm1, sb_sums[j0 + 1], v);
      acc[b] += v;
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
  // Three 20-byte windows (low parts of g = 0/2, of g = 1/3, high parts),
  // three dwords around the unit's scales, and d.
  struct Raw { uint32_t la[5], lb[5], hh[5], sc[3]; uint32_t d; uint32_t s; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }

  __device__ static bool valid(const GemvArgs& a, int64_t u) {
    return 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1) < a.in;
  }

  __device__ __forceinline__ static void load20(const uint8_t* p, uint32_t* w) {
    const u32x4 v = load_u32x4(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    w[4] = load_u32(p + 16);
  }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int64_t u, Raw& r) {
    const int h = static_cast<int>((u >> 1) & 1);
    const int c = static_cast<int>(u & 1);
    const uint8_t* sbp = rp + (u >> 2) * 210;
    const uint32_t s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sbp) & 3u);   // 0 or 2
    const uint8_t* base = sbp - s;
    load20(base + 64 * h + 16 * c, r.la);
    load20(base + 64 * h + 32 + 16 * c, r.lb);
    load20(base + 128 + 32 * h + 16 * c, r.hh);
    // int8 scales sc[8h + 2g + c], g = 0..3, live in the 8 bytes at offset
    // 192 + 8h.  The third dword is needed only when s = 2; for s = 0 it is
    // re-read from in-bounds memory.
    const uint8_t* scp = base + 192 + 8 * h;
    r.sc[0] = load_u32(scp);
    r.sc[1] = load_u32(scp + 4);
    r.sc[2] = load_u32(scp + (s ? 8 : 4));
    r.d = load_u16(sbp + 208);
    r.s = s;
  }

  template <int B>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw& r, int64_t u,
                                                 const float* xs, const float*, int64_t,
                                                 const Lane&, float* acc) {
    const int h = static_cast<int>((u >> 1) & 1);
    const int c = static_cast<int>(u & 1);
    const uint32_t s = r.s;
    const uint32_t S0 = align_bytes(r.sc[1], r.sc[0], s) >> (8 * c);
    const uint32_t S1 = align_bytes(r.sc[2], r.sc[1], s) >> (8 * c);
    const float sc[4] = {sbyte<0>(S0), sbyte<2>(S0), sbyte<0>(S1), sbyte<2>(S1)};
    const float dq = 0.25f * f16_lo(r.d);
    float p[4][B];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int b = 0; b < B; ++b) p[g][b] = 0.f;
    const int64_t xbase = 256 * (u >> 2) + 128 * h + 16 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t la = align_bytes(r.la[j + 1], r.la[j], s);
      const uint32_t lb = align_bytes(r.lb[j + 1], r.lb[j], s);
      const uint32_t hf = align_bytes(r.hh[j + 1], r.hh[j], s) ^ 0xAAAAAAAAu;   // high part XOR 2
      uint32_t v[4];
      v[0] = ((la << 2) & 0x3C3C3C3Cu) | ((hf << 6) & 0xC0C0C0C0u);
      v[1] = ((lb << 2) & 0x3C3C3C3Cu) | ((hf << 4) & 0xC0C0C0C0u);
      v[2] = ((la >> 2) & 0x3C3C3C3Cu) | ((hf << 2) & 0xC0C0C0C0u);
      v[3] = ((lb >> 2) & 0x3C3C3C3Cu) | (hf & 0xC0C0C0C0u);
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
      float v = (dq * sc[0]) * p[0][b];
      v = fmaf(dq * sc[1], p[1][b], v);
      v = fmaf(dq * sc[2], p[2][b], v);
      v = fmaf(dq * sc[3], p[3][b], v);
      acc[b] += v;
    }
  }
};

// ---------------------------------------------------------------------------
// i8row: 64 code bytes per unit; the row scale is applied after the sum.  A
// row whose length is 32 mod 64 ends with a half unit.
// ---------------------------------------------------------------------------
struct FmtI8Row {
  static constexpr bool kSums = false;
  static constexpr int kPad = 64;
  struct Raw { uint32_t q[16]; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }
  __device__ static bool valid(const GemvArgs&, int64_t) { return true; }

  __device__ __forceinline__ static void issue_n(const uint8_t* rp, int64_t u, int64_t in, Raw& r) {
    const uint8_t* p = rp + u * 64;
    const u32x4 v0 = load_u32x4_a16(p), v1 = load_u32x4_a16(p + 16);
    u32x4 v2 = {0u, 0u, 0u, 0u}, v3 = {0u, 0u, 0u, 0u};
    if (64 * u + 64 <= in) { v2 = load_u32x4_a16(p + 32); v3 = load_u32x4_a16(p + 48); }
    r.q[0] = v0.x; r.q[1] = v0.y; r.q[2] = v0.z; r.q[3] = v0.w;
    r.q[4] = v1.x; r.q[5] = v1.y; r.q[6] = v1.z; r.q[7] = v1.w;
    r.q[8] = v2.x; r.q[9] = v2.y; r.q[10] = v2.z; r.q[11] = v2.w;
    r.q[12] = v3.x; r.q[13] = v3.y; r.q[14] = v3.z; r.q[15] = v3.w;
  }

  template <int B>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw& r, int64_t u,
                                                 const float* xs, const float*, int64_t,
                                                 const Lane&, float* acc) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t v = r.q[t];
      const float q0 = sbyte<0>(v), q1 = sbyte<1>(v), q2 = sbyte<2>(v), q3 = sbyte<3>(v);
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

template <class F>
__device__ __forceinline__ void issue_unit(const GemvArgs& a, const uint8_t* rp, int64_t u,
                                           typename F::Raw& r) {
  if constexpr (std::is_same<F, FmtI8Row>::value) {
    F::issue_n(rp, u, a.in, r);
  } else {
    F::issue(rp, u, r);
  }
}

// ---------------------------------------------------------------------------
// Staging: x into LDS (padded layout, zero past `in`), and for Q4_K the sum
// of every 32 consecutive x next to it.  A thread holds XS float4 at a time,
// all loaded before any is stored, so x costs one memory round trip per
// XS * kThreads float4 (XS = 1, 2 or 8 for rows of up to 1024, 2048 or 8192
// weights).  The per-32 sums reduce the 8 float4 of a sub-block, held by 8
// consecutive lanes, with DPP.  One barrier follows.
// ---------------------------------------------------------------------------
template <bool kSums, int B, int XS>
__device__ __forceinline__ void stage(const GemvArgs& a, float* xs, float* sums) {
  const int n4 = static_cast<int>(a.xpad >> 2);   // float4 slots per batch row
  const int in4 = static_cast<int>(a.in >> 2);
  const int nsub = static_cast<int>(a.xpad >> 5);
  const int tid = static_cast<int>(threadIdx.x);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.x + b * a.in);
    float* dst = xs + b * a.xstride;
    for (int base = 0; base < n4; base += XS * kThreads) {
      f32x4 v[XS];
#pragma unroll
      for (int r = 0; r < XS; ++r) {
        const int s = base + r * kThreads + tid;
        v[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s < in4) v[r] = src[s];
      }
#pragma unroll
      for (int r = 0; r < XS; ++r) {
        const int s = base + r * kThreads + tid;
        if (s < n4) *reinterpret_cast<f32x4*>(dst + xs_phys(4 * s)) = v[r];
        if constexpr (kSums) {
          float part = (v[r].x + v[r].y) + (v[r].z + v[r].w);
          part += dpp<0xB1>(part);    // lane ^ 1
          part += dpp<0x4E>(part);    // lane ^ 2
          part += dpp<0x141>(part);   // lane i <-> 7 - i within 8
          if ((tid & 7) == 0 && s < n4) sums[b * nsub + (s >> 3)] = part;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped launch: up to kMaxGroup independent mat-vecs of one format (and
// batch) in one grid: workgroup (x, y) serves tile x of op y; the grid is
// as wide as the op with the most tiles.
// ---------------------------------------------------------------------------
constexpr int kMaxGroup = PESTI_MAX_GROUP;

struct GroupArgs {
  GemvArgs op[kMaxGroup];
  int32_t n_ops;
};

// The kernel.  One workgroup = one tile of kRowsPerGroup rows of one op.
// A lane serves units sub + L*j, j = 0 .. ipt-1, in lock step with its wave
// (so the DPP reduction at the end sees a full wave).  When ipt <= U all of
// a lane's units are loaded at once, before x is staged: one memory round
// trip per launch.  Longer rows walk their units with the next unit's loads
// issued before the current one is computed.
template <class F, int L, int B, int U>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GroupArgs g) {
  extern __shared__ float lds[];
  constexpr int XS = L == 16 ? 1 : (L == 32 ? 2 : 8);
  constexpr int kRowsPerWave = kWave / L;
  constexpr int kRowsPerGroup = kWavesPerGroup * kRowsPerWave;

  // blockIdx.y picks the op, so the op's arguments are read in one round
  // trip without first scanning the group.
  const GemvArgs a = g.op[blockIdx.y];
  const int64_t tile = blockIdx.x;
  float* xs = lds;
  float* sums = lds + B * a.xstride;
  const int64_t nsub = a.xpad / 32;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & (L - 1);
  const int64_t row = tile * kRowsPerGroup + wave * kRowsPerWave + lane / L;
  const int64_t ipt = (a.units + L - 1) / L;
  const typename F::Lane ls = F::lane_state(sub);
  const bool row_live = row < a.out;
  const uint8_t* rp = a.w + (row_live ? row : 0) * a.row_bytes;

  auto live = [&](int64_t jj) {
    const int64_t u = sub + L * jj;
    return row_live && u < a.units && F::valid(a, u);
  };

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.f;

  // Rows of up to L units (every launch with L < 64) always take the first
  // path; only whole-wave rows can be longer than U units.
  if (L < 64 || ipt <= U) {
    typename F::Raw r[U];
    bool have[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      have[j] = j < ipt && live(j);
      if (have[j]) issue_unit<F>(a, rp, sub + L * j, r[j]);
    }
    if (tile * kRowsPerGroup >= a.out) return;   // this op has fewer tiles
    stage<F::kSums, B, XS>(a, xs, sums);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (have[j]) F::template compute<B>(a, r[j], sub + L * j, xs, sums, nsub, ls, acc);
  } else if constexpr (L == 64) {
    typename F::Raw cur;
    bool have = live(0);
    if (have) issue_unit<F>(a, rp, sub, cur);
    if (tile * kRowsPerGroup >= a.out) return;   // this op has fewer tiles
    stage<F::kSums, B, XS>(a, xs, sums);
    __syncthreads();
    for (int64_t j = 0; j < ipt; ++j) {
      typename F::Raw nxt;
      bool have_n = false;
      if (j + 1 < ipt) {
        have_n = live(j + 1);
        if (have_n) issue_unit<F>(a, rp, sub + L * (j + 1), nxt);
      }
      if (have) F::template compute<B>(a, cur, sub + L * j, xs, sums, nsub, ls, acc);
      cur = nxt;
      have = have_n;
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = group_sum<L>(acc[b]);
  if (sub == 0 && row_live) {
    const float bv = a.bias ? a.bias[row] : 0.f;
    const float rs = a.scales ? a.scales[row] : 1.f;
#pragma unroll
    for (int b = 0; b < B; ++b) a.y[b * a.out + row] = fmaf(acc[b], rs, bv);
  }
}

}  // namespace pesti

// ---------------------------------------------------------------------------
// Host side: validation, batch chunking to fit LDS, dispatch on (L, B).
// ---------------------------------------------------------------------------
namespace pesti_gemv {

using pesti::GemvArgs;
using pesti::GroupArgs;

template <class F, int L, int B, int U>
int launch_one(const GroupArgs& g, size_t lds_bytes, hipStream_t stream) {
  constexpr int64_t kRowsPerGroup = pesti::kWavesPerGroup * (pesti::kWave / L);
  int64_t tiles = 0;
  for (int i = 0; i < g.n_ops; ++i) {
    const int64_t t = (g.op[i].out + kRowsPerGroup - 1) / kRowsPerGroup;
    if (t > tiles) tiles = t;
  }
  if (tiles <= 0) return PESTI_OK;
  GroupArgs args = g;
  void* params[] = {&args};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemv_kernel<F, L, B, U>),
                                 dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(g.n_ops)),
                                 dim3(pesti::kThreads), params, lds_bytes, stream);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <class F, int L, int U>
int launch_b(const GroupArgs& g, int batch, size_t lds, hipStream_t st) {
  switch (batch) {
    case 1: return launch_one<F, L, 1, U>(g, lds, st);
    case 2: return launch_one<F, L, 2, U>(g, lds, st);
    case 3: return launch_one<F, L, 3, U>(g, lds, st);
    case 4: return launch_one<F, L, 4, U>(g, lds, st);
    case 5: return launch_one<F, L, 5, U>(g, lds, st);
    case 6: return launch_one<F, L, 6, U>(g, lds, st);
    case 7: return launch_one<F, L, 7, U>(g, lds, st);
    case 8: return launch_one<F, L, 8, U>(g, lds, st);
    default: return PESTI_ERR_BATCH;
  }
}

// (lanes per row L, units held per lane U) for the longest row of a launch:
// rows of up to 16 / 32 units take 16 / 32 lanes and one unit per lane;
// longer rows take a whole wave and hold 2 or 4 units per lane at once.
template <class F>
int launch_lu(const GroupArgs& g, int64_t max_units, int batch, size_t lds, hipStream_t st) {
  if (max_units <= 16) return launch_b<F, 16, 1>(g, batch, lds, st);
  if (max_units <= 32) return launch_b<F, 32, 1>(g, batch, lds, st);
  const int64_t ipt = (max_units + 63) / 64;
  if (ipt <= 1) return launch_b<F, 64, 1>(g, batch, lds, st);
  if (ipt <= 2) return launch_b<F, 64, 2>(g, batch, lds, st);
  return launch_b<F, 64, 4>(g, batch, lds, st);
}


// Format-specific packing: packed row bytes and units per row.
template <class F>
void shape_of(int64_t in, int64_t* row_bytes, int64_t* units);
template <> inline void shape_of<pesti::FmtQ8_0x2>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = (in / 32) * 34; *u = in / 64;
}
template <> inline void shape_of<pesti::FmtQ8_0>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = (in / 32) * 34; *u = in / 32;
}
template <> inline void shape_of<pesti::FmtQ4_K>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 255) / 256) * 144; *u = (in + 63) / 64;
}
template <> inline void shape_of<pesti::FmtQ6_K>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 255) / 256) * 210; *u = ((in + 255) / 256) * 4;
}
template <> inline void shape_of<pesti::FmtI8Row>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = in; *u = (in + 63) / 64;
}

// Validate one op; returns PESTI_OK, an error, or 1 for "empty, skip".
template <class F>
int check_op(const pesti_gemv_op& o, int32_t batch) {
  if (o.out_features < 0 || o.in_features < 0) return PESTI_ERR_SHAPE;
  if (o.out_features == 0 || batch == 0) return 1;
  if (o.in_features % 32 != 0 || o.in_features > PESTI_MAX_IN_FEATURES) return PESTI_ERR_SHAPE;
  const bool has_in = o.in_features > 0;
  if (!o.y || (has_in && (!o.w || !o.x))) return PESTI_ERR_NULL;
  if (std::is_same<F, pesti::FmtI8Row>::value && has_in && !o.row_scales) return PESTI_ERR_NULL;
  if (!pesti_host::aligned(o.y, 16) || (o.w && !pesti_host::aligned(o.w, 16)) ||
      (o.x && !pesti_host::aligned(o.x, 16)) || (o.bias && !pesti_host::aligned(o.bias, 4)) ||
      (o.row_scales && !pesti_host::aligned(o.row_scales, 4)))
    return PESTI_ERR_ALIGN;
  return PESTI_OK;
}

template <class F>
int group_dispatch(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream) {
  if (n_ops < 0 || n_ops > PESTI_MAX_GROUP) return PESTI_ERR_SHAPE;
  if (n_ops > 0 && !ops) return PESTI_ERR_NULL;
  if (batch < 0 || batch > PESTI_MAX_BATCH) return PESTI_ERR_BATCH;
  int live[PESTI_MAX_GROUP];
  int n_live = 0;
  for (int i = 0; i < n_ops; ++i) {
    const int st = check_op<F>(ops[i], batch);
    if (st < 0) return st;
    if (st == PESTI_OK) live[n_live++] = i;
  }
  if (n_live == 0) return PESTI_OK;
  int dev = 0;
  size_t lds_limit = 0;
  const int st = pesti_host::current_device(&dev, &lds_limit);
  if (st != PESTI_OK) return st;

  GroupArgs g{};
  int64_t max_units = 0;
  size_t row_lds = 0;
  for (int i = 0; i < n_live; ++i) {
    const pesti_gemv_op& o = ops[live[i]];
    GemvArgs& a = g.op[i];
    a.w = static_cast<const uint8_t*>(o.w);
    a.scales = o.row_scales;
    a.bias = o.bias;
    a.out = o.out_features;
    a.in = o.in_features;
    shape_of<F>(o.in_features, &a.row_bytes, &a.units);
    const int64_t pad = F::kPad;
    a.xpad = ((a.in + pad - 1) / pad) * pad;
    a.xstride = pesti::xs_stride(a.in, pad);
    const size_t r = sizeof(float) * (a.xstride + (F::kSums ? a.xpad / 32 : 0));
    if (r > row_lds) row_lds = r;
    if (a.units > max_units) max_units = a.units;
  }
  g.n_ops = n_live;
  const int per_launch = pesti_host::batch_per_launch(lds_limit, row_lds, 0, batch);
  if (per_launch < 1) return PESTI_ERR_SHAPE;
  hipStream_t stream_h = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < batch; b0 += per_launch) {
    const int nb = batch - b0 < per_launch ? batch - b0 : per_launch;
    GroupArgs c = g;
    for (int i = 0; i < n_live; ++i) {
      const pesti_gemv_op& o = ops[live[i]];
      c.op[i].x = o.x ? o.x + static_cast<int64_t>(b0) * o.in_features : nullptr;
      c.op[i].y = o.y + static_cast<int64_t>(b0) * o.out_features;
    }
    const size_t lds = row_lds * nb;
    const int r = launch_lu<F>(c, max_units, nb, lds, stream_h);
    if (r != PESTI_OK) return r;
  }
  return PESTI_OK;
}

inline pesti_gemv_op make_op(int64_t out, int64_t in, const void* w, const float* scales,
                             const float* x, float* y, const float* bias) {
  pesti_gemv_op o;
  o.out_features = out;
  o.in_features = in;
  o.w = w;
  o.row_scales = scales;
  o.x = x;
  o.y = y;
  o.bias = bias;
  return o;
}

}  // namespace pesti_gemv


namespace pesti_gemv {
// Grouped dispatch for one format, each defined in its own translation unit
// (gemv_<format>.hip) so the kernels of the four formats compile in parallel.
int group_q8_0(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_q4_k(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_q6_k(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_i8row(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
}  // namespace pesti_gemv
