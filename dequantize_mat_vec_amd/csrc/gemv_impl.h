// Fused dequantize + mat-vec kernels for gfx950: y = W x + b with W in
// Q8_0, Q2_K .. Q6_K, per-row int8 or per-row int4, x and y in float32.
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
//   i4row : 4-bit two's complement q, two per byte, rows padded to 64
//           weights, + float32 scale[out]                     w = s q
// (Q2_K, Q3_K and Q5_K are described beside their format structs.)
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
//   i8row 64 consecutive code bytes;
//   i4row 32 consecutive code bytes (64 weights).
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

#include <cstdint>
#include <type_traits>

#include "common.h"

namespace pesti {

struct GemvArgs {
  const uint8_t* w;       // packed rows
  const float* scales;    // i8row / i4row row scales (else null)
  const float* x;         // [batch][in]
  float* y;               // [batch][out]
  const float* bias;      // [out] or null
  int64_t out;
  int64_t in;
  int64_t row_bytes;
  int64_t units;          // units per row
  int64_t xpad;           // logical x length staged (zero filled past in)
  int64_t xstride;        // LDS floats per staged batch row
  const uint8_t* w2;      // paired launches: the up projection's rows
  const float* scales2;   // paired launches: its i8row / i4row row scales
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
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 64;
  struct Raw { uint32_t w[17]; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }
  __device__ static bool valid(const GemvArgs&, int) { return true; }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
    const uint8_t* p = rp + u * 68;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = load_u32x4(p + 16 * i);
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
    r.w[16] = load_u32(p + 64);
  }

  // r[0..R-1]: the same unit of R rows; acc[k * B + b] is row k, column b.
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane&, float* acc) {
    float pa[R][B], pb[R][B];
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int b = 0; b < B; ++b) { pa[k][b] = 0.f; pb[k][b] = 0.f; }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f32x4 xa[B], xc[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        xa[b] = xs4(xs + b * a.xstride, 64 * u + 4 * j);
        xc[b] = xs4(xs + b * a.xstride, 64 * u + 32 + 4 * j);
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t ca = align_bytes(r[k].w[j + 1], r[k].w[j], 2);
        const uint32_t cb = r[k].w[9 + j];
        const float a0 = sbyte<0>(ca), a1 = sbyte<1>(ca), a2 = sbyte<2>(ca), a3 = sbyte<3>(ca);
        const float b0 = sbyte<0>(cb), b1 = sbyte<1>(cb), b2 = sbyte<2>(cb), b3 = sbyte<3>(cb);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          pa[k][b] = fmaf(a0, xa[b].x, pa[k][b]); pa[k][b] = fmaf(a1, xa[b].y, pa[k][b]);
          pa[k][b] = fmaf(a2, xa[b].z, pa[k][b]); pa[k][b] = fmaf(a3, xa[b].w, pa[k][b]);
          pb[k][b] = fmaf(b0, xc[b].x, pb[k][b]); pb[k][b] = fmaf(b1, xc[b].y, pb[k][b]);
          pb[k][b] = fmaf(b2, xc[b].z, pb[k][b]); pb[k][b] = fmaf(b3, xc[b].w, pb[k][b]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float dA = f16_lo(r[k].w[0]), dB = f16_hi(r[k].w[8]);
#pragma unroll
      for (int b = 0; b < B; ++b)
        acc[k * B + b] = fmaf(dB, pb[k][b], fmaf(dA, pa[k][b], acc[k * B + b]));
    }
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
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 64;
  struct Raw { uint32_t w[9]; uint32_t s; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }
  __device__ static bool valid(const GemvArgs&, int) { return true; }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
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

  // The realignment s is per row: with an odd block count, consecutive rows
  // start on alternating dword phases.
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane&, float* acc) {
    float part[R][B];
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int b = 0; b < B; ++b) part[k][b] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f32x4 xv[B];
#pragma unroll
      for (int b = 0; b < B; ++b) xv[b] = xs4(xs + b * a.xstride, u * 32 + 4 * j);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t c = r[k].s ? r[k].w[j + 1] : align_bytes(r[k].w[j + 1], r[k].w[j], 2);
        const float q0 = sbyte<0>(c), q1 = sbyte<1>(c), q2 = sbyte<2>(c), q3 = sbyte<3>(c);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          part[k][b] = fmaf(q0, xv[b].x, part[k][b]);
          part[k][b] = fmaf(q1, xv[b].y, part[k][b]);
          part[k][b] = fmaf(q2, xv[b].z, part[k][b]);
          part[k][b] = fmaf(q3, xv[b].w, part[k][b]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float d = r[k].s ? f16_hi(r[k].w[0]) : f16_lo(r[k].w[0]);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[k * B + b] = fmaf(d, part[k][b], acc[k * B + b]);
    }
  }
};

// ---------------------------------------------------------------------------
// Q4_K: unit u = super-block u/4, run g = u%4.  g is fixed per lane (L is a
// multiple of 4), so the byte selectors that gather its two scales and
// mins are computed once per lane.
// ---------------------------------------------------------------------------
struct FmtQ4_K {
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 256;
  struct Raw { u32x4 hdr, qa, qb; };
  // Per lane (run g = sub % 4, sub-blocks 2g and 2g+1), byte selectors that
  // gather the unit's raw scale/min bytes, a = 2 * (g % 2):
  //   sel_yz: [S[a], S[a+1], S[a+4], S[a+5]]   (header dwords 1 and 2)
  //   sel_w:  [S[a+8], S[a+9], S[a+8], S[a+9]] (header dword 3)
  // For g < 2 the four 6-bit values (sc, sc, m, m) are the low 6 bits of
  // the first gather; for g >= 2 their low 4 bits come from the second
  // gather (low nibbles for sc, high nibbles for m) and their top 2 bits
  // from bits 6-7 of the first.
  struct Lane {
    uint32_t sel_yz, sel_w;
    bool high;   // g >= 2
  };
  __device__ static bool valid(const GemvArgs&, int) { return true; }

  __device__ static Lane lane_state(int sub) {
    const uint32_t a = 2u * (static_cast<uint32_t>(sub) & 1u);
    Lane s;
    // v_perm_b32 numbers the bytes of (src0:src1) 0-3 in src1, 4-7 in src0.
    s.sel_yz = (4u + a) | (5u + a) << 8 | a << 16 | (a + 1u) << 24;
    s.sel_w = a | (a + 1u) << 8 | a << 16 | (a + 1u) << 24;
    s.high = (sub & 2) != 0;
    return s;
  }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
    const uint8_t* sbp = rp + (u >> 2) * 144;
    const int g = static_cast<int>(u & 3);
    r.hdr = load_u32x4_a16(sbp);
    r.qa = load_u32x4_a16(sbp + 16 + 32 * g);
    r.qb = load_u32x4_a16(sbp + 32 + 32 * g);
  }

  // Code dword t (0..7) of the unit: bytes 4t..4t+3 of its 32-byte run.
  __device__ __forceinline__ static uint32_t code_word(const Raw& r, int t) {
    switch (t) {
      case 0: return r.qa.x;
      case 1: return r.qa.y;
      case 2: return r.qa.z;
      case 3: return r.qa.w;
      case 4: return r.qb.x;
      case 5: return r.qb.y;
      case 6: return r.qb.z;
      default: return r.qb.w;
    }
  }

  // Scale factors of the unit's two sub-blocks: d*sc (times 2^9, undoing the
  // code conversion's 2^-9) and dmin*m.
  __device__ __forceinline__ static void scales(const u32x4& hdr, const Lane& L, float& ds0,
                                                float& ds1, float& dm0, float& dm1) {
    const float d = f16_lo(hdr.x), dmin = f16_hi(hdr.x);
    const uint32_t p = __builtin_amdgcn_perm(hdr.y, hdr.z, L.sel_yz);   // [sc0 sc1 m0 m1] raw
    const uint32_t q = __builtin_amdgcn_perm(hdr.w, hdr.w, L.sel_w);
    const uint32_t lo4 = (q & 0x00000F0Fu) | ((q >> 4) & 0x0F0F0000u);
    const uint32_t hi = (lo4 | ((p >> 2) & 0x30303030u));
    const uint32_t v = L.high ? hi : (p & 0x3F3F3F3Fu);
    const float d512 = d * 512.0f;
    ds0 = d512 * ubyte<0>(v);
    ds1 = d512 * ubyte<1>(v);
    dm0 = dmin * ubyte<2>(v);
    dm1 = dmin * ubyte<3>(v);
  }

  // Every weight is dequantized on its own, w = d sc q - dmin m with one
  // rounding (the FMA of the exact d sc 2^9 and q 2^-9 against the exact
  // dmin m: the weight's float32 value, bit for bit), and then multiplied
  // into the sum.  Taking the two terms apart per sub-block (d sc sum q x -
  // dmin m sum x) would cost one FMA less per weight, but when d sc q and
  // dmin m nearly cancel the two large partial sums leave a rounding error
  // that is not bounded by sum |w x|.
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane& L, float* acc) {
    float ds0[R], ds1[R], ndm0[R], ndm1[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float dm0, dm1;
      scales(r[k].hdr, L, ds0[k], ds1[k], dm0, dm1);
      ndm0[k] = -dm0;
      ndm1[k] = -dm1;
    }
    const int x0 = 64 * u;   // first weight of the run (sub-block 2g)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4 xl[B], xh[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        xl[b] = xs4(xs + b * a.xstride, x0 + 4 * t);
        xh[b] = xs4(xs + b * a.xstride, x0 + 32 + 4 * t);
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t q = code_word(r[k], t);
        float l0, l1, l2, l3, h0, h1, h2, h3;
        nibbles_x512(q & 0x0F0F0F0Fu, l0, l1, l2, l3);
        nibbles_x512((q >> 4) & 0x0F0F0F0Fu, h0, h1, h2, h3);
        l0 = fmaf(ds0[k], l0, ndm0[k]); l1 = fmaf(ds0[k], l1, ndm0[k]);
        l2 = fmaf(ds0[k], l2, ndm0[k]); l3 = fmaf(ds0[k], l3, ndm0[k]);
        h0 = fmaf(ds1[k], h0, ndm1[k]); h1 = fmaf(ds1[k], h1, ndm1[k]);
        h2 = fmaf(ds1[k], h2, ndm1[k]); h3 = fmaf(ds1[k], h3, ndm1[k]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float& s = acc[k * B + b];
          s = fmaf(l0, xl[b].x, s); s = fmaf(l1, xl[b].y, s);
          s = fmaf(l2, xl[b].z, s); s = fmaf(l3, xl[b].w, s);
          s = fmaf(h0, xh[b].x, s); s = fmaf(h1, xh[b].y, s);
          s = fmaf(h2, xh[b].z, s); s = fmaf(h3, xh[b].w, s);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Q4_K in half units, for short rows at batch 1: unit u is half h = u % 2 of
// run r = u / 2 (super-block r / 4, run g = r % 4), i.e. code bytes
// 32g + 16h .. +15, whose low nibbles are weights 64r + 16h + [0, 16) of
// sub-block 2g and high nibbles weights 64r + 32 + 16h + [0, 16) of
// sub-block 2g + 1.  A 896-weight row is 28 half units on 32 lanes: each
// lane dequantizes and sums 32 weights instead of 64, which halves the
// arithmetic after a launch's one memory round trip (the decode step's
// launches are that short).  g = (u / 2) % 4 is fixed per lane (L is a
// multiple of 8), so the scale gather is FmtQ4_K's for lane sub / 2.
// ---------------------------------------------------------------------------
#ifndef PESTI_Q4K_HALF_UNITS
#define PESTI_Q4K_HALF_UNITS 1
#endif
constexpr bool kQ4KHalfUnits = PESTI_Q4K_HALF_UNITS != 0;
#ifndef PESTI_HALF_UNIT_MAX_ROWS
#define PESTI_HALF_UNIT_MAX_ROWS 2048
#endif
constexpr int64_t kHalfUnitMaxRows = PESTI_HALF_UNIT_MAX_ROWS;

struct FmtQ4_KH {
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 256;
  struct Raw { u32x4 hdr, q; };
  using Lane = FmtQ4_K::Lane;
  __device__ static Lane lane_state(int sub) { return FmtQ4_K::lane_state(sub >> 1); }
  __device__ static bool valid(const GemvArgs&, int) { return true; }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
    const uint8_t* sbp = rp + (u >> 3) * 144;
    r.hdr = load_u32x4_a16(sbp);
    r.q = load_u32x4_a16(sbp + 16 + 16 * (u & 7));   // 32g + 16h = 16 (u % 8)
  }

  // Each weight dequantized on its own (see FmtQ4_K::compute).
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane& L, float* acc) {
    float ds0[R], ds1[R], ndm0[R], ndm1[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float dm0, dm1;
      FmtQ4_K::scales(r[k].hdr, L, ds0[k], ds1[k], dm0, dm1);
      ndm0[k] = -dm0;
      ndm1[k] = -dm1;
    }
    const int x0 = 64 * (u >> 1) + 16 * (u & 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 xl[B], xh[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        xl[b] = xs4(xs + b * a.xstride, x0 + 4 * t);
        xh[b] = xs4(xs + b * a.xstride, x0 + 32 + 4 * t);
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t q = t == 0 ? r[k].q.x : (t == 1 ? r[k].q.y : (t == 2 ? r[k].q.z : r[k].q.w));
        float l0, l1, l2, l3, h0, h1, h2, h3;
        nibbles_x512(q & 0x0F0F0F0Fu, l0, l1, l2, l3);
        nibbles_x512((q >> 4) & 0x0F0F0F0Fu, h0, h1, h2, h3);
        l0 = fmaf(ds0[k], l0, ndm0[k]); l1 = fmaf(ds0[k], l1, ndm0[k]);
        l2 = fmaf(ds0[k], l2, ndm0[k]); l3 = fmaf(ds0[k], l3, ndm0[k]);
        h0 = fmaf(ds1[k], h0, ndm1[k]); h1 = fmaf(ds1[k], h1, ndm1[k]);
        h2 = fmaf(ds1[k], h2, ndm1[k]); h3 = fmaf(ds1[k], h3, ndm1[k]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float& s = acc[k * B + b];
          s = fmaf(l0, xl[b].x, s); s = fmaf(l1, xl[b].y, s);
          s = fmaf(l2, xl[b].z, s); s = fmaf(l3, xl[b].w, s);
          s = fmaf(h0, xh[b].x, s); s = fmaf(h1, xh[b].y, s);
          s = fmaf(h2, xh[b].z, s); s = fmaf(h3, xh[b].w, s);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Q4_K stream layout: the matrix's weights in row-major order cut into
// 256-weight super-blocks in order (only the last one padded), so a row of
// `in` weights (in % 64 == 0) starts at run R0 = row * in / 64 of the
// stream - super-block R0 / 4, run R0 % 4 - and a 896-weight row takes 504
// bytes instead of the row layout's 576.  Unit u of a row is stream run
// R0 + u: FmtQ4_K's unit, addressed from the row's first super-block with
// the row's phase R0 % 4 added (the lane's run, and so its scale gather, is
// (sub + phase) % 4).  Rows are handled one per lane group (all units of a
// lane group's rows then share one phase).
// ---------------------------------------------------------------------------
struct FmtQ4_KS {
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 64;
  using Raw = FmtQ4_K::Raw;
  struct Lane {
    FmtQ4_K::Lane k;
    int phase;
  };
  __device__ static bool valid(const GemvArgs&, int) { return true; }
  __device__ static Lane lane_state(int sub, const GemvArgs& a, int64_t row) {
    const int phase = static_cast<int>((row * (a.in >> 6)) & 3);
    return Lane{FmtQ4_K::lane_state((sub + phase) & 3), phase};
  }
  __device__ static const uint8_t* row_ptr(const GemvArgs& a, int64_t row) {
    return a.w + ((row * (a.in >> 6)) >> 2) * 144;
  }
  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, const Lane& L, Raw& r) {
    FmtQ4_K::issue(rp, u + L.phase, r);
  }
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane& L, float* acc) {
    FmtQ4_K::compute<B, R>(a, r, u, xs, L.k, acc);
  }
};

// The stream layout in half units, for rows of at most 1024 weights at
// batch 1 (as FmtQ4_KH for the row layout): half unit u of a row is stream
// half unit u + 2 * phase from the row's first super-block, and its scale
// gather is FmtQ4_K's for run ((sub / 2) + phase) % 4.
struct FmtQ4_KSH {
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 64;
  using Raw = FmtQ4_KH::Raw;
  using Lane = FmtQ4_KS::Lane;
  __device__ static bool valid(const GemvArgs&, int) { return true; }
  __device__ static Lane lane_state(int sub, const GemvArgs& a, int64_t row) {
    const int phase = static_cast<int>((row * (a.in >> 6)) & 3);
    return Lane{FmtQ4_K::lane_state(((sub >> 1) + phase) & 3), phase};
  }
  __device__ static const uint8_t* row_ptr(const GemvArgs& a, int64_t row) { return FmtQ4_KS::row_ptr(a, row); }
  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, const Lane& L, Raw& r) {
    FmtQ4_KH::issue(rp, u + 2 * L.phase, r);
  }
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane& L, float* acc) {
    FmtQ4_KH::compute<B, R>(a, r, u, xs, L.k, acc);
  }
};

template <class F>
constexpr bool kStreamLayout = std::is_same<F, FmtQ4_KS>::value || std::is_same<F, FmtQ4_KSH>::value;

// ---------------------------------------------------------------------------
// Q2_K and Q3_K share a unit: half h and column c of super-block u / 4
// (h = (u >> 1) & 1, c = u & 1), i.e. code bytes 32h + 16c .. +15 of the
// super-block, whose bits 2j, 2j+1 hold weights 128h + 32j + 16c + [0, 16)
// (16-weight sub-block 8h + 2j + c) for j = 0..3.  A row has
// 2 * ceil(in / 128) units, so every unit's super-block holds real weights
// (padding weights inside a unit meet x = 0).  u % 4 is the lane's sub % 4.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4u2 __attribute__((ext_vector_type(4), aligned(2)));

// Q2_K, 84-byte super-blocks: 16 scale bytes (4-bit scale, 4-bit min per
// sub-block), 64 code bytes, d, dmin.  w = d*sc*q - dmin*m with q in 0..3:
// the codes convert as e4m3 bytes (q * 2^-9, exact).
struct FmtQ2_K {
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 256;
  struct Raw { u32x4 q; uint32_t sc0, sc1, dd; };
  struct Lane { uint32_t h, c; };
  __device__ static bool valid(const GemvArgs&, int) { return true; }
  __device__ static Lane lane_state(int sub) {
    return Lane{static_cast<uint32_t>((sub >> 1) & 1), static_cast<uint32_t>(sub & 1)};
  }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
    const uint8_t* sbp = rp + (u >> 2) * 84;
    const int h = (u >> 1) & 1, c = u & 1;
    r.q = load_u32x4(sbp + 16 + 32 * h + 16 * c);
    r.sc0 = load_u32(sbp + 8 * h);       // scale bytes of sub-blocks 8h .. 8h+3
    r.sc1 = load_u32(sbp + 8 * h + 4);   // and 8h+4 .. 8h+7
    r.dd = load_u32(sbp + 80);           // d | dmin << 16
  }

  // Each weight dequantized on its own (see FmtQ4_K::compute): the 2-bit
  // code converts as q 2^-9, and w = (d sc 2^9) (q 2^-9) - dmin m is one
  // rounding of the exact value.
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane& L, float* acc) {
    const int x0 = 256 * (u >> 2) + 128 * static_cast<int>(L.h) + 16 * static_cast<int>(L.c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // scale byte of sub-block 8h + 2j + c: byte 2j + c of the lane's eight
      float ds[R], ndm[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t word = j < 2 ? r[k].sc0 : r[k].sc1;
        const uint32_t sbyte_v = (word >> (8 * (2 * (j & 1) + L.c))) & 0xFFu;
        ds[k] = f16_lo(r[k].dd) * 512.0f * static_cast<float>(sbyte_v & 15u);
        ndm[k] = -(f16_hi(r[k].dd) * static_cast<float>(sbyte_v >> 4));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 xv[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xv[b] = xs4(xs + b * a.xstride, x0 + 32 * j + 4 * t);
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const uint32_t w = t == 0 ? r[k].q.x : (t == 1 ? r[k].q.y : (t == 2 ? r[k].q.z : r[k].q.w));
          float q0, q1, q2, q3;
          nibbles_x512((w >> (2 * j)) & 0x03030303u, q0, q1, q2, q3);
          q0 = fmaf(ds[k], q0, ndm[k]); q1 = fmaf(ds[k], q1, ndm[k]);
          q2 = fmaf(ds[k], q2, ndm[k]); q3 = fmaf(ds[k], q3, ndm[k]);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            float& s = acc[k * B + b];
            s = fmaf(q0, xv[b].x, s); s = fmaf(q1, xv[b].y, s);
            s = fmaf(q2, xv[b].z, s); s = fmaf(q3, xv[b].w, s);
          }
        }
      }
    }
  }
};

// Q3_K, 110-byte super-blocks (2-byte aligned every other one): 32
// high-bit bytes, 64 low-bit bytes (the Q2_K arrangement), 12 scale bytes,
// d.  Weight 128h + 32j + 16c + l has its high bit at bit 4h + j of
// high-bit byte 16c + l; its code is the low two bits, minus 4 where the
// high bit is clear - as a signed byte, low2 | 0xFC where clear (-4..-1),
// converted with the signed-byte convert.  Scale k (6 bits, minus 32): bits
// 0-3 at bit 4(k / 8) of byte k % 8, bits 4-5 at bit 2(k / 4) of byte
// 8 + k % 4; w = d * (scale - 32) * q.
struct FmtQ3_K {
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 256;
  struct Raw { u32x4 q, hm; uint32_t s0, s1, s2, d; };
  using Lane = FmtQ2_K::Lane;
  __device__ static bool valid(const GemvArgs&, int) { return true; }
  __device__ static Lane lane_state(int sub) { return FmtQ2_K::lane_state(sub); }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
    const uint8_t* sbp = rp + (u >> 2) * 110;
    const int h = (u >> 1) & 1, c = u & 1;
    const u32x4u2 qv = *reinterpret_cast<const u32x4u2*>(sbp + 32 + 32 * h + 16 * c);
    const u32x4u2 hv = *reinterpret_cast<const u32x4u2*>(sbp + 16 * c);
    r.q = u32x4{qv.x, qv.y, qv.z, qv.w};
    r.hm = u32x4{hv.x, hv.y, hv.z, hv.w};
    typedef uint32_t u32a2 __attribute__((aligned(2)));
    r.s0 = *reinterpret_cast<const u32a2*>(sbp + 96);
    r.s1 = *reinterpret_cast<const u32a2*>(sbp + 100);
    r.s2 = *reinterpret_cast<const u32a2*>(sbp + 104);
    r.d = load_u16(sbp + 108);
  }

  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane& L, float* acc) {
    const int x0 = 256 * (u >> 2) + 128 * static_cast<int>(L.h) + 16 * static_cast<int>(L.c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hs = 4u * L.h + static_cast<uint32_t>(j);   // high-bit position
      float p[R][B];
#pragma unroll
      for (int k = 0; k < R; ++k)
#pragma unroll
        for (int b = 0; b < B; ++b) p[k][b] = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 xv[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xv[b] = xs4(xs + b * a.xstride, x0 + 32 * j + 4 * t);
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const uint32_t w = t == 0 ? r[k].q.x : (t == 1 ? r[k].q.y : (t == 2 ? r[k].q.z : r[k].q.w));
          const uint32_t hw = t == 0 ? r[k].hm.x : (t == 1 ? r[k].hm.y : (t == 2 ? r[k].hm.z : r[k].hm.w));
          const uint32_t low2 = (w >> (2 * j)) & 0x03030303u;
          const uint32_t clear = (~(hw >> hs)) & 0x01010101u;   // 1 where the high bit is clear
          const uint32_t qb = low2 | (clear * 0xFCu);            // signed bytes -4..3
          const float q0 = sbyte<0>(qb), q1 = sbyte<1>(qb), q2 = sbyte<2>(qb), q3 = sbyte<3>(qb);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            p[k][b] = fmaf(q0, xv[b].x, p[k][b]); p[k][b] = fmaf(q1, xv[b].y, p[k][b]);
            p[k][b] = fmaf(q2, xv[b].z, p[k][b]); p[k][b] = fmaf(q3, xv[b].w, p[k][b]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        // local scale index 8h + 2j + c: low bits in byte 2j + c (nibble h),
        // high bits in byte 8 + 2(j % 2) + c at bit 4h + 2(j / 2)
        const uint32_t lw = j < 2 ? r[k].s0 : r[k].s1;
        const uint32_t lo4 = (lw >> (8 * (2 * (j & 1) + L.c) + 4 * L.h)) & 15u;
        const uint32_t hi2 = (r[k].s2 >> (8 * (2 * (j & 1) + L.c) + 4 * L.h + 2 * (j >> 1))) & 3u;
        const float ds = f16_lo(r[k].d) * static_cast<float>(static_cast<int>(lo4 | (hi2 << 4)) - 32);
#pragma unroll
        for (int b = 0; b < B; ++b) acc[k * B + b] = fmaf(ds, p[k][b], acc[k * B + b]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Q5_K: Q4_K's units (run g = u % 4 of super-block u / 4: sub-blocks 2g and
// 2g+1) on 176-byte super-blocks whose codes have a fifth bit: weight
// 64g + 32c + l takes bit 2g + c of high-bit byte l (bytes 16..47, shared by
// the four runs); the runs' low nibbles start at byte 48.  Codes reach 31,
// past the e4m3 nibble trick, so they convert with v_cvt_f32_ubyte (exact);
// the scale gather is Q4_K's.
// ---------------------------------------------------------------------------
struct FmtQ5_K {
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 256;
  struct Raw { u32x4 hdr, ha, hb, qa, qb; };
  using Lane = FmtQ4_K::Lane;
  __device__ static bool valid(const GemvArgs&, int) { return true; }
  __device__ static Lane lane_state(int sub) { return FmtQ4_K::lane_state(sub); }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
    const uint8_t* sbp = rp + (u >> 2) * 176;
    const int g = static_cast<int>(u & 3);
    r.hdr = load_u32x4_a16(sbp);
    r.ha = load_u32x4_a16(sbp + 16);
    r.hb = load_u32x4_a16(sbp + 32);
    r.qa = load_u32x4_a16(sbp + 48 + 32 * g);
    r.qb = load_u32x4_a16(sbp + 64 + 32 * g);
  }

  __device__ __forceinline__ static uint32_t high_word(const Raw& r, int t) {
    switch (t) {
      case 0: return r.ha.x;
      case 1: return r.ha.y;
      case 2: return r.ha.z;
      case 3: return r.ha.w;
      case 4: return r.hb.x;
      case 5: return r.hb.y;
      case 6: return r.hb.z;
      default: return r.hb.w;
    }
  }
  __device__ __forceinline__ static uint32_t code_word(const Raw& r, int t) {
    switch (t) {
      case 0: return r.qa.x;
      case 1: return r.qa.y;
      case 2: return r.qa.z;
      case 3: return r.qa.w;
      case 4: return r.qb.x;
      case 5: return r.qb.y;
      case 6: return r.qb.z;
      default: return r.qb.w;
    }
  }

  // Each weight dequantized on its own (see FmtQ4_K::compute).
  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane& L, float* acc) {
    float ds0[R], ds1[R], ndm0[R], ndm1[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float dm0, dm1;
      FmtQ4_K::scales(r[k].hdr, L, ds0[k], ds1[k], dm0, dm1);   // d*sc*2^9: Q4_K's codes carry 2^-9
      ds0[k] *= 1.0f / 512.0f;
      ds1[k] *= 1.0f / 512.0f;
      ndm0[k] = -dm0;
      ndm1[k] = -dm1;
    }
    const int x0 = 64 * u;
    const uint32_t g2 = 2u * static_cast<uint32_t>(u & 3);   // fifth-bit position of the first half
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4 xl[B], xh[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        xl[b] = xs4(xs + b * a.xstride, x0 + 4 * t);
        xh[b] = xs4(xs + b * a.xstride, x0 + 32 + 4 * t);
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t q = code_word(r[k], t);
        const uint32_t hq = high_word(r[k], t);
        const uint32_t lo = (q & 0x0F0F0F0Fu) | (((hq >> g2) & 0x01010101u) << 4);
        const uint32_t hi = ((q >> 4) & 0x0F0F0F0Fu) | (((hq >> (g2 + 1u)) & 0x01010101u) << 4);
        const float l0 = fmaf(ds0[k], ubyte<0>(lo), ndm0[k]), l1 = fmaf(ds0[k], ubyte<1>(lo), ndm0[k]);
        const float l2 = fmaf(ds0[k], ubyte<2>(lo), ndm0[k]), l3 = fmaf(ds0[k], ubyte<3>(lo), ndm0[k]);
        const float h0 = fmaf(ds1[k], ubyte<0>(hi), ndm1[k]), h1 = fmaf(ds1[k], ubyte<1>(hi), ndm1[k]);
        const float h2 = fmaf(ds1[k], ubyte<2>(hi), ndm1[k]), h3 = fmaf(ds1[k], ubyte<3>(hi), ndm1[k]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float& s = acc[k * B + b];
          s = fmaf(l0, xl[b].x, s); s = fmaf(l1, xl[b].y, s);
          s = fmaf(l2, xl[b].z, s); s = fmaf(l3, xl[b].w, s);
          s = fmaf(h0, xh[b].x, s); s = fmaf(h1, xh[b].y, s);
          s = fmaf(h2, xh[b].z, s); s = fmaf(h3, xh[b].w, s);
        }
      }
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
  static constexpr bool kRowScales = false;
  static constexpr int kPad = 256;
  // Three 20-byte windows (low parts of g = 0/2, of g = 1/3, high parts),
  // three dwords around the unit's scales, and d.
  struct Raw { uint32_t la[5], lb[5], hh[5], sc[3]; uint32_t d; uint32_t s; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }

  __device__ static bool valid(const GemvArgs& a, int u) {
    return 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1) < a.in;
  }

  __device__ __forceinline__ static void load20(const uint8_t* p, uint32_t* w) {
    const u32x4 v = load_u32x4(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    w[4] = load_u32(p + 16);
  }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
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

  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane&, float* acc) {
    const int h = static_cast<int>((u >> 1) & 1);
    const int c = static_cast<int>(u & 1);
    float p[R][4][B];
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int b = 0; b < B; ++b) p[k][g][b] = 0.f;
    const int xbase = 256 * (u >> 2) + 128 * h + 16 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t v[R][4];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t s = r[k].s;
        const uint32_t la = align_bytes(r[k].la[j + 1], r[k].la[j], s);
        const uint32_t lb = align_bytes(r[k].lb[j + 1], r[k].lb[j], s);
        const uint32_t hf = align_bytes(r[k].hh[j + 1], r[k].hh[j], s) ^ 0xAAAAAAAAu;   // high part XOR 2
        v[k][0] = ((la << 2) & 0x3C3C3C3Cu) | ((hf << 6) & 0xC0C0C0C0u);
        v[k][1] = ((lb << 2) & 0x3C3C3C3Cu) | ((hf << 4) & 0xC0C0C0C0u);
        v[k][2] = ((la >> 2) & 0x3C3C3C3Cu) | ((hf << 2) & 0xC0C0C0C0u);
        v[k][3] = ((lb >> 2) & 0x3C3C3C3Cu) | (hf & 0xC0C0C0C0u);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 xv[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xv[b] = xs4(xs + b * a.xstride, xbase + 32 * g + 4 * j);
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const uint32_t w = v[k][g];
          const float q0 = sbyte<0>(w), q1 = sbyte<1>(w), q2 = sbyte<2>(w), q3 = sbyte<3>(w);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            p[k][g][b] = fmaf(q0, xv[b].x, p[k][g][b]);
            p[k][g][b] = fmaf(q1, xv[b].y, p[k][g][b]);
            p[k][g][b] = fmaf(q2, xv[b].z, p[k][g][b]);
            p[k][g][b] = fmaf(q3, xv[b].w, p[k][g][b]);
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const uint32_t s = r[k].s;
      const uint32_t S0 = align_bytes(r[k].sc[1], r[k].sc[0], s) >> (8 * c);
      const uint32_t S1 = align_bytes(r[k].sc[2], r[k].sc[1], s) >> (8 * c);
      const float sc[4] = {sbyte<0>(S0), sbyte<2>(S0), sbyte<0>(S1), sbyte<2>(S1)};
      const float dq = 0.25f * f16_lo(r[k].d);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float t = (dq * sc[0]) * p[k][0][b];
        t = fmaf(dq * sc[1], p[k][1][b], t);
        t = fmaf(dq * sc[2], p[k][2][b], t);
        t = fmaf(dq * sc[3], p[k][3][b], t);
        acc[k * B + b] += t;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// i8row: 64 code bytes per unit; the row scale is applied after the sum.  A
// row whose length is 32 mod 64 ends with a half unit.
// ---------------------------------------------------------------------------
struct FmtI8Row {
  static constexpr bool kRowScales = true;
  static constexpr int kPad = 64;
  struct Raw { uint32_t q[16]; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }
  __device__ static bool valid(const GemvArgs&, int) { return true; }

  __device__ __forceinline__ static void issue_n(const uint8_t* rp, int u, int64_t in, Raw& r) {
    const uint8_t* p = rp + u * 64;
    // A half unit (the last of a row 32 mod 64 long) re-reads its own first
    // half instead of the missing second half (loads stay branch-free) and
    // zeroes it.
    const bool full = 64 * u + 64 <= in;
    const uint8_t* p2 = full ? p + 32 : p;
    const u32x4 v0 = load_u32x4_a16(p), v1 = load_u32x4_a16(p + 16);
    u32x4 v2 = load_u32x4_a16(p2), v3 = load_u32x4_a16(p2 + 16);
    if (!full) { v2 = u32x4{0u, 0u, 0u, 0u}; v3 = u32x4{0u, 0u, 0u, 0u}; }
    r.q[0] = v0.x; r.q[1] = v0.y; r.q[2] = v0.z; r.q[3] = v0.w;
    r.q[4] = v1.x; r.q[5] = v1.y; r.q[6] = v1.z; r.q[7] = v1.w;
    r.q[8] = v2.x; r.q[9] = v2.y; r.q[10] = v2.z; r.q[11] = v2.w;
    r.q[12] = v3.x; r.q[13] = v3.y; r.q[14] = v3.z; r.q[15] = v3.w;
  }

  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane&, float* acc) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      f32x4 xv[B];
#pragma unroll
      for (int b = 0; b < B; ++b) xv[b] = xs4(xs + b * a.xstride, 64 * u + 4 * t);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t v = r[k].q[t];
        const float q0 = sbyte<0>(v), q1 = sbyte<1>(v), q2 = sbyte<2>(v), q3 = sbyte<3>(v);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float& s = acc[k * B + b];
          s = fmaf(q0, xv[b].x, s);
          s = fmaf(q1, xv[b].y, s);
          s = fmaf(q2, xv[b].z, s);
          s = fmaf(q3, xv[b].w, s);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// i4row: 32 code bytes per unit (64 weights; rows are padded to whole
// units).  Dword t of the unit holds weights 8t .. 8t+7, the even ones in
// the low nibbles.  A two's complement nibble moved to the top of an
// otherwise zero byte reads as the signed byte 16 q, so masking the high
// nibbles in place (odd weights) and shifting the low ones up by 4 (even
// weights) gives every code exactly through the sign-extending byte
// converts; the sum carries the factor 16, which the epilogue removes with
// an exact multiplication by 2^-4 before the row scale.
// ---------------------------------------------------------------------------
struct FmtI4Row {
  static constexpr bool kRowScales = true;
  static constexpr int kPad = 64;
  static constexpr float kAccScale = 0.0625f;
  struct Raw { u32x4 a, b; };
  struct Lane {};
  __device__ static Lane lane_state(int) { return {}; }
  __device__ static bool valid(const GemvArgs&, int) { return true; }

  __device__ __forceinline__ static void issue(const uint8_t* rp, int u, Raw& r) {
    const uint8_t* p = rp + u * 32;
    r.a = load_u32x4_a16(p);
    r.b = load_u32x4_a16(p + 16);
  }

  __device__ __forceinline__ static uint32_t word(const Raw& r, int t) {
    switch (t) {
      case 0: return r.a.x;
      case 1: return r.a.y;
      case 2: return r.a.z;
      case 3: return r.a.w;
      case 4: return r.b.x;
      case 5: return r.b.y;
      case 6: return r.b.z;
      default: return r.b.w;
    }
  }

  template <int B, int R>
  __device__ __forceinline__ static void compute(const GemvArgs& a, const Raw* r, int u,
                                                 const float* xs, const Lane&, float* acc) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4 xa[B], xb[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        xa[b] = xs4(xs + b * a.xstride, 64 * u + 8 * t);
        xb[b] = xs4(xs + b * a.xstride, 64 * u + 8 * t + 4);
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t v = word(r[k], t);
        const uint32_t ev = (v << 4) & 0xF0F0F0F0u;   // even weights, 16 q each
        const uint32_t od = v & 0xF0F0F0F0u;          // odd weights
        const float e0 = sbyte<0>(ev), e1 = sbyte<1>(ev), e2 = sbyte<2>(ev), e3 = sbyte<3>(ev);
        const float o0 = sbyte<0>(od), o1 = sbyte<1>(od), o2 = sbyte<2>(od), o3 = sbyte<3>(od);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float& s = acc[k * B + b];
          s = fmaf(e0, xa[b].x, s); s = fmaf(o0, xa[b].y, s);
          s = fmaf(e1, xa[b].z, s); s = fmaf(o1, xa[b].w, s);
          s = fmaf(e2, xb[b].x, s); s = fmaf(o2, xb[b].y, s);
          s = fmaf(e3, xb[b].z, s); s = fmaf(o3, xb[b].w, s);
        }
      }
    }
  }
};

// Factor the kernel epilogue applies to a finished row sum before the row
// scale and bias: 1 except where a format's codes enter scaled by a power
// of two.
template <class F, class = void>
struct AccScale { static constexpr float value = 1.0f; };
template <class F>
struct AccScale<F, std::void_t<decltype(F::kAccScale)>> { static constexpr float value = F::kAccScale; };

template <class F>
__device__ __forceinline__ void issue_unit(const GemvArgs& a, const uint8_t* rp, int u,
                                           const typename F::Lane& ls, typename F::Raw& r) {
  if constexpr (std::is_same<F, FmtI8Row>::value) {
    F::issue_n(rp, u, a.in, r);
  } else if constexpr (kStreamLayout<F>) {
    F::issue(rp, u, ls, r);
  } else {
    F::issue(rp, u, r);
  }
}

// ---------------------------------------------------------------------------
// Staging: x into LDS (padded layout, zero past `in`).  A thread holds XS
// float4 at a time, all loaded before any is stored, so x costs one memory
// round trip per XS * kThreads float4 (XS = 1, 2 or 8 for rows of up to
// 1024, 2048 or 8192 weights).  One barrier follows.
// ---------------------------------------------------------------------------
template <int B, int XS>
struct XChunk {
  f32x4 v[B][XS];
};

template <int B, int XS>
__device__ __forceinline__ void stage_load(const GemvArgs& a, int base, XChunk<B, XS>& c) {
  const int in4 = static_cast<int>(a.in >> 2);
  const int tid = static_cast<int>(threadIdx.x);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.x + b * a.in);
#pragma unroll
    for (int r = 0; r < XS; ++r) {
      const int s = base + r * kThreads + tid;
      // Branch-free: slot 0 stands in past the row, and stage_store zeroes
      // it there.  Selecting here would make the kernel wait for x before
      // the branch that issues the weight loads.
      c.v[b][r] = src[s < in4 ? s : 0];
    }
  }
}

template <int B, int XS>
__device__ __forceinline__ void stage_store(const GemvArgs& a, float* xs, int base, const XChunk<B, XS>& c) {
  const int n4 = static_cast<int>(a.xpad >> 2);   // float4 slots per batch row
  const int in4 = static_cast<int>(a.in >> 2);
  const int tid = static_cast<int>(threadIdx.x);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    float* dst = xs + b * a.xstride;
#pragma unroll
    for (int r = 0; r < XS; ++r) {
      const int s = base + r * kThreads + tid;
      const f32x4 v = s < in4 ? c.v[b][r] : f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < n4) *reinterpret_cast<f32x4*>(dst + xs_phys(4 * s)) = v;
    }
  }
}

// Chunks after the first (rows longer than 1024, 2048 or 8192 weights for
// XS = 1, 2, 8), one batch column at a time.
template <int B, int XS>
__device__ __forceinline__ void stage_rest(const GemvArgs& a, float* xs, int from) {
  const int n4 = static_cast<int>(a.xpad >> 2);
  for (int base = from; base < n4; base += XS * kThreads) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      GemvArgs ab = a;
      ab.x = a.x + b * a.in;
      XChunk<1, XS> c;
      stage_load<1, XS>(ab, base, c);
      stage_store<1, XS>(ab, xs + b * a.xstride, base, c);
    }
  }
}

// Whether a kernel loads its first x chunk ahead of its weights: when the
// chunk is small (the registers it holds stay live across the weight
// loads), and always at batch 1, where even a whole-wave row's 8 float4
// per thread pay for themselves (the down projection of a decode step is
// short, so x's L2 round trip otherwise adds to every launch).
template <int B, int XS>
constexpr bool kEarlyX = (XS <= 2 && XS * B <= 8) || B == 1;

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

// The kernel.  One workgroup = one tile of kRowsPerTile rows of one op.
// A group of L lanes serves R rows, kRowsPerSlab apart, with one lane
// layout: lane `sub` holds units sub + L*j, j = 0 .. ipt-1, of every one of
// the R rows, so each x value it reads from LDS feeds R rows.  Lanes walk
// in lock step with their wave (the DPP reduction at the end sees a full
// wave).  When ipt <= U all of a lane's units are loaded at once, before x
// is staged: one memory round trip per launch.  Longer rows (whole-wave
// lane groups only) walk their units with the next unit's loads issued
// before the current one is computed.  Rows past the op's end read the
// tile's first row (in bounds) and are not stored.
//
// Paired launches (P) compute row r of W (the gate projection) and row r of
// w2 (the up projection) together and write silu(gate) * up with silu(g) =
// g * sigmoid(g) ("PESTI ..." README, "Conformance": SwiGLU with the
// sigmoid-based SiLU), so the feed-forward input never leaves registers
// between the two products.  With 16 or 32 lanes per row (R = 1) adjacent
// lane groups of a wave take the gate and the up row, one exchange across
// the pair joins their sums, and a tile keeps the unpaired launch's lanes
// per row; whole-wave rows (R = 2) hold both rows in one lane group.
template <int L, int R, bool P>
constexpr int kTileRows = P ? (R == 1 ? kWavesPerGroup * (kWave / L) / 2 : kWavesPerGroup * (kWave / L))
                            : kWavesPerGroup * (kWave / L) * R;

template <class F, int L, int B, int U, int R, bool P = false>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GroupArgs g) {
  extern __shared__ float lds[];
  constexpr int XS = L <= 16 ? 1 : (L == 32 ? 2 : 8);
  constexpr int kRowsPerWave = kWave / L;
  constexpr int kRowsPerSlab = kWavesPerGroup * kRowsPerWave;
  constexpr int kRowsPerTile = kTileRows<L, R, P>;
  static_assert(R == 1 || L < 64 || U == 1, "several rows per lane group need short rows");
  static_assert(!P || (R == 1 && L < 64) || R == 2, "paired rows: lane-group pairs or two rows per group");
  static_assert(!kStreamLayout<F> || (R == 1 && !P), "stream rows: one row per lane group, unpaired");

  // blockIdx.y picks the op, so the op's arguments are read without first
  // scanning the group.  All of its fields are loaded before the first
  // branch: left to itself the compiler sinks each scalar load to its
  // first use behind the branches below, which costs a kernel-argument
  // round trip per branch before the first weight load is issued.
  const GemvArgs a = g.op[blockIdx.y];
  asm volatile("" ::"s"(a.w), "s"(a.scales), "s"(a.x), "s"(a.y), "s"(a.bias), "s"(a.out), "s"(a.in),
               "s"(a.row_bytes), "s"(a.units), "s"(a.xpad), "s"(a.xstride));
  if constexpr (P) asm volatile("" ::"s"(a.w2), "s"(a.scales2));
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t first = tile * kRowsPerTile;
  if (first >= a.out) return;   // this op has fewer tiles (uniform)
  float* xs = lds;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & (L - 1);
  const int rofs = wave * kRowsPerWave + lane / L;   // row within a slab
  const int ipt = static_cast<int>((a.units + L - 1) / L);
  // Row k of the lane sits rofs + k * kRowsPerSlab rows past the tile's
  // first row; rows past the end read the first row instead.  Offsets
  // within a tile fit 24 bits (at most 256 rows of at most 34816 bytes).
  const uint8_t* tile_base = a.w + first * a.row_bytes;
  const int64_t left = a.out - first;
  const typename F::Lane ls = [&]() {
    if constexpr (kStreamLayout<F>) return F::lane_state(sub, a, first + (rofs < left ? rofs : 0));
    else return F::lane_state(sub);
  }();
  const uint8_t* rp[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if constexpr (kStreamLayout<F>) {   // one row per lane group (R = 1)
      rp[k] = F::row_ptr(a, first + (rofs < left ? rofs : 0));
    } else if constexpr (P && R == 1) {   // even lane groups: gate row rofs / 2; odd: up row
      const int pr = rofs >> 1;
      const uint8_t* base = ((rofs & 1) ? a.w2 : a.w) + first * a.row_bytes;
      rp[k] = base + (pr < left ? __umul24(static_cast<uint32_t>(pr),
                                           static_cast<uint32_t>(a.row_bytes)) : 0u);
    } else if constexpr (P) {   // row rofs of the gate (k = 0) and up (k = 1) rows
      const uint8_t* base = (k == 0 ? a.w : a.w2) + first * a.row_bytes;
      rp[k] = base + (rofs < left ? __umul24(static_cast<uint32_t>(rofs),
                                             static_cast<uint32_t>(a.row_bytes)) : 0u);
    } else {
      const int r = rofs + k * kRowsPerSlab;
      rp[k] = tile_base + (r < left ? __umul24(static_cast<uint32_t>(r),
                                                static_cast<uint32_t>(a.row_bytes)) : 0u);
    }
  }

  auto live = [&](int jj) {
    const int u = sub + L * jj;
    return u < a.units && F::valid(a, u);
  };

  float acc[R * B];
#pragma unroll
  for (int i = 0; i < R * B; ++i) acc[i] = 0.f;

  // x is loaded before the weights: vector loads retire in order, so x can
  // reach LDS (and the barrier pass) while the weights are still in flight.
  constexpr bool kEarly = kEarlyX<B, XS>;
  XChunk<kEarly ? B : 1, XS> xc;
  if constexpr (kEarly) stage_load<B, XS>(a, 0, xc);
  // A lane's unit j (j < ipt): sub + L*j when it exists, else unit 0 of the
  // same row as an in-bounds stand-in (loads stay branch-free).
  auto unit = [&](int j) { return (j < ipt && live(j)) ? sub + L * j : 0; };
  // The epilogue's per-row operands (bias, row scales) are loaded with the
  // weights, not after the reduction, where they would add a memory round
  // trip to the end of the launch.  Each lane loads those of the row it may
  // store (row `sub` of its R, or the pair's gate row); absent operands and
  // rows past the end read a stand-in inside the lane's weight row (loads
  // stay branch-free), and the value is not used.
  float ep[3] = {0.f, 0.f, 0.f};
  auto epilogue_loads = [&]() {
    int er;
    if constexpr (P && R == 1) er = rofs >> 1;
    else if constexpr (P) er = rofs;
    else er = rofs + (sub < R ? sub : 0) * kRowsPerSlab;
    const bool in_rows = er < left;
    const float* stand_in = reinterpret_cast<const float*>(tile_base);   // 4-byte aligned
    const int64_t row = first + er;
    ep[0] = *((a.bias && in_rows) ? a.bias + row : stand_in);
    ep[1] = *((a.scales && in_rows) ? a.scales + row : stand_in);
    ep[2] = P ? *((a.scales2 && in_rows) ? a.scales2 + row : stand_in) : 0.f;
  };
  // Rows of more than U units exist only for whole-wave lane groups (16
  // and 32 lanes per row always hold all units at once); such a lane walks
  // its units with two register buffers.  Both paths issue their first
  // weight loads in their own branch and then share the x staging, so no
  // use of x can be hoisted above the weight loads (which would make the
  // launch wait for x before asking for its weights).
  constexpr bool kWalk = R == 1 && L == 64;
  const bool at_once = !kWalk || ipt <= U;
  typename F::Raw r[U][R];
  typename F::Raw rb[1];   // the walk's second buffer
  bool have[U];
  if (at_once) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      // Every lane loads (lanes without a unit load unit 0 of their row, in
      // bounds): branch-free loads keep the in-order load count exact, so
      // the x stores below wait for x alone.
      have[j] = j < ipt && live(j);
#pragma unroll
      for (int k = 0; k < R; ++k) issue_unit<F>(a, rp[k], unit(j), ls, r[j][k]);
    }
  } else if constexpr (kWalk) {
    issue_unit<F>(a, rp[0], unit(0), ls, r[0][0]);
    issue_unit<F>(a, rp[0], unit(1), ls, rb[0]);
  }
  epilogue_loads();
  if constexpr (kEarly) stage_store<B, XS>(a, xs, 0, xc);
  stage_rest<B, XS>(a, xs, kEarly ? XS * kThreads : 0);
  __syncthreads();
  if (at_once) {
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (have[j]) F::template compute<B, R>(a, r[j], sub + L * j, xs, ls, acc);
  } else if constexpr (kWalk) {
    // Two units in flight: unit j + 2 is requested as soon as unit j's
    // registers are free.  Requests past the last unit read unit 0 (in
    // bounds, unused), which keeps the loop branch-free.
    for (int j = 0; j < ipt; j += 2) {
      if (live(j)) F::template compute<B, 1>(a, r[0], sub + L * j, xs, ls, acc);
      if (j + 1 >= ipt) break;
      issue_unit<F>(a, rp[0], unit(j + 2), ls, r[0][0]);
      if (live(j + 1)) F::template compute<B, 1>(a, rb, sub + L * (j + 1), xs, ls, acc);
      issue_unit<F>(a, rp[0], unit(j + 3), ls, rb[0]);
    }
  }
#pragma unroll
  for (int i = 0; i < R * B; ++i) acc[i] = group_sum<L>(acc[i]);
  // Every lane of the group now holds all R * B sums; lane k of the group
  // stores row k (a paired launch: lane 0 stores silu(gate) * up).
  if constexpr (P && R == 1) {
    // The up sums sit in the odd lane group of the pair, L lanes up.
    float up[B];
#pragma unroll
    for (int b = 0; b < B; ++b) up[b] = __shfl_xor(acc[b], L, kWave);
    const int pr = rofs >> 1;
    if (sub == 0 && (rofs & 1) == 0 && pr < left) {
      const int64_t row = first + pr;
      const float rs0 = a.scales ? ep[1] : 1.f;
      const float rs1 = a.scales2 ? ep[2] : 1.f;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float gv = (acc[b] * AccScale<F>::value) * rs0;
        const float uv = (up[b] * AccScale<F>::value) * rs1;
        a.y[b * a.out + row] = gv / (1.f + expf(-gv)) * uv;
      }
    }
    return;
  } else if constexpr (P) {
    if (sub == 0 && rofs < left) {
      const int64_t row = first + rofs;
      const float rs0 = a.scales ? ep[1] : 1.f;
      const float rs1 = a.scales2 ? ep[2] : 1.f;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float gv = (acc[b] * AccScale<F>::value) * rs0;
        const float uv = (acc[B + b] * AccScale<F>::value) * rs1;
        a.y[b * a.out + row] = gv / (1.f + expf(-gv)) * uv;
      }
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int r = rofs + k * kRowsPerSlab;
    if (sub == k && r < left) {
      const int64_t row = first + r;
      const float bv = a.bias ? ep[0] : 0.f;
      const float rs = a.scales ? ep[1] : 1.f;
#pragma unroll
      for (int b = 0; b < B; ++b)
        a.y[b * a.out + row] = fmaf(acc[k * B + b] * AccScale<F>::value, rs, bv);
    }
  }
}

}  // namespace pesti

// ---------------------------------------------------------------------------
// Host side: validation, batch chunking to fit LDS, dispatch on (L, B).
// ---------------------------------------------------------------------------
namespace pesti_gemv {

using pesti::GemvArgs;
using pesti::GroupArgs;

template <class F, int L, int B, int U, int R, bool P = false>
int launch_one(const GroupArgs& g, size_t lds_bytes, hipStream_t stream) {
  constexpr int64_t kRowsPerTile = pesti::kTileRows<L, R, P>;
  int64_t tiles = 0;
  for (int i = 0; i < g.n_ops; ++i) {
    const int64_t t = (g.op[i].out + kRowsPerTile - 1) / kRowsPerTile;
    if (t > tiles) tiles = t;
  }
  if (tiles <= 0) return PESTI_OK;
  GroupArgs args = g;
  void* params[] = {&args};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemv_kernel<F, L, B, U, R, P>),
                                 dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(g.n_ops)),
                                 dim3(pesti::kThreads), params, lds_bytes, stream);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <class F, int L, int U, int R>
int launch_b(const GroupArgs& g, int batch, size_t lds, hipStream_t st) {
  switch (batch) {
    case 1:
      if constexpr (R == 1) return launch_one<F, L, 1, U, R>(g, lds, st);
      return PESTI_ERR_BATCH;   // several rows per lane group serve batches of 2+
    case 2: return launch_one<F, L, 2, U, R>(g, lds, st);
    case 3: return launch_one<F, L, 3, U, R>(g, lds, st);
    case 4: return launch_one<F, L, 4, U, R>(g, lds, st);
    case 5: return launch_one<F, L, 5, U, R>(g, lds, st);
    case 6: return launch_one<F, L, 6, U, R>(g, lds, st);
    case 7: return launch_one<F, L, 7, U, R>(g, lds, st);
    case 8: return launch_one<F, L, 8, U, R>(g, lds, st);
    default: return PESTI_ERR_BATCH;
  }
}

// Rows per lane group for short rows: with two or more batch columns a
// lane group serves 2 rows of a tall matrix (each x value read from LDS
// feeds both, and the workgroup carries twice the bytes), as long as the
// launch keeps at least kMinTiles workgroups.  With one batch column the
// extra registers cost more occupancy than the sharing gains.
#ifndef PESTI_MIN_TILES
#define PESTI_MIN_TILES 2048
#endif
constexpr int64_t kMinTiles = PESTI_MIN_TILES;

template <class F, int L>
int launch_r(const GroupArgs& g, int64_t max_out, int batch, size_t lds, hipStream_t st) {
  const int64_t tiles1 = (max_out + 4 * (64 / L) - 1) / (4 * (64 / L));
  if constexpr (!pesti::kStreamLayout<F>) {
    if (batch >= 2 && tiles1 >= 2 * kMinTiles) return launch_b<F, L, 1, 2>(g, batch, lds, st);
  }
  return launch_b<F, L, 1, 1>(g, batch, lds, st);
}

// (lanes per row L, units held per lane U, rows per lane group R) for the
// longest row of a launch: rows of up to 16 / 32 units take 16 / 32 lanes
// and one unit per lane; longer rows take a whole wave and hold 2 or 4
// units per lane at once.
template <class F>
int launch_lu(const GroupArgs& g, int64_t max_units, int64_t max_out, int batch, size_t lds,
              hipStream_t st) {
  if (max_units <= 16) return launch_r<F, 16>(g, max_out, batch, lds, st);
  if (max_units <= 32) return launch_r<F, 32>(g, max_out, batch, lds, st);
  const int64_t ipt = (max_units + 63) / 64;
  if (ipt <= 1) return launch_b<F, 64, 1, 1>(g, batch, lds, st);
  if (ipt <= 2) return launch_b<F, 64, 2, 1>(g, batch, lds, st);
  return launch_b<F, 64, 4, 1>(g, batch, lds, st);
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
template <> inline void shape_of<pesti::FmtQ4_KH>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 255) / 256) * 144; *u = 2 * ((in + 63) / 64);
}
template <> inline void shape_of<pesti::FmtQ4_KS>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = 0; *u = in / 64;   // rows have no fixed stride: FmtQ4_KS::row_ptr
}
template <> inline void shape_of<pesti::FmtQ2_K>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 255) / 256) * 84; *u = ((in + 127) / 128) * 2;
}
template <> inline void shape_of<pesti::FmtQ3_K>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 255) / 256) * 110; *u = ((in + 127) / 128) * 2;
}
template <> inline void shape_of<pesti::FmtQ5_K>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 255) / 256) * 176; *u = (in + 63) / 64;
}
template <> inline void shape_of<pesti::FmtQ6_K>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 255) / 256) * 210; *u = ((in + 255) / 256) * 4;
}
template <> inline void shape_of<pesti::FmtI8Row>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = in; *u = (in + 63) / 64;
}
template <> inline void shape_of<pesti::FmtI4Row>(int64_t in, int64_t* rb, int64_t* u) {
  *rb = ((in + 63) / 64) * 32; *u = (in + 63) / 64;
}

// y[b][o] = bias[o] (or 0) for every op of `g` and b < batch (ops with
// in_features == 0); defined in gemv.hip.
int fill_bias(const GroupArgs& g, int batch, hipStream_t stream);

// Validate one op; returns PESTI_OK, an error, or 1 for "empty, skip".
template <class F>
int check_op(const pesti_gemv_op& o, int32_t batch) {
  if (o.out_features < 0 || o.in_features < 0) return PESTI_ERR_SHAPE;
  if (o.out_features == 0 || batch == 0) return 1;
  if (o.in_features % 32 != 0 || o.in_features > PESTI_MAX_IN_FEATURES) return PESTI_ERR_SHAPE;
  if (pesti::kStreamLayout<F> && o.in_features % 64 != 0) return PESTI_ERR_SHAPE;   // rows of whole runs
  const bool has_in = o.in_features > 0;
  if (!o.y || (has_in && (!o.w || !o.x))) return PESTI_ERR_NULL;
  if (F::kRowScales && has_in && !o.row_scales) return PESTI_ERR_NULL;
  if (!pesti_host::aligned(o.y, 16) || (o.w && !pesti_host::aligned(o.w, 16)) ||
      (o.x && !pesti_host::aligned(o.x, 16)) || (o.bias && !pesti_host::aligned(o.bias, 4)) ||
      (o.row_scales && !pesti_host::aligned(o.row_scales, 4)))
    return PESTI_ERR_ALIGN;
  return PESTI_OK;
}

// K-quant, per-row INT4 and even-block-count Q8_0 ops of at least this
// many rows, with rows of at most 1024 weights, at batch kMfmaMinBatch..8
// go to the matrix-core mat-vec (gemv_mfma.hip), which overtakes the
// vector-ALU kernel on the 151936 x 896 LM head from batch 3 (Q2_K, Q3_K,
// Q4_K, Q5_K), 4 (Q8_0), 5 (Q6_K) and 2 (per-row INT4).  The choice
// depends on the op alone (never on the other ops of a group), so a
// grouped op gives the same bits as its own single call.
#ifndef PESTI_MFMA_MIN_ROWS
#define PESTI_MFMA_MIN_ROWS 16384
#endif
#ifndef PESTI_MFMA_MIN_BATCH
#define PESTI_MFMA_MIN_BATCH 3
#endif
#ifndef PESTI_MFMA_MIN_BATCH_Q6_K
#define PESTI_MFMA_MIN_BATCH_Q6_K 5
#endif
#ifndef PESTI_MFMA_MIN_BATCH_Q5_K
#define PESTI_MFMA_MIN_BATCH_Q5_K 3
#endif
#ifndef PESTI_MFMA_MIN_BATCH_I4ROW
#define PESTI_MFMA_MIN_BATCH_I4ROW 2
#endif
#ifndef PESTI_MFMA_MIN_BATCH_Q2_K
#define PESTI_MFMA_MIN_BATCH_Q2_K 3
#endif
#ifndef PESTI_MFMA_MIN_BATCH_Q3_K
#define PESTI_MFMA_MIN_BATCH_Q3_K 3
#endif
#ifndef PESTI_MFMA_MIN_BATCH_Q8_0
#define PESTI_MFMA_MIN_BATCH_Q8_0 4
#endif
constexpr int64_t kMfmaMinRows = PESTI_MFMA_MIN_ROWS;
template <class F>
constexpr int kMfmaMinBatch = std::is_same<F, pesti::FmtQ6_K>::value    ? PESTI_MFMA_MIN_BATCH_Q6_K
                              : std::is_same<F, pesti::FmtQ5_K>::value  ? PESTI_MFMA_MIN_BATCH_Q5_K
                              : std::is_same<F, pesti::FmtI4Row>::value ? PESTI_MFMA_MIN_BATCH_I4ROW
                              : std::is_same<F, pesti::FmtQ2_K>::value  ? PESTI_MFMA_MIN_BATCH_Q2_K
                              : std::is_same<F, pesti::FmtQ3_K>::value  ? PESTI_MFMA_MIN_BATCH_Q3_K
                              : std::is_same<F, pesti::FmtQ8_0x2>::value ? PESTI_MFMA_MIN_BATCH_Q8_0
                                                                        : PESTI_MFMA_MIN_BATCH;
template <class F>
constexpr bool kHasMfma = std::is_same<F, pesti::FmtQ4_K>::value || std::is_same<F, pesti::FmtQ6_K>::value ||
                          std::is_same<F, pesti::FmtQ5_K>::value || std::is_same<F, pesti::FmtI4Row>::value ||
                          std::is_same<F, pesti::FmtQ2_K>::value || std::is_same<F, pesti::FmtQ3_K>::value ||
                          std::is_same<F, pesti::FmtQ8_0x2>::value;
template <class F>
inline bool mfma_op(const GemvArgs& a, int batch) {
  return kHasMfma<F> && batch >= kMfmaMinBatch<F> && batch <= PESTI_MAX_BATCH && a.out >= kMfmaMinRows &&
         a.in > 0 && a.in <= 1024;
}
// Tall Q4_K, Q5_K, Q2_K, Q3_K and per-row INT4 matrices with rows of at most 1024 weights at
// batch 1 (2 but for INT4) take the kernel of gemv_tall.hip (128-weight units, a row per U
// lanes); in the Q4_K stream layout and for per-row INT4 only rows of a
// whole number of 128-weight units, so that no unit straddles two
// super-blocks or reads past its row.
#ifndef PESTI_TALL_MIN_ROWS
#define PESTI_TALL_MIN_ROWS 16384
#endif
constexpr int64_t kTallMinRows = PESTI_TALL_MIN_ROWS;
template <class F>
constexpr bool kHasTall = std::is_same<F, pesti::FmtQ4_K>::value || std::is_same<F, pesti::FmtQ5_K>::value ||
                          std::is_same<F, pesti::FmtQ2_K>::value || std::is_same<F, pesti::FmtQ3_K>::value ||
                          std::is_same<F, pesti::FmtI4Row>::value || pesti::kStreamLayout<F>;
// Largest batch the tall kernel takes: 2 (one dequantized weight feeds both
// columns), below the batch at which the matrix cores take over.
#ifndef PESTI_TALL_MAX_BATCH
#define PESTI_TALL_MAX_BATCH 2
#endif
template <class F>
constexpr int kTallMaxBatch = PESTI_TALL_MAX_BATCH < kMfmaMinBatch<F> - 1 ? PESTI_TALL_MAX_BATCH
                                                                           : kMfmaMinBatch<F> - 1;
template <class F>
inline bool tall_op(const GemvArgs& a, int batch) {
  constexpr bool kWholeUnits = pesti::kStreamLayout<F> || std::is_same<F, pesti::FmtI4Row>::value;
  return kHasTall<F> && batch >= 1 && batch <= kTallMaxBatch<F> && a.out >= kTallMinRows && a.in > 0 &&
         a.in <= 1024 && (!kWholeUnits || a.in % 128 == 0);
}
// One launch of ops that all pass tall_op and share one row length in
// 128-weight units; x and y of every op set.
int launch_tall_q4_k(const GroupArgs& g, bool stream_layout, int batch, hipStream_t st);
int launch_tall_q5_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_tall_q2_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_tall_q3_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_tall_i4row(const GroupArgs& g, int batch, hipStream_t st);
template <class F>
inline int launch_tall(const GroupArgs& g, int batch, hipStream_t st) {
  if constexpr (std::is_same<F, pesti::FmtQ5_K>::value) return launch_tall_q5_k(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtQ2_K>::value) return launch_tall_q2_k(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtQ3_K>::value) return launch_tall_q3_k(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtI4Row>::value) return launch_tall_i4row(g, batch, st);
  else return launch_tall_q4_k(g, pesti::kStreamLayout<F>, batch, st);
}

// One launch of ops that all pass mfma_op and share one row length in
// super-blocks; x and y of every op set.
int launch_mfma_q4_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_mfma_q6_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_mfma_q5_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_mfma_i4row(const GroupArgs& g, int batch, hipStream_t st);
int launch_mfma_q2_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_mfma_q3_k(const GroupArgs& g, int batch, hipStream_t st);
int launch_mfma_q8_0(const GroupArgs& g, int batch, hipStream_t st);
template <class F>
inline int launch_mfma(const GroupArgs& g, int batch, hipStream_t st) {
  if constexpr (std::is_same<F, pesti::FmtQ6_K>::value) return launch_mfma_q6_k(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtQ5_K>::value) return launch_mfma_q5_k(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtI4Row>::value) return launch_mfma_i4row(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtQ2_K>::value) return launch_mfma_q2_k(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtQ3_K>::value) return launch_mfma_q3_k(g, batch, st);
  else if constexpr (std::is_same<F, pesti::FmtQ8_0x2>::value) return launch_mfma_q8_0(g, batch, st);
  else return launch_mfma_q4_k(g, batch, st);
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

  // Ops with no columns only write their bias (or zeros); the mat-vec
  // kernel assumes every row has at least one unit.
  GroupArgs g{}, fill{};
  int n_mv = 0;
  int64_t max_units = 0, max_out = 0;
  size_t row_lds = 0;
  for (int i = 0; i < n_live; ++i) {
    const pesti_gemv_op& o = ops[live[i]];
    if (o.in_features == 0) {
      GemvArgs& f = fill.op[fill.n_ops++];
      f.y = o.y;
      f.bias = o.bias;
      f.out = o.out_features;
      continue;
    }
    live[n_mv] = live[i];
    GemvArgs& a = g.op[n_mv++];
    a.w = static_cast<const uint8_t*>(o.w);
    a.scales = o.row_scales;
    a.bias = o.bias;
    a.out = o.out_features;
    a.in = o.in_features;
    shape_of<F>(o.in_features, &a.row_bytes, &a.units);
    const int64_t pad = F::kPad;
    a.xpad = ((a.in + pad - 1) / pad) * pad;
    a.xstride = pesti::xs_stride(a.in, pad);
    const size_t r = sizeof(float) * a.xstride;
    if (r > row_lds) row_lds = r;
    if (a.units > max_units) max_units = a.units;
    if (a.out > max_out) max_out = a.out;
  }
  g.n_ops = n_mv;
  hipStream_t stream_h = static_cast<hipStream_t>(stream);
  // Every check before the first launch: an error enqueues nothing.
  const int per_launch = pesti_host::batch_per_launch(lds_limit, row_lds, 0, batch);
  if (n_mv > 0 && per_launch < 1) return PESTI_ERR_SHAPE;
  if (fill.n_ops > 0) {
    const int r = fill_bias(fill, batch, stream_h);
    if (r != PESTI_OK) return r;
  }
  if (n_mv == 0) return PESTI_OK;
  if constexpr (kHasTall<F>) {
    // Tall batch-1 ops leave the group: one launch per row length in
    // 128-weight units.
    GroupArgs rest{};
    int rest_live[PESTI_MAX_GROUP];
    bool taken[PESTI_MAX_GROUP] = {};
    for (int i = 0; i < n_mv; ++i) {
      if (taken[i] || !tall_op<F>(g.op[i], batch)) continue;
      GroupArgs t{};
      for (int j = i; j < n_mv; ++j) {
        if (taken[j] || !tall_op<F>(g.op[j], batch) || (g.op[j].in + 127) / 128 != (g.op[i].in + 127) / 128)
          continue;
        taken[j] = true;
        t.op[t.n_ops] = g.op[j];
        t.op[t.n_ops].x = ops[live[j]].x;
        t.op[t.n_ops].y = ops[live[j]].y;
        ++t.n_ops;
      }
      const int r = launch_tall<F>(t, batch, stream_h);
      if (r != PESTI_OK) return r;
    }
    max_units = 0;
    max_out = 0;
    for (int i = 0; i < n_mv; ++i) {
      if (taken[i]) continue;
      rest_live[rest.n_ops] = live[i];
      rest.op[rest.n_ops++] = g.op[i];
      if (g.op[i].units > max_units) max_units = g.op[i].units;
      if (g.op[i].out > max_out) max_out = g.op[i].out;
    }
    if (rest.n_ops == 0) return PESTI_OK;
    g = rest;
    n_mv = rest.n_ops;
    for (int i = 0; i < n_mv; ++i) live[i] = rest_live[i];
  }
  if constexpr (kHasMfma<F>) {
    // Matrix-core ops leave the group: one launch per row length (every
    // batch column at once); the rest stay for the vector-ALU kernel.
    GroupArgs rest{};
    int rest_live[PESTI_MAX_GROUP];
    bool taken[PESTI_MAX_GROUP] = {};
    for (int i = 0; i < n_mv; ++i) {
      if (taken[i] || !mfma_op<F>(g.op[i], batch)) continue;
      GroupArgs m{};
      for (int j = i; j < n_mv; ++j) {
        if (taken[j] || !mfma_op<F>(g.op[j], batch) || g.op[j].row_bytes != g.op[i].row_bytes) continue;
        taken[j] = true;
        m.op[m.n_ops] = g.op[j];
        m.op[m.n_ops].x = ops[live[j]].x;
        m.op[m.n_ops].y = ops[live[j]].y;
        ++m.n_ops;
      }
      const int r = launch_mfma<F>(m, batch, stream_h);
      if (r != PESTI_OK) return r;
    }
    max_units = 0;
    max_out = 0;
    for (int i = 0; i < n_mv; ++i) {
      if (taken[i]) continue;
      rest_live[rest.n_ops] = live[i];
      rest.op[rest.n_ops++] = g.op[i];
      if (g.op[i].units > max_units) max_units = g.op[i].units;
      if (g.op[i].out > max_out) max_out = g.op[i].out;
    }
    if (rest.n_ops == 0) return PESTI_OK;
    g = rest;
    n_mv = rest.n_ops;
    for (int i = 0; i < n_mv; ++i) live[i] = rest_live[i];
  }
  for (int b0 = 0; b0 < batch; b0 += per_launch) {
    const int nb = batch - b0 < per_launch ? batch - b0 : per_launch;
    GroupArgs c = g;
    for (int i = 0; i < n_mv; ++i) {
      const pesti_gemv_op& o = ops[live[i]];
      c.op[i].x = o.x ? o.x + static_cast<int64_t>(b0) * o.in_features : nullptr;
      c.op[i].y = o.y + static_cast<int64_t>(b0) * o.out_features;
    }
    const size_t lds = row_lds * nb;
    int r = 1;
    if constexpr ((std::is_same<F, pesti::FmtQ4_K>::value || std::is_same<F, pesti::FmtQ4_KS>::value) &&
                  pesti::kQ4KHalfUnits) {
      if (nb == 1) {
        // Ops of at most kHalfUnitMaxRows rows of at most 1024 weights take
        // half units at batch 1 (FmtQ4_KH, FmtQ4_KSH in the stream layout):
        // they halve each lane's arithmetic after a short launch's one memory
        // round trip, while on larger ops the extra workgroups and header
        // reads cost more than that saves.  The choice is made per op, so a
        // group of both kinds is two launches and every op gives the bits
        // of its own single call.
        using H = typename std::conditional<std::is_same<F, pesti::FmtQ4_K>::value, pesti::FmtQ4_KH,
                                            pesti::FmtQ4_KSH>::type;
        GroupArgs sh{}, lg{};
        int64_t sh_units = 0, lg_units = 0, lg_out = 0;
        size_t sh_lds = 0, lg_lds = 0;
        for (int i = 0; i < n_mv; ++i) {
          const size_t op_lds = sizeof(float) * static_cast<size_t>(c.op[i].xstride);
          if (c.op[i].units <= 16 && c.op[i].out <= pesti::kHalfUnitMaxRows) {
            sh.op[sh.n_ops] = c.op[i];
            sh.op[sh.n_ops].units = 2 * c.op[i].units;
            ++sh.n_ops;
            if (c.op[i].units > sh_units) sh_units = c.op[i].units;
            if (op_lds > sh_lds) sh_lds = op_lds;
          } else {
            lg.op[lg.n_ops++] = c.op[i];
            if (c.op[i].units > lg_units) lg_units = c.op[i].units;
            if (c.op[i].out > lg_out) lg_out = c.op[i].out;
            if (op_lds > lg_lds) lg_lds = op_lds;
          }
        }
        r = PESTI_OK;
        if (sh.n_ops > 0)
          r = sh_units <= 8 ? launch_one<H, 16, 1, 1, 1>(sh, sh_lds, stream_h)
                            : launch_one<H, 32, 1, 1, 1>(sh, sh_lds, stream_h);
        if (r == PESTI_OK && lg.n_ops > 0) r = launch_lu<F>(lg, lg_units, lg_out, nb, lg_lds, stream_h);
      }
    }
    if (r == 1) r = launch_lu<F>(c, max_units, max_out, nb, lds, stream_h);
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
int group_q4_k_stream(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_q2_k(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_q3_k(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_q5_k(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_q6_k(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_i8row(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
int group_i4row(int32_t n_ops, const pesti_gemv_op* ops, int32_t batch, void* stream);
// Paired gate/up launches with the SwiGLU epilogue (swiglu_dispatch below).
#define PESTI_SWIGLU_ARGS                                                                          \
  int64_t out_features, int64_t in_features, const void *w_gate, const void *w_up,                 \
      const float *gate_scales, const float *up_scales, const float *x, float *h, int32_t batch,    \
      void *stream
int swiglu_q8_0(PESTI_SWIGLU_ARGS);
int swiglu_q4_k(PESTI_SWIGLU_ARGS);
int swiglu_q2_k(PESTI_SWIGLU_ARGS);
int swiglu_q3_k(PESTI_SWIGLU_ARGS);
int swiglu_q5_k(PESTI_SWIGLU_ARGS);
int swiglu_q6_k(PESTI_SWIGLU_ARGS);
int swiglu_i8row(PESTI_SWIGLU_ARGS);
int swiglu_i4row(PESTI_SWIGLU_ARGS);

// ---------------------------------------------------------------------------
// Paired gate/up launch with the SwiGLU epilogue: h = silu(W_gate x) *
// (W_up x), both matrices of one format and shape.  Rows must fit the
// one-round path (at most 64 units, all held at once).
// ---------------------------------------------------------------------------
template <class F, int L>
int launch_pair_b(const GroupArgs& g, int batch, size_t lds, hipStream_t st) {
  constexpr int R = L < 64 ? 1 : 2;   // lane-group pairs, or both rows in a whole wave
  switch (batch) {
    case 1: return launch_one<F, L, 1, 1, R, true>(g, lds, st);
    case 2: return launch_one<F, L, 2, 1, R, true>(g, lds, st);
    case 3: return launch_one<F, L, 3, 1, R, true>(g, lds, st);
    case 4: return launch_one<F, L, 4, 1, R, true>(g, lds, st);
    case 5: return launch_one<F, L, 5, 1, R, true>(g, lds, st);
    case 6: return launch_one<F, L, 6, 1, R, true>(g, lds, st);
    case 7: return launch_one<F, L, 7, 1, R, true>(g, lds, st);
    case 8: return launch_one<F, L, 8, 1, R, true>(g, lds, st);
    default: return PESTI_ERR_BATCH;
  }
}

template <class F>
int swiglu_dispatch(int64_t out_features, int64_t in_features, const void* w_gate, const void* w_up,
                    const float* gate_scales, const float* up_scales, const float* x, float* h,
                    int32_t batch, void* stream) {
  if (batch < 0 || batch > PESTI_MAX_BATCH) return PESTI_ERR_BATCH;
  const pesti_gemv_op gate = make_op(out_features, in_features, w_gate, gate_scales, x, h, nullptr);
  const pesti_gemv_op up = make_op(out_features, in_features, w_up, up_scales, x, h, nullptr);
  int st = check_op<F>(gate, batch);
  if (st < 0) return st;
  const int st_up = check_op<F>(up, batch);
  if (st_up < 0) return st_up;
  if (st == 1) return PESTI_OK;   // nothing to compute
  int64_t rb = 0, units = 0;
  shape_of<F>(in_features, &rb, &units);
  if (units > 64) return PESTI_ERR_SHAPE;   // rows beyond the one-round path
  int dev = 0;
  size_t lds_limit = 0;
  st = pesti_host::current_device(&dev, &lds_limit);
  if (st != PESTI_OK) return st;
  hipStream_t sh = static_cast<hipStream_t>(stream);
  GroupArgs g{};
  g.n_ops = 1;
  GemvArgs& a = g.op[0];
  if (in_features == 0) {   // silu(0) * 0 = 0
    a.y = h;
    a.out = out_features;
    return fill_bias(g, batch, sh);
  }
  a.w = static_cast<const uint8_t*>(w_gate);
  a.w2 = static_cast<const uint8_t*>(w_up);
  a.scales = gate_scales;
  a.scales2 = up_scales;
  a.out = out_features;
  a.in = in_features;
  a.row_bytes = rb;
  a.units = units;
  const int64_t pad = F::kPad;
  a.xpad = ((a.in + pad - 1) / pad) * pad;
  a.xstride = pesti::xs_stride(a.in, pad);
  const size_t row_lds = sizeof(float) * a.xstride;
  const int per_launch = pesti_host::batch_per_launch(lds_limit, row_lds, 0, batch);
  if (per_launch < 1) return PESTI_ERR_SHAPE;
  for (int b0 = 0; b0 < batch; b0 += per_launch) {
    const int nb = batch - b0 < per_launch ? batch - b0 : per_launch;
    GroupArgs c = g;
    c.op[0].x = x + static_cast<int64_t>(b0) * in_features;
    c.op[0].y = h + static_cast<int64_t>(b0) * out_features;
    const size_t lds = row_lds * nb;
    int r;
    if (units <= 16) r = launch_pair_b<F, 16>(c, nb, lds, sh);
    else if (units <= 32) r = launch_pair_b<F, 32>(c, nb, lds, sh);
    else r = launch_pair_b<F, 64>(c, nb, lds, sh);
    if (r != PESTI_OK) return r;
  }
  return PESTI_OK;
}

}  // namespace pesti_gemv
