// Batch-1 and batch-2 mat-vec for tall Q4_K, Q5_K, Q2_K, Q3_K and per-row
// INT4 matrices with short rows (the LM head, 151936 x 896): y = W x + b.
//
// The operation is the decode step's row-major matrix-vector product with
// the weights kept in GGUF Q4_K, Q5_K, Q2_K or Q3_K blocks ("Project scaffold:
// modules, CLI, and correctness harness", file summaries of tensor.rs and
// quant.rs; "PESTI - Portable Execution Substrate for Transformer
// Inference", "What This Is"): w = d sc q - dmin m per sub-block (32
// weights; 16 for Q2_K), w = d (sc - 32) q for Q3_K (16), w = s q for
// per-row INT4 (s per row).
//
// At batch 1 the general kernel (gemv_impl.h) spends most of a lane's
// instructions on work that does not scale with the weights it reads - x
// staging, address set-up, scale decode, the reduction - for one 64-weight
// unit per lane, and 2 of each 16-lane row group stay idle on 896-weight
// rows (14 units).  Here a lane takes a 128-weight unit (two runs of one
// super-block: for Q4_K its 16-byte header and 64 code bytes, five 16-byte
// loads; TallQ5K, TallQ2K, TallQ3K and TallI4 below) and a row takes U =
// in / 128 consecutive lanes, so a wave holds floor(64 / U) rows (9 rows of 7
// lanes at 896 columns, one lane idle), and a workgroup of 4 waves stages x
// once for 36 rows (measured on the 151936 x 896 head: 2 / 4 / 8 / 16 waves
// 21.5 / 20.0 / 22.6 / 26.8 us).  Each weight is dequantized on its own, w =
// (d sc 2^9)(q 2^-9) - dmin m, one rounding of the exact value (the float32
// weight, bit for bit), then multiplied into the lane's sum (at batch 2
// into both columns' sums: the decode is paid once for two products); the U
// partial sums of a row are added in lane order by cross-lane reads (a fixed
// order: results do not depend on timing).
#include "gemv_impl.h"

namespace pesti {

#ifndef PESTI_TALL_WAVES
#define PESTI_TALL_WAVES 4
#endif
constexpr int kTallWaves = PESTI_TALL_WAVES;
constexpr int kTallThreads = kTallWaves * kWave;
constexpr int kTallMaxIn = 1024;

// One lane's 128-weight unit: runs 2h and 2h + 1 (sub-blocks 4h .. 4h + 3)
// of one super-block.  In the row layout unit u of a row is half h = u % 2
// of the row's super-block u / 2, weights 128u .. 128u + 127; in the stream
// layout (rows of a whole number of units) it is stream unit g = row U + u,
// half g % 2 of stream super-block g / 2, again weights 128u .. of the row.
struct TallQ4K {
  static constexpr int kBytes = 144;
  struct Raw { u32x4 hdr, c0, c1, c2, c3; };

  // g: the unit's index in 128-weight units from `base` (a row's start in
  // the row layout, the matrix's in the stream layout).
  __device__ __forceinline__ static void issue(const uint8_t* base, int64_t g, Raw& r) {
    const uint8_t* sb = base + (g >> 1) * kBytes;
    const uint8_t* cp = sb + 16 + 64 * (g & 1);
    r.hdr = load_u32x4_a16(sb);
    r.c0 = load_u32x4_a16(cp);
    r.c1 = load_u32x4_a16(cp + 16);
    r.c2 = load_u32x4_a16(cp + 32);
    r.c3 = load_u32x4_a16(cp + 48);
  }

  // Code dword i (0..15) of the unit: bytes 4i..4i+3 of its 64 code bytes.
  __device__ __forceinline__ static uint32_t word(const Raw& r, int i) {
    const u32x4& v = i < 4 ? r.c0 : (i < 8 ? r.c1 : (i < 12 ? r.c2 : r.c3));
    switch (i & 3) {
      case 0: return v.x;
      case 1: return v.y;
      case 2: return v.z;
      default: return v.w;
    }
  }

  // acc += sum over the unit's 128 weights of w * x (x from logical
  // column 128u of the row).  Sub-block 4h + t: t = 0..3 for h = 0 take
  // sc = S[t] & 63, m = S[t + 4] & 63; for h = 1 sc = (S[t + 8] & 15) |
  // (S[t] >> 6) << 4, m = (S[t + 8] >> 4) | (S[t + 4] >> 6) << 4 (S = header
  // bytes 4..15, dwords y, z, w).
  template <int B>
  __device__ __forceinline__ static void compute(const Raw& r, int u, bool h1, const float* xs, int xst,
                                                 float (&acc)[B]) {
    const uint32_t y = r.hdr.y, z = r.hdr.z, w = r.hdr.w;
    const uint32_t scv = h1 ? ((w & 0x0F0F0F0Fu) | ((y >> 2) & 0x30303030u)) : (y & 0x3F3F3F3Fu);
    const uint32_t mv = h1 ? (((w >> 4) & 0x0F0F0F0Fu) | ((z >> 2) & 0x30303030u)) : (z & 0x3F3F3F3Fu);
    const float d512 = f16_lo(r.hdr.x) * 512.0f, dmin = f16_hi(r.hdr.x);
    const float ds[4] = {d512 * ubyte<0>(scv), d512 * ubyte<1>(scv), d512 * ubyte<2>(scv), d512 * ubyte<3>(scv)};
    const float ndm[4] = {-(dmin * ubyte<0>(mv)), -(dmin * ubyte<1>(mv)), -(dmin * ubyte<2>(mv)),
                          -(dmin * ubyte<3>(mv))};
    const int x0 = 128 * u;
#pragma unroll
    for (int k = 0; k < 2; ++k) {   // run 2h + k: low nibbles sub-block 4h + 2k, high 4h + 2k + 1
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t q = word(r, 8 * k + i);
        float l[4], g[4];
        nibbles_x512(q & 0x0F0F0F0Fu, l[0], l[1], l[2], l[3]);
        nibbles_x512((q >> 4) & 0x0F0F0F0Fu, g[0], g[1], g[2], g[3]);
        float wl[4], wg[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wl[e] = fmaf(ds[2 * k], l[e], ndm[2 * k]);
          wg[e] = fmaf(ds[2 * k + 1], g[e], ndm[2 * k + 1]);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const f32x4 xl = xs4(xs + b * xst, x0 + 64 * k + 4 * i);
          const f32x4 xh = xs4(xs + b * xst, x0 + 64 * k + 32 + 4 * i);
          acc[b] = fmaf(wl[0], xl.x, acc[b]);
          acc[b] = fmaf(wl[1], xl.y, acc[b]);
          acc[b] = fmaf(wl[2], xl.z, acc[b]);
          acc[b] = fmaf(wl[3], xl.w, acc[b]);
          acc[b] = fmaf(wg[0], xh.x, acc[b]);
          acc[b] = fmaf(wg[1], xh.y, acc[b]);
          acc[b] = fmaf(wg[2], xh.z, acc[b]);
          acc[b] = fmaf(wg[3], xh.w, acc[b]);
        }
      }
    }
  }
};

// Q5_K (176-byte super-blocks): Q4_K's 16-byte header, 32 fifth-bit
// bytes at 16, the 128 low-nibble bytes at 48.  Weight 64r + 32c + l of a
// super-block (run r, nibble c, l = 0..31) has its low 4 bits in nibble c
// of byte 48 + 32r + l and its fifth bit at bit 2r + c of byte 16 + l.  A
// lane's 128-weight unit is runs 2h and 2h + 1 (h = g % 2): the header, all
// 32 fifth-bit bytes and 64 low-nibble bytes, seven 16-byte loads.  The
// 5-bit codes convert exactly with one unsigned-byte convert each, and
// w = d sc q - dmin m is one rounding of the exact value, as for Q4_K.
struct TallQ5K {
  static constexpr int kBytes = 176;
  struct Raw { u32x4 hdr, h0, h1, c0, c1, c2, c3; };

  __device__ __forceinline__ static void issue(const uint8_t* base, int64_t g, Raw& r) {
    const uint8_t* sb = base + (g >> 1) * kBytes;
    const uint8_t* cp = sb + 48 + 64 * (g & 1);
    r.hdr = load_u32x4_a16(sb);
    r.h0 = load_u32x4_a16(sb + 16);
    r.h1 = load_u32x4_a16(sb + 32);
    r.c0 = load_u32x4_a16(cp);
    r.c1 = load_u32x4_a16(cp + 16);
    r.c2 = load_u32x4_a16(cp + 32);
    r.c3 = load_u32x4_a16(cp + 48);
  }

  __device__ __forceinline__ static uint32_t pick(const u32x4& v, int i) {
    switch (i & 3) {
      case 0: return v.x;
      case 1: return v.y;
      case 2: return v.z;
      default: return v.w;
    }
  }

  // acc += sum over the unit's 128 weights of w * x; scales and mins of
  // sub-blocks 4h + t as TallQ4K::compute.
  template <int B>
  __device__ __forceinline__ static void compute(const Raw& r, int u, bool h1, const float* xs, int xst,
                                                 float (&acc)[B]) {
    const uint32_t y = r.hdr.y, z = r.hdr.z, w = r.hdr.w;
    const uint32_t scv = h1 ? ((w & 0x0F0F0F0Fu) | ((y >> 2) & 0x30303030u)) : (y & 0x3F3F3F3Fu);
    const uint32_t mv = h1 ? (((w >> 4) & 0x0F0F0F0Fu) | ((z >> 2) & 0x30303030u)) : (z & 0x3F3F3F3Fu);
    const float d = f16_lo(r.hdr.x), dmin = f16_hi(r.hdr.x);
    const float ds[4] = {d * ubyte<0>(scv), d * ubyte<1>(scv), d * ubyte<2>(scv), d * ubyte<3>(scv)};
    const float ndm[4] = {-(dmin * ubyte<0>(mv)), -(dmin * ubyte<1>(mv)), -(dmin * ubyte<2>(mv)),
                          -(dmin * ubyte<3>(mv))};
    const uint32_t hshift = h1 ? 4u : 0u;   // fifth bits of runs 2h, 2h + 1: bits 4h .. 4h + 3
    const int x0 = 128 * u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t hb = (i < 4 ? pick(r.h0, i) : pick(r.h1, i)) >> hshift;
#pragma unroll
      for (int k = 0; k < 2; ++k) {   // run 2h + k: low nibbles sub-block 2k, high 2k + 1
        const uint32_t q = k == 0 ? (i < 4 ? pick(r.c0, i) : pick(r.c1, i)) : (i < 4 ? pick(r.c2, i) : pick(r.c3, i));
        const uint32_t lo = (q & 0x0F0F0F0Fu) | (((hb >> (2 * k)) & 0x01010101u) << 4);
        const uint32_t hi = ((q >> 4) & 0x0F0F0F0Fu) | (((hb >> (2 * k + 1)) & 0x01010101u) << 4);
        const float wl[4] = {fmaf(ds[2 * k], ubyte<0>(lo), ndm[2 * k]), fmaf(ds[2 * k], ubyte<1>(lo), ndm[2 * k]),
                             fmaf(ds[2 * k], ubyte<2>(lo), ndm[2 * k]), fmaf(ds[2 * k], ubyte<3>(lo), ndm[2 * k])};
        const float wg[4] = {fmaf(ds[2 * k + 1], ubyte<0>(hi), ndm[2 * k + 1]),
                             fmaf(ds[2 * k + 1], ubyte<1>(hi), ndm[2 * k + 1]),
                             fmaf(ds[2 * k + 1], ubyte<2>(hi), ndm[2 * k + 1]),
                             fmaf(ds[2 * k + 1], ubyte<3>(hi), ndm[2 * k + 1])};
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const f32x4 xl = xs4(xs + b * xst, x0 + 64 * k + 4 * i);
          const f32x4 xh = xs4(xs + b * xst, x0 + 64 * k + 32 + 4 * i);
          acc[b] = fmaf(wl[0], xl.x, acc[b]);
          acc[b] = fmaf(wl[1], xl.y, acc[b]);
          acc[b] = fmaf(wl[2], xl.z, acc[b]);
          acc[b] = fmaf(wl[3], xl.w, acc[b]);
          acc[b] = fmaf(wg[0], xh.x, acc[b]);
          acc[b] = fmaf(wg[1], xh.y, acc[b]);
          acc[b] = fmaf(wg[2], xh.z, acc[b]);
          acc[b] = fmaf(wg[3], xh.w, acc[b]);
        }
      }
    }
  }
};

// Q2_K (84-byte super-blocks: 16 scale bytes, scale in the low nibble and
// min in the high nibble of byte k for 16-weight sub-block k; 64 code
// bytes from 16; d, dmin at 80).  Weight 128h + 32j + 16c + l has its
// 2-bit code at bit 2j of code byte 32h + 16c + l, sub-block 8h + 2j + c.
// A lane's 128-weight unit is half h = g % 2: its 32 code bytes, its 8
// scale bytes and d, dmin (four loads).  Codes convert as q 2^-9 (the fp8
// nibble trick) and w = (d sc 2^9)(q 2^-9) - dmin m is one rounding of the
// exact value, as for Q4_K.
struct TallQ2K {
  static constexpr int kBytes = 84;
  struct Raw { u32x4 q0, q1; uint32_t s0, s1, dd; };

  __device__ __forceinline__ static void issue(const uint8_t* base, int64_t g, Raw& r) {
    const uint8_t* sb = base + (g >> 1) * kBytes;
    const int h = static_cast<int>(g & 1);
    r.q0 = load_u32x4(sb + 16 + 32 * h);
    r.q1 = load_u32x4(sb + 32 + 32 * h);
    r.s0 = load_u32(sb + 8 * h);
    r.s1 = load_u32(sb + 8 * h + 4);
    r.dd = load_u32(sb + 80);
  }

  template <int B>
  __device__ __forceinline__ static void compute(const Raw& r, int u, bool, const float* xs, int xst,
                                                 float (&acc)[B]) {
    const float d512 = f16_lo(r.dd) * 512.0f, dmin = f16_hi(r.dd);
    const int x0 = 128 * u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const u32x4& qv = c ? r.q1 : r.q0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 2 * j + c;   // sub-block within the unit (scale byte k)
        const uint32_t sbyte_v = ((k < 4 ? r.s0 : r.s1) >> (8 * (k & 3))) & 0xFFu;
        const float ds = d512 * static_cast<float>(sbyte_v & 15u);
        const float ndm = -(dmin * static_cast<float>(sbyte_v >> 4));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = t == 0 ? qv.x : (t == 1 ? qv.y : (t == 2 ? qv.z : qv.w));
          float q0, q1, q2, q3;
          nibbles_x512((w >> (2 * j)) & 0x03030303u, q0, q1, q2, q3);
          const float w0 = fmaf(ds, q0, ndm), w1 = fmaf(ds, q1, ndm), w2 = fmaf(ds, q2, ndm), w3 = fmaf(ds, q3, ndm);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const f32x4 xv = xs4(xs + b * xst, x0 + 32 * j + 16 * c + 4 * t);
            acc[b] = fmaf(w0, xv.x, acc[b]);
            acc[b] = fmaf(w1, xv.y, acc[b]);
            acc[b] = fmaf(w2, xv.z, acc[b]);
            acc[b] = fmaf(w3, xv.w, acc[b]);
          }
        }
      }
    }
  }
};

// Q3_K (110-byte super-blocks: hmask[32], qs[64], 12 scale bytes, d): unit
// g is half h = g & 1 of super-block g / 2, weights 128h + 32j + l (j, l =
// 0..3, 0..31): the low two bits at bit 2j of qs byte 32h + l, the high bit
// at bit 4h + j of hmask byte l (clear: the code is 4 less), 16-weight
// sub-block 8h + 2j + (l >= 16) with a 6-bit scale less 32 (low 4 bits in
// nibble h of scale byte 2j + (l >= 16), high 2 bits in byte 8 + (2j + (l >=
// 16)) % 4 at bit 4h + 2(j / 2)).  Super-blocks are only 2-byte aligned; the
// unit takes five 16-byte loads (hmask, its half of qs, and bytes 94..109
// for the scale bytes and d), the scale dwords realigned in registers.
// Codes are exact signed bytes (-4..3); with no mins, a sub-block's sum of
// code times x scaled once by d (sc - 32) is its weights times x, rounding
// aside, with nothing to cancel.
struct TallQ3K {
  static constexpr int kBytes = 110;
  struct Raw { u32x4 h0, h1, q0, q1, sd; };

  __device__ __forceinline__ static u32x4 load2(const uint8_t* p) {
    const u32x4u2 v = *reinterpret_cast<const u32x4u2*>(p);
    return u32x4{v.x, v.y, v.z, v.w};
  }
  __device__ __forceinline__ static void issue(const uint8_t* base, int64_t g, Raw& r) {
    const uint8_t* sb = base + (g >> 1) * kBytes;
    const int h = static_cast<int>(g & 1);
    r.h0 = load2(sb);
    r.h1 = load2(sb + 16);
    r.q0 = load2(sb + 32 + 32 * h);
    r.q1 = load2(sb + 48 + 32 * h);
    r.sd = load2(sb + 94);
  }

  template <int B>
  __device__ __forceinline__ static void compute(const Raw& r, int u, bool half, const float* xs, int xst,
                                                 float (&acc)[B]) {
    // scale bytes 0..3, 4..7, 8..11 (super-block bytes 96..107) and d (108)
    const uint32_t s0 = __builtin_amdgcn_alignbyte(r.sd.y, r.sd.x, 2);
    const uint32_t s1 = __builtin_amdgcn_alignbyte(r.sd.z, r.sd.y, 2);
    const uint32_t s2 = __builtin_amdgcn_alignbyte(r.sd.w, r.sd.z, 2);
    const float d = f16_hi(r.sd.w);
    const uint32_t h4 = half ? 4u : 0u;
    const int x0 = 128 * u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hs = h4 + static_cast<uint32_t>(j);   // high-bit position
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4& qv = c ? r.q1 : r.q0;
        const u32x4& hv = c ? r.h1 : r.h0;
        const int k = 2 * j + c;   // sub-block within the unit
        const uint32_t lo4 = ((k < 4 ? s0 : s1) >> (8 * (k & 3) + h4)) & 15u;
        const uint32_t hi2 = (s2 >> (8 * (k & 3) + h4 + 2 * (j >> 1))) & 3u;
        const float ds = d * static_cast<float>(static_cast<int>(lo4 | (hi2 << 4)) - 32);
        float p[B];
#pragma unroll
        for (int b = 0; b < B; ++b) p[b] = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = t == 0 ? qv.x : (t == 1 ? qv.y : (t == 2 ? qv.z : qv.w));
          const uint32_t hw = t == 0 ? hv.x : (t == 1 ? hv.y : (t == 2 ? hv.z : hv.w));
          const uint32_t low2 = (w >> (2 * j)) & 0x03030303u;
          const uint32_t hb = (hw >> hs) & 0x01010101u;   // 1 where the high bit is set
          // 0xFF in the bytes whose high bit is clear: byte selector 13 of
          // v_perm gives 0xFF, 12 gives 0 (no multiply)
          const uint32_t neg = __builtin_amdgcn_perm(0u, 0u, 0x0D0D0D0Du - hb);
          const uint32_t qb = low2 | (neg & 0xFCFCFCFCu);   // signed bytes -4..3
          const float c0 = sbyte<0>(qb), c1 = sbyte<1>(qb), c2 = sbyte<2>(qb), c3 = sbyte<3>(qb);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const f32x4 xv = xs4(xs + b * xst, x0 + 32 * j + 16 * c + 4 * t);
            p[b] = fmaf(c0, xv.x, p[b]);
            p[b] = fmaf(c1, xv.y, p[b]);
            p[b] = fmaf(c2, xv.z, p[b]);
            p[b] = fmaf(c3, xv.w, p[b]);
          }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = fmaf(ds, p[b], acc[b]);
      }
    }
  }
};

// Per-row INT4 (rows of in / 2 code bytes, weights 2i and 2i + 1 in the low
// and high nibble of byte i, two's complement; w = s q with the row's scale
// s): a unit is 64 code bytes, four 16-byte loads, and rows must be a whole
// number of units (in % 128 == 0) so that no unit reads past its row.  A
// nibble moved to the top of a byte is the exact signed byte 16 q,
// converted with one sign-extending convert; the 1/16 and the row scale
// multiply the row's sum (kRowScales).
struct TallI4 {
  static constexpr bool kRowScales = true;
  static constexpr float kAccScale = 0.0625f;
  struct Raw { u32x4 c0, c1, c2, c3; };

  __device__ __forceinline__ static void issue(const uint8_t* base, int64_t g, Raw& r) {
    const uint8_t* p = base + 64 * g;
    r.c0 = load_u32x4_a16(p);
    r.c1 = load_u32x4_a16(p + 16);
    r.c2 = load_u32x4_a16(p + 32);
    r.c3 = load_u32x4_a16(p + 48);
  }

  template <int B>
  __device__ __forceinline__ static void compute(const Raw& r, int u, bool, const float* xs, int xst,
                                                 float (&acc)[B]) {
    const int x0 = 128 * u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4& cv = i < 4 ? r.c0 : (i < 8 ? r.c1 : (i < 12 ? r.c2 : r.c3));
      const uint32_t v = (i & 3) == 0 ? cv.x : ((i & 3) == 1 ? cv.y : ((i & 3) == 2 ? cv.z : cv.w));
      const uint32_t ev = (v << 4) & 0xF0F0F0F0u;   // even weights, 16 q each
      const uint32_t od = v & 0xF0F0F0F0u;          // odd weights
      const float q[8] = {sbyte<0>(ev), sbyte<0>(od), sbyte<1>(ev), sbyte<1>(od),
                          sbyte<2>(ev), sbyte<2>(od), sbyte<3>(ev), sbyte<3>(od)};
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const f32x4 xa = xs4(xs + b * xst, x0 + 8 * i);
        const f32x4 xb = xs4(xs + b * xst, x0 + 8 * i + 4);
        acc[b] = fmaf(q[0], xa.x, acc[b]);
        acc[b] = fmaf(q[1], xa.y, acc[b]);
        acc[b] = fmaf(q[2], xa.z, acc[b]);
        acc[b] = fmaf(q[3], xa.w, acc[b]);
        acc[b] = fmaf(q[4], xb.x, acc[b]);
        acc[b] = fmaf(q[5], xb.y, acc[b]);
        acc[b] = fmaf(q[6], xb.z, acc[b]);
        acc[b] = fmaf(q[7], xb.w, acc[b]);
      }
    }
  }
};

// Whether a unit policy scales each row's sum (T::kRowScales, per-row INT4).
template <class T, class = void>
struct TallRowScales { static constexpr bool value = false; };
template <class T>
struct TallRowScales<T, std::void_t<decltype(T::kRowScales)>> { static constexpr bool value = T::kRowScales; };

// U = 128-weight units per row (row layout: rows of up to 128 U weights,
// padded to whole super-blocks; stream layout, S: rows of exactly 128 U);
// a wave serves 64 / U rows, a workgroup kTallWaves times that.  Measured
// and not taken: two or four row groups per wave with all their loads in
// flight at once (24.2 / 36.0 us), register caps of 80 or 64 VGPRs for
// more waves per SIMD (26.8 us; 46.6 us with spills), and workgroups that
// take 2, 4 or 8 row blocks in turn with the next block's loads issued
// before the current block's arithmetic (in one run: 23.2 us for one block against
// 24.0 / 26.5 / 33.2: fewer workgroups keep fewer loads in flight).
template <class T, int U, bool S, int B>
__global__ __launch_bounds__(kTallThreads) void gemv_tall_kernel(GroupArgs g) {
  static_assert(!S || std::is_same<T, TallQ4K>::value, "the stream layout is Q4_K's");
  constexpr int kXS = static_cast<int>(xs_phys(kTallMaxIn));   // LDS floats per batch column
  __shared__ float xs[B * kXS];
  constexpr int kRowsPerWave = kWave / U;
  constexpr int kRowsPerGroup = kRowsPerWave * kTallWaves;
  const GemvArgs a = g.op[blockIdx.y];
  asm volatile("" ::"s"(a.w), "s"(a.x), "s"(a.y), "s"(a.bias), "s"(a.out), "s"(a.in), "s"(a.row_bytes));
  const int64_t first_wg = xcd_tile(blockIdx.x, gridDim.x) * kRowsPerGroup;
  if (first_wg >= a.out) return;   // this op has fewer row groups (uniform)
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int rr = lane / U;   // row of the lane within the wave
  const int u = lane - rr * U;
  const int64_t row = first_wg + wave * kRowsPerWave + rr;
  const bool live = rr < kRowsPerWave && row < a.out;
  // x first (slots past `in` are zero), then the unit's loads: rows past
  // the end and the idle lanes read unit 0 of the workgroup's first row (in
  // bounds).
  constexpr int kX4 = 32 * U;   // float4 slots of the padded row
  constexpr int kXPer = (kX4 + kTallThreads - 1) / kTallThreads;
  const int in4 = static_cast<int>(a.in >> 2);
  f32x4 xv[B][kXPer];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
      const int s = tid + k * kTallThreads;
      xv[b][k] = reinterpret_cast<const f32x4*>(a.x + b * a.in)[s < in4 ? s : 0];
    }
  const int64_t lrow = live ? row : first_wg;
  const int lu = live ? u : 0;
  const int64_t gu = S ? lrow * U + lu : lu;
  typename T::Raw r;
  T::issue(S ? a.w : a.w + lrow * a.row_bytes, gu, r);
  const float bv = *(a.bias ? a.bias + lrow : reinterpret_cast<const float*>(a.w));
  float rs = 1.f;
  if constexpr (TallRowScales<T>::value) rs = a.scales[lrow];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
      const int s = tid + k * kTallThreads;
      if (s < kX4)
        *reinterpret_cast<f32x4*>(xs + b * kXS + xs_phys(4 * s)) = s < in4 ? xv[b][k] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  __syncthreads();
  float part[B];
#pragma unroll
  for (int b = 0; b < B; ++b) part[b] = 0.f;
  if (live) T::template compute<B>(r, u, (gu & 1) != 0, xs, kXS, part);
  // each column's U partial sums of the row, added in lane order (reads past
  // the wave take the lane's own value; only the row's first lane stores)
#pragma unroll
  for (int b = 0; b < B; ++b) {
    float sum = part[b];
#pragma unroll
    for (int k = 1; k < U; ++k) sum += __shfl(part[b], lane + k < kWave ? lane + k : lane, kWave);
    if constexpr (TallRowScales<T>::value) {
      if (u == 0 && live) a.y[b * a.out + row] = fmaf(sum * T::kAccScale, rs, a.bias ? bv : 0.f);
    } else {
      if (u == 0 && live) a.y[b * a.out + row] = sum + (a.bias ? bv : 0.f);
    }
  }
}

}  // namespace pesti

namespace pesti_gemv {

template <class T, int U, bool S, int B>
int launch_tall_u(const GroupArgs& g, hipStream_t st) {
  constexpr int64_t kRows = (pesti::kWave / U) * pesti::kTallWaves;
  int64_t max_out = 0;
  for (int i = 0; i < g.n_ops; ++i) max_out = g.op[i].out > max_out ? g.op[i].out : max_out;
  const int64_t groups = (max_out + kRows - 1) / kRows;
  GroupArgs args = g;
  void* params[] = {&args};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemv_tall_kernel<T, U, S, B>),
                                       dim3(static_cast<unsigned>(groups), static_cast<unsigned>(g.n_ops)),
                                       dim3(pesti::kTallThreads), params, 0, st);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <class T, bool S, int B>
int launch_tall_b(const GroupArgs& g, hipStream_t st) {
  switch ((g.op[0].in + 127) / 128) {
    case 1: return launch_tall_u<T, 1, S, B>(g, st);
    case 2: return launch_tall_u<T, 2, S, B>(g, st);
    case 3: return launch_tall_u<T, 3, S, B>(g, st);
    case 4: return launch_tall_u<T, 4, S, B>(g, st);
    case 5: return launch_tall_u<T, 5, S, B>(g, st);
    case 6: return launch_tall_u<T, 6, S, B>(g, st);
    case 7: return launch_tall_u<T, 7, S, B>(g, st);
    case 8: return launch_tall_u<T, 8, S, B>(g, st);
    default: return PESTI_ERR_SHAPE;
  }
}

template <class T, bool S>
int launch_tall_s(const GroupArgs& g, int batch, hipStream_t st) {
  if (batch == 1) return launch_tall_b<T, S, 1>(g, st);
  if (batch == 2 && !pesti::TallRowScales<T>::value) return launch_tall_b<T, S, 2>(g, st);
  return PESTI_ERR_BATCH;
}

// One launch of tall Q4_K ops that share one row length; in the
// stream layout every row is a whole number of 128-weight units.
int launch_tall_q4_k(const GroupArgs& g, bool stream_layout, int batch, hipStream_t st) {
  if (g.n_ops < 1) return PESTI_ERR_SHAPE;
  if (!stream_layout) return launch_tall_s<pesti::TallQ4K, false>(g, batch, st);
  for (int i = 0; i < g.n_ops; ++i)
    if (g.op[i].in % 128 != 0 || g.op[i].in != g.op[0].in) return PESTI_ERR_SHAPE;
  return launch_tall_s<pesti::TallQ4K, true>(g, batch, st);
}

// The same for Q5_K, Q2_K and Q3_K (row layout).
int launch_tall_q5_k(const GroupArgs& g, int batch, hipStream_t st) {
  if (g.n_ops < 1) return PESTI_ERR_SHAPE;
  return launch_tall_s<pesti::TallQ5K, false>(g, batch, st);
}

int launch_tall_q2_k(const GroupArgs& g, int batch, hipStream_t st) {
  if (g.n_ops < 1) return PESTI_ERR_SHAPE;
  return launch_tall_s<pesti::TallQ2K, false>(g, batch, st);
}

int launch_tall_q3_k(const GroupArgs& g, int batch, hipStream_t st) {
  if (g.n_ops < 1) return PESTI_ERR_SHAPE;
  return launch_tall_s<pesti::TallQ3K, false>(g, batch, st);
}

// Per-row INT4: rows of a whole number of 128-weight units only.
int launch_tall_i4row(const GroupArgs& g, int batch, hipStream_t st) {
  if (g.n_ops < 1) return PESTI_ERR_SHAPE;
  for (int i = 0; i < g.n_ops; ++i)
    if (g.op[i].in % 128 != 0 || !g.op[i].scales) return PESTI_ERR_SHAPE;
  return launch_tall_s<pesti::TallI4, false>(g, batch, st);
}

}  // namespace pesti_gemv
