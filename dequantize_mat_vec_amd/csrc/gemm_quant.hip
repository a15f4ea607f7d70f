// Small-M prefill GEMM with block-quantized weights: Y = X W^T + b with W in
// Q8_0 or a K-family format, Q2_K .. Q6_K (packed rows, the layouts of the
// mat-vec), X binary16 [m][K], Y float32 [m][N].  This is the prompt-width case of the decode step's
// linear layer ("inferno" README, "Benchmarks": linear = x @ w + b at prompt
// width, the products that page finds dominate prefill) with the weights kept
// in the quantized form of the mat-vec ("Project scaffold ...", quant.rs:
// the fused dequantize + mat-vec that never expands W to float32).
//
// The product runs on the matrix cores on exact operands.  Every code is an
// integer that binary16 represents exactly (Q8_0 int8 through a float32 and
// a round-to-zero pack; Q4_K nibbles through v_cvt_scalef32_pk_f16_fp8 of
// the nibble read as an e4m3 byte, exactly q * 2^-9; the other K-family
// codes through binary16 1024 + q built by a byte permute), and X is binary16, so
// every product is exact in the float32 accumulator of
// v_mfma_f32_16x16x32_f16.  One MFMA k-step is one 32-weight sub-block
// (a Q8_0 block, a Q4_K sub-block), so its scales are applied to the
// step's 16x16 partial tile in float32: acc += (d * sc) * sum(q x).  Formats
// with mins take the codes less the sub-block's nearest code c
// (nearest_code in common.h) and add (d sc c - dmin m) * sum(x), sum(x)
// coming from a second MFMA against a tile of ones: that remainder is
// exactly 0 where a sub-block's weights all are.
//
// Work split as in the binary16 GEMM: a workgroup owns 16 output columns
// (16 rows of W) and 16 * MT rows of X, its NW wavefronts take contiguous
// slices of K, each streamed one pair of k-steps ahead with two register
// buffers (branch-free loads; steps past the slice read in-bounds
// stand-ins and are skipped), and the partial tiles are summed in a
// fixed order through LDS.
//
// MFMA operand layout, lane l (i = l % 16, kg = l / 16): A = X row i,
// k = 8kg..8kg+7; B = W row i (output column i), the same k; C = column i,
// rows 4kg..4kg+3.
#include <type_traits>

#include "gemm_wide.h"

namespace pesti {

typedef _Float16 qhalf8 __attribute__((ext_vector_type(8)));
typedef _Float16 qhalf2 __attribute__((ext_vector_type(2)));
typedef float qfloat4 __attribute__((ext_vector_type(4)));

struct QGemmArgs {
  const uint8_t* w;    // packed rows of W [N]
  const uint16_t* x;   // [M][K] binary16
  float* y;            // [M][N]
  const float* bias;   // [N] or null
  int64_t m, n, k;
  int64_t row_bytes;
};

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// ---------------------------------------------------------------------------
// Q8_0: k-step s = block s of the row (34 bytes: binary16 d, 32 int8).  A
// lane's 8 codes start at byte 2 + 8kg of the block, 2 bytes off a dword
// boundary in every other block; the lane reads the two dwords that start
// at or before them and, when misaligned, the 16 bits that follow (else an
// in-bounds re-read), never a byte outside the block, and realigns them.
// ---------------------------------------------------------------------------
struct QPolQ8_0 {
  static constexpr int32_t kFormat = PESTI_FMT_Q8_0;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr int kParts = 1;
  struct Step { uint32_t c[3]; uint32_t d; uint32_t s; };

  __device__ __forceinline__ static void load(const uint8_t* row, int s, int kg, Step& st) {
    const uint8_t* blk = row + 34 * s;
    const uint8_t* p = blk + 2 + 8 * kg;
    const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);   // 0 or 2
    const uint8_t* pa = p - mis;
    st.c[0] = load_u32(pa);
    st.c[1] = load_u32(pa + 4);
    st.c[2] = load_u16(pa + (mis ? 8 : 4));
    st.d = load_u16(blk);
    st.s = mis;
  }

  __device__ __forceinline__ static qhalf8 codes(const Step& st) {
    const uint32_t lo = align_bytes(st.c[1], st.c[0], st.s);
    const uint32_t hi = align_bytes(st.c[2], st.c[1], st.s);
    uint32_t h[4];
    h[0] = pack_f16(sbyte<0>(lo), sbyte<1>(lo));
    h[1] = pack_f16(sbyte<2>(lo), sbyte<3>(lo));
    h[2] = pack_f16(sbyte<0>(hi), sbyte<1>(hi));
    h[3] = pack_f16(sbyte<2>(hi), sbyte<3>(hi));
    return __builtin_bit_cast(qhalf8, h);
  }

  __device__ __forceinline__ static void scales(const Step& st, float& ds, float& dm) {
    ds = f16_lo(st.d);
    dm = 0.f;
  }
  __device__ __forceinline__ static qhalf8 codes(const Step& st, int, int) { return codes(st); }
  __device__ __forceinline__ static void scales(const Step& st, int, float& ds, float& dm) {
    scales(st, ds, dm);
  }
};

// Eight int8 codes (two dwords) as exact binary16 operands: q + 128 (the
// sign bit flipped) becomes 1152 + q by writing 0x64 above each byte, and
// an exact packed subtraction of 1152 leaves q.
__device__ __forceinline__ qhalf8 q8_codes(uint32_t lo, uint32_t hi) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  uint32_t h[4];
  h[0] = __builtin_amdgcn_perm(0x64646464u, a, 0x04010400u);
  h[1] = __builtin_amdgcn_perm(0x64646464u, a, 0x04030402u);
  h[2] = __builtin_amdgcn_perm(0x64646464u, b, 0x04010400u);
  h[3] = __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u);
  const qhalf2 base{static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(qhalf2, h[e]) - base);
  return __builtin_bit_cast(qhalf8, h);
}

// Q8_0 block pairs, for rows of an even number of blocks (rows then start
// on a dword boundary): steps s and s + 1 (s even) are blocks s and s + 1,
// 68 bytes from byte 34s.  A lane reads bytes 8kg..8kg+11 of the pair (its
// 8 codes of the first block, 2 bytes in, and for kg = 0 that block's d)
// and bytes 36 + 8kg..+7 (its 8 codes of the second block); the second
// block's d is the top half of the last dword lane kg = 3 reads.  Two
// loads per pair instead of eight; each d reaches the other lanes of its
// column by a cross-lane read when the step is used (all lanes active).
struct QPolQ8_0P {
  static constexpr int32_t kFormat = PESTI_FMT_Q8_0;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr int kParts = 1;
  // w: first block (odd 0) the three dwords at 8kg; second block (odd 1)
  // its two code dwords and the first block's third dword (for its d).
  struct Step { uint32_t w[3]; uint32_t odd; };

  __device__ __forceinline__ static void load_pair(const uint8_t* row, int s, int kg, Step& a, Step& b) {
    const uint8_t* pp = row + 34 * s;
    const uint32_t* ev = reinterpret_cast<const uint32_t*>(pp + 8 * kg);
    const uint32_t* ov = reinterpret_cast<const uint32_t*>(pp + 36 + 8 * kg);
    a.w[0] = ev[0];
    a.w[1] = ev[1];
    a.w[2] = ev[2];
    a.odd = 0;
    b.w[0] = ov[0];
    b.w[1] = ov[1];
    b.w[2] = a.w[2];
    b.odd = 1;
  }
  __device__ __forceinline__ static qhalf8 codes(const Step& st, int, int) {
    if (st.odd) return q8_codes(st.w[0], st.w[1]);
    return q8_codes(__builtin_amdgcn_alignbyte(st.w[1], st.w[0], 2), __builtin_amdgcn_alignbyte(st.w[2], st.w[1], 2));
  }
  __device__ __forceinline__ static void scales(const Step& st, int, float& ds, float& dm) {
    const int i = static_cast<int>(__lane_id()) & 15;
    ds = st.odd ? f16_hi(static_cast<uint32_t>(__shfl(static_cast<int>(st.w[2]), i + 48, kWave)))
                : f16_lo(static_cast<uint32_t>(__shfl(static_cast<int>(st.w[0]), i, kWave)));
    dm = 0.f;
  }
};

// ---------------------------------------------------------------------------
// Q4_K: k-step s = sub-block j = s % 8 of super-block s / 8 (144 bytes:
// d, dmin, 12 bytes of 6-bit scales/mins, 128 code bytes).  Sub-blocks 2g
// and 2g+1 are the low and high nibbles of code bytes 32g..32g+31; a lane's
// 8 codes are bytes 32g + 8kg..+7 (8-byte aligned: rows are whole 144-byte
// super-blocks).
// ---------------------------------------------------------------------------
struct QPolQ4_K {
  static constexpr int32_t kFormat = PESTI_FMT_Q4_K;
  static constexpr bool kMin = true;
  static constexpr bool kScaled = true;
  static constexpr int kParts = 1;
  static constexpr int kNarrowLongNW = 16;
  struct Step { uint32_t c[2]; u32x4 hdr; uint32_t j; };

  // Steps s and s + 1 (s even: sub-blocks 2g and 2g + 1, the low and high
  // nibbles of the same code bytes) share all their bytes: 3 loads for the
  // pair instead of 6.
  __device__ __forceinline__ static void load_pair(const uint8_t* row, int s, int kg, Step& a, Step& b) {
    const uint8_t* sb = row + 144 * (s >> 3);
    const int j = s & 6;
    const uint8_t* p = sb + 16 + 32 * (j >> 1) + 8 * kg;
    a.c[0] = b.c[0] = load_u32(p);
    a.c[1] = b.c[1] = load_u32(p + 4);
    a.hdr = b.hdr = load_u32x4_a16(sb);
    a.j = static_cast<uint32_t>(j);
    b.j = static_cast<uint32_t>(j + 1);
  }

  // The codes less c, (q - c) 2^-9: a nibble in an otherwise zero e4m3 byte
  // is q * 2^-9 (scale 1), and the binary16 subtraction is exact.
  __device__ __forceinline__ static qhalf8 codes(const Step& st) {
    float ds, dm, c;
    sub_block(st, ds, dm, c);
    const qhalf2 off = __builtin_bit_cast(qhalf2, pack_f16(c * (1.0f / 512.0f), c * (1.0f / 512.0f)));
    const uint32_t sh = 4u * (st.j & 1u);   // high nibbles for odd sub-blocks
    const uint32_t a = (st.c[0] >> sh) & 0x0F0F0F0Fu;
    const uint32_t b = (st.c[1] >> sh) & 0x0F0F0F0Fu;
    qhalf2 h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false) - off;
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true) - off;
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false) - off;
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true) - off;
    return __builtin_bit_cast(qhalf8, h);
  }

  // d * sc * 2^9 (undoing the 2^-9 of the code conversion) and the part of
  // the min term the codes leave, dmin * m - d * sc * c (exact).
  __device__ __forceinline__ static void scales(const Step& st, float& ds, float& dm) {
    float c;
    sub_block(st, ds, dm, c);
    dm = -fmaf(ds, c, -dm);
    ds *= 512.0f;
  }

  // d * sc, dmin * m and nearest_code of sub-block j.  Sub-blocks 0..3:
  // sc = S[j] & 63, m = S[j+4] & 63; 4..7 (t = j - 4): sc = (S[j+4] & 15) |
  // (S[t] >> 6) << 4, m = (S[j+4] >> 4) | (S[j] >> 6) << 4, where S[0..11]
  // are header bytes 4..15.
  __device__ __forceinline__ static void sub_block(const Step& st, float& ds, float& dm, float& c) {
    const uint32_t j = st.j;
    const uint32_t t = j & 3u;
    const uint32_t y = st.hdr.y, z = st.hdr.z, w = st.hdr.w;
    const uint32_t sy = (y >> (8 * t)) & 0xFFu, sz = (z >> (8 * t)) & 0xFFu, sw = (w >> (8 * t)) & 0xFFu;
    uint32_t sc, mn;
    if (j < 4) {
      sc = sy & 63u;
      mn = sz & 63u;
    } else {
      sc = (sw & 15u) | ((sy >> 6) << 4);
      mn = (sw >> 4) | ((sz >> 6) << 4);
    }
    const float d = f16_lo(st.hdr.x), dmin = f16_hi(st.hdr.x);
    ds = d * static_cast<float>(sc);
    dm = dmin * static_cast<float>(mn);
    c = nearest_code(dm, ds, 15.f);
  }
  __device__ __forceinline__ static qhalf8 codes(const Step& st, int, int) { return codes(st); }
  __device__ __forceinline__ static void scales(const Step& st, int, float& ds, float& dm) {
    scales(st, ds, dm);
  }
};

// ---------------------------------------------------------------------------
// Q6_K: 210-byte super-blocks (ql[128], qh[64], 16 int8 scales, binary16 d)
// of sixteen 16-weight sub-blocks.  Weight 128h + 32g + l (h < 2, g < 4,
// l < 32) has its low 4 bits in ql[64h + 32(g % 2) + l] (high nibble for
// g >= 2) and its high 2 bits at bit 2g of qh[32h + l]; k-step t = 4h + g
// covers l = 0..31, so a lane's 8 codes (l = 8kg..8kg+7) are 8 bytes of ql
// and 8 of qh, and the step spans sub-blocks 2t (lanes kg < 2) and 2t + 1.
// Super-blocks sit 2 bytes off a dword boundary every other one; the loads
// are 2-byte aligned vector loads (measured faster than dword loads
// realigned in registers).  A code q (0..63) becomes binary16
// 1024 + q by placing 0x64 above its byte, and q - 32 by one exact packed
// subtraction of 1056.  (q - 32) * sc can exceed binary16's integers, so
// the two sub-blocks of a step are two products with the other half of
// the operand zeroed, each scaled by its own d * sc in float32.
// ---------------------------------------------------------------------------
typedef uint32_t q6u2 __attribute__((ext_vector_type(2), aligned(2)));
typedef uint32_t q6u4 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t q6u1 __attribute__((aligned(2)));

__device__ __forceinline__ qhalf8 q6_k_codes(uint32_t l0, uint32_t l1, uint32_t h0, uint32_t h1, int g) {
  const uint32_t ls = 4u * static_cast<uint32_t>(g >> 1);
  const uint32_t hs = 2u * static_cast<uint32_t>(g);
  const uint32_t q0 = ((l0 >> ls) & 0x0F0F0F0Fu) | (((h0 >> hs) & 0x03030303u) << 4);
  const uint32_t q1 = ((l1 >> ls) & 0x0F0F0F0Fu) | (((h1 >> hs) & 0x03030303u) << 4);
  qhalf2 v[4];
  v[0] = __builtin_bit_cast(qhalf2, __builtin_amdgcn_perm(0x64646464u, q0, 0x04010400u));
  v[1] = __builtin_bit_cast(qhalf2, __builtin_amdgcn_perm(0x64646464u, q0, 0x04030402u));
  v[2] = __builtin_bit_cast(qhalf2, __builtin_amdgcn_perm(0x64646464u, q1, 0x04010400u));
  v[3] = __builtin_bit_cast(qhalf2, __builtin_amdgcn_perm(0x64646464u, q1, 0x04030402u));
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = v[e] - qhalf2{1056, 1056};
  return __builtin_bit_cast(qhalf8, v);
}

// The half of a step's operand that belongs to sub-block part (lanes
// kg = 2 part, 2 part + 1); the other lanes' codes are zeroed.
__device__ __forceinline__ qhalf8 q6_k_part(qhalf8 v, int part, int kg) {
  return (kg >> 1) == part ? v : qhalf8{0, 0, 0, 0, 0, 0, 0, 0};
}

struct QPolQ6_K {
  static constexpr int32_t kFormat = PESTI_FMT_Q6_K;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr int kParts = 2;
  struct Step { uint32_t l[2]; uint32_t h[2]; uint32_t sc; uint32_t d; uint32_t g; };

  // Steps s and s + 1 (s even: groups g and g + 1 of one half h, one
  // super-block) share the high-part bytes, d and one dword of scales:
  // 5 loads for the pair instead of 8.
  __device__ __forceinline__ static void load_pair(const uint8_t* row, int s, int kg, Step& a, Step& b) {
    const uint8_t* sb = row + 210 * (s >> 3);
    const int t = s & 6, h = t >> 2, g = t & 3;   // g = 0 or 2
    const q6u2 l0 = *reinterpret_cast<const q6u2*>(sb + 64 * h + 8 * kg);
    const q6u2 l1 = *reinterpret_cast<const q6u2*>(sb + 64 * h + 32 + 8 * kg);
    const q6u2 hv = *reinterpret_cast<const q6u2*>(sb + 128 + 32 * h + 8 * kg);
    const uint32_t sc = *reinterpret_cast<const q6u1*>(sb + 192 + 2 * t);   // scales 2t .. 2t + 3
    const uint32_t d = load_u16(sb + 208);
    a.l[0] = l0.x; a.l[1] = l0.y;
    b.l[0] = l1.x; b.l[1] = l1.y;
    a.h[0] = b.h[0] = hv.x;
    a.h[1] = b.h[1] = hv.y;
    a.sc = sc & 0xFFFFu;
    b.sc = sc >> 16;
    a.d = b.d = d;
    a.g = static_cast<uint32_t>(g);
    b.g = static_cast<uint32_t>(g + 1);
  }
  __device__ __forceinline__ static qhalf8 codes(const Step& st, int part, int kg) {
    return q6_k_part(q6_k_codes(st.l[0], st.l[1], st.h[0], st.h[1], static_cast<int>(st.g)), part, kg);
  }
  __device__ __forceinline__ static void scales(const Step& st, int part, float& ds, float& dm) {
    ds = f16_lo(st.d) * static_cast<float>(static_cast<int8_t>(st.sc >> (8 * part)));
    dm = 0.f;
  }
};

// ---------------------------------------------------------------------------
// Operands carrying their scale: 8 small unsigned code bytes v (two dwords)
// become binary16 1024 + v by writing 0x64 above each byte (v_perm_b32);
// an exact packed subtraction of base (1024 plus the code offset) and an
// exact packed product by the lane's scale s follow, giving
// (v - (base - 1024)) * s: Q5_K (q - c) * sc (|.| <= 31 * 63), Q2_K
// (q - c) * sc (<= 45), Q3_K (v - 4) * (sc - 32) (<= 128), all binary16
// integers.  s is per lane, so a k-step whose lanes belong to different
// sub-blocks needs no second product.
// ---------------------------------------------------------------------------
__device__ __forceinline__ qhalf8 offset_codes(uint32_t lo, uint32_t hi, qhalf2 s, qhalf2 base) {
  uint32_t h[4];
  h[0] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u);
  h[1] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u);
  h[2] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u);
  h[3] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u);
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(qhalf2, h[e]) - base) * s);
  return __builtin_bit_cast(qhalf8, h);
}

// A small non-negative integer as a binary16 pair, exactly.
__device__ __forceinline__ qhalf2 half_pair(uint32_t v) {
  const _Float16 f = static_cast<_Float16>(static_cast<float>(v));
  return qhalf2{f, f};
}
__device__ __forceinline__ qhalf2 half_pair_signed(int v) {
  const _Float16 f = static_cast<_Float16>(static_cast<float>(v));
  return qhalf2{f, f};
}

// 6-bit scale / min of Q4_K-style packing for sub-block j (0..7) from the
// header dwords y, z, w (bytes 4..15).
__device__ __forceinline__ void k4_scale_min(uint32_t y, uint32_t z, uint32_t w, int j, uint32_t& sc,
                                             uint32_t& mn) {
  const uint32_t t = static_cast<uint32_t>(j & 3);
  const uint32_t sy = (y >> (8 * t)) & 0xFFu, sz = (z >> (8 * t)) & 0xFFu, sw = (w >> (8 * t)) & 0xFFu;
  if (j < 4) {
    sc = sy & 63u;
    mn = sz & 63u;
  } else {
    sc = (sw & 15u) | ((sy >> 6) << 4);
    mn = (sw >> 4) | ((sz >> 6) << 4);
  }
}

// The wide kernel's per-unit preparation for Q4_K and Q5_K: the scale sc_j
// and nearest code c_j of all eight sub-blocks of the row's super-block,
// which every lane of the row needs.  Lane kg decodes sub-blocks 2kg and
// 2kg + 1 (sc | c << 6, 16 bits each, in one dword) and the row's four
// lanes (i + 16 kg') exchange their dwords: 2 decodes and 4 shuffles per
// lane instead of 8 decodes.
struct K4Prep {
  uint32_t w[4];   // w[k]: sub-block 2k in bits 0-15, 2k + 1 in bits 16-31
  __device__ __forceinline__ uint32_t sc(int j) const { return (w[j >> 1] >> (16 * (j & 1))) & 63u; }
  __device__ __forceinline__ float c(int j) const { return static_cast<float>((w[j >> 1] >> (16 * (j & 1) + 6)) & 63u); }
};
__device__ __forceinline__ K4Prep k4_prep(const u32x4& hdr, int kg, float cmax) {
  const float d = f16_lo(hdr.x), dmin = f16_hi(hdr.x);
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint32_t sc, mn;
    k4_scale_min(hdr.y, hdr.z, hdr.w, 2 * kg + e, sc, mn);
    const float c = nearest_code(dmin * static_cast<float>(mn), d * static_cast<float>(sc), cmax);
    mine |= (sc | (static_cast<uint32_t>(c) << 6)) << (16 * e);
  }
  K4Prep p;
  const int i = static_cast<int>(__lane_id()) & 15;
#pragma unroll
  for (int k = 0; k < 4; ++k) p.w[k] = static_cast<uint32_t>(__shfl(static_cast<int>(mine), i + 16 * k, kWave));
  return p;
}

// Q5_K step s (sub-block j = s % 8 of super-block s / 8, 176 bytes): the
// lane's 8 low nibbles (bytes 48 + 32(j / 2) + 8kg) and their fifth bits
// (bit j of bytes 16 + 8kg); operand (q - c) * sc_j with c the sub-block's
// nearest_code, scaled by d; the remainder dmin * m_j - d sc_j c times the
// step's sum of x (product against ones).
struct QPolQ5_K {
  static constexpr int32_t kFormat = PESTI_FMT_Q5_K;
  static constexpr bool kMin = true;
  static constexpr bool kScaled = true;
  static constexpr int kParts = 1;
  static constexpr int kNarrowLongNW = 16;
  struct Step { uint32_t c[2]; uint32_t h[2]; u32x4 hdr; uint32_t j; };

  // Steps s and s + 1 (s even) share all their bytes: 5 loads for the pair
  // instead of 10.
  __device__ __forceinline__ static void load_pair(const uint8_t* row, int s, int kg, Step& a, Step& b) {
    const uint8_t* sb = row + 176 * (s >> 3);
    const int j = s & 6;
    const uint8_t* p = sb + 48 + 32 * (j >> 1) + 8 * kg;
    a.c[0] = b.c[0] = load_u32(p);
    a.c[1] = b.c[1] = load_u32(p + 4);
    a.h[0] = b.h[0] = load_u32(sb + 16 + 8 * kg);
    a.h[1] = b.h[1] = load_u32(sb + 20 + 8 * kg);
    a.hdr = b.hdr = load_u32x4_a16(sb);
    a.j = static_cast<uint32_t>(j);
    b.j = static_cast<uint32_t>(j + 1);
  }
  __device__ __forceinline__ static qhalf8 codes(const Step& st, int, int) {
    const uint32_t sh = 4u * (st.j & 1u);
    const uint32_t lo = ((st.c[0] >> sh) & 0x0F0F0F0Fu) | (((st.h[0] >> st.j) & 0x01010101u) << 4);
    const uint32_t hi = ((st.c[1] >> sh) & 0x0F0F0F0Fu) | (((st.h[1] >> st.j) & 0x01010101u) << 4);
    uint32_t sc, mn;
    k4_scale_min(st.hdr.y, st.hdr.z, st.hdr.w, static_cast<int>(st.j), sc, mn);
    const float c = nearest_code(f16_hi(st.hdr.x) * static_cast<float>(mn), f16_lo(st.hdr.x) * static_cast<float>(sc),
                                 31.f);
    const qhalf2 base = __builtin_bit_cast(qhalf2, pack_f16(1024.0f + c, 1024.0f + c));
    return offset_codes(lo, hi, half_pair(sc), base);
  }
  __device__ __forceinline__ static void scales(const Step& st, int, float& ds, float& dm) {
    uint32_t sc, mn;
    k4_scale_min(st.hdr.y, st.hdr.z, st.hdr.w, static_cast<int>(st.j), sc, mn);
    ds = f16_lo(st.hdr.x);
    const float dsc = ds * static_cast<float>(sc);
    dm = f16_hi(st.hdr.x) * static_cast<float>(mn);
    dm = -fmaf(dsc, nearest_code(dm, dsc, 31.f), -dm);
  }
};

// Q3_K step s (t = s % 8 of super-block s / 8, 110 bytes, 2-byte aligned):
// t = 4h + j covers weights 128h + 32j + [0, 32); lane kg holds c = kg / 2,
// l = 8(kg % 2) .. +7 of sub-block 8h + 2j + c: low bits at bit 2j of bytes
// 32 + 32h + 16c + l, high bit at bit 4h + j of bytes 16c + l.  Operand
// (low | high << 2) - 4 = q times the lane's own scale - 32, scaled by d.
struct QPolQ3_K {
  static constexpr int32_t kFormat = PESTI_FMT_Q3_K;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr int kParts = 1;
  struct Step { uint32_t q[2]; uint32_t hm[2]; uint32_t s01, s2; uint32_t d; uint32_t t; };

  // Steps s and s + 1 (s even: j and j + 1 of one half h, one
  // super-block) share the code bytes, the high-bit bytes, d and one dword
  // of each scale run: 5 loads for the pair instead of 10.  The lane's scale
  // k = 8h + 2j + c has its low bits in byte k % 8 = 2j + c (nibble h) and
  // its high bits in byte 8 + k % 4 (bits 4h + 2(j / 2)).
  __device__ __forceinline__ static void load_pair(const uint8_t* row, int s, int kg, Step& a, Step& b) {
    const uint8_t* sb = row + 110 * (s >> 3);
    const int t = s & 6, h = t >> 2, c = kg >> 1, l = 8 * (kg & 1);
    const int j = t & 3;   // 0 or 2
    const q6u2 qv = *reinterpret_cast<const q6u2*>(sb + 32 + 32 * h + 16 * c + l);
    const q6u2 hv = *reinterpret_cast<const q6u2*>(sb + 16 * c + l);
    const uint32_t s01 = *reinterpret_cast<const q6u1*>(sb + 96 + 2 * j);   // bytes 2j .. 2j + 3
    const uint32_t s2 = *reinterpret_cast<const q6u1*>(sb + 104);           // bytes 8 .. 11
    const uint32_t d = load_u16(sb + 108);
    a.q[0] = b.q[0] = qv.x;
    a.q[1] = b.q[1] = qv.y;
    a.hm[0] = b.hm[0] = hv.x;
    a.hm[1] = b.hm[1] = hv.y;
    a.s01 = s01 & 0xFFFFu;
    b.s01 = s01 >> 16;
    a.s2 = s2 & 0xFFFFu;   // j even: bytes 8, 9
    b.s2 = s2 >> 16;       // j + 1 odd: bytes 10, 11
    a.d = b.d = d;
    a.t = static_cast<uint32_t>(t | (kg << 3));
    b.t = static_cast<uint32_t>((t + 1) | (kg << 3));
  }
  __device__ __forceinline__ static qhalf8 codes(const Step& st, int, int kg) {
    const uint32_t t = st.t & 7u, h = t >> 2, j = t & 3u, c = static_cast<uint32_t>(kg >> 1);
    const uint32_t hs = 4u * h + j;
    const uint32_t lo = ((st.q[0] >> (2 * j)) & 0x03030303u) | (((st.hm[0] >> hs) & 0x01010101u) << 2);
    const uint32_t hi = ((st.q[1] >> (2 * j)) & 0x03030303u) | (((st.hm[1] >> hs) & 0x01010101u) << 2);
    const uint32_t lo4 = (st.s01 >> (8 * c + 4 * h)) & 15u;
    const uint32_t hi2 = (st.s2 >> (8 * c + 4 * h + 2 * (j >> 1))) & 3u;
    const int sc = static_cast<int>(lo4 | (hi2 << 4)) - 32;
    const qhalf2 s = half_pair_signed(sc);
    return offset_codes(lo, hi, s, qhalf2{1028, 1028});   // (v - 4) * s, v = q + 4
  }
  __device__ __forceinline__ static void scales(const Step& st, int, float& ds, float& dm) {
    ds = f16_lo(st.d);
    dm = 0.f;
  }
};

// Q2_K step s (t = 4h + j of super-block s / 8, 84 bytes): lane kg holds
// c = kg / 2, l = 8(kg % 2) .. +7 of sub-block k = 8h + 2j + c: codes at bit
// 2j of bytes 16 + 32h + 16c + l, scale and min nibbles of byte k.  Operand
// (q - c_k) * sc with c_k the sub-block's nearest_code, scaled by d; the
// remainders dmin m - d sc c_k of the step's two sub-blocks multiply sums
// of x over its two 16-weight halves (products against ones on one half).
struct QPolQ2_K {
  static constexpr int32_t kFormat = PESTI_FMT_Q2_K;
  static constexpr bool kMin = true;
  static constexpr bool kHalfMins = true;
  static constexpr bool kScaled = true;
  static constexpr int kParts = 1;
  struct Step { uint32_t q[2]; uint32_t scb; uint32_t dd; uint32_t j; };

  // Steps s and s + 1 (s even: j and j + 1 of one half h) share their code
  // bytes, d and dmin and one dword of scale/min bytes: 4 loads for the
  // pair instead of 8.
  __device__ __forceinline__ static void load_pair(const uint8_t* row, int s, int kg, Step& a, Step& b) {
    const uint8_t* sb = row + 84 * (s >> 3);
    const int t = s & 6, h = t >> 2, j = t & 3, c = kg >> 1, l = 8 * (kg & 1);   // j = 0 or 2
    const uint8_t* p = sb + 16 + 32 * h + 16 * c + l;
    a.q[0] = b.q[0] = load_u32(p);
    a.q[1] = b.q[1] = load_u32(p + 4);
    const uint32_t sw = load_u32(sb + 8 * h + 2 * j);   // bytes 8h + 2j .. + 3
    a.scb = sw >> (8 * c);                              // byte k = 8h + 2j + c in bits 0-7
    b.scb = sw >> (16 + 8 * c);                         // byte 8h + 2(j + 1) + c
    a.dd = b.dd = load_u32(sb + 80);
    a.j = static_cast<uint32_t>(j);
    b.j = static_cast<uint32_t>(j + 1);
  }
  // d * sc, dmin * m and nearest_code of the lane's sub-block
  __device__ __forceinline__ static void sub_block(const Step& st, float& ds, float& dm, float& c) {
    ds = f16_lo(st.dd) * static_cast<float>(st.scb & 15u);
    dm = f16_hi(st.dd) * static_cast<float>((st.scb >> 4) & 15u);
    c = nearest_code(dm, ds, 3.f);
  }
  __device__ __forceinline__ static qhalf8 codes(const Step& st, int, int) {
    float ds, dm, c;
    sub_block(st, ds, dm, c);
    const uint32_t lo = (st.q[0] >> (2 * st.j)) & 0x03030303u;
    const uint32_t hi = (st.q[1] >> (2 * st.j)) & 0x03030303u;
    const qhalf2 base = __builtin_bit_cast(qhalf2, pack_f16(1024.0f + c, 1024.0f + c));
    return offset_codes(lo, hi, half_pair(st.scb & 15u), base);
  }
  // ds = d; dm = the lane's sub-block's remainder dmin m - d sc c (exact)
  __device__ __forceinline__ static void scales(const Step& st, int, float& ds, float& dm) {
    float dsc, c;
    sub_block(st, dsc, dm, c);
    ds = f16_lo(st.dd);
    dm = -fmaf(dsc, c, -dm);
  }
};

// ---------------------------------------------------------------------------
// Units of the wide-layer kernel (whole rows per wavefront, X in LDS).
// Q8_0: one block per unit, the step's loads as above.  Q4_K: one
// super-block per unit - the 16-byte header once, and each lane's 8 code
// bytes of the four sub-block pairs - so a unit feeds eight k-steps.
// The super-block formats keep two units in flight per wavefront: deeper
// rings measured slower at the 151936x896 LM head (m 16, Q4_K 32.2 / 32.7 /
// 33.4 / 40.4 us for 2 / 3 / 4 / 6 units, Q6_K 47.5 / 51.4 / 53.5 / 68.5;
// m 64 within 1-3%).
// ---------------------------------------------------------------------------
#ifndef PESTI_WIDE_Q8P_RING
#define PESTI_WIDE_Q8P_RING 4
#endif

struct WPolQ8_0 {
  static constexpr int kSumWidth = 32;
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr bool kChained = false;
  static constexpr int kSteps = 1;
  static constexpr int kRing = 8;
  static constexpr int kParts = 1;
  using Unit = QPolQ8_0::Step;
  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    QPolQ8_0::load(row, u, kg, un);
  }
  __device__ __forceinline__ static qhalf8 codes(const Unit& un, int, int, int) { return QPolQ8_0::codes(un); }
  __device__ __forceinline__ static float scale(const Unit& un, int, int) { return f16_lo(un.d); }
};

// Q8_0 pair unit, for rows of an even number of blocks: blocks 2u and
// 2u + 1, 68 bytes that start on a dword boundary.  A lane reads bytes
// 8kg..8kg+11 of the pair (its 8 codes of the first block, 2 bytes in, and
// for kg = 0 that block's d) and bytes 36 + 8kg..+7 (its 8 codes of the
// second block); the second block's d is the top half of the last dword
// that lane kg = 3 reads.  Two loads for two k-steps instead of eight; the
// d of each block reaches the other lanes of its column by a cross-lane
// read.  Codes as in q8_codes.
struct WPolQ8_0P {
  static constexpr int kSumWidth = 32;
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr bool kChained = false;
  static constexpr int kSteps = 2;
  static constexpr int kRing = PESTI_WIDE_Q8P_RING;
  static constexpr int kParts = 1;
  struct Unit { uint32_t e[3]; uint32_t o[2]; };

  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    const uint32_t* ev = reinterpret_cast<const uint32_t*>(row + 68 * u + 8 * kg);
    const uint32_t* ov = reinterpret_cast<const uint32_t*>(row + 68 * u + 36 + 8 * kg);
    un.e[0] = ev[0];
    un.e[1] = ev[1];
    un.e[2] = ev[2];
    un.o[0] = ov[0];
    un.o[1] = ov[1];
  }
  __device__ __forceinline__ static qhalf8 codes(const Unit& un, int j, int, int) {
    if (j == 0)
      return q8_codes(__builtin_amdgcn_alignbyte(un.e[1], un.e[0], 2), __builtin_amdgcn_alignbyte(un.e[2], un.e[1], 2));
    return q8_codes(un.o[0], un.o[1]);
  }
  // d of block j of the pair, for the lane's column i: from lane i (kg 0)
  // for the first block, lane i + 48 (kg 3) for the second.  Every lane of
  // the wavefront takes part (the kernel calls this on wave-uniform paths).
  __device__ __forceinline__ static float scale(const Unit& un, int j, int) {
    const int i = static_cast<int>(__lane_id()) & 15;
    if (j == 0) return f16_lo(static_cast<uint32_t>(__shfl(static_cast<int>(un.e[0]), i, kWave)));
    return f16_hi(static_cast<uint32_t>(__shfl(static_cast<int>(un.e[2]), i + 48, kWave)));
  }
};

// Q6_K unit: one super-block - per lane its 8-byte pieces of ql (four) and
// qh (two), the 16 scale bytes and d; a unit feeds eight k-steps of two
// scaled parts each.
// The wide kernel takes layers from 1024 16-column tiles in every format:
// at the 4864-column gate/up layers (304 tiles) the K-split kernel, with
// its pair loads, is faster (m 16, Q2_K .. Q6_K: 5.9 / 6.6 / 5.7 / 6.1 /
// 6.9 us against 9.2 / 7.9 / 8.8 / 9.0 / 11.6 on the wide kernel), and at
// the 151936-column LM head (9496 tiles) the wide kernel is.
struct WPolQ6_K {
  static constexpr int kSumWidth = 32;
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr bool kChained = false;
  static constexpr int kParts = 2;
  static constexpr int kSteps = 8;
  static constexpr int kRing = 2;
  struct Unit { uint32_t l[4][2]; uint32_t h[2][2]; q6u4 sc; uint32_t d; };

  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    const uint8_t* sb = row + 210 * u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // e = 2h + g % 2
      const q6u2 v = *reinterpret_cast<const q6u2*>(sb + 32 * e + 8 * kg);
      un.l[e][0] = v.x;
      un.l[e][1] = v.y;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const q6u2 v = *reinterpret_cast<const q6u2*>(sb + 128 + 32 * h + 8 * kg);
      un.h[h][0] = v.x;
      un.h[h][1] = v.y;
    }
    un.sc = *reinterpret_cast<const q6u4*>(sb + 192);
    un.d = load_u16(sb + 208);
  }
  __device__ __forceinline__ static qhalf8 codes(const Unit& un, int j, int part, int kg) {
    const int h = j >> 2, g = j & 3, e = 2 * h + (g & 1);
    return q6_k_part(q6_k_codes(un.l[e][0], un.l[e][1], un.h[h][0], un.h[h][1], g), part, kg);
  }
  // d * sc[2j + part]
  __device__ __forceinline__ static float scale(const Unit& un, int j, int part) {
    const int b = 2 * j + part;
    const uint32_t w = b < 4 ? un.sc.x : (b < 8 ? un.sc.y : (b < 12 ? un.sc.z : un.sc.w));
    return f16_lo(un.d) * static_cast<float>(static_cast<int8_t>(w >> (8 * (b & 3))));
  }
};

struct WPolQ4_K {
  static constexpr int kSumWidth = 32;
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr bool kMin = true;
  static constexpr bool kScaled = true;
  static constexpr bool kChained = true;
  static constexpr int kParts = 1;
  static constexpr int kSteps = 8;
  static constexpr int kRing = 2;
  struct Unit { u32x4 hdr; uint32_t c[4][2]; };

  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    const uint8_t* sb = row + 144 * u;
    un.hdr = load_u32x4_a16(sb);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint8_t* p = sb + 16 + 32 * g + 8 * kg;
      un.c[g][0] = load_u32(p);
      un.c[g][1] = load_u32(p + 4);
    }
  }

  // Operand of sub-block j: (q - c_j) * sc_j with c_j its nearest_code, an
  // integer of magnitude at most 945, exact in binary16, so the
  // super-block's eight k-steps accumulate in the matrix core and d is
  // applied once.  A code byte q becomes binary16 1024 + q by placing 0x64
  // above it (v_perm_b32); an exact packed subtraction of 1024 + c_j and an
  // exact packed product by sc_j follow.
  using Prep = K4Prep;
  __device__ __forceinline__ static Prep prep(const Unit& un, int kg) { return k4_prep(un.hdr, kg, 15.f); }
  __device__ __forceinline__ static qhalf8 codes(const Unit& un, const Prep& pr, int j, int) {
    const uint32_t sh = 4u * static_cast<uint32_t>(j & 1);
    const uint32_t a = (un.c[j >> 1][0] >> sh) & 0x0F0F0F0Fu;
    const uint32_t b = (un.c[j >> 1][1] >> sh) & 0x0F0F0F0Fu;
    const float c = pr.c(j);
    return offset_codes(a, b, half_pair(pr.sc(j)), __builtin_bit_cast(qhalf2, pack_f16(1024.0f + c, 1024.0f + c)));
  }

  __device__ __forceinline__ static float d(const Unit& un) { return f16_lo(un.hdr.x); }

  // d sc_j c_j - dmin m_j for sub-block j = 4 * half + kg (exact, zero for a
  // sub-block of zero weights): the B operand of the 16x16x4 float32
  // product that adds what the codes leave of the mins.
  __device__ __forceinline__ static float neg_min(const Unit& un, int half, int kg) {
    uint32_t sc, mn;
    k4_scale_min(un.hdr.y, un.hdr.z, un.hdr.w, 4 * half + kg, sc, mn);
    const float ds = d(un) * static_cast<float>(sc);
    const float dm = f16_hi(un.hdr.x) * static_cast<float>(mn);
    return fmaf(ds, nearest_code(dm, ds, 15.f), -dm);
  }
  __device__ __forceinline__ static float scale(const Unit&, int, int) { return 0.f; }
};

// Q5_K unit: one super-block - the header, the lane's 8 low-nibble bytes of
// each run and its 8 fifth-bit bytes; chained like Q4_K with (q - c_j) *
// sc_j (q <= 31) in the operand.
struct WPolQ5_K {
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr int kSumWidth = 32;
  static constexpr bool kMin = true;
  static constexpr bool kScaled = true;
  static constexpr bool kChained = true;
  static constexpr int kParts = 1;
  static constexpr int kSteps = 8;
  static constexpr int kRing = 2;
  struct Unit { u32x4 hdr; uint32_t c[4][2]; uint32_t h[2]; };

  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    const uint8_t* sb = row + 176 * u;
    un.hdr = load_u32x4_a16(sb);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint8_t* p = sb + 48 + 32 * g + 8 * kg;
      un.c[g][0] = load_u32(p);
      un.c[g][1] = load_u32(p + 4);
    }
    un.h[0] = load_u32(sb + 16 + 8 * kg);
    un.h[1] = load_u32(sb + 20 + 8 * kg);
  }
  using Prep = K4Prep;
  __device__ __forceinline__ static Prep prep(const Unit& un, int kg) { return k4_prep(un.hdr, kg, 31.f); }
  __device__ __forceinline__ static qhalf8 codes(const Unit& un, const Prep& pr, int j, int) {
    const uint32_t sh = 4u * static_cast<uint32_t>(j & 1);
    const uint32_t lo = ((un.c[j >> 1][0] >> sh) & 0x0F0F0F0Fu) | (((un.h[0] >> j) & 0x01010101u) << 4);
    const uint32_t hi = ((un.c[j >> 1][1] >> sh) & 0x0F0F0F0Fu) | (((un.h[1] >> j) & 0x01010101u) << 4);
    const float c = pr.c(j);
    return offset_codes(lo, hi, half_pair(pr.sc(j)), __builtin_bit_cast(qhalf2, pack_f16(1024.0f + c, 1024.0f + c)));
  }
  __device__ __forceinline__ static float d(const Unit& un) { return f16_lo(un.hdr.x); }
  __device__ __forceinline__ static float neg_min(const Unit& un, int half, int kg) {
    uint32_t sc, mn;
    k4_scale_min(un.hdr.y, un.hdr.z, un.hdr.w, 4 * half + kg, sc, mn);
    const float ds = d(un) * static_cast<float>(sc);
    const float dm = f16_hi(un.hdr.x) * static_cast<float>(mn);
    return fmaf(ds, nearest_code(dm, ds, 31.f), -dm);
  }
  __device__ __forceinline__ static float scale(const Unit&, int, int) { return 0.f; }
};

// Q3_K unit: one super-block (2-byte aligned) - the lane's code bytes of
// both halves (c = kg / 2, l = 8(kg % 2) .. +7), its high-bit bytes, the 12
// scale bytes and d; step j = 4h + jj carries (q) * (scale - 32) of the
// lane's sub-block 8h + 2jj + c in the operand.
struct WPolQ3_K {
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr int kSumWidth = 32;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = true;
  static constexpr bool kChained = true;
  static constexpr int kParts = 1;
  static constexpr int kSteps = 8;
  static constexpr int kRing = 2;
  struct Unit { uint32_t q[2][2]; uint32_t hm[2]; uint32_t s0, s1, s2; uint32_t d; };

  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    const uint8_t* sb = row + 110 * u;
    const int c = kg >> 1, l = 8 * (kg & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const q6u2 v = *reinterpret_cast<const q6u2*>(sb + 32 + 32 * h + 16 * c + l);
      un.q[h][0] = v.x;
      un.q[h][1] = v.y;
    }
    const q6u2 hv = *reinterpret_cast<const q6u2*>(sb + 16 * c + l);
    un.hm[0] = hv.x;
    un.hm[1] = hv.y;
    const q6u2 sv = *reinterpret_cast<const q6u2*>(sb + 96);
    un.s0 = sv.x;
    un.s1 = sv.y;
    typedef uint32_t u32a2 __attribute__((aligned(2)));
    un.s2 = *reinterpret_cast<const u32a2*>(sb + 104);
    un.d = load_u16(sb + 108);
  }
  __device__ __forceinline__ static qhalf8 codes(const Unit& un, int j, int kg) {
    const int h = j >> 2, jj = j & 3;
    const uint32_t c = static_cast<uint32_t>(kg >> 1);
    const uint32_t hs = static_cast<uint32_t>(4 * h + jj);
    const uint32_t lo = ((un.q[h][0] >> (2 * jj)) & 0x03030303u) | (((un.hm[0] >> hs) & 0x01010101u) << 2);
    const uint32_t hi = ((un.q[h][1] >> (2 * jj)) & 0x03030303u) | (((un.hm[1] >> hs) & 0x01010101u) << 2);
    const uint32_t idx = static_cast<uint32_t>(2 * jj) + c;                    // byte k % 8
    const uint32_t lw = jj < 2 ? un.s0 : un.s1;
    const uint32_t lo4 = (lw >> (8 * (idx & 3u) + 4u * h)) & 15u;
    const uint32_t hi2 = (un.s2 >> (8 * (idx & 3u) + 4u * h + 2u * (jj >> 1))) & 3u;
    const qhalf2 sv = half_pair_signed(static_cast<int>(lo4 | (hi2 << 4)) - 32);
    return offset_codes(lo, hi, sv, qhalf2{1028, 1028});
  }
  __device__ __forceinline__ static float d(const Unit& un) { return f16_lo(un.d); }
  __device__ __forceinline__ static float neg_min(const Unit&, int, int) { return 0.f; }
  __device__ __forceinline__ static float scale(const Unit&, int, int) { return 0.f; }
};

// Q2_K unit: one super-block - the lane's code bytes of both halves, the 16
// scale bytes and d, dmin; operand (q - c) * sc of the lane's sub-block (c
// its nearest_code); the 16 remainders d sc c - dmin m (one per 16 weights)
// take 16-weight sums of X, four per product.
struct WPolQ2_K {
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr int kSumWidth = 16;
  static constexpr bool kMin = true;
  static constexpr bool kScaled = true;
  static constexpr bool kChained = true;
  static constexpr int kParts = 1;
  static constexpr int kSteps = 8;
  static constexpr int kRing = 2;
  struct Unit { uint32_t q[2][2]; u32x4 sc; uint32_t dd; };

  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    const uint8_t* sb = row + 84 * u;
    const int c = kg >> 1, l = 8 * (kg & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint8_t* p = sb + 16 + 32 * h + 16 * c + l;
      un.q[h][0] = load_u32(p);
      un.q[h][1] = load_u32(p + 4);
    }
    un.sc = load_u32x4(sb);
    un.dd = load_u32(sb + 80);
  }
  __device__ __forceinline__ static uint32_t scale_byte(const Unit& un, uint32_t k) {
    const uint32_t w = k < 4 ? un.sc.x : (k < 8 ? un.sc.y : (k < 12 ? un.sc.z : un.sc.w));
    return (w >> (8 * (k & 3u))) & 0xFFu;
  }
  __device__ __forceinline__ static qhalf8 codes(const Unit& un, int j, int kg) {
    const int h = j >> 2, jj = j & 3;
    const uint32_t lo = (un.q[h][0] >> (2 * jj)) & 0x03030303u;
    const uint32_t hi = (un.q[h][1] >> (2 * jj)) & 0x03030303u;
    const uint32_t k = static_cast<uint32_t>(8 * h + 2 * jj + (kg >> 1));
    const uint32_t sb = scale_byte(un, k);
    const float c = nearest_code(f16_hi(un.dd) * static_cast<float>(sb >> 4), d(un) * static_cast<float>(sb & 15u),
                                 3.f);
    return offset_codes(lo, hi, half_pair(sb & 15u), __builtin_bit_cast(qhalf2, pack_f16(1024.0f + c, 1024.0f + c)));
  }
  __device__ __forceinline__ static float d(const Unit& un) { return f16_lo(un.dd); }
  // sub-block 4h + kg (16 weights each)
  __device__ __forceinline__ static float neg_min(const Unit& un, int h, int kg) {
    const uint32_t sb = scale_byte(un, static_cast<uint32_t>(4 * h + kg));
    const float ds = d(un) * static_cast<float>(sb & 15u);
    const float dm = f16_hi(un.dd) * static_cast<float>(sb >> 4);
    return fmaf(ds, nearest_code(dm, ds, 3.f), -dm);
  }
  __device__ __forceinline__ static float scale(const Unit&, int, int) { return 0.f; }
};

// Formats whose k-step spans two sub-blocks with mins (Q2_K).
template <class Q, class = void>
struct HalfMins { static constexpr bool value = false; };
template <class Q>
struct HalfMins<Q, std::void_t<decltype(Q::kHalfMins)>> { static constexpr bool value = Q::kHalfMins; };

template <class Q, int MT>
struct QBuf {
  typename Q::Step w[2];
  qhalf8 x[2][MT];
};

// Wavefronts per workgroup on narrow layers of over 128 k-steps (8 unless
// the policy says otherwise).
template <class Q, class = void>
struct NarrowLongNW { static constexpr int value = 8; };
template <class Q>
struct NarrowLongNW<Q, std::void_t<decltype(Q::kNarrowLongNW)>> { static constexpr int value = Q::kNarrowLongNW; };

template <class Q, class = void>
struct PairLoad : std::false_type {};
template <class Q>
struct PairLoad<Q, std::void_t<decltype(&Q::load_pair)>> : std::true_type {};

// Split form (kpart non-null, gridDim.z = splits > 1): workgroup z takes
// the z-th run of whole k-step pairs and writes its partial tile, without
// bias, to kpart[z][m][n]; a second launch sums them.
template <class Q, int NW, int MT, bool SW>
__global__ __launch_bounds__(NW * 64) void gemm_quant_kernel(QGemmArgs a, float* kpart) {
  __shared__ qfloat4 part[NW][MT][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar
  const int i = lane & 15;
  const int kg = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
  const int ksteps = static_cast<int>(a.k / 32);
  // Slices of whole k-step pairs (of the workgroup's split of K).
  const int split = static_cast<int>(blockIdx.z);
  const int split_pairs = ((ksteps + 1) / 2 + static_cast<int>(gridDim.z) - 1) / static_cast<int>(gridDim.z);
  const int g_begin = 2 * split_pairs * split < ksteps ? 2 * split_pairs * split : ksteps;
  const int g_end = g_begin + 2 * split_pairs < ksteps ? g_begin + 2 * split_pairs : ksteps;
  const int pairs = (g_end - g_begin + 1) / 2;
  const int per_wave = 2 * ((pairs + NW - 1) / NW);
  const int s_begin = g_begin + wave * per_wave;
  const int s_end = s_begin + per_wave < g_end ? s_begin + per_wave : g_end;

  const int64_t wn = n0 + i < a.n ? n0 + i : a.n - 1;
  // The bias of the lane's output column, loaded first (branch-free: without
  // a bias, a word of X scaled by 0), so the epilogue never waits on a load
  // issued after the weights.
  static_assert(NW >= MT, "one epilogue element per thread");
  const float bias_v = (a.bias ? 1.f : 0.f) *
                       (a.bias ? a.bias : reinterpret_cast<const float*>(a.x))[a.bias ? wn : 0];
  const uint8_t* wrow = a.w + wn * a.row_bytes;
  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t xm = m0 + 16 * t + i < a.m ? m0 + 16 * t + i : a.m - 1;
    xrow[t] = a.x + xm * a.k + 8 * kg;
  }

  // Steps past the slice read in-bounds stand-ins (the slice's first step)
  // and are skipped.  Formats with a pair load read steps s and s + 1 (s is
  // even, so both lie in one super-block, and s + 1 is inside the row's
  // padded blocks even past the last step) in one go.
  // X rows of whole 128-byte lines (SW: K a multiple of 64, at most 1024):
  // odd rows load the two steps of a buffer in the opposite order (x slot
  // c holds step s + (c ^ swap)) and pick them back, as in the binary16
  // GEMM.  Same operands, same order: the sums are unchanged bit for bit.
  const int swap = SW ? (i & 1) : 0;
  auto load = [&](int s, QBuf<Q, MT>& b) {
    if constexpr (PairLoad<Q>::value) {
      const int s0 = s < s_end ? s : (s_begin < ksteps ? s_begin : 0);
      Q::load_pair(wrow, s0, kg, b.w[0], b.w[1]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int sc = s + c < s_end ? s + c : (s_begin < ksteps ? s_begin : 0);
      const int sl = s + (c ^ swap);
      const int sx = sl < s_end ? sl : (s_begin < ksteps ? s_begin : 0);
      if constexpr (!PairLoad<Q>::value) Q::load(wrow, sc, kg, b.w[c]);
#pragma unroll
      for (int t = 0; t < MT; ++t) b.x[c][t] = *reinterpret_cast<const qhalf8*>(xrow[t] + 32 * sx);
    }
  };
  qfloat4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = qfloat4{0.f, 0.f, 0.f, 0.f};
  const qhalf8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  auto mma = [&](int s, const QBuf<Q, MT>& b) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (s + c >= s_end) continue;   // wave-uniform
#pragma unroll
      for (int pt = 0; pt < Q::kParts; ++pt) {
        float ds, dm;
        Q::scales(b.w[c], pt, ds, dm);
        const qhalf8 wv = Q::codes(b.w[c], pt, kg);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const qhalf8 xv = swap ? b.x[c ^ 1][t] : b.x[c][t];
          const qfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, qfloat4{0.f, 0.f, 0.f, 0.f},
                                                                   0, 0, 0);
          acc[t] += ds * p;
          if constexpr (HalfMins<Q>::value) {
            // two sub-blocks per step: the sums of x over each 16-weight
            // half, times the remainders of the column's two sub-blocks (a
            // lane holds its own; the other half's lanes are 32 away)
            const float dm_other = __shfl_xor(dm, 32, kWave);
            const bool first = kg < 2;
            const qhalf8 zeros = {0, 0, 0, 0, 0, 0, 0, 0};
            const qfloat4 s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, first ? ones : zeros,
                                                                      qfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const qfloat4 s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, first ? zeros : ones,
                                                                      qfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            acc[t] -= (first ? dm : dm_other) * s0;
            acc[t] -= (first ? dm_other : dm) * s1;
          } else if constexpr (Q::kMin) {
            // the step's sum of x (ones)
            const qfloat4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, ones,
                                                                      qfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            acc[t] -= dm * sx;
          }
        }
      }
    }
  };

  // One buffer of two k-steps, refilled right after it is consumed and
  // only while steps remain (the last pass is peeled, so no pass skips a
  // refill: a buffer kept across a skipped refill would make the compiler
  // copy it, and the copy wait for every load in flight).  Deeper rings
  // measured slower: a layer runs hundreds of wavefronts, whose own loads
  // overlap, and more loads in flight per wavefront congest the memory
  // pipeline.
  QBuf<Q, MT> buf;
  load(s_begin, buf);
  int s = s_begin;
  for (; s + 2 < s_end; s += 2) {
    mma(s, buf);
    load(s + 2, buf);
  }
  mma(s, buf);

#pragma unroll
  for (int t = 0; t < MT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  for (int e = threadIdx.x; e < MT * kWave; e += NW * kWave) {
    const int t = e / kWave, l = e % kWave;
    qfloat4 r = part[0][t][l];
#pragma unroll
    for (int w = 1; w < NW; ++w) r += part[w][t][l];
    const int64_t col = n0 + (l & 15);
    if (col < a.n) {
      const float bv = kpart ? 0.f : bias_v;   // e = threadIdx.x: column n0 + i
      float* dst = kpart ? kpart + split * a.m * a.n : a.y;
      const float v[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + 16 * t + 4 * (l >> 4) + q;
        if (row < a.m) dst[row * a.n + col] = v[q] + bv;
      }
    }
  }
}

// y[r][c] = bias[c] (or 0): the K = 0 case.
__global__ __launch_bounds__(256) void gemm_quant_bias_kernel(QGemmArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= a.m * a.n) return;
  a.y[e] = a.bias ? a.bias[e % a.n] : 0.f;
}

}  // namespace pesti

namespace {

using pesti::QGemmArgs;
using pesti::NarrowLongNW;

template <class Q, int NW, int MT>
int launch_q(const QGemmArgs& a, float* ws, hipStream_t st) {
  const int splits = ws ? pesti_host::gemm_splits(Q::kFormat, a.m, a.n, a.k) : 1;
  float* kpart = splits > 1 ? ws : nullptr;
  dim3 grid(static_cast<unsigned>((a.n + 15) / 16), static_cast<unsigned>((a.m + 16 * MT - 1) / (16 * MT)),
            static_cast<unsigned>(splits));
  QGemmArgs args = a;
  void* params[] = {&args, &kpart};
  const void* fn = reinterpret_cast<const void*>(&pesti::gemm_quant_kernel<Q, NW, MT, false>);
  if (a.k % 64 == 0 && a.k <= 1024) fn = reinterpret_cast<const void*>(&pesti::gemm_quant_kernel<Q, NW, MT, true>);
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(NW * 64), params, 0, st);
  if (e != hipSuccess) return PESTI_ERR_LAUNCH;
  return splits > 1 ? pesti_host::launch_split_sum(a.m, a.n, kpart, splits, a.bias, a.y, st) : PESTI_OK;
}

// Launch shape as for the binary16 GEMM: narrow layers give every 16-row
// tile of X its own workgroup of 8 K slices (16 for Q4_K and Q5_K over 128
// k-steps: Qwen down m16 10.4 -> 8.9 and 11.3 -> 10.9 us; the other formats
// measured the same or slower with 16); wider ones share each W load across
// 1, 2 or 4 row tiles, in workgroups of 8 K slices when there are at least
// 256 workgroups (gate/up 4864x896, us for 16 -> 8 slices: m 16 Q6_K 7.3
// -> 7.0, Q3_K 7.0 -> 6.6; m 32 Q4_K 7.7 -> 6.6, Q8_0 7.1 -> 5.9; m 64 Q4_K
// 11.1 -> 8.7, Q6_K 12.4 -> 10.4), else 16.
template <class Q>
int launch_quant(const QGemmArgs& a, float* ws, hipStream_t st) {
  const int64_t tiles_n = (a.n + 15) / 16, tiles_m = (a.m + 15) / 16;
  constexpr int kLongNW = NarrowLongNW<Q>::value;
  if (tiles_n < 96 && a.k / 32 > 128 && ws && pesti_host::gemm_split_row_tiles(Q::kFormat, a.m) == 2)
    return launch_q<Q, kLongNW, 2>(a, ws, st);
  if (tiles_n < 96 && a.k / 32 > 128) return launch_q<Q, kLongNW, 1>(a, ws, st);
  if (tiles_n < 96) return launch_q<Q, 8, 1>(a, nullptr, st);
  if (tiles_m <= 1) return tiles_n >= 256 ? launch_q<Q, 8, 1>(a, nullptr, st) : launch_q<Q, 16, 1>(a, nullptr, st);
  if (tiles_m <= 2) return tiles_n >= 256 ? launch_q<Q, 8, 2>(a, nullptr, st) : launch_q<Q, 16, 2>(a, nullptr, st);
  return tiles_n * ((tiles_m + 3) / 4) >= 256 ? launch_q<Q, 8, 4>(a, nullptr, st)
                                              : launch_q<Q, 16, 4>(a, nullptr, st);
}

template <class Q, class W>
int gemm_quant(int64_t m, int64_t out_features, int64_t in_features, const void* blocks,
               const uint16_t* x, float* y, const float* bias, int64_t row_bytes, float* ws, hipStream_t sh) {
  if (out_features < 0 || in_features < 0) return PESTI_ERR_SHAPE;
  if (m < 0 || m > PESTI_MAX_GEMM_M) return PESTI_ERR_BATCH;
  if (m == 0 || out_features == 0) return PESTI_OK;
  if (in_features % 32 != 0 || in_features > PESTI_MAX_IN_FEATURES) return PESTI_ERR_SHAPE;
  if (!y || (in_features > 0 && (!blocks || !x))) return PESTI_ERR_NULL;
  if (!pesti_host::aligned(y, 16) || (blocks && !pesti_host::aligned(blocks, 16)) ||
      (x && !pesti_host::aligned(x, 16)) || (bias && !pesti_host::aligned(bias, 4)))
    return PESTI_ERR_ALIGN;
  int dev = 0;
  size_t lds_limit = 0;
  const int st = pesti_host::current_device(&dev, &lds_limit);
  if (st != PESTI_OK) return st;
  QGemmArgs a{static_cast<const uint8_t*>(blocks), x, y, bias, m, out_features, in_features, row_bytes};
  const int wide = pesti_host::launch_wide<W>(
      pesti::WideArgs{a.w, x, y, bias, m, out_features, in_features, row_bytes}, lds_limit, sh);
  if (wide != 1) return wide;
  if (in_features == 0) {
    void* params[] = {&a};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemm_quant_bias_kernel),
                                         dim3(static_cast<unsigned>((m * out_features + 255) / 256)),
                                         dim3(256), params, 0, sh);
    return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
  }
  return launch_quant<Q>(a, ws, sh);
}

}  // namespace

int pesti_host::gemm_quant_run(int32_t format, int64_t m, int64_t n, int64_t k, const void* blocks,
                               const uint16_t* x, float* y, const float* bias, float* ws, hipStream_t st) {
  using namespace pesti;
  switch (format) {
    case PESTI_FMT_Q8_0:
      if ((k / 32) % 2 == 0)
        return gemm_quant<QPolQ8_0P, WPolQ8_0P>(m, n, k, blocks, x, y, bias, (k / 32) * 34, ws, st);
      return gemm_quant<QPolQ8_0, WPolQ8_0>(m, n, k, blocks, x, y, bias, (k / 32) * 34, ws, st);
    case PESTI_FMT_Q4_K:
      return gemm_quant<QPolQ4_K, WPolQ4_K>(m, n, k, blocks, x, y, bias, ((k + 255) / 256) * 144, ws, st);
    case PESTI_FMT_Q2_K:
      return gemm_quant<QPolQ2_K, WPolQ2_K>(m, n, k, blocks, x, y, bias, ((k + 255) / 256) * 84, ws, st);
    case PESTI_FMT_Q3_K:
      return gemm_quant<QPolQ3_K, WPolQ3_K>(m, n, k, blocks, x, y, bias, ((k + 255) / 256) * 110, ws, st);
    case PESTI_FMT_Q5_K:
      return gemm_quant<QPolQ5_K, WPolQ5_K>(m, n, k, blocks, x, y, bias, ((k + 255) / 256) * 176, ws, st);
    case PESTI_FMT_Q6_K:
      return gemm_quant<QPolQ6_K, WPolQ6_K>(m, n, k, blocks, x, y, bias, ((k + 255) / 256) * 210, ws, st);
    default:
      return PESTI_ERR_SHAPE;
  }
}

extern "C" {

int pesti_gemm_q8_0_smallm(int64_t m, int64_t out_features, int64_t in_features, const void* blocks,
                           const uint16_t* x, float* y, const float* bias, void* stream) {
  return pesti_host::gemm_quant_run(PESTI_FMT_Q8_0, m, out_features, in_features, blocks, x, y, bias, nullptr,
                                    static_cast<hipStream_t>(stream));
}

int pesti_gemm_q4_k_smallm(int64_t m, int64_t out_features, int64_t in_features, const void* blocks,
                           const uint16_t* x, float* y, const float* bias, void* stream) {
  return pesti_host::gemm_quant_run(PESTI_FMT_Q4_K, m, out_features, in_features, blocks, x, y, bias, nullptr,
                                    static_cast<hipStream_t>(stream));
}

int pesti_gemm_q2_k_smallm(int64_t m, int64_t out_features, int64_t in_features, const void* blocks,
                           const uint16_t* x, float* y, const float* bias, void* stream) {
  return pesti_host::gemm_quant_run(PESTI_FMT_Q2_K, m, out_features, in_features, blocks, x, y, bias, nullptr,
                                    static_cast<hipStream_t>(stream));
}

int pesti_gemm_q3_k_smallm(int64_t m, int64_t out_features, int64_t in_features, const void* blocks,
                           const uint16_t* x, float* y, const float* bias, void* stream) {
  return pesti_host::gemm_quant_run(PESTI_FMT_Q3_K, m, out_features, in_features, blocks, x, y, bias, nullptr,
                                    static_cast<hipStream_t>(stream));
}

int pesti_gemm_q5_k_smallm(int64_t m, int64_t out_features, int64_t in_features, const void* blocks,
                           const uint16_t* x, float* y, const float* bias, void* stream) {
  return pesti_host::gemm_quant_run(PESTI_FMT_Q5_K, m, out_features, in_features, blocks, x, y, bias, nullptr,
                                    static_cast<hipStream_t>(stream));
}

int pesti_gemm_q6_k_smallm(int64_t m, int64_t out_features, int64_t in_features, const void* blocks,
                           const uint16_t* x, float* y, const float* bias, void* stream) {
  return pesti_host::gemm_quant_run(PESTI_FMT_Q6_K, m, out_features, in_features, blocks, x, y, bias, nullptr,
                                    static_cast<hipStream_t>(stream));
}

}  // extern "C"
