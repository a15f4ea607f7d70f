// Matrix-core mat-vec for tall K-quant (Q2_K to Q6_K), Q8_0 and per-row
// INT4 matrices (the LM head):
// y = W x + b with W in one of those formats, x and y in float32, batch
// 1..8, rows of at most 1024 weights.
//
// The operation is the decode step's row-major matrix-vector product with
// the weights kept quantized ("Project scaffold: modules, CLI, and
// correctness harness", file summaries of tensor.rs and quant.rs); the
// block layouts are the GGUF ones of "PESTI - Portable Execution
// Substrate for Transformer Inference" ("What This Is"): Q4_K w = d sc q -
// dmin m per 32-weight sub-block (Q5_K the same with 5-bit codes), Q6_K
// w = d sc (q - 32), Q2_K w = d sc q - dmin m and Q3_K w = d (sc - 32) q
// per 16 weights (described at MfmaQ5K, MfmaQ6K, MfmaQ2K and MfmaQ3K).
//
// The vector-ALU kernel spends one FMA per weight and batch column, so on
// the 151936-row LM head its time grows with the batch well past the time
// of reading the bytes.  Here the k-reduction runs on the matrix cores,
// where up to 8 batch columns share each instruction; the group entry
// points choose this kernel from batch 3 (Q2_K, Q3_K, Q4_K, Q5_K), 4 (Q8_0
// rows of an even block count), 5 (Q6_K) and 2 (per-row INT4), below which
// the vector-ALU kernel is faster.  One v_mfma_f32_16x16x32_f16 k-step is one sub-block of 16
// rows: the B operand is the rows' 4-bit codes less the sub-block's
// nearest_code c (a nibble read as an e4m3 byte is q * 2^-9, which
// v_cvt_scalef32_pk_f16_fp8 turns into binary16 exactly; subtracting
// c 2^-9 is exact too), the A operand is x in binary16.  binary16 cannot hold float32
// x, so x is split: each 32-weight block of x is scaled by a power of two
// 2^e (its largest magnitude lands in [2^14, 2^15)), then xs = hi + lo with
// hi = f16(xs), lo = f16(xs - hi); hi and lo of batch column b are rows 2b
// and 2b + 1 of A, so batches up to 8 share one instruction.  Every
// product q * hi, q * lo is exact in the float32 accumulator; the split
// loses at most 2^-22 |xs| + 2^-25 per element.  Per k-step and row:
//   acc_b += (d sc 2^9 2^-e) (C[2b] + C[2b+1]) + (d sc c - dmin m) sum(x block)
// with the block sums of x computed in float32 while staging; the second
// term is exactly 0 for a sub-block whose weights are all 0.
//
// Layout (MFMA operand layout, lane l: n = l % 16, kg = l / 16): A = row n
// of the staged x operand, k = 8kg..8kg+7; B = W row n of the wave's 16-row
// tile, the same k (code bytes 32g + 8kg..+7 of the run g = j / 2, low
// nibbles for even sub-blocks j, high for odd); C = column n, rows
// 4kg..4kg+3, i.e. batch columns 2kg and 2kg + 1 of row n.  A workgroup is
// 8 waves = 128 rows; all of a lane's code and header loads are issued
// before x is staged, so a launch costs one memory round trip.
#include "gemv_impl.h"

namespace pesti {

typedef _Float16 mhalf8 __attribute__((ext_vector_type(8)));
typedef _Float16 mhalf2 __attribute__((ext_vector_type(2)));
typedef float mfloat4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(8)));

// Wavefronts per workgroup: a workgroup stages x once and serves 16 rows
// per wave.  Measured on the 151936 x 896 LM head (batch 1 / 4 / 8): 1 wave
// 26.3 / 42.3 / 82.2 us, 2 waves 24.7 / 32.2 / 44.4, 4 waves 24.9 / 28.2 /
// 31.3, 8 waves 24.7 / 26.3 / 30.0, 16 waves 35.3 / 36.9 / 37.8.
#ifndef PESTI_MFMA_WAVES
#define PESTI_MFMA_WAVES 8
#endif
constexpr int kMfmaWaves = PESTI_MFMA_WAVES;
constexpr int kMfmaThreads = kMfmaWaves * kWave;
constexpr int kMfmaTileRows = 16;
constexpr int kMfmaGroupRows = kMfmaWaves * kMfmaTileRows;

// Scale and min of sub-block j (0..7) from the header dwords y, z, w
// (bytes S[0..11]): j < 4: sc = S[j] & 63, m = S[j+4] & 63; j >= 4:
// sc = (S[j+4] & 15) | (S[j-4] >> 6) << 4, m = (S[j+4] >> 4) | (S[j] >> 6) << 4.
template <int J>
__device__ __forceinline__ void q4k_scale_min(const u32x4& h, uint32_t& sc, uint32_t& m) {
  auto byte = [&](int k) -> uint32_t {
    const uint32_t w = k < 4 ? h.y : (k < 8 ? h.z : h.w);
    return (w >> (8 * (k & 3))) & 0xFFu;
  };
  if constexpr (J < 4) {
    sc = byte(J) & 63u;
    m = byte(J + 4) & 63u;
  } else {
    sc = (byte(J + 4) & 15u) | (byte(J - 4) >> 6) << 4;
    m = (byte(J + 4) >> 4) | (byte(J) >> 6) << 4;
  }
}

// Packed binary16 pair (v, v) of a float32 value exact in binary16.
__device__ __forceinline__ uint32_t f16_pair(float v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(v, v));
}

// One k-step of the tile: the lane's 8 codes of sub-block J (packed
// nibbles c), its x operand, and the scaled update of its two batch sums
// ((2^-e, block sum of x) per column).  The codes enter as (q - c) 2^-9,
// c = nearest_code of the sub-block: a binary16 subtraction of exact
// values.
template <int B, int J>
__device__ __forceinline__ void q4k_step(const u32x2& c, const u32x4& hdr, float d, float dmin,
                                         const uint8_t* xop, const f32x2& e0, const f32x2& e1, float& acc0,
                                         float& acc1) {
  constexpr uint32_t sh = 4u * (J & 1);
  uint32_t sc, m;
  q4k_scale_min<J>(hdr, sc, m);
  const float ds = d * static_cast<float>(sc);
  const float dm = dmin * static_cast<float>(m);
  const float cq = nearest_code(dm, ds, 15.f);
  const mhalf2 off = __builtin_bit_cast(mhalf2, f16_pair(cq * (1.0f / 512.0f)));
  const uint32_t qa = (c.x >> sh) & 0x0F0F0F0Fu;
  const uint32_t qb = (c.y >> sh) & 0x0F0F0F0Fu;
  mhalf2 h[4];
  h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qa, 1.0f, false) - off;
  h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qa, 1.0f, true) - off;
  h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qb, 1.0f, false) - off;
  h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qb, 1.0f, true) - off;
  const mhalf8 wv = __builtin_bit_cast(mhalf8, h);
  const mhalf8 xv = *reinterpret_cast<const mhalf8*>(xop);
  const mfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  const float ds512 = ds * 512.0f;
  const float rest = fmaf(ds, cq, -dm);   // ds c - dm, exactly 0 when the sub-block cancels
  acc0 = fmaf(ds512 * e0.x, p[0] + p[1], acc0);
  acc0 = fmaf(rest, e0.y, acc0);
  if constexpr (B > 1) {
    acc1 = fmaf(ds512 * e1.x, p[2] + p[3], acc1);
    acc1 = fmaf(rest, e1.y, acc1);
  }
}

// ---------------------------------------------------------------------------
// Per-format parts of the kernel: a row's loads (every super-block of the
// lane's row, issued at once) and its k-steps.  xa / xb: the lane's x
// operand for the step's product(s) (see the kernel), es0 / es1: (2^-e,
// block sum) of the lane's two batch columns per block.
// ---------------------------------------------------------------------------
struct MfmaQ4K {
  static constexpr int kBytes = 144;
  template <int NSB>
  struct Tile {
    u32x4 hdr[NSB];
    u32x2 cw[NSB][4];
  };
  // the header and the lane's 8 code bytes of each 64-weight run
  template <int NSB>
  __device__ __forceinline__ static void issue(const uint8_t* rp, int kg, Tile<NSB>& w) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const uint8_t* sb = rp + 144 * S;
      w.hdr[S] = load_u32x4_a16(sb);
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        w.cw[S][gi] = *reinterpret_cast<const u32x2*>(sb + 16 + 32 * gi + 8 * kg);
    }
  }
  template <int B, int NSB>
  __device__ __forceinline__ static void run(const Tile<NSB>& w, int nsteps, const uint8_t* xa, int xsa,
                                             const uint8_t*, int, const f32x2* es0, const f32x2* es1,
                                             float& acc0, float& acc1) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const float d = f16_lo(w.hdr[S].x);
      const float dmin = f16_hi(w.hdr[S].x);
      const int s0 = 8 * S;
      // A whole super-block runs its 8 steps as straight-line code (they
      // overlap); the padded last one tests each step (uniform).
#define PESTI_Q4K_STEP(J)                                                                          \
        q4k_step<B, J>(w.cw[S][J / 2], w.hdr[S], d, dmin, xa + (s0 + J) * xsa, es0[s0 + J],        \
                       es1[s0 + J], acc0, acc1);
      if (s0 + 8 <= nsteps) {
        PESTI_Q4K_STEP(0) PESTI_Q4K_STEP(1) PESTI_Q4K_STEP(2) PESTI_Q4K_STEP(3)
        PESTI_Q4K_STEP(4) PESTI_Q4K_STEP(5) PESTI_Q4K_STEP(6) PESTI_Q4K_STEP(7)
      } else {
        if (s0 + 0 < nsteps) PESTI_Q4K_STEP(0) if (s0 + 1 < nsteps) PESTI_Q4K_STEP(1)
        if (s0 + 2 < nsteps) PESTI_Q4K_STEP(2) if (s0 + 3 < nsteps) PESTI_Q4K_STEP(3)
        if (s0 + 4 < nsteps) PESTI_Q4K_STEP(4) if (s0 + 5 < nsteps) PESTI_Q4K_STEP(5)
        if (s0 + 6 < nsteps) PESTI_Q4K_STEP(6)
      }
#undef PESTI_Q4K_STEP
    }
  }
};

// Q6_K (210-byte super-blocks: ql[128], qh[64], int8 sc[16], d).  k-step
// s = 8S + 4h + g covers weights 128h + 32g + l, l = 0..31, of super-block
// S: low 4 bits in ql[64h + 32(g % 2) + l] (low nibble for g < 2, high
// for g >= 2), high 2 bits at bit 2g of qh[32h + l].  Lane kg holds
// l = 8kg..8kg+7, so lanes kg < 2 belong to 16-weight sub-block 8h + 2g and
// lanes kg >= 2 to sub-block 8h + 2g + 1: each step is two products with
// the same codes, one against x with the second half's lanes pointed at a
// zero row (xa), one with the first half's (xb), each scaled by its own
// d sc.  The codes enter as q - 32 (binary16 1024 + q built by a byte
// permute, minus 1056: exact).  Super-blocks sit 2 bytes off a dword
// boundary every other one; their pieces are read with 2-byte-aligned
// loads.
typedef uint32_t u32x2u2 __attribute__((ext_vector_type(2), aligned(2)));

__device__ __forceinline__ uint32_t q6k_pair(uint32_t q, uint32_t sel) {
  // bytes [q_i, 0x64, q_j, 0x64]: binary16 1024 + q_i, 1024 + q_j; minus 1056
  const uint32_t v = __builtin_amdgcn_perm(0x64646464u, q, sel);
  const mhalf2 h = __builtin_bit_cast(mhalf2, v) + mhalf2{static_cast<_Float16>(-1056.0f),
                                                          static_cast<_Float16>(-1056.0f)};
  return __builtin_bit_cast(uint32_t, h);
}

struct MfmaQ6K {
  static constexpr int kBytes = 210;
  template <int NSB>
  struct Tile {
    u32x2u2 lo[NSB][2][2];   // [S][h][g % 2]: ql bytes 64h + 32(g % 2) + 8kg..+7
    u32x2u2 hq[NSB][2];      // [S][h]: qh bytes 128 + 32h + 8kg..+7
    u32x4u2 sc[NSB];         // the 16 scales
    uint32_t d[NSB];
  };
  template <int NSB>
  __device__ __forceinline__ static void issue(const uint8_t* rp, int kg, Tile<NSB>& w) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const uint8_t* sb = rp + 210 * S;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        w.lo[S][h][0] = *reinterpret_cast<const u32x2u2*>(sb + 64 * h + 8 * kg);
        w.lo[S][h][1] = *reinterpret_cast<const u32x2u2*>(sb + 64 * h + 32 + 8 * kg);
        w.hq[S][h] = *reinterpret_cast<const u32x2u2*>(sb + 128 + 32 * h + 8 * kg);
      }
      w.sc[S] = *reinterpret_cast<const u32x4u2*>(sb + 192);
      w.d[S] = load_u16(sb + 208);
    }
  }
  template <int B, int H, int G>
  __device__ __forceinline__ static void step(const u32x2u2& l, const u32x2u2& hq, const u32x4u2& scv, float d,
                                              const uint8_t* xa, const uint8_t* xb, const f32x2& e0,
                                              const f32x2& e1, float& acc0, float& acc1) {
    constexpr int kLoShift = 4 * (G >> 1);
    constexpr int kHiShift = 2 * G;
    const uint32_t q0 = ((l.x >> kLoShift) & 0x0F0F0F0Fu) | (((hq.x >> kHiShift) & 0x03030303u) << 4);
    const uint32_t q1 = ((l.y >> kLoShift) & 0x0F0F0F0Fu) | (((hq.y >> kHiShift) & 0x03030303u) << 4);
    uint32_t hw[4];
    hw[0] = q6k_pair(q0, 0x04010400u);
    hw[1] = q6k_pair(q0, 0x04030402u);
    hw[2] = q6k_pair(q1, 0x04010400u);
    hw[3] = q6k_pair(q1, 0x04030402u);
    const mhalf8 wv = __builtin_bit_cast(mhalf8, hw);
    const mhalf8 x0 = *reinterpret_cast<const mhalf8*>(xa);
    const mhalf8 x1 = *reinterpret_cast<const mhalf8*>(xb);
    const mfloat4 pa = __builtin_amdgcn_mfma_f32_16x16x32_f16(x0, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    const mfloat4 pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(x1, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    // scales 8H + 2G and 8H + 2G + 1: bytes 2G, 2G + 1 of dword 2H + G / 2
    constexpr int kSc = 8 * H + 2 * G;
    const uint32_t sw = kSc < 4 ? scv.x : (kSc < 8 ? scv.y : (kSc < 12 ? scv.z : scv.w));
    const float da = d * static_cast<float>(static_cast<int8_t>(sw >> (8 * (kSc & 3))));
    const float db = d * static_cast<float>(static_cast<int8_t>(sw >> (8 * ((kSc & 3) + 1))));
    acc0 = fmaf(e0.x, fmaf(da, pa[0] + pa[1], db * (pb[0] + pb[1])), acc0);
    if constexpr (B > 1) acc1 = fmaf(e1.x, fmaf(da, pa[2] + pa[3], db * (pb[2] + pb[3])), acc1);
  }
  template <int B, int NSB>
  __device__ __forceinline__ static void run(const Tile<NSB>& w, int nsteps, const uint8_t* xa, int xsa,
                                             const uint8_t* xb, int xsb, const f32x2* es0, const f32x2* es1,
                                             float& acc0, float& acc1) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const float d = f16_lo(w.d[S]);
      const int s0 = 8 * S;
      // A whole super-block runs its 8 steps as straight-line code (they
      // overlap); the padded last one tests each step (uniform).
#define PESTI_Q6K_STEP(H, G)                                                                       \
        step<B, H, G>(w.lo[S][H][G & 1], w.hq[S][H], w.sc[S], d, xa + (s0 + 4 * H + G) * xsa,       \
                      xb + (s0 + 4 * H + G) * xsb, es0[s0 + 4 * H + G], es1[s0 + 4 * H + G], acc0, acc1);
      if (s0 + 8 <= nsteps) {
        PESTI_Q6K_STEP(0, 0) PESTI_Q6K_STEP(0, 1) PESTI_Q6K_STEP(0, 2) PESTI_Q6K_STEP(0, 3)
        PESTI_Q6K_STEP(1, 0) PESTI_Q6K_STEP(1, 1) PESTI_Q6K_STEP(1, 2) PESTI_Q6K_STEP(1, 3)
      } else {
        if (s0 + 0 < nsteps) PESTI_Q6K_STEP(0, 0) if (s0 + 1 < nsteps) PESTI_Q6K_STEP(0, 1)
        if (s0 + 2 < nsteps) PESTI_Q6K_STEP(0, 2) if (s0 + 3 < nsteps) PESTI_Q6K_STEP(0, 3)
        if (s0 + 4 < nsteps) PESTI_Q6K_STEP(1, 0) if (s0 + 5 < nsteps) PESTI_Q6K_STEP(1, 1)
        if (s0 + 6 < nsteps) PESTI_Q6K_STEP(1, 2)
      }
#undef PESTI_Q6K_STEP
    }
  }
};

// Q5_K (176-byte super-blocks: Q4_K's d, dmin and 12 scale/min bytes, 32
// bytes of fifth bits, then Q4_K's 128 low-nibble bytes from byte 48).
// k-step j = 2g + c of a super-block is Q4_K's: lane kg holds weights
// 64g + 32c + 8kg..+7, low 4 bits from nibble c of bytes 48 + 32g + 8kg..+7,
// fifth bit j of bytes 16 + 8kg..+7.  Codes reach 31, past the e4m3 nibble
// trick, so they enter as binary16 1024 + q (a byte permute) minus 1024:
// exact.  Scales and mins as Q4_K.
struct MfmaQ5K {
  static constexpr int kBytes = 176;
  template <int NSB>
  struct Tile {
    u32x4 hdr[NSB];
    u32x2 qs[NSB][4];
    u32x2 qh[NSB];
  };
  template <int NSB>
  __device__ __forceinline__ static void issue(const uint8_t* rp, int kg, Tile<NSB>& w) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const uint8_t* sb = rp + 176 * S;
      w.hdr[S] = load_u32x4_a16(sb);
      w.qh[S] = *reinterpret_cast<const u32x2*>(sb + 16 + 8 * kg);
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        w.qs[S][gi] = *reinterpret_cast<const u32x2*>(sb + 48 + 32 * gi + 8 * kg);
    }
  }
  __device__ __forceinline__ static uint32_t pair(uint32_t q, uint32_t sel, mhalf2 off) {
    // bytes [q_i, 0x64, q_j, 0x64]: binary16 1024 + q_i, 1024 + q_j; minus
    // 1024 + c
    const uint32_t v = __builtin_amdgcn_perm(0x64646464u, q, sel);
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(mhalf2, v) - off);
  }
  // The codes enter as q - c (c = nearest_code of the sub-block, see
  // q4k_step).
  template <int B, int J>
  __device__ __forceinline__ static void step(const u32x2& lo, const u32x2& hb, const u32x4& hdr, float d,
                                              float dmin, const uint8_t* xa, const f32x2& e0, const f32x2& e1,
                                              float& acc0, float& acc1) {
    uint32_t sc, m;
    q4k_scale_min<J>(hdr, sc, m);
    const float ds = d * static_cast<float>(sc);
    const float dm = dmin * static_cast<float>(m);
    const float cq = nearest_code(dm, ds, 31.f);
    const mhalf2 off = __builtin_bit_cast(mhalf2, f16_pair(1024.0f + cq));
    constexpr uint32_t sh = 4u * (J & 1);
    const uint32_t q0 = ((lo.x >> sh) & 0x0F0F0F0Fu) | (((hb.x >> J) & 0x01010101u) << 4);
    const uint32_t q1 = ((lo.y >> sh) & 0x0F0F0F0Fu) | (((hb.y >> J) & 0x01010101u) << 4);
    uint32_t hw[4];
    hw[0] = pair(q0, 0x04010400u, off);
    hw[1] = pair(q0, 0x04030402u, off);
    hw[2] = pair(q1, 0x04010400u, off);
    hw[3] = pair(q1, 0x04030402u, off);
    const mhalf8 wv = __builtin_bit_cast(mhalf8, hw);
    const mhalf8 xv = *reinterpret_cast<const mhalf8*>(xa);
    const mfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    const float rest = fmaf(ds, cq, -dm);
    acc0 = fmaf(ds * e0.x, p[0] + p[1], acc0);
    acc0 = fmaf(rest, e0.y, acc0);
    if constexpr (B > 1) {
      acc1 = fmaf(ds * e1.x, p[2] + p[3], acc1);
      acc1 = fmaf(rest, e1.y, acc1);
    }
  }
  template <int B, int NSB>
  __device__ __forceinline__ static void run(const Tile<NSB>& w, int nsteps, const uint8_t* xa, int xsa,
                                             const uint8_t*, int, const f32x2* es0, const f32x2* es1,
                                             float& acc0, float& acc1) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const float d = f16_lo(w.hdr[S].x);
      const float dmin = f16_hi(w.hdr[S].x);
      const int s0 = 8 * S;
      // A whole super-block runs its 8 steps as straight-line code; the
      // padded last one tests each step (uniform).
#define PESTI_Q5K_STEP(J)                                                                          \
        step<B, J>(w.qs[S][J / 2], w.qh[S], w.hdr[S], d, dmin, xa + (s0 + J) * xsa, es0[s0 + J],    \
                   es1[s0 + J], acc0, acc1);
      if (s0 + 8 <= nsteps) {
        PESTI_Q5K_STEP(0) PESTI_Q5K_STEP(1) PESTI_Q5K_STEP(2) PESTI_Q5K_STEP(3)
        PESTI_Q5K_STEP(4) PESTI_Q5K_STEP(5) PESTI_Q5K_STEP(6) PESTI_Q5K_STEP(7)
      } else {
        if (s0 + 0 < nsteps) PESTI_Q5K_STEP(0) if (s0 + 1 < nsteps) PESTI_Q5K_STEP(1)
        if (s0 + 2 < nsteps) PESTI_Q5K_STEP(2) if (s0 + 3 < nsteps) PESTI_Q5K_STEP(3)
        if (s0 + 4 < nsteps) PESTI_Q5K_STEP(4) if (s0 + 5 < nsteps) PESTI_Q5K_STEP(5)
        if (s0 + 6 < nsteps) PESTI_Q5K_STEP(6)
      }
#undef PESTI_Q5K_STEP
    }
  }
};

// Per-row INT4 (4-bit two's complement codes, two per byte - weight 2k in
// the low nibble of byte k, 2k + 1 in the high one - rows padded to 64
// weights, one float32 scale per row applied to the finished sum).  With
// no per-block scale, a k-step may take its 32 weights from anywhere: in
// each 128-weight group G a lane kg loads the 16 contiguous bytes
// 64G + 16kg..+15 (weights 128G + 32kg..+31) and k-step s = 4G + t takes
// their weights 8t..8t+7 (dword t), so step s's k-value 8kg + i is weight
// 128G + 32kg + 8t + i; the x operand is staged in that order (kGrouped),
// with its power-of-two scale per step.  XOR 0x88 per byte makes each
// nibble q + 8 (0..15); the even and odd weights' nibbles are paired by a
// byte permute into binary16 1024 + q + 8, minus 1032: q exactly.  Groups
// past the row's bytes read a stand-in (their x is zero).
struct MfmaI4 {
  static constexpr int kBytes = 128;   // a 256-weight "super-block" of the row loop
  static constexpr bool kGrouped = true;
  template <int NSB>
  struct Tile {
    u32x4 c[2 * NSB];
    float scale;
  };
  template <int NSB>
  __device__ __forceinline__ static void issue(const uint8_t* rp, int kg, Tile<NSB>& w, int64_t row_bytes,
                                               const float* scale) {
#pragma unroll
    for (int G = 0; G < 2 * NSB; ++G) {
      const int off = 64 * G + 16 * kg;
      w.c[G] = *reinterpret_cast<const u32x4*>(rp + (off + 16 <= row_bytes ? off : 0));
    }
    w.scale = *scale;
  }
  __device__ __forceinline__ static uint32_t pair(uint32_t hi, uint32_t lo, uint32_t sel) {
    const uint32_t v = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;   // 1024 + q + 8
    const mhalf2 h = __builtin_bit_cast(mhalf2, v) + mhalf2{static_cast<_Float16>(-1032.0f),
                                                            static_cast<_Float16>(-1032.0f)};
    return __builtin_bit_cast(uint32_t, h);
  }
  template <int B>
  __device__ __forceinline__ static void step(uint32_t c, const uint8_t* xa, const f32x2& e0, const f32x2& e1,
                                              float& acc0, float& acc1) {
    const uint32_t v = c ^ 0x88888888u;
    const uint32_t lo = v & 0x0F0F0F0Fu;          // weights 0, 2, 4, 6 of the lane's 8
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;   // weights 1, 3, 5, 7
    uint32_t hw[4];
    // byte selectors of v_perm_b32(hi, lo): 0..3 pick lo's bytes, 4..7 hi's, 12 a zero
    hw[0] = pair(hi, lo, 0x0C040C00u);
    hw[1] = pair(hi, lo, 0x0C050C01u);
    hw[2] = pair(hi, lo, 0x0C060C02u);
    hw[3] = pair(hi, lo, 0x0C070C03u);
    const mhalf8 wv = __builtin_bit_cast(mhalf8, hw);
    const mhalf8 xv = *reinterpret_cast<const mhalf8*>(xa);
    const mfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    acc0 = fmaf(e0.x, p[0] + p[1], acc0);
    if constexpr (B > 1) acc1 = fmaf(e1.x, p[2] + p[3], acc1);
  }
  template <int B, int NSB>
  __device__ __forceinline__ static void run(const Tile<NSB>& w, int nsteps, const uint8_t* xa, int xsa,
                                             const uint8_t*, int, const f32x2* es0, const f32x2* es1,
                                             float& acc0, float& acc1) {
#pragma unroll
    for (int G = 0; G < 2 * NSB; ++G) {
      const int s0 = 4 * G;
      if (s0 < nsteps) {   // uniform: nsteps is a multiple of 4 here
        step<B>(w.c[G].x, xa + (s0 + 0) * xsa, es0[s0 + 0], es1[s0 + 0], acc0, acc1);
        step<B>(w.c[G].y, xa + (s0 + 1) * xsa, es0[s0 + 1], es1[s0 + 1], acc0, acc1);
        step<B>(w.c[G].z, xa + (s0 + 2) * xsa, es0[s0 + 2], es1[s0 + 2], acc0, acc1);
        step<B>(w.c[G].w, xa + (s0 + 3) * xsa, es0[s0 + 3], es1[s0 + 3], acc0, acc1);
      }
    }
  }
};

// Q2_K (84-byte super-blocks: 16 scale bytes, 4-bit sc | 4-bit m << 4 per
// 16-weight sub-block; 64 code bytes; d; dmin).  k-step s = 8S + 4h + j
// covers weights 128h + 32j + l, l = 0..31, of super-block S, whose 2-bit
// codes sit at bits 2j of code byte 32h + l; lane kg's weights l = 8kg..+7
// belong to sub-block 8h + 2j + kg / 2.  The codes enter as sc (q - c)
// 2^-9 with c the lane's sub-block's nearest_code (one binary16 FMA, exact:
// |sc (q - c)| <= 45), so one product covers both sub-blocks of the step;
// the two sub-blocks' remainders ds c - dm (exactly 0 where a sub-block's
// weights all are) multiply the staged sums of x over each 16-weight half
// of the block, the other half's remainder coming from the lane 32 away
// (kg ^ 2).  Per step: acc += 2^-e d 2^9 C + r_lo sum_lo + r_hi sum_hi.
typedef uint32_t u32x2w __attribute__((ext_vector_type(2), aligned(4)));

struct MfmaQ2K {
  static constexpr int kBytes = 84;
  static constexpr bool kHalfSums = true;
  template <int NSB>
  struct Tile {
    u32x4 sc[NSB];       // the 16 scale bytes
    u32x2w q[NSB][2];    // [S][h]: code bytes 32h + 8kg..+7
    uint32_t dd[NSB];    // d | dmin << 16
    uint32_t sh;         // bit offset of the lane's sub-block in a scale byte pair
  };
  template <int NSB>
  __device__ __forceinline__ static void issue(const uint8_t* rp, int kg, Tile<NSB>& w) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const uint8_t* sb = rp + 84 * S;
      w.sc[S] = *reinterpret_cast<const u32x4*>(sb);
      w.q[S][0] = *reinterpret_cast<const u32x2w*>(sb + 16 + 8 * kg);
      w.q[S][1] = *reinterpret_cast<const u32x2w*>(sb + 48 + 8 * kg);
      w.dd[S] = *reinterpret_cast<const uint32_t*>(sb + 80);
    }
    w.sh = 8u * static_cast<uint32_t>(kg >> 1);
  }
  template <int B, int J>
  __device__ __forceinline__ static void step(const u32x2w& c, uint32_t word, uint32_t sh, float d512, float d,
                                              float dmin, const uint8_t* xop, const f32x2& e0,
                                              const f32x2& e1, const f32x2& hs0, const f32x2& hs1,
                                              float& acc0, float& acc1) {
    const uint32_t qa = (c.x >> (2 * J)) & 0x03030303u;
    const uint32_t qb = (c.y >> (2 * J)) & 0x03030303u;
    // scale bytes of sub-blocks 8h + 2j (low) and 8h + 2j + 1 (high)
    const uint32_t pair = word >> (16 * (J & 1));
    const float scf = static_cast<float>((pair >> sh) & 15u);
    const float ds = d * scf;
    const float dm = dmin * static_cast<float>((pair >> (sh + 4)) & 15u);
    const float cq = nearest_code(dm, ds, 3.f);
    const mhalf2 s2 = __builtin_bit_cast(mhalf2, f16_pair(scf));
    const mhalf2 o2 = __builtin_bit_cast(mhalf2, f16_pair(-scf * cq * (1.0f / 512.0f)));
    mhalf2 h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qa, 1.0f, false) * s2 + o2;
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qa, 1.0f, true) * s2 + o2;
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qb, 1.0f, false) * s2 + o2;
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qb, 1.0f, true) * s2 + o2;
    const mhalf8 wv = __builtin_bit_cast(mhalf8, h);
    const mhalf8 xv = *reinterpret_cast<const mhalf8*>(xop);
    const mfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    const float rest = fmaf(ds, cq, -dm);
    const float other = __shfl_xor(rest, 32, kWave);
    const bool low = sh == 0u;   // lanes kg < 2 hold the step's first sub-block
    const float r_lo = low ? rest : other, r_hi = low ? other : rest;
    acc0 = fmaf(e0.x * d512, p[0] + p[1], acc0);
    acc0 = fmaf(r_lo, hs0.x, fmaf(r_hi, hs0.y, acc0));
    if constexpr (B > 1) {
      acc1 = fmaf(e1.x * d512, p[2] + p[3], acc1);
      acc1 = fmaf(r_lo, hs1.x, fmaf(r_hi, hs1.y, acc1));
    }
  }
  template <int B, int NSB>
  __device__ __forceinline__ static void run(const Tile<NSB>& w, int nsteps, const uint8_t* xa, int xsa,
                                             const uint8_t*, int, const f32x2* es0, const f32x2* es1,
                                             const f32x2* hs0, const f32x2* hs1, float& acc0, float& acc1) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const float d = f16_lo(w.dd[S]);
      const float d512 = d * 512.0f;
      const float dmin = f16_hi(w.dd[S]);
      const int s0 = 8 * S;
#define PESTI_Q2K_STEP(H, J)                                                                       \
      step<B, J>(w.q[S][H], H == 0 ? (J < 2 ? w.sc[S].x : w.sc[S].y) : (J < 2 ? w.sc[S].z : w.sc[S].w), \
                 w.sh, d512, d, dmin, xa + (s0 + 4 * H + J) * xsa, es0[s0 + 4 * H + J], es1[s0 + 4 * H + J], \
                 hs0[s0 + 4 * H + J], hs1[s0 + 4 * H + J], acc0, acc1);
      if (s0 + 8 <= nsteps) {
        PESTI_Q2K_STEP(0, 0) PESTI_Q2K_STEP(0, 1) PESTI_Q2K_STEP(0, 2) PESTI_Q2K_STEP(0, 3)
        PESTI_Q2K_STEP(1, 0) PESTI_Q2K_STEP(1, 1) PESTI_Q2K_STEP(1, 2) PESTI_Q2K_STEP(1, 3)
      } else {
        if (s0 + 0 < nsteps) PESTI_Q2K_STEP(0, 0) if (s0 + 1 < nsteps) PESTI_Q2K_STEP(0, 1)
        if (s0 + 2 < nsteps) PESTI_Q2K_STEP(0, 2) if (s0 + 3 < nsteps) PESTI_Q2K_STEP(0, 3)
        if (s0 + 4 < nsteps) PESTI_Q2K_STEP(1, 0) if (s0 + 5 < nsteps) PESTI_Q2K_STEP(1, 1)
        if (s0 + 6 < nsteps) PESTI_Q2K_STEP(1, 2)
      }
#undef PESTI_Q2K_STEP
    }
  }
};

// Q3_K (110-byte super-blocks, 2 bytes off a dword boundary every other
// one: 32 high-bit bytes, 64 low-bit bytes as Q2_K, 12 bytes of sixteen
// 6-bit scales, d).  k-step s = 8S + 4h + j as for Q2_K: lane kg's weights
// 128h + 32j + 8kg + i (i = 0..7) take their low bits from bits 2j of code
// bytes 32 + 32h + 8kg + i and their high bit from bit 4h + j of high-bit
// bytes 8kg + i; q = low + 4 high - 4, and they belong to sub-block
// 8h + 2j + kg / 2 (scale k: low 4 bits at bit 4(k / 8) of byte k % 8, top
// 2 at bit 2(k / 4) of byte 8 + k % 4; w = d (scale - 32) q).  The byte
// low | high << 2 converts as e4m3 (b 2^-9), and one binary16 FMA by the
// lane's signed scale s = scale - 32 gives s (b - 4) 2^-9 = s q 2^-9
// exactly (|s q| <= 128), so one product covers both sub-blocks of the
// step and there is no min term: acc += 2^-e d 2^9 C.
struct MfmaQ3K {
  static constexpr int kBytes = 110;
  template <int NSB>
  struct Tile {
    u32x2u2 hm[NSB];     // high-bit bytes 8kg..+7
    u32x2u2 q[NSB][2];   // [S][h]: low-bit bytes 32 + 32h + 8kg..+7
    u32x2u2 s01[NSB];    // scale bytes 0..7
    uint32_t s2[NSB];    // scale bytes 8..11
    uint32_t d[NSB];     // binary16 d in the low half
    uint32_t c8;         // 8 (kg / 2): the lane's byte within a scale byte pair
  };
  template <int NSB>
  __device__ __forceinline__ static void issue(const uint8_t* rp, int kg, Tile<NSB>& w) {
    typedef uint32_t u32a2 __attribute__((aligned(2)));
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const uint8_t* sb = rp + 110 * S;
      w.hm[S] = *reinterpret_cast<const u32x2u2*>(sb + 8 * kg);
      w.q[S][0] = *reinterpret_cast<const u32x2u2*>(sb + 32 + 8 * kg);
      w.q[S][1] = *reinterpret_cast<const u32x2u2*>(sb + 64 + 8 * kg);
      w.s01[S] = *reinterpret_cast<const u32x2u2*>(sb + 96);
      w.s2[S] = *reinterpret_cast<const u32a2*>(sb + 104);
      w.d[S] = *reinterpret_cast<const uint16_t*>(sb + 108);
    }
    w.c8 = 8u * static_cast<uint32_t>(kg >> 1);
  }
  template <int B, int H, int J>
  __device__ __forceinline__ static void step(const u32x2u2& c, const u32x2u2& hm, uint32_t slo, uint32_t s2,
                                              uint32_t c8, float d512, const uint8_t* xop, const f32x2& e0,
                                              const f32x2& e1, float& acc0, float& acc1) {
    constexpr uint32_t hb = 4 * H + J;
    const uint32_t ba = ((c.x >> (2 * J)) & 0x03030303u) | (((hm.x >> hb) & 0x01010101u) << 2);
    const uint32_t bb = ((c.y >> (2 * J)) & 0x03030303u) | (((hm.y >> hb) & 0x01010101u) << 2);
    // scale 8h + 2j + kg/2: low 4 bits in byte 2j + kg/2 (nibble h), top 2
    // in byte 8 + 2(j % 2) + kg/2 at bit 4h + 2(j / 2)
    const uint32_t pos = 16u * (J & 1) + c8;
    const uint32_t lo4 = (slo >> (pos + 4 * H)) & 15u;
    const uint32_t hi2 = (s2 >> (pos + 4 * H + 2 * (J >> 1))) & 3u;
    const _Float16 s = static_cast<_Float16>(static_cast<float>(static_cast<int>(lo4 | hi2 << 4) - 32));
    const mhalf2 s2h{s, s};
    const _Float16 off = s * static_cast<_Float16>(-4.0f / 512.0f);
    const mhalf2 o2{off, off};
    mhalf2 h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ba, 1.0f, false) * s2h + o2;
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ba, 1.0f, true) * s2h + o2;
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bb, 1.0f, false) * s2h + o2;
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bb, 1.0f, true) * s2h + o2;
    const mhalf8 wv = __builtin_bit_cast(mhalf8, h);
    const mhalf8 xv = *reinterpret_cast<const mhalf8*>(xop);
    const mfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    acc0 = fmaf(d512 * e0.x, p[0] + p[1], acc0);
    if constexpr (B > 1) acc1 = fmaf(d512 * e1.x, p[2] + p[3], acc1);
  }
  template <int B, int NSB>
  __device__ __forceinline__ static void run(const Tile<NSB>& w, int nsteps, const uint8_t* xa, int xsa,
                                             const uint8_t*, int, const f32x2* es0, const f32x2* es1,
                                             float& acc0, float& acc1) {
#pragma unroll
    for (int S = 0; S < NSB; ++S) {
      const float d512 = f16_lo(w.d[S]) * 512.0f;
      const int s0 = 8 * S;
#define PESTI_Q3K_STEP(H, J)                                                                       \
      step<B, H, J>(w.q[S][H], w.hm[S], J < 2 ? w.s01[S].x : w.s01[S].y, w.s2[S], w.c8, d512,       \
                    xa + (s0 + 4 * H + J) * xsa, es0[s0 + 4 * H + J], es1[s0 + 4 * H + J], acc0, acc1);
      if (s0 + 8 <= nsteps) {
        PESTI_Q3K_STEP(0, 0) PESTI_Q3K_STEP(0, 1) PESTI_Q3K_STEP(0, 2) PESTI_Q3K_STEP(0, 3)
        PESTI_Q3K_STEP(1, 0) PESTI_Q3K_STEP(1, 1) PESTI_Q3K_STEP(1, 2) PESTI_Q3K_STEP(1, 3)
      } else {
        if (s0 + 0 < nsteps) PESTI_Q3K_STEP(0, 0) if (s0 + 1 < nsteps) PESTI_Q3K_STEP(0, 1)
        if (s0 + 2 < nsteps) PESTI_Q3K_STEP(0, 2) if (s0 + 3 < nsteps) PESTI_Q3K_STEP(0, 3)
        if (s0 + 4 < nsteps) PESTI_Q3K_STEP(1, 0) if (s0 + 5 < nsteps) PESTI_Q3K_STEP(1, 1)
        if (s0 + 6 < nsteps) PESTI_Q3K_STEP(1, 2)
      }
#undef PESTI_Q3K_STEP
    }
  }
};

// Q8_0 rows of an even block count (34-byte blocks: binary16 d, 32 int8
// codes).  Two blocks are 68 bytes, so pair P of a row starts on a dword
// boundary: k-step s is block s, and lane kg reads, for the even block of
// the pair, the 12 aligned bytes 68P + 8kg..+11 (its codes are bytes 2..9
// of them, realigned with two byte-aligns) and, for the odd block, the 8
// aligned bytes 68P + 36 + 8kg..+7.  The even block's d is bytes 0..1 of
// lane kg = 0's read and the odd block's bytes 10..11 of lane kg = 3's; the
// other lanes of the row take them with a shuffle.  Codes enter as binary16
// 1024 + (q + 128) from a byte permute, minus 1152: exact.  Per step:
// acc += d 2^-e C.  Pairs past the row's end read pair 0 (in bounds) and
// are skipped.
__device__ __forceinline__ uint32_t q8_pair(uint32_t u, uint32_t sel) {
  const uint32_t v = __builtin_amdgcn_perm(0x64646464u, u, sel);
  const mhalf2 h = __builtin_bit_cast(mhalf2, v) + mhalf2{static_cast<_Float16>(-1152.0f),
                                                          static_cast<_Float16>(-1152.0f)};
  return __builtin_bit_cast(uint32_t, h);
}

struct MfmaQ8 {
  static constexpr int kBytes = 272;   // 8 blocks: a 256-weight "super-block" of the row loop
  template <int NSB>
  struct Tile {
    uint32_t e[4 * NSB][3];   // even block of pair P: bytes 68P + 8kg..+11
    u32x2w o[4 * NSB];        // odd block: bytes 68P + 36 + 8kg..+7
  };
  template <int NSB>
  __device__ __forceinline__ static void issue(const uint8_t* rp, int kg, Tile<NSB>& w, int64_t row_bytes) {
#pragma unroll
    for (int P = 0; P < 4 * NSB; ++P) {
      const uint8_t* pp = rp + (68 * (P + 1) <= row_bytes ? 68 * P : 0);
      const uint32_t* ev = reinterpret_cast<const uint32_t*>(pp + 8 * kg);
      w.e[P][0] = ev[0];
      w.e[P][1] = ev[1];
      w.e[P][2] = ev[2];
      w.o[P] = *reinterpret_cast<const u32x2w*>(pp + 36 + 8 * kg);
    }
  }
  template <int B>
  __device__ __forceinline__ static void step(uint32_t c0, uint32_t c1, float d, const uint8_t* xop,
                                              const f32x2& e0, const f32x2& e1, float& acc0, float& acc1) {
    const uint32_t u0 = c0 ^ 0x80808080u, u1 = c1 ^ 0x80808080u;   // q + 128
    uint32_t hw[4];
    // byte selectors of v_perm_b32(0x64646464, u): 0..3 pick u's bytes, 4 a 0x64
    hw[0] = q8_pair(u0, 0x04010400u);
    hw[1] = q8_pair(u0, 0x04030402u);
    hw[2] = q8_pair(u1, 0x04010400u);
    hw[3] = q8_pair(u1, 0x04030402u);
    const mhalf8 wv = __builtin_bit_cast(mhalf8, hw);
    const mhalf8 xv = *reinterpret_cast<const mhalf8*>(xop);
    const mfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    acc0 = fmaf(d * e0.x, p[0] + p[1], acc0);
    if constexpr (B > 1) acc1 = fmaf(d * e1.x, p[2] + p[3], acc1);
  }
  template <int B, int NSB>
  __device__ __forceinline__ static void run(const Tile<NSB>& w, int nsteps, const uint8_t* xa, int xsa,
                                             const uint8_t*, int, const f32x2* es0, const f32x2* es1,
                                             float& acc0, float& acc1) {
    const int n = static_cast<int>(__lane_id()) & 15;
#pragma unroll
    for (int P = 0; P < 4 * NSB; ++P) {
      const int s = 2 * P;
      if (s < nsteps) {   // uniform; nsteps is even here
        const float de = f16_lo(static_cast<uint32_t>(__shfl(static_cast<int>(w.e[P][0]), n, kWave)));
        const float dodd = f16_hi(static_cast<uint32_t>(__shfl(static_cast<int>(w.e[P][2]), n + 48, kWave)));
        const uint32_t c0 = __builtin_amdgcn_alignbyte(w.e[P][1], w.e[P][0], 2);
        const uint32_t c1 = __builtin_amdgcn_alignbyte(w.e[P][2], w.e[P][1], 2);
        step<B>(c0, c1, de, xa + s * xsa, es0[s], es1[s], acc0, acc1);
        step<B>(w.o[P].x, w.o[P].y, dodd, xa + (s + 1) * xsa, es0[s + 1], es1[s + 1], acc0, acc1);
      }
    }
  }
};

// Formats that take the sums of x over each 16-weight half of a block.
template <class P, class = void>
struct HalfSums { static constexpr bool value = false; };
template <class P>
struct HalfSums<P, std::void_t<decltype(P::kHalfSums)>> { static constexpr bool value = P::kHalfSums; };
template <class P>
constexpr bool kHalfSumsOf = HalfSums<P>::value;

// Formats whose x is staged in 128-weight groups (see MfmaI4) and whose
// rows carry a float32 scale.
template <class P>
constexpr bool kGroupedX = std::is_same<P, MfmaI4>::value;

// Index in x of staged item (block s, quarter q): 32 s + 8 q, or for x
// staged in 128-weight groups 128 (s / 4) + 32 q + 8 (s % 4).
template <bool kGrouped>
__device__ __forceinline__ int x_index(int s, int q) {
  return kGrouped ? 128 * (s >> 2) + 32 * q + 8 * (s & 3) : 32 * s + 8 * q;
}

// P = format, NSB = super-blocks per row (every op of the launch has this
// many).
template <class P, int B, int NSB>
__global__ __launch_bounds__(kMfmaThreads) void gemv_mfma_kernel(GroupArgs g) {
  extern __shared__ float lds[];
  static_assert(B >= 1 && B <= 8 && NSB >= 1 && NSB <= 4, "batch 1..8, rows of at most 1024 weights");
  // The op's arguments, all loaded before the first branch (see gemv_kernel).
  const GemvArgs a = g.op[blockIdx.y];
  asm volatile("" ::"s"(a.w), "s"(a.x), "s"(a.y), "s"(a.bias), "s"(a.out), "s"(a.in), "s"(a.row_bytes));
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kMfmaGroupRows;
  if (first >= a.out) return;   // this op has fewer tiles (uniform)
  // k-steps: 32-weight blocks holding weights (whole 128-weight groups for
  // grouped x)
  const int nsteps = kGroupedX<P> ? static_cast<int>(4 * ((a.in + 127) >> 7)) : static_cast<int>(a.in >> 5);
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int kg = lane >> 4;

  // x, first: work item (b, s, q) = batch column b, block s, quarter q
  // (8 floats at 32 s + 8 q); items past the end load item 0 (in bounds)
  // and store nothing.  Branch-free, so the weight loads below are issued
  // while x is in flight.
  constexpr int kRounds = (32 * B * NSB + kMfmaThreads - 1) / kMfmaThreads;   // B * nsteps * 4 <= 32 B NSB items
  const int per_b = nsteps * 4;
  const int total = B * per_b;
  f32x4 xv[kRounds][2];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int item = tid + r * kMfmaThreads;
    const int b = item / per_b;
    const int rem = item - b * per_b;   // 4 s + q
    const int idx = x_index<kGroupedX<P>>(rem >> 2, rem & 3);
    const bool real = item < total && idx < a.in;
    const float* src = real ? a.x + b * a.in + idx : a.x;
    xv[r][0] = *reinterpret_cast<const f32x4*>(src);
    xv[r][1] = *reinterpret_cast<const f32x4*>(src + 4);
  }

  // Weights: the lane's row of the wave's tile (rows past the end read the
  // launch tile's first row and are not stored).
  const int64_t row = first + wave * kMfmaTileRows + n;
  const bool live = row < a.out;
  const uint8_t* rp = a.w + (live ? row : first) * a.row_bytes;
  typename P::template Tile<NSB> w;
  if constexpr (kGroupedX<P>) {
    // with the row's scale (rows past the end read the tile's first row's)
    P::template issue<NSB>(rp, kg, w, a.row_bytes, a.scales + (live ? row : first));
  } else if constexpr (std::is_same<P, MfmaQ8>::value) {
    P::template issue<NSB>(rp, kg, w, a.row_bytes);
  } else {
    P::template issue<NSB>(rp, kg, w);
  }
  const float bv = *(a.bias ? a.bias + (live ? row : first) : reinterpret_cast<const float*>(rp));

  // Stage x: operand rows [nsteps][2B][32 binary16] (64 bytes each), a zero
  // row for the lanes of unused A rows, then (2^-e, block sum) per [b][s].
  uint8_t* base = reinterpret_cast<uint8_t*>(lds);
  const int op_bytes = nsteps * 2 * B * 64;
  uint8_t* zero_row = base + op_bytes;
  f32x2* xsc = reinterpret_cast<f32x2*>(base + op_bytes + 64);
  f32x2* hsc = xsc + B * nsteps;   // per-16 sums of x (formats with 16-weight sub-blocks)
  if (tid < 16) reinterpret_cast<float*>(zero_row)[tid] = 0.f;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int item = tid + r * kMfmaThreads;
    const int rem0 = item % per_b;
    const bool real = item < total && x_index<kGroupedX<P>>(rem0 >> 2, rem0 & 3) < a.in;
    float v[8] = {xv[r][0].x, xv[r][0].y, xv[r][0].z, xv[r][0].w,
                  xv[r][1].x, xv[r][1].y, xv[r][1].z, xv[r][1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = real ? v[i] : 0.f;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
    float sm = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    // the block's 4 quarters sit in 4 consecutive lanes
    mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 2, kWave));
    sm += __shfl_xor(sm, 1, kWave);   // the sum of the lane's 16-weight half
    const float other_half = __shfl_xor(sm, 2, kWave);
    const f32x2 halves{sm, other_half};   // (first, second) in quarter 0's lane
    sm += other_half;
    int e = 0;
    if (mx > 0.f) {
      int E;
      (void)frexpf(mx, &E);   // mx = f 2^E, f in [0.5, 1)
      e = 15 - E;
      e = e < -126 ? -126 : (e > 126 ? 126 : e);
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = ldexpf(v[2 * i], e), x1 = ldexpf(v[2 * i + 1], e);
      const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
      const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
      const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
      hi[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
              static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16;
      lo[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l0)) |
              static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16;
    }
    if (item < total) {
      const int b = item / per_b;
      const int rem = item - b * per_b;
      const int s = rem >> 2, q = rem & 3;
      uint8_t* dst = base + (s * 2 * B + 2 * b) * 64 + 16 * q;
      *reinterpret_cast<u32x4a*>(dst) = u32x4a{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<u32x4a*>(dst + 64) = u32x4a{lo[0], lo[1], lo[2], lo[3]};
      if (q == 0) {
        xsc[b * nsteps + s] = f32x2{ldexpf(1.0f, -e), sm};
        if constexpr (kHalfSumsOf<P>) hsc[b * nsteps + s] = halves;
      }
    }
  }
  __syncthreads();

  // Lane (n, kg): A row n (x hi/lo of batch n / 2, or the zero row), batch
  // columns 2kg and 2kg + 1 (clamped to a real column; unused ones are not
  // stored).  xa / xb: the operand with lanes kg >= 2 / kg < 2 at the zero
  // row (Q6_K's two sub-blocks per step); Q4_K uses the whole operand.
  const bool arow = n < 2 * B;
  const uint8_t* xop = arow ? base + n * 64 + 16 * kg : zero_row + 16 * kg;
  const int xstep = arow ? 2 * B * 64 : 0;
  const bool half0 = kg < 2;
  const uint8_t* xa = std::is_same<P, MfmaQ6K>::value && !half0 ? zero_row + 16 * kg : xop;
  const int xsa = std::is_same<P, MfmaQ6K>::value && !half0 ? 0 : xstep;
  const uint8_t* xb = half0 ? zero_row + 16 * kg : xop;
  const int xsb = half0 ? 0 : xstep;
  const int b0 = 2 * kg, b1 = 2 * kg + 1;
  const f32x2* xs0 = xsc + (b0 < B ? b0 : B - 1) * nsteps;
  const f32x2* xs1 = xsc + (b1 < B ? b1 : B - 1) * nsteps;
  float acc0 = 0.f, acc1 = 0.f;
  if constexpr (kHalfSumsOf<P>) {
    P::template run<B, NSB>(w, nsteps, xa, xsa, xb, xsb, xs0, xs1, hsc + (xs0 - xsc), hsc + (xs1 - xsc),
                            acc0, acc1);
  } else {
    P::template run<B, NSB>(w, nsteps, xa, xsa, xb, xsb, xs0, xs1, acc0, acc1);
  }
  if constexpr (kGroupedX<P>) {
    acc0 *= w.scale;
    acc1 *= w.scale;
  }
  if (live) {
    const float bias = a.bias ? bv : 0.f;
    if (b0 < B) a.y[b0 * a.out + row] = acc0 + bias;
    if (b1 < B) a.y[b1 * a.out + row] = acc1 + bias;
  }
}

}  // namespace pesti

namespace pesti_gemv {

template <class P, int B, int NSB>
int launch_mfma_bn(const GroupArgs& g, hipStream_t st) {
  int64_t max_in = 0, max_out = 0;
  for (int i = 0; i < g.n_ops; ++i) {
    max_in = g.op[i].in > max_in ? g.op[i].in : max_in;
    max_out = g.op[i].out > max_out ? g.op[i].out : max_out;
  }
  const int64_t nsteps = pesti::kGroupedX<P> ? 4 * ((max_in + 127) / 128) : max_in / 32;
  const size_t lds = static_cast<size_t>(nsteps * 2 * B * 64 + 64 + 8 * B * nsteps * (pesti::kHalfSumsOf<P> ? 2 : 1));
  const int64_t tiles = (max_out + pesti::kMfmaGroupRows - 1) / pesti::kMfmaGroupRows;
  GroupArgs args = g;
  void* params[] = {&args};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemv_mfma_kernel<P, B, NSB>),
                                       dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(g.n_ops)),
                                       dim3(pesti::kMfmaThreads), params, lds, st);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <class P, int NSB>
int launch_mfma_n(const GroupArgs& g, int batch, hipStream_t st) {
  switch (batch) {
    case 1: return launch_mfma_bn<P, 1, NSB>(g, st);
    case 2: return launch_mfma_bn<P, 2, NSB>(g, st);
    case 3: return launch_mfma_bn<P, 3, NSB>(g, st);
    case 4: return launch_mfma_bn<P, 4, NSB>(g, st);
    case 5: return launch_mfma_bn<P, 5, NSB>(g, st);
    case 6: return launch_mfma_bn<P, 6, NSB>(g, st);
    case 7: return launch_mfma_bn<P, 7, NSB>(g, st);
    case 8: return launch_mfma_bn<P, 8, NSB>(g, st);
    default: return PESTI_ERR_BATCH;
  }
}

template <class P>
int launch_mfma_p(const GroupArgs& g, int batch, hipStream_t st) {
  if (g.n_ops < 1) return PESTI_ERR_SHAPE;
  // per-row INT4 rows are whole 64-weight units and may end inside a
  // 256-weight group of the row loop; the other formats' rows are whole
  // super-blocks
  if (!pesti::kGroupedX<P> && !std::is_same<P, pesti::MfmaQ8>::value && g.op[0].row_bytes % P::kBytes != 0)
    return PESTI_ERR_SHAPE;
  switch ((g.op[0].row_bytes + P::kBytes - 1) / P::kBytes) {
    case 1: return launch_mfma_n<P, 1>(g, batch, st);
    case 2: return launch_mfma_n<P, 2>(g, batch, st);
    case 3: return launch_mfma_n<P, 3>(g, batch, st);
    case 4: return launch_mfma_n<P, 4>(g, batch, st);
    default: return PESTI_ERR_SHAPE;
  }
}

int launch_mfma_q4_k(const GroupArgs& g, int batch, hipStream_t st) {
  return launch_mfma_p<pesti::MfmaQ4K>(g, batch, st);
}

int launch_mfma_q6_k(const GroupArgs& g, int batch, hipStream_t st) {
  return launch_mfma_p<pesti::MfmaQ6K>(g, batch, st);
}

int launch_mfma_q5_k(const GroupArgs& g, int batch, hipStream_t st) {
  return launch_mfma_p<pesti::MfmaQ5K>(g, batch, st);
}

int launch_mfma_i4row(const GroupArgs& g, int batch, hipStream_t st) {
  return launch_mfma_p<pesti::MfmaI4>(g, batch, st);
}

int launch_mfma_q2_k(const GroupArgs& g, int batch, hipStream_t st) {
  return launch_mfma_p<pesti::MfmaQ2K>(g, batch, st);
}

int launch_mfma_q3_k(const GroupArgs& g, int batch, hipStream_t st) {
  return launch_mfma_p<pesti::MfmaQ3K>(g, batch, st);
}

int launch_mfma_q8_0(const GroupArgs& g, int batch, hipStream_t st) {
  return launch_mfma_p<pesti::MfmaQ8>(g, batch, st);
}

}  // namespace pesti_gemv
