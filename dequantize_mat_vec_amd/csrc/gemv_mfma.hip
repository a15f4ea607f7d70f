// Matrix-core mat-vec for tall Q4_K matrices (the LM head, wide projections):
// y = W x + b with W in Q4_K, x and y in float32, batch 1..8, rows of at
// most 1024 weights.
//
// The operation is the decode step's row-major matrix-vector product with
// the weights kept quantized ("Project scaffold: modules, CLI, and
// correctness harness", file summaries of tensor.rs and quant.rs); the
// block layout is the GGUF Q4_K one of "PESTI - Portable Execution
// Substrate for Transformer Inference" ("What This Is"), w = d sc q - dmin m
// per 32-weight sub-block.
//
// At batch 1 the vector-ALU kernel spends one FMA, half a convert and a
// quarter of a mask per weight, which on the 151936-row LM head is more
// time than reading its bytes.  Here the k-reduction runs on the matrix
// cores instead.  One v_mfma_f32_16x16x32_f16 k-step is one sub-block of 16
// rows: the B operand is the rows' 4-bit codes (a nibble read as an e4m3
// byte is q * 2^-9, which v_cvt_scalef32_pk_f16_fp8 turns into binary16
// exactly), the A operand is x in binary16.  binary16 cannot hold float32
// x, so x is split: each 32-weight block of x is scaled by a power of two
// 2^e (its largest magnitude lands in [2^14, 2^15)), then xs = hi + lo with
// hi = f16(xs), lo = f16(xs - hi); hi and lo of batch column b are rows 2b
// and 2b + 1 of A, so batches up to 8 share one instruction.  Every
// product q * hi, q * lo is exact in the float32 accumulator; the split
// loses at most 2^-22 |xs| + 2^-25 per element.  Per k-step and row:
//   acc_b += (d sc 2^9 2^-e) (C[2b] + C[2b+1]) - (dmin m) sum(x block)
// with the block sums of x computed in float32 while staging.
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

// One k-step of the tile: the lane's 8 codes of sub-block J (packed
// nibbles c), its x operand, and the scaled update of its two batch sums
// ((2^-e, block sum of x) per column).
template <int B, int J>
__device__ __forceinline__ void q4k_step(const u32x2& c, const u32x4& hdr, float d512, float dmin,
                                         const uint8_t* xop, const f32x2& e0, const f32x2& e1, float& acc0,
                                         float& acc1) {
  constexpr uint32_t sh = 4u * (J & 1);
  const uint32_t qa = (c.x >> sh) & 0x0F0F0F0Fu;
  const uint32_t qb = (c.y >> sh) & 0x0F0F0F0Fu;
  uint32_t h[4];
  h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qa, 1.0f, false));
  h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qa, 1.0f, true));
  h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qb, 1.0f, false));
  h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qb, 1.0f, true));
  const mhalf8 wv = __builtin_bit_cast(mhalf8, h);
  const mhalf8 xv = *reinterpret_cast<const mhalf8*>(xop);
  const mfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, mfloat4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  uint32_t sc, m;
  q4k_scale_min<J>(hdr, sc, m);
  const float ds = d512 * static_cast<float>(sc);
  const float dm = dmin * static_cast<float>(m);
  acc0 = fmaf(ds * e0.x, p[0] + p[1], acc0);
  acc0 = fmaf(-dm, e0.y, acc0);
  if constexpr (B > 1) {
    acc1 = fmaf(ds * e1.x, p[2] + p[3], acc1);
    acc1 = fmaf(-dm, e1.y, acc1);
  }
}

// NSB = super-blocks per row (every op of the launch has this many).
template <int B, int NSB>
__global__ __launch_bounds__(kMfmaThreads) void gemv_mfma_q4k_kernel(GroupArgs g) {
  extern __shared__ float lds[];
  static_assert(B >= 1 && B <= 8 && NSB >= 1 && NSB <= 4, "batch 1..8, rows of at most 1024 weights");
  // The op's arguments, all loaded before the first branch (see gemv_kernel).
  const GemvArgs a = g.op[blockIdx.y];
  asm volatile("" ::"s"(a.w), "s"(a.x), "s"(a.y), "s"(a.bias), "s"(a.out), "s"(a.in), "s"(a.row_bytes));
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kMfmaGroupRows;
  if (first >= a.out) return;   // this op has fewer tiles (uniform)
  const int nsteps = static_cast<int>(a.in >> 5);   // sub-blocks holding weights
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
    const int it = item < total ? item : 0;
    const int b = it / per_b;
    const float* src = a.x + b * a.in + 8 * (it - b * per_b);
    xv[r][0] = *reinterpret_cast<const f32x4*>(src);
    xv[r][1] = *reinterpret_cast<const f32x4*>(src + 4);
  }

  // Weights: the lane's row of the wave's tile (rows past the end read the
  // launch tile's first row and are not stored), every super-block's
  // header and the lane's 8 code bytes of each 64-weight run.
  const int64_t row = first + wave * kMfmaTileRows + n;
  const bool live = row < a.out;
  const uint8_t* rp = a.w + (live ? row : first) * a.row_bytes;
  u32x4 hdr[NSB];
  u32x2 cw[NSB][4];
#pragma unroll
  for (int S = 0; S < NSB; ++S) {
    const uint8_t* sb = rp + 144 * S;
    hdr[S] = load_u32x4_a16(sb);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) cw[S][gi] = *reinterpret_cast<const u32x2*>(sb + 16 + 32 * gi + 8 * kg);
  }
  const float bv = *(a.bias ? a.bias + (live ? row : first) : reinterpret_cast<const float*>(rp));

  // Stage x: operand rows [nsteps][2B][32 binary16] (64 bytes each), a zero
  // row for the lanes of unused A rows, then (2^-e, block sum) per [b][s].
  uint8_t* base = reinterpret_cast<uint8_t*>(lds);
  const int op_bytes = nsteps * 2 * B * 64;
  uint8_t* zero_row = base + op_bytes;
  f32x2* xsc = reinterpret_cast<f32x2*>(base + op_bytes + 64);
  if (tid < 16) reinterpret_cast<float*>(zero_row)[tid] = 0.f;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int item = tid + r * kMfmaThreads;
    const float v[8] = {xv[r][0].x, xv[r][0].y, xv[r][0].z, xv[r][0].w,
                        xv[r][1].x, xv[r][1].y, xv[r][1].z, xv[r][1].w};
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
    float sm = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    // the block's 4 quarters sit in 4 consecutive lanes
    mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 2, kWave));
    sm += __shfl_xor(sm, 1, kWave);
    sm += __shfl_xor(sm, 2, kWave);
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
      if (q == 0) xsc[b * nsteps + s] = f32x2{ldexpf(1.0f, -e), sm};
    }
  }
  __syncthreads();

  // Lane (n, kg): A row n (x hi/lo of batch n / 2, or the zero row), batch
  // columns 2kg and 2kg + 1 (clamped to a real column; unused ones are not
  // stored).
  const bool arow = n < 2 * B;
  const uint8_t* xop = arow ? base + n * 64 + 16 * kg : zero_row + 16 * kg;
  const int xstep = arow ? 2 * B * 64 : 0;
  const int b0 = 2 * kg, b1 = 2 * kg + 1;
  const f32x2* xs0 = xsc + (b0 < B ? b0 : B - 1) * nsteps;
  const f32x2* xs1 = xsc + (b1 < B ? b1 : B - 1) * nsteps;
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int S = 0; S < NSB; ++S) {
    const float d512 = f16_lo(hdr[S].x) * 512.0f;
    const float dmin = f16_hi(hdr[S].x);
    const int s0 = 8 * S;
    // Sub-blocks past in (a padded super-block) are skipped (uniform).
#define PESTI_Q4K_STEP(J)                                                                          \
    if (s0 + J < nsteps)                                                                           \
      q4k_step<B, J>(cw[S][J / 2], hdr[S], d512, dmin, xop + (s0 + J) * xstep, xs0[s0 + J], xs1[s0 + J], \
                     acc0, acc1);
    PESTI_Q4K_STEP(0) PESTI_Q4K_STEP(1) PESTI_Q4K_STEP(2) PESTI_Q4K_STEP(3)
    PESTI_Q4K_STEP(4) PESTI_Q4K_STEP(5) PESTI_Q4K_STEP(6) PESTI_Q4K_STEP(7)
#undef PESTI_Q4K_STEP
  }
  if (live) {
    const float bias = a.bias ? bv : 0.f;
    if (b0 < B) a.y[b0 * a.out + row] = acc0 + bias;
    if (b1 < B) a.y[b1 * a.out + row] = acc1 + bias;
  }
}

}  // namespace pesti

namespace pesti_gemv {

template <int B, int NSB>
int launch_mfma_bn(const GroupArgs& g, hipStream_t st) {
  int64_t max_in = 0, max_out = 0;
  for (int i = 0; i < g.n_ops; ++i) {
    max_in = g.op[i].in > max_in ? g.op[i].in : max_in;
    max_out = g.op[i].out > max_out ? g.op[i].out : max_out;
  }
  const int64_t nsteps = max_in / 32;
  const size_t lds = static_cast<size_t>(nsteps * 2 * B * 64 + 64 + 8 * B * nsteps);
  const int64_t tiles = (max_out + pesti::kMfmaGroupRows - 1) / pesti::kMfmaGroupRows;
  GroupArgs args = g;
  void* params[] = {&args};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemv_mfma_q4k_kernel<B, NSB>),
                                       dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(g.n_ops)),
                                       dim3(pesti::kMfmaThreads), params, lds, st);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <int NSB>
int launch_mfma_n(const GroupArgs& g, int batch, hipStream_t st) {
  switch (batch) {
    case 1: return launch_mfma_bn<1, NSB>(g, st);
    case 2: return launch_mfma_bn<2, NSB>(g, st);
    case 3: return launch_mfma_bn<3, NSB>(g, st);
    case 4: return launch_mfma_bn<4, NSB>(g, st);
    case 5: return launch_mfma_bn<5, NSB>(g, st);
    case 6: return launch_mfma_bn<6, NSB>(g, st);
    case 7: return launch_mfma_bn<7, NSB>(g, st);
    case 8: return launch_mfma_bn<8, NSB>(g, st);
    default: return PESTI_ERR_BATCH;
  }
}

int launch_mfma_q4_k(const GroupArgs& g, int batch, hipStream_t st) {
  if (g.n_ops < 1 || g.op[0].row_bytes % 144 != 0) return PESTI_ERR_SHAPE;
  switch (g.op[0].row_bytes / 144) {
    case 1: return launch_mfma_n<1>(g, batch, st);
    case 2: return launch_mfma_n<2>(g, batch, st);
    case 3: return launch_mfma_n<3>(g, batch, st);
    case 4: return launch_mfma_n<4>(g, batch, st);
    default: return PESTI_ERR_SHAPE;
  }
}

}  // namespace pesti_gemv
