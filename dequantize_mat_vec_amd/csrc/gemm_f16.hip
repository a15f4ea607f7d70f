// Small-M binary16 linear layer Y = X W^T + b ("inferno" README,
// "Benchmarks": linear = x @ w + b at prompt width, e.g. 32x768 @ 768x2304,
// which the page names as where the prefill time goes).  X binary16 [m][K],
// W binary16 [N][K] (same row orientation as the mat-vec), Y float32 [m][N],
// float32 accumulation.
//
// For m >= 16 the product is a dense contraction and runs on the matrix
// cores (v_mfma_f32_16x16x32_f16); below 16 rows the matrix cores would
// idle most of their rows, so a vector-ALU kernel treats the rows of X as a
// batch of mat-vecs over binary16 weights.
#include "gemm_wide.h"

namespace pesti {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint16_t* w;   // [N][K]
  const uint16_t* x;   // [M][K]
  float* y;            // [M][N]
  const float* bias;   // [N] or null
  int64_t m, n, k;
};

// MFMA path (m >= 16).  A workgroup of NW wavefronts owns 16 output
// columns (16 rows of W) and up to 16 * MT rows of X; its wavefronts split K
// into NW contiguous slices, so even a narrow layer (N = 768) runs
// 48 * NW wavefronts per 16 * MT rows of X.  Each wavefront streams its
// slice C k-steps (32 weights each) at a time with two register buffers:
// the loads of the next C steps are in flight while the current ones feed
// the matrix cores.  Every load is unconditional (k-steps past the slice,
// rows past N or M read in-bounds stand-ins whose W operand is zeroed), so
// the in-order load count stays exact.  The NW partial tiles are summed in
// a fixed order through LDS, so results do not depend on timing.
//
// Operand layout of v_mfma_f32_16x16x32_f16 for lane l (i = l % 16,
// kg = l / 16): A row i, k = 8kg..8kg+7; B column i, the same k; C column i,
// rows 4kg..4kg+3.  Only the pairing of A and B k-slots matters for the sum,
// so both read the same 8 consecutive k of their row.
//
// A k-step reads 64 bytes of each of 16 rows.  When the row stride is a
// whole number of 128-byte lines (K a multiple of 64), those 16 pieces sit
// at the same offset in their lines and one load instruction crowds one half
// of the memory path (K = 768 and 3072 ran 10-20% slower than K = 800 or
// 3040).  Odd rows of W and X therefore load the two k-steps of a buffer in
// the opposite order, so each instruction reads both halves, and pick their
// operands back in step order: the matrix cores see the same operands in the
// same order, so the sums are unchanged bit for bit.
constexpr int kGemmC = 2;   // k-steps per buffer (even: swapped in pairs)

template <int NW, int MT, int C>
struct GemmBuf {
  half8 w[C];
  half8 x[C][MT];
};

// Split form (kpart non-null, gridDim.z = splits > 1): workgroup z takes
// the z-th run of whole k-step pairs and writes its partial tile, without
// bias, to kpart[z][m][n]; a second launch sums them.
template <int NW, int MT, int C, bool SW>
__global__ __launch_bounds__(NW * 64) void gemm_f16_mfma_kernel(GemmArgs a, float* kpart) {
  __shared__ floatx4 part[NW][MT][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar
  const int i = lane & 15;
  const int kg = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
  const int ksteps = static_cast<int>(a.k / 32);
  const int split = static_cast<int>(blockIdx.z);
  const int per_split = 2 * ((ksteps + 2 * static_cast<int>(gridDim.z) - 1) / (2 * static_cast<int>(gridDim.z)));
  const int g_begin = per_split * split < ksteps ? per_split * split : ksteps;
  const int g_end = g_begin + per_split < ksteps ? g_begin + per_split : ksteps;
  const int per_wave = (g_end - g_begin + NW - 1) / NW;
  const int s_begin = g_begin + wave * per_wave;
  const int s_end = s_begin + per_wave < g_end ? s_begin + per_wave : g_end;

  const int64_t wn = n0 + i < a.n ? n0 + i : a.n - 1;
  const uint16_t* wrow = a.w + wn * a.k + 8 * kg;
  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t xm = m0 + 16 * t + i < a.m ? m0 + 16 * t + i : a.m - 1;
    xrow[t] = a.x + xm * a.k + 8 * kg;
  }

  // With SW (K a multiple of 64) slot c of a buffer holds k-step
  // s + (c ^ swap); W row i and X rows 16t + i share the parity of i.
  static_assert(C % 2 == 0, "k-steps are swapped in pairs");
  const int swap = SW ? (i & 1) : 0;
  auto load = [&](int s, GemmBuf<NW, MT, C>& b) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int sl = s + (c ^ swap);
      const int sc = sl < s_end ? sl : (s_begin < ksteps ? s_begin : 0);
      b.w[c] = *reinterpret_cast<const half8*>(wrow + 32 * sc);
#pragma unroll
      for (int t = 0; t < MT; ++t) b.x[c][t] = *reinterpret_cast<const half8*>(xrow[t] + 32 * sc);
    }
  };
  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int s, const GemmBuf<NW, MT, C>& b) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const half8 wsel = swap ? b.w[c ^ 1] : b.w[c];
      const half8 wv = s + c < s_end ? wsel : half8{};
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const half8 xv = swap ? b.x[c ^ 1][t] : b.x[c][t];
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, acc[t], 0, 0, 0);
      }
    }
  };

  GemmBuf<NW, MT, C> ba, bb;
  load(s_begin, ba);
  for (int s = s_begin; s < s_end; s += 2 * C) {
    load(s + C, bb);
    mma(s, ba);
    if (s + C >= s_end) break;
    load(s + 2 * C, ba);
    mma(s + C, bb);
  }

#pragma unroll
  for (int t = 0; t < MT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  // Thread e sums entry e (tile e / 64, lane e % 64) over the NW slices in
  // slice order, adds the bias and stores its four values.
  for (int e = threadIdx.x; e < MT * kWave; e += NW * kWave) {
    const int t = e / kWave, l = e % kWave;
    floatx4 r = part[0][t][l];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const floatx4 p = part[w][t][l];
      r.x += p.x; r.y += p.y; r.z += p.z; r.w += p.w;
    }
    const int64_t col = n0 + (l & 15);
    if (col < a.n) {
      const float bv = kpart ? 0.f : (a.bias ? a.bias[col] : 0.f);
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
__global__ __launch_bounds__(256) void gemm_bias_fill_kernel(GemmArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= a.m * a.n) return;
  a.y[e] = a.bias ? a.bias[e % a.n] : 0.f;
}

// Vector-ALU path for m < 16: the rows of X are a batch of B <= 8 columns
// applied to every W row, which is read once.  L lanes per W row, a unit
// is 32 weights (64 bytes); a lane loads up to U units of its row at once
// (longer rows take several such rounds).  X stays binary16 in LDS and
// v_dot2_f32_f16 multiplies two weight/activation pairs per instruction
// into a float32 sum (the products of two binary16 values are exact in
// float32).  Rows past N and lanes past the row end load in-bounds
// stand-ins that are dropped, keeping every load unconditional.
typedef _Float16 half2 __attribute__((ext_vector_type(2)));

// LDS position (in halves) of x element i: 8 halves of padding every 128.
__device__ __forceinline__ int xh_phys(int i) { return i + 8 * (i >> 7); }
__host__ __device__ constexpr int64_t xh_stride(int64_t k) { return ((k + 127) / 128) * 136; }

template <int L, int U, int B>
__global__ __launch_bounds__(kThreads) void gemm_f16_valu_kernel(GemmArgs a) {
  extern __shared__ uint16_t xh[];
  constexpr int kRowsPerWave = kWave / L;
  constexpr int kRowsPerGroup = kWavesPerGroup * kRowsPerWave;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (L - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup + wave * kRowsPerWave + lane / L;
  const int units = static_cast<int>(a.k / 32);
  const int stride = static_cast<int>(xh_stride(a.k));
  const uint16_t* wr = a.w + (row < a.n ? row : a.n - 1) * a.k;

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.f;
  for (int j0 = 0; j0 * L < units; j0 += U) {
    u32x4 wv[U][4];
    bool have[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = sub + L * (j0 + j);
      have[j] = u < units;
      const uint16_t* p = wr + 32 * (have[j] ? u : 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) wv[j][c] = load_u32x4_a16(p + 8 * c);
    }
    if (j0 == 0) {
      // X (B rows of K halves) into LDS, 16 bytes per thread and step.  With
      // more than four steps per thread (long rows), four steps' loads are
      // issued before their stores (slots past the end re-read the thread's
      // first chunk and are not stored) so that they overlap instead of
      // paying one round trip each: 3072-deep rows at m = 8 6.56 -> 6.04 us;
      // shorter rows keep one step at a time (batching them measured 2-5%
      // slower: the stand-in loads cost more than they hide).
      const int chunks = B * (units * 4);
      if (chunks > 4 * kThreads) {
        constexpr int kBatch = 4;
        for (int e0 = threadIdx.x; e0 < chunks; e0 += kBatch * kThreads) {
          u32x4 v[kBatch];
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int e = e0 + i * kThreads < chunks ? e0 + i * kThreads : e0;
            const int b = e / (units * 4), q = e % (units * 4);
            v[i] = load_u32x4_a16(a.x + b * a.k + 8 * q);
          }
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int e = e0 + i * kThreads;
            if (e < chunks) {
              const int b = e / (units * 4), q = e % (units * 4);
              *reinterpret_cast<u32x4*>(xh + b * stride + xh_phys(8 * q)) = v[i];
            }
          }
        }
      } else {
        for (int e = threadIdx.x; e < chunks; e += kThreads) {
          const int b = e / (units * 4), q = e % (units * 4);
          const u32x4 v = load_u32x4_a16(a.x + b * a.k + 8 * q);
          *reinterpret_cast<u32x4*>(xh + b * stride + xh_phys(8 * q)) = v;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (!have[j]) continue;
      const int u = sub + L * (j0 + j);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w4[4] = {wv[j][c].x, wv[j][c].y, wv[j][c].z, wv[j][c].w};
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xh + b * stride + xh_phys(32 * u + 8 * c));
          const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2, w4[e]),
                                            __builtin_bit_cast(half2, x4[e]), acc[b], false);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = group_sum<L>(acc[b]);
  if (sub == 0 && row < a.n) {
    const float bv = a.bias ? a.bias[row] : 0.f;
#pragma unroll
    for (int b = 0; b < B; ++b) a.y[b * a.n + row] = acc[b] + bv;
  }
}

}  // namespace pesti

namespace {

using pesti::GemmArgs;

template <int L, int U, int B>
int launch_valu(const GemmArgs& a, hipStream_t st) {
  constexpr int kRowsPerGroup = pesti::kWavesPerGroup * (pesti::kWave / L);
  const size_t lds = sizeof(uint16_t) * pesti::xh_stride(a.k) * B;
  const int64_t tiles = (a.n + kRowsPerGroup - 1) / kRowsPerGroup;
  GemmArgs args = a;
  void* params[] = {&args};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemm_f16_valu_kernel<L, U, B>),
                                 dim3(static_cast<unsigned>(tiles)), dim3(pesti::kThreads), params, lds, st);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <int L, int U>
int launch_valu_b(const GemmArgs& a, int b, hipStream_t st) {
  switch (b) {
    case 1: return launch_valu<L, U, 1>(a, st);
    case 2: return launch_valu<L, U, 2>(a, st);
    case 3: return launch_valu<L, U, 3>(a, st);
    case 4: return launch_valu<L, U, 4>(a, st);
    case 5: return launch_valu<L, U, 5>(a, st);
    case 6: return launch_valu<L, U, 6>(a, st);
    case 7: return launch_valu<L, U, 7>(a, st);
    case 8: return launch_valu<L, U, 8>(a, st);
    default: return PESTI_ERR_BATCH;
  }
}

template <int NW, int MT>
int launch_mfma_t(const GemmArgs& a, float* ws, hipStream_t st) {
  const int splits = ws ? pesti_host::gemm_splits(PESTI_FMT_F16, a.m, a.n, a.k) : 1;
  float* kpart = splits > 1 ? ws : nullptr;
  dim3 grid(static_cast<unsigned>((a.n + 15) / 16), static_cast<unsigned>((a.m + 16 * MT - 1) / (16 * MT)),
            static_cast<unsigned>(splits));
  GemmArgs args = a;
  void* params[] = {&args, &kpart};
  const void* fn = a.k % 64 == 0
                       ? reinterpret_cast<const void*>(&pesti::gemm_f16_mfma_kernel<NW, MT, pesti::kGemmC, true>)
                       : reinterpret_cast<const void*>(&pesti::gemm_f16_mfma_kernel<NW, MT, pesti::kGemmC, false>);
  hipError_t e = hipLaunchKernel(fn, grid, dim3(NW * 64), params, 0, st);
  if (e != hipSuccess) return PESTI_ERR_LAUNCH;
  return splits > 1 ? pesti_host::launch_split_sum(a.m, a.n, kpart, splits, a.bias, a.y, st) : PESTI_OK;
}

// Launch shape by how many 16-column tiles the layer has: narrow layers
// (under 96 tiles, e.g. N = 768) give every 16-row tile of X its own
// workgroup, so that enough workgroups stream W; wider ones let a
// workgroup of 16 K slices reuse each W load for 2 or 4 tiles of X.  A
// narrow layer's workgroup takes 16 K slices when K is short (at most 32
// k-steps: one buffer round per wavefront instead of two) or long (over 128
// k-steps), else 8 (measured at N = 768 and 896, m = 16..64: K = 768 4.05 ->
// 3.43 us, K = 4864 11.3 -> 10.6 us, K = 1536..3072 0.3-1.1 us slower).
int launch_mfma(const GemmArgs& a, float* ws, hipStream_t st) {
  const int64_t tiles_n = (a.n + 15) / 16, tiles_m = (a.m + 15) / 16;
  const int64_t ksteps = a.k / 32;
  if (tiles_n < 96 && (ksteps <= 32 || ksteps > 128)) return launch_mfma_t<16, 1>(a, ws, st);
  if (tiles_n < 96) return launch_mfma_t<8, 1>(a, ws, st);
  // 8 K slices once there are at least 256 workgroups (4864x896: m 16 6.3
  // -> 5.6 us, m 32 7.7 -> 7.2, m 64 10.3 -> 9.2), else 16 (GPT-2 c_attn
  // m 32: 4.2 against 5.1 with 8)
  if (tiles_m <= 1) return tiles_n >= 256 ? launch_mfma_t<8, 1>(a, nullptr, st) : launch_mfma_t<16, 1>(a, nullptr, st);
  if (tiles_m <= 2) return tiles_n >= 256 ? launch_mfma_t<8, 2>(a, nullptr, st) : launch_mfma_t<16, 2>(a, nullptr, st);
  return tiles_n * ((tiles_m + 3) / 4) >= 256 ? launch_mfma_t<8, 4>(a, nullptr, st)
                                              : launch_mfma_t<16, 4>(a, nullptr, st);
}

#ifndef PESTI_WIDE_F16_RING
#define PESTI_WIDE_F16_RING 8
#endif

// binary16 weights for the wide-layer kernel: a unit is one k-step, 32
// consecutive weights of the row, the lane's 8 of them one 16-byte load.
struct WPolF16 {
  static constexpr int kSumWidth = 32;
  static constexpr int64_t kWideMinTiles = 1024;
  static constexpr bool kMin = false;
  static constexpr bool kScaled = false;
  static constexpr bool kChained = false;
  static constexpr int kSteps = 1;
  static constexpr int kRing = PESTI_WIDE_F16_RING;
  struct Unit { pesti::u32x4 v; };
  __device__ __forceinline__ static void load(const uint8_t* row, int u, int kg, Unit& un) {
    un.v = pesti::load_u32x4_a16(row + 64 * u + 16 * kg);
  }
  __device__ __forceinline__ static pesti::whalf8 codes(const Unit& un, int, int, int) {
    return __builtin_bit_cast(pesti::whalf8, un.v);
  }
  __device__ __forceinline__ static float scale(const Unit&, int, int) { return 1.f; }
};

}  // namespace

int pesti_host::gemm_f16_run(int64_t m, int64_t out_features, int64_t in_features, const uint16_t* w,
                             const uint16_t* x, float* y, const float* bias, float* ws, hipStream_t sh) {
  if (out_features < 0 || in_features < 0) return PESTI_ERR_SHAPE;
  if (m < 0 || m > PESTI_MAX_GEMM_M) return PESTI_ERR_BATCH;
  if (m == 0 || out_features == 0) return PESTI_OK;
  if (in_features % 32 != 0 || in_features > PESTI_MAX_IN_FEATURES) return PESTI_ERR_SHAPE;
  if (!y || (in_features > 0 && (!w || !x))) return PESTI_ERR_NULL;
  if (!pesti_host::aligned(y, 16) || (w && !pesti_host::aligned(w, 16)) ||
      (x && !pesti_host::aligned(x, 16)) || (bias && !pesti_host::aligned(bias, 4)))
    return PESTI_ERR_ALIGN;
  int dev = 0;
  size_t lds_limit = 0;
  int st = pesti_host::current_device(&dev, &lds_limit);
  if (st != PESTI_OK) return st;
  GemmArgs a{w, x, y, bias, m, out_features, in_features};
  if (in_features == 0) {
    void* params[] = {&a};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemm_bias_fill_kernel),
                                         dim3(static_cast<unsigned>((m * out_features + 255) / 256)),
                                         dim3(256), params, 0, sh);
    return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
  }
  if (m >= 16) {
    const int wide = pesti_host::launch_wide<WPolF16>(
        pesti::WideArgs{reinterpret_cast<const uint8_t*>(w), x, y, bias, m, out_features, in_features,
                        2 * in_features},
        lds_limit, sh);
    if (wide != 1) return wide;
    return launch_mfma(a, ws, sh);
  }
  // m < 16: rows of X in chunks of up to 8 as a batch of binary16 mat-vecs;
  // 32 lanes per W row holding up to 2 units each (rows of up to 2048
  // weights), 64 lanes holding up to 2 (up to 4096 weights: the 3072-deep
  // GPT-2 projection, 6.75 us at m = 8 against 7.49 with 32 lanes holding
  // 3) and up to 4 in several rounds beyond that.
  const size_t row_lds = sizeof(uint16_t) * pesti::xh_stride(in_features);
  int per_launch = pesti_host::batch_per_launch(lds_limit, row_lds, 0, 8);
  if (per_launch < 1) return PESTI_ERR_SHAPE;
  const int64_t units = in_features / 32;
  for (int64_t r0 = 0; r0 < m; r0 += per_launch) {
    const int nb = static_cast<int>(m - r0 < per_launch ? m - r0 : per_launch);
    GemmArgs c = a;
    c.x = x + r0 * in_features;
    c.y = y + r0 * out_features;
    c.m = nb;
    int r;
    if (units <= 32) r = launch_valu_b<32, 1>(c, nb, sh);
    else if (units <= 64) r = launch_valu_b<32, 2>(c, nb, sh);
    else if (units <= 128) r = launch_valu_b<64, 2>(c, nb, sh);
    else r = launch_valu_b<64, 4>(c, nb, sh);
    if (r != PESTI_OK) return r;
  }
  return PESTI_OK;
}

extern "C" int pesti_gemm_f16_smallm(int64_t m, int64_t out_features, int64_t in_features,
                                     const uint16_t* w, const uint16_t* x, float* y,
                                     const float* bias, void* stream) {
  return pesti_host::gemm_f16_run(m, out_features, in_features, w, x, y, bias, nullptr,
                                  static_cast<hipStream_t>(stream));
}
