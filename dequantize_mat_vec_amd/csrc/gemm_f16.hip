// Small-M binary16 linear layer Y = X W^T + b ("inferno" README,
// "Benchmarks": linear = x @ w + b at prompt width, e.g. 32x768 @ 768x2304;
// "Bottlenecks are the big prompt-width GEMMs").  X binary16 [m][K],
// W binary16 [N][K] (same row orientation as the mat-vec), Y float32 [m][N],
// float32 accumulation.
//
// For m >= 16 the product is a dense contraction and runs on the matrix
// cores (v_mfma_f32_16x16x32_f16): a workgroup owns 16 output columns and up
// to 64 rows of X; its 4 wavefronts split K four ways, each streaming its
// slice of the 16 W rows once and reusing it for every 16-row tile of X;
// the four partial tiles are summed through LDS.  Below 16 rows the matrix
// cores would idle most of their rows, so a vector-ALU kernel treats the
// rows of X as a batch of mat-vecs over binary16 weights.
#include "common.h"

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

constexpr int kGemmRowsPerGroup = 64;   // rows of X per workgroup (4 MFMA tiles)

// Operand layout of v_mfma_f32_16x16x32_f16 for lane l (i = l % 16,
// kg = l / 16): A row i, k = 8kg..8kg+7; B column i, the same k; C column i,
// rows 4kg..4kg+3.  Only the pairing of A and B k-slots matters for the sum,
// so both read the same 8 consecutive k of their row.
__global__ __launch_bounds__(256) void gemm_f16_mfma_kernel(GemmArgs a) {
  __shared__ floatx4 part[kWavesPerGroup][4][kWave];   // per wave: 4 row tiles
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;
  const int kg = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kGemmRowsPerGroup;
  const int64_t ksteps = a.k / 32;
  const int64_t per_wave = (ksteps + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t s_begin = wave * per_wave;
  const int64_t s_end = s_begin + per_wave < ksteps ? s_begin + per_wave : ksteps;
  const int64_t mtiles = (a.m - m0 + 15) / 16 < 4 ? (a.m - m0 + 15) / 16 : 4;

  floatx4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int64_t wn = n0 + i;
  const bool wvalid = wn < a.n;
  const uint16_t* wrow = a.w + (wvalid ? wn : 0) * a.k + 8 * kg;
  for (int64_t s = s_begin; s < s_end; ++s) {
    half8 bv = {};
    if (wvalid) bv = *reinterpret_cast<const half8*>(wrow + 32 * s);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < mtiles) {
        const int64_t xm = m0 + 16 * t + i;
        half8 av = {};
        if (xm < a.m) av = *reinterpret_cast<const half8*>(a.x + xm * a.k + 32 * s + 8 * kg);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  // wave w finishes row tile w: sum the four K-slices, add bias, store.
  const int t = wave;
  if (t < mtiles) {
    floatx4 r = part[0][t][lane];
#pragma unroll
    for (int w = 1; w < kWavesPerGroup; ++w) {
      const floatx4 p = part[w][t][lane];
      r.x += p.x; r.y += p.y; r.z += p.z; r.w += p.w;
    }
    const int64_t col = n0 + i;
    if (col < a.n) {
      const float bv = a.bias ? a.bias[col] : 0.f;
      const float v[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + 16 * t + 4 * kg + q;
        if (row < a.m) a.y[row * a.n + col] = v[q] + bv;
      }
    }
  }
}

// Vector-ALU path for m < 16: every W row is read once and applied to all
// rows of X (staged in LDS as float32).  L lanes per W row, 32 weights
// (64 bytes) per unit.
template <int L, int B>
__global__ __launch_bounds__(kThreads) void gemm_f16_valu_kernel(GemmArgs a, int64_t xstride) {
  extern __shared__ float xs[];
  const int64_t kpad = ((a.k + 63) / 64) * 64;
  for (int b = 0; b < B; ++b) {
    for (int64_t i = threadIdx.x; i < kpad; i += kThreads) {
      float v = 0.f;
      if (i < a.k) v = static_cast<float>(__builtin_bit_cast(_Float16, a.x[b * a.k + i]));
      xs[b * xstride + xs_phys(i)] = v;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (L - 1);
  const int grp = lane / L;
  constexpr int kRowsPerWave = kWave / L;
  constexpr int kRowsPerGroup = kWavesPerGroup * kRowsPerWave;
  const int64_t units = a.k / 32;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup; r0 < a.n;
       r0 += static_cast<int64_t>(gridDim.x) * kRowsPerGroup) {
    const int64_t row = r0 + wave * kRowsPerWave + grp;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    if (row < a.n) {
      const uint16_t* wr = a.w + row * a.k;
      for (int64_t u = sub; u < units; u += L) {
        const uint16_t* p = wr + 32 * u;
        u32x4 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = load_u32x4_a16(p + 8 * c);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t d4[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float w0 = f16_lo(d4[e]), w1 = f16_hi(d4[e]);
            const int64_t kk = 32 * u + 8 * c + 2 * e;
#pragma unroll
            for (int b = 0; b < B; ++b) {
              const float* xb = xs + b * xstride;
              acc[b] = fmaf(w0, xb[xs_phys(kk)], acc[b]);
              acc[b] = fmaf(w1, xb[xs_phys(kk + 1)], acc[b]);
            }
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
}

}  // namespace pesti

namespace {

using pesti::GemmArgs;

template <int L, int B>
int launch_valu(const GemmArgs& a, hipStream_t st) {
  constexpr int kRowsPerGroup = pesti::kWavesPerGroup * (pesti::kWave / L);
  const int64_t xstride = pesti::xs_stride(a.k, 64);
  const size_t lds = sizeof(float) * xstride * B;
  const int64_t tiles = (a.n + kRowsPerGroup - 1) / kRowsPerGroup;
  GemmArgs args = a;
  int64_t xs = xstride;
  void* params[] = {&args, &xs};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemm_f16_valu_kernel<L, B>),
                                 dim3(pesti_host::grid_for(tiles, 8192)), dim3(pesti::kThreads), params,
                                 lds, st);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <int L>
int launch_valu_b(const GemmArgs& a, int b, hipStream_t st) {
  switch (b) {
    case 1: return launch_valu<L, 1>(a, st);
    case 2: return launch_valu<L, 2>(a, st);
    case 3: return launch_valu<L, 3>(a, st);
    case 4: return launch_valu<L, 4>(a, st);
    case 5: return launch_valu<L, 5>(a, st);
    case 6: return launch_valu<L, 6>(a, st);
    case 7: return launch_valu<L, 7>(a, st);
    case 8: return launch_valu<L, 8>(a, st);
    default: return PESTI_ERR_BATCH;
  }
}

}  // namespace

extern "C" int pesti_gemm_f16_smallm(int64_t m, int64_t out_features, int64_t in_features,
                                     const uint16_t* w, const uint16_t* x, float* y,
                                     const float* bias, void* stream) {
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
  hipStream_t sh = static_cast<hipStream_t>(stream);
  GemmArgs a{w, x, y, bias, m, out_features, in_features};
  if (m >= 16) {
    dim3 grid(static_cast<unsigned>((out_features + 15) / 16),
              static_cast<unsigned>((m + pesti::kGemmRowsPerGroup - 1) / pesti::kGemmRowsPerGroup));
    void* params[] = {&a};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemm_f16_mfma_kernel), grid,
                                   dim3(256), params, 0, sh);
    return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
  }
  // m < 16: rows of X in chunks of up to 8 as a batch of binary16 mat-vecs
  const size_t row_lds = sizeof(float) * pesti::xs_stride(in_features, 64);
  int per_launch = pesti_host::batch_per_launch(lds_limit, row_lds, 0, 8);
  if (per_launch < 1) return PESTI_ERR_SHAPE;
  const int64_t units = in_features / 32;
  for (int64_t r0 = 0; r0 < m; r0 += per_launch) {
    const int nb = static_cast<int>(m - r0 < per_launch ? m - r0 : per_launch);
    GemmArgs c = a;
    c.x = x ? x + r0 * in_features : nullptr;
    c.y = y + r0 * out_features;
    c.m = nb;
    int r;
    if (units <= 16) r = launch_valu_b<16>(c, nb, sh);
    else if (units <= 32) r = launch_valu_b<32>(c, nb, sh);
    else r = launch_valu_b<64>(c, nb, sh);
    if (r != PESTI_OK) return r;
  }
  return PESTI_OK;
}
