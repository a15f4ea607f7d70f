// Small-M linear layer Y = X W^T + b for wide layers (many 16-column tiles
// of W, a K short enough that the workgroup's rows of X fit in LDS), shared
// by the binary16-weight and quantized-weight entry points.
//
// The K-split kernels give each workgroup one 16-column tile, so every 16
// columns of W re-read the whole tile of X and pay a cross-wavefront
// reduction.  Here the workgroup stages its 16 * MT rows of X in LDS once,
// already in the operand order of v_mfma_f32_16x16x32_f16, and each
// wavefront then streams whole rows of W for one column tile after another
// (tiles blockIdx.x * NWV + wave, stepping by gridDim.x * NWV): every k-step
// is one 32-weight block of the weight format, its W operand decoded from
// registers, its X operand one 16-byte LDS read per lane and M-tile.  Loads
// of W run several units ahead in a ring of registers, across tile boundaries;
// past the wavefront's last tile they re-read its last rows, so every load
// is unconditional and in bounds.  No reduction: a wavefront owns its
// tile's outputs over all of K and writes them once.
//
// Weight policy Q (kWideMinTiles: the layer width, in 16-column tiles,
// from which this kernel is used): a Unit holds the raw bytes of kSteps consecutive k-steps
// (a Q4_K super-block, a Q8_0 block, 32 binary16 weights), kRing units are
// in flight per wavefront; load(row, u, kg, Unit&) reads unit u of a row
// (whole units stay inside the row's padded length).  Unscaled (binary16)
// weights: codes(Unit, j, 0, kg) gives step j's 8 operand values, which
// accumulate in the matrix core directly.  Scaled formats: each of the
// step's kParts parts - codes(Unit, j, part, kg), scale(Unit, j, part) - is
// its own product, added to the float32 sum times its scale.  Chained
// formats (kChained) carry the sub-block scales in the operand:
// codes(Unit, j, kg) for the steps of a unit accumulate in the matrix core,
// d(Unit) scales the sum once, and for kMin formats neg_min(Unit, h, kg)
// times the sums of X over each kSumWidth weights (taken once per
// workgroup into LDS) removes the mins, four sum groups per 16x16x4
// product.  j, part and h are constants after unrolling.
//
// Operand layout, lane l (i = l % 16, kg = l / 16): A = X row i,
// k = 8kg..8kg+7 of the step; B = W row i (output column i), the same k;
// C = column i, rows 4kg..4kg+3.
#pragma once
#include <type_traits>

#include "common.h"

namespace pesti {

typedef _Float16 whalf8 __attribute__((ext_vector_type(8)));
typedef float wfloat4 __attribute__((ext_vector_type(4)));

// Chained policies may decode per-unit data once for the wave (Q::Prep,
// Q::prep(unit, kg)); codes(unit, prep, j, kg) then reads it.
template <class Q, class = void>
struct HasPrep : std::false_type {};
template <class Q>
struct HasPrep<Q, std::void_t<typename Q::Prep>> : std::true_type {};
struct NoPrep {};
template <class Q>
__device__ __forceinline__ auto prep_of(const typename Q::Unit& un, int kg) {
  if constexpr (HasPrep<Q>::value) return Q::prep(un, kg);
  else return NoPrep{};
}

struct WideArgs {
  const uint8_t* w;    // N rows of row_bytes
  const uint16_t* x;   // [M][K] binary16
  float* y;            // [M][N]
  const float* bias;   // [N] or null
  int64_t m, n, k;
  int64_t row_bytes;
};

// LDS bytes: X fragments [MT][S][64] of 16 bytes, then (kMin) the sums of
// X over each kSumWidth (32 or 16) weights, [K / kSumWidth][16 * MT] float32.
template <class Q>
__host__ __device__ constexpr int64_t wide_lds_bytes(int mt, int64_t k) {
  return static_cast<int64_t>(mt) * (k / 32) * 64 * 16 + (Q::kMin ? (k / Q::kSumWidth) * 16 * mt * 4 : 0);
}

template <class Q, int MT, int NWV>
__global__ __launch_bounds__(NWV * 64) void gemm_wide_kernel(WideArgs a) {
  constexpr int P = Q::kRing;
  constexpr int KS = Q::kSteps;
  extern __shared__ __attribute__((aligned(16))) uint8_t wide_lds[];
  const int S = static_cast<int>(a.k / 32);
  const int UR = (S + KS - 1) / KS;   // units per row
  whalf8* xf = reinterpret_cast<whalf8*>(wide_lds);
  float* sx = reinterpret_cast<float*>(wide_lds + static_cast<int64_t>(MT) * S * 64 * 16);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wavefront index is uniform; readfirstlane tells the compiler, so
  // the tile and unit cursors derived from it live in scalar registers and
  // their tests are scalar branches, not exec-mask ones.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15;
  const int kg = lane >> 4;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);

  // Stage rows m0 .. m0 + 16MT - 1 of X (zeros past M): 16-byte chunk q of
  // row r goes to fragment (r / 16, q / 4), lane (r % 16) + 16 (q % 4).
  // Eight chunks per thread are loaded before any is stored, so the loads
  // overlap instead of paying one round trip each.
  // The thread's chunk (r, q) advances by NWV * 64 chunks at a time without
  // a division; offsets within the workgroup's 16 * MT rows of X are 32-bit.
  const int qpr = 4 * S;   // chunks per row
  constexpr int kNT = NWV * 64;
  const int rows_here = a.m - m0 < 16 * MT ? static_cast<int>(a.m - m0) : 16 * MT;
  const int dr = kNT / qpr, dq = kNT - (kNT / qpr) * qpr;
  const uint16_t* xb = a.x + m0 * a.k;
  const int kk = static_cast<int>(a.k);
  int r = tid / qpr, q = tid - (tid / qpr) * qpr;
  constexpr int kBatch = 8;
  while (r < 16 * MT) {
    whalf8 v[kBatch];
    int rr[kBatch], qq[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      rr[b] = r;
      qq[b] = q;
      v[b] = whalf8{0, 0, 0, 0, 0, 0, 0, 0};
      if (r < rows_here) v[b] = *reinterpret_cast<const whalf8*>(xb + r * kk + 8 * q);
      r += dr;
      q += dq;
      if (q >= qpr) { q -= qpr; ++r; }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (rr[b] < 16 * MT)
        xf[((rr[b] >> 4) * S + (qq[b] >> 2)) * 64 + (rr[b] & 15) + 16 * (qq[b] & 3)] = v[b];
  }
  constexpr int SPS = 32 / Q::kSumWidth;   // sums per k-step
  if constexpr (Q::kMin) {
    __syncthreads();
    // sx[q][r]: the kSumWidth values of row r in sum group q (lanes
    // kg = 4 / SPS * (q % SPS) .. of step q / SPS) summed in float32, in k
    // order.
    for (int c = tid; c < 16 * MT * S * SPS; c += NWV * 64) {
      const int q = c / (16 * MT), r = c - q * (16 * MT);
      const int s = q / SPS, g0 = (4 / SPS) * (q % SPS);
      float t = 0.f;
#pragma unroll
      for (int g = 0; g < 4 / SPS; ++g) {
        const whalf8 v = xf[((r >> 4) * S + s) * 64 + (r & 15) + 16 * (g0 + g)];
#pragma unroll
        for (int e = 0; e < 8; ++e) t += static_cast<float>(v[e]);
      }
      sx[c] = t;
    }
  }
  __syncthreads();

  const int64_t tiles = (a.n + 15) / 16;
  const int64_t t_first = static_cast<int64_t>(blockIdx.x) * NWV + wave;
  const int64_t t_step = static_cast<int64_t>(gridDim.x) * NWV;
  if (t_first >= tiles) return;   // no barrier follows
  const int64_t my_tiles = (tiles - 1 - t_first) / t_step + 1;
  const int64_t units = my_tiles * UR;

  auto row_of = [&](int64_t tile) {
    const int64_t col = tile * 16 + i;
    return a.w + (col < a.n ? col : a.n - 1) * a.row_bytes;
  };
  // A ring slot: one unit of W and the bias of its output column, loaded
  // together.  Loads retire in order, so a bias load in the epilogue would
  // wait for every unit issued before it and empty the ring; loaded with
  // the unit it is ready when that unit is.  Without a bias the slot reads
  // the first bias-sized word of X and the epilogue scales it by 0.
  struct Slot {
    typename Q::Unit un;
    float b;
  };
  const float* bias_src = a.bias ? a.bias : reinterpret_cast<const float*>(a.x);
  const int64_t bias_step = a.bias ? 1 : 0;
  const float bias_mul = a.bias ? 1.f : 0.f;
  // Issue cursor: tile and unit of the next load.
  int64_t i_tile = t_first;
  int i_u = 0;
  const uint8_t* i_row = row_of(t_first);
  const float* i_bias = bias_src + bias_step * (t_first * 16 + i < a.n ? t_first * 16 + i : a.n - 1);
  auto issue = [&](Slot& sl) {
    Q::load(i_row, i_u, kg, sl.un);
    sl.b = *i_bias;
    if (++i_u == UR) {
      i_u = 0;
      i_tile += t_step;
      if (i_tile < tiles) {   // else: re-read the last rows
        i_row = row_of(i_tile);
        i_bias = bias_src + bias_step * (i_tile * 16 + i < a.n ? i_tile * 16 + i : a.n - 1);
      }
    }
  };

  Slot ring[P];
#pragma unroll
  for (int u = 0; u < P; ++u) issue(ring[u]);

  // acc: the scaled products; accm: the chained formats' min terms (kept
  // apart so the matrix-core chain does not wait on vector-ALU updates).
  wfloat4 acc[MT], accm[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc[t] = wfloat4{0.f, 0.f, 0.f, 0.f};
    accm[t] = wfloat4{0.f, 0.f, 0.f, 0.f};
  }
  int c_u = 0;
  int64_t c_tile = t_first;

  for (int64_t f = 0; f < units; f += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const bool live = f + u < units;   // wave-uniform
      if constexpr (Q::kChained) {
        // The unit's k-steps accumulate in the matrix core on operands that
        // carry their sub-block scales; d scales the sum once, and the mins
        // are subtracted by 16x16x4 float32 products of the sums of X (A:
        // lane (i, kg) = row i, sum group 4h + kg of the unit) with
        // -dmin * m (B: the same group, column i).
        if (live) {
          wfloat4 pc[MT];
#pragma unroll
          for (int t = 0; t < MT; ++t) pc[t] = wfloat4{0.f, 0.f, 0.f, 0.f};
          [[maybe_unused]] const auto pr = prep_of<Q>(ring[u].un, kg);
#pragma unroll
          for (int j = 0; j < KS; ++j) {
            const int s = c_u * KS + j;
            if (s >= S) break;   // wave-uniform: the row's last, partial unit
            whalf8 wv;
            if constexpr (HasPrep<Q>::value) wv = Q::codes(ring[u].un, pr, j, kg);
            else wv = Q::codes(ring[u].un, j, kg);
#pragma unroll
            for (int t = 0; t < MT; ++t)
              pc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xf[(t * S + s) * 64 + lane], wv, pc[t], 0, 0, 0);
          }
          const float dd = Q::d(ring[u].un);
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[t] += dd * pc[t];
          if constexpr (Q::kMin) {
#pragma unroll
            for (int h = 0; h < KS * SPS / 4; ++h) {
              const int s0 = c_u * KS * SPS + 4 * h;   // first sum group of the product
              if (s0 >= S * SPS) break;   // wave-uniform
              const float bm = Q::neg_min(ring[u].un, h, kg);
              const int sk = s0 + kg < S * SPS ? s0 + kg : S * SPS - 1;
              const float keep = s0 + kg < S * SPS ? 1.f : 0.f;
#pragma unroll
              for (int t = 0; t < MT; ++t) {
                const float av = keep * sx[sk * 16 * MT + 16 * t + i];
                accm[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bm, accm[t], 0, 0, 0);
              }
            }
          }
        }
      } else if (live) {
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          const int s = c_u * KS + j;
          if (KS > 1 && s >= S) break;   // wave-uniform: the row's last, partial unit
          if constexpr (Q::kScaled) {
            // Each scaled part (a block, or a sub-block's half of the
            // operand) is its own product, added times its scale.
#pragma unroll
            for (int pt = 0; pt < Q::kParts; ++pt) {
              const whalf8 wv = Q::codes(ring[u].un, j, pt, kg);
              const float ds = Q::scale(ring[u].un, j, pt);
#pragma unroll
              for (int t = 0; t < MT; ++t) {
                const whalf8 xv = xf[(t * S + s) * 64 + lane];
                const wfloat4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, wfloat4{0.f, 0.f, 0.f, 0.f},
                                                                         0, 0, 0);
                acc[t] += ds * p;
              }
            }
          } else {
            const whalf8 wv = Q::codes(ring[u].un, j, 0, kg);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              const whalf8 xv = xf[(t * S + s) * 64 + lane];
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, wv, acc[t], 0, 0, 0);
            }
          }
        }
      }
      if (live) {
        if (++c_u == UR) {   // the tile's last unit: write its outputs
          c_u = 0;
          const float bv = bias_mul * ring[u].b;
          const int64_t col = c_tile * 16 + i;
          if (col < a.n) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              const wfloat4 r4 = acc[t] + accm[t];
              const float v[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int64_t row = m0 + 16 * t + 4 * kg + q;
                if (row < a.m) a.y[row * a.n + col] = v[q] + bv;
              }
            }
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            acc[t] = wfloat4{0.f, 0.f, 0.f, 0.f};
            accm[t] = wfloat4{0.f, 0.f, 0.f, 0.f};
          }
          c_tile += t_step;
        }
      }
      // The slot is refilled on every pass, live or not (past the last unit
      // with in-bounds stand-ins), and only after everything that reads its
      // old contents: a value kept across the refill, or a merge of old and
      // new contents, would need a register copy, and the copy a wait for
      // the load - which, loads retiring in order, empties the ring.
      issue(ring[u]);
    }
  }
}

}  // namespace pesti

namespace pesti_host {

// Launches the wide-layer kernel when it applies: at least Q::kWideMinTiles
// column tiles (below that the K-split kernels, whose wavefronts split K
// and so issue more loads at once, finish sooner), and the workgroup's rows
// of X (16 per M-tile; 1, 2 or 4 M-tiles by m, more rows in further
// workgroups along y) fit in LDS.  Returns 1 (and launches nothing) when it
// does not apply.
// Workgroups per CU that the grid is sized for (also capped by LDS): each
// stages its rows of X once, so fewer, longer-lived workgroups amortise the
// staging, more of them balance the tiles better.
#ifndef PESTI_WIDE_WG_PER_CU
#define PESTI_WIDE_WG_PER_CU 2
#endif

template <class Q, int MT, int NWV>
int launch_wide_t(const pesti::WideArgs& a, int64_t lds, size_t lds_limit, hipStream_t st) {
  const int64_t tiles = (a.n + 15) / 16;
  // Workgroups resident per CU by LDS, at most PESTI_WIDE_WG_PER_CU
  // counted; 256 CUs.
  int64_t per_cu = static_cast<int64_t>(lds_limit) / lds;
  per_cu = per_cu > PESTI_WIDE_WG_PER_CU ? PESTI_WIDE_WG_PER_CU : (per_cu < 1 ? 1 : per_cu);
  int64_t gx = (tiles + NWV - 1) / NWV;
  if (gx > 256 * per_cu) gx = 256 * per_cu;
  const int64_t gy = (a.m + 16 * MT - 1) / (16 * MT);
  pesti::WideArgs args = a;
  void* params[] = {&args};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pesti::gemm_wide_kernel<Q, MT, NWV>),
                                       dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                                       dim3(NWV * 64), params, static_cast<size_t>(lds), st);
  return e == hipSuccess ? PESTI_OK : PESTI_ERR_LAUNCH;
}

template <class Q, int MT>
int launch_wide_m(const pesti::WideArgs& a, int64_t lds, size_t lds_limit, hipStream_t st) {
  const int64_t tiles = (a.n + 15) / 16;
  if (tiles >= 8 * 256) return launch_wide_t<Q, MT, 8>(a, lds, lds_limit, st);
  return launch_wide_t<Q, MT, 4>(a, lds, lds_limit, st);
}

template <class Q>
int launch_wide(const pesti::WideArgs& a, size_t lds_limit, hipStream_t st) {
  const int64_t tiles = (a.n + 15) / 16;
  if (tiles < Q::kWideMinTiles || a.k == 0) return 1;
  const int mt = a.m <= 16 ? 1 : (a.m <= 32 ? 2 : 4);
  const int64_t lds = pesti::wide_lds_bytes<Q>(mt, a.k);
  if (lds > static_cast<int64_t>(lds_limit)) return 1;
  if (mt == 1) return launch_wide_m<Q, 1>(a, lds, lds_limit, st);
  if (mt == 2) return launch_wide_m<Q, 2>(a, lds, lds_limit, st);
  return launch_wide_m<Q, 4>(a, lds, lds_limit, st);
}

}  // namespace pesti_host
