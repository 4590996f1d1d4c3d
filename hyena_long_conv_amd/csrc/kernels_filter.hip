// kernels_filter.hip -- implicit filter generation and spectrum export.
//
// h_n[d](t) = Window_d(t) * FFN(e(t))[n*D + d] with the positional features
// e(t) = [t/L, sin(2 pi k t/L), cos(2 pi k t/L)] and an exponential-decay
// window exp(-alpha_d t / L) (jisaku.com glossary "Hyena（ハイエナ）", section
// "暗黙的畳み込みフィルタ"; paper digest of Hyena Hierarchy, framework figure,
// HyenaFilter node: positional encoding -> FFN -> window).  The FFN is
// affine -> sin -> affine -> sin -> affine.
#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {

// One workgroup = 64 positions t x a tile of filter rows.  Layers 1 and 2
// (H hidden units each) are computed once per workgroup into LDS, stored
// unit-major ([q][t], so the lanes of a wave, which differ in t, read
// consecutive words); then every lane keeps the H values of its position in
// registers and runs the last layer for its share of the tile's rows.  A
// wave's lanes share one filter row at a time, so the weights are read with
// scalar (wave-uniform) loads.  Sums run in the same order as the plain
// definition (bias, then m = 0..H-1).
constexpr int kFgThreads = 256, kFgT = 64, kFgWaves = kFgThreads / 64;
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int H>
__global__ void __launch_bounds__(kFgThreads) k_filter_gen(FilterGenArgs a, int rows_per_wg) {
  __shared__ float A1[H][kFgT];
  __shared__ float A2[H][kFgT];
  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);     // wave index (uniform)
  const int64_t t = (int64_t)blockIdx.x * kFgT + lane;
  const int K = a.K, F = 1 + 2 * K;
  const float tl = (float)t / (float)a.L;
  constexpr int QW = H / kFgWaves > 0 ? H / kFgWaves : 1;               // hidden units per wave
  // layer 1: units g*QW .. g*QW + QW - 1 of position t
  {
    float es[kMaxFreq + 1], ec[kMaxFreq + 1];
#pragma unroll
    for (int k = 1; k <= kMaxFreq; ++k) {
      es[k] = 0.f; ec[k] = 0.f;
      if (k <= K) {
        const int64_t m = ((int64_t)k * t) % a.L;    // phase k t / L reduced modulo 1 exactly
        sincospif(2.0f * (float)m / (float)a.L, &es[k], &ec[k]);
      }
    }
    for (int i = 0; i < QW; ++i) {
      const int q = g * QW + i;
      if (q >= H) break;
      const float* w = a.W1 + q * F;
      float acc = a.b1 ? a.b1[q] : 0.f;
      acc = fmaf(w[0], tl, acc);
#pragma unroll
      for (int k = 1; k <= kMaxFreq; ++k) {
        if (k <= K) {
          acc = fmaf(w[k], es[k], acc);
          acc = fmaf(w[K + k], ec[k], acc);
        }
      }
      A1[q][lane] = sinf(acc);
    }
  }
  __syncthreads();
  // layer 2
  {
    float x[H];
#pragma unroll
    for (int m = 0; m < H; ++m) x[m] = A1[m][lane];
    for (int i = 0; i < QW; ++i) {
      const int q = g * QW + i;
      if (q >= H) break;
      const float* w = a.W2 + q * H;
      float acc = a.b2 ? a.b2[q] : 0.f;
#pragma unroll
      for (int m = 0; m < H; ++m) acc = fmaf(w[m], x[m], acc);
      A2[q][lane] = sinf(acc);
    }
  }
  __syncthreads();
  // Layer 3 on the matrix cores (v_mfma_f32_32x32x2f32, fp32 products and
  // sums): per wave, 32-row tiles of the workgroup's rows times the 64
  // positions as two 32-column blocks.  Step s of the K loop takes hidden
  // unit k = s + (H/2)*(lane/32) for lanes on either half, so a lane reads a
  // contiguous half-row of W3 and its B values are fixed for the workgroup.
  constexpr int KS = H / 2;
  const int half = lane >> 5, col = lane & 31;
  float bv[2][KS];                                   // A2[s + KS*half][n*32 + col]
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) bv[n][s2] = A2[s2 + KS * half][n * 32 + col];
  const int NF = a.N * a.D;
  const int f0 = blockIdx.y * rows_per_wg;
  const int f1 = (f0 + rows_per_wg < NF) ? f0 + rows_per_wg : NF;
  for (int r0 = f0 + 32 * g; r0 < f1; r0 += 32 * kFgWaves) {
    const int fa = r0 + col;                         // A row of this lane
    float av[KS];
    if (fa < f1) {
      const float* w = a.W3 + (int64_t)fa * H + KS * half;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) av[s2] = w[s2];
    } else {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) av[s2] = 0.f;
    }
    f32x16 acc[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s2], bv[n][s2], acc[n], 0, 0, 0);
    // accumulator r of this lane: row 8(r/4) + 4*half + r%4, column col
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int f = r0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (f >= f1) continue;
      const float bias = a.b3 ? a.b3[f] : 0.f;
      const float al = a.alpha[f % a.D];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int64_t tt = (int64_t)blockIdx.x * kFgT + n * 32 + col;
        if (tt < a.L) a.h[(int64_t)f * a.L + tt] = expf(-al * ((float)tt / (float)a.L)) * (acc[n][r] + bias);
      }
    }
  }
}

hipError_t filter_gen(const FilterGenArgs& a, hipStream_t s) {
  const int NF = a.N * a.D;
  const int64_t tiles = (a.L + kFgT - 1) / kFgT;
  // Row tiles: enough for ~512 workgroups (two per CU) and no more, since
  // every row tile recomputes layers 1-2 of its positions.
  const int64_t max_tiles = (NF + 32 * kFgWaves - 1) / (32 * kFgWaves);   // one 32-row tile per wave
  int64_t row_tiles = (512 + tiles - 1) / tiles;
  if (row_tiles > max_tiles) row_tiles = max_tiles;
  if (row_tiles < 1) row_tiles = 1;
  const int per = (int)((NF + row_tiles - 1) / row_tiles);
  const int rows_per_wg = (per + 32 * kFgWaves - 1) / (32 * kFgWaves) * (32 * kFgWaves);
  const dim3 grid((unsigned)tiles, (unsigned)((NF + rows_per_wg - 1) / rows_per_wg));
  const dim3 block(kFgThreads);
  switch (a.H) {
    case 8: hipLaunchKernelGGL((k_filter_gen<8>), grid, block, 0, s, a, rows_per_wg); break;
    case 16: hipLaunchKernelGGL((k_filter_gen<16>), grid, block, 0, s, a, rows_per_wg); break;
    case 32: hipLaunchKernelGGL((k_filter_gen<32>), grid, block, 0, s, a, rows_per_wg); break;
    case 64: hipLaunchKernelGGL((k_filter_gen<64>), grid, block, 0, s, a, rows_per_wg); break;
    case 128: hipLaunchKernelGGL((k_filter_gen<128>), grid, block, 0, s, a, rows_per_wg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// H(k)/M of filter row `row` from the single path's pair coefficients:
// P = (a1 + conj a2)/2, sQ = (conj a2 - a1)/2, cQ = bq, Q = s*sQ + c*cQ;
// H(p) = (P + Q)/2, H(N-p) = conj(P - Q)/2 with p = min(k, N-k).
__device__ __forceinline__ cf single_bin(const cf* row, int64_t k, int64_t N, int64_t stride) {
  const int64_t qs = stride / 3;
  const int64_t p = k <= N / 2 ? k : N - k;
  const cf a1 = row[p], a2 = row[qs + p], bq = row[2 * qs + p];
  float sn, cs;
  sincospif((float)p / (float)N, &sn, &cs);
  const float Px = 0.5f * (a1.x + a2.x), Py = 0.5f * (a1.y - a2.y);
  const float sQx = 0.5f * (a2.x - a1.x), sQy = 0.5f * (-a2.y - a1.y);
  const float Qx = sn * sQx + cs * bq.x, Qy = sn * sQy + cs * bq.y;
  return (k == p) ? make_float2(0.5f * (Px + Qx), 0.5f * (Py + Qy)) : make_float2(0.5f * (Px - Qx), -0.5f * (Py - Qy));
}

// Library spectrum layout -> natural order, undoing the 1/(2N) scale.
__global__ void k_spectrum_export(const cf* __restrict__ spec, float* __restrict__ out, int NF, int64_t N,
                                  int path, int n1, int n2, int64_t stride) {
  const int64_t half = N + 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)NF * half) return;
  const int64_t f = idx / half, k = idx - f * half;
  const cf* row = spec + f * stride;
  cf g;
  if (path == PATH_SINGLE) {
    g = single_bin(row, k, N, stride);
  } else {
    int64_t src = k;
    if (k < N) src = (k % n1) * n2 + k / n1;
    g = row[src];
  }
  out[2 * idx] = g.x * (float)(2 * N);
  out[2 * idx + 1] = g.y * (float)(2 * N);
}

// A single-path spectrum rewritten in the four-step layout (n1 x n2) of the
// same FFT length: H(k)/M at (k mod n1) * n2 + k / n1, H(N)/M at N.
__global__ void k_spectrum_to_fourstep(const cf* __restrict__ spec, cf* __restrict__ out, int NF, int64_t N,
                                       int64_t stride_in, int n1, int n2, int64_t stride_out) {
  const int64_t half = N + 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)NF * half) return;
  const int64_t f = idx / half, k = idx - f * half;
  const int64_t dst = k < N ? (k % n1) * n2 + k / n1 : N;
  out[f * stride_out + dst] = single_bin(spec + f * stride_in, k, N, stride_in);
}

hipError_t spectrum_to_fourstep(const void* spec, int NF, const PlanInfo& single, const PlanInfo& fs, void* out,
                                hipStream_t s) {
  const int64_t total = (int64_t)NF * (single.N + 1);
  const int threads = 256;
  hipLaunchKernelGGL(k_spectrum_to_fourstep, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, s,
                     (const cf*)spec, (cf*)out, NF, single.N, single.spec_stride, fs.n1, fs.n2, fs.spec_stride);
  return hipGetLastError();
}

hipError_t spectrum_export(const void* spec, int NF, const PlanInfo& p, float* out, hipStream_t s) {
  const int64_t total = (int64_t)NF * (p.N + 1);
  const int threads = 256;
  hipLaunchKernelGGL(k_spectrum_export, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, s,
                     (const cf*)spec, out, NF, p.N, p.path, p.n1, p.n2, p.spec_stride);
  return hipGetLastError();
}

}  // namespace hyena
