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

constexpr int kFgThreads = 256;
constexpr int kFgChunk = 64;   // filter rows per block (layer 1-2 recomputed per chunk)

template <int H>
__global__ void __launch_bounds__(kFgThreads) k_filter_gen(FilterGenArgs a) {
  const int64_t t = (int64_t)blockIdx.x * kFgThreads + threadIdx.x;
  if (t >= a.L) return;
  const int K = a.K;
  const float tl = (float)t / (float)a.L;
  float es[kMaxFreq + 1], ec[kMaxFreq + 1];
#pragma unroll
  for (int k = 1; k <= kMaxFreq; ++k) {
    es[k] = 0.f; ec[k] = 0.f;
    if (k <= K) {
      // phase k t / L reduced modulo 1 exactly in integers
      const int64_t m = ((int64_t)k * t) % a.L;
      sincospif(2.0f * (float)m / (float)a.L, &es[k], &ec[k]);
    }
  }
  const int F = 1 + 2 * K;
  float a1[H];
#pragma unroll
  for (int q = 0; q < H; ++q) {
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
    a1[q] = sinf(acc);
  }
  float a2[H];
#pragma unroll
  for (int q = 0; q < H; ++q) {
    const float* w = a.W2 + q * H;
    float acc = a.b2 ? a.b2[q] : 0.f;
#pragma unroll
    for (int m = 0; m < H; ++m) acc = fmaf(w[m], a1[m], acc);
    a2[q] = sinf(acc);
  }
  const int NF = a.N * a.D;
  const int f0 = blockIdx.y * kFgChunk;
  const int f1 = (f0 + kFgChunk < NF) ? f0 + kFgChunk : NF;
  for (int f = f0; f < f1; ++f) {
    const float* w = a.W3 + (int64_t)f * H;
    float acc = a.b3 ? a.b3[f] : 0.f;
#pragma unroll
    for (int m = 0; m < H; ++m) acc = fmaf(w[m], a2[m], acc);
    const int d = f % a.D;
    const float win = expf(-a.alpha[d] * tl);
    a.h[(int64_t)f * a.L + t] = win * acc;
  }
}

hipError_t filter_gen(const FilterGenArgs& a, hipStream_t s) {
  const int NF = a.N * a.D;
  const dim3 grid((unsigned)((a.L + kFgThreads - 1) / kFgThreads), (unsigned)((NF + kFgChunk - 1) / kFgChunk));
  const dim3 block(kFgThreads);
  switch (a.H) {
    case 8: hipLaunchKernelGGL((k_filter_gen<8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_filter_gen<16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_filter_gen<32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_filter_gen<64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((k_filter_gen<128>), grid, block, 0, s, a); break;
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
