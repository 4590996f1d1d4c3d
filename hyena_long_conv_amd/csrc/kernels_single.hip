// kernels_single.hip -- single-pass Hyena forward and filter spectrum for
// complex FFT lengths N <= 16384 (sequence length L <= 16384).
//
// One workgroup owns one real row (b, d) for the whole order-N recurrence:
// per order n it runs the forward FFT, the spectral product with filter
// h_n[d], the inverse FFT and the gate with x_n.  The state z_n stays in
// registers/LDS between orders and never goes back to HBM (the fused-kernel
// principle of the gist.science HyenaND summary, section "実装: nSubQ";
// recurrence of the Hyena Hierarchy explainer, section "Hyena 演算子の形").
#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {

#ifndef HYENA_SINGLE_WAVES
#define HYENA_SINGLE_WAVES 1
#endif
#ifndef HYENA_SINGLE_E16_MIN
#define HYENA_SINGLE_E16_MIN 16384
#endif

// 8 points per thread below N = HYENA_SINGLE_E16_MIN (fewer registers, more
// waves per CU; measured faster than 16 on the 2K-context shape), 16 above.
template <int N> struct SinglePlan {
  static constexpr bool E16 = N >= HYENA_SINGLE_E16_MIN;
  static constexpr int E = E16 ? 16 : 8;
  static constexpr int T = N / E;
  using R = typename std::conditional<E16, typename Plan16<(N >= 1024 ? N : 1024)>::R,
                                      typename Plan8<(N < 16384 ? N : 8192)>::R>::type;
};

// Spectral step of one order on the registers of a single-pass workgroup:
// u[i] holds C(k), k = j + i*S, on entry and C'(k) on exit.  Bins pair up
// as (k, N-k); the thread owning the low index i < E/2 of a pair computes
// both results (the partner bin lives in thread S-j at index E-1-i, or in
// thread 0 itself at E-i), exchanging through LDS.  k = 0 and k = N/2 pair
// with themselves.
template <int N, int E, class Lds>
__device__ __forceinline__ void spectral_step(cf (&u)[E], const Lds& lds, int j, const cf* g, cf wb) {
  constexpr int S = N / E;
  __syncthreads();
#pragma unroll
  for (int i = E / 2; i < E; ++i) lds(j + i * S) = u[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    const int k = j + i * S;
    if (i == 0 && j == 0) {
      u[0] = realconv_bin(u[0], u[0], g[0], g[N], make_float2(1.f, 0.f));
    } else {
      const int km = N - k;
      cf b = lds(km);
      realconv_pair(u[i], b, g[k], g[km], cmul(wb, w2e<E>(i)));
      lds(km) = b;
    }
  }
  if (j == 0) {
    const cf a = lds(N / 2), gh = g[N / 2];
    lds(N / 2) = realconv_bin(a, a, gh, gh, make_float2(0.f, -1.f));
  }
  __syncthreads();
#pragma unroll
  for (int i = E / 2; i < E; ++i) u[i] = lds(j + i * S);
}

// Spectrum layout on this path: row f = n*D + d holds S(k) = H(k)/(2N) for
// k = 0..N in natural order, rows spec_stride complex values apart.
template <int N, int IOT, bool EVEN>
__global__ void __launch_bounds__(SinglePlan<N>::T, HYENA_SINGLE_WAVES)
k_single_forward(const void* __restrict__ v, XPtrs x, const cf* __restrict__ spec, void* __restrict__ y,
                 int D, int NORD, int L, int64_t spec_stride) {
  using P = SinglePlan<N>;
  constexpr int E = P::E, S = N / E;
  __shared__ cf smem[RowLds::padded(N)];
  const RowLds lds{smem};
  const int j = threadIdx.x;
  const int r = blockIdx.x, d = r % D;
  const int64_t off = (int64_t)r * L;
  BlockFFT<N, E, typename P::R> fft;
  fft.init(j);
  const cf wbase = twiddle<false>((uint32_t)j, (uint32_t)(2 * N));   // W_M^j

  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i)
    u[i] = (i < E / 2) ? ld_pair<IOT, EVEN>(v, off, 2 * (int64_t)(j + i * S), L) : make_float2(0.f, 0.f);

  for (int n = 0; n < NORD; ++n) {
    fft.template run<false>(u, lds, j);
    spectral_step<N, E>(u, lds, j, spec + (int64_t)(n * D + d) * spec_stride, opaque(wbase));
    fft.template run<true>(u, lds, j);
    const void* xn = x.p[n];
    const bool last = (n == NORD - 1);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      cf z = make_float2(0.f, 0.f);
      if (i < E / 2) {
        const int64_t t = 2 * (int64_t)(j + i * S);
        const cf xv = ld_pair<IOT, EVEN>(xn, off, t, L);
        z = make_float2(xv.x * u[i].x, xv.y * u[i].y);
        if (last) st_pair<IOT, EVEN>(y, off, t, L, z);
      }
      u[i] = z;
    }
  }
}

// One filter row f of the NF = N*D rows of h per workgroup.
template <int N, bool EVEN>
__global__ void __launch_bounds__(SinglePlan<N>::T)
k_single_spectrum(const float* __restrict__ h, cf* __restrict__ spec, int L, int64_t spec_stride) {
  using P = SinglePlan<N>;
  constexpr int E = P::E, S = N / E;
  __shared__ cf smem[RowLds::padded(N)];
  const RowLds lds{smem};
  const int j = threadIdx.x;
  const int64_t off = (int64_t)blockIdx.x * L;
  BlockFFT<N, E, typename P::R> fft;
  fft.init(j);
  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i)
    u[i] = (i < E / 2) ? ld_pair<0, EVEN>(h, off, 2 * (int64_t)(j + i * S), L) : make_float2(0.f, 0.f);
  fft.template run<false>(u, lds, j);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) lds(j + i * S) = u[i];
  __syncthreads();
  cf* out = spec + (int64_t)blockIdx.x * spec_stride;
  const cf wbase = twiddle<false>((uint32_t)j, (uint32_t)(2 * N));
  const float sc = 1.0f / (float)(2 * N);
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int k = j + i * S;
    const cf am = lds((N - k) & (N - 1));
    out[k] = realfft_bin(u[i], am, cmul(wbase, w2e<E>(i)), sc);
    if (k == 0) out[N] = make_float2((u[i].x - u[i].y) * sc, 0.f);   // Nyquist bin
  }
}

template <int N, int IOT>
static hipError_t launch_fwd(const ForwardArgs& a, hipStream_t s) {
  if (a.L % 2 == 0)
    hipLaunchKernelGGL((k_single_forward<N, IOT, true>), dim3(a.n_rows), dim3(SinglePlan<N>::T), 0, s, a.v,
                       a.x, (const cf*)a.spec, a.y, a.D, a.NORD, (int)a.L, a.spec_stride);
  else
    hipLaunchKernelGGL((k_single_forward<N, IOT, false>), dim3(a.n_rows), dim3(SinglePlan<N>::T), 0, s, a.v,
                       a.x, (const cf*)a.spec, a.y, a.D, a.NORD, (int)a.L, a.spec_stride);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_spec(const SpectrumArgs& a, hipStream_t s) {
  if (a.L % 2 == 0)
    hipLaunchKernelGGL((k_single_spectrum<N, true>), dim3(a.NF), dim3(SinglePlan<N>::T), 0, s, a.h,
                       (cf*)a.spec, (int)a.L, a.spec_stride);
  else
    hipLaunchKernelGGL((k_single_spectrum<N, false>), dim3(a.NF), dim3(SinglePlan<N>::T), 0, s, a.h,
                       (cf*)a.spec, (int)a.L, a.spec_stride);
  return hipGetLastError();
}

hipError_t single_forward(const ForwardArgs& a, int64_t N, hipStream_t s) {
#define HY_CASE(NN)                                                       \
  case NN:                                                                \
    return a.io == 0 ? launch_fwd<NN, 0>(a, s) : launch_fwd<NN, 1>(a, s);
  switch (N) {
    HY_CASE(64) HY_CASE(128) HY_CASE(256) HY_CASE(512) HY_CASE(1024) HY_CASE(2048)
    HY_CASE(4096) HY_CASE(8192) HY_CASE(16384)
    default: return hipErrorInvalidValue;
  }
#undef HY_CASE
}

hipError_t single_spectrum(const SpectrumArgs& a, int64_t N, hipStream_t s) {
#define HY_CASE(NN) \
  case NN: return launch_spec<NN>(a, s);
  switch (N) {
    HY_CASE(64) HY_CASE(128) HY_CASE(256) HY_CASE(512) HY_CASE(1024) HY_CASE(2048)
    HY_CASE(4096) HY_CASE(8192) HY_CASE(16384)
    default: return hipErrorInvalidValue;
  }
#undef HY_CASE
}

}  // namespace hyena
