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
#define HYENA_SINGLE_E16_MIN 1024
#endif

// 16 points per thread from N = HYENA_SINGLE_E16_MIN up, 8 below.
template <int N> struct SinglePlan {
  static constexpr bool E16 = N >= HYENA_SINGLE_E16_MIN;
  static constexpr int E = E16 ? 16 : 8;
  static constexpr int T = N / E;
  using R = typename std::conditional<E16, typename Plan16<(N >= 1024 ? N : 1024)>::R,
                                      typename Plan8<(N < 16384 ? N : 8192)>::R>::type;
};

// Spectrum layout on this path: row f = n*D + d holds S(k) = H(k)/(2N) for
// k = 0..N in natural order, rows spec_stride complex values apart.
template <int N, int IOT>
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
  for (int i = 0; i < E; ++i) {
    const int64_t t = 2 * (int64_t)(j + i * S);
    u[i] = make_float2(0.f, 0.f);
    if (i < E / 2) u[i] = make_float2(ld_masked<IOT>(v, off, t, L), ld_masked<IOT>(v, off, t + 1, L));
  }

  for (int n = 0; n < NORD; ++n) {
    fft.template run<false>(u, lds, j);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E; ++i) lds(j + i * S) = u[i];
    __syncthreads();
    const cf* g = spec + (int64_t)(n * D + d) * spec_stride;
    const cf wb = opaque(wbase);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k = j + i * S;
      const cf am = lds((N - k) & (N - 1));
      u[i] = realconv_bin(u[i], am, g[k], g[N - k], cmul(wb, w2e<E>(i)));
    }
    fft.template run<true>(u, lds, j);
    const void* xn = x.p[n];
    const bool last = (n == NORD - 1);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t t = 2 * (int64_t)(j + i * S);
      cf z = make_float2(0.f, 0.f);
      if (i < E / 2) {
        z.x = ld_masked<IOT>(xn, off, t, L) * u[i].x;
        z.y = ld_masked<IOT>(xn, off, t + 1, L) * u[i].y;
        if (last) {
          if (t < L) IO<IOT>::st(y, off + t, z.x);
          if (t + 1 < L) IO<IOT>::st(y, off + t + 1, z.y);
        }
      }
      u[i] = z;
    }
  }
}

// One filter row f of the NF = N*D rows of h per workgroup.
template <int N>
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
  for (int i = 0; i < E; ++i) {
    const int64_t t = 2 * (int64_t)(j + i * S);
    u[i] = make_float2(0.f, 0.f);
    if (i < E / 2) u[i] = make_float2(t < L ? h[off + t] : 0.f, t + 1 < L ? h[off + t + 1] : 0.f);
  }
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
  hipLaunchKernelGGL((k_single_forward<N, IOT>), dim3(a.n_rows), dim3(SinglePlan<N>::T), 0, s, a.v, a.x,
                     (const cf*)a.spec, a.y, a.D, a.NORD, (int)a.L, a.spec_stride);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_spec(const SpectrumArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_single_spectrum<N>), dim3(a.NF), dim3(SinglePlan<N>::T), 0, s, a.h, (cf*)a.spec,
                     (int)a.L, a.spec_stride);
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
