// kernels_single.hip -- single-pass Hyena forward and filter spectrum for
// FFT lengths M <= 16384 (sequence length L <= 8192).
//
// One workgroup owns one complex signal of M points (two real rows packed as
// real and imaginary parts) for the whole order-N recurrence.  Per order n:
// forward FFT, pointwise product with the filter spectrum, inverse FFT,
// gate with x_n.  The state z_n stays in registers/LDS between orders and
// never goes back to HBM (the fused-kernel principle of the gist.science
// HyenaND summary, section "実装: nSubQ"; recurrence of the Hyena Hierarchy
// explainer, section "Hyena 演算子の形").
#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {

template <int M> struct SinglePlan {
  static constexpr int E = (M >= 1024) ? 16 : 8;
  static constexpr int T = M / E;
  using R = typename std::conditional<(M >= 1024), typename Plan16<(M >= 1024 ? M : 1024)>::R,
                                      typename Plan8<(M < 1024 ? M : 512)>::R>::type;
};

// Spectrum layout on this path: row f = n*D + d holds G(k) = H(k)/M for
// k = 0..M/2 (natural order), rows spaced spec_stride complex values apart.
template <int M, int IOT>
__global__ void __launch_bounds__(SinglePlan<M>::T)
k_single_forward(const void* __restrict__ v, XPtrs x, const cf* __restrict__ spec, void* __restrict__ y,
                 int B, int D, int N, int L, int64_t spec_stride, int n_batch_pairs, int half_b) {
  using P = SinglePlan<M>;
  constexpr int E = P::E, S = M / E;
  __shared__ cf smem[RowLds::padded(M)];
  const RowLds lds{smem};
  const int j = threadIdx.x;
  const Pair pr = decode_pair(blockIdx.x, B, D, L, n_batch_pairs, half_b);
  BlockFFT<M, E, typename P::R> fft;
  fft.init(j);

  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int t = j + i * S;
    u[i] = make_float2(0.f, 0.f);
    if (i < E / 2 && t < L) {
      u[i].x = IO<IOT>::ld(v, pr.off_a + t);
      if (pr.has_b) u[i].y = IO<IOT>::ld(v, pr.off_b + t);
    }
  }

  for (int n = 0; n < N; ++n) {
    fft.template run<false>(u, lds, j);
    const cf* ga = spec + (int64_t)(n * D + pr.da) * spec_stride;
    const cf* gb = spec + (int64_t)(n * D + pr.db) * spec_stride;
    if (pr.same) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int k = j + i * S;
        const cf g = (k <= M / 2) ? ga[k] : cconj(ga[M - k]);
        u[i] = cmul(g, u[i]);
      }
    } else {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < E; ++i) lds(j + i * S) = u[i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int k = j + i * S;
        const int km = (M - k) & (M - 1);
        const cf zm = lds(km);
        const cf gak = (k <= M / 2) ? ga[k] : cconj(ga[M - k]);
        const cf gbk = (k <= M / 2) ? gb[k] : cconj(gb[M - k]);
        u[i] = pair_multiply(u[i], zm, gak, gbk);
      }
    }
    fft.template run<true>(u, lds, j);
    const void* xn = x.p[n];
    const bool last = (n == N - 1);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int t = j + i * S;
      float za = 0.f, zb = 0.f;
      if (i < E / 2 && t < L) {
        za = IO<IOT>::ld(xn, pr.off_a + t) * u[i].x;
        if (pr.has_b) zb = IO<IOT>::ld(xn, pr.off_b + t) * u[i].y;
        if (last) {
          IO<IOT>::st(y, pr.off_a + t, za);
          if (pr.has_b) IO<IOT>::st(y, pr.off_b + t, zb);
        }
      }
      u[i] = make_float2(za, zb);
    }
  }
}

// Filter pair (fa, fb) = (2p, 2p+1) over the NF = N*D rows of h.
template <int M>
__global__ void __launch_bounds__(SinglePlan<M>::T)
k_single_spectrum(const float* __restrict__ h, cf* __restrict__ spec, int NF, int L, int64_t spec_stride) {
  using P = SinglePlan<M>;
  constexpr int E = P::E, S = M / E;
  __shared__ cf smem[RowLds::padded(M)];
  const RowLds lds{smem};
  const int j = threadIdx.x;
  const int fa = 2 * blockIdx.x, fb = fa + 1;
  const bool has_b = fb < NF;
  BlockFFT<M, E, typename P::R> fft;
  fft.init(j);
  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int t = j + i * S;
    u[i] = make_float2(0.f, 0.f);
    if (i < E / 2 && t < L) {
      u[i].x = h[(int64_t)fa * L + t];
      if (has_b) u[i].y = h[(int64_t)fb * L + t];
    }
  }
  fft.template run<false>(u, lds, j);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) lds(j + i * S) = u[i];
  __syncthreads();
  const float sc = 0.5f / (float)M;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int k = j + i * S;
    if (k <= M / 2) {
      const cf zm = lds((M - k) & (M - 1));
      const cf z = u[i];
      // Ha = (Z + conj Zm)/2, Hb = (Z - conj Zm)/(2i); stored divided by M.
      spec[(int64_t)fa * spec_stride + k] = make_float2((z.x + zm.x) * sc, (z.y - zm.y) * sc);
      if (has_b) spec[(int64_t)fb * spec_stride + k] = make_float2((z.y + zm.y) * sc, (zm.x - z.x) * sc);
    }
  }
}

template <int M, int IOT>
static hipError_t launch_fwd(const ForwardArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_single_forward<M, IOT>), dim3(a.n_pairs), dim3(SinglePlan<M>::T), 0, s,
                     a.v, a.x, (const cf*)a.spec, a.y, a.B, a.D, a.N, (int)a.L, a.spec_stride,
                     a.n_batch_pairs, a.half_b);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_spec(const SpectrumArgs& a, hipStream_t s) {
  const int npairs = (a.NF + 1) / 2;
  hipLaunchKernelGGL((k_single_spectrum<M>), dim3(npairs), dim3(SinglePlan<M>::T), 0, s, a.h,
                     (cf*)a.spec, a.NF, (int)a.L, a.spec_stride);
  return hipGetLastError();
}

hipError_t single_forward(const ForwardArgs& a, int64_t M, hipStream_t s) {
#define HY_CASE(MM)                                                       \
  case MM:                                                                \
    return a.io == 0 ? launch_fwd<MM, 0>(a, s) : launch_fwd<MM, 1>(a, s);
  switch (M) {
    HY_CASE(64) HY_CASE(128) HY_CASE(256) HY_CASE(512) HY_CASE(1024) HY_CASE(2048)
    HY_CASE(4096) HY_CASE(8192) HY_CASE(16384)
    default: return hipErrorInvalidValue;
  }
#undef HY_CASE
}

hipError_t single_spectrum(const SpectrumArgs& a, int64_t M, hipStream_t s) {
#define HY_CASE(MM) \
  case MM: return launch_spec<MM>(a, s);
  switch (M) {
    HY_CASE(64) HY_CASE(128) HY_CASE(256) HY_CASE(512) HY_CASE(1024) HY_CASE(2048)
    HY_CASE(4096) HY_CASE(8192) HY_CASE(16384)
    default: return hipErrorInvalidValue;
  }
#undef HY_CASE
}

}  // namespace hyena
