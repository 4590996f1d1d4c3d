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
#ifndef HYENA_XCD_MAP
#define HYENA_XCD_MAP 1
#endif
#ifndef HYENA_SINGLE_PERSIST
#define HYENA_SINGLE_PERSIST 1
#endif
#ifndef HYENA_SINGLE_E16_MIN
#define HYENA_SINGLE_E16_MIN 16384
#endif

// 8 points per thread below N = HYENA_SINGLE_E16_MIN (fewer registers, more
// waves per CU; measured faster than 16 on the 2K-context shape), 16 above.
// SW: XOR-swizzled LDS exchange buffers; PP: two exchange buffers (one
// barrier per FFT stage instead of two; 16*N bytes of LDS).  Both chosen per
// length from timings at D = 768 with the batch rows of a channel on one XCD
// (swizzle off only at 16384, where it costs registers and spills; two
// buffers from 2048 to 8192, where together with the swizzle they were
// faster by 1.5-3%).
template <int N> struct SinglePlan {
  static constexpr bool E16 = N >= HYENA_SINGLE_E16_MIN;
  static constexpr int E = E16 ? 16 : 8;
  static constexpr int T = N / E;
#ifdef HYENA_SINGLE_SW
  static constexpr bool SW = HYENA_SINGLE_SW;
#else
  static constexpr bool SW = N != 16384;
#endif
#ifdef HYENA_SINGLE_PP
  static constexpr bool PP = HYENA_SINGLE_PP && N <= 8192;
#else
  static constexpr bool PP = N >= 2048 && N <= 8192;
#endif
  // PF: request each order's filter coefficients and gate inputs before its
  // forward FFT (their latency hides behind it), where the registers allow.
#ifdef HYENA_SINGLE_PF
  static constexpr bool PF = HYENA_SINGLE_PF && N <= 4096;
#else
  static constexpr bool PF = N <= 2048;
#endif
  using Lds = RowLdsT<SW>;
  using R = typename std::conditional<E16, typename Plan16<(N >= 1024 ? N : 1024)>::R,
                                      typename Plan8<(N < 16384 ? N : 8192)>::R>::type;
};

// Pair coefficients of one filter for the bins a thread owns, loaded ahead
// of the forward FFT so the loads are in flight while it runs.
template <int N, int E>
struct PairCoeffs {
  cf a1[E / 2], a2[E / 2], bq[E / 2];
  cf half;   // a1 of p = N/2 (used by thread 0)
  __device__ __forceinline__ void load(const cf* g, int64_t qs, int j) {
    constexpr int S = N / E;
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      const int p = j + i * S;
      a1[i] = g[p];
      a2[i] = g[qs + p];
      bq[i] = g[2 * qs + p];
    }
    half = g[N / 2];
  }
};

// Spectral step of one order on the registers of a single-pass workgroup:
// u[i] holds C(k), k = j + i*S, on entry and C'(k) on exit.  Bins pair up
// as (p, N-p); the thread owning the low index i < E/2 of a pair computes
// both results (the partner bin lives in thread S-j at index E-1-i, or in
// thread 0 itself at E-i), exchanging through LDS.  p = 0 and p = N/2 pair
// with themselves.
template <int N, int E, bool LEAD_BARRIER, class Lds>
__device__ __forceinline__ void spectral_step(cf (&u)[E], const Lds& lds, int j, const PairCoeffs<N, E>& c) {
  constexpr int S = N / E;
  if constexpr (LEAD_BARRIER) __syncthreads();
#pragma unroll
  for (int i = E / 2; i < E; ++i) lds(j + i * S) = u[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    const int p = j + i * S;
    if (i == 0 && j == 0) {
      u[0] = conv_self(u[0], c.a1[0], c.bq[0]);
    } else {
      cf b = lds(N - p);
      conv_pair(u[i], b, c.a1[i], c.a2[i], c.bq[i]);
      lds(N - p) = b;
    }
  }
  if (j == 0) lds(N / 2) = cmul(lds(N / 2), c.half);   // p = N/2: bq = 0
  __syncthreads();
#pragma unroll
  for (int i = E / 2; i < E; ++i) u[i] = lds(j + i * S);
}

// Spectrum layout on this path: filter row f = n*D + d starts at
// f*spec_stride and holds the pair coefficients a1[p], a2[p], bq[p]
// (p = 0..N/2) of conv_pair as three arrays qs = spec_stride/3 values apart.
// Row handled by workgroup wg.  Workgroups are dispatched round-robin over
// the 8 XCDs (wg mod 8), each with its own L2; when D is a multiple of 8 the
// B rows of one channel, which share a filter spectrum, go to consecutive
// workgroups of the same XCD so the spectrum is fetched into that L2 once.
__device__ __forceinline__ int row_of_workgroup(int wg, int B, int D) {
  if (HYENA_XCD_MAP && (D & 7) == 0) {
    const int xcd = wg & 7, slot = wg >> 3;
    const int d = (slot / B) * 8 + xcd, b = slot - (slot / B) * B;
    return b * D + d;
  }
  return wg;
}

// FULL: circular mode, the row fills all M = 2N samples (no zero half);
// otherwise the row occupies the first half of each thread's points.
// EXACT: L = N, so (like FULL) every sample a thread reads or writes is in
// the row and the accesses need no mask.
template <int N, int IOT, bool EVEN, bool FULL, bool EXACT = false>
__global__ void __launch_bounds__(SinglePlan<N>::T, HYENA_SINGLE_WAVES)
k_single_forward(const void* __restrict__ v, XPtrs x, const cf* __restrict__ spec, void* __restrict__ y,
                 int B, int D, int NORD, int L, int64_t spec_stride, int n_rows) {
  using P = SinglePlan<N>;
  constexpr int E = P::E, S = N / E, NV = FULL ? E : E / 2;
  constexpr bool IN = FULL || EXACT;
  const auto ldp = [&](const void* p, int64_t o, int t) {
    if constexpr (IN) return ld_pair_in<IOT>(p, o, t);
    else return ld_pair<IOT, EVEN, true>(p, o, (int64_t)t, L);
  };
  __shared__ cf smem[P::PP ? 2 * N : N];
  using Lds = typename P::Lds;
  const Lds lds2[2] = {Lds{smem}, Lds{smem + (P::PP ? N : 0)}};
  const int j = threadIdx.x;
  BlockFFT<N, E, typename P::R> fft;
  fft.init(j);
  const int64_t qs = spec_stride / 3;
  // A workgroup takes rows wg, wg + gridDim.x, ... (one row when the grid
  // covers them all).  Each row's first LDS store follows a barrier inside
  // the forward FFT, so consecutive rows need no extra synchronisation.
  for (int wg = blockIdx.x; wg < n_rows; wg += gridDim.x) {
  const int r = row_of_workgroup(wg, B, D), d = r % D;
  const int64_t off = (int64_t)r * L;

  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i) u[i] = (i < NV) ? ldp(v, off, 2 * (j + i * S)) : make_float2(0.f, 0.f);

  for (int n = 0; n < NORD; ++n) {
    const cf* g = spec + (int64_t)(n * D + d) * spec_stride;
    const void* xn = x.p[n];
    PairCoeffs<N, E> pc;
    cf xv[NV];
    if constexpr (P::PF) {
      pc.load(g, qs, j);
#pragma unroll
      for (int i = 0; i < NV; ++i) xv[i] = ldp(xn, off, 2 * (j + i * S));
    }
    if constexpr (P::PP) {
      fft.template run_pp<false>(u, lds2, j);
      if constexpr (!P::PF) pc.load(g, qs, j);
      // the buffer the forward FFT's last stage did not read is free, so the
      // exchange needs no leading barrier
      spectral_step<N, E, false>(u, lds2[fft.last_buf() ^ 1], j, pc);
      fft.template run_pp<true>(u, lds2, j);
    } else {
      fft.template run<false>(u, lds2[0], j);
      if constexpr (!P::PF) pc.load(g, qs, j);
      spectral_step<N, E, true>(u, lds2[0], j, pc);
      fft.template run<true>(u, lds2[0], j);
    }
    if constexpr (!P::PF) {
#pragma unroll
      for (int i = 0; i < NV; ++i) xv[i] = ldp(xn, off, 2 * (j + i * S));
    }
    const bool last = (n == NORD - 1);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      cf z = make_float2(0.f, 0.f);
      if (i < NV) {
        const int t = 2 * (j + i * S);
        z = make_float2(xv[i].x * u[i].x, xv[i].y * u[i].y);
        if (last) {
          if constexpr (IN) st_pair_in<IOT>(y, off, t, z);
          else st_pair<IOT, EVEN>(y, off, (int64_t)t, L, z);
        }
      }
      u[i] = z;
    }
  }
  }
}

// One filter row f of the NF = N*D rows of h per workgroup: the real FFT
// H(k)/M of the zero-padded row (k = 0..N, staged in LDS), then the pair
// coefficients of conv_pair for p = 0..N/2.
template <int N, bool EVEN, bool FULL>
__global__ void __launch_bounds__(SinglePlan<N>::T)
k_single_spectrum(const float* __restrict__ h, cf* __restrict__ spec, int L, int64_t spec_stride) {
  using P = SinglePlan<N>;
  constexpr int E = P::E, S = N / E, NV = FULL ? E : E / 2;
  __shared__ cf smem[N];
  __shared__ cf nyq;
  const typename P::Lds lds{smem};
  const int j = threadIdx.x;
  const int64_t off = (int64_t)blockIdx.x * L;
  BlockFFT<N, E, typename P::R> fft;
  fft.init(j);
  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i)
    u[i] = (i < NV) ? ld_pair<0, EVEN>(h, off, 2 * (int64_t)(j + i * S), L) : make_float2(0.f, 0.f);
  fft.template run<false>(u, lds, j);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) lds(j + i * S) = u[i];
  __syncthreads();
  const cf wbase = twiddle<false>((uint32_t)j, (uint32_t)(2 * N));
  const float sc = 1.0f / (float)(2 * N);
  cf hv[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int k = j + i * S;
    const cf am = lds((N - k) & (N - 1));
    hv[i] = realfft_bin(u[i], am, cmul(wbase, w2e<E>(i)), sc);
    if (k == 0) nyq = make_float2((u[i].x - u[i].y) * sc, 0.f);   // H(N)/M
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) lds(j + i * S) = hv[i];               // H(k)/M, k < N
  __syncthreads();
  const int64_t qs = spec_stride / 3;
  cf* out = spec + (int64_t)blockIdx.x * spec_stride;
  for (int p = j; p <= N / 2; p += S) {
    float sn, cs;
    sincospif((float)p / (float)N, &sn, &cs);
    cf a1, a2, bq;
    pair_coeffs(lds(p), p == 0 ? nyq : lds(N - p), sn, cs, a1, a2, bq);
    out[p] = a1;
    out[qs + p] = a2;
    out[2 * qs + p] = bq;
  }
}

// ------------------------------------------------------------------ backward
//
// Gradients of the recurrence by the chain rule; the adjoint of a causal
// convolution is the correlation with the same filter, i.e. the spectral
// step with conjugated coefficients.  One workgroup per channel d walks the
// B rows of that channel, so the filter gradients sum over the batch in its
// own accumulators (deterministically).  Per row: the forward is recomputed
// and each convolution output c_n saved (cbuf); then for n = N..1, with g the
// gradient of z_{n+1}:  gx_n = g * c_n,  gc = g * x_n,  the spectra of z_n and
// gc,  the filter-gradient term (spectral step whose "filter" is conj of z_n's
// spectrum, pair coefficients built on the fly) added into hacc[n], and the
// adjoint step plus inverse FFT give the gradient of z_n.  Finally each
// hacc[n] is inverse transformed into gh_n.
// HL: the filter-gradient accumulators live in LDS (NORD x N values of
// dynamic shared memory; each thread only touches its own points, so no
// barrier guards them) instead of the hacc workspace.
// FULL: circular mode (L = 2N, every point of the row is a sample).
template <int N, int IOT, bool EVEN, bool HL, bool FULL>
__global__ void __launch_bounds__(SinglePlan<N>::T, 1)
k_single_backward(const void* __restrict__ v, XPtrs x, const cf* __restrict__ spec, const void* __restrict__ gy,
                  void* __restrict__ gv, OutPtrs gx, float* __restrict__ gh, cf* __restrict__ cbuf,
                  cf* __restrict__ hacc, int B, int D, int NORD, int L, int64_t spec_stride) {
  using P = SinglePlan<N>;
  constexpr int E = P::E, S = N / E, H2 = N / 2;
  constexpr int NV = FULL ? E : E / 2;           // points of a thread that hold samples
  constexpr int CBS = FULL ? N : H2;             // saved c_n per row (packed points)
  __shared__ cf smem[N];
  extern __shared__ cf hl[];
  const typename P::Lds lds{smem};
  const int j = threadIdx.x, d = blockIdx.x;
  BlockFFT<N, E, typename P::R> fft;
  fft.init(j);
  const int64_t qs = spec_stride / 3;
  const cf wbase = twiddle<false>((uint32_t)j, (uint32_t)(2 * N));   // W_M^j
  const float scM = 1.0f / (float)(2 * N);
  const auto had = [](cf a, cf b) { return make_float2(a.x * b.x, a.y * b.y); };   // sample-wise product

  for (int b = 0; b < B; ++b) {
    const int64_t off = ((int64_t)b * D + d) * L;
    cf u[E];
#pragma unroll
    for (int i = 0; i < E; ++i)
      u[i] = (i < NV) ? ld_pair<IOT, EVEN, true>(v, off, 2 * (int64_t)(j + i * S), L) : make_float2(0.f, 0.f);
    // forward, saving c_n (packed points j + i*S, i < E/2)
    for (int n = 0; n < NORD; ++n) {
      PairCoeffs<N, E> pc;
      pc.load(spec + (int64_t)(n * D + d) * spec_stride, qs, j);
      fft.template run<false>(u, lds, j);
      spectral_step<N, E, true>(u, lds, j, pc);
      fft.template run<true>(u, lds, j);
      cf* cb = cbuf + (((int64_t)n * B + b) * D + d) * CBS;
      const void* xn = x.p[n];
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (i < NV) {
          cb[j + i * S] = u[i];
          u[i] = had(ld_pair<IOT, EVEN, true>(xn, off, 2 * (int64_t)(j + i * S), L), u[i]);
        } else {
          u[i] = make_float2(0.f, 0.f);
        }
      }
    }
    // backward
    cf g[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) g[i] = ld_pair<IOT, EVEN, true>(gy, off, 2 * (int64_t)(j + i * S), L);
    for (int n = NORD - 1; n >= 0; --n) {
      const cf* cb = cbuf + (((int64_t)n * B + b) * D + d) * CBS;
      const cf* cbp = cbuf + (((int64_t)(n > 0 ? n - 1 : 0) * B + b) * D + d) * CBS;
      const void* xn = x.p[n];
      const void* xp = x.p[n > 0 ? n - 1 : 0];
      PairCoeffs<N, E> pc;
      pc.load(spec + (int64_t)(n * D + d) * spec_stride, qs, j);
      cf zt[E], gt[E];
      {
        // every load of the step first (one branch on the order for z_n's
        // inputs), then the products and the gx_n stores: loads and stores
        // interleaved point by point waited for each other
        cf cv[NV], xv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int64_t t = 2 * (int64_t)(j + i * S);
          cv[i] = cb[j + i * S];
          xv[i] = ld_pair<IOT, EVEN, true>(xn, off, t, L);
        }
        if (n == 0) {
#pragma unroll
          for (int i = 0; i < NV; ++i) zt[i] = ld_pair<IOT, EVEN, true>(v, off, 2 * (int64_t)(j + i * S), L);
        } else {
#pragma unroll
          for (int i = 0; i < NV; ++i)
            zt[i] = had(ld_pair<IOT, EVEN, true>(xp, off, 2 * (int64_t)(j + i * S), L), cbp[j + i * S]);   // z_n
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          st_pair<IOT, EVEN>(gx.p[n], off, 2 * (int64_t)(j + i * S), L, had(g[i], cv[i]));   // gx_n = g * c_n
          gt[i] = had(g[i], xv[i]);                                                       // gc = g * x_n
        }
#pragma unroll
        for (int i = NV; i < E; ++i) {
          zt[i] = make_float2(0.f, 0.f);
          gt[i] = make_float2(0.f, 0.f);
        }
      }
      fft.template run<false>(zt, lds, j);
      fft.template run<false>(gt, lds, j);
      // exchange: high halves of Z at k (k >= N/2), of G at k - N/2
      __syncthreads();
#pragma unroll
      for (int i = E / 2; i < E; ++i) {
        lds(j + i * S) = zt[i];
        lds(j + i * S - H2) = gt[i];
      }
      __syncthreads();
      cf pz[E];
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const cf w = cmul(wbase, w2e<E>(i));                 // W_M^p, p = j + i*S
        if (i == 0 && j == 0) {                              // p = 0: its own partner
          const cf z0 = zt[0];
          cf f1, f2, fq;
          pair_coeffs(make_float2((z0.x + z0.y) * scM, 0.f), make_float2((z0.x - z0.y) * scM, 0.f), 0.f, 1.f,
                      f1, f2, fq);
          pz[0] = conv_self(gt[0], f1, fq);
          gt[0] = conv_self(gt[0], cconj(pc.a1[0]), cconj(pc.bq[0]));
        } else {
          const int m = N - (j + i * S);
          const cf zm = lds(m), gm = lds(m - H2);
          const cf xk = realfft_bin(zt[i], zm, w, scM);                     // X_z(p) / M
          const cf xm = realfft_bin(zm, zt[i], make_float2(-w.x, w.y), scM);  // X_z(N-p) / M
          cf f1, f2, fq;
          pair_coeffs(cconj(xk), cconj(xm), -w.y, w.x, f1, f2, fq);
          cf pa = gt[i], pb = gm;
          conv_pair(pa, pb, f1, f2, fq);                     // filter-gradient spectrum at p, N-p
          cf ga = gt[i], gb = gm;
          conv_pair(ga, gb, cconj(pc.a1[i]), cconj(pc.a2[i]), cconj(pc.bq[i]));   // adjoint step
          pz[i] = pa;
          gt[i] = ga;
          lds(m) = pb;
          lds(m - H2) = gb;
        }
      }
      if (j == 0) {                                          // p = N/2: its own partner
        const cf zh = lds(H2), gq = lds(0);
        const cf xh = realfft_bin(zh, zh, make_float2(0.f, -1.f), scM);
        cf f1, f2, fq;
        pair_coeffs(cconj(xh), cconj(xh), 1.f, 0.f, f1, f2, fq);
        lds(H2) = cmul(f1, gq);
        lds(0) = cmul(cconj(pc.half), gq);
      }
      __syncthreads();
#pragma unroll
      for (int i = E / 2; i < E; ++i) {
        pz[i] = lds(j + i * S);
        gt[i] = lds(j + i * S - H2);
      }
      cf* ha = HL ? hl + n * N : hacc + ((int64_t)n * D + d) * N;
#pragma unroll
      for (int i = 0; i < E; ++i) ha[j + i * S] = (b == 0) ? pz[i] : cadd(ha[j + i * S], pz[i]);
      fft.template run<true>(gt, lds, j);
#pragma unroll
      for (int i = 0; i < NV; ++i) g[i] = gt[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) st_pair<IOT, EVEN>(gv, off, 2 * (int64_t)(j + i * S), L, g[i]);
  }
  // filter gradients: inverse transform of each accumulated spectrum
  for (int n = 0; n < NORD; ++n) {
    const cf* ha = HL ? hl + n * N : hacc + ((int64_t)n * D + d) * N;
    cf u[E];
#pragma unroll
    for (int i = 0; i < E; ++i) u[i] = ha[j + i * S];
    fft.template run<true>(u, lds, j);
    float* out = gh + ((int64_t)n * D + d) * L;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t t = 2 * (int64_t)(j + i * S);
      if (t < L) out[t] = u[i].x;
      if (t + 1 < L) out[t + 1] = u[i].y;
    }
  }
}

#ifndef HYENA_BWD_LDS_ACC
#define HYENA_BWD_LDS_ACC (52 * 1024)   // LDS budget per workgroup for accumulators in LDS (0: never)
#endif

template <int N, int IOT, bool EVEN, bool HL, bool FULL = false>
static void launch_bwd_k(const BackwardArgs& a, size_t shared, hipStream_t s) {
  hipLaunchKernelGGL((k_single_backward<N, IOT, EVEN, HL, FULL>), dim3(a.D), dim3(SinglePlan<N>::T), shared, s, a.v, a.x,
                     (const cf*)a.spec, a.gy, a.gv, a.gx, a.gh, (cf*)a.cbuf, (cf*)a.hacc, a.B, a.D, a.NORD,
                     (int)a.L, a.spec_stride);
}

template <int N, int IOT>
static hipError_t launch_bwd(const BackwardArgs& a, hipStream_t s) {
  // Accumulators in LDS when they and the FFT buffer fit the budget that
  // keeps three workgroups per CU (the launch has only D workgroups).
  const size_t acc = (size_t)a.NORD * N * sizeof(cf);
  const bool hl = acc + N * sizeof(cf) <= (size_t)HYENA_BWD_LDS_ACC;
  if (a.circular) {   // L = 2N, even
    if (hl) launch_bwd_k<N, IOT, true, true, true>(a, acc, s);
    else launch_bwd_k<N, IOT, true, false, true>(a, 0, s);
  } else if (a.L % 2 == 0) {
    if (hl) launch_bwd_k<N, IOT, true, true>(a, acc, s);
    else launch_bwd_k<N, IOT, true, false>(a, 0, s);
  } else {
    if (hl) launch_bwd_k<N, IOT, false, true>(a, acc, s);
    else launch_bwd_k<N, IOT, false, false>(a, 0, s);
  }
  return hipGetLastError();
}

// Workgroups of kernel k that fit the GPU at once (0 if the query fails).
template <class K>
static int resident_workgroups(K k, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

// ------------------------------------------- cross-lane variant (N = 2048)
//
// HYENA_SINGLE_XLANE=1 builds a variant of the forward for N = 2048 complex
// points (rows of L <= 2048) whose FFT exchanges data inside a wave with
// lane permutations instead of LDS: of the three exchanges per FFT of the
// LDS version, only the one across the four waves stays in LDS.  Index
// n = j + 256 i (thread j = 64 w + l, lane l = l0 + 8 l1, register i):
//   1. DFT_8 over i in registers, twiddle W_2048^(j k_i);
//   2. DFT_4 over w (LDS exchange: wave w' takes the series k_i = 2w', 2w'+1),
//      twiddle W_256^(l k_w);
//   3. DFT_64 over l: swap register bits with lane bits 3..5 (8x8
//      register/lane transpose: DPP row_ror:8, v_permlane16_swap,
//      v_permlane32_swap), DFT_8 over l1, twiddle W_64^(l0 k0), swap register
//      bits with lane bits 0..2 (DPP quad permutations and row shifts), DFT_8
//      over l0.
// Thread (w, L) then holds bin k = 2w + (L >> 5) + 8 ((L >> 3) & 3) +
// 32 (L & 7) + 256 r in register r.  The spectral step pairs bins through
// LDS, each thread computing its own bins' outputs, and the inverse FFT is
// the forward's adjoint (same steps in reverse, conjugate twiddles), which
// returns the natural layout for the gate.  Built to measure the cross-lane
// exchanges against LDS exchanges on the VALU-bound single-pass kernel.
#ifndef HYENA_SINGLE_XLANE
#define HYENA_SINGLE_XLANE 0
#endif
#if HYENA_SINGLE_XLANE

namespace xlane {

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// value of lane l ^ 4 (within rows of 16): row_shr:4 into lanes 4-7, 12-15,
// row_shl:4 into lanes 0-3, 8-11
__device__ __forceinline__ float xor4(float v) {
  const int x = __builtin_bit_cast(int, v);
  const int t = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xA, false);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(t, x, 0x104, 0xF, 0x5, false));
}
template <int LB>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (LB == 0) return dpp<0xB1>(v);        // quad_perm [1,0,3,2]
  else if constexpr (LB == 1) return dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  else if constexpr (LB == 2) return xor4(v);
  else return dpp<0x128>(v);                         // row_ror:8
}

// One 2x2 block step of a register/lane transpose: lane bit LB <-> register
// bit RB.  For lanes L0 (bit clear) and L1 (bit set) and registers r0 (bit
// clear) and r1 (bit set): L0.r1 <- L1.r0 and L1.r0 <- L0.r1.
template <int LB, int RB>
__device__ __forceinline__ void tstep(cf (&u)[8], int lane) {
#pragma unroll
  for (int r0 = 0; r0 < 8; ++r0) {
    if (r0 & (1 << RB)) continue;
    const int r1 = r0 | (1 << RB);
    if constexpr (LB == 4 || LB == 5) {
      uint32_t ax = __float_as_uint(u[r0].x), bx = __float_as_uint(u[r1].x);
      uint32_t ay = __float_as_uint(u[r0].y), by = __float_as_uint(u[r1].y);
      if constexpr (LB == 4) {
        const auto px = __builtin_amdgcn_permlane16_swap(ax, bx, false, false);
        const auto py = __builtin_amdgcn_permlane16_swap(ay, by, false, false);
        ax = px[0]; bx = px[1]; ay = py[0]; by = py[1];
      } else {
        const auto px = __builtin_amdgcn_permlane32_swap(ax, bx, false, false);
        const auto py = __builtin_amdgcn_permlane32_swap(ay, by, false, false);
        ax = px[0]; bx = px[1]; ay = py[0]; by = py[1];
      }
      u[r0] = make_float2(__uint_as_float(ax), __uint_as_float(ay));
      u[r1] = make_float2(__uint_as_float(bx), __uint_as_float(by));
    } else {
      // value selects only: selecting between array elements became a
      // run-time index, i.e. a trip through scratch memory
      const bool hi = (lane >> LB) & 1;
      const cf a0 = u[r0], a1 = u[r1];
      const float sx = hi ? a0.x : a1.x, sy = hi ? a0.y : a1.y;
      const float rx = lane_xor<LB>(sx), ry = lane_xor<LB>(sy);
      u[r0] = make_float2(hi ? rx : a0.x, hi ? ry : a0.y);
      u[r1] = make_float2(hi ? a1.x : rx, hi ? a1.y : ry);
    }
  }
}

// register bits 0..2 <-> lane bits 0..2, and <-> lane bits 3..5
__device__ __forceinline__ void transpose_low(cf (&u)[8], int lane) {
  tstep<0, 0>(u, lane);
  tstep<1, 1>(u, lane);
  tstep<2, 2>(u, lane);
}
__device__ __forceinline__ void transpose_high(cf (&u)[8], int lane) {
  tstep<3, 0>(u, lane);
  tstep<4, 1>(u, lane);
  tstep<5, 2>(u, lane);
}

template <bool INV>
__device__ __forceinline__ void twiddle_powers(cf (&u)[8], cf w, int mask) {
  // u[r] *= w^(r & mask), w conjugated for the inverse; the powers are
  // recomputed at every use rather than kept live across the row loop
  const cf b = opaque(INV ? cconj(w) : w);
#pragma unroll
  for (int r = 1; r < 8; ++r)
    if (r & mask) u[r] = cmul(u[r], step_power<8>(make_float2(1.f, 0.f), b, r & mask));
}

template <bool INV>
__device__ __forceinline__ void fft2048(cf (&u)[8], cf* smem, int j, cf t1, cf t2, cf t3) {
  const int w = j >> 6, lane = j & 63;
  if constexpr (!INV) {
    dft<8, false>(u);
    twiddle_powers<false>(u, t1, 7);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) smem[k * 256 + j] = u[k];
    __syncthreads();
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int v = 0; v < 4; ++v) u[sl * 4 + v] = smem[(2 * w + sl) * 256 + v * 64 + lane];
    dft4<false>(u[0], u[1], u[2], u[3]);
    dft4<false>(u[4], u[5], u[6], u[7]);
    twiddle_powers<false>(u, t2, 3);
    transpose_high(u, lane);
    dft<8, false>(u);
    twiddle_powers<false>(u, t3, 7);
    transpose_low(u, lane);
    dft<8, false>(u);
  } else {
    dft<8, true>(u);
    transpose_low(u, lane);
    twiddle_powers<true>(u, t3, 7);
    dft<8, true>(u);
    transpose_high(u, lane);
    twiddle_powers<true>(u, t2, 3);
    dft4<true>(u[0], u[1], u[2], u[3]);
    dft4<true>(u[4], u[5], u[6], u[7]);
    __syncthreads();
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int v = 0; v < 4; ++v) smem[(2 * w + sl) * 256 + v * 64 + lane] = u[sl * 4 + v];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = smem[k * 256 + j];
    twiddle_powers<true>(u, t1, 7);
    dft<8, true>(u);
  }
}

}  // namespace xlane

template <int IOT, bool EVEN, bool EXACT>
__global__ void __launch_bounds__(256, HYENA_SINGLE_WAVES)
k_single_forward_xl(const void* __restrict__ v, XPtrs x, const cf* __restrict__ spec, void* __restrict__ y,
                    int B, int D, int NORD, int L, int64_t spec_stride, int n_rows) {
  constexpr int N = 2048, E = 8, S = N / E, NV = E / 2;
  const auto ldp = [&](const void* p, int64_t o, int t) {
    if constexpr (EXACT) return ld_pair_in<IOT>(p, o, t);
    else return ld_pair<IOT, EVEN, true>(p, o, (int64_t)t, L);
  };
  __shared__ cf smem[N];
  const int j = threadIdx.x, w = j >> 6, lane = j & 63;
  const cf t1 = twiddle<false>((uint32_t)j, 2048u);
  const cf t2 = twiddle<false>((uint32_t)lane, 256u);
  const cf t3 = twiddle<false>((uint32_t)(lane & 7), 64u);
  // bins of this thread: k(r) = kb + 256 r
  const int kb = 2 * w + (lane >> 5) + 8 * ((lane >> 3) & 3) + 32 * (lane & 7);
  const int64_t qs = spec_stride / 3;
  for (int wg = blockIdx.x; wg < n_rows; wg += gridDim.x) {
    const int r = row_of_workgroup(wg, B, D), d = r % D;
    const int64_t off = (int64_t)r * L;
    cf u[E];
#pragma unroll
    for (int i = 0; i < E; ++i) u[i] = (i < NV) ? ldp(v, off, 2 * (j + i * S)) : make_float2(0.f, 0.f);
    for (int n = 0; n < NORD; ++n) {
      const cf* g = spec + (int64_t)(n * D + d) * spec_stride;
      xlane::fft2048<false>(u, smem, j, t1, t2, t3);
      // spectral step: every bin meets its partner N - k through LDS
      __syncthreads();
#pragma unroll
      for (int i = 0; i < E; ++i) smem[kb + 256 * i] = u[i];
      __syncthreads();
      // every bin k: C'(k) = A C(k) + i Bq conj C(N - k), with (A, Bq) =
      // (a1[k], bq[k]) below N/2, (a2[N-k], conj bq[N-k]) above, (a1[N/2], 0)
      // at N/2 (bin 0 pairs with itself)
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int k = kb + 256 * i;
        const int p = k <= N / 2 ? k : N - k;
        const cf A = g[(k <= N / 2 ? 0 : qs) + p];
        cf Bq = g[2 * qs + p];
        Bq = k < N / 2 ? Bq : (k == N / 2 ? make_float2(0.f, 0.f) : cconj(Bq));
        const cf c = u[i], o = smem[(N - k) & (N - 1)];
        u[i] = make_float2(fmaf(A.x, c.x, fmaf(-A.y, c.y, fmaf(Bq.x, o.y, -Bq.y * o.x))),
                           fmaf(A.x, c.y, fmaf(A.y, c.x, fmaf(Bq.x, o.x, Bq.y * o.y))));
      }
      xlane::fft2048<true>(u, smem, j, t1, t2, t3);
      const void* xn = x.p[0];   // uniform select: indexing the argument array would copy it to scratch
#pragma unroll
      for (int q = 1; q < kMaxOrder; ++q) xn = (n == q) ? x.p[q] : xn;
      const bool last = (n == NORD - 1);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        cf z = make_float2(0.f, 0.f);
        if (i < NV) {
          const int t = 2 * (j + i * S);
          const cf xv = ldp(xn, off, t);
          z = make_float2(xv.x * u[i].x, xv.y * u[i].y);
          if (last) {
            if constexpr (EXACT) st_pair_in<IOT>(y, off, t, z);
            else st_pair<IOT, EVEN>(y, off, (int64_t)t, L, z);
          }
        }
        u[i] = z;
      }
    }
  }
}

template <int IOT, bool EVEN, bool EXACT>
static void launch_fwd_xl(const ForwardArgs& a, hipStream_t s) {
  const auto k = k_single_forward_xl<IOT, EVEN, EXACT>;
  int grid = a.n_rows;
#if HYENA_SINGLE_PERSIST
  static const int cap = resident_workgroups(k, 256) & ~7;
  if (cap > 0 && grid > cap) grid = cap;
#endif
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, a.v, a.x, (const cf*)a.spec, a.y, a.B, a.D, a.NORD, (int)a.L,
                     a.spec_stride, a.n_rows);
}

template <int IOT>
static hipError_t launch_fwd_xlane(const ForwardArgs& a, hipStream_t s) {
  if (a.L == 2048) launch_fwd_xl<IOT, true, true>(a, s);
  else if (a.L % 2 == 0) launch_fwd_xl<IOT, true, false>(a, s);
  else launch_fwd_xl<IOT, false, false>(a, s);
  return hipGetLastError();
}

#endif  // HYENA_SINGLE_XLANE

template <int N, int IOT, bool EVEN, bool FULL, bool EXACT>
static void launch_fwd_k(const ForwardArgs& a, hipStream_t s) {
  const auto k = k_single_forward<N, IOT, EVEN, FULL, EXACT>;
  int grid = a.n_rows;
#if HYENA_SINGLE_PERSIST
  // One resident set of workgroups walks all rows (a multiple of 8, so the
  // XCD of virtual workgroup wg is still wg mod 8).
  static const int cap = resident_workgroups(k, SinglePlan<N>::T) & ~7;
  if (cap > 0 && grid > cap) grid = cap;
#endif
  hipLaunchKernelGGL(k, dim3(grid), dim3(SinglePlan<N>::T), 0, s, a.v, a.x, (const cf*)a.spec, a.y, a.B, a.D,
                     a.NORD, (int)a.L, a.spec_stride, a.n_rows);
}

template <int N, int IOT>
static hipError_t launch_fwd(const ForwardArgs& a, hipStream_t s) {
  if (a.circular) launch_fwd_k<N, IOT, true, true, false>(a, s);   // L = 2N, even
  else if (a.L == N) launch_fwd_k<N, IOT, true, false, true>(a, s);
  else if (a.L % 2 == 0) launch_fwd_k<N, IOT, true, false, false>(a, s);
  else launch_fwd_k<N, IOT, false, false, false>(a, s);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_spec(const SpectrumArgs& a, hipStream_t s) {
  const dim3 grid(a.NF), block(SinglePlan<N>::T);
  if (a.circular)
    hipLaunchKernelGGL((k_single_spectrum<N, true, true>), grid, block, 0, s, a.h, (cf*)a.spec, (int)a.L,
                       a.spec_stride);
  else if (a.L % 2 == 0)
    hipLaunchKernelGGL((k_single_spectrum<N, true, false>), grid, block, 0, s, a.h, (cf*)a.spec, (int)a.L,
                       a.spec_stride);
  else
    hipLaunchKernelGGL((k_single_spectrum<N, false, false>), grid, block, 0, s, a.h, (cf*)a.spec, (int)a.L,
                       a.spec_stride);
  return hipGetLastError();
}

hipError_t single_forward(const ForwardArgs& a, int64_t N, hipStream_t s) {
#if HYENA_SINGLE_XLANE
  if (N == 2048 && !a.circular) return a.io == 0 ? launch_fwd_xlane<0>(a, s) : launch_fwd_xlane<1>(a, s);
#endif
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

hipError_t single_backward(const BackwardArgs& a, int64_t N, hipStream_t s) {
#define HY_CASE(NN)                                                       \
  case NN:                                                                \
    return a.io == 0 ? launch_bwd<NN, 0>(a, s) : launch_bwd<NN, 1>(a, s);
  switch (N) {
    HY_CASE(64) HY_CASE(128) HY_CASE(256) HY_CASE(512) HY_CASE(1024) HY_CASE(2048)
    HY_CASE(4096) HY_CASE(8192)
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
