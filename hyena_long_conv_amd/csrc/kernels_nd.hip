// kernels_nd.hip -- the order-N recurrence with convolutions on 2-D and 3-D
// grids (the gist.science HyenaND summary, "手法: HyenaND": native N-D
// convolution through the N-D FFT; boundary handling, circular for periodic
// systems and every axis zero-padded to twice its size otherwise; section
// "実装: nSubQ": forward FFT, spectral product and inverse FFT fused, the
// intermediate kept on chip).
//
// One workgroup owns one grid (b, d) for all N orders, as on the 1-D
// single-pass path.  The padded real grid P^(k-1) x P (a power-of-two cube,
// every side >= 2L-1 or, circular, = L) travels as a complex grid whose last
// axis is packed in even/odd pairs: c[.., m] = x[.., 2m] + i x[.., 2m+1], so
// NC = P^k / 2 complex points, held E per thread in registers.
//
// The k-dimensional DFT runs as one Stockham pass over the flattened index
// (row-major, first axis slowest) whose stages are grouped by axis: the
// stages of the first (slowest) axis come first, and every later stage
// drops the cross-axis part of the usual twiddle, keeping only the power of
// W over its own axis.  The result lands with the axes reversed (first axis
// fastest); the inverse pass is planned over that reversed layout and
// returns the original one, so a forward/inverse pair needs no transposes.
#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {
namespace {

#ifndef HYENA_ND_E16_MIN
#define HYENA_ND_E16_MIN 16384      // circular grids
#endif
#ifndef HYENA_ND_E16_MIN_PAD
#define HYENA_ND_E16_MIN_PAD 8192   // zero-padded grids
#endif
#ifndef HYENA_ND_SW
#define HYENA_ND_SW 1
#endif

// --------------------------------------------------------------- plans

template <int... Bs> struct Bounds {};   // flattened sizes at which an axis ends

// The product of the axes completed by the stages before NS points (1 if none).
template <int... Bs>
__host__ __device__ constexpr int axis_base(Bounds<Bs...>, int ns) {
  const int bs[] = {0, Bs...};
  int a = 1;
  for (int i = 1; i < (int)(sizeof(bs) / sizeof(int)); ++i)
    if (bs[i] <= ns) a = bs[i];
  return a;
}

template <class A, class B> struct RadCat;
template <int... X, int... Y> struct RadCat<Radices<X...>, Radices<Y...>> {
  using type = Radices<X..., Y...>;
};

// Radices of one axis of length A (a power of two): the leftover radix
// first (its stage opens the axis and needs no twiddle), then radix E.
template <int A, int E, bool LEAD = true> struct AxisRad {
  static constexpr int lg = ilog2(A), le = ilog2(E);
  static constexpr int r = (A <= E) ? A : ((LEAD && lg % le != 0) ? (1 << (lg % le)) : E);
  using type = typename RadCat<Radices<r>, typename AxisRad<A / r, E, false>::type>::type;
};
template <int E, bool LEAD> struct AxisRad<1, E, LEAD> { using type = Radices<>; };

template <int NDIM, int P, bool CIRC> struct NdPlan {
  static_assert(NDIM == 2 || NDIM == 3, "2-D or 3-D grids");
  static constexpr int NL = P / 2;                        // packed last axis
  static constexpr int Q = (NDIM == 2) ? P : P * P;       // points over the other axes
  static constexpr int NC = Q * NL;
  // 16 points per thread from HYENA_ND_E16_MIN(_PAD) complex points on (fewer
  // stages; measured faster on zero-padded 8192-point grids, where half of
  // every thread's points are padding), 8 below
  static constexpr int E = NC >= (CIRC ? HYENA_ND_E16_MIN : HYENA_ND_E16_MIN_PAD) ? 16 : 8;
  static constexpr int T = NC / E;
  static constexpr int S = NC / E;
  static constexpr int LQ = ilog2(Q), LNL = ilog2(NL), LP = ilog2(P);
  using RP = typename AxisRad<P, E>::type;
  using RN = typename AxisRad<NL, E>::type;
  using RF = typename std::conditional<NDIM == 2, typename RadCat<RP, RN>::type,
                                       typename RadCat<typename RadCat<RP, RP>::type, RN>::type>::type;
  using RI = typename std::conditional<NDIM == 2, typename RadCat<RN, RP>::type,
                                       typename RadCat<typename RadCat<RN, RP>::type, RP>::type>::type;
  using BF = typename std::conditional<NDIM == 2, Bounds<P>, Bounds<P, P * P>>::type;
  using BI = typename std::conditional<NDIM == 2, Bounds<NL>, Bounds<NL, NL * P>>::type;
  using Lds = RowLdsT<HYENA_ND_SW != 0>;
};

// --------------------------------------------------------------- the FFT

template <int E, class Bnd, int NS, int R, int... Rest>
constexpr int nd_tw_count() {
  constexpr int c = (axis_base(Bnd{}, NS) == NS) ? 0 : E / R;
  if constexpr (sizeof...(Rest) > 0) return c + nd_tw_count<E, Bnd, NS * R, Rest...>();
  else return c;
}

template <int NPT, int E, class Bnd, int NS, int OFF, int R, int... Rest>
__device__ __forceinline__ void nd_tw_init(cf* tw, int j) {
  constexpr int A = axis_base(Bnd{}, NS);
  constexpr int BPT = E / R;
  if constexpr (A != NS) {
#pragma unroll
    for (int m = 0; m < BPT; ++m) {
      const uint32_t beta = (uint32_t)j + (uint32_t)m * (NPT / E);
      tw[OFF + m] = twiddle<false>((beta & (NS - 1)) / A, (uint32_t)(R * NS / A));
    }
  }
  if constexpr (sizeof...(Rest) > 0) nd_tw_init<NPT, E, Bnd, NS * R, OFF + (A != NS ? BPT : 0), Rest...>(tw, j);
}

template <int NPT, int E, bool INV, class Bnd, int NS, int OFF, int SHPREV, class Lds, int R, int... Rest>
__device__ __forceinline__ void nd_fft_tail(cf (&u)[E], const Lds& lds, int j, const cf* tw) {
  constexpr int A = axis_base(Bnd{}, NS);
  stage_load<NPT, E, R, SHPREV>(u, lds, j);
  if constexpr (A == NS) stage_first<E, R, INV>(u);      // first stage of an axis
  else stage_twiddled<E, R, INV>(u, tw + OFF);
  if constexpr (sizeof...(Rest) > 0) {
    __syncthreads();
    stage_store<NPT, E, R, NS>(u, lds, j);
    __syncthreads();
    nd_fft_tail<NPT, E, INV, Bnd, NS * R, OFF + (A != NS ? E / R : 0), swz_key(R, NS), Lds, Rest...>(u, lds, j,
                                                                                                     tw);
  }
}

template <int NPT, int E, class Rad, class Bnd> struct NdFFT;

// Same register layout contract as BlockFFT: point (or bin) j + i*NPT/E in
// reg[i] on entry and exit; every thread calls run(); callers put a barrier
// before their next LDS write.
template <int NPT, int E, int R0, int... Rs, class Bnd>
struct NdFFT<NPT, E, Radices<R0, Rs...>, Bnd> {
  static_assert(sizeof...(Rs) > 0, "at least two stages");
  static constexpr int NTW = nd_tw_count<E, Bnd, R0, Rs...>();
  cf tw[NTW > 0 ? NTW : 1];

  __device__ __forceinline__ void init(int j) { nd_tw_init<NPT, E, Bnd, R0, 0, Rs...>(tw, j); }

  template <bool INV, class Lds>
  __device__ __forceinline__ void run(cf (&u)[E], const Lds& lds, int j) const {
    stage_first<E, R0, INV>(u);
    __syncthreads();
    stage_store<NPT, E, R0, 1>(u, lds, j);
    __syncthreads();
    nd_fft_tail<NPT, E, INV, Bnd, R0, 0, swz_key(R0, 1), Lds, Rs...>(u, lds, j, tw);
  }
};

// --------------------------------------------------------------- indexing

// Bin k of the reversed layout: a = k mod Q over the other axes (first axis
// fastest), p = k / Q on the packed axis.  The Hermitian partner negates
// every axis index.
template <int NDIM, int P>
__device__ __forceinline__ int nd_neg_other(int a) {
  if constexpr (NDIM == 2) {
    return (P - a) & (P - 1);
  } else {
    const int a1 = a & (P - 1), a2 = a >> ilog2(P);
    return ((P - a1) & (P - 1)) + P * ((P - a2) & (P - 1));
  }
}

// Grid point t of the original layout (first axis slowest, packed axis
// fastest): its offset inside the grid (elements) and its first real index
// on the last axis; false if it lies in the padding.  Grids hold at most
// 2^24 points, so the offset fits 32 bits.
template <int NDIM, int P>
__device__ __forceinline__ bool nd_point(int t, int Lo, int Lm, int Ll, int& off, int& tl) {
  using PL = NdPlan<NDIM, P, false>;
  const int m = t & (PL::NL - 1);
  const int rest = t >> PL::LNL;
  const int n2 = (NDIM == 3) ? (rest & (P - 1)) : 0;
  const int n1 = (NDIM == 3) ? (rest >> PL::LP) : rest;
  off = (n1 * Lm + n2) * Ll;
  tl = 2 * m;
  return n1 < Lo && n2 < Lm && tl < Ll;
}

// A value the compiler must not treat as loop-invariant: per-order index
// arithmetic is cheaper to redo than to keep E copies live across orders.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int IOT>
__device__ __forceinline__ const void* advance(const void* p, int64_t n) {
  return IOT == 0 ? (const void*)(static_cast<const float*>(p) + n) : (const void*)(static_cast<const uint16_t*>(p) + n);
}
template <int IOT>
__device__ __forceinline__ void* advance(void* p, int64_t n) {
  return IOT == 0 ? (void*)(static_cast<float*>(p) + n) : (void*)(static_cast<uint16_t*>(p) + n);
}

// --------------------------------------------------------------- kernels

// Spectrum of one kernel row f: the real k-D DFT H/M (M = 2 NC) of the
// kernel placed on the padded grid (offset o at o mod P on every axis),
// stored in the reversed layout: bins k < NC, then the plane p = NL of the
// packed axis (Q values) that the Hermitian pairing of p = 0 refers to.
template <int NDIM, int P, bool CIRC>
__global__ void __launch_bounds__((NdPlan<NDIM, P, CIRC>::T))
k_nd_spectrum(const float* __restrict__ K, cf* __restrict__ spec, int Lo, int Lm, int Ll, int64_t spec_stride) {
  using PL = NdPlan<NDIM, P, CIRC>;
  constexpr int E = PL::E, S = PL::S, NC = PL::NC, NL = PL::NL, Q = PL::Q;
  __shared__ cf smem[NC];
  const typename PL::Lds lds{smem};
  const int j = threadIdx.x;
  const int eo = CIRC ? Lo : 2 * Lo - 1, em = CIRC ? Lm : (NDIM == 3 ? 2 * Lm - 1 : 1), el = CIRC ? Ll : 2 * Ll - 1;
  const float* kr = K + (int64_t)blockIdx.x * eo * em * el;
  // kernel index of padded-grid position n on an axis of side L (-1: gap)
  const auto kidx = [](int n, int L) { return CIRC ? n : (n < L ? n + L - 1 : (n > P - L ? n - P + L - 1 : -1)); };
  NdFFT<NC, E, typename PL::RF, typename PL::BF> ff;
  ff.init(j);
  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int t = j + i * S;
    const int m = t & (NL - 1), rest = t >> PL::LNL;
    const int n2 = (NDIM == 3) ? (rest & (P - 1)) : 0;
    const int n1 = (NDIM == 3) ? (rest >> PL::LP) : rest;
    const int i1 = kidx(n1, Lo), i2 = (NDIM == 3) ? kidx(n2, Lm) : 0;
    const int i3a = kidx(2 * m, Ll), i3b = kidx(2 * m + 1, Ll);
    const bool ok = i1 >= 0 && i2 >= 0;
    const int64_t rb = ((int64_t)i1 * em + i2) * el;
    u[i] = make_float2((ok && i3a >= 0) ? kr[rb + i3a] : 0.f, (ok && i3b >= 0) ? kr[rb + i3b] : 0.f);
  }
  ff.template run<false>(u, lds, j);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) lds(j + i * S) = u[i];
  __syncthreads();
  const float sc = 1.0f / (float)(2 * NC);
  cf* out = spec + (int64_t)blockIdx.x * spec_stride;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int k = j + i * S;
    const int a = k & (Q - 1), p = k >> PL::LQ;
    const int na = nd_neg_other<NDIM, P>(a);
    const cf cm = lds(na + Q * ((NL - p) & (NL - 1)));
    float sn, cs;
    sincospif((float)p / (float)NL, &sn, &cs);
    out[k] = realfft_bin(u[i], cm, make_float2(cs, -sn), sc);
    if (p == 0) out[NC + a] = realfft_bin(u[i], cm, make_float2(-1.f, 0.f), sc);
  }
}

// The recurrence on one grid (b, d).  Per order: forward k-D FFT, the
// spectral step, inverse k-D FFT, gate.  Spectral step per bin k with data
// partner k' and filter values G = H(k)/M, G'' = H(k'')/M (k'' the filter's
// Hermitian partner, p = 0 pairing with the plane p = NL):
//   C'(k) = A C(k) + i B conj C(k'),  A = Pg - s Qg,  B = c Qg,
//   Pg = G + conj G'',  Qg = G - conj G'',  (s, c) = (sin, cos)(pi p / NL)
// -- the per-bin form of the 1-D pair step (real-FFT untangling, product
// with H and re-packing folded into one linear map).
template <int NDIM, int P, int IOT, bool CIRC, bool EVEN>
__global__ void __launch_bounds__((NdPlan<NDIM, P, CIRC>::T))
k_nd_forward(const void* __restrict__ v, XPtrs x, const cf* __restrict__ spec, void* __restrict__ y, int D,
             int NORD, int Lo, int Lm, int Ll, int per_sample, int64_t spec_stride) {
  using PL = NdPlan<NDIM, P, CIRC>;
  constexpr int E = PL::E, S = PL::S, NC = PL::NC, NL = PL::NL, Q = PL::Q;
  // bins whose filter values are loaded together (bounds the registers
  // they hold while the partner exchange runs)
  constexpr int CH = E > 8 ? 4 : E;
  // Non-circular grids fill less than half of the first (slowest) axis, so
  // the points of registers i >= E/2 are padding on every order.
  constexpr int NV = CIRC ? E : E / 2;
  __shared__ cf smem[NC];
  __shared__ float2 tws[NL];
  const typename PL::Lds lds{smem};
  const int j = threadIdx.x;
  const int row = blockIdx.x, b = row / D, d = row - b * D;
  const int64_t gbase = (int64_t)row * Lo * Lm * Ll;
  const void* vg = advance<IOT>(v, gbase);
  void* yg = advance<IOT>(y, gbase);
  for (int p = j; p < NL; p += PL::T) {
    float sn, cs;
    sincospif((float)p / (float)NL, &sn, &cs);
    tws[p] = make_float2(sn, cs);
  }
  NdFFT<NC, E, typename PL::RF, typename PL::BF> ff;
  NdFFT<NC, E, typename PL::RI, typename PL::BI> fi;
  ff.init(j);
  fi.init(j);
  cf u[E];
  // Loads run unconditionally: points outside the grid (zero padding) read
  // the grid's first pair and are masked afterwards.  A branch around a load
  // whose value is converted inside it makes the wave wait for each load
  // before issuing the next.
#pragma unroll
  for (int i = 0; i < E; ++i) {
    int off, tl;
    const bool ok = CIRC || nd_point<NDIM, P>(j + i * S, Lo, Lm, Ll, off, tl);
    if constexpr (CIRC) nd_point<NDIM, P>(j + i * S, Lo, Lm, Ll, off, tl);
    if (i < NV) {
      const cf w = ld_pair<IOT, EVEN, true>(vg, ok ? off : 0, ok ? tl : 0, Ll);
      u[i] = ok ? w : make_float2(0.f, 0.f);
    } else {
      u[i] = make_float2(0.f, 0.f);
    }
  }
  for (int n = 0; n < NORD; ++n) {
    const int jj = fresh(j);
    const int f = per_sample ? ((b * NORD + n) * D + d) : (n * D + d);
    const cf* hs = spec + (int64_t)f * spec_stride;
    ff.template run<false>(u, lds, jj);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E; ++i) lds(jj + i * S) = u[i];
    __syncthreads();
#pragma unroll
    for (int i0 = 0; i0 < E; i0 += CH) {
      const int jc = (CH < E) ? fresh(jj) : jj;
      cf g[CH], gm[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int k = jc + (i0 + c) * S;
        const int a = k & (Q - 1), p = k >> PL::LQ;
        g[c] = hs[k];
        gm[c] = hs[nd_neg_other<NDIM, P>(a) + Q * (NL - p)];
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int i = i0 + c;
        const int k = jc + i * S;
        const int a = k & (Q - 1), p = k >> PL::LQ;
        const cf cm = lds(nd_neg_other<NDIM, P>(a) + Q * ((NL - p) & (NL - 1)));
        const float2 w = tws[p];
        const cf Pg = make_float2(g[c].x + gm[c].x, g[c].y - gm[c].y);
        const cf Qg = make_float2(g[c].x - gm[c].x, g[c].y + gm[c].y);
        const cf A = make_float2(fmaf(-w.x, Qg.x, Pg.x), fmaf(-w.x, Qg.y, Pg.y));
        const cf Bc = make_float2(w.y * Qg.x, w.y * Qg.y);
        const cf z = u[i];
        u[i] = make_float2(fmaf(A.x, z.x, fmaf(-A.y, z.y, fmaf(Bc.x, cm.y, -Bc.y * cm.x))),
                           fmaf(A.x, z.y, fmaf(A.y, z.x, fmaf(Bc.x, cm.x, Bc.y * cm.y))));
      }
    }
    fi.template run<true>(u, lds, jj);
    const void* xg = advance<IOT>(x.p[n], gbase);
    const bool last = (n == NORD - 1);
    const int jg = fresh(jj);
    // gates requested in batches of 8 and pinned (not sunk into the stores'
    // masks; the fence keeps the next batch's loads after the pins)
    constexpr int GB = NV < 8 ? NV : 8;
#pragma unroll
    for (int i0 = 0; i0 < E; i0 += GB) {
      RawPair<IOT> xr[GB];
      if (i0 < NV) {
#pragma unroll
        for (int c = 0; c < GB; ++c) {
          int off, tl;
          const bool ok = nd_point<NDIM, P>(jg + (i0 + c) * S, Lo, Lm, Ll, off, tl) || CIRC;
          xr[c] = ld_pair_raw<IOT, EVEN>(xg, ok ? off : 0, ok ? tl : 0, Ll);
        }
#pragma unroll
        for (int c = 0; c < GB; ++c) pin<IOT, true>(xr[c]);
      }
#pragma unroll
      for (int c = 0; c < GB; ++c) {
        const int i = i0 + c;
        int off, tl;
        const bool ok = nd_point<NDIM, P>(jg + i * S, Lo, Lm, Ll, off, tl) || CIRC;
        cf z = make_float2(0.f, 0.f);
        if (i < NV && ok) {
          const cf xv = unpack(xr[c]);
          z = make_float2(xv.x * u[i].x, xv.y * u[i].y);
          if (last) st_pair<IOT, EVEN>(yg, off, tl, Ll, z);
        }
        u[i] = z;
      }
    }
  }
}

// Plane pass of the 3-D multi-pass grids: after the column pass over the
// first axis, plane k1 of a grid is a P x P/2 complex array (rows i2, packed
// columns m).  A workgroup takes planes k1 and P-k1 (each bin's Hermitian
// partner (-k1, -k2, -k3) lies in the mirror plane; planes 0 and P/2 are
// their own mirrors and go together), runs the 2-D FFT of each (the grid
// FFT above, two axes), the per-bin spectral step, and the inverse 2-D FFT.
// Spectrum layout: H/M of plane k1 at k1*NCp + k (k in the plane FFT's
// reversed layout), then the packed axis' Nyquist plane at NC + k1*P + a.
struct PlaneArgs {
  cf* work;
  const cf* spec;
  cf* spec_out;
  int64_t spec_stride;
  int order, NORD, D, per_sample, r0;
};

template <int P, bool SPEC>
__global__ void __launch_bounds__((2 * NdPlan<2, P, false>::T)) k_grid_plane(PlaneArgs a) {
  using PL = NdPlan<2, P, false>;
  constexpr int E = PL::E, S = PL::S, NCP = PL::NC, NL = PL::NL, T = PL::T;
  constexpr int64_t NC = (int64_t)P * NCP;
  __shared__ cf smem[2 * NCP];
  __shared__ float2 tws[NL];
  const int b = threadIdx.x / T, j = threadIdx.x - b * T;
  const int w = blockIdx.x % (P / 2), g = blockIdx.x / (P / 2);
  const int k1 = (b == 0) ? w : (w == 0 ? P / 2 : P - w);
  const bool self_mirror = (k1 == 0) || (2 * k1 == P);
  const int mb = self_mirror ? b : 1 - b;
  const int k1m = (P - k1) & (P - 1);
  const typename PL::Lds lds{smem + b * NCP}, ldsm{smem + mb * NCP};
  cf* plane = a.work + (int64_t)g * NC + (int64_t)k1 * NCP;
  for (int p = threadIdx.x; p < NL; p += 2 * T) {
    float sn, cs;
    sincospif((float)p / (float)NL, &sn, &cs);
    tws[p] = make_float2(sn, cs);
  }
  NdFFT<NCP, E, typename PL::RF, typename PL::BF> ff;
  ff.init(j);
  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i) u[i] = plane[j + i * S];
  ff.template run<false>(u, lds, j);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) lds(j + i * S) = u[i];
  __syncthreads();
  const float sc = 1.0f / (float)(2 * NC);
  if constexpr (SPEC) {
    cf* out = a.spec_out + (int64_t)(a.r0 + g) * a.spec_stride;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k = j + i * S;
      const int ka = k & (P - 1), p = k >> PL::LQ;
      const int na = nd_neg_other<2, P>(ka);
      const cf cm = ldsm(na + P * ((NL - p) & (NL - 1)));
      const float2 t = tws[p];
      out[(int64_t)k1 * NCP + k] = realfft_bin(u[i], cm, make_float2(t.y, -t.x), sc);
      if (p == 0) out[NC + (int64_t)k1 * P + ka] = realfft_bin(u[i], cm, make_float2(-1.f, 0.f), sc);
    }
  } else {
    const int rowid = a.r0 + g, bb = rowid / a.D, d = rowid - bb * a.D;
    const int64_t f = a.per_sample ? ((int64_t)bb * a.NORD + a.order) * a.D + d : (int64_t)a.order * a.D + d;
    const cf* gs = a.spec + f * a.spec_stride;
    constexpr int CH = E > 8 ? 4 : E;       // bins whose filter values are in flight together
#pragma unroll
    for (int i0 = 0; i0 < E; i0 += CH) {
      const int jc = (CH < E) ? fresh(j) : j;
      cf G[CH], Gm[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int k = jc + (i0 + c) * S;
        const int ka = k & (P - 1), p = k >> PL::LQ;
        const int na = nd_neg_other<2, P>(ka);
        G[c] = gs[(int64_t)k1 * NCP + k];
        Gm[c] = (p == 0) ? gs[NC + (int64_t)k1m * P + na] : gs[(int64_t)k1m * NCP + na + P * (NL - p)];
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int i = i0 + c, k = jc + i * S;
        const int ka = k & (P - 1), p = k >> PL::LQ;
        const cf cm = ldsm(nd_neg_other<2, P>(ka) + P * ((NL - p) & (NL - 1)));
        const float2 t = tws[p];
        const cf Pg = make_float2(G[c].x + Gm[c].x, G[c].y - Gm[c].y);
        const cf Qg = make_float2(G[c].x - Gm[c].x, G[c].y + Gm[c].y);
        const cf A = make_float2(fmaf(-t.x, Qg.x, Pg.x), fmaf(-t.x, Qg.y, Pg.y));
        const cf Bc = make_float2(t.y * Qg.x, t.y * Qg.y);
        const cf z = u[i];
        u[i] = make_float2(fmaf(A.x, z.x, fmaf(-A.y, z.y, fmaf(Bc.x, cm.y, -Bc.y * cm.x))),
                           fmaf(A.x, z.y, fmaf(A.y, z.x, fmaf(Bc.x, cm.x, Bc.y * cm.y))));
      }
    }
    // the inverse's twiddles are made here, so they are not live during the step above
    NdFFT<NCP, E, typename PL::RI, typename PL::BI> fi;
    fi.init(fresh(j));
    fi.template run<true>(u, lds, j);
#pragma unroll
    for (int i = 0; i < E; ++i) plane[j + i * S] = u[i];
  }
}

template <int P>
hipError_t launch_grid_plane(const NdArgs& a, int r0, int groups, int n, bool spec, hipStream_t s) {
  PlaneArgs pa{};
  pa.work = (cf*)a.work;
  pa.spec = (const cf*)a.spec;
  pa.spec_out = (cf*)a.spec;
  pa.spec_stride = a.spec_stride;
  pa.order = n; pa.NORD = a.NORD; pa.D = a.D; pa.per_sample = a.per_sample; pa.r0 = r0;
  const dim3 grid((unsigned)(groups * (P / 2))), block(2 * NdPlan<2, P, false>::T);
  if (spec) hipLaunchKernelGGL((k_grid_plane<P, true>), grid, block, 0, s, pa);
  else hipLaunchKernelGGL((k_grid_plane<P, false>), grid, block, 0, s, pa);
  return hipGetLastError();
}

template <int NDIM, int P>
hipError_t launch_nd_spectrum(const NdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.rows);
  const dim3 block(a.circular ? NdPlan<NDIM, P, true>::T : NdPlan<NDIM, P, false>::T);
  if (a.circular)
    hipLaunchKernelGGL((k_nd_spectrum<NDIM, P, true>), grid, block, 0, s, a.kernel, (cf*)a.spec, a.Lo, a.Lm, a.Ll,
                       a.spec_stride);
  else
    hipLaunchKernelGGL((k_nd_spectrum<NDIM, P, false>), grid, block, 0, s, a.kernel, (cf*)a.spec, a.Lo, a.Lm, a.Ll,
                       a.spec_stride);
  return hipGetLastError();
}

template <int NDIM, int P, int IOT>
hipError_t launch_nd_forward_io(const NdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.rows);
  const dim3 block(a.circular ? NdPlan<NDIM, P, true>::T : NdPlan<NDIM, P, false>::T);
  const cf* sp = (const cf*)a.spec;
  if (a.circular)
    hipLaunchKernelGGL((k_nd_forward<NDIM, P, IOT, true, true>), grid, block, 0, s, a.v, a.x, sp, a.y, a.D, a.NORD,
                       a.Lo, a.Lm, a.Ll, a.per_sample, a.spec_stride);
  else if ((a.Ll & 1) == 0)
    hipLaunchKernelGGL((k_nd_forward<NDIM, P, IOT, false, true>), grid, block, 0, s, a.v, a.x, sp, a.y, a.D,
                       a.NORD, a.Lo, a.Lm, a.Ll, a.per_sample, a.spec_stride);
  else
    hipLaunchKernelGGL((k_nd_forward<NDIM, P, IOT, false, false>), grid, block, 0, s, a.v, a.x, sp, a.y, a.D,
                       a.NORD, a.Lo, a.Lm, a.Ll, a.per_sample, a.spec_stride);
  return hipGetLastError();
}

template <int NDIM, int P>
hipError_t launch_nd_forward(const NdArgs& a, hipStream_t s) {
  return a.io == 0 ? launch_nd_forward_io<NDIM, P, 0>(a, s) : launch_nd_forward_io<NDIM, P, 1>(a, s);
}

}  // namespace

hipError_t nd_spectrum(const NdArgs& a, hipStream_t s) {
  if (a.ndim == 2) {
    switch (a.P) {
      case 16: return launch_nd_spectrum<2, 16>(a, s);
      case 32: return launch_nd_spectrum<2, 32>(a, s);
      case 64: return launch_nd_spectrum<2, 64>(a, s);
      case 128: return launch_nd_spectrum<2, 128>(a, s);
    }
  } else if (a.ndim == 3) {
    switch (a.P) {
      case 8: return launch_nd_spectrum<3, 8>(a, s);
      case 16: return launch_nd_spectrum<3, 16>(a, s);
      case 32: return launch_nd_spectrum<3, 32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t nd_forward(const NdArgs& a, hipStream_t s) {
  if (a.ndim == 2) {
    switch (a.P) {
      case 16: return launch_nd_forward<2, 16>(a, s);
      case 32: return launch_nd_forward<2, 32>(a, s);
      case 64: return launch_nd_forward<2, 64>(a, s);
      case 128: return launch_nd_forward<2, 128>(a, s);
    }
  } else if (a.ndim == 3) {
    switch (a.P) {
      case 8: return launch_nd_forward<3, 8>(a, s);
      case 16: return launch_nd_forward<3, 16>(a, s);
      case 32: return launch_nd_forward<3, 32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t grid_plane_pass(const NdArgs& a, int r0, int groups, int n, bool spec, hipStream_t s) {
  switch (a.P) {
    case 64: return launch_grid_plane<64>(a, r0, groups, n, spec, s);
    case 128: return launch_grid_plane<128>(a, r0, groups, n, spec, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hyena
