// fft_engine.hpp -- workgroup-level complex FFT building blocks for gfx950.
//
// A workgroup computes one or more complex FFTs of NPT points.  Each thread
// owns E = (a multiple of every radix used) points in registers.  Stages are
// Stockham autosort (decimation in time, twiddle on the inputs): a radix-R
// stage that follows stages of total size NS reads leg r of butterfly beta
// from index beta + r*NPT/R, multiplies it by W_{R*NS}^{(beta mod NS)*r},
// applies an R-point DFT and writes output q to (beta/NS)*NS*R + beta mod NS
// + q*NS.  The output comes out in natural order with no bit reversal.
//
// Thread j handles butterflies beta = j + m*(NPT/E), m < E/R.  With that
// assignment the thread's register set is {j + i*(NPT/E) : i < E} both at the
// input of the first stage and at the output of the last stage, for any
// radix sequence.  Consequences used throughout the kernels:
//   * a forward FFT leaves bin k = j + i*NPT/E in reg[i];
//   * an inverse FFT started from those registers needs no data exchange and
//     leaves time sample t = j + i*NPT/E in reg[i];
//   * the next forward FFT starts from those same registers.
// Only the stages in between go through LDS.
//
// The math is the textbook Cooley-Tukey factorisation of the DFT; the
// Stockham ordering avoids a separate bit-reversal pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "plan.hpp"

namespace hyena {

typedef float2 cf;
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ cf cadd(cf a, cf b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ cf csub(cf a, cf b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ cf cscale(cf a, float s) { return make_float2(a.x * s, a.y * s); }
__device__ __forceinline__ cf cconj(cf a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ cf cmul(cf a, cf b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
// a * conj(b)
__device__ __forceinline__ cf cmulc(cf a, cf b) {
  return make_float2(fmaf(a.x, b.x, a.y * b.y), fmaf(a.y, b.x, -a.x * b.y));
}

// Multiply by -i (forward transform) or +i (inverse transform).
template <bool INV>
__device__ __forceinline__ cf rot90(cf a) {
  return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// exp(-2 pi i k / n) (forward) or its conjugate (inverse), for k, n < 2^24.
// The angle is k/n turns.  Its nearest quarter turn q is taken out in exact
// integer arithmetic (4k - q n fits a float exactly), leaving r = (4k - q n)
// / 4n turns with |r| <= 1/8, i.e. |2 pi r| <= pi/4; cos and sin of 2 pi r
// come from their Taylor series about 0 through the r^10 and r^9 terms
// (truncation error below 2e-9 on that range), and the result is rotated by
// q quarter turns.  Absolute error about 1.5 x 2^-24 for power-of-two n and
// 2 x 2^-24 otherwise (checked on the CPU against double precision for n up
// to 2^22); half the instructions of a general sincos, and no division:
// 1/n is a reciprocal refined by one Newton step, folded when n is a
// compile-time constant.
template <bool INV>
__device__ __forceinline__ cf twiddle(uint32_t k, uint32_t n) {
  const float fk4 = 4.0f * (float)k, fn = (float)n;
  const float rn0 = __builtin_amdgcn_rcpf(fn);
  const float rn = fmaf(fmaf(-fn, rn0, 1.0f), rn0, rn0);
  const float q = __builtin_rintf(fk4 * rn);
  const float r = fmaf(-q, fn, fk4) * (0.25f * rn);
  const float r2 = r * r;
  // (2 pi)^j / j! with alternating signs: sin(2 pi r) = r * S(r^2), cos = C(r^2)
  float sp = fmaf(r2, 42.058693944897634f, -76.70585975306136f);
  sp = fmaf(r2, sp, 81.60524927607504f);
  sp = fmaf(r2, sp, -41.341702240399755f);
  sp = fmaf(r2, sp, 6.283185307179586f);
  const float sr = r * sp;
  float cp = fmaf(r2, -26.426256783374388f, 60.24464137187664f);
  cp = fmaf(r2, cp, -85.45681720669371f);
  cp = fmaf(r2, cp, 64.93939402266828f);
  cp = fmaf(r2, cp, -19.739208802178716f);
  const float cr = fmaf(r2, cp, 1.0f);
  // rotation by q quarter turns: (c, s) -> (-s, c) per quarter
  const uint32_t qi = (uint32_t)(int)q;
  const bool odd = (qi & 1u) != 0;
  const float c = __uint_as_float(__float_as_uint(odd ? sr : cr) ^ (((qi + 1u) & 2u) << 30));
  const float s = __uint_as_float(__float_as_uint(odd ? cr : sr) ^ ((qi & 2u) << 30));
  return INV ? make_float2(c, s) : make_float2(c, -s);
}

// ---------------------------------------------------------------- small DFTs

template <bool INV>
__device__ __forceinline__ void dft2(cf& a0, cf& a1) {
  cf t = a0;
  a0 = cadd(t, a1);
  a1 = csub(t, a1);
}

template <bool INV>
__device__ __forceinline__ void dft4(cf& a0, cf& a1, cf& a2, cf& a3) {
  cf t0 = cadd(a0, a2), t1 = csub(a0, a2);
  cf t2 = cadd(a1, a3), t3 = rot90<INV>(csub(a1, a3));
  a0 = cadd(t0, t2);
  a2 = csub(t0, t2);
  a1 = cadd(t1, t3);
  a3 = csub(t1, t3);
}

// times exp(-+ i pi / 4)
template <bool INV>
__device__ __forceinline__ cf mul_w8(cf a) {
  const float r = 0.70710678118654752440f;
  return INV ? make_float2((a.x - a.y) * r, (a.x + a.y) * r)
             : make_float2((a.x + a.y) * r, (a.y - a.x) * r);
}

template <bool INV>
__device__ __forceinline__ void dft8(cf* a) {
  // even / odd halves, then combine with W8^k
  cf e0 = a[0], e1 = a[2], e2 = a[4], e3 = a[6];
  cf o0 = a[1], o1 = a[3], o2 = a[5], o3 = a[7];
  dft4<INV>(e0, e1, e2, e3);
  dft4<INV>(o0, o1, o2, o3);
  o1 = mul_w8<INV>(o1);
  o2 = rot90<INV>(o2);
  o3 = rot90<INV>(mul_w8<INV>(o3));
  a[0] = cadd(e0, o0); a[4] = csub(e0, o0);
  a[1] = cadd(e1, o1); a[5] = csub(e1, o1);
  a[2] = cadd(e2, o2); a[6] = csub(e2, o2);
  a[3] = cadd(e3, o3); a[7] = csub(e3, o3);
}

template <bool INV>
__device__ __forceinline__ void dft16(cf* a) {
  // 4 x 4: inner DFT4 over n1 for each n2, twiddle W16^{n2 k1}, outer DFT4.
  const float c1 = 0.92387953251128675613f;  // cos(pi/8)
  const float s1 = 0.38268343236508977173f;  // sin(pi/8)
#pragma unroll
  for (int n2 = 0; n2 < 4; ++n2) dft4<INV>(a[n2], a[n2 + 4], a[n2 + 8], a[n2 + 12]);
  // a[n2 + 4*k1] now holds b[n2][k1]
  const cf w1 = INV ? make_float2(c1, s1) : make_float2(c1, -s1);   // W16^1
  const cf w3 = INV ? make_float2(s1, c1) : make_float2(s1, -c1);   // W16^3
  a[1 + 4 * 1] = cmul(a[1 + 4 * 1], w1);
  a[1 + 4 * 2] = mul_w8<INV>(a[1 + 4 * 2]);
  a[1 + 4 * 3] = cmul(a[1 + 4 * 3], w3);
  a[2 + 4 * 1] = mul_w8<INV>(a[2 + 4 * 1]);
  a[2 + 4 * 2] = rot90<INV>(a[2 + 4 * 2]);
  a[2 + 4 * 3] = rot90<INV>(mul_w8<INV>(a[2 + 4 * 3]));
  a[3 + 4 * 1] = cmul(a[3 + 4 * 1], w3);
  a[3 + 4 * 2] = rot90<INV>(mul_w8<INV>(a[3 + 4 * 2]));
  a[3 + 4 * 3] = cmul(a[3 + 4 * 3], make_float2(-w1.x, -w1.y));     // W16^9 = -W16^1
#pragma unroll
  for (int k1 = 0; k1 < 4; ++k1) dft4<INV>(a[4 * k1 + 0], a[4 * k1 + 1], a[4 * k1 + 2], a[4 * k1 + 3]);
  // a[4*k1 + k2] holds X[k1 + 4*k2]; transpose the 4x4 index into natural order
  cf t[16];
#pragma unroll
  for (int k1 = 0; k1 < 4; ++k1)
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) t[k1 + 4 * k2] = a[4 * k1 + k2];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = t[i];
}

template <int R, bool INV>
__device__ __forceinline__ void dft(cf* a) {
  if constexpr (R == 2) dft2<INV>(a[0], a[1]);
  else if constexpr (R == 4) dft4<INV>(a[0], a[1], a[2], a[3]);
  else if constexpr (R == 8) dft8<INV>(a);
  else if constexpr (R == 16) dft16<INV>(a);
  else static_assert(R == 2, "unsupported radix");
}

// ------------------------------------------------- twiddled DIT butterflies
//
// A Stockham stage after stages of total size NS evaluates, for butterfly
// beta with p = beta mod NS and w = W_{R*NS}^p,
//     X_q = sum_r a_r (w W_R^q)^r,   q = 0..R-1,
// i.e. the polynomial sum_r a_r z^r at the R points w W_R^q.  Splitting r
// into even and odd terms gives X_q = E_q + w W_R^q O_q and
// X_{q+R/2} = E_q - w W_R^q O_q, where E and O are the same problem of size
// R/2 for base w^2.  Each radix-2 step below costs six FMAs; the only
// twiddles needed are powers w^(2^k) (squarings) times the constants W_R^q.

// Hide a value from loop-invariant code motion: derived twiddles are cheaper
// to recompute per use than to keep live across a whole FFT pair.
__device__ __forceinline__ cf opaque(cf w) {
  asm volatile("" : "+v"(w.x), "+v"(w.y));
  return w;
}

__device__ __forceinline__ cf csq(cf w) {
  return make_float2(fmaf(w.x, w.x, -w.y * w.y), 2.0f * w.x * w.y);
}

// (a, b) <- (a + t b, a - t b) with six FMAs.
__device__ __forceinline__ void bfly2(cf& a, cf& b, cf t) {
  const float rx = fmaf(-b.y, t.y, fmaf(b.x, t.x, a.x));
  const float ry = fmaf(b.x, t.y, fmaf(b.y, t.x, a.y));
  b = make_float2(fmaf(2.0f, a.x, -rx), fmaf(2.0f, a.y, -ry));
  a = make_float2(rx, ry);
}

// w * W_R^q (W_R = exp(-2 pi i / R) forward, its conjugate inverse).
template <int R, int Q, bool INV>
__device__ __forceinline__ cf tw_const(cf w) {
  constexpr int q = Q % R;
  if constexpr (q == 0) return w;
  else if constexpr (4 * q == R) return rot90<INV>(w);
  else if constexpr (4 * q > R) return rot90<INV>(tw_const<R, q - R / 4, INV>(w));
  else if constexpr (8 * q == R) return mul_w8<INV>(w);
  else {
    static_assert(R == 16 && (q == 1 || q == 3), "unsupported constant twiddle");
    const float c1 = 0.92387953251128675613f, s1 = 0.38268343236508977173f;
    const cf k = (q == 1) ? make_float2(c1, INV ? s1 : -s1) : make_float2(s1, INV ? c1 : -c1);
    return cmul(w, k);
  }
}

template <int R, bool INV>
struct Dit {
  static __device__ __forceinline__ void run(cf* a, cf w) {
    if constexpr (R == 1) {
      return;
    } else {
      cf e[R / 2], o[R / 2];
#pragma unroll
      for (int r = 0; r < R / 2; ++r) { e[r] = a[2 * r]; o[r] = a[2 * r + 1]; }
      if constexpr (R > 2) {
        const cf w2 = csq(w);
        Dit<R / 2, INV>::run(e, w2);
        Dit<R / 2, INV>::run(o, w2);
      }
      twiddle_combine(e, o, w, std::make_integer_sequence<int, R / 2>{});
#pragma unroll
      for (int q = 0; q < R / 2; ++q) { a[q] = e[q]; a[q + R / 2] = o[q]; }
    }
  }
  template <int... Q>
  static __device__ __forceinline__ void twiddle_combine(cf* e, cf* o, cf w, std::integer_sequence<int, Q...>) {
    (bfly2(e[Q], o[Q], tw_const<R, Q, INV>(w)), ...);
  }
};

// One butterfly of a twiddled stage: a[r] in, X_q out (natural order).
template <int R, bool INV>
__device__ __forceinline__ void bfly_tw(cf* a, cf w) {
  Dit<R, INV>::run(a, INV ? cconj(w) : w);
}

// b * s^i for a compile-time i < E (binary powers of s, CSE'd across i).
template <int E>
__device__ __forceinline__ cf step_power(cf b, cf s, int i) {
  cf p = b, sp = s;
#pragma unroll
  for (int bit = 1; bit < E; bit <<= 1) {
    if (i & bit) p = cmul(p, sp);
    if ((bit << 1) < E) sp = csq(sp);
  }
  return p;
}

// ---------------------------------------------------------------- LDS layouts

// One FFT per row, point index fastest.  The buffer written by a radix-R
// stage (and read by the next one) stores point p at p ^ ((p >> log2 R) & 31):
// the stage's strided writes (stride R at the first stage) then spread over
// all LDS banks, while the next stage's unit-stride reads stay conflict-free.
// (Checked offline for every radix sequence used, against 32-bank/16-lane and
// 64-bank/32-lane models: 1.03x the conflict-free cycle count on average,
// 1.31x worst, against 1.9x for one pad slot per 16 points.)  operator()
// addresses the buffer unswizzled, for the spectral exchanges.  SW = false
// turns the swizzle off (plain addressing needs fewer VALU operations, which
// some lengths value more than the conflicts it removes).
template <bool SW>
struct RowLdsT {
  cf* base;
  static constexpr __host__ __device__ int padded(int npt) { return npt; }
  template <int SH>
  __device__ __forceinline__ cf& at(int i) const {
    if constexpr (SH == 0 || !SW) return base[i];
    else return base[i ^ ((i >> SH) & 31)];
  }
  __device__ __forceinline__ cf& operator()(int i) const { return base[i]; }
};
using RowLds = RowLdsT<false>;

// Many FFTs side by side, FFT instance fastest: element i of instance c sits
// at i*NB + c.  Lanes that differ in c touch consecutive words, so no swizzle.
template <int NB>
struct ColLds {
  cf* base;  // already offset by the instance index c
  template <int SH>
  __device__ __forceinline__ cf& at(int i) const { return base[i * NB]; }
  __device__ __forceinline__ cf& operator()(int i) const { return base[i * NB]; }
};

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// Swizzle key of the buffer a radix-R stage after stages of size NS writes:
// only stores with NS < 32 are strided across lanes; wider ones already write
// runs of >= 32 consecutive points and stay unswizzled (cheaper addressing).
constexpr int swz_key(int R, int NS) { return NS < 32 ? ilog2(R) : 0; }

// ---------------------------------------------------------------- stages

template <int... Rs>
struct Radices {};

// Butterflies of the first stage (NS = 1: no twiddles).  u[m + r*BPT] holds
// leg r of butterfly m on entry and output q at u[m + q*BPT] on exit.
template <int E, int R, bool INV>
__device__ __forceinline__ void stage_first(cf (&u)[E]) {
  constexpr int BPT = E / R;
  static_assert(E % R == 0, "radix must divide the per-thread count");
#pragma unroll
  for (int m = 0; m < BPT; ++m) {
    cf a[R];
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = u[m + r * BPT];
    dft<R, INV>(a);
#pragma unroll
    for (int q = 0; q < R; ++q) u[m + q * BPT] = a[q];
  }
}

template <int E, int R, bool INV>
__device__ __forceinline__ void stage_twiddled(cf (&u)[E], const cf* tw) {
  constexpr int BPT = E / R;
  static_assert(E % R == 0, "radix must divide the per-thread count");
#pragma unroll
  for (int m = 0; m < BPT; ++m) {
    cf a[R];
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = u[m + r * BPT];
    bfly_tw<R, INV>(a, opaque(tw[m]));
#pragma unroll
    for (int q = 0; q < R; ++q) u[m + q * BPT] = a[q];
  }
}

template <int NPT, int E, int R, int NS, class Lds>
__device__ __forceinline__ void stage_store(const cf (&u)[E], const Lds& lds, int j) {
  constexpr int BPT = E / R, SH = swz_key(R, NS);
#pragma unroll
  for (int m = 0; m < BPT; ++m) {
    const int beta = j + m * (NPT / E);
    const int base = (beta / NS) * NS * R + (beta & (NS - 1));
#pragma unroll
    for (int q = 0; q < R; ++q) lds.template at<SH>(base + q * NS) = u[m + q * BPT];
  }
}

// Loads of a radix-R stage from a buffer written by a stage of radix 2^SH.
template <int NPT, int E, int R, int SH, class Lds>
__device__ __forceinline__ void stage_load(cf (&u)[E], const Lds& lds, int j) {
  constexpr int BPT = E / R;
#pragma unroll
  for (int m = 0; m < BPT; ++m) {
    const int beta = j + m * (NPT / E);
#pragma unroll
    for (int r = 0; r < R; ++r) u[m + r * BPT] = lds.template at<SH>(beta + r * (NPT / R));
  }
}

// Base twiddles w = W_{R*NS}^{beta mod NS} of every later stage, in stage order.
template <int NPT, int E, int NS, int OFF, int R, int... Rest>
__device__ __forceinline__ void tw_init(cf* tw, int j) {
  constexpr int BPT = E / R;
#pragma unroll
  for (int m = 0; m < BPT; ++m) {
    const uint32_t beta = (uint32_t)j + (uint32_t)m * (NPT / E);
    tw[OFF + m] = twiddle<false>(beta & (NS - 1), (uint32_t)(R * NS));
  }
  if constexpr (sizeof...(Rest) > 0) tw_init<NPT, E, NS * R, OFF + BPT, Rest...>(tw, j);
}

template <int NPT, int E, bool INV, int NS, int OFF, int SHPREV, class Lds, int R, int... Rest>
__device__ __forceinline__ void fft_tail(cf (&u)[E], const Lds& lds, int j, const cf* tw) {
  stage_load<NPT, E, R, SHPREV>(u, lds, j);
  stage_twiddled<E, R, INV>(u, tw + OFF);
  if constexpr (sizeof...(Rest) > 0) {
    __syncthreads();                       // all reads of this stage done
    stage_store<NPT, E, R, NS>(u, lds, j);
    __syncthreads();                       // writes visible to the next stage
    fft_tail<NPT, E, INV, NS * R, OFF + E / R, swz_key(R, NS), Lds, Rest...>(u, lds, j, tw);
  }
}

// Ping-pong variant: stage s stores into buffer s & 1, so a stage's loads and
// the next stage's stores never share a buffer and one barrier per stage
// suffices.  L[0], L[1] are the two buffers.
template <int NPT, int E, bool INV, int NS, int OFF, int SHPREV, int P, class Lds, int R, int... Rest>
__device__ __forceinline__ void fft_tail_pp(cf (&u)[E], const Lds* L, int j, const cf* tw) {
  stage_load<NPT, E, R, SHPREV>(u, L[P], j);
  stage_twiddled<E, R, INV>(u, tw + OFF);
  if constexpr (sizeof...(Rest) > 0) {
    stage_store<NPT, E, R, NS>(u, L[P ^ 1], j);
    __syncthreads();                       // writes visible to the next stage
    fft_tail_pp<NPT, E, INV, NS * R, OFF + E / R, swz_key(R, NS), P ^ 1, Lds, Rest...>(u, L, j, tw);
  }
}

template <int NPT, int E, class Rad> struct BlockFFT;

// Complex FFT of NPT points by the threads of a workgroup, E points each,
// radix sequence R0, Rs...  Registers in and out in the invariant layout.
// Every thread of the workgroup must call run() (it has barriers when there
// is more than one stage).  On return other threads may still read LDS:
// callers put a barrier before their next LDS write.
template <int NPT, int E, int R0, int... Rs>
struct BlockFFT<NPT, E, Radices<R0, Rs...>> {
  static constexpr int NTW = (0 + ... + (E / Rs));
  cf tw[NTW > 0 ? NTW : 1];

  __device__ __forceinline__ void init(int j) {
    if constexpr (NTW > 0) tw_init<NPT, E, R0, 0, Rs...>(tw, j);
  }

  template <bool INV, class Lds>
  __device__ __forceinline__ void run(cf (&u)[E], const Lds& lds, int j) const {
    stage_first<E, R0, INV>(u);
    if constexpr (sizeof...(Rs) > 0) {
      __syncthreads();
      stage_store<NPT, E, R0, 1>(u, lds, j);
      __syncthreads();
      fft_tail<NPT, E, INV, R0, 0, swz_key(R0, 1), Lds, Rs...>(u, lds, j, tw);
    }
  }

  // Two-buffer form (stages - 1 + 1 barriers).  The leading barrier keeps the
  // first store clear of reads still pending from the caller's previous use
  // of buffer 0.  The last stage reads buffer last_buf(); the other one is
  // free for the caller until the next run_pp().
  static constexpr int NSTAGES = 1 + sizeof...(Rs);
  static constexpr int last_buf() { return (NSTAGES - 2) & 1; }

  template <bool INV, class Lds>
  __device__ __forceinline__ void run_pp(cf (&u)[E], const Lds* L, int j) const {
    static_assert(sizeof...(Rs) > 0, "ping-pong needs at least two stages");
    stage_first<E, R0, INV>(u);
    __syncthreads();
    stage_store<NPT, E, R0, 1>(u, L[0], j);
    __syncthreads();
    fft_tail_pp<NPT, E, INV, R0, 0, swz_key(R0, 1), 0, Lds, Rs...>(u, L, j, tw);
  }
};

// Radix sequences per FFT length for 16 (or 8) points per thread.  First and
// last radix equal E so a thread's register set stays put.
template <int NPT> struct Plan16;
template <> struct Plan16<16> { using R = Radices<16>; };
template <> struct Plan16<32> { using R = Radices<16, 2>; };
template <> struct Plan16<64> { using R = Radices<16, 4>; };
template <> struct Plan16<128> { using R = Radices<16, 8>; };
template <> struct Plan16<256> { using R = Radices<16, 16>; };
template <> struct Plan16<512> { using R = Radices<16, 2, 16>; };
template <> struct Plan16<1024> { using R = Radices<16, 4, 16>; };
template <> struct Plan16<2048> { using R = Radices<16, 8, 16>; };
template <> struct Plan16<4096> { using R = Radices<16, 16, 16>; };
template <> struct Plan16<8192> { using R = Radices<16, 2, 16, 16>; };
template <> struct Plan16<16384> { using R = Radices<16, 4, 16, 16>; };

template <int NPT> struct Plan8;
template <> struct Plan8<64> { using R = Radices<8, 8>; };
template <> struct Plan8<128> { using R = Radices<8, 2, 8>; };
template <> struct Plan8<256> { using R = Radices<8, 4, 8>; };
template <> struct Plan8<512> { using R = Radices<8, 8, 8>; };
template <> struct Plan8<1024> { using R = Radices<8, 2, 8, 8>; };
template <> struct Plan8<2048> { using R = Radices<8, 4, 8, 8>; };
template <> struct Plan8<4096> { using R = Radices<8, 8, 8, 8>; };
template <> struct Plan8<8192> { using R = Radices<8, 2, 8, 8, 8>; };

// ---------------------------------------------------------------- I/O types

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats to packed bf16 (low half = lo), round to nearest even, by the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <int IOT> struct IO;
template <> struct IO<0> {  // fp32
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return __builtin_nontemporal_load(static_cast<const float*>(p) + i);
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    __builtin_nontemporal_store(v, static_cast<float*>(p) + i);
  }
};
template <> struct IO<1> {  // bf16
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return bf16_bits_to_f32(__builtin_nontemporal_load(static_cast<const uint16_t*>(p) + i));
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    __builtin_nontemporal_store((uint16_t)bf16x2_bits(v, 0.f), static_cast<uint16_t*>(p) + i);
  }
};

// ------------------------------------------------- real rows as half-size FFTs
//
// A real row x of M = 2N samples (zero-padded) travels as the complex signal
// c[m] = x[2m] + i x[2m+1] of N points.  With C = DFT_N(c) and W = W_M^k:
//   even part E(k) = (C(k) + conj C(N-k)) / 2, odd part O(k) = (C(k) - conj C(N-k)) / (2i),
//   X(k) = E(k) + W O(k) is the M-point real DFT (k = 0..N; C(N) means C(0)).
// For the filtered row Y = H X the inverse needs C'(k) = E'(k) + i O'(k) with
// E' = (Y(k) + conj Y(N-k))/2, O' = (Y(k) - conj Y(N-k)) conj(W) / 2.  Folding
// the two steps gives, with s = sin(2 pi k/M), c = cos(2 pi k/M), G = H/(2N),
// G' = conj G(N-k):
//   C'(k) = C(k) [(G + G') + s (G' - G)] + conj C(N-k) [i c (G - G')]
// and the inverse N-point DFT of C' (unnormalised) returns y[2m] + i y[2m+1].
// Each row is processed on its own, so rounding never mixes two rows.

// cos(2 pi q / 32), q = 0..31
__device__ constexpr float kCos32[32] = {1.00000000000000000000f, 0.98078528040323043058f, 0.92387953251128673848f, 0.83146961230254523567f, 0.70710678118654757274f, 0.55557023301960228867f, 0.38268343236508983729f, 0.19509032201612833135f, 0.00000000000000006123f, -0.19509032201612819257f, -0.38268343236508972627f, -0.55557023301960195560f, -0.70710678118654746172f, -0.83146961230254534669f, -0.92387953251128673848f, -0.98078528040323043058f, -1.00000000000000000000f, -0.98078528040323043058f, -0.92387953251128684951f, -0.83146961230254545772f, -0.70710678118654768376f, -0.55557023301960217765f, -0.38268343236509033689f, -0.19509032201612866442f, -0.00000000000000018370f, 0.19509032201612830359f, 0.38268343236509000382f, 0.55557023301960184458f, 0.70710678118654735069f, 0.83146961230254523567f, 0.92387953251128651644f, 0.98078528040323031956f};

// W_{2E}^i = exp(-2 pi i * i / (2E)) for compile-time i < 2E, E in {8, 16}.
template <int E>
__device__ __forceinline__ cf w2e(int i) {
  const int q = i * (16 / E);
  return make_float2(kCos32[q & 31], -kCos32[(q + 24) & 31]);
}

__device__ __forceinline__ cf realconv_bin(cf a, cf am, cf g, cf gm, cf w) {
  const float co = w.x, si = -w.y;
  const float sx = g.x + gm.x, sy = g.y - gm.y;      // G + G'
  const float dx = gm.x - g.x, dy = -gm.y - g.y;     // G' - G
  const cf U = make_float2(fmaf(si, dx, sx), fmaf(si, dy, sy));
  const cf V = make_float2(co * dy, -co * dx);       // i c (G - G')
  // a U + conj(am) V
  return make_float2(fmaf(am.y, V.y, fmaf(am.x, V.x, fmaf(a.x, U.x, -a.y * U.y))),
                     fmaf(-am.y, V.x, fmaf(am.x, V.y, fmaf(a.x, U.y, a.y * U.x))));
}

// Both bins of the pair (k, N-k) at once: a = C(k) -> C'(k), b = C(N-k) ->
// C'(N-k), g = G(k), gm = G(N-k), w = W_M^k.  With P = G(k) + conj G(N-k) and
// Q = conj G(N-k) - G(k):  U_k = P + sQ, V_k = -icQ, U_{N-k} = conj(P - sQ),
// V_{N-k} = -ic conj(Q), and C'(k) = a U_k + conj(b) V_k,
// C'(N-k) = b U_{N-k} + conj(a) V_{N-k}.
__device__ __forceinline__ void realconv_pair(cf& a, cf& b, cf g, cf gm, cf w) {
  const float co = w.x, si = -w.y;
  const float px = g.x + gm.x, py = g.y - gm.y;
  const float qx = gm.x - g.x, qy = -gm.y - g.y;
  const cf U1 = make_float2(fmaf(si, qx, px), fmaf(si, qy, py));
  const cf U2 = make_float2(fmaf(-si, qx, px), fmaf(si, qy, -py));
  const float cqx = co * qx, cqy = co * qy;
  const cf V1 = make_float2(cqy, -cqx), V2 = make_float2(-cqy, -cqx);
  const cf na = cadd(cmul(a, U1), cmul(cconj(b), V1));
  const cf nb = cadd(cmul(b, U2), cmul(cconj(a), V2));
  a = na;
  b = nb;
}

// The same product with the coefficients precomputed per bin pair.  The
// whole step is linear in (C(p), conj C(N-p)):
//   C'(p)   = a1 C(p)   + i bq conj C(N-p),
//   C'(N-p) = a2 C(N-p) + i conj(bq C(p)),
// with, for H = the filter's real-FFT bins over M, s + i c = i W_M^p,
// P = H(p) + conj H(N-p) and Q = H(p) - conj H(N-p):
//   a1 = P - sQ,  a2 = conj(P + sQ),  bq = cQ
// (scaled for an unnormalised inverse FFT).  This is the even/odd split of
// the row spectrum, the product with H and the re-packing, folded together.
// 16 FMA-class operations per pair; no twiddle is needed at run time.
__device__ __forceinline__ void conv_pair(cf& a, cf& b, cf a1, cf a2, cf bq) {
  const cf na = make_float2(fmaf(a1.x, a.x, fmaf(-a1.y, a.y, fmaf(bq.x, b.y, -bq.y * b.x))),
                            fmaf(a1.x, a.y, fmaf(a1.y, a.x, fmaf(bq.x, b.x, bq.y * b.y))));
  const cf nb = make_float2(fmaf(a2.x, b.x, fmaf(-a2.y, b.y, fmaf(bq.x, a.y, bq.y * a.x))),
                            fmaf(a2.x, b.y, fmaf(a2.y, b.x, fmaf(bq.x, a.x, -bq.y * a.y))));
  a = na;
  b = nb;
}

// Bin 0, its own partner: C'(0) = a1 C(0) + i bq conj C(0).
__device__ __forceinline__ cf conv_self(cf a, cf a1, cf bq) {
  return make_float2(fmaf(a1.x, a.x, fmaf(-a1.y, a.y, fmaf(bq.x, a.y, -bq.y * a.x))),
                     fmaf(a1.x, a.y, fmaf(a1.y, a.x, fmaf(bq.x, a.x, bq.y * a.y))));
}

// Pair coefficients (a1, a2, bq) of bins (p, N-p) from hk = H(p)/M,
// hm = H(N-p)/M and (s, c) = (sin, cos)(pi p / N).
__device__ __forceinline__ void pair_coeffs(cf hk, cf hm, float s, float c, cf& a1, cf& a2, cf& bq) {
  const cf P = make_float2(hk.x + hm.x, hk.y - hm.y);
  const cf Q = make_float2(hk.x - hm.x, hk.y + hm.y);
  a1 = make_float2(fmaf(-s, Q.x, P.x), fmaf(-s, Q.y, P.y));
  a2 = make_float2(fmaf(s, Q.x, P.x), -fmaf(s, Q.y, P.y));
  bq = make_float2(c * Q.x, c * Q.y);
}

// X(k) / (2N) of the real row from C(k), C(N-k) and W = W_M^k.
__device__ __forceinline__ cf realfft_bin(cf a, cf am, cf w, float scale) {
  const cf e = make_float2(a.x + am.x, a.y - am.y);          // 2 E
  const cf o = make_float2(a.y + am.y, am.x - a.x);          // 2 O
  return cscale(cadd(e, cmul(w, o)), 0.5f * scale);
}

// x[t] with zero padding beyond L.  CLAMP: the load always runs, from a
// clamped in-row index (L >= 1), so no branch splits the memory counters
// (for loads that are mostly in range); otherwise padding loads are skipped.
template <int IOT, bool CLAMP = false>
__device__ __forceinline__ float ld_masked(const void* p, int64_t row_off, int64_t t, int64_t L) {
  if constexpr (CLAMP) {
    const float w = IO<IOT>::ld(p, row_off + (t < L ? t : L - 1));
    return t < L ? w : 0.f;
  } else {
    return t < L ? IO<IOT>::ld(p, row_off + t) : 0.f;
  }
}

// (x[t], x[t+1]) for even t with zero padding beyond L.  EVEN: the row
// offset and L are even, so the pair is one aligned 8-byte (fp32) or 4-byte
// (bf16) access.  CLAMP as in ld_masked.
template <int IOT, bool EVEN, bool CLAMP = false>
__device__ __forceinline__ cf ld_pair(const void* p, int64_t row_off, int64_t t, int64_t L) {
  if constexpr (EVEN) {
    if constexpr (!CLAMP) {
      if (t >= L) return make_float2(0.f, 0.f);
    }
    const int64_t tc = row_off + ((CLAMP && t >= L) ? L - 2 : t);
    cf v;
    if constexpr (IOT == 0) {
      const f32x2 w = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(static_cast<const float*>(p) + tc));
      v = make_float2(w.x, w.y);
    } else {
      const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + tc));
      v = make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    }
    return (CLAMP && t >= L) ? make_float2(0.f, 0.f) : v;
  } else {
    return make_float2(ld_masked<IOT, CLAMP>(p, row_off, t, L), ld_masked<IOT, CLAMP>(p, row_off, t + 1, L));
  }
}

// The bf16 pair (x[t], x[t+1]) for even t as its raw 32-bit word (x[t] in
// the low half), zero padding beyond L; bf16_pair_cf unpacks it.  One
// register per pair instead of two while a load waits for its use.  The
// load always runs, from a clamped in-row index (as ld_pair with CLAMP).
template <bool EVEN>
__device__ __forceinline__ uint32_t ld_pair_bits(const void* p, int64_t row_off, int64_t t, int64_t L) {
  const uint16_t* q = static_cast<const uint16_t*>(p) + row_off;
  if constexpr (EVEN) {
    const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(q + (t < L ? t : L - 2)));
    return t < L ? w : 0u;
  } else {
    const uint32_t lo = __builtin_nontemporal_load(q + (t < L ? t : L - 1));
    const uint32_t hi = __builtin_nontemporal_load(q + (t + 1 < L ? t + 1 : L - 1));
    return (t < L ? lo : 0u) | (t + 1 < L ? hi << 16 : 0u);
  }
}
__device__ __forceinline__ cf bf16_pair_cf(uint32_t w) {
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// An activation pair as loaded (a bf16 pair's 32-bit word, or two floats,
// zero beyond L, from clamped indices), pinned, then unpacked.  pin() hands
// the value to an empty asm statement, so the load has to complete there and
// the compiler cannot sink it into a later branch (e.g. the mask of a
// store): a load sunk into such a branch waits for its data before the next
// one is issued.  Loading a batch, then pinning it, keeps the batch in flight
// together; FENCE (a memory clobber) also keeps later loads after the pin,
// which bounds the registers a batch holds.
template <int IOT> struct RawPair { cf v; };
template <> struct RawPair<1> { uint32_t w; };
template <int IOT, bool EVEN>
__device__ __forceinline__ RawPair<IOT> ld_pair_raw(const void* p, int64_t row_off, int64_t t, int64_t L) {
  if constexpr (IOT == 0) return {ld_pair<0, EVEN, true>(p, row_off, t, L)};
  else return {ld_pair_bits<EVEN>(p, row_off, t, L)};
}
template <int IOT, bool FENCE = false>
__device__ __forceinline__ void pin(RawPair<IOT>& r) {
  if constexpr (FENCE) {
    if constexpr (IOT == 0) asm volatile("" : "+v"(r.v.x), "+v"(r.v.y) : : "memory");
    else asm volatile("" : "+v"(r.w) : : "memory");
  } else {
    if constexpr (IOT == 0) asm volatile("" : "+v"(r.v.x), "+v"(r.v.y));
    else asm volatile("" : "+v"(r.w));
  }
}
template <int IOT>
__device__ __forceinline__ cf unpack(RawPair<IOT> r) {
  if constexpr (IOT == 0) return r.v;
  else return bf16_pair_cf(r.w);
}

// (x[t], x[t+1]) of a row whose every requested pair is in range (t + 1 < L,
// row offset and t even): one aligned access, no mask.
template <int IOT>
__device__ __forceinline__ cf ld_pair_in(const void* p, int64_t row_off, int t) {
  if constexpr (IOT == 0) {
    const f32x2 w = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(static_cast<const float*>(p) + row_off) + (t >> 1));
    return make_float2(w.x, w.y);
  } else {
    const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + row_off) + (t >> 1));
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  }
}

template <int IOT>
__device__ __forceinline__ void st_pair_in(void* p, int64_t row_off, int t, cf v) {
  if constexpr (IOT == 0) {
    const f32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x2*>(static_cast<float*>(p) + row_off) + (t >> 1));
  } else {
    __builtin_nontemporal_store(bf16x2_bits(v.x, v.y), reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + row_off) + (t >> 1));
  }
}

template <int IOT, bool EVEN>
__device__ __forceinline__ void st_pair(void* p, int64_t row_off, int64_t t, int64_t L, cf v) {
  if constexpr (EVEN) {
    if (t >= L) return;
    if constexpr (IOT == 0) {
      const f32x2 w = {v.x, v.y};
      __builtin_nontemporal_store(w, reinterpret_cast<f32x2*>(static_cast<float*>(p) + row_off + t));
    } else {
      const uint32_t w = bf16x2_bits(v.x, v.y);
      __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + row_off + t));
    }
  } else {
    if (t < L) IO<IOT>::st(p, row_off + t, v.x);
    if (t + 1 < L) IO<IOT>::st(p, row_off + t + 1, v.y);
  }
}

using XPtrs = XPtrsHost;

}  // namespace hyena
