// fft_odd.hpp -- in-register DFTs of odd lengths 3, 5, 9, 15, 25 and 27 for
// one thread, for four-step factorisations N = n1 * n2 whose column length
// n1 is odd (the FFT length of a zero-padded row then only has to be a
// 2^a 3^b 5^c number >= 2L - 1 instead of a power of two).
//
// Prime lengths 3 and 5 are evaluated from the symmetric/antisymmetric input
// sums (the textbook real-coefficient form of a small DFT); composite
// lengths P*Q by the Cooley-Tukey index map n = Q*n1 + n2, k = k1 + P*k2:
// Q DFTs of length P, twiddles W_N^(n2 k1), P DFTs of length Q.  Every
// twiddle is a compile-time constant, evaluated in double by a constexpr
// Taylor series and rounded once to float.  The header stands alone and its
// functions are host-callable too, so the same code is checked on the CPU
// against a library FFT (tests/test_fft_odd.py).
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

namespace hyena {

typedef float2 cf;

namespace odd_detail {

__host__ __device__ inline cf add(cf a, cf b) { return make_float2(a.x + b.x, a.y + b.y); }
__host__ __device__ inline cf sub(cf a, cf b) { return make_float2(a.x - b.x, a.y - b.y); }
__host__ __device__ inline cf scale(cf a, float s) { return make_float2(a.x * s, a.y * s); }
__host__ __device__ inline cf mul(cf a, cf b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

constexpr double kPi = 3.14159265358979323846264338327950288;

// sin and cos of x in [-pi, pi] by their Taylor series (40 terms: the
// remainder is far below double rounding).
constexpr double taylor_sin(double x) {
  double term = x, sum = x;
  for (int n = 1; n < 40; ++n) {
    term *= -x * x / ((2.0 * n) * (2.0 * n + 1.0));
    sum += term;
  }
  return sum;
}
constexpr double taylor_cos(double x) {
  double term = 1.0, sum = 1.0;
  for (int n = 1; n < 40; ++n) {
    term *= -x * x / ((2.0 * n - 1.0) * (2.0 * n));
    sum += term;
  }
  return sum;
}
// angle 2 pi m / n reduced to [-pi, pi]
constexpr double angle(long m, long n) {
  m %= n;
  if (m < 0) m += n;
  if (2 * m > n) m -= n;
  return 2.0 * kPi * (double)m / (double)n;
}
constexpr float cos2pi(long m, long n) { return (float)taylor_cos(angle(m, n)); }
constexpr float sin2pi(long m, long n) { return (float)taylor_sin(angle(m, n)); }

}  // namespace odd_detail

// W_n^m = exp(-2 pi i m / n) (forward) or its conjugate (inverse), m and n
// compile-time.
template <long M, long N, bool INV>
__host__ __device__ inline cf wconst() {
  constexpr float c = odd_detail::cos2pi(M, N), s = odd_detail::sin2pi(M, N);
  return INV ? make_float2(c, s) : make_float2(c, -s);
}

// times -i (forward) or +i (inverse)
template <bool INV>
__host__ __device__ inline cf mul_mi(cf a) {
  return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// X_k = sum_n a_n W_3^(nk):  X_0 = a0 + s, X_(1,2) = a0 - s/2 -+ i (sqrt3/2) d
// with s = a1 + a2, d = a1 - a2 (forward; inverse flips the sign of i).
template <bool INV>
__host__ __device__ inline void dft3(cf* a) {
  using namespace odd_detail;
  constexpr float h = 0.86602540378443864676f;   // sin(2 pi / 3)
  const cf s = add(a[1], a[2]), d = sub(a[1], a[2]);
  const cf m = make_float2(fmaf(-0.5f, s.x, a[0].x), fmaf(-0.5f, s.y, a[0].y));
  const cf r = mul_mi<INV>(scale(d, h));
  a[0] = add(a[0], s);
  a[1] = add(m, r);
  a[2] = sub(m, r);
}

// X_0 = a0 + t1 + t2, X_(1,4) = a0 + c1 t1 + c2 t2 -+ i (s1 u1 + s2 u2),
// X_(2,3) = a0 + c2 t1 + c1 t2 -+ i (s2 u1 - s1 u2), with t1 = a1 + a4,
// t2 = a2 + a3, u1 = a1 - a4, u2 = a2 - a3, c_j = cos(2 pi j / 5),
// s_j = sin(2 pi j / 5) (forward; inverse flips the sign of i).
template <bool INV>
__host__ __device__ inline void dft5(cf* a) {
  using namespace odd_detail;
  constexpr float c1 = odd_detail::cos2pi(1, 5), c2 = odd_detail::cos2pi(2, 5);
  constexpr float s1 = odd_detail::sin2pi(1, 5), s2 = odd_detail::sin2pi(2, 5);
  const cf t1 = add(a[1], a[4]), t2 = add(a[2], a[3]);
  const cf u1 = sub(a[1], a[4]), u2 = sub(a[2], a[3]);
  const cf b1 = make_float2(fmaf(c2, t2.x, fmaf(c1, t1.x, a[0].x)), fmaf(c2, t2.y, fmaf(c1, t1.y, a[0].y)));
  const cf b2 = make_float2(fmaf(c1, t2.x, fmaf(c2, t1.x, a[0].x)), fmaf(c1, t2.y, fmaf(c2, t1.y, a[0].y)));
  const cf d1 = mul_mi<INV>(make_float2(fmaf(s2, u2.x, s1 * u1.x), fmaf(s2, u2.y, s1 * u1.y)));
  const cf d2 = mul_mi<INV>(make_float2(fmaf(-s1, u2.x, s2 * u1.x), fmaf(-s1, u2.y, s2 * u1.y)));
  a[0] = add(a[0], add(t1, t2));
  a[1] = add(b1, d1);
  a[4] = sub(b1, d1);
  a[2] = add(b2, d2);
  a[3] = sub(b2, d2);
}

template <int N, bool INV> struct RegDft;

template <bool INV> struct RegDft<1, INV> {
  static __host__ __device__ inline void run(cf*) {}
};
template <bool INV> struct RegDft<3, INV> {
  static __host__ __device__ inline void run(cf* a) { dft3<INV>(a); }
};
template <bool INV> struct RegDft<5, INV> {
  static __host__ __device__ inline void run(cf* a) { dft5<INV>(a); }
};

// Composite N = P * Q, natural order in and out.
template <int P, int Q, bool INV>
struct RegDftPQ {
  static constexpr int N = P * Q;
  template <int N2, int K1>
  static __host__ __device__ inline void twiddle_one(cf* b) {
    if constexpr (N2 * K1 != 0) b[N2 * P + K1] = odd_detail::mul(b[N2 * P + K1], wconst<(long)N2 * K1, N, INV>());
  }
  template <int N2, int... K1>
  static __host__ __device__ inline void twiddle_row(cf* b, std::integer_sequence<int, K1...>) {
    (twiddle_one<N2, K1>(b), ...);
  }
  template <int... N2>
  static __host__ __device__ inline void twiddle_all(cf* b, std::integer_sequence<int, N2...>) {
    (twiddle_row<N2>(b, std::make_integer_sequence<int, P>{}), ...);
  }
  static __host__ __device__ inline void run(cf* a) {
    cf b[N];
    // inner DFTs over n1 for each n2: b[n2*P + k1]
#pragma unroll
    for (int n2 = 0; n2 < Q; ++n2) {
      cf t[P];
#pragma unroll
      for (int n1 = 0; n1 < P; ++n1) t[n1] = a[Q * n1 + n2];
      RegDft<P, INV>::run(t);
#pragma unroll
      for (int k1 = 0; k1 < P; ++k1) b[n2 * P + k1] = t[k1];
    }
    twiddle_all(b, std::make_integer_sequence<int, Q>{});
    // outer DFTs over n2 for each k1: X[k1 + P*k2]
#pragma unroll
    for (int k1 = 0; k1 < P; ++k1) {
      cf t[Q];
#pragma unroll
      for (int n2 = 0; n2 < Q; ++n2) t[n2] = b[n2 * P + k1];
      RegDft<Q, INV>::run(t);
#pragma unroll
      for (int k2 = 0; k2 < Q; ++k2) a[k1 + P * k2] = t[k2];
    }
  }
};

template <bool INV> struct RegDft<9, INV> : RegDftPQ<3, 3, INV> {};
template <bool INV> struct RegDft<15, INV> : RegDftPQ<3, 5, INV> {};
template <bool INV> struct RegDft<25, INV> : RegDftPQ<5, 5, INV> {};
template <bool INV> struct RegDft<27, INV> : RegDftPQ<3, 9, INV> {};

// Odd column lengths the four-step planner may choose.
constexpr bool odd_col_ok(int n) { return n == 3 || n == 5 || n == 9 || n == 15 || n == 25 || n == 27; }

}  // namespace hyena
