// plan.hpp -- host-side planner for the Hyena forward (pure C++, no HIP).
//
// Chooses the FFT length and the execution path for a sequence length L.
// The causal linear convolution needs a real FFT length M >= 2L - 1 (zero
// padding so the circular wrap never reaches the kept samples); M is the
// next power of two >= 2L.  A real row of M samples is carried as a complex
// signal of N = M/2 points (even samples real, odd samples imaginary).
//   * single pass: one workgroup holds a row's N points in registers/LDS
//     for all orders (N <= kSingleMaxN);
//   * four-step: N = n1 * n2, column FFTs of n1 points and row FFTs of n2
//     points with a twiddle in between (Bailey's decomposition), passes
//     linked through a workspace buffer.
// Circular mode (periodic boundary, gist.science HyenaND summary, section
// "手法: HyenaND", boundary handling) takes M = L with no padding; L must then
// be a power of two >= 128.
#pragma once

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

namespace hyena {

enum { PATH_SINGLE = 1, PATH_FOURSTEP = 2 };

constexpr int64_t kMaxL = int64_t(1) << 22;
#ifndef HYENA_SINGLE_MAX_N
#define HYENA_SINGLE_MAX_N 16384
#endif
#ifndef HYENA_ROW_MAX
#define HYENA_ROW_MAX 2048
#endif
#ifndef HYENA_WORK_MB
#define HYENA_WORK_MB 256
#endif
constexpr int64_t kSingleMaxN = HYENA_SINGLE_MAX_N;
constexpr int64_t kMinN = 64;
constexpr int kRowMax = HYENA_ROW_MAX;   // largest row FFT (a row pair fills one workgroup's LDS)
constexpr int kRowMin = 64;
constexpr int kRowLimit = 8192;  // largest row kernel compiled
constexpr int kColMin = 16;
constexpr int kColMax = 1024;
constexpr int kMaxOrder = 8;
constexpr int kMaxFreq = 16;

struct XPtrsHost {
  const void* p[8];
};

struct PlanInfo {
  int64_t L;
  int64_t M;             // real FFT length (zero-padded row)
  int64_t N;             // complex FFT length, M / 2
  int path;
  int n1, n2;            // four-step factors of N
  int64_t spec_stride;   // complex values per filter row in the spectrum buffer (>= N + 1)
  int circular;          // 1: M = L, periodic convolution
};

// Single path: a filter row holds three planar arrays of N/2 + 1 complex
// values (the pair coefficients), each single_qs(N) values apart.
inline int64_t single_qs(int64_t N) { return (N / 2 + 1 + 15) / 16 * 16; }

inline int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}
inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Returns 0 on success, 2 (shape) for a bad L, 3 (unsupported) when a forced
// path cannot serve L.  force_path: NULL/"" auto, "single", "fourstep".
inline int make_plan(int64_t L, const char* force_path, const char* force_n1, PlanInfo* out, int circular = 0) {
  if (L < 1 || L > kMaxL) return 2;
  int64_t N = next_pow2(2 * L) / 2;
  if (N < kMinN) N = kMinN;
  if (circular) {
    if (!is_pow2(L) || L < 2 * kMinN) return 3;
    N = L / 2;
  }
  int path = (N <= kSingleMaxN) ? PATH_SINGLE : PATH_FOURSTEP;
  if (force_path && *force_path) {
    if (!strcmp(force_path, "single")) {
      if (N > 16384) return 3;
      path = PATH_SINGLE;
    } else if (!strcmp(force_path, "fourstep")) {
      path = PATH_FOURSTEP;
    }
  }
  PlanInfo p{};
  p.L = L;
  p.path = path;
  if (path == PATH_SINGLE) {
    p.n1 = p.n2 = 0;
  } else {
    if (N < (int64_t)kColMin * kRowMin) {
      if (circular) return 3;
      N = (int64_t)kColMin * kRowMin;
    }
    int64_t n1 = N / kRowMax;
    if (n1 < kColMin) n1 = kColMin;
    if (n1 > kColMax) n1 = kColMax;   // longest rows (up to 8192) beyond that
    if (force_n1 && *force_n1) {
      const int64_t f = atoll(force_n1);
      if (!is_pow2(f) || f < kColMin || f > kColMax) return 3;
      n1 = f;
      if (circular && N / n1 < kRowMin) return 3;
      while (N / n1 < kRowMin) N <<= 1;   // a longer FFT is still exact
    }
    const int64_t n2 = N / n1;
    if (n1 > kColMax || n2 > kRowLimit || n2 < kRowMin) return 3;
    p.n1 = (int)n1;
    p.n2 = (int)n2;
  }
  p.N = N;
  p.M = 2 * N;
  p.circular = circular ? 1 : 0;
  p.spec_stride = (path == PATH_SINGLE) ? 3 * single_qs(N) : round_up(N + 1, 16);
  *out = p;
  return 0;
}

// Four-step intermediate: one N-point complex signal per row in flight.
constexpr int64_t kWorkBudget = int64_t(HYENA_WORK_MB) << 20;

inline int rows_per_group(int64_t N, int64_t n_rows) {
  int64_t g = kWorkBudget / (N * 8);
  if (g < 1) g = 1;
  if (g > n_rows) g = n_rows;
  return (int)g;
}

}  // namespace hyena
