// plan.hpp -- host-side planner for the Hyena forward (pure C++, no HIP).
//
// Chooses the FFT length and the execution path for a sequence length L:
//   * single pass: the whole M-point complex signal of one row pair lives in
//     one workgroup's LDS (M <= 16384 points, i.e. L <= 8192);
//   * four-step: M = n1 * n2, column FFTs of n1 points and row FFTs of n2
//     points with a twiddle in between (Bailey's decomposition), passes
//     linked through a workspace buffer.
// The causal linear convolution needs any M >= 2L - 1 (zero padding so the
// circular wrap never reaches the kept samples); M is the next power of two
// >= 2L, at least 64.
#pragma once

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

namespace hyena {

enum { PATH_SINGLE = 1, PATH_FOURSTEP = 2 };

constexpr int64_t kMaxL = int64_t(1) << 22;
constexpr int64_t kSingleMaxM = 16384;
constexpr int64_t kMinM = 64;
constexpr int kRowMax = 8192;   // largest row FFT (a row pair fills one workgroup's LDS)
constexpr int kRowMin = 64;
constexpr int kColMin = 16;
constexpr int kColMax = 1024;
constexpr int kMaxOrder = 8;
constexpr int kMaxFreq = 16;

struct XPtrsHost {
  const void* p[8];
};

struct PlanInfo {
  int64_t L, M;
  int path;
  int n1, n2;
  int64_t spec_stride;   // complex values per filter row in the spectrum buffer
};

inline int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}
inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Returns 0 on success, 2 (shape) for a bad L, 3 (unsupported) when a forced
// path cannot serve L.  force_path: NULL/"" auto, "single", "fourstep".
inline int make_plan(int64_t L, const char* force_path, const char* force_n1, PlanInfo* out) {
  if (L < 1 || L > kMaxL) return 2;
  int64_t M = next_pow2(2 * L);
  if (M < kMinM) M = kMinM;
  int path = (M <= kSingleMaxM) ? PATH_SINGLE : PATH_FOURSTEP;
  if (force_path && *force_path) {
    if (!strcmp(force_path, "single")) {
      if (M > kSingleMaxM) return 3;
      path = PATH_SINGLE;
    } else if (!strcmp(force_path, "fourstep")) {
      path = PATH_FOURSTEP;
    }
  }
  PlanInfo p{};
  p.L = L;
  p.path = path;
  if (path == PATH_SINGLE) {
    p.M = M;
    p.n1 = p.n2 = 0;
    p.spec_stride = round_up(M / 2 + 1, 16);
  } else {
    if (M < (int64_t)kColMin * kRowMin) M = (int64_t)kColMin * kRowMin;
    int64_t n1 = M / kRowMax;
    if (n1 < kColMin) n1 = kColMin;
    if (force_n1 && *force_n1) {
      const int64_t f = atoll(force_n1);
      if (!is_pow2(f) || f < kColMin || f > kColMax) return 3;
      n1 = f;
      while (M / n1 < kRowMin) M <<= 1;   // a larger M is still exact
    }
    const int64_t n2 = M / n1;
    if (n1 > kColMax || n2 > kRowMax || n2 < kRowMin) return 3;
    p.M = M;
    p.n1 = (int)n1;
    p.n2 = (int)n2;
    p.spec_stride = round_up(n1 * (n2 / 2 + 1), 16);
  }
  *out = p;
  return 0;
}

// Pairing of the B*D real rows into complex signals (see decode_pair).
struct Pairing {
  int n_pairs, n_batch_pairs, half_b;
};
inline Pairing make_pairing(int64_t B, int64_t D) {
  Pairing r;
  r.half_b = (int)(B / 2);
  r.n_batch_pairs = (int)((B / 2) * D);
  r.n_pairs = r.n_batch_pairs + ((B & 1) ? (int)((D + 1) / 2) : 0);
  return r;
}

// Four-step intermediate: one M-point complex signal per pair in flight.
constexpr int64_t kWorkBudget = int64_t(256) << 20;

inline int pairs_per_group(int64_t M, int64_t n_pairs) {
  int64_t g = kWorkBudget / (M * 8);
  if (g < 1) g = 1;
  if (g > n_pairs) g = n_pairs;
  return (int)g;
}

}  // namespace hyena
