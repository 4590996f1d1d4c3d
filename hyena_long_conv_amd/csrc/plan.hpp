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
#ifndef HYENA_WORK_MB
#define HYENA_WORK_MB 256
#endif
constexpr int64_t kSingleMaxN = HYENA_SINGLE_MAX_N;
constexpr int64_t kMinN = 64;
constexpr int kRowPref = 1024;           // preferred row length of power-of-two plans
constexpr int kRowPrefMax = 4096;        // longest row a power-of-two plan takes below the 2^22 limit
constexpr int kColPrefMin = 64, kColPrefMax = 512;
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

// Column lengths of the four-step path beyond the powers of two: q odd (one
// thread per column, the whole column DFT in registers) and 2q (a lane pair
// per column).  With power-of-two rows they give complex lengths
// N = n1 * n2 = 2^a 3^b 5^c, so a zero-padded row of a length L that is not
// a power of two needs at most ~20% more points than 2L instead of up to
// 100% more.
constexpr int kOddCols[] = {3, 5, 9, 15, 25, 27};
constexpr int kRowMaxOdd = 4096;    // longest row with an odd column length
constexpr int kRowMaxPair = 2048;   // longest row with a 2q column length
inline bool is_odd_col(int64_t n) {
  for (int q : kOddCols)
    if (n == q) return true;
  return false;
}
inline bool is_pair_col(int64_t n) { return n % 2 == 0 && is_odd_col(n / 2); }

// Relative cost of one complex point per pass on each kind of plan, from
// timings of the order-3, B = 2, D = 1024, bf16 shapes on MI355X (points per
// ms per order): power-of-two plans 14.0, odd or 2q columns with rows of at
// most 2048 points 12.6, odd columns with 4096-point rows 11.3.
inline double plan_cost(int64_t n1, int64_t n2) {
  const double rate = is_pow2(n1) ? 14.0 : (n2 <= 2048 ? 12.6 : 11.3);
  return (double)(n1 * n2) / rate;
}

// Cheapest odd or 2q factorisation with n1 * n2 >= Nmin (n2 a power of two
// in [kRowMin, kRowMaxOdd or kRowMaxPair]); 0 if none.
inline int64_t best_smooth_plan(int64_t Nmin, int64_t* n1_out, int64_t* n2_out) {
  int64_t best = 0;
  double best_cost = 0;
  for (int q : kOddCols) {
    for (int n1 = q; n1 <= 2 * q; n1 += q) {
      int64_t n2 = next_pow2((Nmin + n1 - 1) / n1);
      if (n2 < kRowMin) n2 = kRowMin;
      if (n2 > (n1 % 2 ? kRowMaxOdd : kRowMaxPair)) continue;
      const double c = plan_cost(n1, n2);
      if (best == 0 || c < best_cost) {
        best = n1 * n2;
        best_cost = c;
        *n1_out = n1;
        *n2_out = n2;
      }
    }
  }
  return best;
}

// Returns 0 on success, 2 (shape) for a bad L, 3 (unsupported) when a forced
// path cannot serve L.  force_path: NULL/"" auto, "single", "fourstep".
// A forced column length (force_n1) is a power of two in [kColMin, kColMax],
// an odd q of kOddCols or 2q.  Lengths long enough for the four-step path by
// themselves (and not circular) take the cheaper (plan_cost) of the
// power-of-two and the best 2^a 3^b 5^c factorisation; forced four-step runs
// of shorter lengths keep the power of two, so their spectra match the
// single path's.
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
    // Rows of 1024 points with columns of 64..512 points: from timing sweeps
    // over N = 2^15 .. 2^21 (orders 2-3, B = 1-4, fp32 and bf16), 1024-point
    // rows beat 2048-point ones by 2-10% (the 64K shape 32 x 2048 -> 64 x 1024:
    // -8%) as long as the columns stay at 512 points or fewer (1024-point
    // columns run one workgroup per CU: the 1M shape keeps 512 x 2048;
    // 2^21 takes 512 x 4096, 2.4% faster than 1024 x 2048).
    int64_t n1 = N / kRowPref;
    if (n1 < kColPrefMin) n1 = kColPrefMin;
    if (n1 > kColPrefMax) n1 = kColPrefMax;
    if (N / n1 < kRowMin) n1 = N / kRowMin;   // short (forced) lengths: rows of at least 64
    if (n1 < kColMin) n1 = kColMin;
    if (N / n1 > kRowPrefMax) n1 = N / kRowPrefMax;   // 2^22: 1024 x 4096
    int64_t n2 = N / n1;
    const bool natural = (next_pow2(2 * L) / 2) > kSingleMaxN;
    if (force_n1 && *force_n1) {
      const int64_t f = atoll(force_n1);
      if (is_odd_col(f) || is_pair_col(f)) {
        if (circular) return 3;
        n1 = f;
        n2 = next_pow2((L + f - 1) / f);
        if (n2 < kRowMin) n2 = kRowMin;
        if (n2 > (f % 2 ? kRowMaxOdd : kRowMaxPair)) return 3;
      } else {
        if (!is_pow2(f) || f < kColMin || f > kColMax) return 3;
        n1 = f;
        if (circular && N / n1 < kRowMin) return 3;
        while (N / n1 < kRowMin) N <<= 1;   // a longer FFT is still exact
        n2 = N / n1;
      }
      N = n1 * n2;
    } else if (natural && !circular) {
      int64_t q = 0, r = 0;
      const int64_t smooth = best_smooth_plan(L, &q, &r);
      if (smooth > 0 && plan_cost(q, r) < plan_cost(n1, n2)) {
        n1 = q;
        n2 = r;
        N = smooth;
      }
    }
    if (n1 > kColMax || n2 > kRowLimit || n2 < kRowMin || n1 * n2 != N) return 3;
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

// Bytes of intermediate a pass group may hold.  The environment variable
// HYENA_WORK_MB (a positive number of MiB), when set, overrides the built-in
// budget at run time: tests force several pass groups with it and tuning
// sweeps size the groups.  Host code only.
inline int64_t work_budget_bytes() {
  const char* e = getenv("HYENA_WORK_MB");
  if (e && *e) {
    const long long mb = atoll(e);
    if (mb > 0 && mb < (1LL << 24)) return (int64_t)mb << 20;
  }
  return kWorkBudget;
}

// Rows per pass group for rows of row_bytes each: as many groups as the
// budget needs (at least one row per group), all of equal size (768 rows as
// 384 + 384 rather than 512 + 256), never more than n_rows.
inline int64_t group_rows(int64_t row_bytes, int64_t n_rows) {
  if (n_rows < 1) return 1;
  int64_t g = row_bytes > 0 ? work_budget_bytes() / row_bytes : n_rows;
  if (g < 1) g = 1;
  if (g > n_rows) g = n_rows;
  const int64_t groups = (n_rows + g - 1) / g;
  return (n_rows + groups - 1) / groups;
}

// The same for rows of an N-point complex intermediate of esz bytes per
// point (8: float2; 4: a bf16 pair).
inline int rows_per_group(int64_t N, int64_t n_rows, int64_t esz = 8) { return (int)group_rows(N * esz, n_rows); }

// The four-step forward keeps its intermediate as bf16 pairs for bf16
// activations up to this order: each order rounds it twice and the rounding
// compounds through the gates (max normalised error against the oracle,
// bound 2e-2: 8.4e-3 at order 2 on the 64K shape, 1.8e-2 at order 3 on the
// 128K and 100000 shapes, 3.6e-3 with an fp32 intermediate).
constexpr int kBf16WorkMaxOrder = 2;
inline bool forward_bf16_work(bool bf16_io, int order) { return bf16_io && order <= kBf16WorkMaxOrder; }
// Bytes per intermediate point of the four-step forward.
inline int64_t forward_work_esz(bool bf16_io, int order) { return forward_bf16_work(bf16_io, order) ? 4 : 8; }

}  // namespace hyena
