// kernels_fourstep.hip -- multi-pass Hyena forward and filter spectrum for
// FFT lengths too long for one workgroup's LDS.
//
// Each real row travels as an N-point complex signal c[m] = x[2m] + i x[2m+1]
// (see fft_engine.hpp).  Its DFT is factored as N = n1 * n2 (Bailey's four-
// step): with m = n2*i1 + i2 and k = k1 + n1*k2,
//   A[k1][i2]    = sum_{i1} c[n2*i1 + i2] W_{n1}^{i1 k1}          (column pass)
//   C[k1+n1 k2] = sum_{i2} A[k1][i2] W_N^{i2 k1} W_{n2}^{i2 k2}    (row pass)
// and the inverse runs the same steps backwards with conjugate twiddles.
// Per order the row pass does row FFT -> spectral product -> inverse row
// FFT in one kernel, and the column pass does inverse column FFT -> gate with
// x_n -> forward column FFT of the next order in one kernel, so each order
// costs two passes over an N-point intermediate per row.  The spectral
// product of bin k needs bin N-k, which sits in row n1-k1; each row
// workgroup therefore takes such a pair of rows (rows 0 and n1/2 are their
// own mirrors and go together).
//
// Long convolution by FFT with zero padding (jisaku.com glossary
// "Hyena（ハイエナ）", section "計算効率"; gist.science HyenaND summary, section
// "手法: HyenaND", boundary handling); gating recurrence of the Hyena
// Hierarchy explainer, section "Hyena 演算子の形".
#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {

#ifndef HYENA_ROW_WAVES
#define HYENA_ROW_WAVES 1
#endif
#ifndef HYENA_COL_WAVES
#define HYENA_COL_WAVES 1
#endif


// Columns per workgroup.  Row convolutions: 2048 points per workgroup up to
// N1 = 64 (1-2% faster than 4096 on the 64K and 128K shapes), at most 64 KB
// of LDS from N1 = 256 on, so two workgroups share a CU and one's loads
// overlap the other's FFT, and never fewer than 16 (each row segment a
// whole 128-byte line).  Gate inputs requested before the inverse FFT where two workgroups
// share a CU (N1 = 256, 512: 5% faster); shorter columns run more workgroups
// per CU and lose more by the registers, and at 1024 it spills.  The grid
// passes (GRID) keep 32 columns up to N1 = 512 and no early gate loads: the
// row settings were 14% slower on a padded 224 x 224 grid.
template <int N1, bool GRID = false> struct ColCfg {
  static constexpr int E = 16;
  static constexpr int W = GRID ? (N1 == 16 ? 256 : N1 == 32 ? 128 : N1 == 64 ? 64 : N1 <= 512 ? 32 : 16)
                                : (N1 <= 64 ? 2048 / N1 : N1 <= 256 ? 32 : 16);
  static constexpr int T = W * N1 / E;
  static constexpr bool LDS = N1 > E;
  static constexpr int PFX = (!GRID && (N1 == 256 || N1 == 512)) ? E : 0;
  using R = typename Plan16<N1>::R;
};

#ifndef HYENA_ROW_E
#define HYENA_ROW_E 16
#endif

template <int N2> struct RowCfg {
  static constexpr int E = HYENA_ROW_E;
  static constexpr int TPR = N2 / E;  // threads per row
  static constexpr int T = 2 * TPR;
  using R = typename std::conditional<E == 16, typename Plan16<N2>::R,
                                      typename Plan8<(N2 <= 8192 ? N2 : 8192)>::R>::type;
};

// Intermediate accesses (each element is written by one pass and read back
// by the next, long after it left the caches).
#ifndef HYENA_WORK_NT
#define HYENA_WORK_NT 0
#endif
__device__ __forceinline__ cf ld_work(const cf* p) {
  if constexpr (HYENA_WORK_NT) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 w = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    return make_float2(w.x, w.y);
  } else {
    return *p;
  }
}
__device__ __forceinline__ void st_work(cf* p, cf v) {
  if constexpr (HYENA_WORK_NT) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(f32x2{v.x, v.y}, reinterpret_cast<f32x2*>(p));
  } else {
    *p = v;
  }
}

// COL_OUT: as COL_LAST without the gate (the plain causal convolution).
enum { COL_FIRST = 0, COL_MID = 1, COL_LAST = 2, COL_SPEC = 3, COL_OUT = 4 };
enum { ROW_CONV = 0, ROW_SPEC = 1 };

struct ColArgs {
  const void* v;       // FIRST: z_1 rows
  const void* xg;      // MID/LAST: gate x_n
  void* y;             // LAST: output
  const float* h;      // SPEC: filters [NF][L]
  cf* work;            // [group][n1][n2]
  int64_t L;
  int n2;
  int r0;              // first row of this launch
  int n_col_blocks;
  // grids (GRID kernels): a grid gL1 x gLm x gL2 per row (gLm = 1 for 2-D),
  // padded to n1 x (n1 x) 2*NL, columns col = i2*NL + m (m on the packed axis)
  int64_t gL1, gLm, gL2;
  int gNLs;            // log2 NL
  int gcirc;           // SPEC: kernel of the grid's shape (else extent 2L-1 per axis)
  int cmB, cmD;        // > 1: channel-major launch, see launch_row_of
};

// Activation row (b*D + d) of the launch's local row g.  Natural launches
// (cmB <= 1) cover rows r0, r0 + 1, ...; channel-major ones cover channels
// r0, r0 + 1, ... with their cmB batch rows next to each other (g = c*cmB + b),
// so the batch rows that share a channel's spectrum run in the same launch.
__device__ __forceinline__ int launch_row_of(int r0, int g, int cmB, int D) {
  if (cmB <= 1) return r0 + g;
  const int c = g / cmB;
  return (g - c * cmB) * D + r0 + c;
}

// Kernel index of padded position n on an axis of padded size P and grid
// side L (offset o at o mod P; non-circular index o + L - 1; -1: gap).
__device__ __forceinline__ int64_t grid_kidx(int64_t n, int64_t P, int64_t L, bool circ) {
  if (circ) return n;
  return n < L ? n + L - 1 : (n > P - L ? n - P + L - 1 : -1);
}

// Kernel value at padded-grid position (i1, i2, i3) of an n1 x Pm x P3 grid
// (2-D: Pm = Lm = 1, i2 = 0).
__device__ __forceinline__ float grid_kernel_at(const float* k, int64_t koff, int i1, int i2, int i3, int n1,
                                                int Pm, int P3, int64_t L1, int64_t Lm, int64_t L3, bool circ) {
  const int64_t a = grid_kidx(i1, n1, L1, circ);
  const int64_t b = Lm == 1 && Pm == 1 ? 0 : grid_kidx(i2, Pm, Lm, circ);
  const int64_t c = grid_kidx(i3, P3, L3, circ);
  const int64_t em = circ ? Lm : 2 * Lm - 1, e3 = circ ? L3 : 2 * L3 - 1;
  return (a >= 0 && b >= 0 && c >= 0) ? k[koff + (a * em + b) * e3 + c] : 0.f;
}

// GRID: each row is a 2-D grid gL1 x gL2 (row-major) zero-padded to
// n1 x 2*n2; the column FFT runs over the grid's first axis and no twiddle
// follows (a 2-D DFT), the packed column index col covering grid columns
// 2col, 2col+1.
template <int N1, int IOT, int KIND, bool EVEN, bool GRID = false>
__global__ void __launch_bounds__((ColCfg<N1, GRID>::T), HYENA_COL_WAVES) k_col(ColArgs a) {
  using C = ColCfg<N1, GRID>;
  constexpr int E = C::E, W = C::W, S1 = N1 / E;
  __shared__ cf smem[C::LDS ? N1 * W : 1];
  const int c = threadIdx.x % W, j = threadIdx.x / W;
  const int g = blockIdx.x / a.n_col_blocks, cb = blockIdx.x - g * a.n_col_blocks;
  const int col = cb * W + c;
  const bool valid = col < a.n2;
  const int64_t N = (int64_t)N1 * a.n2;
  cf* buf = a.work + (int64_t)g * N;
  const int64_t off = (int64_t)launch_row_of(a.r0, g, a.cmB, a.cmD) * (GRID ? a.gL1 * a.gLm * a.gL2 : a.L);
  const int gi2 = col >> a.gNLs, gm = col & ((1 << a.gNLs) - 1);     // GRID: column -> (i2, packed m)
  const ColLds<W> lds{smem + c};
  BlockFFT<N1, E, typename C::R> fft;
  fft.init(j);
  cf u[E];
  // element pair of column point i1: row offset, first real index, row length
  const auto at = [&](int i1, int64_t& ro, int64_t& t, int64_t& len) {
    if constexpr (GRID) {
      ro = off + ((int64_t)i1 * a.gLm + gi2) * a.gL2;
      t = 2 * (int64_t)gm;
      len = a.gL2;
      return valid && i1 < a.gL1 && gi2 < a.gLm;
    } else {
      ro = off;
      t = 2 * ((int64_t)a.n2 * i1 + col);
      len = a.L;
      return valid;
    }
  };

  if constexpr (KIND == COL_SPEC && GRID) {
    const int64_t e = a.gcirc ? a.gL1 * a.gLm * a.gL2 : (2 * a.gL1 - 1) * (2 * a.gLm - 1) * (2 * a.gL2 - 1);
    const int64_t koff = (int64_t)(a.r0 + g) * e;
    const int P3 = 2 << a.gNLs, Pm = a.gLm == 1 && (a.n2 >> a.gNLs) == 1 ? 1 : N1;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int i1 = j + i * S1;
      u[i] = make_float2(0.f, 0.f);
      if (valid)
        u[i] = make_float2(
            grid_kernel_at(a.h, koff, i1, gi2, 2 * gm, N1, Pm, P3, a.gL1, a.gLm, a.gL2, a.gcirc),
            grid_kernel_at(a.h, koff, i1, gi2, 2 * gm + 1, N1, Pm, P3, a.gL1, a.gLm, a.gL2, a.gcirc));
    }
  } else if constexpr (KIND == COL_FIRST || KIND == COL_SPEC) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      int64_t ro, t, len;
      const bool ok = at(j + i * S1, ro, t, len);
      u[i] = make_float2(0.f, 0.f);
      if (ok) {
        if constexpr (KIND == COL_SPEC) u[i] = ld_pair<0, EVEN>(a.h, ro, t, len);
        else u[i] = ld_pair<IOT, EVEN>(a.v, ro, t, len);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i)
      u[i] = valid ? ld_work(buf + (int64_t)(j + i * S1) * a.n2 + col) : make_float2(0.f, 0.f);
    constexpr int PFX = KIND == COL_OUT ? 0 : C::PFX;
    cf xp[PFX > 0 ? PFX : 1];
#pragma unroll
    for (int i = 0; i < PFX; ++i) {
      int64_t ro, t, len;
      xp[i] = at(j + i * S1, ro, t, len) ? ld_pair<IOT, EVEN>(a.xg, ro, t, len) : make_float2(0.f, 0.f);
    }
    fft.template run<true>(u, lds, j);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      int64_t ro, t, len;
      const bool ok = at(j + i * S1, ro, t, len);
      cf z = make_float2(0.f, 0.f);
      if (ok) {
        if constexpr (KIND == COL_OUT) {
          z = u[i];
        } else {
          const cf xv = i < PFX ? xp[i < PFX ? i : 0] : ld_pair<IOT, EVEN>(a.xg, ro, t, len);
          z = make_float2(xv.x * u[i].x, xv.y * u[i].y);
        }
        if constexpr (KIND == COL_LAST || KIND == COL_OUT) st_pair<IOT, EVEN>(a.y, ro, t, len, z);
      }
      u[i] = z;
    }
  }
  if constexpr (KIND != COL_LAST && KIND != COL_OUT) {
    fft.template run<false>(u, lds, j);
    if (valid) {
#pragma unroll
      for (int i = 0; i < E; ++i) st_work(buf + (int64_t)(j + i * S1) * a.n2 + col, u[i]);
    }
  }
}

struct RowArgs {
  cf* work;
  const cf* spec;      // CONV: spectrum (read)
  cf* spec_out;        // SPEC: spectrum (written)
  int n1;
  int64_t spec_stride;
  int order;           // CONV: order n (filters n*D + d)
  int D;
  int r0;              // first row (CONV: activation row b*D + d; SPEC: filter row)
  int n_row_pairs;     // n1 / 2
  int cmB;             // CONV, > 1: channel-major launch (r0 = first channel, cmB batch rows each)
};

// Spectrum layout on this path: row f holds S(k) = H(k)/(2N) at k1*n2 + k2
// for k = k1 + n1*k2 < N, and S(N) at index N.
template <int N2, int KIND>
__global__ void __launch_bounds__(RowCfg<N2>::T, HYENA_ROW_WAVES) k_row(RowArgs a) {
  using C = RowCfg<N2>;
  constexpr int E = C::E, TPR = C::TPR, S2 = N2 / E;
  constexpr int PADN = RowLds::padded(N2);
  __shared__ cf smem[2 * PADN];
  const int b = threadIdx.x / TPR, j = threadIdx.x - b * TPR;
  int g, w;
  if (KIND == ROW_CONV && a.cmB > 1) {
    // Channel-major launch: the cmB workgroups of one (channel, row pair)
    // read the same spectrum slice, so they are placed on one XCD (workgroup
    // i runs on XCD i mod 8) one after another, and the slice is fetched
    // into that XCD's L2 once.  n_row_pairs is a multiple of 8.
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int unit = (slot / a.cmB) * 8 + x, c = unit / a.n_row_pairs;
    w = unit - c * a.n_row_pairs;
    g = c * a.cmB + (slot - (slot / a.cmB) * a.cmB);
  } else {
    g = blockIdx.x / a.n_row_pairs;
    w = blockIdx.x - g * a.n_row_pairs;
  }
  const int n1 = a.n1;
  const int k1 = (b == 0) ? w : (w == 0 ? n1 / 2 : n1 - w);
  const bool self_mirror = (k1 == 0) || (2 * k1 == n1);
  const int mb = self_mirror ? b : 1 - b;          // row holding the mirror bins
  const int k1m = (k1 == 0) ? 0 : n1 - k1;         // its k1
  const uint32_t N = (uint32_t)n1 * (uint32_t)N2;
  cf* row = a.work + (int64_t)g * N + (int64_t)k1 * N2;
  const RowLds lds{smem + b * PADN};
  const RowLds ldsm{smem + mb * PADN};
  BlockFFT<N2, E, typename C::R> fft;
  fft.init(j);
  cf u[E];

  // four-step twiddle W_N^{k1 i2} for i2 = j + i*S2: base W_N^{k1 j} times
  // powers of the step W_N^{k1 S2}
  const cf tb = twiddle<false>((uint32_t)k1 * (uint32_t)j, N);
  const cf ts = twiddle<false>((uint32_t)k1 * (uint32_t)S2, N);
#pragma unroll
  for (int i = 0; i < E; ++i) u[i] = cmul(ld_work(row + j + i * S2), step_power<E>(tb, ts, i));
  fft.template run<false>(u, lds, j);

  // bins k = k1 + n1*k2 with k2 = j + i*S2; mirror N-k at (k1m, k2m)
  // W_{2N}^k = W_{2N}^{k1 + n1 j} * W_{2E}^i
  const cf wk = twiddle<false>((uint32_t)k1 + (uint32_t)n1 * (uint32_t)j, 2 * N);

  if constexpr (KIND == ROW_SPEC) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E; ++i) lds(j + i * S2) = u[i];
    __syncthreads();
    cf* out = a.spec_out + (int64_t)(a.r0 + g) * a.spec_stride;
    const float sc = 1.0f / (float)(2 * N);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k2 = j + i * S2;
      const int k2m = (k1 == 0) ? ((N2 - k2) & (N2 - 1)) : (N2 - 1 - k2);
      const cf am = ldsm(k2m);
      out[(int64_t)k1 * N2 + k2] = realfft_bin(u[i], am, cmul(wk, w2e<E>(i)), sc);
      if (k1 == 0 && k2 == 0) out[N] = make_float2((u[i].x - u[i].y) * sc, 0.f);   // Nyquist bin
    }
  } else {
    // Pair-wise spectral step: the owner of the low index i < E/2 of a bin
    // pair (k, N-k) computes both results; the partner bin is the high index
    // E-1-i of thread S2-1-j in the mirror row (row 0 pairs inside itself:
    // thread S2-j, or index E-i in thread 0; k = 0 and k = N/2 are their own
    // partners).
    const int d = (a.cmB > 1) ? a.r0 + g / a.cmB : (a.r0 + g) % a.D;
    const cf* gs = a.spec + (int64_t)(a.order * a.D + d) * a.spec_stride;
    const cf* gk = gs + (int64_t)k1 * N2;
    const cf* gmr = gs + (int64_t)k1m * N2;
    const cf wkb = opaque(wk);
    __syncthreads();
#pragma unroll
    for (int i = E / 2; i < E; ++i) lds(j + i * S2) = u[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      const int k2 = j + i * S2;
      if (k1 == 0 && i == 0 && j == 0) {
        u[0] = realconv_bin(u[0], u[0], gs[0], gs[N], make_float2(1.f, 0.f));
      } else {
        const int k2m = (k1 == 0) ? (N2 - k2) : (N2 - 1 - k2);
        cf bm = ldsm(k2m);
        realconv_pair(u[i], bm, gk[k2], gmr[k2m], cmul(wkb, w2e<E>(i)));
        ldsm(k2m) = bm;
      }
    }
    if (k1 == 0 && j == 0) {
      const cf am = lds(N2 / 2), gh = gs[N2 / 2];
      lds(N2 / 2) = realconv_bin(am, am, gh, gh, make_float2(0.f, -1.f));
    }
    __syncthreads();
#pragma unroll
    for (int i = E / 2; i < E; ++i) u[i] = lds(j + i * S2);
    fft.template run<true>(u, lds, j);
#pragma unroll
    for (int i = 0; i < E; ++i) st_work(row + j + i * S2, cmulc(u[i], step_power<E>(opaque(tb), opaque(ts), i)));
  }
}

// ---------------------------------------------------------------- launchers

template <int N1, bool EVEN, bool GRID>
static void launch_col_t(int kind, int io, const ColArgs& c, dim3 grid, dim3 block, hipStream_t s) {
  if (kind == COL_SPEC) {
    hipLaunchKernelGGL((k_col<N1, 0, COL_SPEC, EVEN, GRID>), grid, block, 0, s, c);
  } else if (kind == COL_OUT) {
    if constexpr (!GRID) hipLaunchKernelGGL((k_col<N1, 0, COL_OUT, EVEN, false>), grid, block, 0, s, c);
  } else if (io == 0) {
    if (kind == COL_FIRST) hipLaunchKernelGGL((k_col<N1, 0, COL_FIRST, EVEN, GRID>), grid, block, 0, s, c);
    else if (kind == COL_MID) hipLaunchKernelGGL((k_col<N1, 0, COL_MID, EVEN, GRID>), grid, block, 0, s, c);
    else hipLaunchKernelGGL((k_col<N1, 0, COL_LAST, EVEN, GRID>), grid, block, 0, s, c);
  } else {
    if (kind == COL_FIRST) hipLaunchKernelGGL((k_col<N1, 1, COL_FIRST, EVEN, GRID>), grid, block, 0, s, c);
    else if (kind == COL_MID) hipLaunchKernelGGL((k_col<N1, 1, COL_MID, EVEN, GRID>), grid, block, 0, s, c);
    else hipLaunchKernelGGL((k_col<N1, 1, COL_LAST, EVEN, GRID>), grid, block, 0, s, c);
  }
}

// Grid columns exist for the first axes the grid paths plan (2-D 256..1024,
// 3-D 64 and 128).
constexpr bool grid_col_ok(int n1) { return n1 >= 64; }

template <int N1>
static hipError_t launch_col(int kind, int io, const ColArgs& c, int groups, hipStream_t s, bool grid_mode = false) {
  const dim3 grid(groups * c.n_col_blocks), block(ColCfg<N1>::T);
  if (grid_mode) {
    const dim3 block(ColCfg<N1, true>::T);
    if constexpr (grid_col_ok(N1)) {
      if (c.gL2 % 2 == 0) launch_col_t<N1, true, true>(kind, io, c, grid, block, s);
      else launch_col_t<N1, false, true>(kind, io, c, grid, block, s);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (c.L % 2 == 0) {
    launch_col_t<N1, true, false>(kind, io, c, grid, block, s);
  } else {
    launch_col_t<N1, false, false>(kind, io, c, grid, block, s);
  }
  return hipGetLastError();
}

static int col_width(int n1, bool grid = false) {
  switch (n1) {
    case 16: return ColCfg<16>::W;
    case 32: return ColCfg<32>::W;
    case 64: return grid ? ColCfg<64, true>::W : ColCfg<64>::W;
    case 128: return grid ? ColCfg<128, true>::W : ColCfg<128>::W;
    case 256: return grid ? ColCfg<256, true>::W : ColCfg<256>::W;
    case 512: return grid ? ColCfg<512, true>::W : ColCfg<512>::W;
    case 1024: return grid ? ColCfg<1024, true>::W : ColCfg<1024>::W;
  }
  return 0;
}

static hipError_t dispatch_col(int n1, int kind, int io, const ColArgs& c, int groups, hipStream_t s,
                               bool grid_mode = false) {
  switch (n1) {
    case 16: return launch_col<16>(kind, io, c, groups, s, grid_mode);
    case 32: return launch_col<32>(kind, io, c, groups, s, grid_mode);
    case 64: return launch_col<64>(kind, io, c, groups, s, grid_mode);
    case 128: return launch_col<128>(kind, io, c, groups, s, grid_mode);
    case 256: return launch_col<256>(kind, io, c, groups, s, grid_mode);
    case 512: return launch_col<512>(kind, io, c, groups, s, grid_mode);
    case 1024: return launch_col<1024>(kind, io, c, groups, s, grid_mode);
  }
  return hipErrorInvalidValue;
}

template <int N2>
static hipError_t launch_row(int kind, const RowArgs& r, int groups, hipStream_t s) {
  const dim3 grid(groups * r.n_row_pairs), block(RowCfg<N2>::T);
  if (kind == ROW_SPEC) hipLaunchKernelGGL((k_row<N2, ROW_SPEC>), grid, block, 0, s, r);
  else hipLaunchKernelGGL((k_row<N2, ROW_CONV>), grid, block, 0, s, r);
  return hipGetLastError();
}

static hipError_t dispatch_row(int n2, int kind, const RowArgs& r, int groups, hipStream_t s) {
  switch (n2) {
    case 64: return launch_row<64>(kind, r, groups, s);
    case 128: return launch_row<128>(kind, r, groups, s);
    case 256: return launch_row<256>(kind, r, groups, s);
    case 512: return launch_row<512>(kind, r, groups, s);
    case 1024: return launch_row<1024>(kind, r, groups, s);
    case 2048: return launch_row<2048>(kind, r, groups, s);
    case 4096: return launch_row<4096>(kind, r, groups, s);
    case 8192: return launch_row<8192>(kind, r, groups, s);
  }
  return hipErrorInvalidValue;
}

hipError_t fourstep_forward(const ForwardArgs& a, const PlanInfo& p, hipStream_t s) {
  const int W = col_width(p.n1);
  if (W == 0) return hipErrorInvalidValue;
  ColArgs c{};
  c.v = a.v; c.y = a.y; c.h = nullptr; c.work = (cf*)a.work;
  c.L = a.L; c.n2 = p.n2;
  c.n_col_blocks = (p.n2 + W - 1) / W;
  RowArgs r{};
  r.work = (cf*)a.work; r.spec = (const cf*)a.spec; r.spec_out = nullptr;
  r.n1 = p.n1; r.spec_stride = a.spec_stride; r.D = a.D; r.n_row_pairs = p.n1 / 2;
  // With B > 1 a launch covers whole channels (all their batch rows), so the
  // row pass reads each channel's spectrum once instead of once per batch row.
  const bool cm = a.B > 1 && a.n_rows == a.B * a.D && a.rows_per_group >= a.B && r.n_row_pairs % 8 == 0;
  const int units = cm ? a.D : a.n_rows, per = cm ? a.rows_per_group / a.B : a.rows_per_group;
  c.cmB = r.cmB = cm ? a.B : 1;
  c.cmD = a.D;
  for (int r0 = 0; r0 < units; r0 += per) {
    const int groups = ((units - r0 < per) ? units - r0 : per) * (cm ? a.B : 1);
    c.r0 = r0; r.r0 = r0;
    hipError_t e = dispatch_col(p.n1, COL_FIRST, a.io, c, groups, s);
    if (e != hipSuccess) return e;
    for (int n = 0; n < a.NORD; ++n) {
      r.order = n;
      e = dispatch_row(p.n2, ROW_CONV, r, groups, s);
      if (e != hipSuccess) return e;
      c.xg = a.x.p[n];
      e = dispatch_col(p.n1, n < a.NORD - 1 ? COL_MID : (a.no_gate ? COL_OUT : COL_LAST), a.io, c, groups, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t fourstep_spectrum(const SpectrumArgs& a, const PlanInfo& p, hipStream_t s) {
  const int W = col_width(p.n1);
  if (W == 0) return hipErrorInvalidValue;
  ColArgs c{};
  c.h = a.h; c.work = (cf*)a.work; c.L = a.L; c.n2 = p.n2;
  c.n_col_blocks = (p.n2 + W - 1) / W;
  RowArgs r{};
  r.work = (cf*)a.work; r.spec_out = (cf*)a.spec; r.n1 = p.n1; r.spec_stride = a.spec_stride;
  r.n_row_pairs = p.n1 / 2;
  for (int r0 = 0; r0 < a.NF; r0 += a.rows_per_group) {
    const int groups = (a.NF - r0 < a.rows_per_group) ? a.NF - r0 : a.rows_per_group;
    c.r0 = r0; r.r0 = r0;
    hipError_t e = dispatch_col(p.n1, COL_SPEC, 0, c, groups, s);
    if (e != hipSuccess) return e;
    e = dispatch_row(p.n2, ROW_SPEC, r, groups, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------- 2-D grids, multi-pass
//
// A grid row (b, d) holds a gL1 x gL2 grid, zero-padded (or, circular,
// exactly) to P1 x P2 = n1 x 2*n2 and packed along its last axis into an
// n1 x n2 complex array: the column pass above (GRID) transforms the first
// axis, and the row kernel below transforms rows k1 and P1-k1 together --
// the row holding each bin's Hermitian partner (-k1, -k2) -- with no
// twiddle between the passes (a 2-D DFT).  Spectral step per bin, as on the
// single-pass grid path: C'(k) = A C(k) + i B conj C(k'), A = Pg - s Qg,
// B = c Qg from G = H(k)/M and G'' = H at the filter's partner (p = 0 pairs
// with the packed axis' Nyquist plane), (s, c) = (sin, cos)(pi k2 / n2).
// Spectrum layout: H/M at k1*n2 + k2, then the Nyquist plane at n1*n2 + k1.

template <int N2> struct GridRowCfg {
  static constexpr int E = 8;
  static constexpr int TPR = N2 / E;                        // threads per row
  static constexpr int RP = (2 * TPR >= 256) ? 1 : 256 / (2 * TPR);   // row pairs per workgroup
  static constexpr int T = RP * 2 * TPR;
  using R = typename Plan8<N2>::R;
};

struct GridRowArgs {
  cf* work;
  const cf* spec;
  cf* spec_out;
  int n1;
  int64_t spec_stride;
  int order, NORD, D, per_sample;
  int r0;
  int pairs_per_grid;   // n1 / 2
  int cmB;              // CONV, > 1: channel-major launch (r0 = first channel, cmB batch rows each)
};

template <int N2, int KIND>
__global__ void __launch_bounds__(GridRowCfg<N2>::T) k_grid_row(GridRowArgs a) {
  using C = GridRowCfg<N2>;
  constexpr int E = C::E, TPR = C::TPR, S2 = N2 / E;
  __shared__ cf smem[C::RP * 2 * N2];
  const int pr = threadIdx.x / (2 * TPR), tb = threadIdx.x - pr * 2 * TPR;
  const int b = tb / TPR, j = tb - b * TPR;
  int g, w;
  if (KIND == ROW_CONV && a.cmB > 1) {
    // channel-major launch: the cmB workgroups of one (channel, row pairs)
    // share the spectrum slice and run one after another on one XCD
    const int wpg = a.pairs_per_grid / C::RP;     // workgroups per grid, a multiple of 8
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int unit = (slot / a.cmB) * 8 + x, c = unit / wpg;
    g = c * a.cmB + (slot - (slot / a.cmB) * a.cmB);
    w = (unit - c * wpg) * C::RP + pr;
  } else {
    const int pair = blockIdx.x * C::RP + pr;
    g = pair / a.pairs_per_grid;
    w = pair - g * a.pairs_per_grid;
  }
  const int n1 = a.n1;
  const int k1 = (b == 0) ? w : (w == 0 ? n1 / 2 : n1 - w);
  const bool self_mirror = (k1 == 0) || (2 * k1 == n1);
  const int mb = self_mirror ? b : 1 - b;
  const int k1m = (n1 - k1) & (n1 - 1);
  const int64_t NC = (int64_t)n1 * N2;
  cf* row = a.work + (int64_t)g * NC + (int64_t)k1 * N2;
  const RowLds lds{smem + (pr * 2 + b) * N2};
  const RowLds ldsm{smem + (pr * 2 + mb) * N2};
  BlockFFT<N2, E, typename C::R> fft;
  fft.init(j);
  cf u[E];
#pragma unroll
  for (int i = 0; i < E; ++i) u[i] = row[j + i * S2];
  fft.template run<false>(u, lds, j);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) lds(j + i * S2) = u[i];
  __syncthreads();
  const cf wb = twiddle<false>((uint32_t)j, (uint32_t)(2 * N2));     // W_{2 n2}^{k2}, k2 = j + i*S2
  const float sc = 1.0f / (float)(2 * NC);
  if constexpr (KIND == ROW_SPEC) {
    cf* out = a.spec_out + (int64_t)(a.r0 + g) * a.spec_stride;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k2 = j + i * S2;
      const cf cm = ldsm((N2 - k2) & (N2 - 1));
      out[(int64_t)k1 * N2 + k2] = realfft_bin(u[i], cm, cmul(wb, w2e<E>(i)), sc);
      if (k2 == 0) out[NC + k1] = realfft_bin(u[i], cm, make_float2(-1.f, 0.f), sc);
    }
  } else {
    const int rowid = launch_row_of(a.r0, g, a.cmB, a.D), bb = rowid / a.D, d = rowid - bb * a.D;
    const int64_t f = a.per_sample ? ((int64_t)bb * a.NORD + a.order) * a.D + d : (int64_t)a.order * a.D + d;
    const cf* gs = a.spec + f * a.spec_stride;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k2 = j + i * S2;
      const cf cm = ldsm((N2 - k2) & (N2 - 1));
      const cf G = gs[(int64_t)k1 * N2 + k2];
      const cf Gm = (k2 == 0) ? gs[NC + k1m] : gs[(int64_t)k1m * N2 + (N2 - k2)];
      const cf wk = cmul(wb, w2e<E>(i));          // (c, -s)
      const float sn = -wk.y, cs = wk.x;
      const cf Pg = make_float2(G.x + Gm.x, G.y - Gm.y);
      const cf Qg = make_float2(G.x - Gm.x, G.y + Gm.y);
      const cf A = make_float2(fmaf(-sn, Qg.x, Pg.x), fmaf(-sn, Qg.y, Pg.y));
      const cf Bc = make_float2(cs * Qg.x, cs * Qg.y);
      const cf z = u[i];
      u[i] = make_float2(fmaf(A.x, z.x, fmaf(-A.y, z.y, fmaf(Bc.x, cm.y, -Bc.y * cm.x))),
                         fmaf(A.x, z.y, fmaf(A.y, z.x, fmaf(Bc.x, cm.x, Bc.y * cm.y))));
    }
    fft.template run<true>(u, lds, j);
#pragma unroll
    for (int i = 0; i < E; ++i) row[j + i * S2] = u[i];
  }
}

template <int N2>
static hipError_t launch_grid_row(int kind, const GridRowArgs& r, int groups, hipStream_t s) {
  using C = GridRowCfg<N2>;
  const int pairs = groups * r.pairs_per_grid;
  if (pairs % C::RP) return hipErrorInvalidValue;
  const dim3 grid(pairs / C::RP), block(C::T);
  if (kind == ROW_SPEC) hipLaunchKernelGGL((k_grid_row<N2, ROW_SPEC>), grid, block, 0, s, r);
  else hipLaunchKernelGGL((k_grid_row<N2, ROW_CONV>), grid, block, 0, s, r);
  return hipGetLastError();
}

static hipError_t dispatch_grid_row(int n2, int kind, const GridRowArgs& r, int groups, hipStream_t s) {
  switch (n2) {
    case 128: return launch_grid_row<128>(kind, r, groups, s);
    case 256: return launch_grid_row<256>(kind, r, groups, s);
    case 512: return launch_grid_row<512>(kind, r, groups, s);
  }
  return hipErrorInvalidValue;
}

hipError_t grid2d_forward(const NdArgs& a, hipStream_t s) {
  const int n1 = a.P, n2 = a.P / 2;
  const int W = col_width(n1, true);
  if (W == 0 || a.ndim != 2) return hipErrorInvalidValue;
  ColArgs c{};
  c.v = a.v; c.y = a.y; c.work = (cf*)a.work; c.n2 = n2;
  c.n_col_blocks = (n2 + W - 1) / W;
  c.gL1 = a.Lo; c.gLm = 1; c.gL2 = a.Ll; c.gNLs = ilog2(n2); c.gcirc = a.circular;
  GridRowArgs r{};
  r.work = (cf*)a.work; r.spec = (const cf*)a.spec; r.n1 = n1; r.spec_stride = a.spec_stride;
  r.NORD = a.NORD; r.D = a.D; r.per_sample = a.per_sample; r.pairs_per_grid = n1 / 2;
  // Shared kernels and B > 1: launches of whole channels, as in fourstep_forward.
  const int B = a.rows / a.D, tpr = n2 / 8, rp = (2 * tpr >= 256) ? 1 : 256 / (2 * tpr);
  const bool cm = !a.per_sample && B > 1 && a.rows == B * a.D && a.rows_per_group >= B &&
                  (n1 / 2) % (8 * rp) == 0;
  const int units = cm ? a.D : a.rows, per = cm ? a.rows_per_group / B : a.rows_per_group;
  c.cmB = r.cmB = cm ? B : 1;
  c.cmD = a.D;
  for (int r0 = 0; r0 < units; r0 += per) {
    const int groups = ((units - r0 < per) ? units - r0 : per) * (cm ? B : 1);
    c.r0 = r0; r.r0 = r0;
    hipError_t e = dispatch_col(n1, COL_FIRST, a.io, c, groups, s, true);
    if (e != hipSuccess) return e;
    for (int n = 0; n < a.NORD; ++n) {
      r.order = n;
      e = dispatch_grid_row(n2, ROW_CONV, r, groups, s);
      if (e != hipSuccess) return e;
      c.xg = a.x.p[n];
      e = dispatch_col(n1, n == a.NORD - 1 ? COL_LAST : COL_MID, a.io, c, groups, s, true);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t grid2d_spectrum(const NdArgs& a, hipStream_t s) {
  const int n1 = a.P, n2 = a.P / 2;
  const int W = col_width(n1, true);
  if (W == 0 || a.ndim != 2) return hipErrorInvalidValue;
  ColArgs c{};
  c.h = a.kernel; c.work = (cf*)a.work; c.n2 = n2;
  c.n_col_blocks = (n2 + W - 1) / W;
  c.gL1 = a.Lo; c.gLm = 1; c.gL2 = a.Ll; c.gNLs = ilog2(n2); c.gcirc = a.circular;
  GridRowArgs r{};
  r.work = (cf*)a.work; r.spec_out = (cf*)a.spec; r.n1 = n1; r.spec_stride = a.spec_stride;
  r.pairs_per_grid = n1 / 2;
  for (int r0 = 0; r0 < a.rows; r0 += a.rows_per_group) {
    const int groups = (a.rows - r0 < a.rows_per_group) ? a.rows - r0 : a.rows_per_group;
    c.r0 = r0; r.r0 = r0;
    hipError_t e = dispatch_col(n1, COL_SPEC, 0, c, groups, s, true);
    if (e != hipSuccess) return e;
    e = dispatch_grid_row(n2, ROW_SPEC, r, groups, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// 3-D grids, multi-pass: the column pass transforms the first axis (columns
// = (i2, m) of a P x P/2 plane), and the plane pass (kernels_nd.hip) takes
// planes k1 and P-k1 together through a 2-D FFT, the spectral step and back.
hipError_t grid3d_forward(const NdArgs& a, hipStream_t s) {
  const int P = a.P, NL = P / 2, n2 = P * NL;
  const int W = col_width(P, true);
  if (W == 0 || a.ndim != 3) return hipErrorInvalidValue;
  ColArgs c{};
  c.v = a.v; c.y = a.y; c.work = (cf*)a.work; c.n2 = n2;
  c.n_col_blocks = (n2 + W - 1) / W;
  c.gL1 = a.Lo; c.gLm = a.Lm; c.gL2 = a.Ll; c.gNLs = ilog2(NL); c.gcirc = a.circular;
  for (int r0 = 0; r0 < a.rows; r0 += a.rows_per_group) {
    const int groups = (a.rows - r0 < a.rows_per_group) ? a.rows - r0 : a.rows_per_group;
    c.r0 = r0;
    hipError_t e = dispatch_col(P, COL_FIRST, a.io, c, groups, s, true);
    if (e != hipSuccess) return e;
    for (int n = 0; n < a.NORD; ++n) {
      e = grid_plane_pass(a, r0, groups, n, false, s);
      if (e != hipSuccess) return e;
      c.xg = a.x.p[n];
      e = dispatch_col(P, n == a.NORD - 1 ? COL_LAST : COL_MID, a.io, c, groups, s, true);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t grid3d_spectrum(const NdArgs& a, hipStream_t s) {
  const int P = a.P, NL = P / 2, n2 = P * NL;
  const int W = col_width(P, true);
  if (W == 0 || a.ndim != 3) return hipErrorInvalidValue;
  ColArgs c{};
  c.h = a.kernel; c.work = (cf*)a.work; c.n2 = n2;
  c.n_col_blocks = (n2 + W - 1) / W;
  c.gL1 = a.Lo; c.gLm = a.Lm; c.gL2 = a.Ll; c.gNLs = ilog2(NL); c.gcirc = a.circular;
  for (int r0 = 0; r0 < a.rows; r0 += a.rows_per_group) {
    const int groups = (a.rows - r0 < a.rows_per_group) ? a.rows - r0 : a.rows_per_group;
    c.r0 = r0;
    hipError_t e = dispatch_col(P, COL_SPEC, 0, c, groups, s, true);
    if (e != hipSuccess) return e;
    e = grid_plane_pass(a, r0, groups, 0, true, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace hyena
