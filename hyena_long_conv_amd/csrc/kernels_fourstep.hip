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
#include "fft_odd.hpp"
#include "launch.hpp"

namespace hyena {

#ifndef HYENA_ROW_WAVES
#define HYENA_ROW_WAVES 1
#endif
// Points per workgroup of the column pass for columns of up to 64 points
// (its width W = HYENA_COL_POINTS / n1 columns).
#ifndef HYENA_COL_POINTS
#define HYENA_COL_POINTS 2048
#endif
// Gate loads of the middle and last column passes issued before the inverse
// column FFT (PFX points per thread): for 256- and 512-point columns, or for
// every length with HYENA_COL_PFX_ALL=1.
#ifndef HYENA_COL_PFX_ALL
#define HYENA_COL_PFX_ALL 0
#endif
// bf16 gate inputs of the first half of each column requested before the
// inverse column FFT where PFX does not apply.
#ifndef HYENA_COL_PFB
#define HYENA_COL_PFB 1
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
                                : (N1 <= 64 ? HYENA_COL_POINTS / N1 : N1 <= 256 ? 32 : 16);
  static constexpr int T = W * N1 / E;
  static constexpr bool LDS = N1 > E;
  static constexpr int PFX = (!GRID && (HYENA_COL_PFX_ALL || N1 == 256 || N1 == 512)) ? E : 0;
  using R = typename Plan16<N1>::R;
};

// Points per thread of the row pass: HYENA_ROW_E (16), except rows of up
// to 1024 points: HYENA_ROW_E_BF16 (8).  With a bf16 intermediate those
// passes move half the bytes and are bound by VALU issue; at 8 points per
// thread they ran 2% faster on the 64K and 1% on the 128K bf16 shapes, but
// 4% slower with 2048-point rows (L = 100000) and, with an fp32
// intermediate, 4% slower on the 1M shape (2048-point rows).  fp32 rows of
// up to 1024 points (HYENA_ROW_E8_F32) take 8 as well: the order-3 128K
// forward 2.7% and the 64K backward 2.2% faster.
#ifndef HYENA_ROW_E
#define HYENA_ROW_E 16
#endif
#ifndef HYENA_ROW_E_BF16
#define HYENA_ROW_E_BF16 8
#endif

#ifndef HYENA_ROW_E8_F32
#define HYENA_ROW_E8_F32 1
#endif
template <int N2, bool WB = false> struct RowCfg {
  static constexpr int E = ((WB || HYENA_ROW_E8_F32) && N2 <= 1024) ? HYENA_ROW_E_BF16 : HYENA_ROW_E;
  static constexpr int TPR = N2 / E;  // threads per row
  static constexpr int T = 2 * TPR;
  using R = typename std::conditional<E == 16, typename Plan16<N2>::R,
                                      typename Plan8<(N2 <= 8192 ? N2 : 8192)>::R>::type;
};

// Intermediate accesses (each element is written by one pass and read back
// by the next, long after it left the caches).  An element is one complex
// point: a float2, or with bf16 activations (WB) a pair of bf16 in 4 bytes
// (real part in the low half, rounded to nearest even), which halves the
// intermediate traffic of those forwards; the arithmetic stays fp32.
#ifndef HYENA_WORK_NT
#define HYENA_WORK_NT 0
#endif
template <bool WB> struct WorkElem { using T = cf; };
template <> struct WorkElem<true> { using T = uint32_t; };
template <bool WB> using work_t = typename WorkElem<WB>::T;

template <bool WB>
__device__ __forceinline__ cf ld_work(const work_t<WB>* p) {
  if constexpr (WB) {
    const uint32_t w = HYENA_WORK_NT ? __builtin_nontemporal_load(p) : *p;
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  } else if constexpr (HYENA_WORK_NT) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 w = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    return make_float2(w.x, w.y);
  } else {
    return *p;
  }
}
template <bool WB>
__device__ __forceinline__ void st_work(work_t<WB>* p, cf v) {
  if constexpr (WB) {
    if constexpr (HYENA_WORK_NT) __builtin_nontemporal_store(bf16x2_bits(v.x, v.y), p);
    else *p = bf16x2_bits(v.x, v.y);
  } else if constexpr (HYENA_WORK_NT) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(f32x2{v.x, v.y}, reinterpret_cast<f32x2*>(p));
  } else {
    *p = v;
  }
}

// Spectrum reads of the row pass.  Each slice is read once per forward (by
// one workgroup, or by the B consecutive workgroups of one XCD when batch
// rows share a channel), so the loads are nontemporal, like those of the
// activations: 7% faster than plain loads on the 1M shape, 1.5% on 64K.
#ifndef HYENA_SPEC_NT
#define HYENA_SPEC_NT 1
#endif
__device__ __forceinline__ cf ld_spec(const cf* p) {
  if constexpr (HYENA_SPEC_NT) {
    const f32x2 w = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    return make_float2(w.x, w.y);
  } else {
    return *p;
  }
}

// COL_OUT: as COL_LAST without the gate (the plain causal convolution).
// COL_MIDSAVE: as COL_MID, and the ungated convolution is stored too (fp32,
// to y).  COL_FIRSTG: as COL_FIRST with the input formed as x * c (x = xg
// in the activation type, c = v in fp32).  COL_SPECG / COL_SPECGF: a
// spectrum's first pass whose rows are g * x (g = v in the activation type /
// in fp32, x = xg), also storing g * c to y (c = h, fp32; y in the
// activation type).  COL_OUTREV: as COL_OUT, the row stored reversed,
// t -> (rev_c - t) mod L.  These serve the backward.
// ROW_SMUL: the row pass of a convolution whose input rows are given by
// their spectra (the ROW_SPEC layout) instead of a column-transformed
// intermediate; no column pass precedes it.
enum { COL_FIRST = 0, COL_MID = 1, COL_LAST = 2, COL_SPEC = 3, COL_OUT = 4, COL_MIDSAVE = 5, COL_FIRSTG = 6,
       COL_SPECG = 7, COL_SPECGF = 8, COL_OUTREV = 9 };
enum { ROW_CONV = 0, ROW_SPEC = 1, ROW_SMUL = 2 };

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
  int64_t rev_c;       // OUTREV: position t is stored at (rev_c - t) mod L
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
// Column-pass activation type: IOT 0 fp32, 1 bf16, 2 bf16 with the
// intermediate kept as bf16 pairs.
constexpr int io_of(int iot) { return iot == 2 ? 1 : iot; }

// COL_SPECG/F: the g * c stores after the column FFT's stores (1) or before
// the FFT (0; 1M backward 16.83 against 16.96 ms, 64K 2.776 against 2.789).
#ifndef HYENA_SPECG_LATE
#define HYENA_SPECG_LATE 1
#endif

// COL_OUTREV store of the pair at position t (even) of a row of length L:
// t -> (rev_c - t) mod L.  With L even and rev_c = L - 1 the mirrored pair
// (L-2-t, L-1-t) is one aligned 8-byte store; otherwise (odd L, periodic
// rows) two 4-byte stores.
template <bool EVEN>
__device__ __forceinline__ void st_pair_rev(void* y, int64_t off, int64_t t, int64_t L, int64_t rev_c, cf z) {
  if (EVEN && (rev_c & 1) && rev_c == L - 1) {
    if (t < L) {
      const f32x2 w = {z.y, z.x};
      __builtin_nontemporal_store(w, reinterpret_cast<f32x2*>(static_cast<float*>(y) + off + (L - 2 - t)));
    }
    return;
  }
  int64_t q0 = rev_c - t, q1 = q0 - 1;
  if (q0 < 0) q0 += L;
  if (q1 < 0) q1 += L;
  if (t < L) IO<0>::st(y, off + q0, z.x);
  if (t + 1 < L) IO<0>::st(y, off + q1, z.y);
}

template <int N1, int IOT, int KIND, bool EVEN, bool GRID = false>
__global__ void __launch_bounds__((ColCfg<N1, GRID>::T), HYENA_COL_WAVES) k_col(ColArgs a) {
  using C = ColCfg<N1, GRID>;
  constexpr bool OUTK = KIND == COL_OUT || KIND == COL_OUTREV;   // ungated output passes
  constexpr int E = C::E, W = C::W, S1 = N1 / E;
  __shared__ cf smem[C::LDS ? N1 * W : 1];
  const int c = threadIdx.x % W, j = threadIdx.x / W;
  const int g = blockIdx.x / a.n_col_blocks, cb = blockIdx.x - g * a.n_col_blocks;
  const int col = cb * W + c;
  const bool valid = col < a.n2;
  const int64_t N = (int64_t)N1 * a.n2;
  constexpr bool WB = IOT == 2;                      // bf16 intermediate (bf16 activations, low orders)
  work_t<WB>* buf = reinterpret_cast<work_t<WB>*>(a.work) + (int64_t)g * N;
  const int64_t off = (int64_t)launch_row_of(a.r0, g, a.cmB, a.cmD) * (GRID ? a.gL1 * a.gLm * a.gL2 : a.L);
  const int gi2 = col >> a.gNLs, gm = col & ((1 << a.gNLs) - 1);     // GRID: column -> (i2, packed m)
  const ColLds<W> lds{smem + c};
  BlockFFT<N1, E, typename C::R> fft;
  fft.init(j);
  cf u[E];
  // Loads of row passes (not GRID) run unconditionally, from in-range
  // addresses: lanes past the last column work on column 0 (columns never
  // mix, and those lanes store nothing) and positions past the row end read
  // its last pair, masked to zero (CLAMP).  A branch around a load whose
  // value is converted before the branch ends makes the wave wait for each
  // load before it issues the next one.
  const int colc = valid ? col : 0;
  // element pair of column point i1: row offset, first real index, row length
  const auto at = [&](int i1, int64_t& ro, int64_t& t, int64_t& len) {
    if constexpr (GRID) {
      ro = off + ((int64_t)i1 * a.gLm + gi2) * a.gL2;
      t = 2 * (int64_t)gm;
      len = a.gL2;
      return valid && i1 < a.gL1 && gi2 < a.gLm;
    } else {
      ro = off;
      t = 2 * ((int64_t)a.n2 * i1 + colc);
      len = a.L;
      return valid;
    }
  };
  // activation pair of column point i1 (zero where at() fails)
  const auto act = [&](const void* p, int i1) {
    int64_t ro, t, len;
    const bool ok = at(i1, ro, t, len);
    if constexpr (GRID) {
      return ok ? ld_pair<io_of(IOT), EVEN>(p, ro, t, len) : make_float2(0.f, 0.f);
    } else {
      (void)ok;
      return ld_pair<io_of(IOT), EVEN, true>(p, ro, t, len);
    }
  };
  constexpr bool SPECG = KIND == COL_SPECG || KIND == COL_SPECGF;
  cf gc[SPECG ? E : 1];   // SPECG: g * c of the column's points
  const auto store_gc = [&]() {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      int64_t ro, t, len;
      if (at(j + i * S1, ro, t, len)) st_pair<io_of(IOT), EVEN>(a.y, ro, t, len, gc[SPECG ? i : 0]);
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
  } else if constexpr (SPECG) {
    // all loads of the column first, then the stores of g * c (after the
    // column FFT's stores with HYENA_SPECG_LATE)
    constexpr int GT = KIND == COL_SPECGF ? 0 : io_of(IOT);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      int64_t ro, t, len;
      at(j + i * S1, ro, t, len);
      const cf gv = ld_pair<GT, EVEN, true>(a.v, ro, t, len), cv = ld_pair<0, EVEN, true>(a.h, ro, t, len);
      const cf xv = act(a.xg, j + i * S1);
      gc[i] = make_float2(gv.x * cv.x, gv.y * cv.y);
      u[i] = make_float2(gv.x * xv.x, gv.y * xv.y);
    }
    if constexpr (!HYENA_SPECG_LATE) store_gc();
  } else if constexpr (KIND == COL_FIRST || KIND == COL_SPEC || KIND == COL_FIRSTG) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if constexpr (KIND == COL_SPEC) {
        int64_t ro, t, len;
        at(j + i * S1, ro, t, len);
        u[i] = ld_pair<0, EVEN, true>(a.h, ro, t, len);
      } else if constexpr (KIND == COL_FIRSTG) {
        int64_t ro, t, len;
        at(j + i * S1, ro, t, len);
        const cf cv = ld_pair<0, EVEN, true>(a.v, ro, t, len), xv = act(a.xg, j + i * S1);
        u[i] = make_float2(xv.x * cv.x, xv.y * cv.y);
      } else {
        u[i] = act(a.v, j + i * S1);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if constexpr (GRID) {   // (unmasked, these loads held 40 more registers and spilled at n1 = 512)
        u[i] = valid ? ld_work<WB>(buf + (int64_t)(j + i * S1) * a.n2 + col) : make_float2(0.f, 0.f);
      } else {
        u[i] = ld_work<WB>(buf + (int64_t)(j + i * S1) * a.n2 + colc);
      }
    }
    constexpr int PFX = OUTK ? 0 : C::PFX;
    cf xp[PFX > 0 ? PFX : 1];
    // (the column's second half holds samples only on circular rows)
#pragma unroll
    for (int i = 0; i < PFX; ++i) xp[i] = (GRID || i < E / 2) ? act(a.xg, j + i * S1) : make_float2(0.f, 0.f);
    if (!GRID && a.L > N) {
#pragma unroll
      for (int i = E / 2; i < PFX; ++i) xp[i] = act(a.xg, j + i * S1);
    }
    // bf16 gates of the first half of the column (on a zero-padded row the
    // only points that hold samples) requested before the inverse FFT too,
    // kept packed: one register per point.
    constexpr int PFB = (OUTK || PFX > 0 || GRID || io_of(IOT) != 1 || !HYENA_COL_PFB) ? 0 : E / 2;
    uint32_t xb[PFB > 0 ? PFB : 1];
#pragma unroll
    for (int i = 0; i < PFB; ++i) {
      int64_t ro, t, len;
      at(j + i * S1, ro, t, len);
      xb[i] = ld_pair_bits<EVEN>(a.xg, ro, t, len);
    }
    fft.template run<true>(u, lds, j);
    // the other gates (not GRID): requested together, then pinned; points of
    // the column's second half hold samples only on circular rows
    constexpr int G0 = (GRID || OUTK) ? E : (PFX > PFB ? PFX : PFB);
    RawPair<io_of(IOT)> xl[G0 < E ? E - G0 : 1];
    if constexpr (G0 < E) {
      const auto ld_gate = [&](int i) {
        int64_t ro, t, len;
        at(j + i * S1, ro, t, len);
        xl[i - G0] = ld_pair_raw<io_of(IOT), EVEN>(a.xg, ro, t, len);
      };
#pragma unroll
      for (int i = G0; i < E; ++i) {
        if (i < E / 2) ld_gate(i);
        else xl[i - G0] = RawPair<io_of(IOT)>{};
      }
      if (a.L > N) {
#pragma unroll
        for (int i = (G0 > E / 2 ? G0 : E / 2); i < E; ++i) ld_gate(i);
      }
#pragma unroll
      for (int i = G0; i < E; ++i) pin(xl[i - G0]);
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      int64_t ro, t, len;
      const bool ok = at(j + i * S1, ro, t, len);
      cf z = u[i];
      if constexpr (GRID) {   // grid passes: the gate and the store under the point's mask
        z = make_float2(0.f, 0.f);
        if (ok) {
          if constexpr (KIND == COL_OUT) {
            z = u[i];
          } else {
            const cf xv = ld_pair<io_of(IOT), EVEN>(a.xg, ro, t, len);
            z = make_float2(xv.x * u[i].x, xv.y * u[i].y);
          }
          if constexpr (KIND == COL_LAST || KIND == COL_OUT) st_pair<io_of(IOT), EVEN>(a.y, ro, t, len, z);
        }
      } else {
        if constexpr (KIND == COL_MIDSAVE) {
          if (ok) st_pair<0, EVEN>(a.y, ro, t, len, z);
        }
        if constexpr (!OUTK) {
          const cf xv = i < PFX   ? xp[i < PFX ? i : 0]
                        : i < PFB ? bf16_pair_cf(xb[i < PFB ? i : 0])
                                  : unpack(xl[i >= G0 && i - G0 < E ? i - G0 : 0]);
          z = make_float2(xv.x * z.x, xv.y * z.y);
        }
        if constexpr (KIND == COL_LAST || KIND == COL_OUT) {
          if (ok) st_pair<io_of(IOT), EVEN>(a.y, ro, t, len, z);
        }
        if constexpr (KIND == COL_OUTREV) {   // fp32 rows, t -> (rev_c - t) mod L
          if (ok) st_pair_rev<EVEN>(a.y, ro, t, len, a.rev_c, z);
        }
      }
      u[i] = z;
    }
  }
  if constexpr (KIND != COL_LAST && !OUTK) {
    fft.template run<false>(u, lds, j);
    if (valid) {
#pragma unroll
      for (int i = 0; i < E; ++i) st_work<WB>(buf + (int64_t)(j + i * S1) * a.n2 + col, u[i]);
    }
  }
  if constexpr (SPECG && HYENA_SPECG_LATE) store_gc();
}

// Column pass for odd column lengths (n1 in 3, 5, 9, 15, 25, 27: FFT
// lengths 2^a 3^b 5^c, fft_odd.hpp): one thread per column holds the whole
// n1-point column in registers, so the pass needs no LDS and no barrier.
// A wave covers 64 consecutive columns, i.e. 512-byte runs of every row of
// the intermediate.  Same kinds and arguments as k_col (no grids).
constexpr int kColOddThreads = 128;
// Gate loads of these passes go out in batches of this many points: a batch
// is in flight together, and the registers it holds stay bounded.
#ifndef HYENA_GATE_BATCH
#define HYENA_GATE_BATCH 8
#endif
constexpr int kGateBatch = HYENA_GATE_BATCH;

// The same pointer, hidden from common-subexpression elimination: the stores
// at the end of a column pass then recompute their addresses instead of
// keeping the loads' (one 64-bit address per point) live through the DFTs.
template <class T>
__device__ __forceinline__ T* fresh_ptr(T* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+v"(v));
  return reinterpret_cast<T*>(v);
}

// First pass of the backward's fused spectrum (COL_SPECG/F) on one lane's
// points: u[m] = g x, and g c stored to y, for the pair positions pos(m) of
// row offset off.  Loads go out in batches of kGateBatch points, pinned
// before the batch's stores, so a batch stays in flight together.
template <int NP, int IOT, int KIND, bool EVEN, class Pos>
__device__ __forceinline__ void specg_points(const ColArgs& a, int64_t off, cf (&u)[NP], Pos pos) {
  constexpr int GT = KIND == COL_SPECGF ? 0 : io_of(IOT);
#pragma unroll
  for (int m0 = 0; m0 < NP; m0 += kGateBatch) {
    RawPair<GT> gr[kGateBatch];
    RawPair<0> cr[kGateBatch];
    RawPair<io_of(IOT)> xr[kGateBatch];
#pragma unroll
    for (int k = 0; k < kGateBatch; ++k) {
      if (m0 + k < NP) {
        gr[k] = ld_pair_raw<GT, EVEN>(a.v, off, pos(m0 + k), a.L);
        cr[k] = ld_pair_raw<0, EVEN>(a.h, off, pos(m0 + k), a.L);
        xr[k] = ld_pair_raw<io_of(IOT), EVEN>(a.xg, off, pos(m0 + k), a.L);
      }
    }
#pragma unroll
    for (int k = 0; k < kGateBatch; ++k) {
      if (m0 + k < NP) { pin<GT, true>(gr[k]); pin<0, true>(cr[k]); pin<io_of(IOT), true>(xr[k]); }
    }
#pragma unroll
    for (int k = 0; k < kGateBatch; ++k) {
      if (m0 + k < NP) {
        const cf gv = unpack(gr[k]), cv = unpack(cr[k]), xv = unpack(xr[k]);
        u[m0 + k] = make_float2(gv.x * xv.x, gv.y * xv.y);
        st_pair<io_of(IOT), EVEN>(a.y, off, pos(m0 + k), a.L, make_float2(gv.x * cv.x, gv.y * cv.y));
      }
    }
  }
}

template <int N1, int IOT, int KIND, bool EVEN>
__global__ void __launch_bounds__(kColOddThreads) k_col_odd(ColArgs a) {
  const int g = blockIdx.x / a.n_col_blocks, cb = blockIdx.x - g * a.n_col_blocks;
  const int col = cb * kColOddThreads + (int)threadIdx.x;
  if (col >= a.n2) return;
  const int64_t N = (int64_t)N1 * a.n2;
  constexpr bool WB = IOT == 2;                      // bf16 intermediate (bf16 activations, low orders)
  work_t<WB>* buf = reinterpret_cast<work_t<WB>*>(a.work) + (int64_t)g * N + col;
  const int64_t off = (int64_t)launch_row_of(a.r0, g, a.cmB, a.cmD) * a.L;
  cf u[N1];
  constexpr bool OUTK = KIND == COL_OUT || KIND == COL_OUTREV;   // ungated output passes
  if constexpr (KIND == COL_SPECG || KIND == COL_SPECGF) {
    specg_points<N1, IOT, KIND, EVEN>(a, off, u, [&](int i) { return 2 * ((int64_t)a.n2 * i + col); });
  } else if constexpr (KIND == COL_FIRST || KIND == COL_SPEC || KIND == COL_FIRSTG) {
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      const int64_t t = 2 * ((int64_t)a.n2 * i + col);
      if constexpr (KIND == COL_SPEC) {
        u[i] = ld_pair<0, EVEN, true>(a.h, off, t, a.L);
      } else if constexpr (KIND == COL_FIRSTG) {
        const cf cv = ld_pair<0, EVEN, true>(a.v, off, t, a.L), xv = ld_pair<io_of(IOT), EVEN, true>(a.xg, off, t, a.L);
        u[i] = make_float2(xv.x * cv.x, xv.y * cv.y);
      } else {
        u[i] = ld_pair<io_of(IOT), EVEN, true>(a.v, off, t, a.L);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < N1; ++i) u[i] = ld_work<WB>(buf + (int64_t)i * a.n2);
    RegDft<N1, true>::run(u);
    RawPair<io_of(IOT)> xl[N1];
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      const int64_t t = 2 * ((int64_t)a.n2 * i + col);
      if constexpr (!OUTK) {
        if (i % kGateBatch == 0) {   // the batch's gates requested together, then pinned
#pragma unroll
          for (int k = i; k < i + kGateBatch && k < N1; ++k)
            xl[k] = ld_pair_raw<io_of(IOT), EVEN>(a.xg, off, 2 * ((int64_t)a.n2 * k + col), a.L);
#pragma unroll
          for (int k = i; k < i + kGateBatch && k < N1; ++k) pin<io_of(IOT), true>(xl[k]);
        }
      }
      cf z = u[i];
      if constexpr (KIND == COL_MIDSAVE) st_pair<0, EVEN>(a.y, off, t, a.L, z);
      if constexpr (!OUTK) {
        const cf xv = unpack(xl[i]);
        z = make_float2(xv.x * z.x, xv.y * z.y);
      }
      if constexpr (KIND == COL_LAST || KIND == COL_OUT) st_pair<io_of(IOT), EVEN>(a.y, off, t, a.L, z);
      if constexpr (KIND == COL_OUTREV) st_pair_rev<EVEN>(a.y, off, t, a.L, a.rev_c, z);
      u[i] = z;
    }
  }
  if constexpr (KIND != COL_LAST && !OUTK) {
    RegDft<N1, false>::run(u);
    work_t<WB>* dst = fresh_ptr(buf);
#pragma unroll
    for (int i = 0; i < N1; ++i) st_work<WB>(dst + (int64_t)i * a.n2, u[i]);
  }
}

// Column pass for column lengths n1 = 2q (q odd, as above): the two lanes
// of a lane pair (lane bit 0 = a) share a column, q points each, so rows stay
// at most 2048 points (the 4096-point row pass ran 11% slower per point).
// Forward DFT of a column whose lane a holds the interleaved samples
// x[a + 2m] (m < q):  Y_a = DFT_q(x[a + 2m]),  Y_a[k] *= W_2q^(a k),  then the
// 2-point DFT across the pair, X[k + q a] = Y_0[k] + (-1)^a Y_1[k], leaves
// the contiguous half X[q a + k] in lane a.  The inverse runs the same steps
// backwards (2-point DFT across the pair, conjugate twiddle, inverse DFT_q),
// returning the interleaved samples, so every pass reads what the previous
// one wrote.  The exchange is one DPP quad permutation per float (lanes
// 2i <-> 2i+1); no LDS, no barrier.
__device__ __forceinline__ float swap_lane_pair(float v) {
  // quad_perm [1, 0, 3, 2]: each lane reads its pair partner
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

// X = partner + s * own for both components (s = +1 in lane 0 of the pair, -1 in lane 1)
__device__ __forceinline__ cf cross_pair(cf v, float s) {
  const float px = swap_lane_pair(v.x), py = swap_lane_pair(v.y);
  return make_float2(fmaf(s, v.x, px), fmaf(s, v.y, py));
}

template <int Q, bool INV, int K>
__device__ __forceinline__ void pair_twiddle_one(cf* u, bool odd_lane) {
  if constexpr (K != 0) {
    const cf w = wconst<K, 2 * Q, INV>();
    const cf t = cmul(u[K], w);
    u[K] = odd_lane ? t : u[K];
  }
}
template <int Q, bool INV, int... K>
__device__ __forceinline__ void pair_twiddle(cf* u, bool odd_lane, std::integer_sequence<int, K...>) {
  (pair_twiddle_one<Q, INV, K>(u, odd_lane), ...);
}

// forward: interleaved samples in, contiguous half of the spectrum out
template <int Q>
__device__ __forceinline__ void pair_dft_fwd(cf (&u)[Q], int a) {
  RegDft<Q, false>::run(u);
  pair_twiddle<Q, false>(u, a != 0, std::make_integer_sequence<int, Q>{});
  const float s = a ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < Q; ++k) u[k] = cross_pair(u[k], s);
}

// inverse (unnormalised): contiguous half in, interleaved samples out
template <int Q>
__device__ __forceinline__ void pair_dft_inv(cf (&u)[Q], int a) {
  const float s = a ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < Q; ++k) u[k] = cross_pair(u[k], s);
  pair_twiddle<Q, true>(u, a != 0, std::make_integer_sequence<int, Q>{});
  RegDft<Q, true>::run(u);
}

template <int Q, int IOT, int KIND, bool EVEN>
__global__ void __launch_bounds__(kColOddThreads) k_col_pair(ColArgs a) {
  constexpr int CPB = kColOddThreads / 2;   // columns per workgroup
  const int g = blockIdx.x / a.n_col_blocks, cb = blockIdx.x - g * a.n_col_blocks;
  const int lane_a = (int)threadIdx.x & 1;
  const int col = cb * CPB + ((int)threadIdx.x >> 1);
  if (col >= a.n2) return;                  // both lanes of a pair leave together
  const int64_t N = (int64_t)(2 * Q) * a.n2;
  constexpr bool WB = IOT == 2;                      // bf16 intermediate (bf16 activations, low orders)
  work_t<WB>* buf = reinterpret_cast<work_t<WB>*>(a.work) + (int64_t)g * N + col;
  const int64_t off = (int64_t)launch_row_of(a.r0, g, a.cmB, a.cmD) * a.L;
  // time row of point m: lane_a + 2m;  spectrum row of point k: Q*lane_a + k
  const auto trow = [&](int m) { return 2 * ((int64_t)a.n2 * (lane_a + 2 * m) + col); };
  cf u[Q];
  constexpr bool OUTK = KIND == COL_OUT || KIND == COL_OUTREV;   // ungated output passes
  if constexpr (KIND == COL_SPECG || KIND == COL_SPECGF) {
    specg_points<Q, IOT, KIND, EVEN>(a, off, u, trow);
  } else if constexpr (KIND == COL_FIRST || KIND == COL_SPEC || KIND == COL_FIRSTG) {
#pragma unroll
    for (int m = 0; m < Q; ++m) {
      if constexpr (KIND == COL_SPEC) {
        u[m] = ld_pair<0, EVEN, true>(a.h, off, trow(m), a.L);
      } else if constexpr (KIND == COL_FIRSTG) {
        const cf cv = ld_pair<0, EVEN, true>(a.v, off, trow(m), a.L);
        const cf xv = ld_pair<io_of(IOT), EVEN, true>(a.xg, off, trow(m), a.L);
        u[m] = make_float2(xv.x * cv.x, xv.y * cv.y);
      } else {
        u[m] = ld_pair<io_of(IOT), EVEN, true>(a.v, off, trow(m), a.L);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < Q; ++k) u[k] = ld_work<WB>(buf + (int64_t)(Q * lane_a + k) * a.n2);
    pair_dft_inv<Q>(u, lane_a);
    RawPair<io_of(IOT)> xl[Q];
#pragma unroll
    for (int m = 0; m < Q; ++m) {
      if constexpr (!OUTK) {
        if (m % kGateBatch == 0) {   // the batch's gates requested together, then pinned
#pragma unroll
          for (int k = m; k < m + kGateBatch && k < Q; ++k) xl[k] = ld_pair_raw<io_of(IOT), EVEN>(a.xg, off, trow(k), a.L);
#pragma unroll
          for (int k = m; k < m + kGateBatch && k < Q; ++k) pin<io_of(IOT), true>(xl[k]);
        }
      }
      cf z = u[m];
      if constexpr (KIND == COL_MIDSAVE) st_pair<0, EVEN>(a.y, off, trow(m), a.L, z);
      if constexpr (!OUTK) {
        const cf xv = unpack(xl[m]);
        z = make_float2(xv.x * z.x, xv.y * z.y);
      }
      if constexpr (KIND == COL_LAST || KIND == COL_OUT) st_pair<io_of(IOT), EVEN>(a.y, off, trow(m), a.L, z);
      if constexpr (KIND == COL_OUTREV) st_pair_rev<EVEN>(a.y, off, trow(m), a.L, a.rev_c, z);
      u[m] = z;
    }
  }
  if constexpr (KIND != COL_LAST && !OUTK) {
    pair_dft_fwd<Q>(u, lane_a);
    work_t<WB>* dst = fresh_ptr(buf + (int64_t)Q * lane_a * a.n2);
#pragma unroll
    for (int k = 0; k < Q; ++k) st_work<WB>(dst + (int64_t)k * a.n2, u[k]);
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
  int n_row_pairs;     // workgroups per row: n1 / 2 (even n1) or (n1 + 1) / 2 (odd n1)
  int cmB;             // CONV, > 1: channel-major launch (r0 = first channel, cmB batch rows each)
  int n_units;         // channel-major launch: (channel, row pair) units; the grid is padded to a multiple of 8
  int wb;              // CONV: the intermediate holds bf16 pairs (bf16 activations)
  const cf* spec_in;   // SMUL: spectra of the input rows, one per activation row (ROW_SPEC layout)
  int rev;             // SPEC: spectrum of the row reversal t -> (rev_c - t) mod 2N; SMUL: output reversed so
  int64_t rev_c;
};

// W_{2N}^(c k) for the thread's bins k = k1 + n1 (j + i S2), i < E: the
// spectrum of a row reversal t -> (c - t) mod 2N is W^(c k) conj X(k).
template <int E>
struct RevTwiddle {
  cf st, p;   // step W^(c n1 S2); the running power W^(c k_i)
  __device__ __forceinline__ RevTwiddle(int64_t c, int k1, int n1, int j, int S2, uint32_t M) {
    const uint64_t kb = (uint64_t)k1 + (uint64_t)n1 * (uint64_t)j, ks = (uint64_t)n1 * (uint64_t)S2;
    p = twiddle<false>((uint32_t)(((uint64_t)c * kb) % M), M);
    st = twiddle<false>((uint32_t)(((uint64_t)c * ks) % M), M);
  }
  // W^(c k_i) conj v for the thread's points in order i = 0, 1, ...: the
  // power by a running product, as the four-step twiddles with
  // HYENA_ROW_TW_SEQ
  __device__ __forceinline__ cf apply_next(cf v) {
    const cf r = cmul(p, cconj(v));
    p = cmul(p, st);
    return r;
  }
};

// Four-step twiddles of the row pass, W_N^{k1 i2} for the thread's points
// i2 = j + i*S2: the base W_N^{k1 j} times the i-th power of the step
// W_N^{k1 S2}, the powers by repeated multiplication (HYENA_ROW_TW_SEQ = 1:
// E - 1 products, rounding growing with i up to ~E ulp) or by binary
// powers (0: about twice the products for E = 16).
#ifndef HYENA_ROW_TW_SEQ
#define HYENA_ROW_TW_SEQ 1
#endif

// LDS of the row pass.  HYENA_ROW_SW: 0 plain addressing; 1 XOR-swizzled
// FFT stage buffers (RowLdsT<true>); 2 one padding slot after every 16
// points, for every access (the first stage's stores, 16 points apart per
// lane, then spread over the banks at the cost of a shift and an add).
// Plain is the default: the pass keeps the VALU ~81% busy, and the other two
// remove the bank conflicts (1.4 -> 0.02 / 0.3 per access) at the cost of
// registers and address arithmetic, measured 14% and 1-2% slower.
#ifndef HYENA_ROW_SW
#define HYENA_ROW_SW 0
#endif
struct RowLdsPad16 {
  cf* base;
  static constexpr __host__ __device__ int padded(int npt) { return npt + npt / 16; }
  template <int SH>
  __device__ __forceinline__ cf& at(int i) const { return base[i + (i >> 4)]; }
  __device__ __forceinline__ cf& operator()(int i) const { return base[i + (i >> 4)]; }
};
using RowPassLds = std::conditional<HYENA_ROW_SW == 2, RowLdsPad16, RowLdsT<HYENA_ROW_SW == 1>>::type;

// Spectrum layout on this path: row f holds S(k) = H(k)/(2N) at k1*n2 + k2
// for k = k1 + n1*k2 < N, and S(N) at index N.
template <int N2, int KIND, bool WB = false>
__global__ void __launch_bounds__((RowCfg<N2, WB>::T), HYENA_ROW_WAVES) k_row(RowArgs a) {
  using C = RowCfg<N2, WB>;
  constexpr int E = C::E, TPR = C::TPR, S2 = N2 / E;
  constexpr int PADN = RowPassLds::padded(N2);
  __shared__ cf smem[2 * PADN];
  const int b = threadIdx.x / TPR, j = threadIdx.x - b * TPR;
  int g, w;
  const int bid = blockIdx.x;
  if (KIND != ROW_SPEC && a.cmB > 1) {
    // Channel-major launch: the cmB workgroups of one (channel, row pair)
    // read the same spectrum slice, so they are placed on one XCD (workgroup
    // i runs on XCD i mod 8) one after another, and the slice is fetched
    // into that XCD's L2 once.  The grid holds 8 * ceil(n_units / 8) * cmB
    // workgroups; those of the padding units leave before any barrier.
    const int x = bid & 7, slot = bid >> 3;
    const int unit = (slot / a.cmB) * 8 + x;
    if (unit >= a.n_units) return;
    const int c = unit / a.n_row_pairs;
    w = unit - c * a.n_row_pairs;
    g = c * a.cmB + (slot - (slot / a.cmB) * a.cmB);
  } else {
    g = bid / a.n_row_pairs;
    w = bid - g * a.n_row_pairs;
  }
  const int n1 = a.n1;
  // Row k1 pairs with row n1 - k1 (its bins' Hermitian partners).  Even n1:
  // rows 0 and n1/2 are their own mirrors and share workgroup 0.  Odd n1:
  // row 0 is the only self-mirror row, and the second half of workgroup 0
  // repeats it as a shadow that stores nothing (its loads stay unconditional:
  // predicating them kept the compiler from issuing them early).
  const bool odd = (n1 & 1) != 0;
  const int k1 = (b == 0) ? w : (w == 0 ? (odd ? 0 : n1 / 2) : n1 - w);
  const bool live = !(odd && w == 0 && b == 1);
  const bool self_mirror = (k1 == 0) || (2 * k1 == n1);
  const int mb = self_mirror ? b : 1 - b;          // row holding the mirror bins
  const int k1m = (k1 == 0) ? 0 : n1 - k1;         // its k1
  const uint32_t N = (uint32_t)n1 * (uint32_t)N2;
  work_t<WB>* row = reinterpret_cast<work_t<WB>*>(a.work) + (int64_t)g * N + (int64_t)k1 * N2;
  const RowPassLds lds{smem + b * PADN};
  const RowPassLds ldsm{smem + mb * PADN};
  BlockFFT<N2, E, typename C::R> fft;
  fft.init(j);
  cf u[E];

  // four-step twiddle W_N^{k1 i2} for i2 = j + i*S2: base W_N^{k1 j} times
  // powers of the step W_N^{k1 S2}
  const cf tb = twiddle<false>((uint32_t)k1 * (uint32_t)j, N);
  const cf ts = twiddle<false>((uint32_t)k1 * (uint32_t)S2, N);
  if constexpr (KIND != ROW_SMUL) {
    if constexpr (HYENA_ROW_TW_SEQ) {
      cf p = tb;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        u[i] = cmul(ld_work<WB>(row + j + i * S2), p);
        if (i + 1 < E) p = cmul(p, ts);
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) u[i] = cmul(ld_work<WB>(row + j + i * S2), step_power<E>(tb, ts, i));
    }
    fft.template run<false>(u, lds, j);
  }

  // bins k = k1 + n1*k2 with k2 = j + i*S2; mirror N-k at (k1m, k2m)
  // W_{2N}^k = W_{2N}^{k1 + n1 j} * W_{2E}^i
  const cf wk = twiddle<false>((uint32_t)k1 + (uint32_t)n1 * (uint32_t)j, 2 * N);

  if constexpr (KIND == ROW_SMUL) {
    // The input row's real-FFT bins X(k) are given as S(k) = X(k)/(2N), the
    // filter's as G(k) = H(k)/(2N).  With Y = X H / (2N) = 2N S G, the
    // half-length bins whose unnormalised inverse DFT is y[2m] + i y[2m+1]
    // are C'(k) = Y(k) (1 + i conj W) + conj Y(N-k) (1 - i conj W),
    // W = W_{2N}^k -- the even/odd re-packing that realconv_pair folds into
    // its product.  Y(N-k) comes from the thread holding bin N-k (mirror row,
    // through LDS); Y(N), the partner of bin 0, is loaded directly.
    static_assert(!WB, "spectral-input rows use a float2 intermediate");
    const int arow = launch_row_of(a.r0, g, a.cmB, a.D);
    const int d = (a.cmB > 1) ? a.r0 + g / a.cmB : (a.r0 + g) % a.D;
    const cf* xs = a.spec_in + (int64_t)arow * a.spec_stride;
    const cf* gs = a.spec + (int64_t)(a.order * a.D + d) * a.spec_stride;
    const float sc = 2.0f * (float)N;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t k = (int64_t)k1 * N2 + j + i * S2;
      u[i] = cscale(cmul(ld_spec(xs + k), ld_spec(gs + k)), sc);
    }
    cf yn = make_float2(0.f, 0.f);
    if (k1 == 0 && j == 0) yn = cscale(cmul(ld_spec(xs + N), ld_spec(gs + N)), sc);
    if (a.rev) {   // the reversed output row: Y'(k) = W^(c k) conj Y(k), Y'(N) = (-1)^c conj Y(N)
      RevTwiddle<E> rt(a.rev_c, k1, n1, j, S2, 2 * N);
#pragma unroll
      for (int i = 0; i < E; ++i) u[i] = rt.apply_next(u[i]);
      yn = cscale(cconj(yn), a.rev_c & 1 ? -1.f : 1.f);
    }
#pragma unroll
    for (int i = 0; i < E; ++i) lds(j + i * S2) = u[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k2 = j + i * S2;
      const int k2m = (k1 == 0) ? ((N2 - k2) & (N2 - 1)) : (N2 - 1 - k2);
      const cf ym = (k1 == 0 && k2 == 0) ? yn : ldsm(k2m);
      const cf w = cmul(wk, w2e<E>(i));
      const cf p = make_float2(1.f + w.y, w.x), q = make_float2(1.f - w.y, -w.x);
      u[i] = cadd(cmul(u[i], p), cmul(cconj(ym), q));
    }
    __syncthreads();
    fft.template run<true>(u, lds, j);
    if (live) {
      cf p = tb;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        st_work<WB>(row + j + i * S2, cmulc(u[i], HYENA_ROW_TW_SEQ ? p : step_power<E>(tb, ts, i)));
        if (HYENA_ROW_TW_SEQ && i + 1 < E) p = cmul(p, ts);
      }
    }
  } else if constexpr (KIND == ROW_SPEC) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E; ++i) lds(j + i * S2) = u[i];
    __syncthreads();
    cf* out = a.spec_out + (int64_t)(a.r0 + g) * a.spec_stride;
    const float sc = 1.0f / (float)(2 * N);
    if (live) {
      if (a.rev) {
        RevTwiddle<E> rt(a.rev_c, k1, n1, j, S2, 2 * N);
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int k2 = j + i * S2;
          const int k2m = (k1 == 0) ? ((N2 - k2) & (N2 - 1)) : (N2 - 1 - k2);
          const cf am = ldsm(k2m);
          out[(int64_t)k1 * N2 + k2] = rt.apply_next(realfft_bin(u[i], am, cmul(wk, w2e<E>(i)), sc));
          if (k1 == 0 && k2 == 0)   // Nyquist bin, W^(c N) = (-1)^c
            out[N] = make_float2((a.rev_c & 1 ? -1.f : 1.f) * (u[i].x - u[i].y) * sc, 0.f);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int k2 = j + i * S2;
          const int k2m = (k1 == 0) ? ((N2 - k2) & (N2 - 1)) : (N2 - 1 - k2);
          const cf am = ldsm(k2m);
          out[(int64_t)k1 * N2 + k2] = realfft_bin(u[i], am, cmul(wk, w2e<E>(i)), sc);
          if (k1 == 0 && k2 == 0) out[N] = make_float2((u[i].x - u[i].y) * sc, 0.f);   // Nyquist bin
        }
      }
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
        u[0] = realconv_bin(u[0], u[0], ld_spec(gs), ld_spec(gs + N), make_float2(1.f, 0.f));
      } else {
        const int k2m = (k1 == 0) ? (N2 - k2) : (N2 - 1 - k2);
        cf bm = ldsm(k2m);
        realconv_pair(u[i], bm, ld_spec(gk + k2), ld_spec(gmr + k2m), cmul(wkb, w2e<E>(i)));
        ldsm(k2m) = bm;
      }
    }
    if (k1 == 0 && j == 0) {
      const cf am = lds(N2 / 2), gh = ld_spec(gs + N2 / 2);
      lds(N2 / 2) = realconv_bin(am, am, gh, gh, make_float2(0.f, -1.f));
    }
    __syncthreads();
#pragma unroll
    for (int i = E / 2; i < E; ++i) u[i] = lds(j + i * S2);
    fft.template run<true>(u, lds, j);
    if (live) {
      if constexpr (HYENA_ROW_TW_SEQ) {
        cf p = opaque(tb);
        const cf sq = opaque(ts);
#pragma unroll
        for (int i = 0; i < E; ++i) {
          st_work<WB>(row + j + i * S2, cmulc(u[i], p));
          if (i + 1 < E) p = cmul(p, sq);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i)
          st_work<WB>(row + j + i * S2, cmulc(u[i], step_power<E>(opaque(tb), opaque(ts), i)));
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

template <int N1, bool EVEN, bool GRID>
static void launch_col_t(int kind, int io, const ColArgs& c, dim3 grid, dim3 block, hipStream_t s) {
  if (kind == COL_SPEC) {
    hipLaunchKernelGGL((k_col<N1, 0, COL_SPEC, EVEN, GRID>), grid, block, 0, s, c);
  } else if (kind == COL_OUT) {   // io: the output's dtype (the intermediate is float2)
    if constexpr (!GRID) {
      if (io == 1) hipLaunchKernelGGL((k_col<N1, 1, COL_OUT, EVEN, false>), grid, block, 0, s, c);
      else hipLaunchKernelGGL((k_col<N1, 0, COL_OUT, EVEN, false>), grid, block, 0, s, c);
    }
  } else if (kind == COL_OUTREV) {
    if constexpr (!GRID) hipLaunchKernelGGL((k_col<N1, 0, COL_OUTREV, EVEN, false>), grid, block, 0, s, c);
  } else if (kind == COL_SPECG || kind == COL_SPECGF) {
    if constexpr (!GRID) {
      if (kind == COL_SPECGF && io == 0) hipLaunchKernelGGL((k_col<N1, 0, COL_SPECGF, EVEN, false>), grid, block, 0, s, c);
      else if (kind == COL_SPECGF) hipLaunchKernelGGL((k_col<N1, 1, COL_SPECGF, EVEN, false>), grid, block, 0, s, c);
      else if (io == 0) hipLaunchKernelGGL((k_col<N1, 0, COL_SPECG, EVEN, false>), grid, block, 0, s, c);
      else hipLaunchKernelGGL((k_col<N1, 1, COL_SPECG, EVEN, false>), grid, block, 0, s, c);
    }
  } else if (kind == COL_MIDSAVE || kind == COL_FIRSTG) {
    if constexpr (!GRID) {
      if (kind == COL_MIDSAVE && io == 0) hipLaunchKernelGGL((k_col<N1, 0, COL_MIDSAVE, EVEN, false>), grid, block, 0, s, c);
      else if (kind == COL_MIDSAVE) hipLaunchKernelGGL((k_col<N1, 1, COL_MIDSAVE, EVEN, false>), grid, block, 0, s, c);
      else if (io == 0) hipLaunchKernelGGL((k_col<N1, 0, COL_FIRSTG, EVEN, false>), grid, block, 0, s, c);
      else hipLaunchKernelGGL((k_col<N1, 1, COL_FIRSTG, EVEN, false>), grid, block, 0, s, c);
    }
  } else if (io == 0) {
    if (kind == COL_FIRST) hipLaunchKernelGGL((k_col<N1, 0, COL_FIRST, EVEN, GRID>), grid, block, 0, s, c);
    else if (kind == COL_MID) hipLaunchKernelGGL((k_col<N1, 0, COL_MID, EVEN, GRID>), grid, block, 0, s, c);
    else hipLaunchKernelGGL((k_col<N1, 0, COL_LAST, EVEN, GRID>), grid, block, 0, s, c);
  } else if (io == 1 || GRID) {
    if (kind == COL_FIRST) hipLaunchKernelGGL((k_col<N1, 1, COL_FIRST, EVEN, GRID>), grid, block, 0, s, c);
    else if (kind == COL_MID) hipLaunchKernelGGL((k_col<N1, 1, COL_MID, EVEN, GRID>), grid, block, 0, s, c);
    else hipLaunchKernelGGL((k_col<N1, 1, COL_LAST, EVEN, GRID>), grid, block, 0, s, c);
  } else if constexpr (!GRID) {
    if (kind == COL_FIRST) hipLaunchKernelGGL((k_col<N1, 2, COL_FIRST, EVEN, false>), grid, block, 0, s, c);
    else if (kind == COL_MID) hipLaunchKernelGGL((k_col<N1, 2, COL_MID, EVEN, false>), grid, block, 0, s, c);
    else hipLaunchKernelGGL((k_col<N1, 2, COL_LAST, EVEN, false>), grid, block, 0, s, c);
  }
}

// The kernel of one conv kind at one activation type (IOT as in k_col).
#define HYENA_COL_KINDS(KERN, P, IOTV, EVENV)                                                        \
  do {                                                                                               \
    constexpr int IOF = IOTV == 2 ? 0 : IOTV;   /* backward kinds: float2 intermediate */            \
    if (IOTV != 2 && kind == COL_MIDSAVE)                                                            \
      hipLaunchKernelGGL((KERN<P, IOF, COL_MIDSAVE, EVENV>), grid, block, 0, s, c);                  \
    else if (IOTV != 2 && kind == COL_FIRSTG)                                                        \
      hipLaunchKernelGGL((KERN<P, IOF, COL_FIRSTG, EVENV>), grid, block, 0, s, c);                   \
    else if (IOTV != 2 && kind == COL_SPECG)                                                         \
      hipLaunchKernelGGL((KERN<P, IOF, COL_SPECG, EVENV>), grid, block, 0, s, c);                    \
    else if (IOTV != 2 && kind == COL_SPECGF)                                                        \
      hipLaunchKernelGGL((KERN<P, IOF, COL_SPECGF, EVENV>), grid, block, 0, s, c);                   \
    else if (kind == COL_FIRST) hipLaunchKernelGGL((KERN<P, IOTV, COL_FIRST, EVENV>), grid, block, 0, s, c); \
    else if (kind == COL_MID) hipLaunchKernelGGL((KERN<P, IOTV, COL_MID, EVENV>), grid, block, 0, s, c); \
    else hipLaunchKernelGGL((KERN<P, IOTV, COL_LAST, EVENV>), grid, block, 0, s, c);                   \
  } while (0)

template <int N1, bool EVEN>
static void launch_col_odd_t(int kind, int io, const ColArgs& c, dim3 grid, hipStream_t s) {
  const dim3 block(kColOddThreads);
  if (kind == COL_SPEC) hipLaunchKernelGGL((k_col_odd<N1, 0, COL_SPEC, EVEN>), grid, block, 0, s, c);
  else if (kind == COL_OUT && io == 1) hipLaunchKernelGGL((k_col_odd<N1, 1, COL_OUT, EVEN>), grid, block, 0, s, c);
  else if (kind == COL_OUT) hipLaunchKernelGGL((k_col_odd<N1, 0, COL_OUT, EVEN>), grid, block, 0, s, c);
  else if (kind == COL_OUTREV) hipLaunchKernelGGL((k_col_odd<N1, 0, COL_OUTREV, EVEN>), grid, block, 0, s, c);
  else if (io == 0) HYENA_COL_KINDS(k_col_odd, N1, 0, EVEN);
  else if (io == 1) HYENA_COL_KINDS(k_col_odd, N1, 1, EVEN);
  else HYENA_COL_KINDS(k_col_odd, N1, 2, EVEN);
}

template <int Q, bool EVEN>
static void launch_col_pair_t(int kind, int io, const ColArgs& c, dim3 grid, hipStream_t s) {
  const dim3 block(kColOddThreads);
  if (kind == COL_SPEC) hipLaunchKernelGGL((k_col_pair<Q, 0, COL_SPEC, EVEN>), grid, block, 0, s, c);
  else if (kind == COL_OUT && io == 1) hipLaunchKernelGGL((k_col_pair<Q, 1, COL_OUT, EVEN>), grid, block, 0, s, c);
  else if (kind == COL_OUT) hipLaunchKernelGGL((k_col_pair<Q, 0, COL_OUT, EVEN>), grid, block, 0, s, c);
  else if (kind == COL_OUTREV) hipLaunchKernelGGL((k_col_pair<Q, 0, COL_OUTREV, EVEN>), grid, block, 0, s, c);
  else if (io == 0) HYENA_COL_KINDS(k_col_pair, Q, 0, EVEN);
  else if (io == 1) HYENA_COL_KINDS(k_col_pair, Q, 1, EVEN);
  else HYENA_COL_KINDS(k_col_pair, Q, 2, EVEN);
}
#undef HYENA_COL_KINDS

template <int Q>
static hipError_t launch_col_pair(int kind, int io, const ColArgs& c, int groups, hipStream_t s) {
  const dim3 grid(groups * c.n_col_blocks);
  if (c.L % 2 == 0) launch_col_pair_t<Q, true>(kind, io, c, grid, s);
  else launch_col_pair_t<Q, false>(kind, io, c, grid, s);
  return hipGetLastError();
}

template <int N1>
static hipError_t launch_col_odd(int kind, int io, const ColArgs& c, int groups, hipStream_t s) {
  const dim3 grid(groups * c.n_col_blocks);
  if (c.L % 2 == 0) launch_col_odd_t<N1, true>(kind, io, c, grid, s);
  else launch_col_odd_t<N1, false>(kind, io, c, grid, s);
  return hipGetLastError();
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
  if (!grid && odd_col_ok(n1)) return kColOddThreads;
  if (!grid && n1 % 2 == 0 && odd_col_ok(n1 / 2)) return kColOddThreads / 2;
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
  if (!grid_mode) {
    switch (n1) {
      case 3: return launch_col_odd<3>(kind, io, c, groups, s);
      case 5: return launch_col_odd<5>(kind, io, c, groups, s);
      case 9: return launch_col_odd<9>(kind, io, c, groups, s);
      case 15: return launch_col_odd<15>(kind, io, c, groups, s);
      case 25: return launch_col_odd<25>(kind, io, c, groups, s);
      case 27: return launch_col_odd<27>(kind, io, c, groups, s);
      case 6: return launch_col_pair<3>(kind, io, c, groups, s);
      case 10: return launch_col_pair<5>(kind, io, c, groups, s);
      case 18: return launch_col_pair<9>(kind, io, c, groups, s);
      case 30: return launch_col_pair<15>(kind, io, c, groups, s);
      case 50: return launch_col_pair<25>(kind, io, c, groups, s);
      case 54: return launch_col_pair<27>(kind, io, c, groups, s);
    }
  }
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
  // channel-major: n_units (channel, row pair) units padded to a multiple of 8, cmB workgroups each
  const int blocks = (kind != ROW_SPEC && r.cmB > 1) ? (r.n_units + 7) / 8 * 8 * r.cmB : groups * r.n_row_pairs;
  const dim3 grid(blocks);
  if (kind == ROW_SPEC) hipLaunchKernelGGL((k_row<N2, ROW_SPEC>), grid, dim3(RowCfg<N2>::T), 0, s, r);
  else if (kind == ROW_SMUL) hipLaunchKernelGGL((k_row<N2, ROW_SMUL>), grid, dim3(RowCfg<N2>::T), 0, s, r);
  else if (r.wb) hipLaunchKernelGGL((k_row<N2, ROW_CONV, true>), grid, dim3(RowCfg<N2, true>::T), 0, s, r);
  else hipLaunchKernelGGL((k_row<N2, ROW_CONV, false>), grid, dim3(RowCfg<N2>::T), 0, s, r);
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
  r.n1 = p.n1; r.spec_stride = a.spec_stride; r.D = a.D; r.n_row_pairs = (p.n1 + 1) / 2;
  // bf16 activations up to kBf16WorkMaxOrder: bf16 intermediate (column
  // kernels IOT 2, row kernel WB), else float2.
  // The backward's convolutions (no gate) keep a float2 intermediate.
  const int cio = a.io == 0 ? 0 : (!a.no_gate && forward_bf16_work(true, a.NORD) ? 2 : 1);
  r.wb = cio == 2;
  // With B > 1 a launch covers whole channels (all their batch rows), so the
  // row pass reads each channel's spectrum once instead of once per batch row.
  const bool cm = a.B > 1 && a.n_rows == a.B * a.D && a.rows_per_group >= a.B;
  const int units = cm ? a.D : a.n_rows, per = cm ? a.rows_per_group / a.B : a.rows_per_group;
  c.cmB = r.cmB = cm ? a.B : 1;
  c.cmD = a.D;
  // Input rows given by their spectra: one order, no gate, fp32, and the
  // first column pass and forward row FFT are skipped.
  const bool smul = a.spec_in != nullptr;
  if (smul && (a.NORD != 1 || !a.no_gate || cio != 0)) return hipErrorInvalidValue;
  r.spec_in = static_cast<const cf*>(a.spec_in);
  // rev_out: the output row reversed (one order, no gate, float2 intermediate):
  // by the spectral map in the row pass from a spectral input, else by the
  // output column pass's addressing (COL_OUTREV, power-of-two columns)
  if (a.rev_out && (a.NORD != 1 || !a.no_gate || cio == 2)) return hipErrorInvalidValue;
  if (a.rev_out && !smul && !fourstep_fused_spec_ok(p)) return hipErrorInvalidValue;
  r.rev = smul && a.rev_out;
  r.rev_c = a.rev_c;
  c.rev_c = a.rev_c;
  const int rkind = smul ? ROW_SMUL : ROW_CONV;
  // csave: c_n of every order kept (fp32); vc: input rows x * c formed in the
  // first column pass
  const bool save = a.csave != nullptr;
  if ((save || a.vc) && !a.no_gate) return hipErrorInvalidValue;
  if (a.vc && (a.NORD != 1 || smul)) return hipErrorInvalidValue;
  const int first = a.vc ? COL_FIRSTG : COL_FIRST;
  if (a.vc) c.v = a.vc;
  for (int r0 = 0; r0 < units; r0 += per) {
    const int groups = ((units - r0 < per) ? units - r0 : per) * (cm ? a.B : 1);
    c.r0 = r0; r.r0 = r0;
    r.n_units = cm ? groups / a.B * r.n_row_pairs : 0;
    if (a.vc) c.xg = a.v;
    hipError_t e = smul ? hipSuccess : dispatch_col(p.n1, first, cio, c, groups, s);
    if (e != hipSuccess) return e;
    for (int n = 0; n < a.NORD; ++n) {
      r.order = n;
      e = dispatch_row(p.n2, rkind, r, groups, s);
      if (e != hipSuccess) return e;
      c.xg = a.x.p[n];
      if (save) c.y = a.csave + n * a.csave_stride;
      const int kind = n < a.NORD - 1 ? (save ? COL_MIDSAVE : COL_MID)
                                      : (a.no_gate ? (a.rev_out && !smul ? COL_OUTREV : COL_OUT) : COL_LAST);
      // ungated outputs: fp32 rows, bf16 with out_bf16 (float2 intermediate either way)
      e = dispatch_col(p.n1, kind, kind == COL_OUT ? (a.out_bf16 ? 1 : 0) : cio, c, groups, s);
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
  r.n_row_pairs = (p.n1 + 1) / 2;
  r.rev = a.rev; r.rev_c = a.rev_c;
  // rows g * x formed in the column pass (power-of-two columns only)
  const bool fused = a.g != nullptr;
  if (fused && !fourstep_fused_spec_ok(p)) return hipErrorInvalidValue;
  const int kind = fused ? (a.g_f32 ? COL_SPECGF : COL_SPECG) : COL_SPEC;
  if (fused) { c.v = a.g; c.h = a.c; c.xg = a.x; c.y = a.gx; }
  for (int r0 = 0; r0 < a.NF; r0 += a.rows_per_group) {
    const int groups = (a.NF - r0 < a.rows_per_group) ? a.NF - r0 : a.rows_per_group;
    c.r0 = r0; r.r0 = r0;
    hipError_t e = dispatch_col(p.n1, kind, fused ? a.io : 0, c, groups, s);
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
