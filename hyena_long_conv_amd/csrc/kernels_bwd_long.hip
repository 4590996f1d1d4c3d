// kernels_bwd_long.hip -- backward of the recurrence for lengths on the
// four-step path (beyond one workgroup's LDS).
//
// The gradients follow from the recurrence by the chain rule (the pages
// state none; the long-sequence training of the jisaku.com glossary entry,
// section "長いシーケンスへの適応", is what needs them at these lengths).
// Every convolution of the backward is expressed through the causal
// convolution the forward kernels already compute, using the row reversal
// R (R(a)[t] = a[L-1-t]) on [0, L):
//   adjoint of the causal conv:  g[s] = sum_{t>=s} h[t-s] gc[t]
//                                     = R(h conv R(gc))[s],
//   filter gradient:             gh[k] = sum_{t>=k} gc[t] z[t-k]
//                                      = (R(gc) conv z)[L-1-k],
// the latter with R(gc) as a per-row "filter" whose spectrum is built by the
// four-step spectrum kernels (rows of all batch items at once, then summed
// over the batch).  The forward's convolution outputs c_n are recomputed
// once and kept in the workspace.  All intermediates are fp32.
#include <hip/hip_runtime.h>

#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {
namespace {

constexpr int EW_THREADS = 256;

inline dim3 ew_grid(int64_t n) {
  int64_t b = (n / 4 + EW_THREADS - 1) / EW_THREADS;
  if (b > 65536 * 8) b = 65536 * 8;
  return dim3((unsigned)(b < 1 ? 1 : b));
}

// Four consecutive elements per thread (n4 = n / 4 groups), then a scalar
// tail; every buffer here starts 16-byte aligned.
#define EW_LOOP4(n)                                                                              \
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < (n) / 4;                   \
       q += (int64_t)gridDim.x * blockDim.x)

template <int IOT>
__device__ __forceinline__ void ld4_io(const void* p, int64_t i, float (&o)[4]) {
  if constexpr (IOT == 0) {
    const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    o[0] = __uint_as_float(w.x << 16); o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16); o[3] = __uint_as_float(w.y & 0xffff0000u);
  }
}

template <int IOT>
__global__ void k_bw_load(const void* __restrict__ src, float* __restrict__ dst, int64_t n) {
  EW_LOOP4(n) {
    float o[4];
    ld4_io<IOT>(src, 4 * q, o);
    *reinterpret_cast<float4*>(dst + 4 * q) = make_float4(o[0], o[1], o[2], o[3]);
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = (n & ~int64_t(3)) + threadIdx.x;
    dst[i] = IO<IOT>::ld(src, i);
  }
}

// z = x * c  (x in the I/O dtype)
template <int IOT>
__global__ void k_bw_gate(const void* __restrict__ x, const float* __restrict__ c, float* __restrict__ z, int64_t n) {
  EW_LOOP4(n) {
    float o[4];
    ld4_io<IOT>(x, 4 * q, o);
    const float4 cv = *reinterpret_cast<const float4*>(c + 4 * q);
    *reinterpret_cast<float4*>(z + 4 * q) = make_float4(o[0] * cv.x, o[1] * cv.y, o[2] * cv.z, o[3] * cv.w);
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = (n & ~int64_t(3)) + threadIdx.x;
    z[i] = IO<IOT>::ld(x, i) * c[i];
  }
}

// Kernels that reverse rows walk (row, position) on a 2-D grid, so no
// element index is divided by L.
#define ROW_LOOP(rows, L)                                                                         \
  for (int64_t r = blockIdx.y; r < (rows); r += gridDim.y)                                       \
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < (L); t += (int64_t)gridDim.x * blockDim.x)

inline dim3 row_grid(int64_t rows, int64_t L) {
  int64_t bx = (L + EW_THREADS - 1) / EW_THREADS, by = rows;
  if (bx > 1024) bx = 1024;
  if (by > 65535) by = 65535;
  while (bx * by > 65536 * 8 && bx > 1) bx = (bx + 1) / 2;
  return dim3((unsigned)bx, (unsigned)(by < 1 ? 1 : by));
}

// V4 (L a multiple of 4): a thread takes positions t .. t+3 of a row, whose
// mirror images L-4-t .. L-1-t are one aligned group of four as well, so
// every access is a 16-byte (fp32) or 8-byte (bf16) vector.
#define ROW_LOOP4(rows, L)                                                                        \
  for (int64_t r = blockIdx.y; r < (rows); r += gridDim.y)                                       \
    for (int64_t t = 4 * (blockIdx.x * (int64_t)blockDim.x + threadIdx.x); t < (L);                 \
         t += 4 * (int64_t)gridDim.x * blockDim.x)

__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st_f4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <int IOT>
__device__ __forceinline__ void st4_io(void* p, int64_t i, float a, float b, float c, float d) {
  if constexpr (IOT == 0) {
    st_f4(static_cast<float*>(p) + i, a, b, c, d);
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = make_uint2(bf16x2_bits(a, b), bf16x2_bits(c, d));
  }
}

// One order's elementwise work on the incoming gradient g (held reversed,
// g = R(gsrc), when REV: the previous adjoint convolution leaves it so):
//   gx = g * c  (I/O dtype)   and   t2 = R(g * x)  (fp32).
// CIRC: periodic rows, whose reversal is R'(t) = (L - t) mod L instead of
// R(t) = L - 1 - t (one position per thread: the mirrored groups of four
// are not aligned).
__device__ __forceinline__ int64_t mirror(int64_t t, int64_t L, bool circ) {
  return circ ? (t == 0 ? 0 : L - t) : L - 1 - t;
}

template <int IOT, bool REV, bool V4, bool CIRC = false>
__global__ void k_bw_step(const float* __restrict__ gsrc, const float* __restrict__ c, const void* __restrict__ x,
                          void* __restrict__ gx, float* __restrict__ t2, int64_t rows, int64_t L) {
  if constexpr (V4) {
    ROW_LOOP4(rows, L) {
      const int64_t i = r * L + t, ri = r * L + (L - 4 - t);     // ri: mirror of t + 3
      float g[4], xv[4];
      if constexpr (REV) {
        const float4 w = ld_f4(gsrc + ri);
        g[0] = w.w; g[1] = w.z; g[2] = w.y; g[3] = w.x;
      } else {
        const float4 w = ld_f4(gsrc + i);
        g[0] = w.x; g[1] = w.y; g[2] = w.z; g[3] = w.w;
      }
      const float4 cv = ld_f4(c + i);
      ld4_io<IOT>(x, i, xv);
      st4_io<IOT>(gx, i, g[0] * cv.x, g[1] * cv.y, g[2] * cv.z, g[3] * cv.w);
      st_f4(t2 + ri, g[3] * xv[3], g[2] * xv[2], g[1] * xv[1], g[0] * xv[0]);
    }
  } else {
    ROW_LOOP(rows, L) {
      const int64_t i = r * L + t, ri = r * L + mirror(t, L, CIRC);
      const float g = gsrc[REV ? ri : i];
      IO<IOT>::st(gx, i, g * c[i]);
      t2[ri] = g * IO<IOT>::ld(x, i);
    }
  }
}

// out = R(a) in the I/O dtype (the final gradient of v)
template <int IOT, bool V4, bool CIRC = false>
__global__ void k_bw_store_rev(const float* __restrict__ a, void* __restrict__ out, int64_t rows, int64_t L) {
  if constexpr (V4) {
    ROW_LOOP4(rows, L) {
      const float4 w = ld_f4(a + r * L + (L - 4 - t));
      st4_io<IOT>(out, r * L + t, w.w, w.z, w.y, w.x);
    }
  } else {
    ROW_LOOP(rows, L) IO<IOT>::st(out, r * L + t, a[r * L + mirror(t, L, CIRC)]);
  }
}

// gh[d][k] = sum_b t[b*D + d][L-1-k]  (fixed batch order: deterministic)
template <bool V4, bool CIRC = false>
__global__ void k_bw_batch_sum_rev(const float* __restrict__ tt, float* __restrict__ gh, int B, int D, int64_t L) {
  if constexpr (V4) {
    ROW_LOOP4(D, L) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int b = 0; b < B; ++b) {
        const float4 w = ld_f4(tt + ((int64_t)b * D + r) * L + (L - 4 - t));
        acc.x += w.w; acc.y += w.z; acc.z += w.y; acc.w += w.x;
      }
      st_f4(gh + r * L + t, acc.x, acc.y, acc.z, acc.w);
    }
  } else {
    ROW_LOOP(D, L) {
      float acc = 0.f;
      for (int b = 0; b < B; ++b) acc += tt[((int64_t)b * D + r) * L + mirror(t, L, CIRC)];
      gh[r * L + t] = acc;
    }
  }
}

template <int IOT>
hipError_t bw_elementwise_io(int op, const void* a, const void* b, void* out, int64_t n, hipStream_t s) {
  const dim3 g = ew_grid(n), blk(EW_THREADS);
  switch (op) {
    case 0: hipLaunchKernelGGL(k_bw_load<IOT>, g, blk, 0, s, a, (float*)out, n); break;
    case 2: hipLaunchKernelGGL(k_bw_gate<IOT>, g, blk, 0, s, a, (const float*)b, (float*)out, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

enum { BW_LOAD = 0, BW_GATE = 2 };

template <int IOT>
hipError_t bw_step_io(bool rev, const float* g, const float* c, const void* x, void* gx, float* t2, int64_t L,
                      int64_t n, bool circ, hipStream_t s) {
  const int64_t rows = n / L;
  const dim3 blk(EW_THREADS);
  if (circ) {
    const dim3 grid = row_grid(rows, L);
    if (rev) hipLaunchKernelGGL((k_bw_step<IOT, true, false, true>), grid, blk, 0, s, g, c, x, gx, t2, rows, L);
    else hipLaunchKernelGGL((k_bw_step<IOT, false, false, true>), grid, blk, 0, s, g, c, x, gx, t2, rows, L);
  } else if (L % 4 == 0) {
    const dim3 grid = row_grid(rows, L / 4);
    if (rev) hipLaunchKernelGGL((k_bw_step<IOT, true, true>), grid, blk, 0, s, g, c, x, gx, t2, rows, L);
    else hipLaunchKernelGGL((k_bw_step<IOT, false, true>), grid, blk, 0, s, g, c, x, gx, t2, rows, L);
  } else {
    const dim3 grid = row_grid(rows, L);
    if (rev) hipLaunchKernelGGL((k_bw_step<IOT, true, false>), grid, blk, 0, s, g, c, x, gx, t2, rows, L);
    else hipLaunchKernelGGL((k_bw_step<IOT, false, false>), grid, blk, 0, s, g, c, x, gx, t2, rows, L);
  }
  return hipGetLastError();
}

hipError_t bw_ew(int io, int op, const void* a, const void* b, void* out, int64_t n, hipStream_t s) {
  return io == 0 ? bw_elementwise_io<0>(op, a, b, out, n, s) : bw_elementwise_io<1>(op, a, b, out, n, s);
}

// Causal convolution of every row of z with a filter spectrum: an order-1
// four-step forward without the gate.  filters_per_row: the spectrum holds
// one filter per row (else one per channel).
hipError_t bw_conv(const PlanInfo& p, const void* spec, const float* z, float* out, int B, int D,
                   bool filters_per_row, void* work, int rows_per_group, hipStream_t s) {
  ForwardArgs f{};
  f.v = z;
  f.no_gate = 1;
  f.spec = spec;
  f.y = out;
  f.B = filters_per_row ? 1 : B;
  f.D = filters_per_row ? B * D : D;
  f.NORD = 1;
  f.L = p.L;
  f.io = 0;
  f.spec_stride = p.spec_stride;
  f.n_rows = B * D;
  f.work = work;
  f.rows_per_group = rows_per_group;
  f.circular = 0;
  return fourstep_forward(f, p, s);
}

}  // namespace

LongBackwardLayout long_backward_layout(const PlanInfo& p, int64_t B, int64_t D, int64_t NORD) {
  const auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t R = B * D, act = al(R * p.L * 4);
  LongBackwardLayout w{};
  int64_t o = 0;
  w.c = o;     o += NORD * act;
  w.z = o;     o += act;
  w.g = o;     o += act;
  w.t1 = o;    o += act;
  w.t2 = o;    o += act;
  w.sg = o;    o += al(R * p.spec_stride * 8);
  {  // as many pass groups as the work budget needs, of equal size; rows of
     // 8 MiB and more take 224 MB groups, as the forward's
    int64_t g = rows_per_group(p.N, R);
    if ((int64_t)p.N * 8 >= (int64_t(8) << 20)) g = std::min<int64_t>(R, (int64_t(224) << 20) / ((int64_t)p.N * 8));
    const int64_t groups = (R + g - 1) / g;
    w.rows_per_group = (int)((R + groups - 1) / groups);
  }
  w.work = o;  o += al((int64_t)w.rows_per_group * p.N * 8);
  w.total = o;
  return w;
}

hipError_t long_backward(const BackwardArgs& a, const PlanInfo& p, void* workspace, hipStream_t s) {
  const int64_t B = a.B, D = a.D, L = a.L, R = B * D, n = R * L;
  // periodic rows: the same chain with R' (t -> -t mod L) in place of R and
  // periodic convolutions (the four-step passes need no flag: with L equal to
  // the FFT length no sample is padding)
  const bool circ = a.circular != 0;
  const LongBackwardLayout w = long_backward_layout(p, B, D, a.NORD);
  char* ws = static_cast<char*>(workspace);
  float* C = reinterpret_cast<float*>(ws + w.c);
  float* Z = reinterpret_cast<float*>(ws + w.z);
  float* G = reinterpret_cast<float*>(ws + w.g);
  float* T1 = reinterpret_cast<float*>(ws + w.t1);
  float* T2 = reinterpret_cast<float*>(ws + w.t2);
  void* sg = ws + w.sg;
  void* work = ws + w.work;
  const int64_t cstride = (w.z - w.c) / a.NORD / 4;   // floats between saved c_n
  const cf* spec = static_cast<const cf*>(a.spec);
  const auto spec_n = [&](int nn) { return static_cast<const void*>(spec + (int64_t)nn * D * p.spec_stride); };
  hipError_t e;
#define BW_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  // forward: c_n = h_n conv z_n (kept), z_{n+1} = x_n * c_n
  BW_TRY(bw_ew(a.io, BW_LOAD, a.v, nullptr, Z, n, s));
  for (int nn = 0; nn < a.NORD; ++nn) {
    float* Cn = C + nn * cstride;
    BW_TRY(bw_conv(p, spec_n(nn), Z, Cn, (int)B, (int)D, false, work, w.rows_per_group, s));
    if (nn < a.NORD - 1) BW_TRY(bw_ew(a.io, BW_GATE, a.x.p[nn], Cn, Z, n, s));
  }
  // backward, g = dloss/dz_{n+1}; after each adjoint convolution g is left
  // reversed in T1 and read through the reversal by the next step
  BW_TRY(bw_ew(a.io, BW_LOAD, a.gy, nullptr, G, n, s));
  const float* gcur = G;
  bool grev = false;
  for (int nn = a.NORD - 1; nn >= 0; --nn) {
    const float* Cn = C + nn * cstride;
    // gx_n = g * c_n, T2 = R(g * x_n)
    BW_TRY(a.io == 0 ? bw_step_io<0>(grev, gcur, Cn, a.x.p[nn], a.gx.p[nn], T2, L, n, circ, s)
                     : bw_step_io<1>(grev, gcur, Cn, a.x.p[nn], a.gx.p[nn], T2, L, n, circ, s));
    if (nn == 0) BW_TRY(bw_ew(a.io, BW_LOAD, a.v, nullptr, Z, n, s));          // z_1 = v
    else BW_TRY(bw_ew(a.io, BW_GATE, a.x.p[nn - 1], C + (nn - 1) * cstride, Z, n, s));
    // filter gradient: spectra of the rows of T2, then (T2 conv z) reversed and summed over the batch
    SpectrumArgs sa{};
    sa.h = T2; sa.spec = sg; sa.NF = (int)R; sa.L = L; sa.spec_stride = p.spec_stride;
    sa.work = work; sa.rows_per_group = w.rows_per_group; sa.circular = 0;
    BW_TRY(fourstep_spectrum(sa, p, s));
    BW_TRY(bw_conv(p, sg, Z, T1, (int)B, (int)D, true, work, w.rows_per_group, s));
    if (circ)
      hipLaunchKernelGGL((k_bw_batch_sum_rev<false, true>), row_grid(D, L), dim3(EW_THREADS), 0, s, T1,
                         a.gh + (int64_t)nn * D * L, (int)B, (int)D, L);
    else if (L % 4 == 0)
      hipLaunchKernelGGL(k_bw_batch_sum_rev<true>, row_grid(D, L / 4), dim3(EW_THREADS), 0, s, T1,
                         a.gh + (int64_t)nn * D * L, (int)B, (int)D, L);
    else
      hipLaunchKernelGGL(k_bw_batch_sum_rev<false>, row_grid(D, L), dim3(EW_THREADS), 0, s, T1,
                         a.gh + (int64_t)nn * D * L, (int)B, (int)D, L);
    BW_TRY(hipGetLastError());
    // adjoint: g_n = R(h_n conv T2); kept reversed in T1
    BW_TRY(bw_conv(p, spec_n(nn), T2, T1, (int)B, (int)D, false, work, w.rows_per_group, s));
    gcur = T1;
    grev = true;
  }
  const dim3 rg = row_grid(R, L % 4 == 0 && !circ ? L / 4 : L);
  if (circ) {
    if (a.io == 0) hipLaunchKernelGGL((k_bw_store_rev<0, false, true>), rg, dim3(EW_THREADS), 0, s, gcur, a.gv, R, L);
    else hipLaunchKernelGGL((k_bw_store_rev<1, false, true>), rg, dim3(EW_THREADS), 0, s, gcur, a.gv, R, L);
  } else if (L % 4 == 0) {
    if (a.io == 0) hipLaunchKernelGGL((k_bw_store_rev<0, true>), rg, dim3(EW_THREADS), 0, s, gcur, a.gv, R, L);
    else hipLaunchKernelGGL((k_bw_store_rev<1, true>), rg, dim3(EW_THREADS), 0, s, gcur, a.gv, R, L);
  } else {
    if (a.io == 0) hipLaunchKernelGGL((k_bw_store_rev<0, false>), rg, dim3(EW_THREADS), 0, s, gcur, a.gv, R, L);
    else hipLaunchKernelGGL((k_bw_store_rev<1, false>), rg, dim3(EW_THREADS), 0, s, gcur, a.gv, R, L);
  }
  BW_TRY(hipGetLastError());
#undef BW_TRY
  return hipSuccess;
}

}  // namespace hyena
