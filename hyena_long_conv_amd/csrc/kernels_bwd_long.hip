// kernels_bwd_long.hip -- backward of the recurrence for lengths on the
// four-step path (beyond one workgroup's LDS).
//
// The gradients follow from the recurrence by the chain rule (the pages
// state none; the long-sequence training of the jisaku.com glossary entry,
// section "長いシーケンスへの適応", is what needs them at these lengths).
// Every convolution of the backward is expressed through the forward's
// four-step passes, using the row reversal R (R(a)[t] = a[L-1-t]) on [0, L):
//   adjoint of the causal conv:  g[s] = sum_{t>=s} h[t-s] gc[t]
//                                     = R(h conv R(gc))[s],
//   filter gradient:             gh[k] = sum_{t>=k} gc[t] z[t-k]
//                                      = (R(gc) conv z)[L-1-k],
// the latter with R(gc) as a per-row "filter" whose spectrum is built by the
// four-step spectrum kernels (rows of all batch items at once, then summed
// over the batch).  R never runs as a pass of its own: on the spectra it is
// the map X(k) -> W_M^(c k) conj X(k) (c = L - 1, M the FFT length), and on
// the filter gradient's output the column pass's addressing.  The forward's
// convolution outputs c_n are recomputed once and kept in the workspace.
// All intermediates are fp32.
#include <hip/hip_runtime.h>

#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {
namespace {

constexpr int EW_THREADS = 256;

// Row kernels walk (row, position) on a 2-D grid, so no element index is
// divided by L.
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

// V4 (L a multiple of 4): a thread takes positions t .. t+3 of a row, so
// every access is a 16-byte (fp32) or 8-byte (bf16) vector.
#define ROW_LOOP4(rows, L)                                                                        \
  for (int64_t r = blockIdx.y; r < (rows); r += gridDim.y)                                       \
    for (int64_t t = 4 * (blockIdx.x * (int64_t)blockDim.x + threadIdx.x); t < (L);                 \
         t += 4 * (int64_t)gridDim.x * blockDim.x)

__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st_f4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// gh[d][k] = sum_b t[b*D + d][k]  (fixed batch order: deterministic)
template <bool V4>
__global__ void k_bw_batch_sum(const float* __restrict__ tt, float* __restrict__ gh, int B, int D, int64_t L) {
  if constexpr (V4) {
    ROW_LOOP4(D, L) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int b = 0; b < B; ++b) {
        const float4 w = ld_f4(tt + ((int64_t)b * D + r) * L + t);
        acc.x += w.x; acc.y += w.y; acc.z += w.z; acc.w += w.w;
      }
      st_f4(gh + r * L + t, acc.x, acc.y, acc.z, acc.w);
    }
  } else {
    ROW_LOOP(D, L) {
      float acc = 0.f;
      for (int b = 0; b < B; ++b) acc += tt[((int64_t)b * D + r) * L + t];
      gh[r * L + t] = acc;
    }
  }
}

// Causal convolution of every row of z with a filter spectrum: an order-1
// four-step forward without the gate.  filters_per_row: the spectrum holds
// one filter per row (else one per channel).
// zspec: the rows are given by their spectra (filter-spectrum layout, one per
// row) instead of z, which then goes unread; filters per channel only.
// zio: dtype of z (0 fp32, 1 bf16); the intermediate and out are fp32.
// zc: the rows are z * zc (zc fp32), formed in the first column pass.
// rev_c >= 0: the output row reversed, t -> (rev_c - t) mod M.
hipError_t bw_conv(const PlanInfo& p, const void* spec, const void* z, float* out, int B, int D,
                   bool filters_per_row, void* work, int rows_per_group, hipStream_t s,
                   const void* zspec = nullptr, int zio = 0, const float* zc = nullptr, int64_t rev_c = -1,
                   bool out_bf16 = false) {
  ForwardArgs f{};
  f.out_bf16 = out_bf16;
  f.v = z;
  f.spec_in = zspec;
  f.vc = zc;
  f.rev_out = rev_c >= 0;
  f.rev_c = rev_c;
  f.no_gate = 1;
  f.spec = spec;
  f.y = out;
  f.B = filters_per_row ? 1 : B;
  f.D = filters_per_row ? B * D : D;
  f.NORD = 1;
  f.L = p.L;
  f.io = zio;
  f.spec_stride = p.spec_stride;
  f.n_rows = B * D;
  f.work = work;
  f.rows_per_group = rows_per_group;
  f.circular = 0;
  return fourstep_forward(f, p, s);
}

}  // namespace

hipError_t long_backward(const BackwardArgs& a, const PlanInfo& p, void* workspace, hipStream_t s) {
  const int64_t B = a.B, D = a.D, L = a.L, R = B * D;
  // periodic rows: the same chain with R' (t -> -t mod L) in place of R and
  // periodic convolutions (the four-step passes need no flag: with L equal to
  // the FFT length no sample is padding)
  const bool circ = a.circular != 0;
  if (!fourstep_fused_spec_ok(p)) return hipErrorInvalidValue;
  const LongBackwardLayout w = long_backward_layout(p, B, D, a.NORD);
  char* ws = static_cast<char*>(workspace);
  float* C = reinterpret_cast<float*>(ws + w.c);
  float* T1 = reinterpret_cast<float*>(ws + w.t1);
  void* sg = ws + w.sg;
  void* work = ws + w.work;
  const int64_t cstride = (w.t1 - w.c) / a.NORD / 4;  // floats between saved c_n
  const cf* spec = static_cast<const cf*>(a.spec);
  const auto spec_n = [&](int nn) { return static_cast<const void*>(spec + (int64_t)nn * D * p.spec_stride); };
  hipError_t e;
#define BW_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  // forward: c_n = h_n conv z_n (kept), z_{n+1} = x_n * c_n -- the forward's
  // own passes, each order's column pass also storing c_n (fp32)
  {
    ForwardArgs f{};
    f.v = a.v; f.x = a.x; f.spec = a.spec; f.B = (int)B; f.D = (int)D; f.NORD = a.NORD; f.L = L;
    f.io = a.io; f.spec_stride = p.spec_stride; f.n_rows = (int)R; f.work = work;
    f.rows_per_group = w.rows_per_group; f.no_gate = 1; f.csave = C; f.csave_stride = cstride;
    BW_TRY(fourstep_forward(f, p, s));
  }
  // backward, g = dloss/dz_{n+1} in natural order (T1 after the first step,
  // which reads dloss/dy itself).  R enters as the spectral map
  // X(k) -> W_M^(c k) conj X(k) (c = L - 1; periodic rows c = 0).
  const int64_t rev_c = circ ? 0 : L - 1;
  const void* gcur = a.gy;
  for (int nn = a.NORD - 1; nn >= 0; --nn) {
    // spectra of the rows of R(g * x_n); the column pass also stores gx_n = g * c_n
    SpectrumArgs sa{};
    sa.spec = sg; sa.NF = (int)R; sa.L = L; sa.spec_stride = p.spec_stride;
    sa.work = work; sa.rows_per_group = w.rows_per_group; sa.circular = 0;
    sa.g = gcur; sa.g_f32 = nn != a.NORD - 1; sa.c = C + nn * cstride; sa.x = a.x.p[nn]; sa.gx = a.gx.p[nn];
    sa.io = a.io; sa.rev = 1; sa.rev_c = rev_c;
    BW_TRY(fourstep_spectrum(sa, p, s));
    // filter gradient: (R(g * x_n) conv z_n), stored reversed by its output
    // column pass (for B = 1 straight into gh_n) and summed over the batch;
    // z_1 = v, z_n = x_{n-1} * c_{n-1} formed by the first column pass
    float* gh_n = a.gh + (int64_t)nn * D * L;
    float* fout = B == 1 ? gh_n : T1;
    if (nn == 0)
      BW_TRY(bw_conv(p, sg, a.v, fout, (int)B, (int)D, true, work, w.rows_per_group, s, nullptr, a.io, nullptr, rev_c));
    else
      BW_TRY(bw_conv(p, sg, a.x.p[nn - 1], fout, (int)B, (int)D, true, work, w.rows_per_group, s, nullptr, a.io,
                     C + (nn - 1) * cstride, rev_c));
    if (B > 1) {
      if (L % 4 == 0) hipLaunchKernelGGL(k_bw_batch_sum<true>, row_grid(D, L / 4), dim3(EW_THREADS), 0, s, T1, gh_n, (int)B, (int)D, L);
      else hipLaunchKernelGGL(k_bw_batch_sum<false>, row_grid(D, L), dim3(EW_THREADS), 0, s, T1, gh_n, (int)B, (int)D, L);
      BW_TRY(hipGetLastError());
    }
    // adjoint: g_n = R(h_n conv R(g * x_n)).  Those spectra are already in sg,
    // so it starts at its row pass, whose reversal map returns g_n itself
    // (into gv directly for the last step, in the I/O dtype)
    float* gout = nn == 0 ? static_cast<float*>(a.gv) : T1;
    BW_TRY(bw_conv(p, spec_n(nn), nullptr, gout, (int)B, (int)D, false, work, w.rows_per_group, s, sg, 0, nullptr,
                   rev_c, nn == 0 && a.io == 1));
    gcur = T1;
  }
#undef BW_TRY
  return hipSuccess;
}

}  // namespace hyena
