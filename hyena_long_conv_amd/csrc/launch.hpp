// launch.hpp -- internal launch interface between the C ABI (api.cpp) and the
// kernel translation units.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace hyena {

struct ForwardArgs {
  const void* v;
  XPtrsHost x;           // N device pointers
  const void* spec;
  void* y;
  int B, D, NORD;        // batch, channels, order
  int64_t L;
  int io;                // 0 fp32, 1 bf16
  int64_t spec_stride;   // complex64 elements per filter row
  int n_rows;            // B * D real rows
  void* work;            // four-step intermediate (rows_per_group * N complex)
  int rows_per_group;
  int circular;          // single path: rows fill the whole FFT length (no zero half)
  int no_gate;           // four-step, fp32 rows: the last order stores the convolution without a gate
  const void* spec_in;   // four-step, one order, no gate: the input rows' spectra (filter-spectrum
                         // layout, one per row b*D + d) in place of v; nullptr otherwise
  float* csave;          // four-step, no gate: every order's convolution c_n (fp32 [B][D][L]) at
                         // csave + n * csave_stride, the last order's being the only output (y unused)
  int64_t csave_stride;
  const float* vc;       // four-step, one order: the input is xv * vc (xv = v in the I/O dtype, vc fp32)
  int rev_out;           // four-step, one order, no gate: the output row reversed, t -> (rev_c - t) mod L
                         // (by the spectral map with spec_in, else by the output pass's addressing)
  int out_bf16;          // four-step, no gate: unreversed output rows in bf16 instead of fp32
  int64_t rev_c;
};

struct SpectrumArgs {
  const float* h;        // [NF][L]
  void* spec;
  int NF;                // N*D
  int64_t L;
  int64_t spec_stride;
  void* work;
  int rows_per_group;
  int circular;
  // four-step, backward: rows h = g * x formed in the column pass, which also
  // stores gx = g * c (g: the I/O dtype, or fp32 with g_f32; c fp32; x, gx
  // the I/O dtype io); used when g is set
  const void* g;
  const float* c;
  const void* x;
  void* gx;
  int g_f32, io;
  // rev: the spectrum of the reversed row t -> (rev_c - t) mod M instead,
  // i.e. bins W_M^(rev_c k) conj X(k)
  int rev;
  int64_t rev_c;
};

struct FilterGenArgs {
  int D, N, K, H;
  const float *W1, *b1, *W2, *b2, *W3, *b3, *alpha;
  int64_t L;
  float* h;
};

// Dense projections around the operator (kernels_proj.hip).
struct StreamPtrs {
  void* p[9];            // v, x_1..x_N (N <= 8)
};

struct InProjArgs {
  const void* u;         // [B][L][D]
  const void* W;         // [C][D], C = (N+1)*D
  const float* bias;     // [C] or nullptr
  const float* w;        // [C][T]
  StreamPtrs dst;        // N+1 streams, each [B][D][L]
  int B, D, C, T;
  int64_t L;
  int io;
};

struct OutProjArgs {
  const void* y;         // [B][D][L]
  const void* W;         // [D][D]
  const float* bias;     // [D] or nullptr
  void* out;             // [B][L][D]
  int B, D;
  int64_t L;
  int io;
};

hipError_t in_projection(const InProjArgs& a, hipStream_t s);
hipError_t out_projection(const OutProjArgs& a, hipStream_t s);

// Backward of the recurrence (single-pass lengths).
struct OutPtrs {
  void* p[8];            // N device pointers
};

struct BackwardArgs {
  const void* v;
  XPtrsHost x;
  const void* spec;
  const void* gy;
  void* gv;
  OutPtrs gx;
  float* gh;             // [N][D][L]
  void* cbuf;            // workspace: N * B * D * N_c/2 complex (N_c when circular)
  void* hacc;            // workspace: N * D * N_c complex
  int B, D, NORD;
  int64_t L;
  int io;
  int64_t spec_stride;
  int circular;          // single path, L = 2 N_c: periodic convolution
};

hipError_t single_backward(const BackwardArgs& a, int64_t N, hipStream_t s);

// Backward on the four-step path (kernels_bwd_long.hip): byte offsets of its
// workspace buffers (saved c_n, z, g, two temporaries, the per-row spectra
// and the four-step intermediate).
struct LongBackwardLayout {
  int64_t c, t1, sg, work, total;
  int rows_per_group;
};
LongBackwardLayout long_backward_layout(const PlanInfo& p, int64_t B, int64_t D, int64_t NORD);
hipError_t long_backward(const BackwardArgs& a, const PlanInfo& p, void* workspace, hipStream_t s);

// Other filter families (kernels_fir.hip).
hipError_t filter_gen_li(const float* R, const float* lam, int NF, int S, int64_t L, float* h, hipStream_t s);
hipError_t filter_gen_mr(const float* hhat, const float* alpha, int D, int NF, int Lh, float* h, hipStream_t s);
hipError_t fir_forward(const ForwardArgs& a, const float* h, int Lh, hipStream_t s);

// Grid convolutions (kernels_nd.hip).
struct NdArgs {
  int ndim, P;            // 2 or 3 axes; padded FFT side (power of two)
  int Lo, Lm, Ll;         // grid sides: first, middle (1 for 2-D), last (contiguous)
  int circular;
  int64_t spec_stride;    // complex64 elements per kernel row
  void* spec;
  // spectrum
  const float* kernel;    // [rows][extent]
  int rows;
  // forward (rows = B * D grids)
  const void* v;
  XPtrsHost x;
  void* y;
  int D, NORD, per_sample, io;
  // multi-pass grids (2-D, P >= 256): intermediate of rows_per_group grids
  void* work;
  int rows_per_group;
};

hipError_t nd_spectrum(const NdArgs& a, hipStream_t s);
hipError_t nd_forward(const NdArgs& a, hipStream_t s);
hipError_t grid2d_spectrum(const NdArgs& a, hipStream_t s);   // kernels_fourstep.hip
hipError_t grid2d_forward(const NdArgs& a, hipStream_t s);
hipError_t grid3d_spectrum(const NdArgs& a, hipStream_t s);
hipError_t grid3d_forward(const NdArgs& a, hipStream_t s);
// plane pass of the 3-D multi-pass grids over `groups` grids from row r0
// (order n; spec: build the spectrum instead), kernels_nd.hip
hipError_t grid_plane_pass(const NdArgs& a, int r0, int groups, int n, bool spec, hipStream_t s);

// The static device scratch of hyena_forward_static (scratch.hip): its
// address on the current device (looked up once per device) and its size.
constexpr int64_t kStaticScratchBytes = int64_t(128) << 20;
hipError_t static_scratch(void** ptr, int64_t* bytes);

hipError_t single_forward(const ForwardArgs& a, int64_t N, hipStream_t s);
hipError_t single_spectrum(const SpectrumArgs& a, int64_t N, hipStream_t s);
hipError_t fourstep_forward(const ForwardArgs& a, const PlanInfo& p, hipStream_t s);
hipError_t fourstep_spectrum(const SpectrumArgs& a, const PlanInfo& p, hipStream_t s);
// The backward's fused passes (SpectrumArgs.g, reversed outputs) exist for
// every column kernel of the four-step forward: power-of-two columns, odd
// columns in registers and 2q columns on lane pairs.
inline bool fourstep_fused_spec_ok(const PlanInfo& p) {
  const int n1 = p.n1, q = n1 % 2 == 0 ? n1 / 2 : n1;
  const bool odd = q == 3 || q == 5 || q == 9 || q == 15 || q == 25 || q == 27;
  return (n1 >= 16 && (n1 & (n1 - 1)) == 0) || odd;
}
hipError_t filter_gen(const FilterGenArgs& a, hipStream_t s);
hipError_t spectrum_export(const void* spec, int NF, const PlanInfo& p, float* out, hipStream_t s);
hipError_t spectrum_to_fourstep(const void* spec, int NF, const PlanInfo& single, const PlanInfo& fs, void* out,
                                hipStream_t s);

}  // namespace hyena
