// api.cpp -- the extern "C" entry points declared in include/hyena.h.
//
// Every entry point validates its arguments on the host before it enqueues
// anything, so argument errors never reach the GPU.  The library allocates
// nothing: spectrum, workspace and outputs come from the caller.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "hyena.h"
#include "launch.hpp"
#include "plan.hpp"

using namespace hyena;

namespace {

int plan_env(int64_t L, PlanInfo* p, int circular = 0) {
  return make_plan(L, std::getenv("HYENA_FORCE_PATH"), std::getenv("HYENA_FOURSTEP_N1"), p, circular);
}

bool mode_ok(hyena_conv_mode m) { return m == HYENA_CONV_LINEAR || m == HYENA_CONV_CIRCULAR; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

hyena_status from_plan_code(int c) {
  return c == 0 ? HYENA_OK : (c == 2 ? HYENA_ERR_SHAPE : HYENA_ERR_UNSUPPORTED);
}

int64_t spec_bytes(const PlanInfo& p, int64_t NF) { return NF * p.spec_stride * 8; }

int64_t spectrum_ws(const PlanInfo& p, int64_t NF) {
  if (p.path == PATH_SINGLE) return 0;
  return (int64_t)rows_per_group(p.N, NF) * p.N * 8;
}

// Rows per pass group of the four-step forward (equal-size groups under the
// work budget, plan.hpp), for intermediate points of esz bytes.
int64_t forward_group_rows(const PlanInfo& p, int64_t n_rows, int64_t esz) { return rows_per_group(p.N, n_rows, esz); }

int64_t forward_ws(const PlanInfo& p, int64_t B, int64_t D, int N, hyena_dtype io) {
  if (p.path == PATH_SINGLE) return 0;
  const int64_t esz = forward_work_esz(io == HYENA_BF16, N);
  return forward_group_rows(p, B * D, esz) * p.N * esz;
}

// Grid convolutions: padded side P of the square/cube FFT grid.
struct NdPlanH {
  int ndim, P;
  int Lo, Lm, Ll;
  int64_t NC, Q, stride, points;
  bool multi;   // 2-D grids beyond one workgroup: column and row passes through a workspace
};

constexpr int kNdMaxSide = 4096;

int nd_plan(int32_t ndim, const int64_t* dims, int32_t circular, NdPlanH* out) {
  if (!dims) return 1;
  if (ndim != 2 && ndim != 3) return 3;
  if (circular != 0 && circular != 1) return 3;
  int64_t lmax = 0, points = 1;
  for (int a = 0; a < ndim; ++a) {
    if (dims[a] < 1 || dims[a] > kNdMaxSide) return 2;
    lmax = dims[a] > lmax ? dims[a] : lmax;
    points *= dims[a];
  }
  // single pass: 2-D up to 128, 3-D up to 32; multi-pass: 2-D 256..1024, 3-D 64 and 128
  const int pmin = ndim == 2 ? 16 : 8, pmax = ndim == 2 ? 1024 : 128;
  int64_t P;
  if (circular) {
    P = dims[0];
    for (int a = 1; a < ndim; ++a)
      if (dims[a] != P) return 3;
    if ((P & (P - 1)) != 0 || P < pmin || P > pmax) return 3;
  } else {
    P = pmin;
    while (P < 2 * lmax - 1) P *= 2;
    if (P > pmax) return 3;
  }
  NdPlanH p{};
  p.ndim = ndim;
  p.P = (int)P;
  p.Lo = (int)dims[0];
  p.Lm = ndim == 3 ? (int)dims[1] : 1;
  p.Ll = (int)dims[ndim - 1];
  p.Q = ndim == 2 ? P : P * P;
  p.NC = p.Q * (P / 2);
  p.stride = round_up(p.NC + p.Q, 64);
  p.points = points;
  p.multi = (ndim == 2 && P > 128) || (ndim == 3 && P > 32);
  *out = p;
  return 0;
}

// Grids per pass group: as many groups as the work budget needs, of equal size.
int64_t nd_group_rows(const NdPlanH& p, int64_t rows) { return rows_per_group(p.NC, rows); }

int64_t nd_ws(const NdPlanH& p, int64_t rows) {
  return p.multi ? nd_group_rows(p, rows) * p.NC * 8 : 0;
}

// 0: fine; otherwise a status.  Sets the grids per pass group.
hyena_status nd_ws_check(const NdPlanH& p, int64_t rows, void* ws, int64_t wsb, int* group) {
  *group = 0;
  if (!p.multi) return HYENA_OK;
  if (!ws || wsb < p.NC * 8) return HYENA_ERR_WORKSPACE;
  if (!aligned16(ws)) return HYENA_ERR_ALIGN;
  int64_t g = nd_group_rows(p, rows);
  if (g * p.NC * 8 > wsb) g = wsb / (p.NC * 8);
  *group = (int)g;
  return HYENA_OK;
}

int64_t nd_kernel_extent(const NdPlanH& p, int32_t circular) {
  int64_t e = 1;
  const int sides[3] = {p.Lo, p.Lm, p.Ll};
  for (int a = 0; a < 3; ++a) {
    if (p.ndim == 2 && a == 1) continue;
    e *= circular ? sides[a] : 2 * (int64_t)sides[a] - 1;
  }
  return e;
}

bool sizes_ok(int64_t D, int64_t N, int64_t L) {
  return D >= 1 && D <= (1 << 20) && N >= 1 && L >= 1 && L <= kMaxL;
}

}  // namespace

namespace hyena {

// Byte offsets of the long backward's workspace buffers: N saved c_n, one
// temporary (fp32 rows), the per-row spectra and the four-step intermediate
// of one pass group.
LongBackwardLayout long_backward_layout(const PlanInfo& p, int64_t B, int64_t D, int64_t NORD) {
  const auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t R = B * D, act = al(R * p.L * 4);
  LongBackwardLayout w{};
  int64_t o = 0;
  w.c = o;     o += NORD * act;
  w.t1 = o;    o += act;
  w.sg = o;    o += al(R * p.spec_stride * 8);
  // as many pass groups as the work budget needs, of equal size (plan.hpp)
  w.rows_per_group = rows_per_group(p.N, R);
  w.work = o;  o += al((int64_t)w.rows_per_group * p.N * 8);
  w.total = o;
  return w;
}

}  // namespace hyena

extern "C" {

const char* hyena_status_str(hyena_status s) {
  switch (s) {
    case HYENA_OK: return "ok";
    case HYENA_ERR_NULL: return "a required pointer is NULL";
    case HYENA_ERR_SHAPE: return "a size is out of range";
    case HYENA_ERR_UNSUPPORTED: return "unsupported configuration";
    case HYENA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case HYENA_ERR_WORKSPACE: return "workspace missing or too small";
    case HYENA_ERR_ALIAS: return "the output overlaps an input";
    case HYENA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

hyena_status hyena_plan(int64_t L, hyena_plan_info* out) { return hyena_plan_ex(L, HYENA_CONV_LINEAR, out); }

hyena_status hyena_plan_ex(int64_t L, hyena_conv_mode mode, hyena_plan_info* out) {
  if (!out) return HYENA_ERR_NULL;
  if (!mode_ok(mode)) return HYENA_ERR_UNSUPPORTED;
  PlanInfo p;
  const int c = plan_env(L, &p, mode);
  if (c) return from_plan_code(c);
  out->L = p.L;
  out->M = p.M;
  out->path = p.path;
  out->n1 = p.n1;
  out->n2 = p.n2;
  out->reserved = 0;
  out->spec_stride = p.spec_stride;
  return HYENA_OK;
}

hyena_status hyena_filter_gen(const hyena_filter_params* p, int64_t L, float* h, void* stream) {
  if (!p || !h || !p->W1 || !p->W2 || !p->W3 || !p->alpha) return HYENA_ERR_NULL;
  if (!sizes_ok(p->D, p->N, L) || p->K < 0 || p->K > kMaxFreq) return HYENA_ERR_SHAPE;
  if (p->N > kMaxOrder) return HYENA_ERR_UNSUPPORTED;
  if (p->H != 8 && p->H != 16 && p->H != 32 && p->H != 64 && p->H != 128) return HYENA_ERR_UNSUPPORTED;
  if ((int64_t)p->N * p->D > 65535LL * 64) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(h)) return HYENA_ERR_ALIGN;
  FilterGenArgs a{};
  a.D = p->D; a.N = p->N; a.K = p->K; a.H = p->H;
  a.W1 = p->W1; a.b1 = p->b1; a.W2 = p->W2; a.b2 = p->b2; a.W3 = p->W3; a.b3 = p->b3;
  a.alpha = p->alpha; a.L = L; a.h = h;
  return filter_gen(a, (hipStream_t)stream) == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

int64_t hyena_spectrum_bytes(int32_t D, int32_t N, int64_t L) {
  return hyena_spectrum_bytes_ex(D, N, L, HYENA_CONV_LINEAR);
}

int64_t hyena_spectrum_bytes_ex(int32_t D, int32_t N, int64_t L, hyena_conv_mode mode) {
  if (!sizes_ok(D, N, L) || N > kMaxOrder || !mode_ok(mode)) return -1;
  PlanInfo p;
  if (plan_env(L, &p, mode)) return -1;
  return spec_bytes(p, (int64_t)N * D);
}

int64_t hyena_spectrum_workspace_bytes(int32_t D, int32_t N, int64_t L) {
  return hyena_spectrum_workspace_bytes_ex(D, N, L, HYENA_CONV_LINEAR);
}

int64_t hyena_spectrum_workspace_bytes_ex(int32_t D, int32_t N, int64_t L, hyena_conv_mode mode) {
  if (!sizes_ok(D, N, L) || N > kMaxOrder || !mode_ok(mode)) return -1;
  PlanInfo p;
  if (plan_env(L, &p, mode)) return -1;
  return spectrum_ws(p, (int64_t)N * D);
}

hyena_status hyena_filter_spectrum(const float* h, int32_t D, int32_t N, int64_t L, void* spec,
                                   void* workspace, int64_t workspace_bytes, void* stream) {
  return hyena_filter_spectrum_ex(h, D, N, L, HYENA_CONV_LINEAR, spec, workspace, workspace_bytes, stream);
}

hyena_status hyena_filter_spectrum_ex(const float* h, int32_t D, int32_t N, int64_t L, hyena_conv_mode mode,
                                      void* spec, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!h || !spec) return HYENA_ERR_NULL;
  if (!sizes_ok(D, N, L)) return HYENA_ERR_SHAPE;
  if (N > kMaxOrder || !mode_ok(mode)) return HYENA_ERR_UNSUPPORTED;
  PlanInfo p;
  const int c = plan_env(L, &p, mode);
  if (c) return from_plan_code(c);
  const int64_t NF = (int64_t)N * D;
  if (!aligned16(h) || !aligned16(spec) || (workspace && !aligned16(workspace))) return HYENA_ERR_ALIGN;
  const int64_t need = spectrum_ws(p, NF);
  if (need > 0 && (!workspace || workspace_bytes < p.N * 8)) return HYENA_ERR_WORKSPACE;
  if (overlap(spec, spec_bytes(p, NF), h, NF * L * 4)) return HYENA_ERR_ALIAS;
  if (workspace && need > 0 && (overlap(workspace, workspace_bytes, h, NF * L * 4) ||
                                overlap(workspace, workspace_bytes, spec, spec_bytes(p, NF))))
    return HYENA_ERR_ALIAS;
  SpectrumArgs a{};
  a.h = h; a.spec = spec; a.NF = (int)NF; a.L = L; a.spec_stride = p.spec_stride;
  a.work = workspace;
  a.circular = p.circular;
  hipError_t e;
  if (p.path == PATH_SINGLE) {
    e = single_spectrum(a, p.N, (hipStream_t)stream);
  } else {
    int64_t g = rows_per_group(p.N, NF);
    if (g * p.N * 8 > workspace_bytes) g = workspace_bytes / (p.N * 8);
    a.rows_per_group = (int)g;
    e = fourstep_spectrum(a, p, (hipStream_t)stream);
  }
  return e == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

hyena_status hyena_spectrum_export(const void* spec, int32_t D, int32_t N, int64_t L, float* out,
                                   void* stream) {
  return hyena_spectrum_export_ex(spec, D, N, L, HYENA_CONV_LINEAR, out, stream);
}

hyena_status hyena_spectrum_export_ex(const void* spec, int32_t D, int32_t N, int64_t L, hyena_conv_mode mode,
                                      float* out, void* stream) {
  if (!spec || !out) return HYENA_ERR_NULL;
  if (!sizes_ok(D, N, L)) return HYENA_ERR_SHAPE;
  if (N > kMaxOrder || !mode_ok(mode)) return HYENA_ERR_UNSUPPORTED;
  PlanInfo p;
  const int c = plan_env(L, &p, mode);
  if (c) return from_plan_code(c);
  if (!aligned16(spec) || !aligned16(out)) return HYENA_ERR_ALIGN;
  const int64_t NF = (int64_t)N * D;
  if (overlap(out, NF * (p.N + 1) * 8, spec, spec_bytes(p, NF))) return HYENA_ERR_ALIAS;
  return spectrum_export(spec, (int)NF, p, out, (hipStream_t)stream) == hipSuccess ? HYENA_OK
                                                                                   : HYENA_ERR_HIP;
}

int64_t hyena_forward_workspace_bytes(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io) {
  return hyena_forward_workspace_bytes_ex(B, D, N, L, io, HYENA_CONV_LINEAR);
}

int64_t hyena_forward_workspace_bytes_ex(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io,
                                         hyena_conv_mode mode) {
  if (B < 1 || B > (1 << 20) || !sizes_ok(D, N, L) || N > kMaxOrder || !mode_ok(mode)) return -1;
  if (io != HYENA_FP32 && io != HYENA_BF16) return -1;
  PlanInfo p;
  if (plan_env(L, &p, mode)) return -1;
  return forward_ws(p, B, D, N, io);
}

hyena_status hyena_forward(const void* v, const void* const* x, const void* spec, void* y, int64_t B,
                           int32_t D, int32_t N, int64_t L, hyena_dtype io, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  return hyena_forward_ex(v, x, spec, y, B, D, N, L, io, HYENA_CONV_LINEAR, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The forward's argument checks and launch.  static_ws: the four-step
// intermediate goes to the library's static device scratch (looked up on
// the current device) instead of the caller's workspace.
hyena_status forward_impl(const void* v, const void* const* x, const void* spec, void* y, int64_t B, int32_t D,
                          int32_t N, int64_t L, hyena_dtype io, hyena_conv_mode mode, void* workspace,
                          int64_t workspace_bytes, bool static_ws, void* stream) {
  if (!v || !x || !spec || !y) return HYENA_ERR_NULL;
  if (B < 1 || B > (1 << 20) || !sizes_ok(D, N, L)) return HYENA_ERR_SHAPE;
  if (N > kMaxOrder || !mode_ok(mode)) return HYENA_ERR_UNSUPPORTED;
  if (io != HYENA_FP32 && io != HYENA_BF16) return HYENA_ERR_UNSUPPORTED;
  for (int n = 0; n < N; ++n)
    if (!x[n]) return HYENA_ERR_NULL;
  if (B * D > ((int64_t)1 << 30)) return HYENA_ERR_UNSUPPORTED;
  PlanInfo p;
  const int c = plan_env(L, &p, mode);
  if (c) return from_plan_code(c);
  if (!aligned16(v) || !aligned16(y) || !aligned16(spec) || (workspace && !aligned16(workspace)))
    return HYENA_ERR_ALIGN;
  for (int n = 0; n < N; ++n)
    if (!aligned16(x[n])) return HYENA_ERR_ALIGN;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  const int64_t act = B * D * L * esz;
  const int64_t sb = spec_bytes(p, (int64_t)N * D);
  if (overlap(y, act, v, act) || overlap(y, act, spec, sb)) return HYENA_ERR_ALIAS;
  for (int n = 0; n < N; ++n)
    if (overlap(y, act, x[n], act)) return HYENA_ERR_ALIAS;
  if (static_ws) {
    void* sp = nullptr;
    int64_t sbytes = 0;
    if (static_scratch(&sp, &sbytes) != hipSuccess) return HYENA_ERR_HIP;
    workspace = sp;
    workspace_bytes = sbytes;
  }
  ForwardArgs a{};
  a.v = v;
  for (int n = 0; n < N; ++n) a.x.p[n] = x[n];
  a.spec = spec; a.y = y; a.B = (int)B; a.D = D; a.NORD = N; a.L = L;
  a.io = (io == HYENA_FP32) ? 0 : 1;
  a.spec_stride = p.spec_stride;
  a.n_rows = (int)(B * D);
  a.circular = p.circular;
  hipError_t e;
  if (p.path == PATH_SINGLE) {
    e = single_forward(a, p.N, (hipStream_t)stream);
  } else {
    const int64_t esz = forward_work_esz(a.io == 1, N), row_bytes = p.N * esz;
    if (static_ws) {
      if (row_bytes > workspace_bytes) return HYENA_ERR_WORKSPACE;   // one row's intermediate must fit
    } else {
      if (!workspace || workspace_bytes < row_bytes) return HYENA_ERR_WORKSPACE;
      if (overlap(workspace, workspace_bytes, y, act) || overlap(workspace, workspace_bytes, v, act) ||
          overlap(workspace, workspace_bytes, spec, sb))
        return HYENA_ERR_ALIAS;
      for (int n = 0; n < N; ++n)
        if (overlap(workspace, workspace_bytes, x[n], act)) return HYENA_ERR_ALIAS;
    }
    int64_t g = forward_group_rows(p, B * D, esz);
    if (g * row_bytes > workspace_bytes) g = workspace_bytes / row_bytes;
    a.work = workspace;
    a.rows_per_group = (int)g;
    e = fourstep_forward(a, p, (hipStream_t)stream);
  }
  return e == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

}  // namespace

extern "C" {

hyena_status hyena_forward_ex(const void* v, const void* const* x, const void* spec, void* y, int64_t B,
                              int32_t D, int32_t N, int64_t L, hyena_dtype io, hyena_conv_mode mode,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  return forward_impl(v, x, spec, y, B, D, N, L, io, mode, workspace, workspace_bytes, false, stream);
}

static_assert(HYENA_STATIC_SCRATCH_BYTES == kStaticScratchBytes, "header and library disagree on the scratch size");

hyena_status hyena_forward_static(const void* v, const void* const* x, const void* spec, void* y, int64_t B,
                                  int32_t D, int32_t N, int64_t L, hyena_dtype io, void* stream) {
  return forward_impl(v, x, spec, y, B, D, N, L, io, HYENA_CONV_LINEAR, nullptr, 0, true, stream);
}

// ------------------------------------------------------- filter families

hyena_status hyena_filter_gen_li(const float* R, const float* lambda, int32_t D, int32_t N, int32_t S, int64_t L,
                                 float* h, void* stream) {
  if (!R || !lambda || !h) return HYENA_ERR_NULL;
  if (!sizes_ok(D, N, L) || N > kMaxOrder || S < 1 || S > 64) return HYENA_ERR_SHAPE;
  if (!aligned16(h)) return HYENA_ERR_ALIGN;
  const int64_t NF = (int64_t)N * D;
  if (overlap(h, NF * L * 4, R, NF * S * 4) || overlap(h, NF * L * 4, lambda, NF * S * 4)) return HYENA_ERR_ALIAS;
  return filter_gen_li(R, lambda, (int)NF, S, L, h, (hipStream_t)stream) == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

hyena_status hyena_filter_gen_mr(const float* hhat, const float* alpha, int32_t D, int32_t N, int32_t Lh, float* h,
                                 void* stream) {
  if (!hhat || !alpha || !h) return HYENA_ERR_NULL;
  if (!sizes_ok(D, N, 1) || N > kMaxOrder || Lh < 1 || Lh > kMaxL) return HYENA_ERR_SHAPE;
  if (!aligned16(h)) return HYENA_ERR_ALIGN;
  const int64_t NF = (int64_t)N * D;
  if (h != hhat && overlap(h, NF * Lh * 4, hhat, NF * Lh * 4)) return HYENA_ERR_ALIAS;   // in place is fine
  return filter_gen_mr(hhat, alpha, D, (int)NF, Lh, h, (hipStream_t)stream) == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

hyena_status hyena_forward_fir(const void* v, const void* const* x, const float* h, int32_t Lh, void* y, int64_t B,
                               int32_t D, int32_t N, int64_t L, hyena_dtype io, void* stream) {
  if (!v || !x || !h || !y) return HYENA_ERR_NULL;
  if (B < 1 || B > (1 << 20) || !sizes_ok(D, N, L) || Lh < 1 || Lh > HYENA_MAX_FIR) return HYENA_ERR_SHAPE;
  if (N > kMaxOrder) return HYENA_ERR_UNSUPPORTED;
  if (io != HYENA_FP32 && io != HYENA_BF16) return HYENA_ERR_UNSUPPORTED;
  for (int n = 0; n < N; ++n)
    if (!x[n]) return HYENA_ERR_NULL;
  if (B * D > ((int64_t)1 << 30)) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(v) || !aligned16(y) || !aligned16(h)) return HYENA_ERR_ALIGN;
  for (int n = 0; n < N; ++n)
    if (!aligned16(x[n])) return HYENA_ERR_ALIGN;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  const int64_t act = B * D * L * esz;
  if (overlap(y, act, v, act) || overlap(y, act, h, (int64_t)N * D * Lh * 4)) return HYENA_ERR_ALIAS;
  for (int n = 0; n < N; ++n)
    if (overlap(y, act, x[n], act)) return HYENA_ERR_ALIAS;
  ForwardArgs a{};
  a.v = v;
  for (int n = 0; n < N; ++n) a.x.p[n] = x[n];
  a.y = y; a.B = (int)B; a.D = D; a.NORD = N; a.L = L;
  a.io = (io == HYENA_FP32) ? 0 : 1;
  a.n_rows = (int)(B * D);
  return fir_forward(a, h, Lh, (hipStream_t)stream) == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

// --------------------------------------------------------------- backward

namespace {
constexpr int64_t kBackwardMaxN = 8192;   // complex points of the single-pass backward

int64_t bwd_ws_single(const PlanInfo& p, int64_t B, int64_t D, int64_t NORD) {
  const int64_t cb = (NORD * B * D * (p.circular ? p.N : p.N / 2) * 8 + 255) / 256 * 256;
  return cb + NORD * D * p.N * 8;
}

bool bwd_single(const PlanInfo& p) { return p.path == PATH_SINGLE && p.N <= kBackwardMaxN; }

// The four-step plan the long backward runs on (the forward's own plan, or a
// four-step plan of the same length for single-path spectra too long for
// the one-workgroup backward).
int bwd_long_plan(const PlanInfo& p, PlanInfo* fs) {
  if (p.path != PATH_SINGLE) {
    *fs = p;
    return 0;
  }
  return make_plan(p.L, "fourstep", nullptr, fs, p.circular);
}

int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }

// -1 when no backward serves the plan
int64_t bwd_ws(const PlanInfo& p, int64_t B, int64_t D, int64_t NORD) {
  if (bwd_single(p)) return bwd_ws_single(p, B, D, NORD);
  PlanInfo fs;
  if (bwd_long_plan(p, &fs)) return -1;
  int64_t t = long_backward_layout(fs, B, D, NORD).total;
  if (p.path == PATH_SINGLE) t += al256(NORD * D * fs.spec_stride * 8);   // spectrum in the four-step layout
  return t;
}
}  // namespace

int64_t hyena_backward_workspace_bytes(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io) {
  return hyena_backward_workspace_bytes_ex(B, D, N, L, io, HYENA_CONV_LINEAR);
}

int64_t hyena_backward_workspace_bytes_ex(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io,
                                          hyena_conv_mode mode) {
  if (B < 1 || B > (1 << 20) || !sizes_ok(D, N, L) || N > kMaxOrder) return -1;
  if (io != HYENA_FP32 && io != HYENA_BF16) return -1;
  if (mode != HYENA_CONV_LINEAR && mode != HYENA_CONV_CIRCULAR) return -1;
  PlanInfo p;
  if (plan_env(L, &p, mode)) return -1;
  if (B * D > ((int64_t)1 << 30)) return -1;
  return bwd_ws(p, B, D, N);
}

hyena_status hyena_backward(const void* v, const void* const* x, const void* spec, const void* gy, void* gv,
                            void* const* gx, float* gh, int64_t B, int32_t D, int32_t N, int64_t L,
                            hyena_dtype io, void* workspace, int64_t workspace_bytes, void* stream) {
  return hyena_backward_ex(v, x, spec, gy, gv, gx, gh, B, D, N, L, io, HYENA_CONV_LINEAR, workspace,
                           workspace_bytes, stream);
}

hyena_status hyena_backward_ex(const void* v, const void* const* x, const void* spec, const void* gy, void* gv,
                               void* const* gx, float* gh, int64_t B, int32_t D, int32_t N, int64_t L,
                               hyena_dtype io, hyena_conv_mode mode, void* workspace, int64_t workspace_bytes,
                               void* stream) {
  if (!v || !x || !spec || !gy || !gv || !gx || !gh || !workspace) return HYENA_ERR_NULL;
  if (B < 1 || B > (1 << 20) || !sizes_ok(D, N, L)) return HYENA_ERR_SHAPE;
  if (N > kMaxOrder) return HYENA_ERR_UNSUPPORTED;
  if (io != HYENA_FP32 && io != HYENA_BF16) return HYENA_ERR_UNSUPPORTED;
  if (mode != HYENA_CONV_LINEAR && mode != HYENA_CONV_CIRCULAR) return HYENA_ERR_UNSUPPORTED;
  for (int n = 0; n < N; ++n)
    if (!x[n] || !gx[n]) return HYENA_ERR_NULL;
  PlanInfo p;
  const int c = plan_env(L, &p, mode);
  if (c) return from_plan_code(c);
  if (B * D > ((int64_t)1 << 30)) return HYENA_ERR_UNSUPPORTED;
  const int64_t need = bwd_ws(p, B, D, N);
  if (need < 0) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(v) || !aligned16(spec) || !aligned16(gy) || !aligned16(gv) || !aligned16(gh) ||
      !aligned16(workspace))
    return HYENA_ERR_ALIGN;
  for (int n = 0; n < N; ++n)
    if (!aligned16(x[n]) || !aligned16(gx[n])) return HYENA_ERR_ALIGN;
  if (workspace_bytes < need) return HYENA_ERR_WORKSPACE;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  const int64_t act = B * D * L * esz, sb = spec_bytes(p, (int64_t)N * D), ghb = (int64_t)N * D * L * 4;
  // outputs: gv, gx_1..gx_N, gh, workspace; inputs: v, x_1..x_N, spec, gy
  const void* outs[11];
  int64_t osz[11];
  int no = 0;
  outs[no] = gv; osz[no++] = act;
  for (int n = 0; n < N; ++n) { outs[no] = gx[n]; osz[no++] = act; }
  outs[no] = gh; osz[no++] = ghb;
  outs[no] = workspace; osz[no++] = need;
  for (int i = 0; i < no; ++i) {
    if (overlap(outs[i], osz[i], v, act) || overlap(outs[i], osz[i], spec, sb) || overlap(outs[i], osz[i], gy, act))
      return HYENA_ERR_ALIAS;
    for (int n = 0; n < N; ++n)
      if (overlap(outs[i], osz[i], x[n], act)) return HYENA_ERR_ALIAS;
    for (int k = 0; k < i; ++k)
      if (overlap(outs[i], osz[i], outs[k], osz[k])) return HYENA_ERR_ALIAS;
  }
  BackwardArgs a{};
  a.v = v;
  for (int n = 0; n < N; ++n) { a.x.p[n] = x[n]; a.gx.p[n] = gx[n]; }
  a.spec = spec; a.gy = gy; a.gv = gv; a.gh = gh;
  a.B = (int)B; a.D = D; a.NORD = N; a.L = L;
  a.io = (io == HYENA_FP32) ? 0 : 1;
  a.spec_stride = p.spec_stride;
  a.circular = p.circular;
  if (!bwd_single(p)) {
    PlanInfo fs;
    if (bwd_long_plan(p, &fs)) return HYENA_ERR_UNSUPPORTED;
    if (p.path == PATH_SINGLE) {
      // the caller's spectrum has the single-path layout: rewrite it after the long backward's buffers
      void* conv = static_cast<char*>(workspace) + long_backward_layout(fs, B, D, N).total;
      if (spectrum_to_fourstep(spec, N * D, p, fs, conv, (hipStream_t)stream) != hipSuccess) return HYENA_ERR_HIP;
      a.spec = conv;
    }
    a.spec_stride = fs.spec_stride;
    return long_backward(a, fs, workspace, (hipStream_t)stream) == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
  }
  a.cbuf = workspace;
  a.hacc = static_cast<char*>(workspace) + (need - (int64_t)N * D * p.N * 8);
  return single_backward(a, p.N, (hipStream_t)stream) == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

// ------------------------------------------------------------------ block

namespace {

bool block_params_ok(const hyena_block_params* p) {
  return p->D >= 1 && p->D <= (1 << 16) && p->N >= 1 && p->T >= 1 && p->T <= HYENA_MAX_SHORT;
}

hyena_status check_in_projection(const void* u, const hyena_block_params* p, void* const* streams, int64_t B,
                                 int64_t L, hyena_dtype io) {
  if (!u || !p || !streams || !p->W_in || !p->w_short) return HYENA_ERR_NULL;
  if (!block_params_ok(p) || B < 1 || B > (1 << 20) || L < 1 || L > kMaxL) return HYENA_ERR_SHAPE;
  if (p->N > kMaxOrder) return HYENA_ERR_UNSUPPORTED;
  if (io != HYENA_FP32 && io != HYENA_BF16) return HYENA_ERR_UNSUPPORTED;
  for (int s = 0; s <= p->N; ++s)
    if (!streams[s]) return HYENA_ERR_NULL;
  if (!aligned16(u) || !aligned16(p->W_in) || !aligned16(p->w_short) || (p->b_in && !aligned16(p->b_in)))
    return HYENA_ERR_ALIGN;
  for (int s = 0; s <= p->N; ++s)
    if (!aligned16(streams[s])) return HYENA_ERR_ALIGN;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  const int64_t act = B * p->D * L * esz;
  const int64_t C = (int64_t)(p->N + 1) * p->D;
  for (int s = 0; s <= p->N; ++s) {
    if (overlap(streams[s], act, u, act) || overlap(streams[s], act, p->W_in, C * p->D * esz)) return HYENA_ERR_ALIAS;
    for (int r = 0; r < s; ++r)
      if (overlap(streams[s], act, streams[r], act)) return HYENA_ERR_ALIAS;
  }
  return HYENA_OK;
}

hyena_status check_out_projection(const void* y, const hyena_block_params* p, void* out, int64_t B, int64_t L,
                                  hyena_dtype io) {
  if (!y || !p || !out || !p->W_out) return HYENA_ERR_NULL;
  if (!block_params_ok(p) || B < 1 || B > (1 << 20) || L < 1 || L > kMaxL) return HYENA_ERR_SHAPE;
  if (io != HYENA_FP32 && io != HYENA_BF16) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(y) || !aligned16(out) || !aligned16(p->W_out) || (p->b_out && !aligned16(p->b_out)))
    return HYENA_ERR_ALIGN;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  const int64_t act = B * p->D * L * esz;
  if (overlap(out, act, y, act) || overlap(out, act, p->W_out, (int64_t)p->D * p->D * esz)) return HYENA_ERR_ALIAS;
  return HYENA_OK;
}

InProjArgs in_args(const void* u, const hyena_block_params* p, void* const* streams, int64_t B, int64_t L,
                   hyena_dtype io) {
  InProjArgs a{};
  a.u = u; a.W = p->W_in; a.bias = p->b_in; a.w = p->w_short;
  for (int s = 0; s <= p->N; ++s) a.dst.p[s] = streams[s];
  a.B = (int)B; a.D = p->D; a.C = (p->N + 1) * p->D; a.T = p->T; a.L = L;
  a.io = (io == HYENA_FP32) ? 0 : 1;
  return a;
}

OutProjArgs out_args(const void* y, const hyena_block_params* p, void* out, int64_t B, int64_t L, hyena_dtype io) {
  OutProjArgs a{};
  a.y = y; a.W = p->W_out; a.bias = p->b_out; a.out = out;
  a.B = (int)B; a.D = p->D; a.L = L;
  a.io = (io == HYENA_FP32) ? 0 : 1;
  return a;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

hyena_status hyena_in_projection(const void* u, const hyena_block_params* p, void* const* streams, int64_t B,
                                 int64_t L, hyena_dtype io, void* stream) {
  const hyena_status st = check_in_projection(u, p, streams, B, L, io);
  if (st != HYENA_OK) return st;
  return in_projection(in_args(u, p, streams, B, L, io), (hipStream_t)stream) == hipSuccess ? HYENA_OK
                                                                                             : HYENA_ERR_HIP;
}

hyena_status hyena_out_projection(const void* y, const hyena_block_params* p, void* out, int64_t B, int64_t L,
                                  hyena_dtype io, void* stream) {
  const hyena_status st = check_out_projection(y, p, out, B, L, io);
  if (st != HYENA_OK) return st;
  return out_projection(out_args(y, p, out, B, L, io), (hipStream_t)stream) == hipSuccess ? HYENA_OK
                                                                                          : HYENA_ERR_HIP;
}

int64_t hyena_block_workspace_bytes(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io) {
  const int64_t fw = hyena_forward_workspace_bytes(B, D, N, L, io);
  if (fw < 0) return -1;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  return (int64_t)(N + 2) * align256(B * D * L * esz) + align256(fw);
}

hyena_status hyena_block_forward(const void* u, const hyena_block_params* p, const void* spec, void* out, int64_t B,
                                 int64_t L, hyena_dtype io, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!u || !p || !spec || !out || !workspace) return HYENA_ERR_NULL;
  if (!block_params_ok(p) || B < 1 || B > (1 << 20) || L < 1 || L > kMaxL) return HYENA_ERR_SHAPE;
  if (p->N > kMaxOrder) return HYENA_ERR_UNSUPPORTED;
  if (io != HYENA_FP32 && io != HYENA_BF16) return HYENA_ERR_UNSUPPORTED;
  const int64_t need = hyena_block_workspace_bytes(B, p->D, p->N, L, io);
  if (need < 0) return HYENA_ERR_SHAPE;
  if (!aligned16(workspace)) return HYENA_ERR_ALIGN;
  if (workspace_bytes < need) return HYENA_ERR_WORKSPACE;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  const int64_t act = B * p->D * L * esz, slot = align256(act);
  if (overlap(out, act, u, act)) return HYENA_ERR_ALIAS;
  if (overlap(workspace, need, u, act) || overlap(workspace, need, out, act)) return HYENA_ERR_ALIAS;
  char* w = static_cast<char*>(workspace);
  void* streams[9];
  for (int s = 0; s <= p->N; ++s) streams[s] = w + s * slot;
  void* y = w + (p->N + 1) * slot;
  void* fws = w + (p->N + 2) * slot;
  const int64_t fwb = need - (p->N + 2) * slot;
  hyena_status st = hyena_in_projection(u, p, streams, B, L, io, stream);
  if (st != HYENA_OK) return st;
  st = hyena_forward(streams[0], streams + 1, spec, y, B, p->D, p->N, L, io, fwb > 0 ? fws : nullptr, fwb, stream);
  if (st != HYENA_OK) return st;
  return hyena_out_projection(y, p, out, B, L, io, stream);
}

}  // extern "C"

// ------------------------------------------------------- grid convolutions

extern "C" {

hyena_status hyena_nd_plan(int32_t ndim, const int64_t* dims, int32_t circular, int64_t* padded_side) {
  if (!dims || !padded_side) return HYENA_ERR_NULL;
  NdPlanH p;
  const int c = nd_plan(ndim, dims, circular, &p);
  if (c) return c == 2 ? HYENA_ERR_SHAPE : HYENA_ERR_UNSUPPORTED;
  *padded_side = p.P;
  return HYENA_OK;
}

int64_t hyena_nd_spectrum_bytes(int32_t rows, int32_t ndim, const int64_t* dims, int32_t circular) {
  NdPlanH p;
  if (rows < 1 || nd_plan(ndim, dims, circular, &p)) return -1;
  return (int64_t)rows * p.stride * 8;
}

int64_t hyena_nd_workspace_bytes(int64_t rows, int32_t ndim, const int64_t* dims, int32_t circular) {
  NdPlanH p;
  if (rows < 1 || rows > ((int64_t)1 << 30) || nd_plan(ndim, dims, circular, &p)) return -1;
  return nd_ws(p, rows);
}

hyena_status hyena_nd_filter_spectrum(const float* kernel, int32_t rows, int32_t ndim, const int64_t* dims,
                                      int32_t circular, void* spec, void* workspace, int64_t workspace_bytes,
                                      void* stream) {
  if (!kernel || !spec || !dims) return HYENA_ERR_NULL;
  if (rows < 1 || rows > (1 << 24)) return HYENA_ERR_SHAPE;
  NdPlanH p;
  const int c = nd_plan(ndim, dims, circular, &p);
  if (c) return c == 2 ? HYENA_ERR_SHAPE : HYENA_ERR_UNSUPPORTED;
  if (!aligned16(kernel) || !aligned16(spec)) return HYENA_ERR_ALIGN;
  const int64_t kb = (int64_t)rows * nd_kernel_extent(p, circular) * 4, sb = (int64_t)rows * p.stride * 8;
  if (overlap(spec, sb, kernel, kb)) return HYENA_ERR_ALIAS;
  int group;
  const hyena_status ws = nd_ws_check(p, rows, workspace, workspace_bytes, &group);
  if (ws != HYENA_OK) return ws;
  if (p.multi && (overlap(workspace, workspace_bytes, spec, sb) || overlap(workspace, workspace_bytes, kernel, kb)))
    return HYENA_ERR_ALIAS;
  NdArgs a{};
  a.ndim = p.ndim; a.P = p.P; a.Lo = p.Lo; a.Lm = p.Lm; a.Ll = p.Ll;
  a.circular = circular;
  a.spec_stride = p.stride;
  a.spec = spec;
  a.kernel = kernel;
  a.rows = rows;
  a.work = workspace;
  a.rows_per_group = group;
  const hipError_t e = !p.multi ? nd_spectrum(a, (hipStream_t)stream)
                                : (p.ndim == 2 ? grid2d_spectrum(a, (hipStream_t)stream)
                                               : grid3d_spectrum(a, (hipStream_t)stream));
  return e == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

hyena_status hyena_nd_forward(const void* v, const void* const* x, const void* spec, void* y, int64_t B,
                              int32_t D, int32_t N, int32_t ndim, const int64_t* dims, int32_t circular,
                              int32_t per_sample, hyena_dtype io, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  if (!v || !x || !spec || !y || !dims) return HYENA_ERR_NULL;
  if (B < 1 || B > (1 << 20) || D < 1 || D > (1 << 20) || N < 1) return HYENA_ERR_SHAPE;
  if (N > kMaxOrder || (per_sample != 0 && per_sample != 1)) return HYENA_ERR_UNSUPPORTED;
  if (io != HYENA_FP32 && io != HYENA_BF16) return HYENA_ERR_UNSUPPORTED;
  for (int n = 0; n < N; ++n)
    if (!x[n]) return HYENA_ERR_NULL;
  NdPlanH p;
  const int c = nd_plan(ndim, dims, circular, &p);
  if (c) return c == 2 ? HYENA_ERR_SHAPE : HYENA_ERR_UNSUPPORTED;
  if (B * D > ((int64_t)1 << 30)) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(v) || !aligned16(y) || !aligned16(spec)) return HYENA_ERR_ALIGN;
  for (int n = 0; n < N; ++n)
    if (!aligned16(x[n])) return HYENA_ERR_ALIGN;
  const int64_t esz = (io == HYENA_FP32) ? 4 : 2;
  const int64_t act = B * D * p.points * esz;
  const int64_t sb = (per_sample ? B : 1) * (int64_t)N * D * p.stride * 8;
  if (overlap(y, act, v, act) || overlap(y, act, spec, sb)) return HYENA_ERR_ALIAS;
  for (int n = 0; n < N; ++n)
    if (overlap(y, act, x[n], act)) return HYENA_ERR_ALIAS;
  int group;
  const hyena_status ws = nd_ws_check(p, B * D, workspace, workspace_bytes, &group);
  if (ws != HYENA_OK) return ws;
  if (p.multi) {
    if (overlap(workspace, workspace_bytes, y, act) || overlap(workspace, workspace_bytes, v, act) ||
        overlap(workspace, workspace_bytes, spec, sb))
      return HYENA_ERR_ALIAS;
    for (int n = 0; n < N; ++n)
      if (overlap(workspace, workspace_bytes, x[n], act)) return HYENA_ERR_ALIAS;
  }
  NdArgs a{};
  a.work = workspace;
  a.rows_per_group = group;
  a.ndim = p.ndim; a.P = p.P; a.Lo = p.Lo; a.Lm = p.Lm; a.Ll = p.Ll;
  a.circular = circular;
  a.spec_stride = p.stride;
  a.spec = const_cast<void*>(spec);
  a.rows = (int)(B * D);
  a.v = v;
  for (int n = 0; n < N; ++n) a.x.p[n] = x[n];
  a.y = y;
  a.D = D;
  a.NORD = N;
  a.per_sample = per_sample;
  a.io = (io == HYENA_FP32) ? 0 : 1;
  const hipError_t e = !p.multi ? nd_forward(a, (hipStream_t)stream)
                                : (p.ndim == 2 ? grid2d_forward(a, (hipStream_t)stream)
                                               : grid3d_forward(a, (hipStream_t)stream));
  return e == hipSuccess ? HYENA_OK : HYENA_ERR_HIP;
}

}  // extern "C"
