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
};

struct SpectrumArgs {
  const float* h;        // [NF][L]
  void* spec;
  int NF;                // N*D
  int64_t L;
  int64_t spec_stride;
  void* work;
  int rows_per_group;
};

struct FilterGenArgs {
  int D, N, K, H;
  const float *W1, *b1, *W2, *b2, *W3, *b3, *alpha;
  int64_t L;
  float* h;
};

hipError_t single_forward(const ForwardArgs& a, int64_t N, hipStream_t s);
hipError_t single_spectrum(const SpectrumArgs& a, int64_t N, hipStream_t s);
hipError_t fourstep_forward(const ForwardArgs& a, const PlanInfo& p, hipStream_t s);
hipError_t fourstep_spectrum(const SpectrumArgs& a, const PlanInfo& p, hipStream_t s);
hipError_t filter_gen(const FilterGenArgs& a, hipStream_t s);
hipError_t spectrum_export(const void* spec, int NF, const PlanInfo& p, float* out, hipStream_t s);

}  // namespace hyena
