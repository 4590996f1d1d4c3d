// hostcheck_stubs.cpp -- stand-ins for the kernel launchers, linked with
// api.cpp into a host-only build of the C ABI (g++, AddressSanitizer and
// UndefinedBehaviorSanitizer; no GPU code).  That build exercises argument
// validation, planning and the size queries on the CPU.  A call with bad
// arguments must return its status before it reaches a launcher; a call
// that gets this far receives hipErrorNoDevice, which the entry points
// report as HYENA_ERR_HIP, the status a GPU-less host would see anyway.
#include "launch.hpp"

namespace hyena {

namespace {
constexpr hipError_t kNoKernels = hipErrorNoDevice;
}

hipError_t in_projection(const InProjArgs&, hipStream_t) { return kNoKernels; }
hipError_t out_projection(const OutProjArgs&, hipStream_t) { return kNoKernels; }
hipError_t single_backward(const BackwardArgs&, int64_t, hipStream_t) { return kNoKernels; }
hipError_t long_backward(const BackwardArgs&, const PlanInfo&, void*, hipStream_t) { return kNoKernels; }
hipError_t filter_gen_li(const float*, const float*, int, int, int64_t, float*, hipStream_t) { return kNoKernels; }
hipError_t filter_gen_mr(const float*, const float*, int, int, int, float*, hipStream_t) { return kNoKernels; }
hipError_t fir_forward(const ForwardArgs&, const float*, int, hipStream_t) { return kNoKernels; }
hipError_t nd_spectrum(const NdArgs&, hipStream_t) { return kNoKernels; }
hipError_t nd_forward(const NdArgs&, hipStream_t) { return kNoKernels; }
hipError_t grid2d_spectrum(const NdArgs&, hipStream_t) { return kNoKernels; }
hipError_t grid2d_forward(const NdArgs&, hipStream_t) { return kNoKernels; }
hipError_t grid3d_spectrum(const NdArgs&, hipStream_t) { return kNoKernels; }
hipError_t grid3d_forward(const NdArgs&, hipStream_t) { return kNoKernels; }
hipError_t grid_plane_pass(const NdArgs&, int, int, int, bool, hipStream_t) { return kNoKernels; }
hipError_t single_forward(const ForwardArgs&, int64_t, hipStream_t) { return kNoKernels; }
hipError_t single_spectrum(const SpectrumArgs&, int64_t, hipStream_t) { return kNoKernels; }
hipError_t fourstep_forward(const ForwardArgs&, const PlanInfo&, hipStream_t) { return kNoKernels; }
hipError_t fourstep_spectrum(const SpectrumArgs&, const PlanInfo&, hipStream_t) { return kNoKernels; }
hipError_t filter_gen(const FilterGenArgs&, hipStream_t) { return kNoKernels; }
hipError_t spectrum_export(const void*, int, const PlanInfo&, float*, hipStream_t) { return kNoKernels; }
hipError_t static_scratch(void**, int64_t*) { return kNoKernels; }
hipError_t spectrum_to_fourstep(const void*, int, const PlanInfo&, const PlanInfo&, void*, hipStream_t) {
  return kNoKernels;
}

}  // namespace hyena
