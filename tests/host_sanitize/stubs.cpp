// Stand-ins for the kernel launchers, for the host-only sanitizer build of
// the library's host code: every launch reports hipErrorNotSupported, so any
// call that reaches a kernel returns SPIN_EHIP.  The calls the sanitizer
// driver makes never need a GPU.
#include "spin_internal.h"

namespace spin {

namespace {
constexpr hipError_t kNoKernel = hipErrorNotSupported;
}

hipError_t launch_init(const Dev&, hipStream_t) { return kNoKernel; }
hipError_t launch_release(const Dev&, int, hipStream_t) { return kNoKernel; }
hipError_t launch_set_budget(const Dev&, int, int, hipStream_t) { return kNoKernel; }
hipError_t launch_index(const Dev&, int, int, const void*, int, hipStream_t) { return kNoKernel; }
hipError_t launch_append(const Dev&, const uint16_t*, const uint16_t*, hipStream_t) { return kNoKernel; }
hipError_t launch_score(const Dev&, const uint16_t*, float*, hipStream_t) { return kNoKernel; }
hipError_t launch_topk(const Dev&, const float*, int*, hipStream_t) { return kNoKernel; }
hipError_t launch_select_split(const Dev&, const uint16_t*, float*, int*, hipStream_t) { return kNoKernel; }
hipError_t launch_select_fused(const Dev&, const uint16_t*, float*, int*, hipStream_t) { return kNoKernel; }
hipError_t launch_resolve(const Dev&, const int*, int, int*, int*, int*, hipStream_t) { return kNoKernel; }
hipError_t launch_segments(const Dev&, hipStream_t) { return kNoKernel; }
hipError_t launch_step_advance(int*, hipStream_t) { return kNoKernel; }
hipError_t launch_retrieve(const Dev&, hipStream_t) { return kNoKernel; }
hipError_t launch_retrieve_attend(const Dev&, const uint16_t*, hipStream_t) { return kNoKernel; }
hipError_t launch_transfer_attend(const Dev&, const uint16_t*, const int*, const int*, const int*, bool,
                                  hipStream_t) {
  return kNoKernel;
}
hipError_t launch_read_stream(const void*, size_t, unsigned*, hipStream_t) { return kNoKernel; }
hipError_t launch_attend(const Dev&, const uint16_t*, const int*, const int*, const int*, float*, int,
                         hipStream_t, int*) {
  return kNoKernel;
}

}  // namespace spin
