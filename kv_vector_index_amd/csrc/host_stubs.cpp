// Host-only stand-ins for the kernel launchers of the wave-index library, for a build of
// the C ABI's argument validation and workspace layout (api.cpp) with the host compiler and
// its sanitizers. Every launcher reports that nothing can run, so a call that passes
// validation returns WAVE_ERR_HIP; no device code is built or called.
#include "wave_kernels.h"

namespace wave {

hipError_t launch_decode(const DecodeArgs&, hipStream_t, Tracer*) { return hipErrorNotSupported; }
hipError_t launch_dense_decode(const DecodeArgs&, hipStream_t, Tracer*) {
  return hipErrorNotSupported;
}
hipError_t launch_copy_blocks(const CopyArgs&, hipStream_t, Tracer*) {
  return hipErrorNotSupported;
}
hipError_t launch_build(const BuildArgs&, hipStream_t, Tracer*) { return hipErrorNotSupported; }
hipError_t launch_tier_reset(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_listed_attention(const DecodeArgs&, hipStream_t, Tracer*) {
  return hipErrorNotSupported;
}
hipError_t launch_anns_build(const AnnsArgs&, hipStream_t, Tracer*) { return hipErrorNotSupported; }
hipError_t launch_anns_search(const AnnsArgs&, hipStream_t, Tracer*) {
  return hipErrorNotSupported;
}
hipError_t tier_counters_copy(uint32_t*, const void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNotSupported;
}

}  // namespace wave
