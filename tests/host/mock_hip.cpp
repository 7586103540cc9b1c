// A stand-in for the HIP runtime and the kernel launchers, for host-only tests
// of the library's C ABI layer: it records the calls the layer makes and never
// touches memory behind the device pointers it is given.

#include <hip/hip_runtime_api.h>

#include <vector>

#include "kernels.hpp"
#include "mock_hip.hpp"

namespace mock {
Counters counters;
std::vector<bss::FwdParams> fwd_launches;
}  // namespace mock

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t) {
  if (!dst || !src || kind != hipMemcpyHostToDevice) return hipErrorInvalidValue;
  ++mock::counters.memcpy_calls;
  mock::counters.memcpy_bytes += bytes;
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) {
  ++mock::counters.syncs;
  return hipSuccess;
}

const char* hipGetErrorString(hipError_t) { return "mock HIP error"; }

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

namespace bss {

hipError_t launch_fwd(const GroupParams& g, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  ++mock::counters.fwd_launches;
  for (int j = 0; j < g.n_jobs; ++j) mock::fwd_launches.push_back(g.job[j]);
  return hipSuccess;
}
hipError_t launch_bwd(const BwdParams&, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  ++mock::counters.bwd_launches;
  return hipSuccess;
}
hipError_t launch_rr_search(const RrParams&, hipStream_t, hipEvent_t, hipEvent_t) { return hipSuccess; }
hipError_t launch_reorder(const ReorderParams&, hipStream_t, hipEvent_t, hipEvent_t) { return hipSuccess; }
hipError_t launch_decode(const DecodeParams&, int, hipStream_t, hipEvent_t, hipEvent_t) { return hipSuccess; }

// the library's static scratch, at a fixed fake device address
bool checked_build() { return false; }

hipError_t check_bits(uint32_t* bits, bool) {
  *bits = 0;
  return hipSuccess;
}

hipError_t fwd_scratch(void** ptr, size_t* bytes) {
  *ptr = reinterpret_cast<void*>(mock::kScratchAddr);
  *bytes = kFwdScratchBytes;
  return hipSuccess;
}

}  // namespace bss
