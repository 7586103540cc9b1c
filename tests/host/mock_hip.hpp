// Call records of the HIP stand-in (tests/host/mock_hip.cpp).
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "kernels.hpp"

namespace mock {
struct Counters {
  size_t memcpy_calls = 0, memcpy_bytes = 0, syncs = 0, fwd_launches = 0, bwd_launches = 0;
};
extern Counters counters;
constexpr uintptr_t kScratchAddr = 0xC0000000;  // where the stand-in places the library's scratch
extern std::vector<bss::FwdParams> fwd_launches;
}  // namespace mock
