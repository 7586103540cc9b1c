// Call records of the HIP stand-in (tests/host/mock_hip.cpp).
#pragma once

#include <cstddef>
#include <vector>

#include "kernels.hpp"

namespace mock {
struct Counters {
  size_t memcpy_calls = 0, memcpy_bytes = 0, syncs = 0, fwd_launches = 0, bwd_launches = 0;
};
extern Counters counters;
extern std::vector<bss::FwdParams> fwd_launches;
}  // namespace mock
