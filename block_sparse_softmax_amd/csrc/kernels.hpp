// Kernel-side parameter block and launcher declaration (shared by the C ABI
// layer and the HIP translation unit).
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace bss {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t q_sb, q_sl, q_sh;   // element strides
  int64_t k_sb, k_sl, k_sh;
  int64_t v_sb, v_sl, v_sh;
  int64_t o_sb, o_sl, o_sh;
  const int32_t* items;       // n_items x {head, qtile, begin, end}
  const int32_t* kv;          // (kv_tile << 1) | full
  const int32_t* head_left;   // [H] window left reach (WINDOW)
  const uint32_t* block_bits; // unaligned BLOCK masks (unused when aligned)
  const float* sink;          // [H] or nullptr
  float scale_log2;           // softmax scale * log2(e)
  int32_t L, H, n_items;
  int32_t kind, causal;
  int32_t chunk, right;
  int32_t xcd_chunked;        // 1: XCD x runs the x-th contiguous eighth of the schedule
};

// Launch the forward kernel for head dim D on `stream` with grid (n_items, B).
hipError_t launch_fwd(const FwdParams& p, int D, int B, hipStream_t stream);

}  // namespace bss
