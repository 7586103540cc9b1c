// Kernel-side parameter block and launcher declaration (shared by the C ABI
// layer and the HIP translation unit).
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace bss {

// Floats of one partial-state slot of a split item at head dim D: for each of
// the 4 waves, the DT = ceil(D/32) accumulator tiles of O^T (16 floats per
// lane each, stored as 4 float4 per lane, lane-minor) and then the row
// reference m and the denominator l of every lane.
constexpr int64_t partial_slot_floats(int64_t D) { return 4 * (((D + 31) / 32) * 16 * 64 + 2 * 64); }

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t q_sb, q_sl, q_sh;   // element strides
  int64_t k_sb, k_sl, k_sh;
  int64_t v_sb, v_sl, v_sh;
  int64_t o_sb, o_sl, o_sh;
  const int32_t* items;       // n_items x {head, qtile, begin, end, slot, piece, npieces, counter}
  const int32_t* kv;          // (kv_tile << 1) | full
  const int32_t* head_left;   // [H] window left reach (WINDOW)
  const uint32_t* block_bits; // unaligned BLOCK masks (unused when aligned)
  const float* sink;          // [H] or nullptr
  float* partials;            // partial-state slots of split items
  int32_t* counters;          // per split row: pieces finished in this launch (returns to 0)
  float scale_log2;           // softmax scale * log2(e)
  int32_t L, H, n_items;
  int32_t kind, causal;
  int32_t chunk, right;
  int32_t xcd_chunked;        // 1: XCD x runs the x-th of 8 equal-length queues of the schedule
};

// Launch the forward kernel for head dim D on `stream` with grid (n_items, B).
hipError_t launch_fwd(const FwdParams& p, int D, int B, hipStream_t stream);

}  // namespace bss
