// Pieces shared by the forward kernels: attn_fwd.hip (d = 64, 80 and the
// split-row merge), attn_fwd_pp.hip (d = 128, long rows) and attn_fwd_sg.hip
// (d = 128 short rows, d = 256).
#pragma once

#include <hip/hip_runtime.h>

#include "checks.hpp"
#include "kernels.hpp"
#include "tile_common.hpp"

namespace bss {
namespace dev {

// The running reference moves only when a score exceeds it by more than 2^8.
constexpr float kRescaleThreshold = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS tiles.  d = 64 and 80: row-major rows of LRB bytes, 16-byte chunks
// XOR-swizzled by row (the swizzle of tile_common.hpp).  d >= 128: rows
// padded so that every fragment address is one per-lane base plus a constant.
// A 64-key tile is NI = d / 8 DMA wave-instructions of 1 KiB; instruction i
// carries rows i, i + NI, i + 2 NI, ... (1024 / (2 d) rows: 4 at d = 128, 2 at
// d = 256) into 1024 consecutive bytes (row i + k NI at + 2 d k, unswizzled),
// and consecutive instructions sit kKBlk (K) or kVBlk (V) bytes apart.  A K
// fragment read (16 lanes, 16 consecutive rows, one chunk) then sees row
// offsets 16 bytes apart modulo the 256-byte bank width, and a transposed V
// read (32 lanes, 4 consecutive rows x 64 bytes) sees rows 64 bytes apart:
// both conflict-free.
template <int D>
struct Lds {
  static constexpr bool PADDED = (D >= 128);
  static constexpr int NI = 2 * kBN * D / 1024;              // DMA instructions per tile (padded layout)
  static constexpr int kKBlk = 1024 + 16;
  static constexpr int kVBlk = 1024 + 64;
  static constexpr int KT = PADDED ? NI * kKBlk : Shape<D>::TILE;  // bytes of a K tile
  static constexpr int VT = PADDED ? NI * kVBlk : Shape<D>::TILE;  // bytes of a V tile
  static constexpr int BYTES = 2 * KT + 2 * VT;
  // buffers 0-1 hold K tiles, 2-3 V tiles
  __device__ static constexpr int buf_off(int buf) { return buf < 2 ? buf * KT : 2 * KT + (buf - 2) * VT; }
};

#ifdef BSS_CHECKED
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif

// Checked build, at the top of a forward kernel (every wave of the work-group
// runs it, before any barrier): false, with the violations recorded in the
// launch's check word, when the item's fields, the pointers it needs or the
// key tiles it lists are out of range; the work-group then returns without
// touching memory through them.
__device__ inline bool item_checked(const FwdParams& p, int4 item, int4 split) {
  const ItemFields f{item.x, item.y, item.z, item.w, split.x, split.y, split.z};
  uint32_t bits = item_violations(f, p.H, p.L, p.n_entries, p.n_slots);
  if (f.npieces > 1 && p.partials == nullptr) bits |= kCheckPointer;
  if (p.kind == kMaskWindow && p.head_left == nullptr) bits |= kCheckPointer;
  if (p.q == nullptr || p.k == nullptr || p.v == nullptr || p.o == nullptr || p.kv == nullptr) bits |= kCheckPointer;
  if (bits == 0) {
    for (int e = f.begin; e < f.end; ++e) {
      if (!entry_in_range(p.kv[e], p.L)) {
        bits |= kCheckEntry;
        break;
      }
    }
  }
  if (bits == 0) return true;
  if (threadIdx.x == 0 && p.check != nullptr) atomicOr(p.check, bits);
  return false;
}

}  // namespace dev

// Main kernels of the d = 128 and d = 256 forward over `grid` (one work item
// per work-group, as laid out by the plan); launch_fwd queues the split-row
// merge after them.  launch_fwd_sg takes D = 128 or 256.
hipError_t launch_fwd_pp(const GroupParams& g, dim3 grid, bool prefix, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop);
hipError_t launch_fwd_sg(const GroupParams& g, int D, dim3 grid, bool prefix, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop);

}  // namespace bss
