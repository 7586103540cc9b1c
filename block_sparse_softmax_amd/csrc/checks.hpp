// Range checks of the checked build (BSS_CHECKED): the fields of a work item
// and of a split-row record, and the key tiles an item lists, against the
// launch's sizes.  Plain functions of integers, compiled for the host too (the
// CPU tests call them) and used by the forward kernels of the checked build
// before they touch memory through any of these values.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define BSS_HD __host__ __device__
#else
#define BSS_HD
#endif

namespace bss {

// Violation bits (ORed into the launch's check word).
enum CheckBit : uint32_t {
  kCheckHead = 1u << 0,      // item head outside [0, H)
  kCheckQTile = 1u << 1,     // query tile outside [0, ceil(L / 128))
  kCheckRange = 1u << 2,     // list range not inside [0, n_entries) or begin > end
  kCheckPiece = 1u << 3,     // piece / pieces / partial slot out of range
  kCheckEntry = 1u << 4,     // a listed key tile outside [0, ceil(L / 64))
  kCheckMergeRow = 1u << 5,  // a split-row record out of range
  kCheckPointer = 1u << 6,   // a pointer the item needs is NULL
};

struct ItemFields {
  int32_t head, qtile, begin, end, slot0, piece, npieces;
};

// Violations of one work item (head >= 0; head < 0 marks queue padding).
BSS_HD inline uint32_t item_violations(const ItemFields& it, int32_t H, int32_t L, int32_t n_entries,
                                       int32_t n_slots) {
  const int32_t nq = (L + 127) / 128;
  uint32_t bits = 0;
  if (it.head < 0 || it.head >= H) bits |= kCheckHead;
  if (it.qtile < 0 || it.qtile >= nq) bits |= kCheckQTile;
  if (it.begin < 0 || it.begin > it.end || it.end > n_entries) bits |= kCheckRange;
  if (it.npieces < 1 || it.piece < 0 || it.piece >= it.npieces) {
    bits |= kCheckPiece;
  } else if (it.npieces > 1 && (it.slot0 < 0 || it.slot0 > n_slots - it.npieces)) {
    bits |= kCheckPiece;
  }
  return bits;
}

// A list entry ((key tile << 1) | full) inside the sequence.
BSS_HD inline bool entry_in_range(int32_t ent, int32_t L) {
  const int32_t nk = (L + 63) / 64;
  return ent >= 0 && (ent >> 1) < nk;
}

// Violations of one split-row record {head, qtile, first slot, pieces}.
BSS_HD inline uint32_t merge_row_violations(int32_t head, int32_t qtile, int32_t slot0, int32_t npieces,
                                            int32_t H, int32_t L, int32_t n_slots) {
  const int32_t nq = (L + 127) / 128;
  const bool bad = head < 0 || head >= H || qtile < 0 || qtile >= nq || npieces < 2 || slot0 < 0 ||
                   slot0 > n_slots - npieces;
  return bad ? kCheckMergeRow : 0u;
}

}  // namespace bss
