// Mask-descriptor compiler and tile scheduler (host side).
//
// A plan turns a mask descriptor (full / chunk / sliding window / per-head
// causal window / block-selection matrix) into, for every (head, query tile),
// the ascending list of key tiles that contain at least one allowed pair, each
// flagged FULL or PARTIAL.  Masked-out tiles never appear, so the kernel never
// loads or multiplies them.  The tile partition is the block partition of
// "RRAttention", section 2.1 (contiguous blocks, ceil(L/B) of them), applied
// with query tiles of BM rows and key tiles of BN columns.
#pragma once

#include <cstddef>
#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "bss_attn.h"

namespace bss {

constexpr int kBM = 128;  // query rows per work item (4 waves x 32 rows)
constexpr int kBN = 64;   // keys per KV tile
constexpr int kXcds = 8;  // MI355X: 8 accelerator dies, each with its own L2
constexpr int kSlots = 512;  // resident work-groups: 256 CUs x 2

// Device record of one work item (32 bytes).  A (head, query tile) row whose
// list is long compared with the whole launch is cut into `npieces`
// contiguous pieces of its list; each piece leaves its partial softmax state
// in partial slot `slot + piece`, and a second kernel merges the pieces of
// split row `split` (entry `split` of the image's merge list) in piece order.
// Unsplit items have npieces = 1.  Items with head = -1 pad the per-XCD
// queues to equal length and do nothing.
struct Item {
  int32_t head, qtile, begin, end;
  int32_t slot, piece, npieces, split;
};

// Merge-list record of one split row (16 bytes): its head, query tile, first
// partial slot and piece count.
struct MergeRow {
  int32_t head, qtile, slot, npieces;
};

// Layout of the plan's device image inside the caller's workspace, followed
// by the partial-state slots of split items (not part of the image).
struct ImageLayout {
  size_t off_items = 0, off_items_unsplit = 0, off_kv = 0, off_head_left = 0, off_bits = 0,
         off_merge = 0, bytes = 0;
  size_t off_partials = 0, total = 0;
};

// Backward image for one K/V head count (grouped-query attention changes
// which query heads a dK/dV work item visits).  Key blocks are 2 key tiles
// (128 keys, one work-group).  `col` lists, for every (kv head, key block),
// the query tiles of each of the group's query heads whose forward list holds
// one of the block's key tiles, as (group head << 24) | (query tile << 1) |
// full, group heads in order and query tiles ascending; full = every pair of
// the 128 x 128 rectangle is allowed.  `items` are the dK/dV work items
// {kv head, key block, first col entry, one past the last, 0, 0, 1, 0} in
// kXcds equal-length queues (kv head -1 pads).
// `items_split` is the batch-1 schedule: an item whose list is long compared
// with the launch is cut into pieces of consecutive entries, each adding its
// dK and dV sums into partial slot `slot + piece` (n_slots slots of
// dkdv_slot_floats floats after the statistics of a batch-1 workspace), and
// `merge` lists the split items for the merge kernel (MergeRow with the kv
// head in `head` and the key block in `qtile`).
struct BwdImage {
  int64_t kv_heads = 0, nkb = 0;
  std::vector<Item> items, items_split;
  std::vector<MergeRow> merge;
  int64_t n_slots = 0;
  std::vector<int32_t> col_ptr;  // [kv_heads * nkb + 1] (host only): (kv head, key block) row-major
  std::vector<int32_t> col;
  size_t off_items = 0, off_items_split = 0, off_merge = 0, off_col = 0, bytes = 0;  // relative to the image start
};

// Workspace of a backward launch with batch B: the forward workspace
// (image and partial states), the backward image, per-row statistics
// (lse in log2 units and D, float [B][H][2][nq * kBM]), the per query tile
// partial sums of the sink gradient (float [B][H][nq]), the scaled queries
// the scores are recomputed from (bf16 [B][H][L][D]) and, for B = 1, the
// dK/dV partial slots of split key blocks.
struct BwdLayout {
  size_t off_image = 0, off_stat = 0, off_sinkpart = 0, off_qs = 0, off_dkdv = 0, total = 0;
};

void set_error(const std::string& msg);

}  // namespace bss

struct attn_plan {
  // descriptor (copied)
  int32_t kind = 0, causal = 0;
  int64_t chunk = 0, left = 0, right = 0, block = 0;
  int64_t prefix = 0;                 // keys 0 .. prefix-1 added to every row (before the causal cut)
  int32_t block_heads = 0;
  std::vector<int64_t> head_left;     // [H] for WINDOW (left broadcast when no per-head array)
  std::vector<uint8_t> block_mask;    // [Hb][Nb][Nb] for BLOCK
  int64_t nb = 0;                     // ceil(L / block)
  bool block_aligned = true;          // block % BM == 0 and block % BN == 0

  int64_t L = 0, H = 0, D = 0;
  int32_t bm = bss::kBM, bn = bss::kBN;
  int64_t nq = 0, nk = 0;

  // canonical lists
  std::vector<int32_t> row_ptr, kv_tile;
  std::vector<uint8_t> flags;
  std::vector<int64_t> pairs;         // allowed pairs per head
  int64_t pairs_total = 0;

  // schedule and device image: `items` (batch 1, long rows split) and
  // `items_unsplit` (batch > 1: every row one item), each laid out as
  // kXcds equal-length queues
  std::vector<bss::Item> items, items_unsplit;
  int64_t n_partial_slots = 0;
  // forward kernel of head dim 128: the two-group ping-pong kernel when the
  // rows are long on average, else the single-group kernel (two work-groups
  // per CU, for short rows)
  bool pingpong = false;
  std::vector<bss::MergeRow> merge_rows;  // split rows of `items`, merged after the launch
  std::vector<int32_t> kv_entries;    // (kv_tile << 1) | full, in canonical order
  std::vector<int32_t> head_left32;   // [H]
  std::vector<uint32_t> block_bits;   // [Hb][Nb][ceil(Nb/32)] when not block_aligned
  bss::ImageLayout layout;

  // process-wide serial number: names this compilation in the record of
  // which plan image a workspace holds
  uint64_t serial = 0;

  // backward images by K/V head count (built on first use)
  mutable std::mutex bwd_mu;
  mutable std::map<int64_t, std::unique_ptr<bss::BwdImage>> bwd_images;
};

namespace bss {

// Validate and compile.  Returns ATTN_OK and a new plan, or an error status
// with the message set.
attn_status compile_plan(const attn_mask_desc* mask, int64_t L, int64_t H, int64_t D,
                         attn_plan** out);

// Serialise the device image into `dst` (layout.bytes long).
void write_image(const attn_plan& p, uint8_t* dst);

// The backward image of plan p for kv_heads K/V heads (built once, cached in
// the plan; thread-safe).  kv_heads must divide p.H.  Throws std::bad_alloc.
const BwdImage& bwd_image(const attn_plan& p, int64_t kv_heads);

// Byte layout of a backward workspace for batch B.
BwdLayout bwd_layout(const attn_plan& p, const BwdImage& img, int64_t B);

// Serialise the backward image into `dst` (img.bytes long).
void write_bwd_image(const BwdImage& img, uint8_t* dst);

}  // namespace bss
