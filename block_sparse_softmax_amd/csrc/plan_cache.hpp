// Host-side bookkeeping of the one-shot entry point: a bounded cache of
// compiled plans addressed by the descriptor's content, and the record of
// which plan image each caller workspace holds.
#pragma once

#include <cstddef>
#include <cstdint>
#include <list>
#include <memory>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "bss_attn.h"

struct attn_plan;

namespace bss {

// The content a plan is compiled from, in comparable form: the scalar fields
// that matter for the descriptor's kind (with L, H, D) and copies of the
// arrays it points to.
struct DescKey {
  std::vector<int64_t> scalars;
  std::vector<int64_t> head_left;   // WINDOW with per-head reaches
  std::vector<uint8_t> block_mask;  // BLOCK
};

// Scalars of the request, arrays copied.  Requires the array pointers the
// kind uses to be valid for their sizes.
DescKey make_desc_key(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D);

// Whether `key` describes exactly this request (arrays compared in place).
bool desc_matches(const DescKey& key, const attn_mask_desc* m, int64_t L, int64_t H, int64_t D);

// 64-bit hash of the request's content, read a machine word at a time.
uint64_t desc_hash(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D);

// Host bytes a compiled plan holds (its lists, schedules and descriptor copies).
size_t plan_host_bytes(const attn_plan& p);

// Bounded cache of compiled plans.  A lookup hashes the request, and a hit
// needs the stored content to equal the request (so two descriptors whose
// hashes collide get their own plans).  At most max_entries plans and about
// max_bytes of host memory are kept; the least recently used go first (the
// newest is always kept).  Plans are shared: a caller holding one keeps it
// alive after its eviction.  Thread-safe.
class PlanCache {
 public:
  using HashFn = uint64_t (*)(const attn_mask_desc*, int64_t, int64_t, int64_t);
  PlanCache(size_t max_entries, size_t max_bytes, HashFn hash = desc_hash);

  // The plan for this request: cached, or compiled (compile_plan) and cached.
  // The descriptor's array pointers must have been checked by the caller.
  attn_status get(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D,
                  std::shared_ptr<const attn_plan>* out);

  size_t size() const;
  size_t compiles() const;   // compile_plan calls made so far
  size_t bytes() const;      // host bytes of the cached plans

 private:
  struct Entry {
    uint64_t hash;
    DescKey key;
    std::shared_ptr<const attn_plan> plan;
    size_t bytes;
  };
  mutable std::mutex mu_;
  std::list<Entry> lru_;     // front: most recently used
  size_t max_entries_, max_bytes_, bytes_ = 0, compiles_ = 0;
  HashFn hash_;
};

// Which plan image each caller workspace holds, recorded by every call that
// uploads one (attn_plan_upload, attn_bwd_upload, the one-shot forward) and
// dropped by attn_workspace_release.  kv_heads = 0: the forward image only;
// > 0: forward and backward images for that many K/V heads.
struct UploadTag {
  uint64_t plan_serial = 0;
  int64_t kv_heads = 0;
};

class UploadTags {
 public:
  void note(const void* ws, uint64_t plan_serial, int64_t kv_heads);
  // The forward image of plan `plan_serial` is in `ws`.
  bool holds_forward(const void* ws, uint64_t plan_serial) const;
  // The forward and backward images (for kv_heads K/V heads) are in `ws`.
  bool holds_backward(const void* ws, uint64_t plan_serial, int64_t kv_heads) const;
  void forget(const void* ws);
  size_t size() const;

 private:
  mutable std::mutex mu_;
  std::unordered_map<const void*, UploadTag> tags_;
};

}  // namespace bss
