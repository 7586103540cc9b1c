// Plan cache and workspace upload records of the one-shot entry point.
// Host C++17, no HIP calls.

#include "plan_cache.hpp"

#include <cstring>

#include "plan.hpp"

namespace bss {

namespace {

int64_t blocks_per_side(const attn_mask_desc* m, int64_t L) { return (L + m->block - 1) / m->block; }

std::vector<int64_t> scalars_of(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D) {
  std::vector<int64_t> s = {L, H, D, m->kind, m->causal, m->prefix};
  switch (m->kind) {
    case ATTN_MASK_CHUNK: s.push_back(m->chunk); break;
    case ATTN_MASK_WINDOW:
      s.push_back(m->left);
      s.push_back(m->right);
      s.push_back(m->head_left != nullptr);
      break;
    case ATTN_MASK_BLOCK:
      s.push_back(m->block);
      s.push_back(m->block_mask_heads);
      break;
    default: break;
  }
  return s;
}

size_t head_left_count(const attn_mask_desc* m, int64_t H) {
  return (m->kind == ATTN_MASK_WINDOW && m->head_left != nullptr) ? static_cast<size_t>(H) : 0;
}

size_t block_mask_bytes(const attn_mask_desc* m, int64_t L) {
  if (m->kind != ATTN_MASK_BLOCK || m->block_mask == nullptr || m->block < 1) return 0;
  const int64_t nb = blocks_per_side(m, L);
  return static_cast<size_t>(m->block_mask_heads) * static_cast<size_t>(nb) * static_cast<size_t>(nb);
}

// One mixing step per 64-bit word (multiply, then fold the high bits down).
struct WordHash {
  uint64_t h = 0x243F6A8885A308D3ull;
  void word(uint64_t w) {
    h = (h ^ w) * 0x9E3779B97F4A7C15ull;
    h ^= h >> 29;
  }
  void bytes(const void* p, size_t n) {
    const uint8_t* b = static_cast<const uint8_t*>(p);
    size_t i = 0;
    for (; i + 8 <= n; i += 8) {
      uint64_t w;
      std::memcpy(&w, b + i, 8);
      word(w);
    }
    uint64_t tail = 0;
    std::memcpy(&tail, b + i, n - i);
    word(tail ^ (static_cast<uint64_t>(n - i) << 56));
  }
};

}  // namespace

DescKey make_desc_key(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D) {
  DescKey k;
  k.scalars = scalars_of(m, L, H, D);
  const size_t nh = head_left_count(m, H);
  if (nh) k.head_left.assign(m->head_left, m->head_left + nh);
  const size_t nbm = block_mask_bytes(m, L);
  if (nbm) k.block_mask.assign(m->block_mask, m->block_mask + nbm);
  return k;
}

bool desc_matches(const DescKey& key, const attn_mask_desc* m, int64_t L, int64_t H, int64_t D) {
  if (key.scalars != scalars_of(m, L, H, D)) return false;
  const size_t nh = head_left_count(m, H);
  if (key.head_left.size() != nh ||
      (nh && std::memcmp(key.head_left.data(), m->head_left, nh * sizeof(int64_t)) != 0))
    return false;
  const size_t nbm = block_mask_bytes(m, L);
  return key.block_mask.size() == nbm && (nbm == 0 || std::memcmp(key.block_mask.data(), m->block_mask, nbm) == 0);
}

uint64_t desc_hash(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D) {
  WordHash hs;
  for (int64_t s : scalars_of(m, L, H, D)) hs.word(static_cast<uint64_t>(s));
  const size_t nh = head_left_count(m, H);
  if (nh) hs.bytes(m->head_left, nh * sizeof(int64_t));
  const size_t nbm = block_mask_bytes(m, L);
  if (nbm) hs.bytes(m->block_mask, nbm);
  return hs.h;
}

size_t plan_host_bytes(const attn_plan& p) {
  return p.row_ptr.size() * 4 + p.kv_tile.size() * 4 + p.flags.size() + p.pairs.size() * 8 +
         (p.items.size() + p.items_unsplit.size()) * sizeof(Item) + p.merge_rows.size() * sizeof(MergeRow) +
         p.kv_entries.size() * 4 + p.head_left.size() * 8 + p.head_left32.size() * 4 + p.block_mask.size() +
         p.block_bits.size() * 4 + sizeof(attn_plan);
}

PlanCache::PlanCache(size_t max_entries, size_t max_bytes, HashFn hash)
    : max_entries_(max_entries < 1 ? 1 : max_entries), max_bytes_(max_bytes), hash_(hash) {}

attn_status PlanCache::get(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D,
                           std::shared_ptr<const attn_plan>* out) {
  const uint64_t h = hash_(m, L, H, D);
  {
    std::lock_guard<std::mutex> g(mu_);
    for (auto it = lru_.begin(); it != lru_.end(); ++it) {
      if (it->hash == h && desc_matches(it->key, m, L, H, D)) {
        lru_.splice(lru_.begin(), lru_, it);
        *out = lru_.front().plan;
        return ATTN_OK;
      }
    }
  }
  // compile outside the lock (another thread may compile the same content; both results are equal)
  attn_plan* raw = nullptr;
  attn_status st = compile_plan(m, L, H, D, &raw);
  if (st != ATTN_OK) return st;
  std::shared_ptr<const attn_plan> plan(raw);
  Entry e{h, make_desc_key(m, L, H, D), plan, 0};
  e.bytes = plan_host_bytes(*plan) + e.key.block_mask.size() + e.key.head_left.size() * 8;
  std::lock_guard<std::mutex> g(mu_);
  ++compiles_;
  bytes_ += e.bytes;
  lru_.push_front(std::move(e));
  while (lru_.size() > 1 && (lru_.size() > max_entries_ || bytes_ > max_bytes_)) {
    bytes_ -= lru_.back().bytes;
    lru_.pop_back();
  }
  *out = plan;
  return ATTN_OK;
}

size_t PlanCache::size() const {
  std::lock_guard<std::mutex> g(mu_);
  return lru_.size();
}

size_t PlanCache::compiles() const {
  std::lock_guard<std::mutex> g(mu_);
  return compiles_;
}

size_t PlanCache::bytes() const {
  std::lock_guard<std::mutex> g(mu_);
  return bytes_;
}

void UploadTags::note(const void* ws, uint64_t plan_serial, int64_t kv_heads) {
  std::lock_guard<std::mutex> g(mu_);
  tags_[ws] = UploadTag{plan_serial, kv_heads};
}

bool UploadTags::holds_forward(const void* ws, uint64_t plan_serial) const {
  std::lock_guard<std::mutex> g(mu_);
  auto it = tags_.find(ws);
  return it != tags_.end() && it->second.plan_serial == plan_serial;
}

bool UploadTags::holds_backward(const void* ws, uint64_t plan_serial, int64_t kv_heads) const {
  std::lock_guard<std::mutex> g(mu_);
  auto it = tags_.find(ws);
  return it != tags_.end() && it->second.plan_serial == plan_serial && it->second.kv_heads == kv_heads;
}

void UploadTags::forget(const void* ws) {
  std::lock_guard<std::mutex> g(mu_);
  tags_.erase(ws);
}

size_t UploadTags::size() const {
  std::lock_guard<std::mutex> g(mu_);
  return tags_.size();
}

}  // namespace bss
