// Host-only checks of the plan compiler, the plan cache and the one-shot
// entry point's upload bookkeeping, linked against the HIP stand-in
// (mock_hip.cpp) and meant to run under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Prints "ALL OK" and exits 0 when every check
// holds; otherwise prints the failed check and exits 1.

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <string>
#include <vector>

#include "bss_attn.h"
#include "checks.hpp"
#include "mock_hip.hpp"
#include "plan.hpp"
#include "plan_cache.hpp"

namespace {

int g_failures = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);          \
      ++g_failures;                                                          \
    }                                                                        \
  } while (0)

uint64_t same_hash(const attn_mask_desc*, int64_t, int64_t, int64_t) { return 42; }

attn_mask_desc chunk_desc(int64_t c) {
  attn_mask_desc m{};
  m.kind = ATTN_MASK_CHUNK;
  m.chunk = c;
  return m;
}

// Every index of a compiled plan's device image lies in range: the work
// items' heads, query tiles, list ranges, partial slots and split rows, the
// key tiles of the lists, and the merge records.
void check_image(const attn_plan& p) {
  const int64_t nnz = static_cast<int64_t>(p.kv_entries.size());
  CHECK(static_cast<int64_t>(p.kv_tile.size()) == nnz);
  CHECK(static_cast<int64_t>(p.row_ptr.size()) == p.H * p.nq + 1);
  for (int32_t e : p.kv_entries) CHECK((e >> 1) >= 0 && (e >> 1) < p.nk);
  for (int32_t t : p.kv_tile) CHECK(t >= 0 && t < p.nk);
  for (const auto* items : {&p.items, &p.items_unsplit}) {
    CHECK(items->size() % bss::kXcds == 0);
    for (const bss::Item& it : *items) {
      if (it.head < 0) continue;  // queue padding
      CHECK(it.head < p.H && it.qtile >= 0 && it.qtile < p.nq);
      CHECK(it.begin >= 0 && it.begin <= it.end && it.end <= nnz);
      const int32_t r = static_cast<int32_t>(it.head * p.nq + it.qtile);
      CHECK(it.begin >= p.row_ptr[r] && it.end <= p.row_ptr[r + 1]);
      CHECK(it.npieces >= 1 && it.piece >= 0 && it.piece < it.npieces);
      if (it.npieces > 1) {
        CHECK(it.slot >= 0 && it.slot + it.npieces <= p.n_partial_slots);
        CHECK(it.split >= 0 && it.split < static_cast<int32_t>(p.merge_rows.size()));
      }
    }
  }
  for (const bss::MergeRow& m : p.merge_rows) {
    CHECK(m.head >= 0 && m.head < p.H && m.qtile >= 0 && m.qtile < p.nq);
    CHECK(m.npieces >= 2 && m.slot >= 0 && m.slot + m.npieces <= p.n_partial_slots);
  }
  CHECK(p.layout.bytes <= p.layout.total);
  // the checked build's kernel-side range checks pass on every compiled image
  // (split schedule with the plan's partial slots, unsplit with none)
  const int32_t L = static_cast<int32_t>(p.L), H = static_cast<int32_t>(p.H);
  for (int pass = 0; pass < 2; ++pass) {
    const auto& items = pass == 0 ? p.items : p.items_unsplit;
    const int32_t slots = pass == 0 ? static_cast<int32_t>(p.n_partial_slots) : 0;
    for (const bss::Item& it : items) {
      if (it.head < 0) continue;
      const bss::ItemFields f{it.head, it.qtile, it.begin, it.end, it.slot, it.piece, it.npieces};
      CHECK(bss::item_violations(f, H, L, static_cast<int32_t>(nnz), slots) == 0);
    }
  }
  for (int32_t e : p.kv_entries) CHECK(bss::entry_in_range(e, L));
  for (const bss::MergeRow& m : p.merge_rows)
    CHECK(bss::merge_row_violations(m.head, m.qtile, m.slot, m.npieces, H, L,
                                    static_cast<int32_t>(p.n_partial_slots)) == 0);
}

// The checks flag each kind of planted violation, and only that kind.
void test_range_check_predicates() {
  const int32_t H = 4, L = 1000, nnz = 50, slots = 6;  // 8 query tiles, 16 key tiles
  const bss::ItemFields ok{1, 7, 10, 20, 2, 1, 3};
  CHECK(bss::item_violations(ok, H, L, nnz, slots) == 0);
  auto with = [&](auto edit) { bss::ItemFields f = ok; edit(f); return bss::item_violations(f, H, L, nnz, slots); };
  CHECK(with([](bss::ItemFields& f) { f.head = 4; }) == bss::kCheckHead);
  CHECK(with([](bss::ItemFields& f) { f.head = -2; }) == bss::kCheckHead);
  CHECK(with([](bss::ItemFields& f) { f.qtile = 8; }) == bss::kCheckQTile);
  CHECK(with([](bss::ItemFields& f) { f.qtile = -1; }) == bss::kCheckQTile);
  CHECK(with([](bss::ItemFields& f) { f.end = 51; }) == bss::kCheckRange);
  CHECK(with([](bss::ItemFields& f) { f.begin = 21; }) == bss::kCheckRange);
  CHECK(with([](bss::ItemFields& f) { f.begin = -1; }) == bss::kCheckRange);
  CHECK(with([](bss::ItemFields& f) { f.piece = 3; }) == bss::kCheckPiece);
  CHECK(with([](bss::ItemFields& f) { f.npieces = 0; f.piece = 0; }) == bss::kCheckPiece);
  CHECK(with([](bss::ItemFields& f) { f.slot0 = 4; }) == bss::kCheckPiece);    // slots 4..6 of 6
  CHECK(with([](bss::ItemFields& f) { f.slot0 = 3; }) == 0);                    // slots 3..5
  CHECK(with([](bss::ItemFields& f) { f.npieces = 1; f.piece = 0; f.slot0 = 99; }) == 0);  // unsplit: no slot
  CHECK(with([](bss::ItemFields& f) { f.head = 9; f.end = 99; }) == (bss::kCheckHead | bss::kCheckRange));
  CHECK(bss::entry_in_range((15 << 1) | 1, L) && !bss::entry_in_range(16 << 1, L) && !bss::entry_in_range(-1, L));
  CHECK(bss::merge_row_violations(3, 7, 4, 2, H, L, slots) == 0);
  CHECK(bss::merge_row_violations(3, 7, 5, 2, H, L, slots) == bss::kCheckMergeRow);
  CHECK(bss::merge_row_violations(3, 7, 0, 1, H, L, slots) == bss::kCheckMergeRow);
  CHECK(bss::merge_row_violations(4, 0, 0, 2, H, L, slots) == bss::kCheckMergeRow);
}

attn_tensor fake_tensor(uintptr_t addr, int64_t B, int64_t L, int64_t H, int64_t D) {
  attn_tensor t{};
  t.data = reinterpret_cast<void*>(addr);
  t.B = B; t.L = L; t.H = H; t.D = D;
  t.stride_b = L * H * D; t.stride_l = H * D; t.stride_h = D;
  return t;
}

void test_cache_collision() {
  bss::PlanCache cache(8, size_t(1) << 30, same_hash);
  const attn_mask_desc a = chunk_desc(64), b = chunk_desc(32);
  std::shared_ptr<const attn_plan> pa, pb, pa2;
  CHECK(cache.get(&a, 512, 2, 64, &pa) == ATTN_OK);
  CHECK(cache.get(&b, 512, 2, 64, &pb) == ATTN_OK);   // same hash, other content: its own plan
  CHECK(pa != pb && cache.compiles() == 2 && cache.size() == 2);
  CHECK(pa->chunk == 64 && pb->chunk == 32 && pa->pairs_total != pb->pairs_total);
  CHECK(cache.get(&a, 512, 2, 64, &pa2) == ATTN_OK);
  CHECK(pa2 == pa && cache.compiles() == 2);
  // the same descriptor with another shape is another plan
  std::shared_ptr<const attn_plan> pc;
  CHECK(cache.get(&a, 1024, 2, 64, &pc) == ATTN_OK);
  CHECK(pc != pa && cache.compiles() == 3);
}

void test_cache_lru_and_content() {
  bss::PlanCache cache(2, size_t(1) << 30);
  const attn_mask_desc a = chunk_desc(64), b = chunk_desc(32), c = chunk_desc(16);
  std::shared_ptr<const attn_plan> p;
  CHECK(cache.get(&a, 512, 1, 64, &p) == ATTN_OK);
  std::shared_ptr<const attn_plan> held = p;            // stays valid after eviction
  CHECK(cache.get(&b, 512, 1, 64, &p) == ATTN_OK);
  CHECK(cache.get(&c, 512, 1, 64, &p) == ATTN_OK);
  CHECK(cache.size() == 2 && cache.compiles() == 3);
  CHECK(held->chunk == 64 && held->pairs_total == 512 * 64);
  CHECK(cache.get(&a, 512, 1, 64, &p) == ATTN_OK && cache.compiles() == 4);   // a was evicted
  // a block matrix edited in place (same pointer) is new content
  const int64_t L = 1024, nb = 8;
  std::vector<uint8_t> bm(nb * nb, 0);
  for (int m = 0; m < nb; ++m) bm[m * nb + m] = 1;
  attn_mask_desc d{};
  d.kind = ATTN_MASK_BLOCK;
  d.block = 128;
  d.block_mask = bm.data();
  d.block_mask_heads = 1;
  bss::PlanCache c2(4, size_t(1) << 30);
  std::shared_ptr<const attn_plan> q1, q2, q3;
  CHECK(c2.get(&d, L, 1, 128, &q1) == ATTN_OK);
  CHECK(c2.get(&d, L, 1, 128, &q3) == ATTN_OK && q3 == q1);
  bm[5 * nb + 2] = 1;
  CHECK(c2.get(&d, L, 1, 128, &q2) == ATTN_OK);
  CHECK(q2 != q1 && c2.compiles() == 2);
  CHECK(q2->kv_tile.size() == q1->kv_tile.size() + 2);                       // one 128-row tile x two 64-key tiles
  // byte budget: a cache that holds about one plan keeps only the newest
  bss::PlanCache c3(8, 1);
  CHECK(c3.get(&a, 512, 1, 64, &p) == ATTN_OK && c3.get(&b, 512, 1, 64, &p) == ATTN_OK);
  CHECK(c3.size() == 1);
}

void test_oneshot_uploads() {
  const int64_t B = 1, L = 1000, H = 2, D = 80;
  const attn_mask_desc a = chunk_desc(100), b = chunk_desc(50);
  size_t need = 0;
  CHECK(attn_workspace_bytes(&a, L, H, D, &need) == ATTN_OK && need > 0);
  attn_tensor q = fake_tensor(0x10000000, B, L, H, D), k = fake_tensor(0x20000000, B, L, H, D),
              v = fake_tensor(0x30000000, B, L, H, D), o = fake_tensor(0x40000000, B, L, H, D);
  attn_launch ln{};
  ln.workspace = reinterpret_cast<void*>(0x50000000);
  ln.workspace_bytes = need + (1 << 20);
  const size_t m0 = mock::counters.memcpy_calls, s0 = mock::counters.syncs, f0 = mock::counters.fwd_launches;
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &ln) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 1 && mock::counters.syncs == s0 + 1);
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &ln) == ATTN_OK);   // repeat: nothing copied
  CHECK(mock::counters.memcpy_calls == m0 + 1 && mock::counters.syncs == s0 + 1);
  CHECK(mock::counters.fwd_launches == f0 + 2);
  // the launch reads its lists from the workspace
  const bss::FwdParams& fp = mock::fwd_launches.back();
  const uintptr_t w0 = 0x50000000;
  CHECK(reinterpret_cast<uintptr_t>(fp.kv) >= w0 && reinterpret_cast<uintptr_t>(fp.kv) < w0 + need);
  CHECK(reinterpret_cast<uintptr_t>(fp.items) >= w0 && reinterpret_cast<uintptr_t>(fp.items) < w0 + need);
  // another mask into the same workspace copies its image, and then the first one again
  CHECK(attn_masked_fwd(&q, &k, &v, &b, nullptr, &o, &ln) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 2);
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &ln) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 3);
  // another workspace copies; a released workspace copies again
  attn_launch ln2 = ln;
  ln2.workspace = reinterpret_cast<void*>(0x60000000);
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &ln2) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 4);
  CHECK(attn_workspace_release(ln.workspace) == ATTN_OK);
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &ln) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 5);
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &ln2) == ATTN_OK);    // ln2 still holds it
  CHECK(mock::counters.memcpy_calls == m0 + 5);
  // an explicit upload of another plan into the workspace replaces the record
  attn_plan* pb = nullptr;
  CHECK(attn_plan_create(&b, L, H, D, &pb) == ATTN_OK);
  CHECK(attn_plan_upload(pb, ln.workspace, ln.workspace_bytes, nullptr) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 6);
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &ln) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 7);
  // errors leave no record behind: a too-small workspace fails and copies nothing
  attn_launch small = ln;
  small.workspace = reinterpret_cast<void*>(0x70000000);
  small.workspace_bytes = 16;
  CHECK(attn_masked_fwd(&q, &k, &v, &a, nullptr, &o, &small) == ATTN_E_WORKSPACE);
  CHECK(mock::counters.memcpy_calls == m0 + 7);
  attn_plan_destroy(pb);
  attn_workspace_release(ln.workspace);
  attn_workspace_release(ln2.workspace);
}

void test_noalloc() {
  const int64_t B = 1, L = 1000, H = 2, D = 128;
  const attn_mask_desc a = chunk_desc(100), b = chunk_desc(40);
  attn_tensor q = fake_tensor(0x10000000, B, L, H, D), k = fake_tensor(0x20000000, B, L, H, D),
              v = fake_tensor(0x30000000, B, L, H, D), o = fake_tensor(0x40000000, B, L, H, D);
  attn_launch ln{};
  const size_t m0 = mock::counters.memcpy_calls;
  CHECK(attn_masked_fwd_noalloc(&q, &k, &v, &a, nullptr, &o, &ln) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 1);
  CHECK(reinterpret_cast<uintptr_t>(mock::fwd_launches.back().kv) >= mock::kScratchAddr &&
        reinterpret_cast<uintptr_t>(mock::fwd_launches.back().kv) < mock::kScratchAddr + bss::kFwdScratchBytes);
  CHECK(attn_masked_fwd_noalloc(&q, &k, &v, &a, nullptr, &o, &ln) == ATTN_OK);   // the scratch holds it
  CHECK(mock::counters.memcpy_calls == m0 + 1);
  CHECK(attn_masked_fwd_noalloc(&q, &k, &v, &b, nullptr, &o, &ln) == ATTN_OK);
  CHECK(mock::counters.memcpy_calls == m0 + 2);
  attn_launch with_ws = ln;
  with_ws.workspace = reinterpret_cast<void*>(0x50000000);
  with_ws.workspace_bytes = 1 << 20;
  CHECK(attn_masked_fwd_noalloc(&q, &k, &v, &a, nullptr, &o, &with_ws) == ATTN_E_INVAL);
  // a plan larger than the scratch is refused before anything is copied
  const int64_t L2 = 65536, H2 = 16;
  attn_mask_desc full{};
  attn_tensor q2 = fake_tensor(0x10000000, 1, L2, H2, 64), k2 = fake_tensor(0x20000000, 1, L2, H2, 64),
              v2 = fake_tensor(0x30000000, 1, L2, H2, 64), o2 = fake_tensor(0x40000000, 1, L2, H2, 64);
  CHECK(attn_masked_fwd_noalloc(&q2, &k2, &v2, &full, nullptr, &o2, &ln) == ATTN_E_WORKSPACE);
  CHECK(std::string(attn_last_error()).find("bytes of scratch") != std::string::npos);
  CHECK(mock::counters.memcpy_calls == m0 + 2);
}

void test_backward_records() {
  const int64_t B = 1, L = 640, H = 2, D = 64;
  attn_mask_desc m{};
  m.kind = ATTN_MASK_WINDOW;
  m.left = 100;
  m.causal = 1;
  attn_plan* p = nullptr;
  CHECK(attn_plan_create(&m, L, H, D, &p) == ATTN_OK);
  size_t need = 0;
  CHECK(attn_bwd_workspace_bytes(p, B, H, &need) == ATTN_OK);
  attn_tensor t[8];
  for (int i = 0; i < 8; ++i) t[i] = fake_tensor(0x10000000 + 0x1000000 * i, B, L, H, D);
  attn_launch ln{};
  ln.workspace = reinterpret_cast<void*>(0x90000000);
  ln.workspace_bytes = need;
  const float* lse = reinterpret_cast<const float*>(0xA0000000);
  CHECK(attn_masked_bwd(p, &t[0], &t[1], &t[2], &t[3], &t[4], lse, nullptr, &t[5], &t[6], &t[7], nullptr, &ln) ==
        ATTN_E_INVAL);                                                       // not prepared
  CHECK(attn_bwd_upload(p, H, ln.workspace, ln.workspace_bytes, nullptr) == ATTN_OK);
  const size_t b0 = mock::counters.bwd_launches;
  CHECK(attn_masked_bwd(p, &t[0], &t[1], &t[2], &t[3], &t[4], lse, nullptr, &t[5], &t[6], &t[7], nullptr, &ln) ==
        ATTN_OK);
  CHECK(mock::counters.bwd_launches == b0 + 1);
  CHECK(attn_workspace_release(ln.workspace) == ATTN_OK);
  CHECK(attn_masked_bwd(p, &t[0], &t[1], &t[2], &t[3], &t[4], lse, nullptr, &t[5], &t[6], &t[7], nullptr, &ln) ==
        ATTN_E_INVAL);
  attn_plan_destroy(p);
}

void test_images_in_bounds() {
  struct Case {
    attn_mask_desc m;
    int64_t L, H, D;
  };
  std::vector<Case> cases;
  attn_mask_desc full{};
  cases.push_back({full, 4096, 16, 80});
  cases.push_back({chunk_desc(256), 4096, 16, 80});
  attn_mask_desc sw{};
  sw.kind = ATTN_MASK_WINDOW;
  sw.left = sw.right = 128;
  cases.push_back({sw, 4096, 16, 80});
  cases.push_back({sw, 1000, 3, 64});                                        // ragged tail
  static const int64_t hl[4] = {511, 1023, 2047, 4095};
  attn_mask_desc hw{};
  hw.kind = ATTN_MASK_WINDOW;
  hw.causal = 1;
  hw.head_left = hl;
  cases.push_back({hw, 4096, 4, 128});
  attn_mask_desc pf = sw;
  pf.prefix = 4;
  pf.causal = 1;
  cases.push_back({pf, 3000, 2, 128});
  static std::vector<uint8_t> bm;
  const int64_t nb = 64;
  bm.assign(2 * nb * nb, 0);
  uint32_t x = 12345;
  for (int h = 0; h < 2; ++h)
    for (int mrow = 0; mrow < nb; ++mrow)
      for (int n = 0; n <= mrow; ++n) {
        x = x * 1664525u + 1013904223u;
        bm[(h * nb + mrow) * nb + n] = (n == 0 || n == mrow || (x >> 31)) ? 1 : 0;
      }
  attn_mask_desc bk{};
  bk.kind = ATTN_MASK_BLOCK;
  bk.block = 128;
  bk.block_mask = bm.data();
  bk.block_mask_heads = 2;
  cases.push_back({bk, nb * 128, 2, 128});
  for (const Case& c : cases) {
    attn_plan* p = nullptr;
    CHECK(attn_plan_create(&c.m, c.L, c.H, c.D, &p) == ATTN_OK);
    if (p) {
      check_image(*p);
      attn_plan_destroy(p);
    }
  }
  // descriptors the compiler must reject
  attn_mask_desc bad = bk;
  bm[5] = 1;                                                                 // B[0][5] above the diagonal
  attn_plan* p = nullptr;
  CHECK(attn_plan_create(&bad, nb * 128, 2, 128, &p) == ATTN_E_INVAL && p == nullptr);
  attn_mask_desc neg = chunk_desc(0);
  CHECK(attn_plan_create(&neg, 100, 1, 64, &p) == ATTN_E_INVAL);
  CHECK(attn_plan_create(&full, 100, 1, 96, &p) == ATTN_E_UNSUPPORTED);
}

}  // namespace

int main() {
  test_cache_collision();
  test_cache_lru_and_content();
  test_oneshot_uploads();
  test_backward_records();
  test_noalloc();
  test_images_in_bounds();
  test_range_check_predicates();
  if (g_failures) {
    std::printf("%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
