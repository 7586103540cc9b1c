// Mask-descriptor compiler and tile scheduler.  Host C++17, no HIP calls.
//
// Mask semantics (0-based tokens i = query, j = key, both < L):
//   FULL    all j                                  (SHS slides, mask slide)
//   CHUNK   floor(i/C) == floor(j/C)               (same slide, "chunk window")
//   WINDOW  i - left_h <= j <= i + right           (inclusive; the serialisation
//                                                   slide's 7..23 example)
//   BLOCK   B_h[i/Bs][j/Bs] == 1 and j <= i         (RRAttention Eq. 2)
//   prefix  keys 0 .. prefix-1 are added to every row's set (FULL, CHUNK,
//           WINDOW; the StreamingLLM sink tokens kept beside a window).
//   causal = 1 additionally requires j <= i.
// For FULL, CHUNK and WINDOW the allowed keys of row i form one interval
// [lo(i), hi(i)) whose ends never decrease as i grows; the compiler works on
// those intervals.  BLOCK walks the kept blocks of each block row.

#include "plan.hpp"

#include "kernels.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>
#include <numeric>

namespace bss {

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Allowed interval [lo, hi) of row i for the interval kinds.
inline void row_interval(const attn_plan& p, int64_t h, int64_t i, int64_t* lo, int64_t* hi) {
  int64_t a = 0, b = p.L;
  if (p.kind == ATTN_MASK_CHUNK) {
    a = (i / p.chunk) * p.chunk;
    b = std::min(p.L, a + p.chunk);
  } else if (p.kind == ATTN_MASK_WINDOW) {
    a = std::max<int64_t>(0, i - p.head_left[h]);
    b = std::min(p.L, i + p.right + 1);
  }
  if (p.causal) b = std::min(b, i + 1);
  *lo = a;
  *hi = b;
}

// Prefix part [0, pe) of row i's allowed set (empty without a prefix).
inline int64_t row_prefix_end(const attn_plan& p, int64_t i) {
  int64_t pe = std::min(p.prefix, p.L);
  if (p.causal) pe = std::min(pe, i + 1);
  return pe;
}

attn_status validate(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D) {
  if (!m) { set_error("mask descriptor is NULL"); return ATTN_E_INVAL; }
  if (L < 1 || H < 1) { set_error("L and H must be >= 1"); return ATTN_E_INVAL; }
  if (L > (int64_t(1) << 30)) { set_error("L above 2^30 is not supported"); return ATTN_E_UNSUPPORTED; }
  if (H > 65535) { set_error("H above 65535 is not supported"); return ATTN_E_UNSUPPORTED; }
  if (D != 64 && D != 80 && D != 128 && D != 256) {
    set_error("head dim " + std::to_string(D) + " is not supported (64, 80, 128, 256)");
    return ATTN_E_UNSUPPORTED;
  }
  if (m->causal != 0 && m->causal != 1) { set_error("causal must be 0 or 1"); return ATTN_E_INVAL; }
  if (m->prefix < 0) { set_error("prefix must be >= 0"); return ATTN_E_INVAL; }
  if (m->prefix > 0 && m->kind == ATTN_MASK_BLOCK) {
    set_error("prefix tokens are not defined for BLOCK masks");
    return ATTN_E_INVAL;
  }
  switch (m->kind) {
    case ATTN_MASK_FULL:
      break;
    case ATTN_MASK_CHUNK:
      if (m->chunk < 1) { set_error("chunk size must be >= 1"); return ATTN_E_INVAL; }
      break;
    case ATTN_MASK_WINDOW:
      if (m->left < 0 || m->right < 0) { set_error("window reach must be >= 0"); return ATTN_E_INVAL; }
      if (m->head_left) {
        for (int64_t h = 0; h < H; ++h)
          if (m->head_left[h] < 0) { set_error("head_left entries must be >= 0"); return ATTN_E_INVAL; }
      }
      break;
    case ATTN_MASK_BLOCK: {
      if (m->block < 1) { set_error("block size must be >= 1"); return ATTN_E_INVAL; }
      if (!m->block_mask) { set_error("block_mask is NULL"); return ATTN_E_INVAL; }
      if (m->block_mask_heads != 1 && m->block_mask_heads != H) {
        set_error("block_mask_heads must be 1 or H");
        return ATTN_E_INVAL;
      }
      const int64_t nb = ceil_div(L, m->block);
      for (int64_t hb = 0; hb < m->block_mask_heads; ++hb) {
        const uint8_t* b = m->block_mask + hb * nb * nb;
        for (int64_t r = 0; r < nb; ++r)
          for (int64_t c = r + 1; c < nb; ++c)
            if (b[r * nb + c]) {
              set_error("block_mask has B[" + std::to_string(r) + "][" + std::to_string(c) +
                        "] = 1 above the diagonal (causality, RRAttention Eq. 5)");
              return ATTN_E_INVAL;
            }
      }
      break;
    }
    default:
      set_error("unknown mask kind " + std::to_string(m->kind));
      return ATTN_E_INVAL;
  }
  return ATTN_OK;
}

// Lists for FULL / CHUNK / WINDOW.
void compile_intervals(attn_plan& p) {
  const int64_t bm = p.bm, bn = p.bn;
  std::vector<int32_t> diff(p.nk + 1);
  p.row_ptr.assign(1, 0);
  p.pairs.assign(p.H, 0);
  for (int64_t h = 0; h < p.H; ++h) {
    for (int64_t qt = 0; qt < p.nq; ++qt) {
      const int64_t i0 = qt * bm, i1 = std::min(p.L, i0 + bm);
      std::fill(diff.begin(), diff.end(), 0);
      int64_t max_lo = 0, min_hi = p.L;
      for (int64_t i = i0; i < i1; ++i) {
        int64_t lo, hi;
        row_interval(p, h, i, &lo, &hi);
        max_lo = std::max(max_lo, lo);
        min_hi = std::min(min_hi, hi);
        const int64_t pe = row_prefix_end(p, i);
        if (pe > 0) {
          diff[0] += 1;
          diff[(pe - 1) / bn + 1] -= 1;
        }
        if (hi <= lo) {
          p.pairs[h] += pe;
          continue;
        }
        p.pairs[h] += (hi - lo) + pe - std::max<int64_t>(0, std::min(pe, hi) - lo);
        diff[lo / bn] += 1;
        diff[(hi - 1) / bn + 1] -= 1;
      }
      int32_t run = 0;
      const bool rows_full = (i1 - i0) == bm;
      for (int64_t kt = 0; kt < p.nk; ++kt) {
        run += diff[kt];
        if (run <= 0) continue;
        const int64_t j0 = kt * bn, j1 = j0 + bn;
        bool full = rows_full && j1 <= p.L && max_lo <= j0 && min_hi >= j1;
        if (!full && p.prefix > 0 && rows_full && j1 <= p.L) {
          // every row must cover [j0, j1) with its prefix, its window or both joined
          full = true;
          for (int64_t i = i0; full && i < i1; ++i) {
            int64_t lo, hi;
            row_interval(p, h, i, &lo, &hi);
            const int64_t pe = row_prefix_end(p, i);
            const bool joined = hi > lo && lo <= pe;
            const bool covered = (j1 <= pe) || (hi > lo && j0 >= lo && j1 <= hi) ||
                                 (joined && j1 <= std::max(hi, pe));
            full = covered;
          }
        }
        p.kv_tile.push_back(static_cast<int32_t>(kt));
        p.flags.push_back(full ? 1 : 0);
      }
      p.row_ptr.push_back(static_cast<int32_t>(p.kv_tile.size()));
    }
  }
}

// Lists for BLOCK: walk the kept blocks of each block row overlapping the query tile.
void compile_blocks(attn_plan& p) {
  const int64_t bm = p.bm, bn = p.bn, bs = p.block, nb = p.nb;
  std::vector<uint8_t> present(p.nk);
  p.row_ptr.assign(1, 0);
  p.pairs.assign(p.H, 0);
  for (int64_t h = 0; h < p.H; ++h) {
    const uint8_t* B = p.block_mask.data() + (p.block_heads > 1 ? h : 0) * nb * nb;
    // pairs: per block row, full-width kept blocks to the left plus the causal diagonal block
    for (int64_t br = 0; br < nb; ++br) {
      const int64_t r0 = br * bs, r1 = std::min(p.L, r0 + bs);
      int64_t width = 0;
      for (int64_t bc = 0; bc < br; ++bc)
        if (B[br * nb + bc]) width += std::min(p.L, (bc + 1) * bs) - bc * bs;
      int64_t pr = (r1 - r0) * width;
      if (B[br * nb + br]) {
        const int64_t n = r1 - r0;
        pr += n * (n + 1) / 2;
      }
      p.pairs[h] += pr;
    }
    for (int64_t qt = 0; qt < p.nq; ++qt) {
      const int64_t i0 = qt * bm, i1 = std::min(p.L, i0 + bm);
      std::fill(present.begin(), present.end(), 0);
      for (int64_t br = i0 / bs; br <= (i1 - 1) / bs; ++br) {
        const int64_t r1 = std::min(i1, (br + 1) * bs);     // rows of this tile in block row br
        for (int64_t bc = 0; bc <= br; ++bc) {
          if (!B[br * nb + bc]) continue;
          const int64_t c0 = bc * bs;
          const int64_t c1 = std::min({p.L, (bc + 1) * bs, r1});  // j <= i < r1
          if (c1 <= c0) continue;
          for (int64_t kt = c0 / bn; kt <= (c1 - 1) / bn; ++kt) present[kt] = 1;
        }
      }
      for (int64_t kt = 0; kt < p.nk; ++kt) {
        if (!present[kt]) continue;
        const int64_t j0 = kt * bn, j1 = j0 + bn;
        bool full = (i1 - i0) == bm && j1 <= p.L && (j1 - 1) <= i0;
        for (int64_t br = i0 / bs; full && br <= (i1 - 1) / bs; ++br)
          for (int64_t bc = j0 / bs; full && bc <= (j1 - 1) / bs; ++bc)
            if (!B[br * nb + bc]) full = false;
        p.kv_tile.push_back(static_cast<int32_t>(kt));
        p.flags.push_back(full ? 1 : 0);
      }
      p.row_ptr.push_back(static_cast<int32_t>(p.kv_tile.size()));
    }
  }
}

// Work schedule.
//
// Cost of a (head, query tile) row: its listed tiles (a PARTIAL tile counts
// 1.25 for the masking) plus 0.5 for the Q load and the epilogue.  Rows much
// longer than T = max(total / (kPieceShare kSlots), kMinPiece) are cut into
// pieces of about T tiles (batch 1 only), so that a causal or per-head-window
// launch with about as many rows as resident work-groups is not held up by
// its longest rows.  T is 1 / kPieceShare times the fair share of a resident
// work-group: an item's prologue (item record, Q rows, first list entries and
// copies: about three tiles' time) and the merge of a piece's partial state
// cost more than the imbalance that longer pieces leave (per-head windows at
// 4K tokens, pieces of 1, 1.1, 1.25, 1.33, 1.43, 1.67 times the fair share:
// 80.4, 78.9, 78.5, 77.7, 75.9, 81.6 us).  Items are then laid out as kXcds queues:
// heads in descending cost, rows of a head in descending cost, and the
// sequence cut into kXcds consecutive runs of equal total cost (so the work
// that shares an XCD's L2 comes from as few heads as possible; measured
// better than dealing a head's rows to all XCDs for the 16K-token windows and
// the 128K-token block masks).  A queue short enough to run in a few rounds of
// its work-groups is ordered by descending cost.  A launch of at most two
// rounds whose item costs are uneven gives whole heads to XCDs, longest
// first to the least-loaded one, when that balances the XCDs within 5 %
// (else its items are dealt longest first to the least-loaded queue).
// Queues are padded to equal length with null items.
constexpr double kPingPongMinTiles = 32.0;  // d = 128: mean row cost (tiles) from which the ping-pong kernel runs
constexpr double kMinPiece = 12.0;     // tiles: below this a piece's merge costs more than it saves
constexpr double kPieceShare = 0.7;    // pieces are sized for this fraction of the resident work-groups
constexpr double kPieceOverhead = 2.0; // tiles: writing the partial state and the merge
constexpr int kMaxPieces = 16;
constexpr double kHeadSpread = 1.05;   // largest XCD load / mean for whole heads per XCD

std::vector<Item> layout_queues(const std::vector<int64_t>& head_order, const std::vector<Item>& all,
                                const std::vector<double>& icost) {
  // items of each head, in descending cost (stable: query tile, then piece)
  int64_t H = static_cast<int64_t>(head_order.size());
  std::vector<std::vector<int64_t>> by_head(H);
  for (size_t i = 0; i < all.size(); ++i) by_head[all[i].head].push_back(static_cast<int64_t>(i));
  std::vector<int64_t> seq;
  seq.reserve(all.size());
  for (int64_t h : head_order) {
    auto& v = by_head[h];
    std::stable_sort(v.begin(), v.end(), [&](int64_t a, int64_t b) { return icost[a] > icost[b]; });
    seq.insert(seq.end(), v.begin(), v.end());
  }
  std::vector<std::vector<int64_t>> q(kXcds);
  double cmax = 0.0, csum = 0.0;
  for (int64_t i : seq) {
    cmax = std::max(cmax, icost[i]);
    csum += icost[i];
  }
  const bool uneven = !seq.empty() && cmax > 1.5 * csum / static_cast<double>(seq.size());
  if (uneven && seq.size() <= static_cast<size_t>(2 * kSlots)) {
    // At most two rounds of work-groups.  Whole heads go to XCDs, longest
    // first to the least-loaded one, so that a head's key/value tiles are
    // read into one L2 only; if that leaves an XCD more than kHeadSpread
    // above the mean, items go longest first over all queues instead (LPT).
    std::vector<double> hc(H, 0.0);
    for (int64_t i : seq) hc[all[i].head] += icost[i];
    std::vector<int64_t> hs(head_order);
    std::stable_sort(hs.begin(), hs.end(), [&](int64_t a, int64_t b) { return hc[a] > hc[b]; });
    std::vector<double> load(kXcds, 0.0);
    std::vector<int> xcd_of(H, 0);
    for (int64_t h : hs) {
      int x = 0;
      for (int y = 1; y < kXcds; ++y)
        if (load[y] < load[x]) x = y;
      xcd_of[h] = x;
      load[x] += hc[h];
    }
    const double lmax = *std::max_element(load.begin(), load.end());
    if (H >= kXcds && lmax <= kHeadSpread * csum / kXcds) {
      for (int64_t i : seq) q[xcd_of[all[i].head]].push_back(i);
    } else {
      std::stable_sort(seq.begin(), seq.end(), [&](int64_t a, int64_t b) { return icost[a] > icost[b]; });
      std::fill(load.begin(), load.end(), 0.0);
      for (int64_t i : seq) {
        int x = 0;
        for (int y = 1; y < kXcds; ++y)
          if (load[y] < load[x]) x = y;
        q[x].push_back(i);
        load[x] += icost[i];
      }
    }
  } else {
    // consecutive runs of equal cost: an XCD works through few heads at a time
    double total = 0.0;
    for (int64_t i : seq) total += icost[i];
    double cum = 0.0;
    for (int64_t i : seq) {
      const double mid = cum + 0.5 * icost[i];
      int x = total > 0.0 ? static_cast<int>(mid / total * kXcds) : 0;
      x = std::min(std::max(x, 0), kXcds - 1);
      q[x].push_back(i);
      cum += icost[i];
    }
  }
  size_t len = 0;
  for (auto& v : q) {
    if (v.size() <= static_cast<size_t>(4 * kSlots / kXcds))
      std::stable_sort(v.begin(), v.end(), [&](int64_t a, int64_t b) { return icost[a] > icost[b]; });
    len = std::max(len, v.size());
  }
  std::vector<Item> out;
  out.reserve(len * kXcds);
  const Item null_item{-1, 0, 0, 0, 0, 0, 1, 0};
  for (auto& v : q) {
    for (int64_t i : v) out.push_back(all[i]);
    out.insert(out.end(), len - v.size(), null_item);
  }
  return out;
}

void schedule(attn_plan& p) {
  const int64_t rows = p.H * p.nq;
  std::vector<double> cost(rows);
  std::vector<double> head_cost(p.H, 0.0);
  double total = 0.0;
  for (int64_t r = 0; r < rows; ++r) {
    double c = 0.5;  // Q load and epilogue
    for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e) c += p.flags[e] ? 1.0 : 1.25;
    cost[r] = c;
    head_cost[r / p.nq] += c;
    total += c;
  }
  std::vector<int64_t> heads(p.H);
  std::iota(heads.begin(), heads.end(), 0);
  std::stable_sort(heads.begin(), heads.end(),
                   [&](int64_t a, int64_t b) { return head_cost[a] > head_cost[b]; });
  p.pingpong = p.D == 128 && total >= kPingPongMinTiles * static_cast<double>(rows);

  // unsplit schedule (batch > 1)
  std::vector<Item> whole(rows);
  for (int64_t r = 0; r < rows; ++r)
    whole[r] = Item{static_cast<int32_t>(r / p.nq), static_cast<int32_t>(r % p.nq), p.row_ptr[r],
                    p.row_ptr[r + 1], 0, 0, 1, 0};
  p.items_unsplit = layout_queues(heads, whole, cost);

  // batch-1 schedule: long rows cut into pieces
  const double share = std::max(total / (kPieceShare * kSlots), kMinPiece);
  std::vector<Item> all;
  std::vector<double> icost;
  all.reserve(rows);
  icost.reserve(rows);
  int64_t slots = 0, groups = 0;
  for (int64_t r = 0; r < rows; ++r) {
    const int32_t b = p.row_ptr[r], e = p.row_ptr[r + 1], n = e - b;
    int np = 1;
    if (cost[r] > 1.25 * share)
      np = static_cast<int>(std::min<double>({std::ceil(cost[r] / share), double(kMaxPieces), double(n)}));
    if (np <= 1) {
      all.push_back(whole[r]);
      icost.push_back(cost[r]);
      continue;
    }
    for (int k = 0; k < np; ++k) {
      const int32_t pb = b + static_cast<int32_t>(int64_t(n) * k / np);
      const int32_t pe = b + static_cast<int32_t>(int64_t(n) * (k + 1) / np);
      double c = 0.5 + kPieceOverhead;
      for (int32_t x = pb; x < pe; ++x) c += p.flags[x] ? 1.0 : 1.25;
      all.push_back(Item{whole[r].head, whole[r].qtile, pb, pe, static_cast<int32_t>(slots), k, np,
                         static_cast<int32_t>(groups)});
      icost.push_back(c);
    }
    p.merge_rows.push_back(MergeRow{whole[r].head, whole[r].qtile, static_cast<int32_t>(slots), np});
    slots += np;
    groups += 1;
  }
  p.n_partial_slots = slots;
  p.items = layout_queues(heads, all, icost);
}

void build_image(attn_plan& p) {
  p.kv_entries.resize(p.kv_tile.size());
  for (size_t e = 0; e < p.kv_tile.size(); ++e) p.kv_entries[e] = (p.kv_tile[e] << 1) | p.flags[e];
  p.head_left32.assign(p.H, 0);
  if (p.kind == ATTN_MASK_WINDOW)
    for (int64_t h = 0; h < p.H; ++h)
      p.head_left32[h] = static_cast<int32_t>(std::min<int64_t>(p.head_left[h], p.L));
  if (p.kind == ATTN_MASK_BLOCK && !p.block_aligned) {
    const int64_t words = ceil_div(p.nb, 32);
    p.block_bits.assign(static_cast<size_t>(p.block_heads) * p.nb * words, 0u);
    for (int64_t hb = 0; hb < p.block_heads; ++hb)
      for (int64_t r = 0; r < p.nb; ++r)
        for (int64_t c = 0; c <= r; ++c)
          if (p.block_mask[(hb * p.nb + r) * p.nb + c])
            p.block_bits[(hb * p.nb + r) * words + c / 32] |= 1u << (c % 32);
  }
  ImageLayout& l = p.layout;
  l.off_items = 0;
  l.off_items_unsplit = align_up(l.off_items + p.items.size() * sizeof(Item));
  l.off_kv = align_up(l.off_items_unsplit + p.items_unsplit.size() * sizeof(Item));
  l.off_head_left = align_up(l.off_kv + std::max<size_t>(1, p.kv_entries.size()) * sizeof(int32_t));
  l.off_bits = align_up(l.off_head_left + p.head_left32.size() * sizeof(int32_t));
  l.off_merge = align_up(l.off_bits + p.block_bits.size() * sizeof(uint32_t));
  l.bytes = align_up(l.off_merge + p.merge_rows.size() * sizeof(MergeRow));
  l.off_partials = l.bytes;
  l.total = align_up(l.off_partials + static_cast<size_t>(p.n_partial_slots) *
                                          static_cast<size_t>(partial_slot_floats(p.D)) * sizeof(float));
}

}  // namespace

attn_status compile_plan(const attn_mask_desc* m, int64_t L, int64_t H, int64_t D, attn_plan** out) {
  if (!out) { set_error("output pointer is NULL"); return ATTN_E_INVAL; }
  attn_status st = validate(m, L, H, D);
  if (st != ATTN_OK) return st;
  attn_plan* p = nullptr;
  try {
    p = new attn_plan();
    p->kind = m->kind;
    p->causal = m->causal;
    p->prefix = m->prefix;
    p->L = L; p->H = H; p->D = D;
    p->nq = ceil_div(L, p->bm);
    p->nk = ceil_div(L, p->bn);
    if (m->kind == ATTN_MASK_CHUNK) p->chunk = m->chunk;
    if (m->kind == ATTN_MASK_WINDOW) {
      p->left = m->left;
      p->right = std::min<int64_t>(m->right, L);
      p->head_left.resize(H);
      for (int64_t h = 0; h < H; ++h)
        p->head_left[h] = std::min<int64_t>(m->head_left ? m->head_left[h] : m->left, L);
    }
    if (m->kind == ATTN_MASK_BLOCK) {
      p->block = m->block;
      p->block_heads = m->block_mask_heads;
      p->nb = ceil_div(L, m->block);
      p->block_mask.resize(static_cast<size_t>(p->block_heads) * p->nb * p->nb);
      for (size_t i = 0; i < p->block_mask.size(); ++i) p->block_mask[i] = m->block_mask[i] ? 1 : 0;
      p->block_aligned = (p->block % p->bm == 0) && (p->block % p->bn == 0);
      compile_blocks(*p);
    } else {
      compile_intervals(*p);
    }
    p->pairs_total = std::accumulate(p->pairs.begin(), p->pairs.end(), int64_t(0));
    if (p->kv_tile.size() > static_cast<size_t>(INT32_MAX)) {
      delete p;
      set_error("tile list longer than 2^31 entries");
      return ATTN_E_UNSUPPORTED;
    }
    schedule(*p);
    build_image(*p);
    static std::atomic<uint64_t> next_serial{1};
    p->serial = next_serial.fetch_add(1);
  } catch (const std::bad_alloc&) {
    delete p;
    set_error("host allocation failed while compiling the plan");
    return ATTN_E_NOMEM;
  }
  *out = p;
  return ATTN_OK;
}

const BwdImage& bwd_image(const attn_plan& p, int64_t kv_heads) {
  std::lock_guard<std::mutex> lk(p.bwd_mu);
  auto it = p.bwd_images.find(kv_heads);
  if (it != p.bwd_images.end()) return *it->second;
  auto img = std::make_unique<BwdImage>();
  const int64_t g = p.H / kv_heads;
  const int64_t nkb = ceil_div(p.L, 2 * static_cast<int64_t>(kBN));
  img->kv_heads = kv_heads;
  img->nkb = nkb;
  // per (query head, key block): query tiles listing tile 2kb or 2kb+1, and
  // whether every pair of the block is allowed (both tiles FULL, or the
  // block's second tile lies past the sequence end)
  std::vector<std::vector<int32_t>> per(static_cast<size_t>(p.H * nkb));
  for (int64_t h = 0; h < p.H; ++h) {
    for (int64_t qt = 0; qt < p.nq; ++qt) {
      const int64_t r = h * p.nq + qt;
      int64_t last_kb = -1;
      for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e) {
        const int64_t kt = p.kv_tile[e], kb = kt / 2;
        const bool half_full = p.flags[e] != 0;
        std::vector<int32_t>& v = per[static_cast<size_t>(h * nkb + kb)];
        if (kb != last_kb) {
          // first tile of this block in the row: FULL only if it is tile 2kb
          // and tile 2kb+1 either follows FULL or does not exist
          const bool second_exists = 2 * kb + 1 < p.nk;
          bool full = half_full && (kt == 2 * kb);
          if (full && second_exists) {
            const bool next_listed = e + 1 < p.row_ptr[r + 1] && p.kv_tile[e + 1] == kt + 1;
            full = next_listed && p.flags[e + 1] != 0;
          }
          v.push_back(static_cast<int32_t>((qt << 1) | (full ? 1 : 0)));
          last_kb = kb;
        }
      }
    }
  }
  // per (kv head, key block): the group's lists in head order; cost of an item
  std::vector<Item> all;
  std::vector<double> cost;
  std::vector<double> head_cost(static_cast<size_t>(kv_heads), 0.0);
  all.reserve(static_cast<size_t>(kv_heads * nkb));
  img->col_ptr.assign(1, 0);
  for (int64_t hk = 0; hk < kv_heads; ++hk) {
    for (int64_t kb = 0; kb < nkb; ++kb) {
      const int32_t begin = static_cast<int32_t>(img->col.size());
      double c = 1.0;  // K, V fragment loads and the dK, dV stores
      for (int64_t gi = 0; gi < g; ++gi) {
        for (int32_t x : per[static_cast<size_t>((hk * g + gi) * nkb + kb)]) {
          img->col.push_back(static_cast<int32_t>((gi << 24) | x));
          c += (x & 1) ? 2.0 : 2.25;  // two 64-row steps; masking on PARTIAL entries
        }
      }
      all.push_back(Item{static_cast<int32_t>(hk), static_cast<int32_t>(kb), begin,
                         static_cast<int32_t>(img->col.size()), 0, 0, 1, 0});
      img->col_ptr.push_back(static_cast<int32_t>(img->col.size()));
      cost.push_back(c);
      head_cost[static_cast<size_t>(hk)] += c;
    }
  }
  std::vector<int64_t> heads(static_cast<size_t>(kv_heads));
  std::iota(heads.begin(), heads.end(), 0);
  std::stable_sort(heads.begin(), heads.end(), [&](int64_t a, int64_t b) { return head_cost[a] > head_cost[b]; });
  img->items = layout_queues(heads, all, cost);
  // batch-1 schedule: items much longer than the fair share of the resident
  // work-groups (one per CU at d = 128, two otherwise) cut into pieces of
  // consecutive entries; each piece then pays for its partial sums
  {
    double total = 0.0;
    for (double c : cost) total += c;
    const double slots = (p.D >= 128 ? 1.0 : 2.0) * kSlots / 2;
    const double share = std::max(total / slots, kMinPiece);
    std::vector<Item> parts;
    std::vector<double> pcost;
    int64_t nslot = 0;
    for (size_t i = 0; i < all.size(); ++i) {
      const Item& it = all[i];
      const int32_t n = it.end - it.begin;
      int np = 1;
      if (cost[i] > 1.25 * share)
        np = static_cast<int>(std::min<double>({std::ceil(cost[i] / share), double(kMaxPieces), double(n)}));
      if (np <= 1) {
        parts.push_back(it);
        pcost.push_back(cost[i]);
        continue;
      }
      for (int k = 0; k < np; ++k) {
        const int32_t pb = it.begin + static_cast<int32_t>(int64_t(n) * k / np);
        const int32_t pe = it.begin + static_cast<int32_t>(int64_t(n) * (k + 1) / np);
        double c = 1.0 + kPieceOverhead;
        for (int32_t x = pb; x < pe; ++x) c += (img->col[x] & 1) ? 2.0 : 2.25;
        parts.push_back(Item{it.head, it.qtile, pb, pe, static_cast<int32_t>(nslot), k, np,
                             static_cast<int32_t>(img->merge.size())});
        pcost.push_back(c);
      }
      img->merge.push_back(MergeRow{it.head, it.qtile, static_cast<int32_t>(nslot), np});
      nslot += np;
    }
    img->n_slots = nslot;
    img->items_split = img->merge.empty() ? img->items : layout_queues(heads, parts, pcost);
  }
  img->off_items = 0;
  img->off_items_split = align_up(img->items.size() * sizeof(Item));
  img->off_merge = align_up(img->off_items_split + img->items_split.size() * sizeof(Item));
  img->off_col = align_up(img->off_merge + img->merge.size() * sizeof(MergeRow));
  img->bytes = align_up(img->off_col + std::max<size_t>(1, img->col.size()) * sizeof(int32_t));
  const BwdImage& ref = *img;
  p.bwd_images.emplace(kv_heads, std::move(img));
  return ref;
}

BwdLayout bwd_layout(const attn_plan& p, const BwdImage& img, int64_t B) {
  BwdLayout l;
  l.off_image = align_up(p.layout.total);
  l.off_stat = align_up(l.off_image + img.bytes);
  const size_t lpad = static_cast<size_t>(p.nq) * kBM;
  l.off_sinkpart = align_up(l.off_stat + static_cast<size_t>(B) * p.H * 2 * lpad * sizeof(float));
  l.off_qs = align_up(l.off_sinkpart + static_cast<size_t>(B) * p.H * p.nq * sizeof(float));
  l.off_dkdv = align_up(l.off_qs + static_cast<size_t>(B) * p.H * p.L * p.D * sizeof(uint16_t));
  const size_t dkdv = B == 1 ? static_cast<size_t>(img.n_slots) * dkdv_slot_floats(p.D) * sizeof(float) : 0;
  l.total = align_up(l.off_dkdv + dkdv);
  return l;
}

void write_bwd_image(const BwdImage& img, uint8_t* dst) {
  std::memset(dst, 0, img.bytes);
  std::memcpy(dst + img.off_items, img.items.data(), img.items.size() * sizeof(Item));
  std::memcpy(dst + img.off_items_split, img.items_split.data(), img.items_split.size() * sizeof(Item));
  if (!img.merge.empty()) std::memcpy(dst + img.off_merge, img.merge.data(), img.merge.size() * sizeof(MergeRow));
  if (!img.col.empty()) std::memcpy(dst + img.off_col, img.col.data(), img.col.size() * sizeof(int32_t));
}

void write_image(const attn_plan& p, uint8_t* dst) {
  std::memset(dst, 0, p.layout.bytes);
  std::memcpy(dst + p.layout.off_items, p.items.data(), p.items.size() * sizeof(Item));
  std::memcpy(dst + p.layout.off_items_unsplit, p.items_unsplit.data(), p.items_unsplit.size() * sizeof(Item));
  std::memcpy(dst + p.layout.off_kv, p.kv_entries.data(), p.kv_entries.size() * sizeof(int32_t));
  std::memcpy(dst + p.layout.off_head_left, p.head_left32.data(), p.head_left32.size() * sizeof(int32_t));
  if (!p.block_bits.empty())
    std::memcpy(dst + p.layout.off_bits, p.block_bits.data(), p.block_bits.size() * sizeof(uint32_t));
  if (!p.merge_rows.empty())
    std::memcpy(dst + p.layout.off_merge, p.merge_rows.data(), p.merge_rows.size() * sizeof(MergeRow));
}

}  // namespace bss
