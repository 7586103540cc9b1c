// Structured-mask softmax attention forward, head dim 128, for gfx950.
// The computation is attn_fwd_kernel's (attn_fwd.hip: the exact tiled softmax
// over the item's listed key tiles, sink in the denominator, PARTIAL-tile
// masking, split rows); this file arranges it for two wave groups.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fwd_common.hpp"
#include "kernels.hpp"
#include "tile_common.hpp"

namespace bss {
namespace {

using namespace dev;

// Two wave groups in ping-pong.
//
// One work-group of 8 waves takes one work item (128 query rows).  Waves 0-3
// (group A) and waves 4-7 (group B) each hold all 128 rows (wave w of a
// group: rows 32 (w mod 4) .. +31), and each group walks every other tile of
// the item's list (A entries 0, 2, 4, ..., B entries 1, 3, 5, ...) with its
// own double-buffered K/V tiles in LDS.  A group's tile j takes two phases:
//   M_j  S^T_j = K_j Q^T and O^T += V_{j-1}^T P^T_{j-1}: 32 MFMAs, LDS
//        fragment reads, nothing else;
//   V_j  the copies of tile j+2's keys and tile j+1's values into LDS, the
//        mask (PARTIAL tiles), the exponentials of S_j, the row sums, and the
//        first fragments of M_{j+1}.
// Every phase ends at a work-group barrier, and group B runs one phase behind
// group A, so the two waves of each SIMD (wave w and wave w + 4) always run
// different phases: while one issues MFMAs the other does its softmax.  The
// ordering the barriers give is the only exchange between the groups until
// the end, where group B's running state (reference, sum, accumulators) goes
// through LDS and group A merges it into its own and writes the result.
// Buffers: a group's pair p = (K_p, V_{p-1}) sits in its buffer set p mod 2;
// M_j reads pair j, V_j issues pair j+2 into the set M_j has just finished
// with, and the wait for pair j+1 comes before the barrier that ends M_j.
template <bool PREFIX>
__global__ __launch_bounds__(512, 1) void attn_fwd_pp_kernel(const GroupParams g) {
  constexpr int D = 128;
  using S = Shape<D>;
  using L = Lds<D>;
  static_assert(L::PADDED, "the ping-pong kernel uses the padded d = 128 tiles");
  constexpr int64_t kSlotFloats = partial_slot_floats(D);
  constexpr int kSlotM = 4 * S::DT * 16 * 64;
  constexpr int kSlotL = kSlotM + 4 * 64;
  constexpr int kSetBytes = L::KT + L::VT;         // one pair (K tile + V tile)
  constexpr int kGroupBytes = 2 * kSetBytes;       // two pairs per group
  constexpr int NQ = 2 * S::KS;                    // 16 QK MFMAs per tile
  constexpr int NP = 4 * S::DT;                    // 16 PV MFMAs per tile
  // group B's state for the merge (per wave: acc as float4 [DT][4][64], then m, l, redo flag per lane)
  constexpr int kXFloats = S::DT * 16 * 64 + 3 * 64;
  static_assert(4 * kXFloats * 4 <= 2 * kGroupBytes, "merge staging must fit in the tile buffers");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kGroupBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5;
  const int l31 = lane & 31;

  int pos = static_cast<int>(blockIdx.x / 8), jb = 0;
  while (jb + 1 < g.n_jobs && pos >= g.queue_len[jb]) pos -= g.queue_len[jb++];
  const int job = __builtin_amdgcn_readfirstlane(jb);
  pos = __builtin_amdgcn_readfirstlane(pos);
  if (pos >= g.queue_len[job]) return;
  const FwdParams& p = g.job[job];
  const int item_idx = static_cast<int>(blockIdx.x % 8) * g.queue_len[job] + pos;
  const int4 item = reinterpret_cast<const int4*>(p.items)[2 * item_idx];
  const int4 split = reinterpret_cast<const int4*>(p.items)[2 * item_idx + 1];
  const int head = __builtin_amdgcn_readfirstlane(item.x);
  if (head < 0) return;  // queue padding
  if constexpr (kChecked) {
    if (!item_checked(p, item, split)) return;
  }
  const int qtile = __builtin_amdgcn_readfirstlane(item.y);
  const int e_begin = __builtin_amdgcn_readfirstlane(item.z);
  const int e_end = __builtin_amdgcn_readfirstlane(item.w);
  const int slot0 = __builtin_amdgcn_readfirstlane(split.x);
  const int piece = __builtin_amdgcn_readfirstlane(split.y);
  const int npieces = __builtin_amdgcn_readfirstlane(split.z);
  const int b = blockIdx.y;

  // Roles: the two waves that share a SIMD must belong to different groups,
  // and which waves share one is up to the dispatcher, so every wave reads
  // its SIMD from the hardware id and the roles follow: on each SIMD the
  // lower-numbered wave joins group A, the other group B, and both take the
  // rows 32 s .. 32 s + 31 of SIMD s.  (Any other placement falls back to
  // waves 0-3 / 4-7, which is correct but without the alternation.)
  int grp, wq;
  {
    int hw;
    __asm__ volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    const int simd = (hw >> 4) & 3;
    int* simd_of = reinterpret_cast<int*>(smem);
    if (lane == 0) simd_of[wave] = simd;
    wg_barrier();
    int counts = 0, rank = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int sw = simd_of[w];
      counts += 1 << (8 * sw);
      rank += (w < wave && sw == simd) ? 1 : 0;
    }
    const bool paired = counts == 0x02020202;
    grp = __builtin_amdgcn_readfirstlane(paired ? rank : (wave >> 2));
    wq = __builtin_amdgcn_readfirstlane(paired ? simd : (wave & 3));
    wg_barrier();  // every wave has read the table before the tiles reuse the memory
  }

  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q + b * p.q_sb + head * p.q_sh);
  const int kv_head = head / p.kv_group;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k + b * p.k_sb + kv_head * p.k_sh);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v + b * p.v_sb + kv_head * p.v_sh);
  unsigned char* obase = reinterpret_cast<unsigned char*>(p.o + b * p.o_sb + head * p.o_sh);
  const int64_t q_row_bytes = p.q_sl * 2, k_row_bytes = p.k_sl * 2, v_row_bytes = p.v_sl * 2,
                o_row_bytes = p.o_sl * 2;

  // kept in registers: read from the parameter block inside the loop, these
  // would be reloaded after every barrier and copy (a scalar load and a wait
  // that also drains the wave's LDS reads)
  const int32_t* const kv_list = p.kv;
  const int seq_len = p.L;
  const int n = e_end - e_begin;
  const int ng = (n - grp + 1) >> 1;  // this group's tiles: list entries e_begin + grp + 2 t
  const int N = (n + 1) >> 1;         // group A's count (group B has N or N - 1)

  // ---- this lane's query; Q fragments pre-scaled by softmax_scale * log2(e) ----
  const int qi = qtile * kBM + wq * 32 + l31;
  const int qrow = qi < p.L ? qi : p.L - 1;
  bf16x8 qf[S::KS];
  {
    const unsigned char* src = qbase + qrow * q_row_bytes + 16 * h2;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)raw[e] * p.scale_log2);
    }
  }

  // ---- allowed key interval [lo, lo + width) of this query, prefix [0, pend) ----
  int lo = 0, hi = p.L;
  if (p.kind == kMaskChunk) {
    lo = (qi / p.chunk) * p.chunk;
    hi = min(p.L, lo + p.chunk);
  } else if (p.kind == kMaskWindow) {
    lo = max(0, qi - p.head_left[head]);
    hi = min(p.L, qi + p.right + 1);
  }
  if (p.causal || p.kind == kMaskBlock) hi = min(hi, qi + 1);
  hi = max(hi, lo);
  const unsigned width = static_cast<unsigned>(hi - lo);
  int pend = 0;
  if constexpr (PREFIX) {
    pend = min(p.prefix, p.L);
    if (p.causal) pend = min(pend, qi + 1);
  }
  const int wave_lo_max = __builtin_amdgcn_readlane(lo, 31);
  const int wave_hi_min = __builtin_amdgcn_readlane(hi, 0);
  auto unmasked = [&](int ent) __attribute__((always_inline)) {
    const int kv0 = (ent >> 1) * kBN;
    return (ent & 1) || (kv0 >= wave_lo_max && kv0 + kBN <= wave_hi_min);
  };

  // ---- running state of this group (log2 domain); only group A carries the sink ----
  float m_run = -INFINITY, l_run = 0.f, sink_l = 0.f;
  f32x16 acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};
  const float sink_log2 = (p.sink != nullptr && piece == 0 && grp == 0) ? p.sink[head] * kLog2e : -INFINITY;
  if (sink_log2 > -INFINITY) {
    m_run = sink_log2;
    sink_l = 1.f;
  }
  auto ref_of = [&]() __attribute__((always_inline)) { return m_run == -INFINITY ? 0.f : m_run; };

  // ---- LDS addressing (padded rows; see Lds<128>) ----
  const int kbase_off = (l31 & 15) * L::kKBlk + (l31 >> 4) * 256 + 16 * h2;
  const int tr_j = (lane & 15) >> 2, tr_c = lane & 3, dhalf = (lane >> 4) & 1;
  const int vbase_off = (4 * h2 + tr_j) * L::kVBlk + 32 * dhalf + 8 * tr_c;
  const int gbase = grp * kGroupBytes;
  auto kbuf = [&](int set) __attribute__((always_inline)) { return gbase + set * kSetBytes; };
  auto vbuf = [&](int set) __attribute__((always_inline)) { return gbase + set * kSetBytes + L::KT; };
  auto kfrag = [&](int set, int i) __attribute__((always_inline)) {  // QK step i: k-step i/2, key half i%2
    return *reinterpret_cast<const bf16x8*>(smem + kbuf(set) + kbase_off + 32 * (i >> 1) + (i & 1) * 512);
  };
  auto vfrag = [&](int set, int i) __attribute__((always_inline)) {  // PV step i: keys 16 (i/DT) .., O^T tile i%DT
    const unsigned char* src = smem + vbuf(set) + (i / S::DT) * 256 + vbase_off + 64 * (i % S::DT);
    const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src));
    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + 8 * L::kVBlk));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- LDS-DMA: waves 0-1 of a group copy K tiles, waves 2-3 V tiles ----
  const int dma_tensor = wq >> 1;
  const uint32_t dma_row_bytes =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(dma_tensor ? v_row_bytes : k_row_bytes)));
  const unsigned char* dma_base = dma_tensor ? vbase : kbase;
  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t goff_pad = static_cast<uint32_t>(16 * (lane >> 4)) * dma_row_bytes + 16 * (lane & 15);
  const uint32_t blk_bytes = dma_tensor ? L::kVBlk : L::kKBlk;
  // this wave's share of key tile kt into its tensor's buffer of set `set`
  auto issue_tile = [&](int kt, int set) __attribute__((always_inline)) {
    const uint32_t kv0 = static_cast<uint32_t>(kt * kBN);
    const uint64_t tb = uniform_u64(reinterpret_cast<uint64_t>(dma_base) + static_cast<uint64_t>(kv0) * dma_row_bytes);
    constexpr int kPer = 8;
    const int i0 = (wq & 1) * kPer;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        smem_lds + (dma_tensor ? vbuf(set) : kbuf(set)) + i0 * blk_bytes);
    if (static_cast<int>(kv0) + kBN <= seq_len) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        dma16(tb + static_cast<uint64_t>(i0 + i) * dma_row_bytes, goff_pad, dst + i * blk_bytes);
    } else {  // ragged last tile: clamp rows past the end of the sequence (their keys are masked)
      const int last = seq_len - 1 - static_cast<int>(kv0);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int row = i0 + i + 16 * (lane >> 4);
        dma16(tb, min(row, last) * dma_row_bytes + 16 * (lane & 15), dst + i * blk_bytes);
      }
    }
  };
  // list entry of this group's tile t (a uniform load; -1 past the group's end)
  auto entry = [&](int t) __attribute__((always_inline)) {
    return t < ng ? __builtin_amdgcn_readfirstlane(kv_list[e_begin + grp + 2 * t]) : -1;
  };
  // pair t = (K_t, V_{t-1}) into set t mod 2: K-waves copy K_t, V-waves V_{t-1}
  auto issue_pair = [&](int t, int ent_k, int ent_v) __attribute__((always_inline)) {
    if (dma_tensor == 0) {
      if (t < ng) issue_tile(ent_k >> 1, t & 1);
    } else {
      if (t >= 1 && t - 1 < ng) issue_tile(ent_v >> 1, t & 1);
    }
  };

  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16 sn[2];         // S^T of the group's newest tile (relative to the reference)
  bf16x8 pb[4];         // P^T of the previous tile (B operand of the PV MFMAs)
  bf16x8 ka[NQ + 2], va[NP + 2];

  // M phase: S^T_j (kQK) and O^T += V_{j-1}^T P^T_{j-1} (kPV), MFMAs alternating;
  // fragments 0 and 1 of each kind were read at the end of the previous V
  // phase, later ones are read two MFMAs of their kind ahead.
  float rsum = 0.f;
  auto m_phase = [&](int set, auto qk_tag, auto pv_tag) __attribute__((always_inline)) {
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPV = decltype(pv_tag)::value;
    // S^T starts from minus the reference (C operand of the first k-step), built
    // here so that no registers hold it between phases
    f32x16 seedv;
    if constexpr (kQK) {
      const float sd = -ref_of();
#pragma unroll
      for (int r = 0; r < 16; ++r) seedv[r] = sd;
    }
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if constexpr (kQK) {
        if (i + 2 < NQ) ka[i + 2] = kfrag(set, i + 2);
        sn[i & 1] = mfma32(ka[i], qf[i >> 1], i < 2 ? seedv : sn[i & 1]);
      }
      if constexpr (kPV) {
        if (i + 2 < NP) va[i + 2] = vfrag(set, i + 2);
        acc[i % S::DT] = mfma32(va[i], pb[i / S::DT], acc[i % S::DT]);
        // row sum of P_{j-1}: one pair per PV MFMA
        const int t = i / S::DT, e = 2 * (i % S::DT);
        rsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[t][e], pb[t][e + 1]}, ones2, rsum, false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPV) {
      l_run += rsum;
      rsum = 0.f;
    }
  };

  // V phase on S_j: mask (PARTIAL tiles), reference on the group's first tile, exponentials, row sums
  auto v_softmax = [&](int ent, auto mask_tag, auto first_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    constexpr bool kFirst = decltype(first_tag)::value;
    if constexpr (kMask) {
      const unsigned mbase = static_cast<unsigned>((ent >> 1) * kBN + 4 * h2 - lo);
      const int kbase_key = (ent >> 1) * kBN + 4 * h2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned u = mbase + 8 * (r >> 2) + (r & 3);
        if constexpr (PREFIX) {
          const int key = kbase_key + 8 * (r >> 2) + (r & 3);
          sn[0][r] = (u >= width && key >= pend) ? -INFINITY : sn[0][r];
          sn[1][r] = (u + 32 >= width && key + 32 >= pend) ? -INFINITY : sn[1][r];
        } else {
          sn[0][r] = (u >= width) ? -INFINITY : sn[0][r];
          sn[1][r] = (u + 32 >= width) ? -INFINITY : sn[1][r];
        }
      }
    }
    if constexpr (kFirst) {
      float x = fmaxf(sn[0][0], sn[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) x = max3(x, sn[0][r], sn[1][r]);
      const float mt = halves_max(x);  // tile max relative to the reference
      const bool need = (m_run == -INFINITY) ? (mt > -INFINITY) : (mt > kRescaleThreshold);
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float ref = ref_of();
        const float m_new = need ? ref + mt : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 while m_run = -inf
        const float shift = (m_new == -INFINITY ? 0.f : m_new) - ref;
        m_run = m_new;
        l_run *= alpha;
        sink_l *= alpha;
        sn[0] -= shift;
        sn[1] -= shift;
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = t >> 1, src = 8 * (t & 1) + 2 * i;
        pb[t][2 * i] = (__bf16)__builtin_amdgcn_exp2f(sn[h][src]);
        pb[t][2 * i + 1] = (__bf16)__builtin_amdgcn_exp2f(sn[h][src + 1]);
      }
    }
  };

  if (n > 0) {
    // prologue: pairs 0 and 1 of both groups, pair 0 waited for everywhere
    int ent_c = entry(0), ent_n1 = entry(1), ent_n2 = entry(2);
    issue_pair(0, ent_c, 0);
    wait_vmcnt<0>();
    issue_pair(1, ent_n1, ent_c);
    wg_barrier();
    if (ng > 0) {
      ka[0] = kfrag(0, 0);
      ka[1] = kfrag(0, 1);
    }
    if (grp == 1) wg_barrier();  // group B runs one phase behind group A
    using T1 = Bool<true>;
    using F0 = Bool<false>;
    // end of M_j: the next list entry, this wave's copies of pair j+1, the barrier
    auto end_m = [&](int j) __attribute__((always_inline)) {
      const int ent_n3 = entry(j + 3);  // uniform load, used two phases later
      wait_vmcnt<0>();
      wg_barrier();
      return ent_n3;
    };
    // V_j around the softmax: copies of pair j+2 (into the set M_j has finished with) first,
    // the first fragments of M_{j+1} last (pair j+1 is complete: waited before the barrier)
    auto v_begin = [&](int j) __attribute__((always_inline)) { issue_pair(j + 2, ent_n2, ent_n1); };
    auto v_end = [&](int j, int ent_n3) __attribute__((always_inline)) {
      const int set1 = (j + 1) & 1;
      if (j + 1 < ng) {
        ka[0] = kfrag(set1, 0);
        ka[1] = kfrag(set1, 1);
      }
      if (j + 1 <= ng) {
        va[0] = vfrag(set1, 0);
        va[1] = vfrag(set1, 1);
      }
      wg_barrier();
      ent_c = ent_n1;
      ent_n1 = ent_n2;
      ent_n2 = ent_n3;
    };
    int j = 0;
    if (ng > 0) {
      // j = 0: S^T of the first tile only; it sets the group's reference
      m_phase(0, T1{}, F0{});
      int e3 = end_m(0);
      v_begin(0);
      if (unmasked(ent_c)) v_softmax(ent_c, F0{}, T1{});
      else v_softmax(ent_c, T1{}, T1{});
      v_end(0, e3);
      // steady state: one straight body per FULL / PARTIAL tile
      for (j = 1; j < ng; ++j) {
        m_phase(j & 1, T1{}, T1{});
        e3 = end_m(j);
        v_begin(j);
        if (unmasked(ent_c)) v_softmax(ent_c, F0{}, F0{});
        else v_softmax(ent_c, T1{}, F0{});
        v_end(j, e3);
      }
      // j = ng: the value mix of the last tile only
      m_phase(ng & 1, F0{}, T1{});
      wait_vmcnt<0>();
      wg_barrier();
      wg_barrier();
      j = ng + 1;
    }
    for (; j <= N; ++j) {  // a group with one tile fewer keeps the barrier count
      wg_barrier();
      wg_barrier();
    }
    if (grp == 0) wg_barrier();  // matches group B's extra barrier
  }

  // ---- merge: group B's state through LDS into group A ----
  const float lrow = halves_sum(l_run);
  float* xb = reinterpret_cast<float*>(smem) + wq * kXFloats;
  auto row_has_key = [&](int first, int step) __attribute__((always_inline)) {
    bool has = false;
    const int hi_row = lo + static_cast<int>(width);
    for (int e = e_begin + first; e < e_end; e += step) {
      const int ent = p.kv[e];
      const int j0 = (ent >> 1) * kBN;
      has = has || (ent & 1) || (j0 < hi_row && j0 + kBN > lo) || j0 < pend;
    }
    return has;
  };
  // Whether this group's state is out of the fast pass's range for a row it lists keys of:
  // the wave then recomputes its rows exactly (see attn_fwd_kernel).
  bool redo_mine = false;
  if (n > 0) {
    const bool off_range = qi < p.L && (!(lrow <= 0x1p64f) || !(lrow + sink_l >= 0x1p-64f));
    if (__builtin_amdgcn_ballot_w64(off_range) != 0)
      redo_mine = off_range && (!(lrow <= 0x1p64f) || row_has_key(grp, 2));
  }
  if (n > 0) {
    wait_vmcnt<0>();
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const float4 a = make_float4(acc[dt][4 * gg], acc[dt][4 * gg + 1], acc[dt][4 * gg + 2], acc[dt][4 * gg + 3]);
          *reinterpret_cast<float4*>(xb + ((dt * 4 + gg) * 64 + lane) * 4) = a;
        }
      }
      xb[S::DT * 16 * 64 + lane] = m_run;
      xb[S::DT * 16 * 64 + 64 + lane] = lrow;
      xb[S::DT * 16 * 64 + 128 + lane] = redo_mine ? 1.f : 0.f;
    }
    wg_barrier();
    if (grp == 1) return;
  } else if (grp == 1) {
    return;
  }

  // group A: merge, then the epilogue of attn_fwd_kernel
  float m_b = -INFINITY, l_b = 0.f;
  bool redo = redo_mine;
  if (n > 0) {
    m_b = xb[S::DT * 16 * 64 + lane];
    l_b = xb[S::DT * 16 * 64 + 64 + lane];
    redo = redo || xb[S::DT * 16 * 64 + 128 + lane] != 0.f;
  }
  const float ra = ref_of(), ta = lrow + sink_l;
  const float rb = m_b == -INFINITY ? 0.f : m_b, tb = l_b;
  const float mstar = (ta > 0.f && tb > 0.f) ? fmaxf(ra, rb) : (ta > 0.f ? ra : (tb > 0.f ? rb : 0.f));
  const float wa = ta > 0.f ? __builtin_amdgcn_exp2f(ra - mstar) : 0.f;
  const float wb = tb > 0.f ? __builtin_amdgcn_exp2f(rb - mstar) : 0.f;
  const float ltot = wa * ta + wb * tb;
  if (n > 0) {
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float4 x = *reinterpret_cast<const float4*>(xb + ((dt * 4 + gg) * 64 + lane) * 4);
        acc[dt][4 * gg + 0] = __builtin_fmaf(wb, x.x, wa * acc[dt][4 * gg + 0]);
        acc[dt][4 * gg + 1] = __builtin_fmaf(wb, x.y, wa * acc[dt][4 * gg + 1]);
        acc[dt][4 * gg + 2] = __builtin_fmaf(wb, x.z, wa * acc[dt][4 * gg + 2]);
        acc[dt][4 * gg + 3] = __builtin_fmaf(wb, x.w, wa * acc[dt][4 * gg + 3]);
      }
    }
  }

  auto store_lse = [&](float m, float l) __attribute__((always_inline)) {
    if (p.lse != nullptr && h2 == 0 && qi < p.L)
      p.lse[(static_cast<int64_t>(b) * p.H + head) * p.L + qi] =
          l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  };
  if (__builtin_amdgcn_ballot_w64(redo) != 0) {
    // rare: this wave's 32 rows recomputed exactly in fp32 over the whole list
    constexpr int DH = D / 2;
    const unsigned char* qr = qbase + qrow * q_row_bytes + h2 * DH * 2;
    bf16x8 qv[DH / 8];
#pragma unroll
    for (int c = 0; c < DH / 8; ++c) qv[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
    float m = -INFINITY, l = 0.f, o[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] = 0.f;
    const float sink_a = (p.sink != nullptr && piece == 0) ? p.sink[head] * kLog2e : -INFINITY;
#pragma unroll 1
    for (int e = e_begin; e < e_end; ++e) {
      const int ent = p.kv[e];
      const int kv0 = (ent >> 1) * kBN;
#pragma unroll 1
      for (int kk = 0; kk < kBN; ++kk) {
        const int key = kv0 + kk;
        const bool allowed = key < p.L && ((ent & 1) || static_cast<unsigned>(key - lo) < width || key < pend);
        const int krow = key < p.L ? key : p.L - 1;
        const unsigned char* kr = kbase + static_cast<int64_t>(krow) * k_row_bytes + h2 * DH * 2;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < DH / 8; ++c) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(kr + 16 * c);
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) part = __builtin_fmaf((float)qv[c][e8], (float)x[e8], part);
        }
        const float sdot = halves_sum(part);
        const float sc2 = allowed ? sdot * p.scale_log2 : -INFINITY;
        const float m_new = fmaxf(m, sc2);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
        const float pr = allowed ? __builtin_amdgcn_exp2f(sc2 - m_new) : 0.f;
        l = l * alpha + pr;
        const unsigned char* vr = vbase + static_cast<int64_t>(krow) * v_row_bytes + h2 * DH * 2;
#pragma unroll
        for (int c = 0; c < DH / 8; ++c) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(vr + 16 * c);
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) o[8 * c + e8] = __builtin_fmaf(o[8 * c + e8], alpha, pr * (float)x[e8]);
        }
        m = m_new;
      }
    }
    if (sink_a > -INFINITY) {
      const float m_new = fmaxf(m, sink_a);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      l = l * alpha + __builtin_amdgcn_exp2f(sink_a - m_new);
#pragma unroll
      for (int d = 0; d < DH; ++d) o[d] *= alpha;
      m = m_new;
    }
    if (npieces > 1) {
      float* sp = p.partials + static_cast<int64_t>(slot0 + piece) * kSlotFloats;
#pragma unroll
      for (int dd = 0; dd < DH; ++dd) {
        const int d = h2 * DH + dd;
        const int idx = ((((wq * S::DT + (d >> 5)) * 4 + ((d >> 3) & 3)) * 64) + l31 + 32 * ((d >> 2) & 1)) * 4 + (d & 3);
        sp[idx] = o[dd];
      }
      sp[kSlotM + wq * 64 + lane] = l > 0.f ? m : -INFINITY;
      sp[kSlotL + wq * 64 + lane] = l;
      return;
    }
    store_lse(m, l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (qi < p.L) {
      unsigned char* dst = obase + qi * o_row_bytes + h2 * DH * 2;
#pragma unroll
      for (int c = 0; c < DH / 4; ++c) {
        bf16x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (__bf16)(o[4 * c + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + 8 * c) = out;
      }
    }
    return;
  }

  if (npieces == 1) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (qi < p.L) {
      unsigned char* dst = obase + qi * o_row_bytes;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int d = 32 * dt + 8 * gg + 4 * h2;
          bf16x4 out;
          out[0] = (__bf16)(acc[dt][4 * gg + 0] * inv);
          out[1] = (__bf16)(acc[dt][4 * gg + 1] * inv);
          out[2] = (__bf16)(acc[dt][4 * gg + 2] * inv);
          out[3] = (__bf16)(acc[dt][4 * gg + 3] * inv);
          *reinterpret_cast<bf16x4*>(dst + d * 2) = out;
        }
      }
    }
    store_lse(mstar, ltot);
    return;
  }
  float* sp = p.partials + static_cast<int64_t>(slot0 + piece) * kSlotFloats;
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const float4 a = make_float4(acc[dt][4 * gg], acc[dt][4 * gg + 1], acc[dt][4 * gg + 2], acc[dt][4 * gg + 3]);
      *reinterpret_cast<float4*>(sp + (((wq * S::DT + dt) * 4 + gg) * 64 + lane) * 4) = a;
    }
  }
  sp[kSlotM + wq * 64 + lane] = ltot > 0.f ? mstar : -INFINITY;
  sp[kSlotL + wq * 64 + lane] = ltot;
}

}  // namespace

hipError_t launch_fwd_pp(const GroupParams& g, dim3 grid, bool prefix, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop) {
  if (prefix) hipExtLaunchKernelGGL((attn_fwd_pp_kernel<true>), grid, dim3(512), 0, stream, start, stop, 0, g);
  else hipExtLaunchKernelGGL((attn_fwd_pp_kernel<false>), grid, dim3(512), 0, stream, start, stop, 0, g);
  return hipGetLastError();
}

}  // namespace bss
