// Structured-mask softmax attention forward for head dims 128 and 256 on
// gfx950, one wave group per work-group.  The computation is
// attn_fwd_kernel's (attn_fwd.hip): the exact tiled softmax over the item's
// listed key tiles, sink in the denominator, PARTIAL-tile masking, split rows.
//
// 4 waves x 32 query rows per work-group.  Each 64-key tile runs
// S^T = K Q^T (2 d / 16 MFMAs), the mask (PARTIAL tiles), the softmax and
// O^T += V^T P^T (d / 8 MFMAs, with the exponentials of the next 16 keys
// beside the MFMAs of the previous 16) in turn, while the copies of the next
// listed tile stream into the other LDS buffers.
//   * d = 128: two work-groups per CU, so that one work-group's first tiles
//     and epilogue overlap the other's MFMAs.  This is the kernel for items of
//     a few tiles (short windows, small chunks); long items run the ping-pong
//     kernel (attn_fwd_pp.hip).
//   * d = 256 (the grouped-query layer of the sliding-window-vs-linear-
//     attention article's speed test: 16 query heads on 4 key/value heads):
//     a wave's 32 rows hold 64 registers of Q fragments and 128 of fp32
//     accumulators, so one work-group per CU, registers beyond 256 in AGPRs.
// LDS tiles use the padded layout of Lds<D>: copy instruction i carries rows
// i, i + NI, ... (1024 / (2 d) rows of 2 d bytes) into 1 KiB plus a pad.

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

template <int D, bool PREFIX>
__global__ __launch_bounds__(kThreads, D == 128 ? 2 : 1) void attn_fwd_sg_kernel(const GroupParams g) {
  using S = Shape<D>;
  using L = Lds<D>;
  static_assert(L::PADDED && (D == 128 || D == 256), "padded tiles of head dim 128 or 256");
  constexpr int NI = L::NI;          // copy instructions per tile
  constexpr int RB = 2 * D;          // bytes of a row
  constexpr int CPR = D / 8;         // 16-byte chunks of a row
  constexpr int PAIRS = S::DT / 4;   // PV MFMAs per pair of exponentials of the next 16 keys
  constexpr int64_t kSlotFloats = partial_slot_floats(D);
  constexpr int kSlotM = 4 * S::DT * 16 * 64;
  constexpr int kSlotL = kSlotM + 4 * 64;
  static_assert(kSlotL + 4 * 64 == kSlotFloats, "partial slot layout");
  constexpr int NQ = 2 * S::KS;  // QK MFMAs per tile
  constexpr int NP = 4 * S::DT;  // PV MFMAs per tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::BYTES];

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

  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q + b * p.q_sb + head * p.q_sh);
  const int kv_head = head / p.kv_group;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k + b * p.k_sb + kv_head * p.k_sh);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v + b * p.v_sb + kv_head * p.v_sh);
  unsigned char* obase = reinterpret_cast<unsigned char*>(p.o + b * p.o_sb + head * p.o_sh);
  const int64_t q_row_bytes = p.q_sl * 2, k_row_bytes = p.k_sl * 2, v_row_bytes = p.v_sl * 2,
                o_row_bytes = p.o_sl * 2;
  const int n = e_end - e_begin;
  // kept in registers: read from the parameter block inside the loop, these
  // would be reloaded after every barrier and copy
  const int32_t* const kv_list = p.kv;
  const int seq_len = p.L;

  // ---- this lane's query; Q fragments pre-scaled by softmax_scale * log2(e) ----
  const int qi = qtile * kBM + wave * 32 + l31;
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

  // ---- running state (log2 domain) ----
  float m_run = -INFINITY, l_run = 0.f, sink_l = 0.f;
  f32x16 acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};
  const float sink_log2 = (p.sink != nullptr && piece == 0) ? p.sink[head] * kLog2e : -INFINITY;
  if (sink_log2 > -INFINITY) {
    m_run = sink_log2;
    sink_l = 1.f;
  }
  auto ref_of = [&]() __attribute__((always_inline)) { return m_run == -INFINITY ? 0.f : m_run; };

  // ---- LDS addressing (padded rows; Lds<D>): row r sits in block r mod NI at (r / NI) * RB ----
  // K fragment: key row l31 (+32 for the second key half: + 32 RB / NI bytes), chunk 2 ks + h2
  const int kbase_off = (l31 % NI) * L::kKBlk + (l31 / NI) * RB + 16 * h2;
  constexpr int kHalfOff = 32 / NI * RB;
  // V^T fragment: source lane (j, c) of each 16-lane group reads key row 16 t + 8 u + 4 h2 + j,
  // columns 32 dt + 16 dhalf + 4 c .. +3 (u = 0, 1: the two transposed reads)
  const int tr_j = (lane & 15) >> 2, tr_c = lane & 3, dhalf = (lane >> 4) & 1;
  const int vbase_off = (4 * h2 + tr_j) * L::kVBlk + 32 * dhalf + 8 * tr_c;
  auto kfrag = [&](int set, int i) __attribute__((always_inline)) {  // QK step i: k-step i/2, key half i%2
    return *reinterpret_cast<const bf16x8*>(smem + L::buf_off(set) + kbase_off + 32 * (i >> 1) + (i & 1) * kHalfOff);
  };
  auto vfrag = [&](int set, int i) __attribute__((always_inline)) {  // PV step i: keys 16 t .., O^T tile dt
    const int t = i / S::DT, dt = i % S::DT;
    const unsigned char* src = smem + L::buf_off(2 + set) + ((16 * t) % NI) * L::kVBlk + (16 * t / NI) * RB +
                               vbase_off + 64 * dt;
    const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src));
    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + 8 * L::kVBlk));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- LDS-DMA: waves 0-1 copy K tiles, waves 2-3 V tiles, NI / 2 instructions each ----
  const int dma_tensor = wave >> 1;
  const uint32_t dma_row_bytes =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(dma_tensor ? v_row_bytes : k_row_bytes)));
  const unsigned char* dma_base = dma_tensor ? vbase : kbase;
  const uint32_t smem_lds = lds_addr(smem);
  // lane l of instruction i copies chunk l mod CPR of row i + NI (l / CPR)
  const uint32_t goff = static_cast<uint32_t>(NI * (lane / CPR)) * dma_row_bytes + 16 * (lane % CPR);
  const uint32_t blk_bytes = dma_tensor ? L::kVBlk : L::kKBlk;
  auto issue_tile = [&](int kt, int set) __attribute__((always_inline)) {
    const uint32_t kv0 = static_cast<uint32_t>(kt * kBN);
    const uint64_t tb = uniform_u64(reinterpret_cast<uint64_t>(dma_base) + static_cast<uint64_t>(kv0) * dma_row_bytes);
    constexpr int kPer = NI / 2;
    const int i0 = (wave & 1) * kPer;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(smem_lds + L::buf_off(2 * dma_tensor + set) + i0 * blk_bytes);
    if (static_cast<int>(kv0) + kBN <= seq_len) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        dma16(tb + static_cast<uint64_t>(i0 + i) * dma_row_bytes, goff, dst + i * blk_bytes);
    } else {  // ragged last tile: clamp rows past the end of the sequence (their keys are masked)
      const int last = seq_len - 1 - static_cast<int>(kv0);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int row = i0 + i + NI * (lane / CPR);
        dma16(tb, min(row, last) * dma_row_bytes + 16 * (lane % CPR), dst + i * blk_bytes);
      }
    }
  };

  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  // one tile: QK, mask (PARTIAL), reference (first tile), softmax, PV
  auto tile = [&](int j, int ent, int ent_next, auto mask_tag, auto first_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    constexpr bool kFirst = decltype(first_tag)::value;
    const int set = j & 1;
    wait_vmcnt<0>();   // this wave's share of tile j
    wg_barrier();      // ... and everyone else's; the buffers of tile j-1 are free
    bf16x8 ka[NQ], va[NP];
    ka[0] = kfrag(set, 0);
    ka[1] = kfrag(set, 1);
    if (j + 1 < n) issue_tile(ent_next >> 1, set ^ 1);
    f32x16 seedv;
    {
      const float sd = -ref_of();
#pragma unroll
      for (int r = 0; r < 16; ++r) seedv[r] = sd;
    }
    f32x16 sn[2];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i + 2 < NQ) ka[i + 2] = kfrag(set, i + 2);
      if (i == NQ - 2) va[0] = vfrag(set, 0);
      if (i == NQ - 1) va[1] = vfrag(set, 1);
      sn[i & 1] = mfma32(ka[i], qf[i >> 1], i < 2 ? seedv : sn[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
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
    // P^T = exp2(S^T) in bf16, 16 keys (one B operand pb[t]) at a time: the
    // exponentials of keys 16(t+1) .. +15 run beside the PV MFMAs of keys 16t .. +15
    bf16x8 pb[4];
    float rs = 0.f;
    auto exp_pair = [&](int t, int i) __attribute__((always_inline)) {  // pair i (0..3) of pb[t]
      const int h = t >> 1, src = 8 * (t & 1) + 2 * i;
      pb[t][2 * i] = (__bf16)__builtin_amdgcn_exp2f(sn[h][src]);
      pb[t][2 * i + 1] = (__bf16)__builtin_amdgcn_exp2f(sn[h][src + 1]);
      rs = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[t][2 * i], pb[t][2 * i + 1]}, ones2, rs, false);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) exp_pair(0, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = i / S::DT, dt = i % S::DT;
      if (i + 2 < NP) va[i + 2] = vfrag(set, i + 2);
      acc[dt] = mfma32(va[i], pb[t], acc[dt]);
      if (t + 1 < 4 && (dt + 1) % PAIRS == 0) exp_pair(t + 1, dt / PAIRS);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += rs;
  };

  if (n > 0) {
    int ent = __builtin_amdgcn_readfirstlane(kv_list[e_begin]);
    int ent1 = n > 1 ? __builtin_amdgcn_readfirstlane(kv_list[e_begin + 1]) : 0;
    // entry j + 2 is loaded at the top of iteration j and read into a scalar
    // register at the top of iteration j + 1, after the tile's wait for its
    // copies has also covered it (a load used at once would cost a round trip
    // per tile)
    int raw2 = n > 2 ? kv_list[e_begin + 2] : 0;
    issue_tile(ent >> 1, 0);
    if (unmasked(ent)) tile(0, ent, ent1, Bool<false>{}, Bool<true>{});
    else tile(0, ent, ent1, Bool<true>{}, Bool<true>{});
    for (int j = 1; j < n; ++j) {
      ent = ent1;
      ent1 = j + 1 < n ? __builtin_amdgcn_readfirstlane(raw2) : 0;
      raw2 = j + 2 < n ? kv_list[e_begin + j + 2] : 0;
      if (unmasked(ent)) tile(j, ent, ent1, Bool<false>{}, Bool<false>{});
      else tile(j, ent, ent1, Bool<true>{}, Bool<false>{});
    }
  }

  auto store_lse = [&](float m, float l) __attribute__((always_inline)) {
    if (p.lse != nullptr && h2 == 0 && qi < p.L)
      p.lse[(static_cast<int64_t>(b) * p.H + head) * p.L + qi] =
          l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  };
  const float lrow = halves_sum(l_run);
  // Out of the fast pass's range for a row the item lists keys of (see
  // attn_fwd_kernel): the wave recomputes its 32 rows exactly in fp32.
  bool redo = false;
  if (n > 0) {
    const bool off_range = qi < p.L && (!(lrow <= 0x1p64f) || !(lrow + sink_l >= 0x1p-64f));
    if (__builtin_amdgcn_ballot_w64(off_range) != 0) {
      bool has = false;
      const int hi_row = lo + static_cast<int>(width);
      for (int e = e_begin; e < e_end; ++e) {
        const int en = p.kv[e];
        const int j0 = (en >> 1) * kBN;
        has = has || (en & 1) || (j0 < hi_row && j0 + kBN > lo) || j0 < pend;
      }
      redo = off_range && (!(lrow <= 0x1p64f) || has);
    }
  }
  if (__builtin_amdgcn_ballot_w64(redo) != 0) {
    // Lanes l and l + 32 share a query: each takes half of the head dimension.
    constexpr int DH = D / 2;
    const unsigned char* qr = qbase + qrow * q_row_bytes + h2 * DH * 2;
    bf16x8 qv[DH / 8];
#pragma unroll
    for (int c = 0; c < DH / 8; ++c) qv[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
    float m = -INFINITY, l = 0.f, o[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] = 0.f;
#pragma unroll 1
    for (int e = e_begin; e < e_end; ++e) {
      const int en = p.kv[e];
      const int kv0 = (en >> 1) * kBN;
#pragma unroll 1
      for (int kk = 0; kk < kBN; ++kk) {
        const int key = kv0 + kk;
        const bool allowed = key < p.L && ((en & 1) || static_cast<unsigned>(key - lo) < width || key < pend);
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
    if (sink_log2 > -INFINITY) {
      const float m_new = fmaxf(m, sink_log2);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      l = l * alpha + __builtin_amdgcn_exp2f(sink_log2 - m_new);
#pragma unroll
      for (int d = 0; d < DH; ++d) o[d] *= alpha;
      m = m_new;
    }
    if (npieces > 1) {
      float* sp = p.partials + static_cast<int64_t>(slot0 + piece) * kSlotFloats;
#pragma unroll
      for (int dd = 0; dd < DH; ++dd) {
        const int d = h2 * DH + dd;
        const int idx = ((((wave * S::DT + (d >> 5)) * 4 + ((d >> 3) & 3)) * 64) + l31 + 32 * ((d >> 2) & 1)) * 4 + (d & 3);
        sp[idx] = o[dd];
      }
      sp[kSlotM + wave * 64 + lane] = l > 0.f ? m : -INFINITY;
      sp[kSlotL + wave * 64 + lane] = l;
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

  const float ltot = lrow + sink_l;
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
    store_lse(ref_of(), ltot);
    return;
  }
  float* sp = p.partials + static_cast<int64_t>(slot0 + piece) * kSlotFloats;
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const float4 a = make_float4(acc[dt][4 * gg], acc[dt][4 * gg + 1], acc[dt][4 * gg + 2], acc[dt][4 * gg + 3]);
      *reinterpret_cast<float4*>(sp + (((wave * S::DT + dt) * 4 + gg) * 64 + lane) * 4) = a;
    }
  }
  sp[kSlotM + wave * 64 + lane] = ltot > 0.f ? ref_of() : -INFINITY;
  sp[kSlotL + wave * 64 + lane] = ltot;
}

}  // namespace

hipError_t launch_fwd_sg(const GroupParams& g, int D, dim3 grid, bool prefix, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop) {
  if (D == 128) {
    if (prefix) hipExtLaunchKernelGGL((attn_fwd_sg_kernel<128, true>), grid, dim3(kThreads), 0, stream, start, stop, 0, g);
    else hipExtLaunchKernelGGL((attn_fwd_sg_kernel<128, false>), grid, dim3(kThreads), 0, stream, start, stop, 0, g);
  } else if (D == 256) {
    if (prefix) hipExtLaunchKernelGGL((attn_fwd_sg_kernel<256, true>), grid, dim3(kThreads), 0, stream, start, stop, 0, g);
    else hipExtLaunchKernelGGL((attn_fwd_sg_kernel<256, false>), grid, dim3(kThreads), 0, stream, start, stop, 0, g);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bss
