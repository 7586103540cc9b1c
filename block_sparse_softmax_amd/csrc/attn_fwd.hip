// Structured-mask softmax attention forward for gfx950 (MI355X).
//
// What one work-group computes: one work item = (batch b, head h, query tile
// of kBM = 128 rows).  It walks the item's list of KV tiles (kBN = 64 keys
// each; only tiles holding an allowed pair are listed) and keeps a running
// row max m, row sum l and un-normalised output acc, the exact tiled
// softmax of "Vision transformers and hybrid architectures" (section on
// efficient attention: exact softmax, tiled, never materialising the n x n
// score matrix).  The sink logit of "Semantic Head Specialization ..." (the
// sink-bias slide, "Eq. 1") enters the running state as one extra
// denominator term with no value.
//
// This file: attn_fwd_kernel (d = 64 and 80), the merge of split rows and the
// launch for every head dim; d = 128 runs attn_fwd_pp_kernel (attn_fwd_pp.hip:
// two wave groups in ping-pong) for long rows and attn_fwd_sg_kernel
// (attn_fwd_sg.hip: one wave group, two work-groups per CU) for short ones,
// d = 256 attn_fwd_sg_kernel.
//
// Layout of the work in attn_fwd_kernel (per work-group: 4 waves x 32 query rows):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  K (A operand) comes from LDS,
//     Q (B operand) stays in registers for the whole item.  In the S^T output
//     layout lane l owns query (l mod 32) and 16 of every 32 keys; the other
//     16 keys of that query sit in lane l^32, so the row max needs a single
//     cross-half exchange (v_permlane32_swap).
//   * The probabilities P^T are already in the B-operand layout of the next
//     MFMA, O^T += V^T P^T: converted to bf16 in place, no shuffles.  V is
//     kept row-major in LDS and read transposed with ds_read_b64_tr_b16.
//   * d = 80 is padded to 96 rows of O^T for the PV product only; the first
//     pad row of V^T is a row of ones, so the MFMA also produces the row sum
//     of the bf16 probabilities at no extra VALU cost.
//   * K and V tiles go global -> LDS with global_load_lds_dwordx4 (no VGPR
//     staging), double-buffered: the next listed tile streams in while the
//     current one is multiplied.  LDS rows are XOR-swizzled by 16-byte chunk
//     (d = 64, 80; the d = 128 kernel pads them instead) so that fragment
//     reads are conflict-free.
//   * Masking code runs only on tiles flagged PARTIAL: every allowed key set
//     of the interval masks is one interval [lo, hi) per query, and a block
//     matrix whose block size is a multiple of the tile sizes adds only j <= i.
//   * Lazy rescaling: the running max moves only when a score exceeds it by
//     more than 2^8; probabilities stay below 256 and the result is the same
//     softmax (every term shares the reference point).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "fwd_common.hpp"
#include "kernels.hpp"
#include "tile_common.hpp"

namespace bss {
namespace {

using namespace dev;

constexpr int kListCap = 1024;  // KV-list entries staged in LDS at a time

// PREFIX: the launch may add prefix tokens to the rows' sets (a second
// allowed interval [0, pend) checked on PARTIAL tiles); without it the mask
// is the single interval [lo, hi).
template <int D, bool PREFIX>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const GroupParams g) {
  using S = Shape<D>;
  static_assert(S::PIPELINED, "d = 128 runs attn_fwd_pp_kernel");
  constexpr int64_t kSlotFloats = partial_slot_floats(D);
  constexpr int kSlotM = 4 * S::DT * 16 * 64;  // m of every lane of the 4 waves
  constexpr int kSlotL = kSlotM + 4 * 64;       // l of every lane
  static_assert(kSlotL + 4 * 64 == kSlotFloats, "partial slot layout");
  using L = Lds<D>;
  // LDS: K tiles in buffers 0-1, V tiles in buffers 2-3.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::BYTES];
  __shared__ int list_lds[kListCap];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5;    // half of the wave
  const int l31 = lane & 31;

  // Work-groups are dealt to the 8 XCDs round-robin (block i runs on XCD i mod 8);
  // XCD x takes the x-th contiguous chunk of the schedule, so the items that
  // share an XCD's L2 at any time come from the same head.
  // XCD x (blockIdx mod 8) runs queue x of job 0, then of job 1, ...
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
  // A piece of a split row: its list range is a part of the row's list; the
  // sink enters piece 0 only.
  const int slot0 = __builtin_amdgcn_readfirstlane(split.x);
  const int piece = __builtin_amdgcn_readfirstlane(split.y);
  const int npieces = __builtin_amdgcn_readfirstlane(split.z);
  const int b = blockIdx.y;

  const unsigned char* qbase =
      reinterpret_cast<const unsigned char*>(p.q + b * p.q_sb + head * p.q_sh);
  // grouped-query attention: runs of kv_group consecutive query heads share one K/V head
  const int kv_head = head / p.kv_group;
  const unsigned char* kbase =
      reinterpret_cast<const unsigned char*>(p.k + b * p.k_sb + kv_head * p.k_sh);
  const unsigned char* vbase =
      reinterpret_cast<const unsigned char*>(p.v + b * p.v_sb + kv_head * p.v_sh);
  unsigned char* obase = reinterpret_cast<unsigned char*>(p.o + b * p.o_sb + head * p.o_sh);
  const int64_t q_row_bytes = p.q_sl * 2, k_row_bytes = p.k_sl * 2, v_row_bytes = p.v_sl * 2,
                o_row_bytes = p.o_sl * 2;

  // ---- the KV list of this item, staged in LDS kListCap entries at a time ----
  const int n = e_end - e_begin;
  auto stage_list = [&](int first) __attribute__((always_inline)) {
    const int cnt = min(kListCap, n - first);
    for (int i = threadIdx.x; i < cnt; i += kThreads) list_lds[i] = p.kv[e_begin + first + i];
  };
  if (n > 0) stage_list(0);

  // ---- this lane's query; Q fragments (B operand of S^T = K Q^T), pre-scaled ----
  // by softmax_scale * log2(e) so that the MFMA yields log2-domain logits.
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

  // ---- allowed key interval [lo, lo + width) of this query (PARTIAL tiles) ----
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
  // prefix tokens: keys [0, pend) are allowed as well
  int pend = 0;
  if constexpr (PREFIX) {
    pend = min(p.prefix, p.L);
    if (p.causal) pend = min(pend, qi + 1);
  }
  // A tile flagged PARTIAL for the 128 rows of the item can still allow every
  // pair for this wave's 32 rows: the intervals' ends never decrease with the
  // row, so the wave's rows all allow keys [lo of its last row, hi of its
  // first row).  Such tiles take the unmasked path.
  const int wave_lo_max = __builtin_amdgcn_readlane(lo, 31);
  const int wave_hi_min = __builtin_amdgcn_readlane(hi, 0);
  auto unmasked = [&](int ent) __attribute__((always_inline)) {
    const int kv0 = (ent >> 1) * kBN;
    return (ent & 1) || (kv0 >= wave_lo_max && kv0 + kBN <= wave_hi_min);
  };

  // ---- running softmax state (log2 domain) ----
  // m_run: reference max (-inf while no allowed key and no sink has been seen);
  // l_run: sum of this lane's probabilities (d != 80: d = 80 reads the row sum
  // off O^T row 80); sink_l: the sink's term exp2(s_aux log2e - m_run).
  float m_run, l_run, sink_l;
  f32x16 acc[S::DT];
  const float sink_log2 = (p.sink != nullptr && piece == 0) ? p.sink[head] * kLog2e : -INFINITY;
  auto init_state = [&]() __attribute__((always_inline)) {
    m_run = -INFINITY;
    l_run = 0.f;
    sink_l = 0.f;
    if (sink_log2 > -INFINITY) {
      m_run = sink_log2;
      sink_l = 1.f;
    }
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};
  };
  init_state();

  // ---- LDS addressing ----
  // K fragment for k-step ks: row l31 (and l31 + 32: same swizzle), logical chunk 2*ks + h2.
  // d = 128 (padded rows) needs one base per table and immediate offsets.
  int koff[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) koff[ks] = l31 * S::LRB + phys_chunk<D>(l31, 2 * ks + h2) * 16;
  int kbase_off = koff[0];
  // V^T fragment for O^T tile dt and half u of a 16-key k-step: transposed
  // read; source lane (j, c) of each 16-lane group points at row
  // 8*u + 4*h2 + j (+16 per k-step), columns 32*dt + 16*dhalf + 4*c .. +3.
  const int tr_j = (lane & 15) >> 2, tr_c = lane & 3, dhalf = (lane >> 4) & 1;
  int voff[S::DT][2];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 8 * u + 4 * h2 + tr_j;
      const int c = 4 * dt + 2 * dhalf + (tr_c >> 1);
      voff[dt][u] = row * S::LRB + phys_chunk<D>(row, c) * 16 + (tr_c & 1) * 8;
    }
  }
  int vbase_off = voff[0][0];
  if constexpr (S::PAD_ROWSUM) {
    // Constant pad chunks 10-11 of every V row in both V buffers: element 80 = 1, the rest 0.
    for (int i = threadIdx.x; i < 2 * kBN * 4; i += kThreads) {  // 2 buffers x 64 rows x 4 x 8 bytes
      const int buf = i / (kBN * 4), row = (i / 4) % kBN, q4 = i % 4;
      const int c = 10 + (q4 >> 1);
      uint2 v = make_uint2(0u, 0u);
      if (q4 == 0) v.x = 0x3F80u;  // bf16 1.0 in element 80
      *reinterpret_cast<uint2*>(smem + L::buf_off(2 + buf) + row * S::LRB +
                                phys_chunk<D>(row, c) * 16 + (q4 & 1) * 8) = v;
    }
  }

  // LDS-DMA: waves 0-1 fill K tiles and waves 2-3 V tiles; wave-instruction i
  // of a wave fills 64 consecutive 16-byte LDS slots of its half of the tile.
  const int dma_tensor = wave >> 1;
  const uint32_t dma_row_bytes =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(dma_tensor ? v_row_bytes : k_row_bytes)));
  const unsigned char* dma_base = dma_tensor ? vbase : kbase;
  // Lane part of each load's source offset for one swizzle period (16 rows);
  // later periods add 16 rows to the uniform base.  d = 80: lanes whose slot
  // is a pad chunk read chunk 0 of their row instead; for V they are left out
  // of the copy (the pad holds the constant ones row), for K the copy is
  // harmless (K pad chunks are never read).
  uint32_t goff[S::DMA_PERIOD];
  uint64_t gskip[S::DMA_PERIOD];
#pragma unroll
  for (int i = 0; i < S::DMA_PERIOD; ++i) {
    const int slot = ((wave & 1) * S::LOADS + i) * 64 + lane;
    const int row = slot / S::LCPR;
    const int c = phys_chunk<D>(row, slot % S::LCPR);
    const bool pad = c >= S::CPR;
    goff[i] = row * dma_row_bytes + (pad ? 0 : c) * 16;
    gskip[i] = (S::PAD_ROWSUM && dma_tensor == 1) ? __builtin_amdgcn_ballot_w64(pad) : 0;
  }
  const uint32_t smem_lds = lds_addr(smem);
  // Issue this wave's share of tile kt into LDS buffer buf (0-1 K, 2-3 V).
  auto issue_tile = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t kv0 = static_cast<uint32_t>(kt * kBN);
    const uint64_t tb = uniform_u64(reinterpret_cast<uint64_t>(dma_base) + static_cast<uint64_t>(kv0) * dma_row_bytes);
    const uint32_t dst =
        __builtin_amdgcn_readfirstlane(smem_lds + L::buf_off(buf) + (wave & 1) * S::LOADS * 1024);
    if (static_cast<int>(kv0) + kBN <= p.L) {
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const uint64_t b = tb + static_cast<uint64_t>((i / S::DMA_PERIOD) * 16) * dma_row_bytes;
        if constexpr (S::PAD_ROWSUM) dma16_skip(b, goff[i % S::DMA_PERIOD], dst + i * 1024, gskip[i % S::DMA_PERIOD]);
        else dma16(b, goff[i % S::DMA_PERIOD], dst + i * 1024);
      }
    } else {  // ragged last tile: clamp rows past the end of the sequence (their keys are masked)
      const int last = p.L - 1 - static_cast<int>(kv0);
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const int slot = ((wave & 1) * S::LOADS + i) * 64 + lane;
        const int row = slot / S::LCPR;
        const int c = phys_chunk<D>(row, slot % S::LCPR);
        const uint32_t off = min(row, last) * dma_row_bytes + (c < S::CPR ? c : 0) * 16;
        if constexpr (S::PAD_ROWSUM) dma16_skip(tb, off, dst + i * 1024, gskip[i % S::DMA_PERIOD]);
        else dma16(tb, off, dst + i * 1024);
      }
    }
  };

  // ---- LDS fragment reads ----
  // d = 128: XOR of a per-use constant into one base; d = 80: its swizzle
  // only touches the two low chunk bits, so addresses are one of two bases
  // plus an immediate (32 bytes per k-step, 64 bytes per O^T tile).
  auto k_addr = [&](int ks) __attribute__((always_inline)) {
    if constexpr (D == 80) return koff[ks & 1] + 32 * (ks & ~1);
    else return koff[ks];
  };
  auto v_addr = [&](int dt, int u) __attribute__((always_inline)) {
    if constexpr (D == 80) return voff[0][u] + 64 * dt;
    else return voff[dt][u];
  };
  // K fragment (A operand of S^T = K Q^T) for k-step ks, keys 32*half .. +31.
  auto kfrag = [&](int kbuf, int ks, int half) __attribute__((always_inline)) {
    constexpr int kHalf = 32 * S::LRB;  // keys 32 .. 63
    return *reinterpret_cast<const bf16x8*>(smem + L::buf_off(kbuf) + k_addr(ks) + half * kHalf);
  };
  // V^T fragment for PV step p = t * DT + dt (keys 16t .. 16t+15, O^T tile dt).
  auto vfrag = [&](int vbuf, int p) __attribute__((always_inline)) {
    const int t = p / S::DT, dt = p % S::DT;
    const unsigned char* src = smem + L::buf_off(vbuf) + t * (16 * S::LRB);
    const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + v_addr(dt, 0)));
    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + v_addr(dt, 1)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Seed of a tile's S^T accumulators (C operand of its first k-step): minus
  // the reference, so the MFMA output is already relative to it.
  f32x16 seedv;
  auto ref_of = [&]() __attribute__((always_inline)) { return m_run == -INFINITY ? 0.f : m_run; };
  auto set_seed = [&]() __attribute__((always_inline)) {
    if constexpr (S::SEEDED) {
      const float sd = -ref_of();
#pragma unroll
      for (int r = 0; r < 16; ++r) seedv[r] = sd;
    }
  };
  set_seed();

  // ---- main loop: software pipeline over the listed tiles, scheduled by hand ----
  // Iteration j (0 <= j <= n):
  //   part 1: S^T of tile j (2 KS MFMAs), each MFMA followed by a share of
  //           the exponentials of tile j-1, keys 0-31;
  //   part 2: O^T += V^T P^T of tile j-1 (4 DT MFMAs); the first half of them
  //           carry the exponentials of keys 32-63, the second half the mask
  //           (PARTIAL tiles) and row max of tile j.
  // An MFMA hides about four full-rate VALU instructions (VALU work issued
  // while an MFMA runs proceeds at half rate), which sets the shares.  LDS
  // fragments are read two MFMAs ahead; scheduling fences keep this order.
  // A rare branch at the end moves the reference when tile j's max exceeds
  // it by more than 2^kRescaleThreshold (scaling acc, which then holds tile
  // j-1, the row sum, the sink term and tile j's scores).
  // K of tile t sits in buffer t&1 (DMA issued at the top of iteration t-1),
  // V of tile t in buffer 2 + (t&1) (DMA issued at the top of iteration t);
  // the barrier at the top of iteration j guarantees that the buffers of K
  // tile j-1 and V tile j-2 are no longer read.
  // Scores of the newest tile relative to the reference: two register
  // blocks that trade roles every iteration (the loop is unrolled by two),
  // so the hand-over needs no copies and buffer offsets are immediates.
  f32x16 sA[2], sB[2];
  int list_base = 0;
  // List entries (kv_tile << 1 | full) of tiles j and j+1.  Entry j+2 is read
  // from LDS during iteration j and moved to a scalar register only at its
  // end, so the DMA address of the next tile never waits on an LDS read.
  int ent_cur = 0, ent_nxt = 0;
  // Read list entry i (i < n) from the staged list; crossing into the next
  // staged chunk restages it (every wave is past the barrier of this
  // iteration, so no entry of the old chunk is still to be read).
  auto list_entry = [&](int i) __attribute__((always_inline)) {
    if (i - list_base == kListCap) {
      list_base += kListCap;
      stage_list(list_base);
      __syncthreads();
    }
    return list_lds[i - list_base];
  };
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  // sc: scores of tile j-1 (read); sn: scores of tile j (written).
  auto iteration = [&](int j, auto cur_tag, auto prev_tag, auto mask_tag, auto par_tag, auto safe_tag,
                       f32x16 (&sc)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
    constexpr bool kCur = decltype(cur_tag)::value;    // tile j exists
    constexpr bool kPrev = decltype(prev_tag)::value;  // tile j-1 exists
    constexpr bool kMask = decltype(mask_tag)::value;  // tile j is PARTIAL
    constexpr int kPar = decltype(par_tag)::value;     // j & 1
    // Row max and reference update: on the first tile always; on later tiles
    // only in the safe pass (the fast pass keeps the first tile's reference).
    constexpr bool kMax = decltype(safe_tag)::value || !kPrev;
    constexpr int NQ = 2 * S::KS;  // QK MFMAs
    constexpr int NP = 4 * S::DT;  // PV MFMAs
    wait_vmcnt<0>();   // this wave's share of K tile j / V tile j-1
    wg_barrier();      // ... and everyone else's
    constexpr int kb = kPar, vb = 2 + (kPar ^ 1);
    // the first K fragments of tile j go out before the DMA instructions
    // (whose memory clobber would otherwise hold them back)
    bf16x8 ka[NQ + 2];
    if constexpr (kCur) {
      ka[0] = kfrag(kb, 0, 0);
      ka[1] = kfrag(kb, 0, 1);
    }
    const int ent = ent_cur, ent1 = ent_nxt;
    if (j + 1 < n) {
      if (dma_tensor == 0) issue_tile(ent1 >> 1, kPar ^ 1);
    }
    if constexpr (kCur) {
      if (dma_tensor == 1) issue_tile(ent >> 1, 2 + kPar);
    }
    const int raw2 = (j + 2 < n) ? list_entry(j + 2) : 0;

    // exponentials of tile j-1: pair i (0..7) of key block h -> P^T elements
    bf16x8 pb[4];
    float rs = 0.f;
    // (unseeded scores are raw logits: the reference comes off here)
    const float eref = S::SEEDED ? 0.f : ref_of();
    auto exp_pair = [&](int h, int i) __attribute__((always_inline)) {
      const int t = 2 * h + i / 4, e = 2 * (i % 4);
      pb[t][e] = (__bf16)__builtin_amdgcn_exp2f(sc[h][2 * i] - eref);
      pb[t][e + 1] = (__bf16)__builtin_amdgcn_exp2f(sc[h][2 * i + 1] - eref);
      if constexpr (!S::PAD_ROWSUM)
        rs = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[t][e], pb[t][e + 1]}, ones2, rs, false);
    };
    // mask (PARTIAL) and row max of tile j: step r (0..15)
    float x = 0.f;
    const unsigned mbase = static_cast<unsigned>((ent >> 1) * kBN + 4 * h2 - lo);
    const int kbase_key = (ent >> 1) * kBN + 4 * h2;
    auto mask_step = [&](int r) __attribute__((always_inline)) {
      const unsigned u = mbase + 8 * (r >> 2) + (r & 3);
      if constexpr (PREFIX) {
        const int key = kbase_key + 8 * (r >> 2) + (r & 3);
        sn[0][r] = (u >= width && key >= pend) ? -INFINITY : sn[0][r];
        sn[1][r] = (u + 32 >= width && key + 32 >= pend) ? -INFINITY : sn[1][r];
      } else {
        sn[0][r] = (u >= width) ? -INFINITY : sn[0][r];
        sn[1][r] = (u + 32 >= width) ? -INFINITY : sn[1][r];
      }
    };
    auto max_step = [&](int r) __attribute__((always_inline)) {
      x = (r == 0) ? fmaxf(sn[0][0], sn[1][0]) : max3(x, sn[0][r], sn[1][r]);
    };
    // QK MFMA number q: k-step and key half
    auto q_ks = [](int q) __attribute__((always_inline)) { return q / 2; };
    auto q_half = [](int q) __attribute__((always_inline)) { return q % 2; };

    // ---- part 1 ----
    bf16x8 va[NP + 2];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int ks = q_ks(q), half = q_half(q);
      if constexpr (kCur) {
        if (q + 2 < NQ) ka[q + 2] = kfrag(kb, q_ks(q + 2), q_half(q + 2));
        sn[half] = mfma32(ka[q], qf[ks], ks == 0 ? (S::SEEDED ? seedv : f32x16{}) : sn[half]);
      }
      if constexpr (kPrev) {
        if (q == NQ - 2) va[0] = vfrag(vb, 0);
        if (q == NQ - 1) va[1] = vfrag(vb, 1);
#pragma unroll
        for (int i = q * 8 / NQ; i < (q + 1) * 8 / NQ; ++i) exp_pair(0, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- part 2 ----
    // Raised wave priority while the PV MFMAs issue: when both waves of a
    // SIMD are ready, the one feeding the matrix core goes first, and the
    // other wave's VALU work fills the MFMA shadow (measured: +4 % on the
    // 16K-token full launch, +6 % at 4K).
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NB = (kMask ? 16 : 0) + (kMax ? 16 : 0);  // mask + max steps
#pragma unroll
    for (int pidx = 0; pidx < NP; ++pidx) {
      if constexpr (kPrev) {
        if (pidx + 2 < NP) va[pidx + 2] = vfrag(vb, pidx + 2);
        const int t = pidx / S::DT, dt = pidx % S::DT;
        acc[dt] = mfma32(va[pidx], pb[t], acc[dt]);
        if (pidx < 2 * S::DT) {
          constexpr int H = 2 * S::DT;
#pragma unroll
          for (int i = pidx * 8 / H; i < (pidx + 1) * 8 / H; ++i) exp_pair(1, i);
        }
      }
      if constexpr (kCur) {
        constexpr int H = 2 * S::DT;
        if (!kPrev || pidx >= H) {
          const int slot = !kPrev ? pidx : pidx - H;
          const int nslots = !kPrev ? NP : H;
#pragma unroll
          for (int i = slot * NB / nslots; i < (slot + 1) * NB / nslots; ++i) {
            if (kMask && i < 16) mask_step(i);
            else if constexpr (kMax) max_step(kMask ? i - 16 : i);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!S::PAD_ROWSUM && kPrev) l_run += rs;

    if constexpr (kCur && kMax) {
      // ---- rare: move the reference ----
      const float ref = ref_of();
      const float mx = halves_max(x);  // tile max (SEEDED: relative to the reference)
      const float mt = S::SEEDED ? mx : mx - ref;
      const bool need = (m_run == -INFINITY) ? (mt > -INFINITY) : (mt > kRescaleThreshold);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
        const float m_new = need ? ref + mt : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 while m_run = -inf
        const float shift = (m_new == -INFINITY ? 0.f : m_new) - ref;
        m_run = m_new;
        l_run *= alpha;
        sink_l *= alpha;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) acc[dt] *= alpha;
        if constexpr (S::SEEDED) {
          sn[0] -= shift;
          sn[1] -= shift;
        }
        set_seed();
      }
    }
    ent_cur = ent1;
    ent_nxt = __builtin_amdgcn_readfirstlane(raw2);
  };
  // steady-state iteration: the FULL / PARTIAL variant of tile j
  auto steady = [&](int j, auto par_tag, auto safe_tag, f32x16 (&sc)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
    if (unmasked(ent_cur))
      iteration(j, Bool<true>{}, Bool<true>{}, Bool<false>{}, par_tag, safe_tag, sc, sn);
    else
      iteration(j, Bool<true>{}, Bool<true>{}, Bool<true>{}, par_tag, safe_tag, sc, sn);
  };

  // Log-sum-exp of the row (natural log, sink included) from the log2-domain
  // reference m and denominator l: ln(l 2^m); -inf for a row with neither an
  // allowed key nor a sink.  Lanes l and l^32 hold the same row.
  auto store_lse = [&](float m, float l) __attribute__((always_inline)) {
    if (p.lse != nullptr && h2 == 0 && qi < p.L)
      p.lse[(static_cast<int64_t>(b) * p.H + head) * p.L + qi] =
          l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  };

  // Rare path: this wave's 32 query rows recomputed exactly in fp32, K and V
  // read straight from global memory (no LDS, no other wave involved).
  // Lanes l and l+32 share a query: each takes half of the head dimension,
  // for the dot products (summed over the pair) and for the output.
  auto exact_rows = [&]() __attribute__((always_inline)) {
    constexpr int DH = D / 2;
    const unsigned char* qr = qbase + (qi < p.L ? qi : p.L - 1) * q_row_bytes + h2 * DH * 2;
    bf16x8 qv[DH / 8];
#pragma unroll
    for (int c = 0; c < DH / 8; ++c) qv[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
    float m = -INFINITY, l = 0.f, o[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] = 0.f;
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
    if (sink_log2 > -INFINITY) {  // the sink adds exp2(s_aux log2 e - m) to the denominator
      const float m_new = fmaxf(m, sink_log2);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      l = l * alpha + __builtin_amdgcn_exp2f(sink_log2 - m_new);
#pragma unroll
      for (int d = 0; d < DH; ++d) o[d] *= alpha;
      m = m_new;
    }
    if (npieces > 1) {  // partial state of this piece, in the accumulator layout
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
  };
  // Whether some listed tile of this item holds an allowed key of this row.
  auto row_has_key = [&]() __attribute__((always_inline)) {
    bool has = false;
    const int hi_row = lo + static_cast<int>(width);
    for (int e = e_begin; e < e_end; ++e) {
      const int ent = p.kv[e];
      const int j0 = (ent >> 1) * kBN;
      has = has || (ent & 1) || (j0 < hi_row && j0 + kBN > lo) || j0 < pend;
    }
    return has;
  };

  // ---- epilogue: O = acc / (row sum + sink term) ----
  auto store_o = [&](float inv) __attribute__((always_inline)) {
    if (qi < p.L) {
      unsigned char* dst = obase + qi * o_row_bytes;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * h2;
          if (S::PAD_ROWSUM && 32 * dt + 8 * g >= D) continue;
          bf16x4 out;
          out[0] = (__bf16)(acc[dt][4 * g + 0] * inv);
          out[1] = (__bf16)(acc[dt][4 * g + 1] * inv);
          out[2] = (__bf16)(acc[dt][4 * g + 2] * inv);
          out[3] = (__bf16)(acc[dt][4 * g + 3] * inv);
          *reinterpret_cast<bf16x4*>(dst + d * 2) = out;
        }
      }
    }
  };

  // ---- a piece of a split row leaves its partial state in its slot ----
  // Slot layout (per wave): acc as float4 [DT][4][64 lanes], then m and l per
  // lane.  attn_merge_kernel, launched after this kernel on the same stream,
  // merges the pieces of every split row (so no device-scope fence is needed
  // here: the kernel boundary orders the writes before the merge's reads).
  float* slots = p.partials + static_cast<int64_t>(slot0) * kSlotFloats;

  // After the pass (fast pass: the reference is fixed after the first tile,
  // so later tiles need no row max).  Probabilities relative to it stay far
  // inside the bf16 / fp32 range unless a later score exceeds it by more than
  // 2^64.  The reference is a score of the row (or its sink) whenever the
  // first tile allows one of the row's keys, which makes the total at least
  // 1; a row that starts from the placeholder reference 0 instead can end far
  // below it.  A wave with a row (inside the sequence) whose row sum is not
  // finite or above 2^64, or whose total is below 2^-64 although the item
  // lists one of its keys, recomputes its rows exactly (exact_rows; no other
  // wave is involved) and finishes from there.  A piece of a split row may
  // legitimately hold none of a row's keys: that row's total is 0 and it is
  // left as is.
  auto finish_or_redo = [&](float lrow) __attribute__((always_inline)) {
    const bool off_range = qi < p.L && (!(lrow <= 0x1p64f) || !(lrow + sink_l >= 0x1p-64f));
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(off_range) != 0, 0)) {
      const bool redo = off_range && (!(lrow <= 0x1p64f) || row_has_key());
      if (__builtin_amdgcn_ballot_w64(redo) != 0) return true;
    }
    return false;
  };

  {
   // One pass over the item's tiles; `safe` selects the pass that tracks the
   // row max on every tile.
   auto pass = [&](auto safe) __attribute__((always_inline)) {
    __syncthreads();  // list staged, pad regions written
    ent_cur = __builtin_amdgcn_readfirstlane(list_lds[0]);
    ent_nxt = n > 1 ? __builtin_amdgcn_readfirstlane(list_lds[1]) : 0;
    if (dma_tensor == 0) issue_tile(ent_cur >> 1, 0);
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (unmasked(ent_cur)) iteration(0, Bool<true>{}, Bool<false>{}, Bool<false>{}, I0{}, safe, sB, sA);
    else iteration(0, Bool<true>{}, Bool<false>{}, Bool<true>{}, I0{}, safe, sB, sA);
    int j = 1;
    for (; j + 1 < n; j += 2) {
      steady(j, I1{}, safe, sA, sB);
      steady(j + 1, I0{}, safe, sB, sA);
    }
    if (j < n) {  // j = n - 1 (odd)
      steady(j, I1{}, safe, sA, sB);
      iteration(n, Bool<false>{}, Bool<true>{}, Bool<false>{}, I0{}, safe, sB, sA);
    } else {  // j = n (odd)
      iteration(n, Bool<false>{}, Bool<true>{}, Bool<false>{}, I1{}, safe, sA, sB);
    }
   };
   if (n > 0) pass(Bool<false>{});
  }
  const float lrow = S::PAD_ROWSUM ? low_half(acc[S::DT - 1][8])  // O^T row D (ones row of V^T), lanes 0..31
                                   : halves_sum(l_run);
  if (n > 0 && finish_or_redo(lrow)) {
    exact_rows();  // writes O, or this piece's partial state
    return;
  }
  const float ltot = lrow + sink_l;
  if (npieces == 1) {
    store_o(ltot > 0.f ? 1.f / ltot : 0.f);
    store_lse(ref_of(), ltot);
    return;
  }
  {
    float* sp = slots + static_cast<int64_t>(piece) * kSlotFloats;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = make_float4(acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]);
        *reinterpret_cast<float4*>(sp + (((wave * S::DT + dt) * 4 + g) * 64 + lane) * 4) = a;
      }
    }
    sp[kSlotM + wave * 64 + lane] = ltot > 0.f ? ref_of() : -INFINITY;
    sp[kSlotL + wave * 64 + lane] = ltot;
  }
}

// Merge of split rows (batch 1): one work-group per split row, its 4 waves
// with the forward's register layout (wave w, lane (l31, h2) holds query row
// 32 w + l31 of the 128-row tile, O^T elements d = 32 dt + 8 g + 4 h2 + e).
// The pieces' states are merged in piece order (the result does not depend
// on which piece finished first): m* = max of the pieces' references, then
// acc = sum of 2^(m_i - m*) acc_i and l = sum of 2^(m_i - m*) l_i; the sink
// term is already in piece 0's l.  Writes O = acc / l (0 for an empty row)
// and, when requested, the row's log-sum-exp.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(const GroupParams g) {
  using S = Shape<D>;
  constexpr int64_t kSlotFloats = partial_slot_floats(D);
  constexpr int kSlotM = 4 * S::DT * 16 * 64;
  constexpr int kSlotL = kSlotM + 4 * 64;
  int idx = static_cast<int>(blockIdx.x), jb = 0;
  while (jb + 1 < g.n_jobs && idx >= g.job[jb].n_merge) idx -= g.job[jb++].n_merge;
  const int job = __builtin_amdgcn_readfirstlane(jb);
  idx = __builtin_amdgcn_readfirstlane(idx);
  const FwdParams& p = g.job[job];
  if (idx >= p.n_merge) return;
  const int4 row = reinterpret_cast<const int4*>(p.merge_rows)[idx];
  const int head = __builtin_amdgcn_readfirstlane(row.x);
  const int qtile = __builtin_amdgcn_readfirstlane(row.y);
  const int slot0 = __builtin_amdgcn_readfirstlane(row.z);
  const int npieces = __builtin_amdgcn_readfirstlane(row.w);
  if constexpr (kChecked) {
    const uint32_t bits = merge_row_violations(head, qtile, slot0, npieces, p.H, p.L, p.n_slots);
    if (bits != 0) {
      if (threadIdx.x == 0 && p.check != nullptr) atomicOr(p.check, bits);
      return;
    }
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l31 = lane & 31;
  const float* slots = p.partials + static_cast<int64_t>(slot0) * kSlotFloats;

  // every piece's reference and sum first (one batch of loads), then the
  // pieces' accumulators two at a time: piece i + 1's loads are in flight
  // while piece i is added (pieces are still added in piece order)
  constexpr int kMaxMerge = 16;              // pieces per split row (the plan's limit)
  float mv[kMaxMerge], lv[kMaxMerge];
#pragma unroll
  for (int i = 0; i < kMaxMerge; ++i) {
    mv[i] = i < npieces ? slots[static_cast<int64_t>(i) * kSlotFloats + kSlotM + wave * 64 + lane] : -INFINITY;
    lv[i] = i < npieces ? slots[static_cast<int64_t>(i) * kSlotFloats + kSlotL + wave * 64 + lane] : 0.f;
  }
  float mmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxMerge; ++i) mmax = fmaxf(mmax, mv[i]);
  for (int i = kMaxMerge; i < npieces; ++i)  // beyond the plan's limit: read as needed
    mmax = fmaxf(mmax, slots[static_cast<int64_t>(i) * kSlotFloats + kSlotM + wave * 64 + lane]);
  f32x16 acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};
  float lm = 0.f;
  auto load_piece = [&](int i, float4 (&a)[S::DT * 4]) __attribute__((always_inline)) {
    const float* sp = slots + static_cast<int64_t>(i) * kSlotFloats;
#pragma unroll
    for (int k = 0; k < S::DT * 4; ++k) a[k] = *reinterpret_cast<const float4*>(sp + ((wave * S::DT * 4 + k) * 64 + lane) * 4);
  };
  auto add_piece = [&](int i, const float4 (&a)[S::DT * 4]) __attribute__((always_inline)) {
    float mi = mv[0], li = lv[0];
#pragma unroll
    for (int k = 1; k < kMaxMerge; ++k) {
      mi = i == k ? mv[k] : mi;
      li = i == k ? lv[k] : li;
    }
    if (i >= kMaxMerge) {
      mi = slots[static_cast<int64_t>(i) * kSlotFloats + kSlotM + wave * 64 + lane];
      li = slots[static_cast<int64_t>(i) * kSlotFloats + kSlotL + wave * 64 + lane];
    }
    const float w = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - mmax);
    lm = __builtin_fmaf(w, li, lm);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float4& x = a[dt * 4 + gg];
        acc[dt][4 * gg + 0] = __builtin_fmaf(w, x.x, acc[dt][4 * gg + 0]);
        acc[dt][4 * gg + 1] = __builtin_fmaf(w, x.y, acc[dt][4 * gg + 1]);
        acc[dt][4 * gg + 2] = __builtin_fmaf(w, x.z, acc[dt][4 * gg + 2]);
        acc[dt][4 * gg + 3] = __builtin_fmaf(w, x.w, acc[dt][4 * gg + 3]);
      }
    }
  };
  {
    float4 b0[S::DT * 4], b1[S::DT * 4];
    if (npieces > 0) load_piece(0, b0);
    for (int i = 0; i < npieces; i += 2) {
      if (i + 1 < npieces) load_piece(i + 1, b1);
      add_piece(i, b0);
      if (i + 1 < npieces) {
        if (i + 2 < npieces) load_piece(i + 2, b0);
        add_piece(i + 1, b1);
      }
    }
  }
  const int b = blockIdx.y;
  const int qi = qtile * kBM + wave * 32 + l31;
  if (qi >= p.L) return;
  const float inv = lm > 0.f ? 1.f / lm : 0.f;
  unsigned char* dst = reinterpret_cast<unsigned char*>(p.o + b * p.o_sb + head * p.o_sh) + qi * p.o_sl * 2;
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int d = 32 * dt + 8 * gg + 4 * h2;
      if (S::PAD_ROWSUM && 32 * dt + 8 * gg >= D) continue;
      bf16x4 out;
      out[0] = (__bf16)(acc[dt][4 * gg + 0] * inv);
      out[1] = (__bf16)(acc[dt][4 * gg + 1] * inv);
      out[2] = (__bf16)(acc[dt][4 * gg + 2] * inv);
      out[3] = (__bf16)(acc[dt][4 * gg + 3] * inv);
      *reinterpret_cast<bf16x4*>(dst + d * 2) = out;
    }
  }
  if (p.lse != nullptr && h2 == 0)
    p.lse[(static_cast<int64_t>(b) * p.H + head) * p.L + qi] =
        lm > 0.f ? (mmax + __builtin_amdgcn_logf(lm)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const GroupParams& g, int blocks, int B, hipStream_t stream, hipEvent_t start,
                    hipEvent_t stop) {
  dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(B));
  bool prefix = false;
  for (int j = 0; j < g.n_jobs; ++j) prefix = prefix || g.job[j].prefix > 0;
  int64_t merges = 0;
  for (int j = 0; j < g.n_jobs; ++j) merges += g.job[j].n_merge;
  // the extended launch attaches the events to the kernel's own dispatch
  hipEvent_t stop1 = merges > 0 ? nullptr : stop;
  hipError_t e = hipSuccess;
  if constexpr (D == 128 || D == 256) {
    bool pingpong = D == 128;
    for (int j = 0; j < g.n_jobs; ++j) pingpong = pingpong && g.job[j].pingpong != 0;
    e = pingpong ? launch_fwd_pp(g, grid, prefix, stream, start, stop1)
                 : launch_fwd_sg(g, D, grid, prefix, stream, start, stop1);
  } else {
    if (prefix) hipExtLaunchKernelGGL((attn_fwd_kernel<D, true>), grid, dim3(kThreads), 0, stream, start, stop1, 0, g);
    else hipExtLaunchKernelGGL((attn_fwd_kernel<D, false>), grid, dim3(kThreads), 0, stream, start, stop1, 0, g);
    e = hipGetLastError();
  }
  if (e != hipSuccess || merges == 0) return e;
  hipExtLaunchKernelGGL(attn_merge_kernel<D>, dim3(static_cast<unsigned>(merges), static_cast<unsigned>(B)),
                        dim3(kThreads), 0, stream, nullptr, stop, 0, g);
  return hipGetLastError();
}

// Scratch of the allocation-free forward: the plan image and the partial
// states of split rows, for callers that cannot allocate device memory.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// only the address hipGetSymbolAddress returns (per device) is passed on.
static __device__ __align__(256) unsigned char scratch[kFwdScratchBytes];

// Violation bits of the checked build's range checks (one word per device).
static __device__ uint32_t check_word;

// The current device's address of check_word (looked up once per device).
hipError_t check_word_addr(uint32_t** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint32_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_word));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<uint32_t*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace

bool checked_build() { return kChecked; }

hipError_t check_bits(uint32_t* bits, bool clear) {
  uint32_t* w = nullptr;
  hipError_t e = check_word_addr(&w);
  if (e != hipSuccess) return e;
  e = hipMemcpy(bits, w, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0;
  return hipMemcpy(w, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
}

hipError_t fwd_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kFwdScratchBytes;
  return hipSuccess;
}

hipError_t launch_fwd(const GroupParams& g, int D, int B, hipStream_t stream, hipEvent_t start,
                      hipEvent_t stop) {
  int64_t blocks = 0;
  for (int j = 0; j < g.n_jobs; ++j) blocks += 8 * static_cast<int64_t>(g.queue_len[j]);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (blocks == 0 || B == 0) {  // nothing to run: the events still mark this point of the stream
    hipError_t e = hipSuccess;
    if (start != nullptr) e = hipEventRecord(start, stream);
    if (e == hipSuccess && stop != nullptr) e = hipEventRecord(stop, stream);
    return e;
  }
  const GroupParams* gp = &g;
  GroupParams gc;
  if constexpr (dev::kChecked) {  // the kernels report range violations into the device's check word
    uint32_t* w = nullptr;
    hipError_t e = check_word_addr(&w);
    if (e != hipSuccess) return e;
    gc = g;
    for (int j = 0; j < gc.n_jobs; ++j) gc.job[j].check = w;
    gp = &gc;
  }
  switch (D) {
    case 64: return launch_d<64>(*gp, static_cast<int>(blocks), B, stream, start, stop);
    case 80: return launch_d<80>(*gp, static_cast<int>(blocks), B, stream, start, stop);
    case 128: return launch_d<128>(*gp, static_cast<int>(blocks), B, stream, start, stop);
    case 256: return launch_d<256>(*gp, static_cast<int>(blocks), B, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bss
