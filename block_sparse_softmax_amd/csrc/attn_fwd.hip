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
// Layout of the work (per work-group: 4 waves x 32 query rows):
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
//     current one is multiplied.  LDS rows are XOR-swizzled by 16-byte chunk.
//   * Masking code runs only on tiles flagged PARTIAL: every allowed key set
//     of the interval masks is one interval [lo, hi) per query, and a block
//     matrix whose block size is a multiple of the tile sizes adds only j <= i.
//   * Lazy rescaling: the running max moves only when a score exceeds it by
//     more than 2^8; probabilities stay below 256 and the result is the same
//     softmax (every term shares the reference point).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"

namespace bss {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;
constexpr int kListCap = 1024;  // KV-list entries staged in LDS at a time

constexpr int kMaskFull = 0, kMaskChunk = 1, kMaskWindow = 2, kMaskBlock = 3;

template <bool B>
struct Bool {
  static constexpr bool value = B;
};

template <int D>
struct Shape {
  static constexpr int CPR = D / 8;                          // 16-byte chunks per token row in memory
  static constexpr int RB = D * 2;                           // bytes per token row in memory
  // 16-byte chunks per row in LDS: d = 80 rows get two extra chunks whose V
  // slots hold the constant pad of the last O^T tile (element 80 = 1, so that
  // O^T row 80 is the row sum of P); the DMA never writes them.
  static constexpr int LCPR = (D == 80) ? 12 : CPR;
  static constexpr int LRB = LCPR * 16;                      // bytes per row in LDS
  static constexpr int KS = D / 16;                          // k-steps of the Q.K product
  static constexpr int DT = (D + 31) / 32;                   // 32-row tiles of O^T
  static constexpr int TILE = kBN * LRB;                     // bytes of one K (or V) tile in LDS
  static constexpr int LOADS = 2 * kBN * LCPR / 64 / kWaves; // LDS-DMA wave-instructions per wave per tile
  // waves 0-1 fill the K tile, waves 2-3 the V tile, LOADS wave-instructions each
  static_assert(2 * LOADS == LCPR, "each wave must cover half of one tensor's tile");
  // the XOR swizzle repeats every 16 rows; that many rows span DMA_PERIOD loads
  static constexpr int DMA_PERIOD = 16 * LCPR / 64;
  static_assert(LOADS % DMA_PERIOD == 0, "loads per wave must be whole swizzle periods");
  static constexpr bool PAD_ROWSUM = (D % 32) != 0;
};

// Physical 16-byte chunk of logical chunk c in LDS row `row` (an XOR, so its
// own inverse).  Chosen so that the 16 rows read by one K-fragment load, and
// the 4 rows x 64 bytes read by 32 lanes of one transposed V load, fall in
// distinct banks of a 64-bank LDS:
//   d = 128 (16 chunks):  c ^ {row bits 0-1 -> bits 2-3, row bits 2-3 -> bits 0-1}
//   d = 64  (8 chunks):   c ^ {row bit 1 -> bit 2, row bits 2-3 -> bits 0-1}
//   d = 80  (12 chunks):  c ^ row bits 2-3  (stays inside each aligned group of 4)
template <int D>
__device__ __forceinline__ int phys_chunk(int row, int c) {
  if constexpr (D == 128) return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  else if constexpr (D == 64) return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  else return c ^ ((row >> 2) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// One 16-byte global -> LDS copy per lane: lane l writes LDS bytes
// [lds_base + 16 l, lds_base + 16 l + 16).  Issued as inline assembly so the
// compiler does not treat every later LDS read as aliasing it (it would then
// wait for the whole prefetch before any LDS read); completion is tracked by
// the explicit vmcnt waits in the main loop.
__device__ __forceinline__ void dma16(const void* base_ptr, uint32_t voffset, uint32_t lds_base) {
  // readfirstlane yields int: widen through uint32_t so the low half is not sign-extended
  const uint64_t a = reinterpret_cast<uint64_t>(base_ptr);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  const uint64_t base = (static_cast<uint64_t>(hi) << 32) | lo;
  __asm__ volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voffset), "s"(base), "s"(lds_base)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)(p)));
}

__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Max (or sum) of x over lanes l and l^32.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Value of x held by lane (l mod 32), delivered to lanes l and l^32.
__device__ __forceinline__ float low_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const FwdParams p) {
  using S = Shape<D>;
  // LDS: K tiles in buffers 0-1, V tiles in buffers 2-3 (row pitch LRB).
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * S::TILE];
  __shared__ int list_lds[kListCap];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5;    // half of the wave
  const int l31 = lane & 31;

  // Work-groups are dealt to the 8 XCDs round-robin (block i runs on XCD i mod 8);
  // XCD x takes the x-th contiguous chunk of the schedule, so the items that
  // share an XCD's L2 at any time come from the same head.
  const int xcd_chunk = (p.n_items + 7) / 8;
  const int item_idx = p.xcd_chunked ? (blockIdx.x % 8) * xcd_chunk + blockIdx.x / 8 : blockIdx.x;
  if (item_idx >= p.n_items) return;
  const int4 item = reinterpret_cast<const int4*>(p.items)[item_idx];
  const int head = __builtin_amdgcn_readfirstlane(item.x);
  const int qtile = __builtin_amdgcn_readfirstlane(item.y);
  const int e_begin = __builtin_amdgcn_readfirstlane(item.z);
  const int e_end = __builtin_amdgcn_readfirstlane(item.w);
  const int b = blockIdx.y;

  const unsigned char* qbase =
      reinterpret_cast<const unsigned char*>(p.q + b * p.q_sb + head * p.q_sh);
  const unsigned char* kbase =
      reinterpret_cast<const unsigned char*>(p.k + b * p.k_sb + head * p.k_sh);
  const unsigned char* vbase =
      reinterpret_cast<const unsigned char*>(p.v + b * p.v_sb + head * p.v_sh);
  unsigned char* obase = reinterpret_cast<unsigned char*>(p.o + b * p.o_sb + head * p.o_sh);
  const int64_t q_row_bytes = p.q_sl * 2, k_row_bytes = p.k_sl * 2, v_row_bytes = p.v_sl * 2,
                o_row_bytes = p.o_sl * 2;

  // ---- the KV list of this item, staged in LDS kListCap entries at a time ----
  const int n = e_end - e_begin;
  auto stage_list = [&](int first) {
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

  // ---- allowed key interval [lo, hi) of this query (used on PARTIAL tiles) ----
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

  // ---- running softmax state (log2 domain) ----
  // m_run: reference max; l_run: row sum of this lane's keys (d != 80);
  // sink_l: the sink's term exp2(s_aux log2e - m_run).
  float m_run = -INFINITY, l_run = 0.f, sink_l = 0.f;
  if (p.sink != nullptr) {
    const float s = p.sink[head] * kLog2e;
    if (s > -INFINITY) {
      m_run = s;
      sink_l = 1.f;
    }
  }
  f32x16 acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};

  // ---- LDS addressing ----
  // K fragment for k-step ks: row l31 (and l31 + 32: same swizzle), logical chunk 2*ks + h2.
  int koff[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) koff[ks] = l31 * S::LRB + phys_chunk<D>(l31, 2 * ks + h2) * 16;
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
  if constexpr (S::PAD_ROWSUM) {
    // Constant pad chunks 10-11 of every V row in both V buffers: element 80 = 1, the rest 0.
    for (int i = threadIdx.x; i < 2 * kBN * 4; i += kThreads) {  // 2 buffers x 64 rows x 4 x 8 bytes
      const int buf = i / (kBN * 4), row = (i / 4) % kBN, q4 = i % 4;
      const int c = 10 + (q4 >> 1);
      uint2 v = make_uint2(0u, 0u);
      if (q4 == 0) v.x = 0x3F80u;  // bf16 1.0 in element 80
      *reinterpret_cast<uint2*>(smem + (2 + buf) * S::TILE + row * S::LRB +
                                phys_chunk<D>(row, c) * 16 + (q4 & 1) * 8) = v;
    }
  }

  // LDS-DMA: waves 0-1 fill K tiles and waves 2-3 V tiles; wave-instruction i
  // of a wave fills 64 consecutive 16-byte LDS slots of its half of the tile.
  const int dma_tensor = wave >> 1;
  const uint32_t dma_row_bytes = static_cast<uint32_t>(dma_tensor ? v_row_bytes : k_row_bytes);
  const unsigned char* dma_base = dma_tensor ? vbase : kbase;
  // Lane part of each load's source offset for one swizzle period (16 rows);
  // later periods add 16 rows to the uniform base.  Lanes whose slot is a
  // pad chunk (d = 80) load nothing.
  uint32_t goff[S::DMA_PERIOD];
  bool gpad[S::DMA_PERIOD];
#pragma unroll
  for (int i = 0; i < S::DMA_PERIOD; ++i) {
    const int slot = ((wave & 1) * S::LOADS + i) * 64 + lane;
    const int row = slot / S::LCPR;
    const int c = phys_chunk<D>(row, slot % S::LCPR);
    gpad[i] = c >= S::CPR;
    goff[i] = row * dma_row_bytes + (gpad[i] ? 0 : c) * 16;
  }
  const uint32_t smem_lds = lds_addr(smem);
  // Issue this wave's share of tile kt into LDS buffer buf (0-1 K, 2-3 V).
  auto issue_tile = [&](int kt, int buf) {
    const int kv0 = kt * kBN;
    const unsigned char* src = dma_base + static_cast<uint32_t>(kv0) * dma_row_bytes;
    const uint32_t dst =
        __builtin_amdgcn_readfirstlane(smem_lds + buf * S::TILE + (wave & 1) * S::LOADS * 1024);
    if (kv0 + kBN <= p.L) {
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const uint32_t rows_ahead = static_cast<uint32_t>((i / S::DMA_PERIOD) * 16);
        if (!S::PAD_ROWSUM || !gpad[i % S::DMA_PERIOD])
          dma16(src + rows_ahead * dma_row_bytes, goff[i % S::DMA_PERIOD], dst + i * 1024);
      }
    } else {  // ragged last tile: clamp rows past the end of the sequence (their keys are masked)
      const int last = p.L - 1 - kv0;
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const int slot = ((wave & 1) * S::LOADS + i) * 64 + lane;
        const int row = slot / S::LCPR;
        const int c = phys_chunk<D>(row, slot % S::LCPR);
        const uint32_t off = min(row, last) * dma_row_bytes + c * 16;
        if (!S::PAD_ROWSUM || c < S::CPR) dma16(src, off, dst + i * 1024);
      }
    }
  };

  // S^T = K Q^T + seed (log2-domain logits minus the reference max) for a
  // 64-key tile; the seed block is the C operand of the first k-step.
  auto qk = [&](int kbuf, const f32x16& seed, f32x16& s0, f32x16& s1) {
    const unsigned char* kt_lds = smem + kbuf * S::TILE;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kt_lds + koff[ks]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kt_lds + koff[ks] + 32 * S::LRB);
      s0 = mfma32(a0, qf[ks], ks == 0 ? seed : s0);
      s1 = mfma32(a1, qf[ks], ks == 0 ? seed : s1);
    }
  };
  // O^T += V^T P^T for a 64-key tile.
  auto pv = [&](int vbuf, const bf16x8 (&pb)[4]) {
    const unsigned char* vt_lds = smem + vbuf * S::TILE;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {  // consecutive MFMAs use different accumulators
        const unsigned char* src = vt_lds + 16 * t * S::LRB;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + voff[dt][0]));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + voff[dt][1]));
        const s16x8 x = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[dt] = mfma32(__builtin_bit_cast(bf16x8, x), pb[t], acc[dt]);
      }
    }
  };
  // Seed of a tile's S^T accumulators: minus the current reference max (0 while
  // none), kept as a 16-register block rewritten only when the max moves.
  f32x16 seedv;
  auto set_seed = [&]() {
    const float sd = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) seedv[r] = sd;
  };
  set_seed();

  // ---- main loop: one listed tile per iteration ----
  // K and V of tile j sit in buffers (j&1) and 2 + (j&1); the DMA for tile
  // j+1 is issued at the top of iteration j, right after the barrier that
  // guarantees every wave is done with the buffers of tile j-1.
  int list_base = 0;
  int ent_c = 0;
  if (n > 0) {
    __syncthreads();  // list staged, pad regions written
    ent_c = __builtin_amdgcn_readfirstlane(list_lds[0]);
    issue_tile(ent_c >> 1, 2 * dma_tensor);
  }
  for (int j = 0; j < n; ++j) {
    const int ent = __builtin_amdgcn_readfirstlane(ent_c);
    wait_vmcnt<0>();   // this wave's share of tile j (and, at j = 0, the Q fragments)
    wg_barrier();      // everyone's share of tile j; buffers of tile j-1 are free
    if (j + 1 < n) {
      if (j + 1 - list_base == kListCap) {  // next chunk of the list
        list_base += kListCap;
        stage_list(list_base);
        __syncthreads();
      }
      ent_c = __builtin_amdgcn_readfirstlane(list_lds[j + 1 - list_base]);
      issue_tile(ent_c >> 1, 2 * dma_tensor + ((j + 1) & 1));
    }

    // ---- S^T of tile j, relative to the reference max (seeded C operand) ----
    f32x16 s0, s1;
    qk(j & 1, seedv, s0, s1);

    // ---- mask (PARTIAL tiles only), row max, lazy rescale ----
    if (!(ent & 1)) {
      const unsigned base = static_cast<unsigned>((ent >> 1) * kBN + 4 * h2 - lo);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned u = base + 8 * (r >> 2) + (r & 3);
        s0[r] = (u >= width) ? -INFINITY : s0[r];
        s1[r] = (u + 32 >= width) ? -INFINITY : s1[r];
      }
    }
    float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
    mt = halves_max(mt);
    const bool need = (m_run == -INFINITY) ? (mt > -INFINITY) : (mt > kRescaleThreshold);
    if (__builtin_amdgcn_ballot_w64(need)) {
      float alpha = 1.f, shift = 0.f;
      if (need) {
        const float m_new = (m_run == -INFINITY ? 0.f : m_run) + mt;
        alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        shift = mt;
      }
      s0 -= shift;
      s1 -= shift;
      l_run *= alpha;
      sink_l *= alpha;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) acc[dt] *= alpha;
      set_seed();
    }

    // ---- P = exp2(S), O^T += V^T P^T ----
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(s0[r]);
      s1[r] = __builtin_amdgcn_exp2f(s1[r]);
      if (!S::PAD_ROWSUM) rs += s0[r] + s1[r];
    }
    if (!S::PAD_ROWSUM) l_run += rs;
    bf16x8 pb[4];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      pb[0][e8] = (__bf16)s0[e8];
      pb[1][e8] = (__bf16)s0[8 + e8];
      pb[2][e8] = (__bf16)s1[e8];
      pb[3][e8] = (__bf16)s1[8 + e8];
    }
    pv(2 + (j & 1), pb);
  }

  // ---- epilogue: O = acc / (row sum + sink term) ----
  float lsum;
  if (S::PAD_ROWSUM) {
    lsum = low_half(acc[S::DT - 1][8]);  // O^T row D (ones row of V^T), held by lanes 0..31
  } else {
    lsum = halves_sum(l_run);
  }
  const float ltot = lsum + sink_l;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
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
}

template <int D>
hipError_t launch_d(const FwdParams& p, int B, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(8 * ((p.n_items + 7) / 8)), static_cast<unsigned>(B));
  hipLaunchKernelGGL(attn_fwd_kernel<D>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int D, int B, hipStream_t stream) {
  if (p.n_items == 0 || B == 0) return hipSuccess;
  switch (D) {
    case 64: return launch_d<64>(p, B, stream);
    case 80: return launch_d<80>(p, B, stream);
    case 128: return launch_d<128>(p, B, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bss
