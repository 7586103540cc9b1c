// Backward pass of structured-mask softmax attention for gfx950 (MI355X).
//
// For a loss with upstream gradient dO and the forward's per-row log-sum-exp,
// the chain rule through o_i = sum_j p_ij v_j and the masked row softmax
// (with the per-head sink logit of "Semantic Head Specialization ...", the
// sink-bias slide, in the denominator) gives, with s_ij = sigma q_i.k_j on the
// allowed pairs and p_ij = exp(s_ij - lse_i):
//
//   D_i = dO_i . O_i,   dP_ij = dO_i . v_j,   dS_ij = p_ij (dP_ij - D_i),
//   dV_j = sum_i p_ij dO_i,   dK_j = sigma sum_i dS_ij q_i,
//   dQ_i = sigma sum_j dS_ij k_j,   d s_aux = - sum_i exp(s_aux - lse_i) D_i.
//
// The pages train these masks (the SHS slides' ViT variants, the per-head
// windows of "Asymmetric Attention Heads"); the tiling reuses the forward's
// tile lists, so masked-out tiles are skipped here too.  Four kernels run in
// order on one stream:
//   bwd_prep  D_i and the log2-domain lse of every row (padded rows get
//             lse = +inf, so their probabilities are exactly 0), per
//             (batch, head, query tile) partial sums of the sink gradient,
//             and Qs = Q sigma log2(e) rounded to bf16 exactly as the forward
//             rounds it: the scores recomputed from Qs are the forward's
//             (in log2 units), so exp2(s - lse2) are the probabilities the
//             forward normalised (a row with one key gets p = 1 exactly);
//   bwd_dq    query-major, over the forward's per-query-tile KV lists: S^T,
//             dP^T = V dO^T and dQ^T += K^T dS^T on MFMA (the forward's
//             layout: Q and dO stay in registers, K and V tiles stream
//             through LDS, K^T is read transposed);
//   bwd_dkdv  key-major, over the transposed lists: a work-group owns 128
//             keys (32 per wave) of one K/V head and walks every query tile
//             of every query head of its group that lists them.  K and V of
//             the wave's keys stay in registers as B operands; Qs and dO
//             tiles stream through LDS.  S = Qs K^T leaves P and dS in the
//             B-operand layout of dV^T += dO^T P and dK^T += Qs^T dS (dO^T,
//             Qs^T read transposed), so nothing is shuffled; dK = that sum /
//             log2(e) (Qs = sigma log2(e) Q up to the rounding);
//   bwd_sink  the sink gradient, summed in a fixed order (deterministic).
// dQ and dK/dV are written once each (no atomics): the two kernels recompute
// S and dP on their own, which costs two extra matrix products per tile pair
// against a single kernel with atomic dQ accumulation, and keeps the result
// bit-reproducible.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"
#include "tile_common.hpp"

namespace bss {
namespace {

using namespace dev;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// prep: D_i, lse2_i; partial sink-gradient sums
// ---------------------------------------------------------------------------
// One work-group per (batch, head, query tile); a row's 16-byte chunks sit on
// P adjacent lanes (P = D / 8 rounded up to a power of two, lanes past D / 8
// idle), so every load and store of a pass is contiguous; D_i is summed per
// lane over its 8 elements, then over the row's lanes.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p) {
  constexpr int CH = D / 8;                  // 16-byte chunks of a row
  constexpr int P = CH <= 8 ? 8 : 16;        // lanes per row
  constexpr int RPP = 256 / P;               // rows per pass
  static_assert(CH <= P && kBM % RPP == 0, "row layout");
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % P, rsub = threadIdx.x / P;
  const unsigned char* obase = reinterpret_cast<const unsigned char*>(p.o + b * p.o_sb + h * p.o_sh);
  const unsigned char* gbase = reinterpret_cast<const unsigned char*>(p.dout + b * p.do_sb + h * p.do_sh);
  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q + b * p.q_sb + h * p.q_sh);
  unsigned char* qwbase = reinterpret_cast<unsigned char*>(p.qs) + (static_cast<int64_t>(b) * p.H + h) * p.L * (D * 2);
  float* st = p.stat + (static_cast<int64_t>(b) * p.H + h) * 2 * p.Lpad;
  const float sink2 = (p.dsink != nullptr && p.sink != nullptr) ? p.sink[h] * kLog2e : -INFINITY;
  float t = 0.f;                             // this lane's share of the sink-gradient partial sum
  for (int pass = 0; pass < kBM / RPP; ++pass) {
    const int i = qt * kBM + pass * RPP + rsub;
    float dsum = 0.f;
    if (i < p.L && c < CH) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(obase + static_cast<int64_t>(i) * p.o_sl * 2 + 16 * c);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(gbase + static_cast<int64_t>(i) * p.do_sl * 2 + 16 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)x[e], (float)y[e], dsum);
      // this lane's chunk of the scaled query row
      const bf16x8 qx = *reinterpret_cast<const bf16x8*>(qbase + static_cast<int64_t>(i) * p.q_sl * 2 + 16 * c);
      bf16x8 qy;
#pragma unroll
      for (int e = 0; e < 8; ++e) qy[e] = (__bf16)((float)qx[e] * p.scale_log2);
      *reinterpret_cast<bf16x8*>(qwbase + static_cast<int64_t>(i) * (D * 2) + 16 * c) = qy;
    }
#pragma unroll
    for (int off = 1; off < P; off <<= 1) dsum += __shfl_xor(dsum, off);
    if (c == 0) {
      float lse2 = INFINITY;
      if (i < p.L) {
        const float lse = p.lse[(static_cast<int64_t>(b) * p.H + h) * p.L + i];
        lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
      }
      st[i] = lse2;
      st[p.Lpad + i] = i < p.L ? dsum : 0.f;
      // the sink's share of row i is exp2(s_aux log2 e - lse2_i)
      if (i < p.L && sink2 > -INFINITY) t += __builtin_amdgcn_exp2f(sink2 - lse2) * dsum;
    }
  }
  if (p.dsink == nullptr) return;
  __shared__ float red[256];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.sinkpart[(static_cast<int64_t>(b) * p.H + h) * p.nq + qt] = red[0];
}

// d s_aux[h] = - sum over batches and query tiles of the partial sums (fixed order).
__global__ __launch_bounds__(256) void bwd_sink_kernel(const BwdParams p, int B) {
  const int h = blockIdx.x;
  float t = 0.f;
  for (int b = 0; b < B; ++b)
    for (int qt = threadIdx.x; qt < p.nq; qt += 256) t += p.sinkpart[(static_cast<int64_t>(b) * p.H + h) * p.nq + qt];
  __shared__ float red[256];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.dsink[h] = p.sink != nullptr ? -red[0] : 0.f;
}

// ---------------------------------------------------------------------------
// Shared pieces of the two MFMA kernels
// ---------------------------------------------------------------------------

// Global -> LDS copy of 64-row tiles of two tensors in the forward's LDS row
// layout (row pitch LRB, XOR-swizzled chunks): waves 0-1 copy tensor A, waves
// 2-3 tensor B.  d = 80 rows carry two pad chunks, filled with a copy of the
// row's chunk 0 (they only feed output rows beyond d, which are never stored).
template <int D>
struct TileCopy {
  using S = Shape<D>;
  uint32_t goff[S::DMA_PERIOD];
  uint32_t row_bytes;
  int wave;

  __device__ __forceinline__ void init(int wave_, int lane, int64_t row_bytes_a, int64_t row_bytes_b) {
    wave = wave_;
    row_bytes = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>((wave >> 1) ? row_bytes_b : row_bytes_a)));
#pragma unroll
    for (int i = 0; i < S::DMA_PERIOD; ++i) {
      const int slot = ((wave & 1) * S::LOADS + i) * 64 + lane;
      const int row = slot / S::LCPR;
      const int c = phys_chunk<D>(row, slot % S::LCPR);
      goff[i] = row * row_bytes + (c >= S::CPR ? 0 : c) * 16;
    }
  }
  // Rows row0 .. row0+63 of this wave's tensor (base = its element [0] of the
  // head) into LDS bytes dst .. (dst: the tile of this wave's tensor); rows at
  // or past L (row0 itself may be) are copies of row L-1.
  __device__ __forceinline__ void issue(const void* base, int row0, int L, uint32_t dst, int lane) const {
    const uint32_t d0 = __builtin_amdgcn_readfirstlane(dst + (wave & 1) * S::LOADS * 1024);
    if (row0 + kBN <= L) {
      const uint64_t tb = uniform_u64(reinterpret_cast<uint64_t>(base) + static_cast<uint64_t>(row0) * row_bytes);
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i)
        dma16(tb + static_cast<uint64_t>((i / S::DMA_PERIOD) * 16) * row_bytes, goff[i % S::DMA_PERIOD], d0 + i * 1024);
    } else {
      // offsets from the last in-range row at or before row0 (never negative)
      const int rb = min(row0, L - 1);
      const uint64_t tb = uniform_u64(reinterpret_cast<uint64_t>(base) + static_cast<uint64_t>(rb) * row_bytes);
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const int slot = ((wave & 1) * S::LOADS + i) * 64 + lane;
        const int row = slot / S::LCPR;
        const int c = phys_chunk<D>(row, slot % S::LCPR);
        const int src = min(row0 + row, L - 1) - rb;  // 0 .. 63
        dma16(tb, static_cast<uint32_t>(src) * row_bytes + (c < S::CPR ? c : 0) * 16, d0 + i * 1024);
      }
    }
  }
};

// LDS offsets inside a 64-row tile.
//   row fragment (A or B operand whose K dimension is the head dimension):
//     lane (l31, h2) reads row 32 half + l31, elements 16 ks + 8 h2 .. +7;
//   transposed fragment (A operand whose K dimension runs over 16 rows
//     16 t .. 16 t + 15, M over head-dim rows 32 dt ..): two ds_read_b64_tr_b16
//     reads; element e of lane (m, h2) is row 16 t + 8 (e / 4) + 4 h2 + e % 4,
//     the row order in which a 32x32 MFMA result holds its M rows, so an
//     output block converts to the matching B operand in place.
template <int D>
__device__ __forceinline__ int row_frag_off(int lane, int ks) {
  using S = Shape<D>;
  const int l31 = lane & 31, h2 = lane >> 5;
  return l31 * S::LRB + phys_chunk<D>(l31, 2 * ks + h2) * 16;
}
template <int D>
__device__ __forceinline__ int tr_frag_off(int lane, int dt, int u) {
  using S = Shape<D>;
  const int h2 = lane >> 5, tr_j = (lane & 15) >> 2, tr_c = lane & 3, dhalf = (lane >> 4) & 1;
  const int row = 8 * u + 4 * h2 + tr_j;
  const int c = 4 * dt + 2 * dhalf + (tr_c >> 1);
  return row * S::LRB + phys_chunk<D>(row, c) * 16 + (tr_c & 1) * 8;
}
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const unsigned char* tile, int off, int half) {
  return *reinterpret_cast<const bf16x8*>(tile + off + half * 32 * Shape<D>::LRB);
}
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* tile, int off0, int off1, int t) {
  const unsigned char* src = tile + 16 * t * Shape<D>::LRB;
  const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + off0));
  const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + off1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Store a transposed accumulator block (32 head-dim rows per tile, lane =
// token) times `scale` as bf16 into the token row `dst` (16-byte aligned).
template <int D>
__device__ __forceinline__ void store_rows(unsigned char* dst, const f32x16 (&acc)[Shape<D>::DT], float scale,
                                           int h2) {
#pragma unroll
  for (int dt = 0; dt < Shape<D>::DT; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (32 * dt + 8 * g >= D) continue;
      const int d = 32 * dt + 8 * g + 4 * h2;
      bf16x4 out;
      out[0] = (__bf16)(acc[dt][4 * g + 0] * scale);
      out[1] = (__bf16)(acc[dt][4 * g + 1] * scale);
      out[2] = (__bf16)(acc[dt][4 * g + 2] * scale);
      out[3] = (__bf16)(acc[dt][4 * g + 3] * scale);
      *reinterpret_cast<bf16x4*>(dst + d * 2) = out;
    }
  }
}

// Fragments (row layout, K dimension = head dim) of one token row of a
// tensor, straight from global memory: lane (l31, h2) of the wave gets
// elements 16 ks + 8 h2 .. +7 of row `row`.
template <int D>
__device__ __forceinline__ void load_row_frags(bf16x8 (&f)[Shape<D>::KS], const uint16_t* base, int64_t row_elems,
                                               int row, int h2) {
  const unsigned char* src = reinterpret_cast<const unsigned char*>(base) + row * row_elems * 2 + 16 * h2;
#pragma unroll
  for (int ks = 0; ks < Shape<D>::KS; ++ks) f[ks] = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
}

// ---------------------------------------------------------------------------
// dQ: query-major over the forward's lists (work item = head, 128-row query tile)
// ---------------------------------------------------------------------------
template <int D, bool PREFIX>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(const BwdParams p) {
  using S = Shape<D>;
  // K tiles in buffers 0-1, V tiles in 2-3
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * S::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l31 = lane & 31;
  const int pos = static_cast<int>(blockIdx.x / 8);
  if (pos >= p.q_queue) return;
  const int item_idx = static_cast<int>(blockIdx.x % 8) * p.q_queue + pos;
  const int4 item = reinterpret_cast<const int4*>(p.q_items)[2 * item_idx];
  const int4 split = reinterpret_cast<const int4*>(p.q_items)[2 * item_idx + 1];
  const int head = __builtin_amdgcn_readfirstlane(item.x);
  if (head < 0) return;
  const int qtile = __builtin_amdgcn_readfirstlane(item.y);
  const int e_begin = __builtin_amdgcn_readfirstlane(item.z);
  const int e_end = __builtin_amdgcn_readfirstlane(item.w);
  // a piece of a split row (batch 1) sums dQ over its part of the row's list
  const int slot = __builtin_amdgcn_readfirstlane(split.x + split.y);
  const int npieces = __builtin_amdgcn_readfirstlane(split.z);
  const int b = blockIdx.y;
  const int kv_head = head / p.kv_group;
  const uint16_t* kb = p.k + b * p.k_sb + kv_head * p.k_sh;
  const uint16_t* vb = p.v + b * p.v_sb + kv_head * p.v_sh;

  const int qi = qtile * kBM + wave * 32 + l31;
  const int qrow = qi < p.L ? qi : p.L - 1;
  bf16x8 qf[S::KS], gf[S::KS];
  load_row_frags<D>(qf, p.qs + (static_cast<int64_t>(b) * p.H + head) * p.L * D, D, qrow, h2);
  load_row_frags<D>(gf, p.dout + b * p.do_sb + head * p.do_sh, p.do_sl, qrow, h2);
  const float* st = p.stat + (static_cast<int64_t>(b) * p.H + head) * 2 * p.Lpad;
  const float lse2 = st[qi];
  const float drow = st[p.Lpad + qi];

  // allowed key interval [lo, lo + width) of this query, plus prefix keys [0, pend)
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

  TileCopy<D> dma;
  dma.init(wave, lane, p.k_sl * 2, p.v_sl * 2);
  const uint16_t* dma_base = (wave >> 1) ? vb : kb;
  const uint32_t smem_lds = lds_addr(smem);
  int koffs[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) koffs[ks] = row_frag_off<D>(lane, ks);
  int toff[S::DT][2];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
    toff[dt][0] = tr_frag_off<D>(lane, dt, 0);
    toff[dt][1] = tr_frag_off<D>(lane, dt, 1);
  }

  f32x16 acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};

  // list entries (kv_tile << 1 | full) of tiles j and j+1; entry j+2 is
  // fetched during iteration j
  const int n = e_end - e_begin;
  int ent_cur = n > 0 ? __builtin_amdgcn_readfirstlane(p.kv[e_begin]) : 0;
  int ent_nxt = n > 1 ? __builtin_amdgcn_readfirstlane(p.kv[e_begin + 1]) : 0;
  if (n > 0) dma.issue(dma_base, (ent_cur >> 1) * kBN, p.L, smem_lds + 2 * (wave >> 1) * S::TILE, lane);
  for (int j = 0; j < n; ++j) {
    const int ent = ent_cur;
    const int par = j & 1;
    wait_vmcnt<0>();
    wg_barrier();  // tile j is in LDS; every wave is done with tile j-1's buffers
    if (j + 1 < n)
      dma.issue(dma_base, (ent_nxt >> 1) * kBN, p.L, smem_lds + (2 * (wave >> 1) + (par ^ 1)) * S::TILE, lane);
    const int raw2 = (j + 2 < n) ? p.kv[e_begin + j + 2] : 0;
    const unsigned char* kt = smem + par * S::TILE;
    const unsigned char* vt = smem + (2 + par) * S::TILE;

    // S^T = K Qs^T (log2 units) and dP^T = V dO^T, two 32-key halves
    f32x16 s[2], dp[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      s[half] = f32x16{};
      dp[half] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        s[half] = mfma32(row_frag<D>(kt, koffs[ks], half), qf[ks], s[half]);
        dp[half] = mfma32(row_frag<D>(vt, koffs[ks], half), gf[ks], dp[half]);
      }
    }
    const int kv0 = (ent >> 1) * kBN;
    const bool masked = !((ent & 1) || (kv0 >= wave_lo_max && kv0 + kBN <= wave_hi_min));
    if (masked) {
      const unsigned mbase = static_cast<unsigned>(kv0 + 4 * h2 - lo);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned u = mbase + 8 * (r >> 2) + (r & 3);
        const int key = kv0 + 4 * h2 + 8 * (r >> 2) + (r & 3);
        bool out0 = u >= width, out1 = u + 32 >= width;
        if constexpr (PREFIX) {
          out0 = out0 && key >= pend;
          out1 = out1 && key + 32 >= pend;
        }
        s[0][r] = out0 ? -INFINITY : s[0][r];
        s[1][r] = out1 ? -INFINITY : s[1][r];
      }
    }
    // dS^T = P^T (dP^T - D), in bf16 as the B operand of 16-key steps
    bf16x8 dsb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * (t & 1) + e;
        const float pr = __builtin_amdgcn_exp2f(s[t >> 1][r] - lse2);
        dsb[t][e] = (__bf16)(pr * (dp[t >> 1][r] - drow));
      }
    }
    // dQ^T += K^T dS^T.  At d < 128 two waves share a SIMD: the one feeding
    // the matrix core issues first (raised priority), the other's VALU work
    // fills the MFMA shadow (+5 % on the 896-px full backward; at d = 128 it
    // cost 3 %).
    if constexpr (D != 128) {
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) acc[dt] = mfma32(tr_frag<D>(kt, toff[dt][0], toff[dt][1], t), dsb[t], acc[dt]);
    }
    if constexpr (D != 128) {
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    ent_cur = ent_nxt;
    ent_nxt = __builtin_amdgcn_readfirstlane(raw2);
  }
  if (npieces > 1) {  // this piece's dQ^T sum, in the forward's partial-slot layout (acc part)
    float* sp = p.partials + static_cast<int64_t>(slot) * partial_slot_floats(D);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = make_float4(acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]);
        *reinterpret_cast<float4*>(sp + (((wave * S::DT + dt) * 4 + g) * 64 + lane) * 4) = a;
      }
    }
    return;
  }
  if (qi < p.L) {
    unsigned char* dst = reinterpret_cast<unsigned char*>(p.dq + b * p.dq_sb + head * p.dq_sh) +
                         static_cast<int64_t>(qi) * p.dq_sl * 2;
    store_rows<D>(dst, acc, p.scale, h2);
  }
}

// dQ of the split rows (batch 1): one work-group per split row adds its
// pieces' sums in piece order (a fixed order: the result does not depend on
// which piece finished first) and writes dQ = scale * sum.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_merge_kernel(const BwdParams p) {
  using S = Shape<D>;
  const int4 row = reinterpret_cast<const int4*>(p.merge_rows)[blockIdx.x];
  const int head = __builtin_amdgcn_readfirstlane(row.x);
  const int qtile = __builtin_amdgcn_readfirstlane(row.y);
  const int slot0 = __builtin_amdgcn_readfirstlane(row.z);
  const int npieces = __builtin_amdgcn_readfirstlane(row.w);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l31 = lane & 31;
  f32x16 acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};
  for (int i = 0; i < npieces; ++i) {
    const float* sp = p.partials + static_cast<int64_t>(slot0 + i) * partial_slot_floats(D);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = *reinterpret_cast<const float4*>(sp + (((wave * S::DT + dt) * 4 + g) * 64 + lane) * 4);
        acc[dt][4 * g + 0] += a.x;
        acc[dt][4 * g + 1] += a.y;
        acc[dt][4 * g + 2] += a.z;
        acc[dt][4 * g + 3] += a.w;
      }
    }
  }
  const int qi = qtile * kBM + wave * 32 + l31;
  if (qi < p.L) {
    unsigned char* dst = reinterpret_cast<unsigned char*>(p.dq + head * p.dq_sh) + static_cast<int64_t>(qi) * p.dq_sl * 2;
    store_rows<D>(dst, acc, p.scale, h2);
  }
}

// ---------------------------------------------------------------------------
// dK, dV: key-major over the transposed lists (work item = K/V head, 128 keys)
// ---------------------------------------------------------------------------
template <int D>
struct DkdvShape {
  using S = Shape<D>;
  // a stage: Q rows, dO rows (64 each), then lse2[64] and D[64]
  static constexpr int STAGE = 2 * S::TILE + 1024;
  static constexpr int STAT = 2 * S::TILE;
  // d = 128 keeps K, V fragments and both accumulators in registers: one
  // wave per SIMD (512 registers with the accumulation registers)
  static constexpr int OCC = D == 128 ? 1 : 2;
};

template <int D, bool PREFIX>
__global__ __launch_bounds__(kThreads, DkdvShape<D>::OCC) void bwd_dkdv_kernel(const BwdParams p) {
  using S = Shape<D>;
  using T = DkdvShape<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * T::STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l31 = lane & 31;
  const int pos = static_cast<int>(blockIdx.x / 8);
  if (pos >= p.kv_queue) return;
  const int item_idx = static_cast<int>(blockIdx.x % 8) * p.kv_queue + pos;
  const int4 item = reinterpret_cast<const int4*>(p.kv_items)[2 * item_idx];
  const int4 split = reinterpret_cast<const int4*>(p.kv_items)[2 * item_idx + 1];
  const int hk = __builtin_amdgcn_readfirstlane(item.x);
  if (hk < 0) return;
  const int kblk = __builtin_amdgcn_readfirstlane(item.y);
  const int c_begin = __builtin_amdgcn_readfirstlane(item.z);
  const int c_end = __builtin_amdgcn_readfirstlane(item.w);
  // a piece of a split key block (batch 1) sums dK and dV over its part of the block's list
  const int slot = __builtin_amdgcn_readfirstlane(split.x + split.y);
  const int npieces = __builtin_amdgcn_readfirstlane(split.z);
  const int b = blockIdx.y;

  // this lane's key (N index of every product) and its K, V fragments
  const int kj = kblk * 2 * kBN + wave * 32 + l31;
  const int krow = kj < p.L ? kj : p.L - 1;
  bf16x8 kf[S::KS], vf[S::KS];
  load_row_frags<D>(kf, p.k + b * p.k_sb + hk * p.k_sh, p.k_sl, krow, h2);
  load_row_frags<D>(vf, p.v + b * p.v_sb + hk * p.v_sh, p.v_sl, krow, h2);

  // key-side form of the mask: the queries that may see key kj form one
  // interval [qlo, qhi) (chunk: the key's chunk; window: j - right .. j + left;
  // causal and block: from j on; a prefix key: every query, from j on when
  // causal); the chunk bounds do not depend on the head
  int chunk_lo = 0, chunk_hi = p.L;
  if (p.kind == kMaskChunk) {
    chunk_lo = (kj / p.chunk) * p.chunk;
    chunk_hi = min(p.L, chunk_lo + p.chunk);
  }
  const bool causal = p.causal || p.kind == kMaskBlock;

  TileCopy<D> dma;
  dma.init(wave, lane, D * 2, p.do_sl * 2);
  const uint32_t smem_lds = lds_addr(smem);
  int roffs[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) roffs[ks] = row_frag_off<D>(lane, ks);
  int toff[S::DT][2];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
    toff[dt][0] = tr_frag_off<D>(lane, dt, 0);
    toff[dt][1] = tr_frag_off<D>(lane, dt, 1);
  }

  f32x16 dk[S::DT], dv[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // steps: two 64-row halves of every listed query tile
  const int nsteps = 2 * (c_end - c_begin);
  auto step_head = [&](int ent) __attribute__((always_inline)) { return hk * p.kv_group + (ent >> 24); };
  auto step_row0 = [&](int ent, int s) __attribute__((always_inline)) { return ((ent >> 1) & 0x7FFFFF) * kBM + 64 * s; };
  // copy step (ent, s) into stage buffer `stage`: Q rows (waves 0-1), dO rows
  // (waves 2-3), lse2 and D of the 64 rows (wave 0, lanes 0-31)
  auto issue_step = [&](int ent, int s, int stage) __attribute__((always_inline)) {
    const int h = step_head(ent), row0 = step_row0(ent, s);
    const uint16_t* base = (wave >> 1) ? p.dout + b * p.do_sb + h * p.do_sh
                                       : p.qs + (static_cast<int64_t>(b) * p.H + h) * p.L * D;
    const uint32_t dst = smem_lds + stage * T::STAGE + (wave >> 1) * S::TILE;
    dma.issue(base, row0, p.L, dst, lane);
    if (wave == 0) {
      const float* sb = p.stat + (static_cast<int64_t>(b) * p.H + h) * 2 * p.Lpad;
      const uint32_t off = static_cast<uint32_t>(((lane < 16) ? row0 + 4 * lane : p.Lpad + row0 + 4 * (lane - 16)) * 4);
      dma16_skip(uniform_u64(reinterpret_cast<uint64_t>(sb)), off, __builtin_amdgcn_readfirstlane(smem_lds + stage * T::STAGE + T::STAT),
                 0xFFFFFFFF00000000ull);
    }
  };

  int ent_cur = nsteps > 0 ? __builtin_amdgcn_readfirstlane(p.col[c_begin]) : 0;
  if (nsteps > 0) issue_step(ent_cur, 0, 0);
  int ent_nxt = nsteps > 2 ? p.col[c_begin + 1] : 0;
  int qlo = 0, qwidth = 0;
  for (int k = 0; k < nsteps; ++k) {
    const int s = k & 1, stage = k & 1;
    wait_vmcnt<0>();
    wg_barrier();  // step k is in LDS; every wave is done with step k-1's stage
    // next step: the other half of this tile, or the first half of the next
    if (k + 1 < nsteps) {
      if (s == 0) issue_step(ent_cur, 1, stage ^ 1);
      else issue_step(__builtin_amdgcn_readfirstlane(ent_nxt), 0, stage ^ 1);
    }
    const int ent = ent_cur;
    const int h = step_head(ent), row0 = step_row0(ent, s);
    if (s == 0) {
      // this query head's interval for the lane's key
      int lo = chunk_lo, hi = chunk_hi;
      if (p.kind == kMaskWindow) {
        lo = max(0, kj - p.right);
        hi = min(p.L, kj + p.head_left[h] + 1);
      }
      if (causal) lo = max(lo, kj);
      if constexpr (PREFIX) {
        if (kj < p.prefix) {
          lo = causal ? kj : 0;
          hi = p.L;
        }
      }
      if (kj >= p.L) hi = lo;
      qlo = lo;
      qwidth = max(hi - lo, 0);
    }
    const bool masked = (ent & 1) == 0;
    const unsigned char* qt = smem + stage * T::STAGE;
    const unsigned char* gt = qt + S::TILE;
    const float* stl = reinterpret_cast<const float*>(qt + T::STAT);

    if constexpr (D == 128) {
      // One wave per SIMD: the step's two 32-query chunks are software-
      // pipelined so that the vector work of one chunk issues beside the
      // MFMAs of the other:
      //   S, dP of chunk 0;  S, dP of chunk 1 | P, dS of chunk 0;
      //   dV, dK of chunk 0 | P, dS of chunk 1;  dV, dK of chunk 1.
      // Each MFMA step takes one pair of P and dS values (packed to bf16 as
      // the serial loop packs them); the packed words are pinned per step, so
      // that the compiler does not sink the exponentials to their first use.
      float4 l4[2][4], d4[2][4];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          l4[c][g] = *reinterpret_cast<const float4*>(stl + 32 * c + 8 * g + 4 * h2);
          d4[c][g] = *reinterpret_cast<const float4*>(stl + 64 + 32 * c + 8 * g + 4 * h2);
        }
      auto comp = [](const float4& v, int i) __attribute__((always_inline)) {
        return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
      };
      f32x16 sc[2], dp[2];
      u32x4 pw[2][2], dw[2][2];               // P and dS of each chunk, bf16 pairs (B operands)
      auto mask_chunk = [&](int c) __attribute__((always_inline)) {
        if (!masked) return;
        const unsigned ubase = static_cast<unsigned>(row0 + 32 * c + 4 * h2 - qlo);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned u = ubase + 8 * (r >> 2) + (r & 3);
          sc[c][r] = u >= static_cast<unsigned>(qwidth) ? -INFINITY : sc[c][r];
        }
      };
      // P and dS of chunk c, values r = 2 i, 2 i + 1
      auto soft_pair = [&](int c, int i) __attribute__((always_inline)) {
        float pr[2], ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          pr[e] = __builtin_amdgcn_exp2f(sc[c][r] - comp(l4[c][r >> 2], r & 3));
          ds[e] = pr[e] * (dp[c][r] - comp(d4[c][r >> 2], r & 3));
        }
        uint32_t wp = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)pr[0], (__bf16)pr[1]});
        uint32_t wd = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)ds[0], (__bf16)ds[1]});
        __asm__ volatile("" : "+v"(wp), "+v"(wd));
        pw[c][i >> 2][i & 3] = wp;
        dw[c][i >> 2][i & 3] = wd;
      };
      auto bop = [](const u32x4& w) __attribute__((always_inline)) { return __builtin_bit_cast(bf16x8, w); };

      // The step as 32 operations of two MFMAs each: S, dP of chunk 0 (ks 0..7),
      // of chunk 1, then dV, dK of chunk 0 ((t2, dt) pairs), of chunk 1.  Each
      // operation's two LDS fragments are read kAhead operations before it.
      constexpr int kOps = 4 * S::KS;
      static_assert(2 * S::DT == S::KS, "dV/dK operations per chunk match S/dP ones at d = 128");
      constexpr int kAhead = 3;
      auto frags = [&](int j, bf16x8 (&f)[2]) __attribute__((always_inline)) {
        if (j < 2 * S::KS) {
          const int c = j / S::KS, ks = j % S::KS;
          f[0] = row_frag<D>(qt, roffs[ks], c);
          f[1] = row_frag<D>(gt, roffs[ks], c);
        } else {
          const int c = (j - 2 * S::KS) / S::KS, st = (j - 2 * S::KS) % S::KS;
          const int t2 = st / S::DT, dt = st % S::DT;
          f[0] = tr_frag<D>(gt, toff[dt][0], toff[dt][1], 2 * c + t2);
          f[1] = tr_frag<D>(qt, toff[dt][0], toff[dt][1], 2 * c + t2);
        }
      };
      bf16x8 fr[kOps][2];
#pragma unroll
      for (int j = 0; j < kAhead; ++j) frags(j, fr[j]);
      sc[0] = f32x16{};
      dp[0] = f32x16{};
      sc[1] = f32x16{};
      dp[1] = f32x16{};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kOps; ++j) {
        if (j == S::KS) {
          mask_chunk(0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (j == 2 * S::KS) {
          mask_chunk(1);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (j + kAhead < kOps) frags(j + kAhead, fr[j + kAhead]);
        if (j < 2 * S::KS) {
          const int c = j / S::KS, ks = j % S::KS;
          sc[c] = mfma32(fr[j][0], kf[ks], sc[c]);
          if (c == 1) soft_pair(0, ks);
          dp[c] = mfma32(fr[j][1], vf[ks], dp[c]);
        } else {
          const int c = (j - 2 * S::KS) / S::KS, st = (j - 2 * S::KS) % S::KS;
          const int t2 = st / S::DT, dt = st % S::DT;
          dv[dt] = mfma32(fr[j][0], bop(pw[c][t2]), dv[dt]);
          if (c == 0) soft_pair(1, st);
          dk[dt] = mfma32(fr[j][1], bop(dw[c][t2]), dk[dt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
  #pragma unroll
      for (int c = 0; c < 2; ++c) {  // 32-query chunks
        // S = Qs K^T (log2 units), dP = dO V^T (rows: queries 32c .. +31; columns: the wave's keys)
        f32x16 sc = f32x16{}, dp = f32x16{};
  #pragma unroll
        for (int ks = 0; ks < S::KS; ++ks) {
          sc = mfma32(row_frag<D>(qt, roffs[ks], c), kf[ks], sc);
          dp = mfma32(row_frag<D>(gt, roffs[ks], c), vf[ks], dp);
        }
        // row r of the block is query 32c + 8 (r/4) + 4 h2 + r%4 of the step
        float4 l4[4], d4[4];
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          l4[g] = *reinterpret_cast<const float4*>(stl + 32 * c + 8 * g + 4 * h2);
          d4[g] = *reinterpret_cast<const float4*>(stl + 64 + 32 * c + 8 * g + 4 * h2);
        }
        if (masked) {
          const unsigned ubase = static_cast<unsigned>(row0 + 32 * c + 4 * h2 - qlo);
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned u = ubase + 8 * (r >> 2) + (r & 3);
            sc[r] = u >= static_cast<unsigned>(qwidth) ? -INFINITY : sc[r];
          }
        }
        bf16x8 pb[2], dsb[2];
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float4& L4 = l4[r >> 2];
          const float4& D4 = d4[r >> 2];
          const float lr = (r & 3) == 0 ? L4.x : (r & 3) == 1 ? L4.y : (r & 3) == 2 ? L4.z : L4.w;
          const float dr = (r & 3) == 0 ? D4.x : (r & 3) == 1 ? D4.y : (r & 3) == 2 ? D4.z : D4.w;
          const float pr = __builtin_amdgcn_exp2f(sc[r] - lr);
          pb[r >> 3][r & 7] = (__bf16)pr;
          dsb[r >> 3][r & 7] = (__bf16)(pr * (dp[r] - dr));
        }
        // dV^T += dO^T P, dK^T += Q^T dS (K dimension: 16-query steps 2c, 2c+1),
        // at raised priority when two waves share a SIMD (as in the dQ kernel)
        if constexpr (D != 128) {
          __builtin_amdgcn_s_setprio(1);
          __builtin_amdgcn_sched_barrier(0);
        }
  #pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
  #pragma unroll
          for (int dt = 0; dt < S::DT; ++dt) {
            dv[dt] = mfma32(tr_frag<D>(gt, toff[dt][0], toff[dt][1], 2 * c + t2), pb[t2], dv[dt]);
            dk[dt] = mfma32(tr_frag<D>(qt, toff[dt][0], toff[dt][1], 2 * c + t2), dsb[t2], dk[dt]);
          }
        }
        if constexpr (D != 128) {
          __builtin_amdgcn_s_setprio(0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (s == 1) {
      ent_cur = __builtin_amdgcn_readfirstlane(ent_nxt);
      const int next = (k + 1) / 2 + 1;  // entry index of the step after next tile
      ent_nxt = (c_begin + next < c_end) ? p.col[c_begin + next] : 0;
    }
  }
  if (npieces > 1) {  // this piece's dK^T and dV^T sums (dK then dV, float4 [wave][dt][4][lane])
    float* sp = p.dkdv_partials + static_cast<int64_t>(slot) * dkdv_slot_floats(D);
    constexpr int kHalf = 4 * S::DT * 16 * 64;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int off = (((wave * S::DT + dt) * 4 + g) * 64 + lane) * 4;
        *reinterpret_cast<float4*>(sp + off) = make_float4(dk[dt][4 * g], dk[dt][4 * g + 1], dk[dt][4 * g + 2], dk[dt][4 * g + 3]);
        *reinterpret_cast<float4*>(sp + kHalf + off) =
            make_float4(dv[dt][4 * g], dv[dt][4 * g + 1], dv[dt][4 * g + 2], dv[dt][4 * g + 3]);
      }
    }
    return;
  }
  if (kj < p.L) {
    unsigned char* dkr = reinterpret_cast<unsigned char*>(p.dk + b * p.dk_sb + hk * p.dk_sh) +
                         static_cast<int64_t>(kj) * p.dk_sl * 2;
    unsigned char* dvr = reinterpret_cast<unsigned char*>(p.dv + b * p.dv_sb + hk * p.dv_sh) +
                         static_cast<int64_t>(kj) * p.dv_sl * 2;
    store_rows<D>(dkr, dk, 1.f / kLog2e, h2);
    store_rows<D>(dvr, dv, 1.f, h2);
  }
}

// dK and dV of the split key blocks (batch 1): one work-group per split block
// adds its pieces' sums in piece order and writes dK = sum / log2(e) (the
// scores were recomputed from Q scaled by sigma log2(e)) and dV = sum.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_merge_kernel(const BwdParams p) {
  using S = Shape<D>;
  constexpr int kHalf = 4 * S::DT * 16 * 64;
  const int4 row = reinterpret_cast<const int4*>(p.kv_merge)[blockIdx.x];
  const int hk = __builtin_amdgcn_readfirstlane(row.x);
  const int kblk = __builtin_amdgcn_readfirstlane(row.y);
  const int slot0 = __builtin_amdgcn_readfirstlane(row.z);
  const int npieces = __builtin_amdgcn_readfirstlane(row.w);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5, l31 = lane & 31;
  for (int part = 0; part < 2; ++part) {  // dK, then dV
    f32x16 acc[S::DT];
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x16{};
    for (int i = 0; i < npieces; ++i) {
      const float* sp = p.dkdv_partials + static_cast<int64_t>(slot0 + i) * dkdv_slot_floats(D) + part * kHalf;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 a = *reinterpret_cast<const float4*>(sp + (((wave * S::DT + dt) * 4 + g) * 64 + lane) * 4);
          acc[dt][4 * g + 0] += a.x;
          acc[dt][4 * g + 1] += a.y;
          acc[dt][4 * g + 2] += a.z;
          acc[dt][4 * g + 3] += a.w;
        }
      }
    }
    const int kj = kblk * 2 * kBN + wave * 32 + l31;
    if (kj < p.L) {
      uint16_t* base = part == 0 ? p.dk + hk * p.dk_sh : p.dv + hk * p.dv_sh;
      const int64_t sl = part == 0 ? p.dk_sl : p.dv_sl;
      unsigned char* dst = reinterpret_cast<unsigned char*>(base) + static_cast<int64_t>(kj) * sl * 2;
      store_rows<D>(dst, acc, part == 0 ? 1.f / kLog2e : 1.f, h2);
    }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, int B, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const bool prefix = p.prefix > 0;
  const bool sink = p.dsink != nullptr;
  hipExtLaunchKernelGGL((bwd_prep_kernel<D>), dim3(p.nq, p.H, B), dim3(256), 0, stream, start, nullptr, 0, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gq(static_cast<unsigned>(8 * p.q_queue), static_cast<unsigned>(B));
  if (prefix) hipLaunchKernelGGL((bwd_dq_kernel<D, true>), gq, dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL((bwd_dq_kernel<D, false>), gq, dim3(kThreads), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.n_merge > 0) {  // batch 1 only: the split rows' dQ
    hipLaunchKernelGGL((bwd_dq_merge_kernel<D>), dim3(static_cast<unsigned>(p.n_merge)), dim3(kThreads), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 gk(static_cast<unsigned>(8 * p.kv_queue), static_cast<unsigned>(B));
  const bool kv_merge = p.n_kv_merge > 0;
  hipEvent_t last_stop = (sink || kv_merge) ? nullptr : stop;
  if (prefix) hipExtLaunchKernelGGL((bwd_dkdv_kernel<D, true>), gk, dim3(kThreads), 0, stream, nullptr, last_stop, 0, p);
  else hipExtLaunchKernelGGL((bwd_dkdv_kernel<D, false>), gk, dim3(kThreads), 0, stream, nullptr, last_stop, 0, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (kv_merge) {  // batch 1 only: the split key blocks' dK and dV
    hipExtLaunchKernelGGL((bwd_dkdv_merge_kernel<D>), dim3(static_cast<unsigned>(p.n_kv_merge)), dim3(kThreads), 0,
                          stream, nullptr, sink ? nullptr : stop, 0, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (sink) {
    hipExtLaunchKernelGGL(bwd_sink_kernel, dim3(p.H), dim3(256), 0, stream, nullptr, stop, 0, p, B);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int D, int B, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  switch (D) {
    case 64: return launch_bwd_d<64>(p, B, stream, start, stop);
    case 80: return launch_bwd_d<80>(p, B, stream, start, stop);
    case 128: return launch_bwd_d<128>(p, B, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bss
