// One-query (decode) attention with a sliding window, prefix tokens and a sink,
// for gfx950 (MI355X).
//
// Generation reads one new query per sequence against its key/value cache.
// The sliding-window-vs-linear-attention article decodes with a causal window
// of the last W cached tokens, either with a learned per-head sink logit in
// the denominator or with the first few tokens kept as StreamingLLM sink
// tokens (its "comparison at equal memory" section: 576 tokens, or 572 + 4),
// on grouped-query heads (32 query heads on 8 key/value heads, head dim 128;
// its speed test uses 16 on 4 at head dim 256).  The query is the last token
// t = n - 1 of a sequence of n cached tokens; its allowed keys are the window
// [n - W, n) and the prefix [0, P) (the same sets the prefill masks give row
// t), and the softmax is the exact masked softmax with the sink in the
// denominator ("Semantic Head Specialization ...", the sink-bias slide).
//
// The work is memory-bound: every cached K/V row in the window is read once
// and multiplied by the few query heads that share it.  Layout:
//   * one work-group per (key split, K/V head, sequence).  The allowed keys
//     form one virtual list (the prefix keys not already in the window, then
//     the window); split s takes keys [s C, s C + C) of it.  A split count of
//     1 writes O directly; otherwise every split writes its partial state
//     (unnormalised output, reference, denominator) and decode_combine merges
//     them in split order with the sink.
//   * K and V tiles of 64 keys go global -> LDS with global_load_lds_dwordx4
//     (per-lane row addresses follow the virtual list) into two buffers, two
//     tiles in flight: tile t+2 is issued as soon as every wave is done with
//     tile t, so a work-group waits on one tile while the next is already on
//     its way.  LDS rows carry one 16-byte pad chunk so that the fragment
//     reads below fall in distinct banks.
//   * wave w takes keys 16w .. 16w+15 of each tile.  S^T = K Q^T on
//     v_mfma_f32_16x16x32_bf16: K rows from LDS (A operand), the group's
//     query heads as the 16 columns of B (zero columns past the group), so
//     lane l holds query column l mod 16 and 4 keys.  O^T += V^T P^T on
//     v_mfma_f32_16x16x16_bf16: P^T is already that lane layout, V^T comes
//     from LDS with the transposed read ds_read_b64_tr_b16.
//   * online softmax per wave in log2 units (Q pre-scaled by scale log2(e));
//     the four waves' states merge through LDS at the end.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"
#include "tile_common.hpp"

namespace bss {
namespace {

using namespace dev;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecTile = 64;  // keys per K/V tile
constexpr float kNegInf = -INFINITY;

template <int D>
struct DecShape {
  static constexpr int CPR = D / 8;              // 16-byte chunks of a token row
  static constexpr int SPR = CPR + 1;            // LDS slots per row (one pad chunk)
  static constexpr int LRB = SPR * 16;           // LDS bytes per row
  static constexpr int TILE = kDecTile * LRB;    // one K or V tile
  static constexpr int KS = D / 32;              // k-steps of S^T = K Q^T
  static constexpr int DT = D / 16;              // 16-row tiles of O^T
  static constexpr int STATE = 4 * 16 * (D + 2) * 4;  // the waves' final states (floats)
  static_assert(STATE <= 4 * TILE, "wave states must fit in the K/V buffers");
};

// Value pairs across lanes l and l^16 (v_permlane16_swap) or l and l^32.
__device__ __forceinline__ float pair16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (N < 64: the gfx9 vmcnt field is bits 3:0 and 15:14; expcnt and lgkmcnt
// are left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// exp2 of a difference where a -inf first argument gives 0 (and -inf - -inf is not formed).
__device__ __forceinline__ float exp2_rel(float m, float ref) {
  return m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - ref);
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeParams p) {
  using S = DecShape<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * S::TILE];  // [buf][K, V][row][LRB]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;      // 16-lane group
  const int col = lane & 15;    // query column of S^T / O^T
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;

  // ---- the allowed keys of this sequence as one virtual list ----
  const int n = min(max(p.seq_lens[b], 0), p.max_len);         // cached tokens; the query is token n - 1
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;       // window [lo, n)
  const int pre = min(min(p.prefix, n), lo);                    // prefix keys outside the window
  const int nk = pre + (n - lo);
  const int v0 = split * p.chunk;
  const int v1 = min(nk, v0 + p.chunk);
  const int ntiles = v1 > v0 ? (v1 - v0 + kDecTile - 1) / kDecTile : 0;
  auto key_of = [&](int vi) __attribute__((always_inline)) { return vi < pre ? vi : lo + (vi - pre); };

  // ---- query columns: head kvh * G + col, pre-scaled by scale * log2(e), bf16 ----
  bf16x8 qf[S::KS];
  {
    const bool live = col < p.G;
    const uint16_t* qrow = p.q + b * p.q_sb + (kvh * p.G + (live ? col : 0)) * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = live ? (__bf16)((float)raw[e] * p.scale_log2) : (__bf16)0.f;
    }
  }

  const uint64_t kbase = uniform_u64(reinterpret_cast<uint64_t>(p.k + b * p.k_sb + kvh * p.k_sh));
  const uint64_t vbase = uniform_u64(reinterpret_cast<uint64_t>(p.v + b * p.v_sb + kvh * p.v_sh));
  const uint32_t k_row_bytes = static_cast<uint32_t>(p.k_sl * 2), v_row_bytes = static_cast<uint32_t>(p.v_sl * 2);
  const uint32_t smem_lds = lds_addr(smem);

  // Issue tile t into buffer buf: 2 * SPR wave-instructions (K then V), dealt
  // to the waves round-robin; instruction i fills LDS slots 64 (i mod SPR) ..
  // +63 of its tensor.  Rows past the split's end re-read its last key (their
  // scores are masked); pad slots re-read chunk 0 of their row.
  auto issue = [&](int t, int buf) __attribute__((always_inline)) {
    const int row0 = v0 + t * kDecTile;
    for (int i = wave; i < 2 * S::SPR; i += 4) {
      const int tensor = i >= S::SPR ? 1 : 0;
      const int ii = i - tensor * S::SPR;
      const int slot = ii * 64 + lane;
      const int row = slot / S::SPR, c = slot % S::SPR;
      const int vi = min(row0 + row, v1 - 1);
      const uint32_t off = static_cast<uint32_t>(key_of(vi)) * (tensor ? v_row_bytes : k_row_bytes) +
                           static_cast<uint32_t>(c < S::CPR ? c : 0) * 16u;
      const uint32_t dst = static_cast<uint32_t>(
          __builtin_amdgcn_readfirstlane(static_cast<int>(smem_lds + (2 * buf + tensor) * S::TILE + ii * 1024)));
      dma16(tensor ? vbase : kbase, off, dst);
    }
  };

  // ---- per-wave online softmax state (log2 units) ----
  float m_run = kNegInf, l_run = 0.f;   // reference and this lane's share of the denominator
  f32x4 acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS offsets: K fragment row 16 wave + col, chunk 4 ks + g; V^T transposed
  // read: lane (j, c) of group g points at row 16 wave + 4 g + j, columns 4c .. 4c+3 of each 16-column block.
  const int k_off = (16 * wave + col) * S::LRB + 16 * g;
  const int v_off = (16 * wave + 4 * g + (col >> 2)) * S::LRB + 8 * (col & 3);

  // DMA instructions this wave issues per tile (instructions i = wave, wave + 4, ... < 2 SPR)
  constexpr int kLoadsHi = (2 * S::SPR + 3) / 4, kLoadsLo = (2 * S::SPR) / 4;
  const bool loads_hi = (2 * S::SPR - wave + 3) / 4 == kLoadsHi;
  if (ntiles > 0) issue(0, 0);
  if (ntiles > 1) issue(1, 1);
  for (int t = 0; t < ntiles; ++t) {
    // this wave's part of tile t (tile t+1's loads, issued later, may stay in flight)
    if (t + 1 < ntiles) {
      if (loads_hi) wait_vm<kLoadsHi>();
      else wait_vm<kLoadsLo>();
    } else {
      wait_vm<0>();
    }
    wg_barrier();      // every wave's part of tile t has landed
    const unsigned char* kt = smem + (2 * (t & 1)) * S::TILE;
    const unsigned char* vt = kt + S::TILE;

    // S^T for this wave's 16 keys x 16 query columns
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + k_off + 64 * ks);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], s, 0, 0, 0);
    }
    // keys 16 wave + 4 g + e of the tile; past the split's end -> -inf
    const int first = v0 + t * kDecTile + 16 * wave + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = (first + e < v1) ? s[e] : kNegInf;
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mt = halves_max(pair16_max(mt));              // over the wave's 16 keys of this column
    const float m_new = fmaxf(m_run, mt);
    const float ref = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_rel(m_run, ref);
    s16x4 pb;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pe = __builtin_amdgcn_exp2f(s[e] - ref);   // exp2(-inf) = 0
      ps += pe;
      pb[e] = __builtin_bit_cast(short, (__bf16)pe);
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
      acc[dt] *= alpha;
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vt + v_off + 32 * dt));
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[dt], 0, 0, 0);
    }
    if (t + 2 < ntiles) {
      wg_barrier();    // every wave is done with buffer t & 1
      issue(t + 2, t & 1);
    }
  }

  // ---- merge the four waves' states through LDS ----
  const float l_col = halves_sum(pair16_sum(l_run));   // the column's denominator over the wave's keys
  __syncthreads();                                      // K/V buffers are free
  float* st = reinterpret_cast<float*>(smem);           // [wave][col][D + 2]: acc[0..D), m, l
  float* mine = st + (wave * 16 + col) * (D + 2);
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mine[16 * dt + 4 * g + e] = acc[dt][e];
  if (g == 0) {
    mine[D] = m_run;
    mine[D + 1] = l_col;
  }
  __syncthreads();

  const int hq0 = kvh * p.G;
  for (int idx = threadIdx.x; idx < p.G * D; idx += kThreads) {
    const int c = idx / D, d = idx - c * D;
    float mw[4], M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = st[(w * 16 + c) * (D + 2) + D];
      M = fmaxf(M, mw[w]);
    }
    float A = 0.f, Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2_rel(mw[w], M);
      A += f * st[(w * 16 + c) * (D + 2) + d];
      Lsum += f * st[(w * 16 + c) * (D + 2) + D + 1];
    }
    if (M == kNegInf) A = Lsum = 0.f;
    const int hq = hq0 + c;
    if (p.nsplit == 1) {
      const float sl = p.sink ? p.sink[hq] * kLog2e : kNegInf;
      const float M2 = fmaxf(M, sl);
      float out = 0.f;
      if (M2 != kNegInf) {
        const float f = exp2_rel(M, M2);
        const float den = Lsum * f + exp2_rel(sl, M2);
        out = den > 0.f ? A * f / den : 0.f;
      }
      p.o[b * p.o_sb + hq * p.o_sh + d] = __builtin_bit_cast(uint16_t, (__bf16)out);
    } else {
      float* part = p.partials + ((static_cast<int64_t>(b) * p.H + hq) * p.nsplit + split) * (D + 2);
      part[d] = A;
      if (d == 0) {
        part[D] = M;
        part[D + 1] = Lsum;
      }
    }
  }
}

// Merge the splits of one (sequence, query head) with the sink.  The split
// references and denominators are staged in LDS with their weights
// 2^(m_s - M); thread (d, r) of the 256 sums the weighted partial outputs of
// element d over splits r, r + R, ... (R = 256 / D), and the R partial sums
// are added in a fixed order, so the result does not depend on timing.
constexpr int kMaxSplits = 4096;
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeParams p, int D) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[256];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int ns = p.nsplit;
  const float* part = p.partials + (static_cast<int64_t>(b) * p.H + hq) * ns * (D + 2);
  const float sl = p.sink ? p.sink[hq] * kLog2e : kNegInf;
  float mx = sl;
  for (int s = tid; s < ns; s += 256) {
    const float m = part[s * (D + 2) + D];
    wgt[s] = m;
    mx = fmaxf(mx, m);
  }
  red[tid] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float lsum = 0.f;
  for (int s = tid; s < ns; s += 256) {
    const float f = (M == kNegInf) ? 0.f : exp2_rel(wgt[s], M);
    wgt[s] = f;
    lsum += f * part[s * (D + 2) + D + 1];
  }
  red[tid] = lsum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float den = red[0] + ((M == kNegInf) ? 0.f : exp2_rel(sl, M));
  __syncthreads();
  const int R = 256 / D;                 // D in {64, 128, 256}
  const int d = tid % D, r = tid / D;
  float a = 0.f;
#pragma unroll 8
  for (int s = r; s < ns; s += R) a += wgt[s] * part[s * (D + 2) + d];
  red[tid] = a;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
    for (int j = 0; j < R; ++j) acc += red[j * D + tid];
    const float out = den > 0.f ? acc / den : 0.f;
    p.o[b * p.o_sb + hq * p.o_sh + tid] = __builtin_bit_cast(uint16_t, (__bf16)out);
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const dim3 grid(static_cast<unsigned>(p.nsplit), static_cast<unsigned>(p.H / p.G), static_cast<unsigned>(p.B));
  if (p.nsplit == 1) {
    hipExtLaunchKernelGGL(decode_kernel<D>, grid, dim3(kThreads), 0, stream, start, stop, 0, p);
    return hipGetLastError();
  }
  hipExtLaunchKernelGGL(decode_kernel<D>, grid, dim3(kThreads), 0, stream, start, nullptr, 0, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipExtLaunchKernelGGL(decode_combine_kernel, dim3(static_cast<unsigned>(p.H), static_cast<unsigned>(p.B)),
                        dim3(256), 0, stream, nullptr, stop, 0, p, D);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int D, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  switch (D) {
    case 64: return launch_decode_d<64>(p, stream, start, stop);
    case 128: return launch_decode_d<128>(p, stream, start, stop);
    case 256: return launch_decode_d<256>(p, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bss
