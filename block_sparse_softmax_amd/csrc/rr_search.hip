// RRAttention's block-pattern search for gfx950 ("RRAttention", section 3):
// from Q and K to the block-selection matrix B that the masked forward kernel
// consumes as its block mask.
//
//   prep    sampled queries q_P(i,h), P(i,h) = iS + (S - 1 - (h mod S)) (Eq. 6-7),
//           and stride-summed keys sum_{k=jS}^{(j+1)S-1} k_k (Eq. 8), into
//           contiguous bf16 rows of the workspace.  A stride sum is formed in
//           fp32 and kept as two bf16 halves, hi = bf16(sum) and
//           lo = bf16(sum - hi), whose sum is the fp32 sum to about 2^-16
//           relative: the importance GEMM then runs on the matrix cores with
//           the key aggregate at fp32 accuracy (hi and lo are two k-ranges of
//           one product against the same query fragments).
//   kmax    the largest norm of the head's key aggregates.
//   scores  the stride importance I = q . ksum / (S sqrt(d)) (Eq. 8) on
//           v_mfma_f32_32x32x16_bf16, in ONE pass over the causal key
//           strides j <= i: each row's probabilities are taken against a
//           fixed reference r >= every I of the row (|q| |ksum|max, Cauchy-
//           Schwarz), so the pass sums 2^(I - r) per (row, key block) and per
//           row without knowing the row's max; the per-block sums go to the
//           workspace (the stride-level matrix never exists), and once a
//           wave's rows are done it reads its own sums back and writes
//           S_mn = sum over the rows i of block m of u_in / l_i (Eq. 9-10).
//   recompute  rows whose sum against r underflows (r far above the row's
//           max: keys with large norms orthogonal to the query) are redone,
//           per query tile, by the two-pass kernel: pass 1 keeps each row's
//           running max and sum, pass 2 recomputes I, normalises and sums
//           the probabilities into block scores.
//   select  per query block m: of S_m,n (n <= m) ordered descending (ties to
//           the lower n), keep the shortest prefix whose mass reaches tau
//           times the row's mass (Eq. 11), found by a threshold search rather
//           than a sort, and every causal block of the last query block
//           (Eq. 12).
//
// Layout of the two-pass scores kernel: a work-group of 4 waves takes 128
// consecutive sampled queries of one (batch, head); wave w owns queries
// 32w..32w+31 of them.  The stride-summed keys are staged in LDS 64 at a
// time, up to three stages in flight, shared by the 4 waves, and used in
// chunks of 32.  I^T = Ksum Q^T: the key chunk is the A operand (from LDS),
// the sampled queries the B operand (in registers), so lane l holds query
// l mod 32 and 16 of the chunk's 32 key strides.  The single pass uses the
// same staging with 256 queries per work-group (two sets of 32 per wave).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "kernels.hpp"
#include "tile_common.hpp"

namespace bss {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRrThreads = 256;
constexpr int kRrQ = 128;     // sampled queries per work-group
constexpr int kChunk = 32;    // key strides per chunk

// Sum of v over the lanes l ^ x for every x < n (n = 8, 16 or 32: the lanes
// of an aligned group of n), all holding the total: DPP quad and row-mirror
// steps inside a 16-lane row, a row swap (v_permlane16_swap) for n = 32.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);   // row_half_mirror: the other quad of each 8 lanes
  if constexpr (N >= 16) v += dpp_mov<0x140>(v);  // row_mirror: the other 8 lanes of the row
  if constexpr (N >= 32) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// Sum of v over lanes l and l ^ 32.
__device__ __forceinline__ float halves_sum32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- prep ----
// One thread per (batch, head, stride row of the padded table, 8-dim chunk),
// a row's chunks on P lanes in a row (P = D / 8 rounded up to a power of two;
// lanes past D / 8 only join the norm's reduction).
// A stride-summed key row holds hi (D bf16) then lo (D bf16); rows are
// 4 D + 16 bytes apart (the last 16 bytes are never written or read): a run
// of rows is then byte for byte the padded LDS layout of the scores kernel
// and is copied with LDS-DMA as it is.  The row's |hi + lo|^2 (the aggregate
// the products see) is summed over its lanes and stored once per row.
template <int P>
__global__ __launch_bounds__(256) void rr_prep_kernel(const RrParams p) {
  const int cpr = p.D / 8;
  const int64_t n = static_cast<int64_t>(p.B) * p.H * p.ns_pad * P;   // a multiple of 64: whole waves
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int c = static_cast<int>(t % P);
  const int64_t row = t / P;
  const int j = static_cast<int>(row % p.ns_pad);
  const int bh = static_cast<int>(row / p.ns_pad);
  const int h = bh % p.H, b = bh / p.H;
  bf16x8 qo = {}, ko = {}, kl = {};
  float n2 = 0.f;
  if (j < p.ns && c < cpr) {
    const int pos = j * p.S + (p.S - 1 - (h % p.S));
    qo = *reinterpret_cast<const bf16x8*>(p.q + b * p.q_sb + static_cast<int64_t>(pos) * p.q_sl + h * p.q_sh + 8 * c);
    float acc[8] = {};
    const uint16_t* kr = p.k + b * p.k_sb + static_cast<int64_t>(j) * p.S * p.k_sl + (h / p.kv_group) * p.k_sh + 8 * c;
    // the stride's rows in batches of 8 loads issued together (one round trip
    // per batch instead of one per row); the sum stays in row order
    for (int s0 = 0; s0 < p.S; s0 += 8) {
      bf16x8 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        x[u] = *reinterpret_cast<const bf16x8*>(kr + static_cast<int64_t>(min(s0 + u, p.S - 1)) * p.k_sl);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u < p.S) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += static_cast<float>(x[u][e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ko[e] = static_cast<__bf16>(acc[e]);
      kl[e] = static_cast<__bf16>(acc[e] - static_cast<float>(ko[e]));  // the difference is exact in fp32
      const float x = static_cast<float>(ko[e]) + static_cast<float>(kl[e]);
      n2 = __builtin_fmaf(x, x, n2);
    }
  }
#pragma unroll
  for (int off = 1; off < P; off <<= 1) n2 += __shfl_xor(n2, off);
  if (c == 0) p.knorm2[row] = n2;
  if (c < cpr) {
    *reinterpret_cast<bf16x8*>(p.qs + row * p.D + 8 * c) = qo;
    uint16_t* kdst = p.ks + row * (2 * p.D + 8);                     // rows of 4 D + 16 bytes
    *reinterpret_cast<bf16x8*>(kdst + 8 * c) = ko;
    *reinterpret_cast<bf16x8*>(kdst + p.D + 8 * c) = kl;
  }
}

// -------------------------------------------------------------- scores ----
// R = block size / stride (strides per block): 8, 16 or 32.
template <int D, int R>
__global__ __launch_bounds__(kRrThreads) void rr_scores_kernel(const RrParams p) {
  constexpr int KS = D / 16;                 // k-steps of the 32x32x16 product per key half (hi, lo)
  constexpr int PITCH = 4 * D + 16;          // row pitch (table and LDS): 16 rows of a fragment read hit distinct banks
  constexpr int CPR = D / 8;                 // 16-byte pieces per query row
  constexpr int STAGE = 2 * kChunk;          // key strides per copy stage
  constexpr int SBYTES = STAGE * PITCH;      // bytes of one stage
  constexpr int NI = SBYTES / 1024;          // LDS-DMA wave-instructions per stage (wave w takes w, w + 4, ...)
  constexpr int NW_HI = (NI + 3) / 4, NW_LO = NI / 4;
  // stages in LDS: three (two in flight during compute) where two work-groups
  // still fit per CU, else two (one in flight)
  constexpr int NBUF = (3 * SBYTES <= 80 * 1024) ? 3 : 2;
  constexpr int AHEAD = NBUF - 1;            // stages issued ahead of the one computed
  static_assert(SBYTES % 1024 == 0, "a stage is whole 1 KiB copies");
  static_assert(NW_HI < 16, "vmcnt immediate");
  static_assert(R == 8 || R == 16 || R == 32, "strides per block");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NBUF * SBYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = p.ns_pad / kRrQ;
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.x);  // longest (latest) tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh_row = (static_cast<int64_t>(b) * p.H + h) * p.ns_pad;
  const bf16x8* qs = reinterpret_cast<const bf16x8*>(p.qs) + bh_row * CPR;
  const unsigned char* ksb = reinterpret_cast<const unsigned char*>(p.ks) + bh_row * PITCH;

  if (p.gate && p.flags[(static_cast<int64_t>(b) * p.H + h) * n_tiles + tile] == 0) return;  // whole work-group
  const int q0 = tile * kRrQ + 32 * wave;    // this wave's first sampled query
  const int qi = q0 + (lane & 31);           // this lane's query (column of I^T)
  const int half = lane >> 5;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = qs[static_cast<int64_t>(qi) * CPR + 2 * s + half];

  const int last_chunk_wg = (tile * kRrQ + kRrQ - 1) / kChunk;  // chunks the work-group stages
  const int last_chunk = q0 / kChunk;                            // chunks this wave computes
  const int n_chunks = last_chunk_wg + 1;                        // a multiple of 4
  const int n_stage = n_chunks / 2;

  // Stage s (key strides 64 s .. 64 s + 63, contiguous in the table) into
  // buffer s mod 3: wave w issues 1 KiB copies w, w + 4, ... of it.
  const uint32_t smem_lds = dev::lds_addr(smem);
  const int nw = (NI - wave + 3) / 4;        // copies per stage issued by this wave
  auto issue_stage = [&](int st) __attribute__((always_inline)) {
    const uint64_t src = dev::uniform_u64(reinterpret_cast<uint64_t>(ksb) + static_cast<uint64_t>(st) * SBYTES);
    const uint32_t dst = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
        static_cast<int>(smem_lds + (st % NBUF) * SBYTES)));
#pragma unroll
    for (int i = 0; i < NW_HI; ++i) {
      const int ins = wave + 4 * i;
      if (ins < NI) dev::dma16(src + static_cast<uint64_t>(ins) * 1024, 16 * lane, dst + ins * 1024);
    }
  };
  // Wait for this wave's copies of stage st when the copies of stage st + 1
  // (issued after them) may stay in flight (three buffers only); global
  // stores issued in between only make the wait longer, never shorter.
  auto wait_stage = [&](bool next_in_flight) __attribute__((always_inline)) {
    if (!next_in_flight) dev::wait_vmcnt<0>();
    else if (nw == NW_HI) dev::wait_vmcnt<NW_HI>();
    else dev::wait_vmcnt<NW_LO>();
  };
  // I^T tile of chunk c (half `sub` of the stage in buffer buf): lane holds
  // key strides c*32 + 8g + 4*half + e (register 4g + e).  k-steps 0..KS-1
  // take the hi halves of the key rows, KS..2KS-1 the lo halves, both against
  // the same query fragments.
  auto chunk_scores = [&](int buf, int sub) __attribute__((always_inline)) {
    f32x16 acc = {};
    const unsigned char* base = smem + buf * SBYTES + (sub * kChunk + (lane & 31)) * PITCH + half * 16;
#pragma unroll
    for (int s = 0; s < 2 * KS; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(base + 32 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s % KS], acc, 0, 0, 0);
    }
    return acc;
  };
  auto key_of = [&](int c, int r) __attribute__((always_inline)) { return c * kChunk + 8 * (r >> 2) + 4 * half + (r & 3); };
  const bool q_valid = qi < p.ns;

  // ---- pass 1: per-lane running max and sum (log2 domain) over its key strides ----
  float m_run = -INFINITY, l_run = 0.f;
  // ---- pass 2 state: this lane's query's max and sum (both halves combined) ----
  float m_row = 0.f, inv_l = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    issue_stage(0);
    if (AHEAD > 1 && n_stage > 1) issue_stage(1);
    for (int st = 0; st < n_stage; ++st) {
      wait_stage(AHEAD > 1 && st + 1 < n_stage);
      __syncthreads();                         // stage st everywhere; stage st - 1 no longer read
      if (st + AHEAD < n_stage) issue_stage(st + AHEAD);  // into the buffer of stage st - 1
      const int buf = st % NBUF;
      // both chunks' products first: the softmax work of the first runs
      // beside the MFMAs of the second
      f32x16 accs[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
        if (2 * st + sub <= last_chunk) accs[sub] = chunk_scores(buf, sub);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int c = 2 * st + sub;
        if (c <= last_chunk) {
          const f32x16& acc = accs[sub];
          // below the wave's diagonal sub-chunk every key stride precedes every
          // query of the wave: no causal test (and no padded query: q0 + 31 < ns)
          const bool open = c < last_chunk && q0 + 31 < p.ns;
          if (pass == 0 && open) {
            float mx = fmaxf(acc[0], acc[1]);
  #pragma unroll
            for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(acc[r], acc[r + 1]));
            const float m_new = fmaxf(m_run, mx * p.scale_log2);
            float s = 0.f;
  #pragma unroll
            for (int r = 0; r < 16; ++r) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], p.scale_log2, -m_new));
            l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_new) + s;
            m_run = m_new;
          } else if (pass == 0) {
            float mx = -INFINITY;
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = key_of(c, r);
              if (q_valid && j <= qi) mx = fmaxf(mx, acc[r] * p.scale_log2);
            }
            const float m_new = fmaxf(m_run, mx);
            if (m_new > -INFINITY) {
              float s = 0.f;
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int j = key_of(c, r);
                if (q_valid && j <= qi) s += __builtin_amdgcn_exp2f(acc[r] * p.scale_log2 - m_new);
              }
              l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_new) + s;
              m_run = m_new;
            }
          } else {
            // probabilities of this lane's 16 key strides, summed per key block
            constexpr int KB = kChunk / R;     // key blocks in a chunk
            float bs[KB];
  #pragma unroll
            for (int kb = 0; kb < KB; ++kb) bs[kb] = 0.f;
            if (open) {
  #pragma unroll
              for (int r = 0; r < 16; ++r)
                bs[(8 * (r >> 2) + 4 * half + (r & 3)) / R] +=
                    __builtin_amdgcn_exp2f(acc[r] * p.scale_log2 - m_row) * inv_l;
            } else {
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int j = key_of(c, r);
                const float pr = (q_valid && j <= qi) ? __builtin_amdgcn_exp2f(acc[r] * p.scale_log2 - m_row) * inv_l : 0.f;
                bs[(8 * (r >> 2) + 4 * half + (r & 3)) / R] += pr;
              }
            }
            // sum over the lanes of each query block (R consecutive queries, both halves)
  #pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              const float v = halves_sum32(group_sum<R>(bs[kb]));
              const int qb_first = q0 + (lane & 31);     // first query of a block when lane % R == 0
              if (half == 0 && (lane % R) == 0 && qb_first < p.ns_pad) {
                const int qb = (q0 + (lane & 31)) / R;
                const int kblk = (c * kChunk) / R + kb;
                if (qb < p.nb && kblk < p.nb)
                  p.score[(static_cast<int64_t>(b) * p.H + h) * p.nb * p.nb + static_cast<int64_t>(qb) * p.nb + kblk] = v;
              }
            }
          }
        }
      }
    }
    __syncthreads();                           // the next pass restages buffers 0 and 1
    if (pass == 0) {
      // combine the two halves of each query: max and sum over all its key strides
      const float mo = __shfl_xor(m_run, 32), lo = __shfl_xor(l_run, 32);
      const float m = fmaxf(m_run, mo);
      const float l = (m == -INFINITY) ? 0.f
                                       : l_run * __builtin_amdgcn_exp2f(m_run - m) + lo * __builtin_amdgcn_exp2f(mo - m);
      m_row = (m == -INFINITY) ? 0.f : m;
      inv_l = l > 0.f ? 1.f / l : 0.f;
    }
  }
}

// ---------------------------------------------------------------- kmax ----
// One work-group of 1024 threads per (batch, head): the largest |hi + lo|
// over the head's rows (padding rows are 0), stored as the float's bits.
__global__ __launch_bounds__(1024) void rr_kmax_kernel(const RrParams p) {
  __shared__ float wmax[16];
  const int64_t bh = static_cast<int64_t>(blockIdx.y) * p.H + blockIdx.x;
  const float* n2 = p.knorm2 + bh * p.ns_pad;
  float m = 0.f;
  for (int r = threadIdx.x; r < p.ns_pad; r += 1024) m = fmaxf(m, n2[r]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float x = wmax[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) x = fmaxf(x, wmax[w]);
    p.kmax[bh] = __float_as_uint(__builtin_sqrtf(x));
  }
}

// ------------------------------------------------------ scores, one pass ----
// 256 sampled queries per work-group, 64 per wave as two sets of 32 (rows
// q0 .. q0+31 and q0+32 .. q0+63 of the wave): every K fragment read from LDS
// feeds one MFMA per set, so a staged 64-stride stage serves twice the
// products of the two-pass kernel's layout.  Key strides staged 64 at a time
// as there, chunks of 32.  Lane l's rows take the reference
// r_i = |q_i| kmax scale (1 + 2^-8): every computed I_ij scale is at most r_i
// (Cauchy-Schwarz, the products' and sums' rounding far inside the margin), so
// 2^(I_ij scale - r_i) <= 1 and the row's sum l_i and its per-key-block sums
// u_in can be accumulated against r_i from the first stride on.  u_in goes to
// the workspace ([key block][row], one coalesced 128-byte store per set and
// block); 1 / l_i too.  A row whose l_i is below 2^-40 (r_i more than
// 40 + log2 of its strides above its max) flags its 128-row query tile for
// the two-pass recompute.
constexpr int kRrQ1 = 256;    // sampled queries per work-group of the single pass
template <int D, int R>
__global__ __launch_bounds__(kRrThreads, 2) void rr_scores1p_kernel(const RrParams p) {
  constexpr int KS = D / 16;
  constexpr int PITCH = 4 * D + 16;
  constexpr int CPR = D / 8;
  constexpr int STAGE = 2 * kChunk;
  constexpr int SBYTES = STAGE * PITCH;
  constexpr int NI = SBYTES / 1024;
  constexpr int NW_HI = (NI + 3) / 4, NW_LO = NI / 4;
  constexpr int NBUF = (3 * SBYTES <= 80 * 1024) ? 3 : 2;
  constexpr int AHEAD = NBUF - 1;
  constexpr int KB = kChunk / R;             // key blocks in a chunk
  static_assert(SBYTES % 1024 == 0, "a stage is whole 1 KiB copies");
  static_assert(NW_HI < 16, "vmcnt immediate");
  static_assert(R == 8 || R == 16 || R == 32, "strides per block");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NBUF * SBYTES];
  __shared__ int bad_wave[4];
  __shared__ float linv_s[4][64];            // 1 / l of each wave's rows

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = p.ns_pad / kRrQ1;
  // one flat grid, tile-major: every head's longest (latest) tiles go first
  // and the short ones fill the tail
  const int nbh = p.B * p.H;
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.x) / nbh;
  const int64_t bh = static_cast<int>(blockIdx.x) % nbh;
  const int64_t bh_row = bh * p.ns_pad;
  const bf16x8* qs = reinterpret_cast<const bf16x8*>(p.qs) + bh_row * CPR;
  const unsigned char* ksb = reinterpret_cast<const unsigned char*>(p.ks) + bh_row * PITCH;

  const int q0 = tile * kRrQ1 + 64 * wave;   // this wave's first sampled query
  const int half = lane >> 5;
  const float kmx = __uint_as_float(p.kmax[bh]);
  int qi[2];
  bool q_valid[2];
  float rref[2];
  bf16x8 qf[2][KS];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    qi[g] = q0 + 32 * g + (lane & 31);
    q_valid[g] = qi[g] < p.ns;
    float qn2 = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[g][s] = qs[static_cast<int64_t>(qi[g]) * CPR + 2 * s + half];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qn2 = __builtin_fmaf(static_cast<float>(qf[g][s][e]), static_cast<float>(qf[g][s][e]), qn2);
    }
    qn2 = halves_sum32(qn2);                  // |q|^2 over both halves of the lane pair
    rref[g] = __builtin_sqrtf(qn2) * kmx * p.scale_log2 * (1.f + 0x1p-8f);
  }

  const int last_chunk_wg = (tile * kRrQ1 + kRrQ1 - 1) / kChunk;
  const int last0 = q0 / kChunk;              // set g's diagonal chunk is last0 + g
  const int n_chunks = last_chunk_wg + 1;     // a multiple of 8
  const int n_stage = n_chunks / 2;

  const uint32_t smem_lds = dev::lds_addr(smem);
  const int nw = (NI - wave + 3) / 4;
  auto issue_stage = [&](int st) __attribute__((always_inline)) {
    const uint64_t src = dev::uniform_u64(reinterpret_cast<uint64_t>(ksb) + static_cast<uint64_t>(st) * SBYTES);
    const uint32_t dst = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
        static_cast<int>(smem_lds + (st % NBUF) * SBYTES)));
#pragma unroll
    for (int i = 0; i < NW_HI; ++i) {
      const int ins = wave + 4 * i;
      if (ins < NI) dev::dma16(src + static_cast<uint64_t>(ins) * 1024, 16 * lane, dst + ins * 1024);
    }
  };
  auto wait_stage = [&](bool next_in_flight) __attribute__((always_inline)) {
    if (!next_in_flight) dev::wait_vmcnt<0>();
    else if (nw == NW_HI) dev::wait_vmcnt<NW_HI>();
    else dev::wait_vmcnt<NW_LO>();
  };
  // I^T tiles of chunk (buf, sub) for the sets that reach it (set 0 stops one chunk earlier)
  auto chunk_scores = [&](int buf, int sub, bool both, f32x16* acc) __attribute__((always_inline)) {
    acc[0] = f32x16{};
    acc[1] = f32x16{};
    const unsigned char* base = smem + buf * SBYTES + (sub * kChunk + (lane & 31)) * PITCH + half * 16;
#pragma unroll
    for (int s = 0; s < 2 * KS; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(base + 32 * s);
      if (both) acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0][s % KS], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[1][s % KS], acc[1], 0, 0, 0);
    }
  };
  auto key_of = [&](int c, int r) __attribute__((always_inline)) { return c * kChunk + 8 * (r >> 2) + 4 * half + (r & 3); };
  // Key block (within a chunk) of accumulator register r: the half and low
  // row bits add less than 8 <= R strides, so only 8 (r / 4) decides it.
  auto kb_of = [](int r) constexpr { return (8 * (r >> 2)) / R; };

  float l_run[2] = {0.f, 0.f};               // the rows' sums against rref (equal in lanes l and l ^ 32)
  float* ucol[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) ucol[g] = p.u + bh * p.nb * static_cast<int64_t>(p.ns_pad) + qi[g];
  // chunk c's per-block sums of both sets: both halves combined, added to the rows' sums, stored
  auto finish = [&](int c, float (&bsx)[2][KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float v = halves_sum32(bsx[g][kb]);
        l_run[g] += v;
        const int kblk = (c * kChunk) / R + kb;
        if (half == 0 && kblk < p.nb) __builtin_nontemporal_store(v, ucol[g] + static_cast<int64_t>(kblk) * p.ns_pad);
      }
  };

  // Stages whose two chunks lie wholly before both sets' rows (every row of
  // the wave valid) run software-pipelined: a chunk's MFMAs are interleaved
  // step by step with the exponentials of the chunk before it, so matrix and
  // vector work of one wave overlap.  The sums keep chunk and register order.
  constexpr int NS = 2 * KS;                 // MFMA steps per chunk (hi and lo k-ranges)
  auto mfma_exp = [&](const unsigned char* base, f32x16 (&acc)[2], const f32x16 (&accx)[2], float (&bsx)[2][KB],
                      auto&& side) __attribute__((always_inline)) {
    acc[0] = f32x16{};
    acc[1] = f32x16{};
    bf16x8 kf = *reinterpret_cast<const bf16x8*>(base);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 kn{};
      if (s + 1 < NS) kn = *reinterpret_cast<const bf16x8*>(base + 32 * (s + 1));
      // one MFMA, then that set's share of the other chunk's exponentials: the
      // vector work issues while the MFMA runs.  The sums are pinned at each
      // step (without it they sink below the chunk's MFMAs, to their first use).
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[g][s % KS], acc[g], 0, 0, 0);
#pragma unroll
        for (int r = s * 16 / NS; r < (s + 1) * 16 / NS; ++r)
          bsx[g][kb_of(r)] += __builtin_amdgcn_exp2f(__builtin_fmaf(accx[g][r], p.scale_log2, -rref[g]));
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) __asm__ volatile("" : "+v"(bsx[g][kb]));
        if (g == 1) side(s);
        __builtin_amdgcn_sched_barrier(0);
      }
      kf = kn;
    }
  };
  auto exp_only = [&](const f32x16 (&accx)[2], float (&bsx)[2][KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        bsx[g][kb_of(r)] += __builtin_amdgcn_exp2f(__builtin_fmaf(accx[g][r], p.scale_log2, -rref[g]));
  };
  const int n_open = (q0 + 63 < p.ns) ? last0 / 2 : 0;
  f32x16 accp[2];                            // the pending chunk's scores (none yet: exp2 of -inf adds 0)
#pragma unroll
  for (int r = 0; r < 16; ++r) accp[0][r] = accp[1][r] = -__builtin_inff();

  auto next_stage = [&](int st) __attribute__((always_inline)) {
    wait_stage(AHEAD > 1 && st + 1 < n_stage);
    __syncthreads();
    if (st + AHEAD < n_stage) issue_stage(st + AHEAD);
  };
  issue_stage(0);
  if (AHEAD > 1 && n_stage > 1) issue_stage(1);
  // In pipelined stages the copies of stage st + AHEAD are spread over the
  // first chunk's MFMA steps (one per two steps; a wave's last copy, which
  // not every wave has, after them) instead of issued in a burst.
  static_assert(NS / 2 >= NW_LO, "a copy every second step");
  auto no_side = [](int) {};
  auto pipelined = [&](int st, auto copies) __attribute__((always_inline)) {
    const unsigned char* base = smem + (st % NBUF) * SBYTES + (lane & 31) * PITCH + half * 16;
    uint64_t src = 0;
    uint32_t dst = 0;
    if constexpr (decltype(copies)::value) {
      const int sn = st + AHEAD;
      src = dev::uniform_u64(reinterpret_cast<uint64_t>(ksb) + static_cast<uint64_t>(sn) * SBYTES);
      dst = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(smem_lds + (sn % NBUF) * SBYTES)));
    }
    auto copy = [&](int s) __attribute__((always_inline)) {
      if constexpr (decltype(copies)::value) {
        if (s % 2 == 0 && s / 2 < NW_LO) {
          const int ins = wave + 4 * (s / 2);
          dev::dma16(src + static_cast<uint64_t>(ins) * 1024, 16 * lane, dst + ins * 1024);
        }
      }
    };
    float bsp[2][KB] = {}, bsa[2][KB] = {};
    f32x16 acca[2], accb[2];
    mfma_exp(base, acca, accp, bsp, copy);              // chunk 2 st; exponentials of 2 st - 1
    if constexpr (decltype(copies)::value) {
      if (NW_HI > NW_LO && wave + 4 * NW_LO < NI)
        dev::dma16(src + static_cast<uint64_t>(wave + 4 * NW_LO) * 1024, 16 * lane, dst + (wave + 4 * NW_LO) * 1024);
    }
    if (st > 0) finish(2 * st - 1, bsp);
    mfma_exp(base + kChunk * PITCH, accb, acca, bsa, no_side);  // chunk 2 st + 1; exponentials of 2 st
    finish(2 * st, bsa);
    accp[0] = accb[0];
    accp[1] = accb[1];
  };
  int st = 0;
  for (; st < n_open; ++st) {
    wait_stage(AHEAD > 1 && st + 1 < n_stage);
    __syncthreads();
    if (st + AHEAD < n_stage) pipelined(st, std::true_type{});
    else pipelined(st, std::false_type{});
  }
  if (n_open > 0) {                                     // the last pipelined chunk
    float bsp[2][KB] = {};
    exp_only(accp, bsp);
    finish(2 * n_open - 1, bsp);
  }
  for (; st < n_stage; ++st) {
    next_stage(st);
    const int buf = st % NBUF;
    f32x16 accs[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int c = 2 * st + sub;
      if (c <= last0 + 1) chunk_scores(buf, sub, c <= last0, accs[sub]);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int c = 2 * st + sub;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if (c > last0 + g) continue;            // no stride of this chunk precedes the set's rows
        const f32x16& acc = accs[sub][g];
        const bool open = c < last0 + g && q0 + 32 * g + 31 < p.ns;
        float bs[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bs[kb] = 0.f;
        if (open) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            bs[kb_of(r)] += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], p.scale_log2, -rref[g]));
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = key_of(c, r);
            const float pr = (q_valid[g] && j <= qi[g])
                                 ? __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], p.scale_log2, -rref[g]))
                                 : 0.f;
            bs[kb_of(r)] += pr;
          }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const float v = halves_sum32(bs[kb]);
          l_run[g] += v;
          const int kblk = (c * kChunk) / R + kb;
          if (half == 0 && kblk < p.nb) __builtin_nontemporal_store(v, ucol[g] + static_cast<int64_t>(kblk) * p.ns_pad);
        }
      }
    }
  }
  // Block scores of the wave's rows: S_mn = sum over the rows i of block m of
  // u_in / l_i for n <= m, from the per-block sums this wave stored (read
  // back by the wave that wrote them).  Lane (j, b) takes block b of the
  // wave's 64 / R and key blocks n = j, j + R, ...: it reads the block's R
  // row sums for n (contiguous), scales them by the rows' 1 / l (shared
  // through LDS) and adds them in row order.  The table has a row for every
  // block's rows (rows at or past ns hold 0 and 1 / l = 0), so every S_mn with
  // n <= m < nb is written here; rows of flagged tiles are rewritten by the
  // recompute.
  constexpr int MB = 64 / R;                 // query blocks of a wave
  bool bad = false;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float li = (q_valid[g] && l_run[g] > 0.f) ? 1.f / l_run[g] : 0.f;
    bad = bad || (q_valid[g] && !(l_run[g] >= 0x1p-40f));
    if (half == 0) linv_s[wave][32 * g + lane] = li;
  }
  __threadfence_block();                     // this wave's stores of u before its loads of them
  __syncthreads();
  {
    const int bl = lane % MB, j = lane / MB;
    const int m = q0 / R + bl;
    float lr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) lr[r] = linv_s[wave][bl * R + r];
    const int n_row = min(m, p.nb - 1);
    const int n_end = min((q0 + 63) / R, p.nb - 1);     // the wave's last block
    const float* ublk = p.u + bh * p.nb * static_cast<int64_t>(p.ns_pad) + q0 + bl * R;
    float* srow = p.score + (bh * p.nb + m) * static_cast<int64_t>(p.nb);
    constexpr int U = 4;                     // key blocks in flight per lane
    for (int n0 = 0; n0 <= n_end; n0 += U * R) {
      using v4f = float __attribute__((ext_vector_type(4)));
      v4f v[U][R / 4];
#pragma unroll
      for (int k = 0; k < U; ++k) {          // every load issued, at a block the rows have written
        const v4f* src = reinterpret_cast<const v4f*>(
            ublk + static_cast<int64_t>(min(n0 + k * R + j, n_row)) * p.ns_pad);
#pragma unroll
        for (int r4 = 0; r4 < R / 4; ++r4) v[k][r4] = __builtin_nontemporal_load(src + r4);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int n = n0 + k * R + j;
        float sm = 0.f;
#pragma unroll
        for (int r4 = 0; r4 < R / 4; ++r4) {
          sm = __builtin_fmaf(v[k][r4].x, lr[4 * r4], sm);
          sm = __builtin_fmaf(v[k][r4].y, lr[4 * r4 + 1], sm);
          sm = __builtin_fmaf(v[k][r4].z, lr[4 * r4 + 2], sm);
          sm = __builtin_fmaf(v[k][r4].w, lr[4 * r4 + 3], sm);
        }
        if (n <= n_row && m < p.nb) srow[n] = sm;
      }
    }
  }
  const uint64_t any_bad = __builtin_amdgcn_ballot_w64(bad);
  if (lane == 0) bad_wave[wave] = any_bad != 0 ? 1 : 0;
  __syncthreads();
  if (threadIdx.x == 0) {                     // waves 0-1 cover 128-row tile 2 tile, waves 2-3 the next
    const int64_t f = bh * (p.ns_pad / kRrQ) + 2 * tile;
    p.flags[f] = bad_wave[0] | bad_wave[1];
    p.flags[f + 1] = bad_wave[2] | bad_wave[3];
  }
}

// -------------------------------------------------------------- select ----
// One wave per (query block m, head, batch), four block rows per work-group.
// Eq. 11 keeps the shortest prefix of the row's causal blocks, ordered by
// descending score (ties: lower n first), whose mass reaches tau times the
// row's mass.  That prefix is found without sorting.  With F(x) = mass of the
// scores >= x, the last kept score is theta = the largest x with
// F(x) >= tau * total; every block above theta is kept and, of the blocks
// scoring exactly theta, the lowest-n ones until the mass is reached.  Scores
// are >= 0, so their bit patterns order like their values and theta is a
// binary search over bit patterns (31 steps).  Lane l holds the scores of
// n = l, l + 64, ...; each F is summed in one fixed order (the lane's own
// scores in n order, then a butterfly over the wave that leaves every lane
// the same total), so F is monotone in x and reproducible.
constexpr int kSelRows = kRrThreads / 64;
// PER: scores per lane (16 for rows of up to 1024 blocks, 64 up to 4096).
template <int PER>
__global__ __launch_bounds__(kRrThreads) void rr_select_kernel(const RrParams p) {
  constexpr int kPerMax = PER;
  const int lane = threadIdx.x & 63;
  const int m = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kSelRows + (threadIdx.x >> 6));
  const int h = blockIdx.y, b = blockIdx.z;
  if (m >= p.nb) return;                      // the whole wave: no work-group barrier in this kernel
  const int nv = m + 1;                       // causal key blocks n <= m
  const int per = (nv + 63) / 64;
  const int64_t row = (static_cast<int64_t>(b) * p.H + h) * p.nb * p.nb + static_cast<int64_t>(m) * p.nb;
  float* srow = p.score + row;
  uint8_t* brow = p.bmask + row;
  float v[kPerMax];
#pragma unroll
  for (int i = 0; i < kPerMax; ++i) {
    const int n = lane + 64 * i;
    v[i] = (i < per && n < nv) ? fmaxf(srow[n], 0.f) : 0.f;
  }
  auto mass_from = [&](uint32_t xb) __attribute__((always_inline)) {  // F(x), x given by its bits
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kPerMax; ++i)
      if (i < per && __float_as_uint(v[i]) >= xb) s += v[i];
    return halves_sum32(group_sum<32>(s));
  };
  const float total = mass_from(0u);
  const float thr = p.tau * total;
  uint32_t theta = 0xFFFFFFFFu;               // no block kept (a row without mass)
  int need = 0;                               // blocks scoring exactly theta to keep
  if (total > 0.f) {
    uint32_t lo = 0u, hi = 0x7F800000u;       // F(lo) >= thr > F(hi) (thr > 0 = F(+inf))
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      if (mass_from(mid) >= thr) lo = mid;
      else hi = mid;
    }
    theta = lo;
    const float above = mass_from(lo + 1u);   // mass of the scores above theta (< thr)
    const float tv = __uint_as_float(lo);
    const float q = tv > 0.f ? ceilf((thr - above) / tv) : static_cast<float>(nv);
    need = q >= static_cast<float>(nv) ? nv : max(1, static_cast<int>(q));
  }
  const bool protect = p.protect_last && m == p.nb - 1;
  int ties_before = 0;                        // blocks scoring theta at lower n (earlier rounds)
#pragma unroll
  for (int i = 0; i < kPerMax; ++i) {
    const int n = lane + 64 * i;
    const uint32_t vb = __float_as_uint(v[i]);
    const bool tie = theta != 0xFFFFFFFFu && i < per && n < nv && vb == theta;
    const uint64_t tmask = __builtin_amdgcn_ballot_w64(tie);
    const int rank = ties_before + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                       static_cast<uint32_t>(tmask >> 32),
                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(tmask), 0u)));
    ties_before += __builtin_popcountll(tmask);
    const bool keep = (theta != 0xFFFFFFFFu && vb > theta) || (tie && rank < need);
    if (i < per && n < nv) brow[n] = (keep || protect) ? 1 : 0;
  }
  for (int n = nv + lane; n < p.nb; n += 64) {
    brow[n] = 0;
    srow[n] = 0.f;
  }
}

// The single pass (block scores included), then the two-pass kernel on the
// flagged query tiles only (its work-groups for other tiles return at once).
template <int D, int R>
hipError_t launch_scores_r(const RrParams& p, hipStream_t stream) {
  const dim3 grid1(static_cast<unsigned>(p.ns_pad / kRrQ1 * p.H * p.B));
  const dim3 grid(static_cast<unsigned>(p.ns_pad / kRrQ), static_cast<unsigned>(p.H), static_cast<unsigned>(p.B));
  hipLaunchKernelGGL((rr_scores1p_kernel<D, R>), grid1, dim3(kRrThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RrParams g = p;
  g.gate = 1;
  hipLaunchKernelGGL((rr_scores_kernel<D, R>), grid, dim3(kRrThreads), 0, stream, g);
  return hipGetLastError();
}

template <int D>
hipError_t launch_scores(const RrParams& p, hipStream_t stream) {
  switch (p.Bs / p.S) {
    case 8: return launch_scores_r<D, 8>(p, stream);
    case 16: return launch_scores_r<D, 16>(p, stream);
    case 32: return launch_scores_r<D, 32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rr_search(const RrParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  hipError_t e;
  if (start != nullptr && (e = hipEventRecord(start, stream)) != hipSuccess) return e;
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.ns_pad;
  const dim3 pgrid(static_cast<unsigned>((rows * (p.D == 64 ? 8 : 16) + 255) / 256));
  if (p.D == 64) hipLaunchKernelGGL(rr_prep_kernel<8>, pgrid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(rr_prep_kernel<16>, pgrid, dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rr_kmax_kernel, dim3(static_cast<unsigned>(p.H), static_cast<unsigned>(p.B)), dim3(1024), 0,
                     stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (p.D) {
    case 64: e = launch_scores<64>(p, stream); break;
    case 80: e = launch_scores<80>(p, stream); break;
    case 128: e = launch_scores<128>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const dim3 sgrid(static_cast<unsigned>((p.nb + kSelRows - 1) / kSelRows), static_cast<unsigned>(p.H),
                   static_cast<unsigned>(p.B));
  static_assert(kRrMaxBlocks == 64 * 64, "select variants cover up to 4096 blocks");
  if (p.nb <= 1024) hipLaunchKernelGGL(rr_select_kernel<16>, sgrid, dim3(kRrThreads), 0, stream, p);
  else hipLaunchKernelGGL(rr_select_kernel<64>, sgrid, dim3(kRrThreads), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (stop != nullptr && (e = hipEventRecord(stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace bss
