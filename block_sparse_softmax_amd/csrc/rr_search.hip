// RRAttention's block-pattern search for gfx950 ("RRAttention", section 3):
// from Q and K to the block-selection matrix B that the masked forward kernel
// consumes as its block mask.
//
//   prep    sampled queries q_P(i,h), P(i,h) = iS + (S - 1 - (h mod S)) (Eq. 6-7),
//           and stride-summed keys sum_{k=jS}^{(j+1)S-1} k_k (Eq. 8), into
//           contiguous bf16 rows of the workspace (sums in fp32, rounded once).
//   scores  the stride importance I = q . ksum / (S sqrt(d)) (Eq. 8) on
//           v_mfma_f32_32x32x16_bf16, in two passes over the causal key
//           strides j <= i: pass 1 keeps each row's running max and sum
//           (Eq. 9's softmax denominator), pass 2 recomputes I, normalises
//           and sums the probabilities straight into block scores S_mn
//           (Eq. 10).  The stride-level matrix is never stored.
//   select  per query block m: sort S_m,n (n <= m) descending (ties to the
//           lower n), keep the shortest prefix whose mass reaches tau times
//           the row's mass (Eq. 11), and every causal block of the last query
//           block (Eq. 12).
//
// Layout of the scores kernel: a work-group of 4 waves takes 128 consecutive
// sampled queries of one (batch, head); wave w owns queries 32w..32w+31 of
// them.  Chunks of 32 stride-summed keys are staged in LDS (double-buffered,
// shared by the 4 waves).  I^T = Ksum Q^T: the key chunk is the A operand
// (from LDS), the sampled queries the B operand (in registers), so lane l
// holds query l mod 32 and 16 of the chunk's 32 key strides.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"

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
// One thread per (batch, head, stride row of the padded table, 8-dim chunk).
__global__ __launch_bounds__(256) void rr_prep_kernel(const RrParams p) {
  const int cpr = p.D / 8;
  const int64_t n = static_cast<int64_t>(p.B) * p.H * p.ns_pad * cpr;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int c = static_cast<int>(t % cpr);
  const int64_t row = t / cpr;
  const int j = static_cast<int>(row % p.ns_pad);
  const int bh = static_cast<int>(row / p.ns_pad);
  const int h = bh % p.H, b = bh / p.H;
  bf16x8 qo = {}, ko = {};
  if (j < p.ns) {
    const int pos = j * p.S + (p.S - 1 - (h % p.S));
    qo = *reinterpret_cast<const bf16x8*>(p.q + b * p.q_sb + static_cast<int64_t>(pos) * p.q_sl + h * p.q_sh + 8 * c);
    float acc[8] = {};
    const uint16_t* kr = p.k + b * p.k_sb + static_cast<int64_t>(j) * p.S * p.k_sl + (h / p.kv_group) * p.k_sh + 8 * c;
    for (int s = 0; s < p.S; ++s) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(kr + static_cast<int64_t>(s) * p.k_sl);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += static_cast<float>(x[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ko[e] = static_cast<__bf16>(acc[e]);
  }
  *reinterpret_cast<bf16x8*>(p.qs + row * p.D + 8 * c) = qo;
  *reinterpret_cast<bf16x8*>(p.ks + row * p.D + 8 * c) = ko;
}

// -------------------------------------------------------------- scores ----
// R = block size / stride (strides per block): 8, 16 or 32.
template <int D, int R>
__global__ __launch_bounds__(kRrThreads) void rr_scores_kernel(const RrParams p) {
  constexpr int KS = D / 16;                 // k-steps of the 32x32x16 product
  constexpr int PITCH = 2 * D + 16;          // LDS row pitch: 16 rows of a fragment read hit distinct banks
  constexpr int CPR = D / 8;                 // 16-byte pieces per key row
  constexpr int PIECES = kChunk * CPR;       // per chunk
  constexpr int PER_THREAD = (PIECES + kRrThreads - 1) / kRrThreads;
  static_assert(R == 8 || R == 16 || R == 32, "strides per block");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kChunk * PITCH];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = p.ns_pad / kRrQ;
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.x);  // longest (latest) tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh_row = (static_cast<int64_t>(b) * p.H + h) * p.ns_pad;
  const bf16x8* qs = reinterpret_cast<const bf16x8*>(p.qs) + bh_row * CPR;
  const bf16x8* ks = reinterpret_cast<const bf16x8*>(p.ks) + bh_row * CPR;

  const int q0 = tile * kRrQ + 32 * wave;    // this wave's first sampled query
  const int qi = q0 + (lane & 31);           // this lane's query (column of I^T)
  const int half = lane >> 5;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = qs[static_cast<int64_t>(qi) * CPR + 2 * s + half];

  const int last_chunk_wg = (tile * kRrQ + kRrQ - 1) / kChunk;  // chunks the work-group stages
  const int last_chunk = q0 / kChunk;                            // chunks this wave computes
  const int n_chunks = last_chunk_wg + 1;

  // staging: piece t of a chunk = row t / CPR, 16 bytes at column t % CPR
  bf16x8 stage[PER_THREAD];
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int t = threadIdx.x + u * kRrThreads;
      if (t < PIECES) stage[u] = ks[static_cast<int64_t>(c * kChunk + t / CPR) * CPR + t % CPR];
    }
  };
  auto store_chunk = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int t = threadIdx.x + u * kRrThreads;
      if (t < PIECES)
        *reinterpret_cast<bf16x8*>(smem + buf * kChunk * PITCH + (t / CPR) * PITCH + (t % CPR) * 16) = stage[u];
    }
  };
  // I^T tile of chunk c (in buffer buf): lane holds key strides c*32 + 8g + 4*half + e (register 4g + e)
  auto chunk_scores = [&](int buf) __attribute__((always_inline)) {
    f32x16 acc = {};
    const unsigned char* base = smem + buf * kChunk * PITCH + (lane & 31) * PITCH + half * 16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(base + 32 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], acc, 0, 0, 0);
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
    load_chunk(0);
    store_chunk(0);
    if (n_chunks > 1) load_chunk(1);
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
      const int buf = c & 1;
      if (c <= last_chunk) {
        const f32x16 acc = chunk_scores(buf);
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
      if (c + 1 < n_chunks) {
        __syncthreads();                       // everyone is done with buffer buf ^ 1 (chunk c-1)
        store_chunk(buf ^ 1);
        if (c + 2 < n_chunks) load_chunk(c + 2);
        __syncthreads();
      }
    }
    if (pass == 0) {
      // combine the two halves of each query: max and sum over all its key strides
      const float mo = __shfl_xor(m_run, 32), lo = __shfl_xor(l_run, 32);
      const float m = fmaxf(m_run, mo);
      const float l = (m == -INFINITY) ? 0.f
                                       : l_run * __builtin_amdgcn_exp2f(m_run - m) + lo * __builtin_amdgcn_exp2f(mo - m);
      m_row = (m == -INFINITY) ? 0.f : m;
      inv_l = l > 0.f ? 1.f / l : 0.f;
      __syncthreads();                         // pass 2 restages from chunk 0
    }
  }
}

// -------------------------------------------------------------- select ----
// One work-group per (query block m, head, batch).
__global__ __launch_bounds__(kRrThreads) void rr_select_kernel(const RrParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  const int m = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nv = m + 1;                       // causal key blocks n <= m
  int p2 = 1;
  while (p2 < nv) p2 <<= 1;
  float* key = reinterpret_cast<float*>(dyn);
  int* idx = reinterpret_cast<int*>(dyn + static_cast<size_t>(p.sel_cap) * 4);
  float* part = reinterpret_cast<float*>(dyn + static_cast<size_t>(p.sel_cap) * 8);  // kRrThreads partial sums
  const int64_t row = (static_cast<int64_t>(b) * p.H + h) * p.nb * p.nb + static_cast<int64_t>(m) * p.nb;
  float* srow = p.score + row;
  uint8_t* brow = p.bmask + row;
  for (int n = threadIdx.x; n < p2; n += kRrThreads) {
    key[n] = n < nv ? srow[n] : -1.f;         // scores are >= 0: padding sorts last
    idx[n] = n;
  }
  __syncthreads();
  // total mass of the row, in a fixed order (thread t sums n = t, t + 256, ...)
  float s = 0.f;
  for (int n = threadIdx.x; n < nv; n += kRrThreads) s += key[n];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = kRrThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float total = part[0];
  __syncthreads();
  // bitonic sort: descending score, ascending index on ties
  for (int k = 2; k <= p2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < p2; t += kRrThreads) {
        const int u = t ^ j;
        if (u > t) {
          const bool first_before = (key[t] > key[u]) || (key[t] == key[u] && idx[t] < idx[u]);
          const bool up = (t & k) == 0;        // this run is sorted "first before" ascending in t
          if (first_before != up) {
            const float kt = key[t]; key[t] = key[u]; key[u] = kt;
            const int it = idx[t]; idx[t] = idx[u]; idx[u] = it;
          }
        }
      }
      __syncthreads();
    }
  }
  // prefix sums of the sorted scores: thread t owns a contiguous run of positions
  const int per = (p2 + kRrThreads - 1) / kRrThreads;
  const int a0 = threadIdx.x * per, a1 = min(p2, a0 + per);
  float run = 0.f;
  for (int a = a0; a < a1; ++a) run += key[a] > 0.f ? key[a] : 0.f;
  {  // exclusive scan of the run sums in thread order (fixed association: per-wave
     // inclusive scan, then the totals of the preceding waves)
    __shared__ float wave_total[kRrThreads / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float x = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_total[w] = x;
    __syncthreads();
    float base = 0.f;
    for (int i = 0; i < w; ++i) base += wave_total[i];
    part[threadIdx.x] = base + (x - run);
    __syncthreads();
  }
  // keep sorted positions before and at the first one whose prefix reaches tau * total
  const float thr = p.tau * total;
  float c = part[threadIdx.x];
  int cut = -1;                                // first position (in this run) reaching the threshold
  for (int a = a0; a < a1; ++a) {
    c += key[a] > 0.f ? key[a] : 0.f;
    if (cut < 0 && c >= thr && total > 0.f) cut = a;
  }
  __syncthreads();
  int* first = reinterpret_cast<int*>(part);   // reuse: the earliest cut over all threads
  if (threadIdx.x == 0) first[0] = 0x7fffffff;
  __syncthreads();
  if (cut >= 0) atomicMin(first, cut);         // LDS atomic
  __syncthreads();
  const int kcut = total > 0.f ? min(first[0], nv - 1) : -1;
  for (int n = threadIdx.x; n < p.nb; n += kRrThreads) brow[n] = 0;
  __syncthreads();
  for (int a = threadIdx.x; a <= kcut; a += kRrThreads)
    if (idx[a] < nv) brow[idx[a]] = 1;        // (padding sorts last unless a score is NaN)
  if (p.protect_last && m == p.nb - 1)
    for (int n = threadIdx.x; n < nv; n += kRrThreads) brow[n] = 1;
  for (int n = nv + threadIdx.x; n < p.nb; n += kRrThreads) srow[n] = 0.f;
}

template <int D>
hipError_t launch_scores(const RrParams& p, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(p.ns_pad / kRrQ), static_cast<unsigned>(p.H), static_cast<unsigned>(p.B));
  switch (p.Bs / p.S) {
    case 8: hipLaunchKernelGGL((rr_scores_kernel<D, 8>), grid, dim3(kRrThreads), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((rr_scores_kernel<D, 16>), grid, dim3(kRrThreads), 0, stream, p); break;
    case 32: hipLaunchKernelGGL((rr_scores_kernel<D, 32>), grid, dim3(kRrThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rr_search(const RrParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  hipError_t e;
  if (start != nullptr && (e = hipEventRecord(start, stream)) != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(p.B) * p.H * p.ns_pad * (p.D / 8);
  hipLaunchKernelGGL(rr_prep_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (p.D) {
    case 64: e = launch_scores<64>(p, stream); break;
    case 80: e = launch_scores<80>(p, stream); break;
    case 128: e = launch_scores<128>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const size_t lds = static_cast<size_t>(p.sel_cap) * 8 + kRrThreads * 4;
  hipLaunchKernelGGL(rr_select_kernel, dim3(static_cast<unsigned>(p.nb), static_cast<unsigned>(p.H),
                                            static_cast<unsigned>(p.B)),
                     dim3(kRrThreads), lds, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (stop != nullptr && (e = hipEventRecord(stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace bss
