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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;

constexpr int kMaskFull = 0, kMaskChunk = 1, kMaskWindow = 2, kMaskBlock = 3;

template <int D>
struct Shape {
  static constexpr int CPR = D / 8;                          // 16-byte chunks per token row
  static constexpr int RB = D * 2;                           // bytes per token row
  static constexpr int KS = D / 16;                          // k-steps of the Q.K product
  static constexpr int DT = (D + 31) / 32;                   // 32-row tiles of O^T
  static constexpr int TILE = kBN * RB;                      // bytes of one K (or V) tile
  static constexpr int LOADS = 2 * kBN * CPR / 64 / kWaves;  // LDS-DMA loads per lane per tile
  static constexpr bool PAD_ROWSUM = (D % 32) != 0;
  static_assert((2 * kBN * CPR) % (64 * kWaves) == 0, "tile must split evenly over the waves");
};

// Physical 16-byte chunk of logical chunk c in LDS row `row` (an involution).
template <int D>
__device__ __forceinline__ int phys_chunk(int row, int c) {
  if (D == 80 && c >= 8) return c ^ (row & 1);
  return c ^ (row & 7);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
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
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * S::TILE];  // [buffer][K, V]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5;    // half of the wave
  const int l31 = lane & 31;

  const int4 item = reinterpret_cast<const int4*>(p.items)[blockIdx.x];
  const int head = item.x, qtile = item.y, e_begin = item.z, e_end = item.w;
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

  // ---- this lane's query and its Q fragments (B operand of S^T = K Q^T) ----
  const int qi = qtile * kBM + wave * 32 + l31;
  const int qrow = qi < p.L ? qi : p.L - 1;
  bf16x8 qf[S::KS];
  {
    const unsigned char* src = qbase + qrow * q_row_bytes + 16 * h2;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
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
  // K fragment for k-step ks: row l31 (and l31 + 32), logical chunk 2*ks + h2.
  int koff[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) koff[ks] = l31 * S::RB + phys_chunk<D>(l31, 2 * ks + h2) * 16;
  // V^T fragment for O^T tile dt: transposed read; source lane (j, c) of each
  // 16-lane group points at row 4*h2 + j, columns 32*dt + 16*dhalf + 4*c .. +3.
  const int tr_j = (lane & 15) >> 2, tr_c = lane & 3, dhalf = (lane >> 4) & 1;
  int voff[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) {
    const int row = 4 * h2 + tr_j;
    int c = 4 * dt + 2 * dhalf + (tr_c >> 1);
    if (S::PAD_ROWSUM && 8 * c >= D) c = 2 * dhalf + (tr_c >> 1);  // pad lanes: any valid address
    voff[dt] = row * S::RB + phys_chunk<D>(row, c) * 16 + (tr_c & 1) * 8;
  }
  // Pad lanes of the last O^T tile use a constant V^T: row D is all ones, the rest zero.
  bf16x8 pad_ones;
  {
    const __bf16 one = (dhalf == 1 && (lane & 15) == 0) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) pad_ones[e] = one;
  }
  const bool pad_lane = S::PAD_ROWSUM && dhalf == 1;

  // LDS-DMA: wave-instruction idx = wave + 4*i fills 64 consecutive 16-byte slots.
  int goff[S::LOADS];
#pragma unroll
  for (int i = 0; i < S::LOADS; ++i) {
    const int idx = wave + kWaves * i;
    const int tensor = idx >= S::CPR;
    const int blk = tensor ? idx - S::CPR : idx;
    const int slot = blk * 64 + lane;
    const int row = slot / S::CPR;
    const int c = phys_chunk<D>(row, slot % S::CPR);
    goff[i] = row * static_cast<int>(tensor ? v_row_bytes : k_row_bytes) + c * 16;
  }

  auto issue_tile = [&](int kt, int buf) {
    const int kv0 = kt * kBN;
    const unsigned char* kp = kbase + kv0 * k_row_bytes;
    const unsigned char* vp = vbase + kv0 * v_row_bytes;
    unsigned char* dst = smem + buf * 2 * S::TILE;
    const bool ragged = kv0 + kBN > p.L;
#pragma unroll
    for (int i = 0; i < S::LOADS; ++i) {
      const int idx = wave + kWaves * i;
      const int tensor = idx >= S::CPR;
      const int blk = tensor ? idx - S::CPR : idx;
      int off = goff[i];
      if (ragged) {  // clamp rows past the end of the sequence (their keys are masked)
        const int slot = blk * 64 + lane;
        const int row = min(slot / S::CPR, p.L - 1 - kv0);
        const int c = phys_chunk<D>(slot / S::CPR, slot % S::CPR);
        off = row * static_cast<int>(tensor ? v_row_bytes : k_row_bytes) + c * 16;
      }
      const unsigned char* src = (tensor ? vp : kp) + off;
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dst + tensor * S::TILE + blk * 1024), 16, 0, 0);
    }
  };

  const int n = e_end - e_begin;
  if (n > 0) issue_tile(p.kv[e_begin] >> 1, 0);

  for (int e = 0; e < n; ++e) {
    const int ent = p.kv[e_begin + e];
    const int kt = ent >> 1;
    const bool full = ent & 1;
    const int buf = e & 1;
    if (e + 1 < n) {
      issue_tile(p.kv[e_begin + e + 1] >> 1, buf ^ 1);
      wait_vmcnt<S::LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();

    const unsigned char* kt_lds = smem + buf * 2 * S::TILE;
    const unsigned char* vt_lds = kt_lds + S::TILE;

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kt_lds + koff[ks]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kt_lds + koff[ks] + 32 * S::RB);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }

    // ---- mask (PARTIAL tiles only) ----
    if (!full) {
      const unsigned base = static_cast<unsigned>(kt * kBN + 4 * h2 - lo);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned u = base + 8 * (r >> 2) + (r & 3);
        if (u >= width) s0[r] = -INFINITY;
        if (u + 32 >= width) s1[r] = -INFINITY;
      }
    }

    // ---- online softmax ----
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = halves_max(mx) * p.scale_log2;
    const bool need = mx > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      sink_l *= alpha;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) acc[dt] *= alpha;
    }
    const float mneg = (m_run == -INFINITY) ? 0.f : -m_run;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], p.scale_log2, mneg));
      s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], p.scale_log2, mneg));
      if (!S::PAD_ROWSUM) rs += s0[r] + s1[r];
    }
    if (!S::PAD_ROWSUM) l_run += rs;

    // P^T operands for the four 16-key k-steps of this tile
    bf16x8 pb[4];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      pb[0][e8] = (__bf16)s0[e8];
      pb[1][e8] = (__bf16)s0[8 + e8];
      pb[2][e8] = (__bf16)s1[e8];
      pb[3][e8] = (__bf16)s1[8 + e8];
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const unsigned char* src = vt_lds + voff[dt] + 16 * t * S::RB;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + 8 * S::RB));
        bf16x8 a;
        const bf16x4 y0 = __builtin_bit_cast(bf16x4, x0), y1 = __builtin_bit_cast(bf16x4, x1);
        a[0] = y0[0]; a[1] = y0[1]; a[2] = y0[2]; a[3] = y0[3];
        a[4] = y1[0]; a[5] = y1[1]; a[6] = y1[2]; a[7] = y1[3];
        if (S::PAD_ROWSUM && dt == S::DT - 1 && pad_lane) a = pad_ones;
        acc[dt] = mfma32(a, pb[t], acc[dt]);
      }
    }
    wg_barrier();
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
  dim3 grid(static_cast<unsigned>(p.n_items), static_cast<unsigned>(B));
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
