// Token re-permutation between serialisation orders of a 2D patch grid
// ("Semantic Head Specialization ...", the Factor-2 slides and the Ariadne
// design: raster, 2 x 2-block row-major (c) and 2 x 2-block column-major (d)
// orders; Ariadne re-permutes the tokens where the order changes, a
// memory-bound step).  out[b, t, h, :] = in[b, src(t), h, :], where src(t) is
// the position, in the source order, of the patch the target order puts at t.
// One thread per 16-byte piece of a token row; consecutive threads walk the
// output along its smaller stride, so writes are contiguous, and the reads of
// a block order come in runs of a 2 x 2 block's 4 tokens.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include <cstdint>

#include "kernels.hpp"

namespace bss {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Patch (r, c) at sequence position t of order `o`.
__device__ __forceinline__ void patch_at(int o, int t, int gh, int gw, int* r, int* c) {
  if (o == 0) {               // raster
    *r = t / gw;
    *c = t % gw;
  } else if (o == 1) {        // 2 x 2 blocks row-major, row by row inside a block
    const int blk = t >> 2, w = t & 3, bpr = gw >> 1;
    *r = 2 * (blk / bpr) + (w >> 1);
    *c = 2 * (blk % bpr) + (w & 1);
  } else {                    // 2 x 2 blocks column-major, column by column inside a block
    const int blk = t >> 2, w = t & 3, bpc = gh >> 1;
    *c = 2 * (blk / bpc) + (w >> 1);
    *r = 2 * (blk % bpc) + (w & 1);
  }
}

// Sequence position of patch (r, c) in order `o`.
__device__ __forceinline__ int position_of(int o, int r, int c, int gh, int gw) {
  if (o == 0) return r * gw + c;
  if (o == 1) return (((r >> 1) * (gw >> 1) + (c >> 1)) << 2) + ((r & 1) << 1) + (c & 1);
  return (((c >> 1) * (gh >> 1) + (r >> 1)) << 2) + ((c & 1) << 1) + (r & 1);
}

__global__ __launch_bounds__(256) void reorder_kernel(const ReorderParams p) {
  const int cpr = p.D / 8;
  const int64_t n = static_cast<int64_t>(p.B) * p.L * p.H * cpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int c8 = static_cast<int>(i % cpr);
    int64_t rest = i / cpr;
    int h, t;
    if (p.out_sh < p.out_sl) {  // heads interleaved in a token's row ([B, L, H, D]): heads vary fastest
      h = static_cast<int>(rest % p.H);
      rest /= p.H;
      t = static_cast<int>(rest % p.L);
      rest /= p.L;
    } else {                    // each head's rows contiguous ([B, H, L, D]): tokens vary fastest
      t = static_cast<int>(rest % p.L);
      rest /= p.L;
      h = static_cast<int>(rest % p.H);
      rest /= p.H;
    }
    const int b = static_cast<int>(rest);
    int r, c;
    patch_at(p.to, t, p.gh, p.gw, &r, &c);
    const int s = position_of(p.from, r, c, p.gh, p.gw);
    const u32x4 v = *reinterpret_cast<const u32x4*>(p.in + b * p.in_sb + s * p.in_sl + h * p.in_sh + 8 * c8);
    *reinterpret_cast<u32x4*>(p.out + b * p.out_sb + t * p.out_sl + h * p.out_sh + 8 * c8) = v;
  }
}

}  // namespace

hipError_t launch_reorder(const ReorderParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int64_t n = static_cast<int64_t>(p.B) * p.L * p.H * (p.D / 8);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 64);   // grid-stride beyond that
  if (n == 0) return hipSuccess;
  hipExtLaunchKernelGGL(reorder_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, start, stop, 0, p);
  return hipGetLastError();
}

}  // namespace bss
