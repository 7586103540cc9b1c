// Kernel-side parameter block and launcher declaration (shared by the C ABI
// layer and the HIP translation unit).
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace bss {

// Floats of one partial-state slot of a split item at head dim D: for each of
// the 4 waves, the DT = ceil(D/32) accumulator tiles of O^T (16 floats per
// lane each, stored as 4 float4 per lane, lane-minor) and then the row
// reference m and the denominator l of every lane.
constexpr int64_t partial_slot_floats(int64_t D) { return 4 * (((D + 31) / 32) * 16 * 64 + 2 * 64); }

// Floats of one dK/dV partial slot of a split key block (backward): dK then
// dV, each as float4 [4 waves][D/32 tiles][4][64 lanes].
constexpr int64_t dkdv_slot_floats(int64_t D) { return 2 * 4 * ((D + 31) / 32) * 16 * 64; }

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t q_sb, q_sl, q_sh;   // element strides
  int64_t k_sb, k_sl, k_sh;
  int64_t v_sb, v_sl, v_sh;
  int64_t o_sb, o_sl, o_sh;
  const int32_t* items;       // n_items x {head, qtile, begin, end, slot, piece, npieces, counter}
  const int32_t* kv;          // (kv_tile << 1) | full
  const int32_t* head_left;   // [H] window left reach (WINDOW)
  const uint32_t* block_bits; // unaligned BLOCK masks (unused when aligned)
  const float* sink;          // [H] or nullptr
  float* partials;            // partial-state slots of split items
  const int32_t* merge_rows;  // n_merge x {head, qtile, first slot, pieces}: the split rows
  int32_t n_merge;            // split rows of this launch (0 unless batch 1 with split rows)
  float scale_log2;           // softmax scale * log2(e)
  int32_t L, H, n_items;
  int32_t kind, causal;
  int32_t chunk, right;
  int32_t prefix;             // prefix tokens added to every row's set (0 = none)
  int32_t kv_group;           // query heads per K/V head (grouped-query attention; 1 = MHA)
  int32_t pingpong;           // head dim 128: the plan picks the two-group kernel (long rows)
  int32_t n_entries;          // list entries of the plan's image (range checks of the checked build)
  int32_t n_slots;            // partial-state slots of this launch (0 without split rows)
  uint32_t* check;            // violation bits of the checked build (set by launch_fwd)
  float* lse;                 // optional [B][H][L]: row log-sum-exp (natural log), -inf for empty rows
};

// Several launches (jobs) with the same head dim and batch run as one kernel.
// Every job's schedule is 8 equal-length XCD queues of n_items / 8 items; the
// grid's XCD x takes, in job order, queue x of every job.
constexpr int kMaxJobs = 8;
struct GroupParams {
  int32_t n_jobs;
  int32_t queue_len[kMaxJobs];  // job j: items per XCD queue (n_items / 8)
  FwdParams job[kMaxJobs];
};
static_assert(sizeof(GroupParams) <= 4096, "kernel arguments are limited to 4 KiB");

// Launch the forward kernel for head dim D on `stream` with grid
// (8 * sum of queue lengths, B), then, when some job has split rows, the merge
// kernel (one work-group per split row); non-null events record the start of
// the first and the end of the last.
hipError_t launch_fwd(const GroupParams& g, int D, int B, hipStream_t stream, hipEvent_t start,
                      hipEvent_t stop);

// Device scratch of the allocation-free forward (attn_fwd.hip): a file-scope
// device array of kFwdScratchBytes, one per GPU, alive until the process
// ends.  Returns its device address on the current device (looked up once per
// device with hipGetSymbolAddress) and its size.
constexpr size_t kFwdScratchBytes = size_t(32) << 20;
hipError_t fwd_scratch(void** ptr, size_t* bytes);

// Checked build (BSS_CHECKED): whether the kernels carry range checks, and the
// current device's violation bits (read after the device has finished the
// launches; `clear` zeroes them).  Without the checks the bits stay 0.
bool checked_build();
hipError_t check_bits(uint32_t* bits, bool clear);

// Backward pass (attn_bwd.hip).
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int64_t q_sb, q_sl, q_sh;   // element strides
  int64_t k_sb, k_sl, k_sh;
  int64_t v_sb, v_sl, v_sh;
  int64_t o_sb, o_sl, o_sh;
  int64_t do_sb, do_sl, do_sh;
  int64_t dq_sb, dq_sl, dq_sh;
  int64_t dk_sb, dk_sl, dk_sh;
  int64_t dv_sb, dv_sl, dv_sh;
  const float* lse;           // [B][H][L] from the forward (natural log)
  const float* sink;          // [H] or nullptr
  float* dsink;               // [H] or nullptr
  float* stat;                // workspace [B][H][2][Lpad]: lse in log2 units (+inf: no mass), then D
  float* sinkpart;            // workspace [B][H][nq]: per query tile sums of exp(s_aux - lse_i) D_i
  uint16_t* qs;               // workspace [B][H][L][D] bf16: Q * sigma * log2(e) rounded as the forward rounds it
  const int32_t* q_items;     // dQ work items: the forward's schedule (8 queues; batch 1: long rows split)
  float* partials;            // batch 1: the forward's partial slots, reused for the pieces' dQ sums
  const int32_t* merge_rows;  // n_merge x {head, qtile, first slot, pieces}: the split rows
  int32_t n_merge;
  const int32_t* kv;          // the forward's lists: (kv_tile << 1) | full
  const int32_t* kv_items;    // dK/dV work items {kv head, key block, begin, end, slot, piece, pieces, split}
                              // (8 queues; batch 1: long key blocks split)
  float* dkdv_partials;       // batch 1: dK/dV partial slots of split key blocks
  const int32_t* kv_merge;    // n_kv_merge x {kv head, key block, first slot, pieces}
  int32_t n_kv_merge;
  const int32_t* col;         // per (kv head, key block): (group head << 24) | (query tile << 1) | full
  const int32_t* head_left;   // [H] window left reach (WINDOW)
  float scale;                // softmax scale sigma
  float scale_log2;           // sigma * log2(e)
  int32_t L, H, Lpad, nq;     // Lpad = nq * 128
  int32_t kind, causal, chunk, right, prefix, kv_group;
  int32_t q_queue, kv_queue;  // items per XCD queue
};

// Queue the backward kernels (prep, dQ, dK/dV, sink) on `stream`; non-null
// events record the start of the first and the end of the last.
hipError_t launch_bwd(const BwdParams& p, int D, int B, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// RRAttention block-pattern search (rr_search.hip).
constexpr int kRrMaxBlocks = 4096;  // key blocks per row of the pattern search
struct RrParams {
  const uint16_t* q;
  const uint16_t* k;
  int64_t q_sb, q_sl, q_sh;   // element strides
  int64_t k_sb, k_sl, k_sh;
  uint16_t* qs;               // workspace: sampled queries [B][H][ns_pad][D] bf16
  uint16_t* ks;               // workspace: stride-summed keys [B][H][ns_pad][D] bf16
  float* score;               // [B][H][nb][nb] block scores (Eq. 10)
  uint8_t* bmask;             // [B][H][nb][nb] block matrix (Eq. 11-12)
  float scale_log2;           // log2(e) / (S sqrt(D))
  float tau;
  int32_t B, H, L, D, S, Bs;
  int32_t ns, ns_pad, nb, protect_last;
  int32_t kv_group;           // query heads per K head (grouped-query attention)
  // single-pass scores (workspace)
  float* knorm2;              // [B][H][ns_pad]: |hi + lo|^2 of each stride-summed key row
  uint32_t* kmax;             // [B][H]: largest |stride sum| of the head, as float bits
  int32_t* flags;             // [B][H][ns_pad / 128]: query tiles that need the two-pass recompute
  float* u;                   // [B][H][nb][ns_pad]: per (key block, row) sums against the reference
  int32_t gate;               // two-pass kernel: 1 = only the flagged query tiles
};

// Queue the search kernels on `stream`; non-null events are recorded
// before the first and after the last.
hipError_t launch_rr_search(const RrParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Token re-permutation between serialisation orders (reorder.hip).
struct ReorderParams {
  const uint16_t* in;
  uint16_t* out;
  int64_t in_sb, in_sl, in_sh;    // element strides
  int64_t out_sb, out_sl, out_sh;
  int32_t B, L, H, D;             // D a multiple of 8
  int32_t gh, gw;                 // grid rows and columns (L = gh * gw)
  int32_t from, to;               // 0 raster, 1 2x2-block row-major, 2 2x2-block column-major
};

hipError_t launch_reorder(const ReorderParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// One-query decode attention over a key/value cache (decode.hip).
struct DecodeParams {
  const uint16_t* q;          // [B, H, D] (one query token per sequence)
  const uint16_t* k;          // cache [B, Lmax, Hkv, D]
  const uint16_t* v;
  uint16_t* o;                // [B, H, D]
  int64_t q_sb, q_sh;         // element strides
  int64_t k_sb, k_sl, k_sh;
  int64_t v_sb, v_sl, v_sh;
  int64_t o_sb, o_sh;
  const int32_t* seq_lens;    // device [B]: cached tokens n_b (the query is token n_b - 1)
  const float* sink;          // [H] or nullptr
  float* partials;            // [B][H][nsplit][D + 2] when nsplit > 1: acc, reference, denominator
  float scale_log2;           // softmax scale * log2(e)
  int32_t B, H, G;            // G = query heads per K/V head (<= 16)
  int32_t max_len;            // bound applied to seq_lens (<= Lmax)
  int32_t window;             // keys [n - window, n); <= 0: every cached key
  int32_t prefix;             // keys [0, prefix) as well
  int32_t nsplit, chunk;      // key splits and keys per split (a multiple of 64)
};

// Queue the decode kernel (and, with nsplit > 1, the split merge) on `stream`.
hipError_t launch_decode(const DecodeParams& p, int D, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

}  // namespace bss
