/*
 * bss_attn.h — C ABI of the structured-mask softmax attention library (gfx950).
 *
 * The library computes the forward pass
 *
 *     O = Softmax( Q K^T / sqrt(d)  restricted to the allowed keys N(i),
 *                  optionally with a per-head sink logit in the denominator ) V
 *
 * for bf16 Q, K, V with float32 accumulation, writing bf16 O.
 *   - Scores and the row-wise softmax follow "Vision transformers and hybrid
 *     architectures", section 2 (score_ij = q_i.k_j/sqrt(d), row softmax, z_i = sum_j a_ij v_j).
 *   - The allowed-key sets N(i) (full, chunk window, sliding window with l left
 *     and r right) follow the mask slide of "Semantic Head Specialization Guides
 *     Hybrid ViT Attention for Multimodal LLMs"; the sliding window is inclusive
 *     at both ends (that page's serialisation slide: anchor 15 with 8 per side
 *     covers tokens 7..23).
 *   - Per-head causal windows of W keys ("Asymmetric Attention Heads", Table 2)
 *     are the WINDOW kind with causal = 1 and head_left[h] = W_h - 1.
 *   - The block-selection matrix B in {0,1}^{Nb x Nb}, Nb = ceil(L/Bs), is
 *     expanded to tokens as M[i,j] = B[i/Bs][j/Bs] and j <= i ("RRAttention",
 *     section 2.1, Eq. 1-2); B[m][n] = 1 with n > m violates Eq. 5 and is rejected.
 *     A zero entry of B skips the pair (its weight is exactly 0).
 *   - The sink s_aux[h] is a logit with no value that only enlarges the
 *     denominator; -inf means no sink (SHS slides, the sink-bias slide, "Eq. 1").
 *   - A row with no allowed key is written as zeros.
 *
 * Conventions shared by every entry point
 *   - Device tensors are views: element strides for batch, token and head; the
 *     head dimension is contiguous (stride 1).  Every row start must be 16-byte
 *     aligned (D and all strides multiples of 8 elements, 16-byte aligned base).
 *   - The caller owns every device buffer (Q, K, V, O, sink, workspace).  The
 *     library never allocates or frees device memory.  Host arrays passed in a
 *     mask descriptor are only read during the call; a plan copies what it needs.
 *   - Launches are asynchronous on the given HIP stream: they enqueue the
 *     kernel and return.  A kernel fault surfaces at the caller's next
 *     synchronisation as a HIP error.  Copying a plan's device image
 *     (attn_plan_upload, attn_bwd_upload, and attn_masked_fwd when the
 *     workspace does not hold that plan's image yet) stages it in pageable
 *     host memory and synchronises the stream once.
 *   - Functions return attn_status and never throw or abort.  On a non-OK status
 *     attn_last_error() returns a message (thread-local, valid until the next call
 *     on that thread).
 *   - Supported head dims: 64, 80, 128 and 256 for the forward entry points;
 *     64, 80, 128 for the backward and the pattern search.  Batch B >= 1.  Lq == Lk.  K and V may
 *     have fewer heads than Q (grouped-query attention, see attn_tensor).
 */
#ifndef BSS_ATTN_H
#define BSS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVAL = -1,       /* malformed argument: shapes, strides, alignment, descriptor fields */
  ATTN_E_UNSUPPORTED = -2, /* well-formed but outside what the kernels implement (e.g. D = 96)   */
  ATTN_E_WORKSPACE = -3,   /* workspace missing or smaller than attn_plan_workspace_bytes        */
  ATTN_E_HIP = -4,         /* a HIP runtime call failed; the message carries hipGetErrorString   */
  ATTN_E_NOMEM = -5        /* host allocation failed while compiling a plan                      */
} attn_status;

typedef enum {
  ATTN_MASK_FULL = 0,   /* every key                                                   */
  ATTN_MASK_CHUNK = 1,  /* floor(i/chunk) == floor(j/chunk): non-overlapping chunks     */
  ATTN_MASK_WINDOW = 2, /* i - left_h <= j <= i + right (inclusive)                      */
  ATTN_MASK_BLOCK = 3   /* B_h[i/block][j/block] == 1 and j <= i                         */
} attn_mask_kind;

/* A bf16 device tensor view of logical shape [B, L, H, D]. */
/* K and V may have fewer heads than Q (grouped-query attention): Q's head count
 * must be a multiple of theirs, and query head h reads K/V head h / (Hq / Hkv),
 * so each run of Hq / Hkv consecutive query heads shares one ("sliding window
 * vs linear attention" article: 32 query heads sharing 8 key-value heads). */
typedef struct {
  void* data;                 /* device pointer to element [0,0,0,0]                  */
  int64_t B, L, H, D;         /* batch, tokens, heads, head dim                       */
  int64_t stride_b, stride_l, stride_h; /* element strides; the D stride is 1          */
} attn_tensor;

/* Which keys each query may see.  Unused fields are ignored for a given kind. */
typedef struct {
  int32_t kind;               /* attn_mask_kind                                        */
  int32_t causal;             /* 1: additionally require j <= i (FULL, CHUNK, WINDOW); BLOCK is always causal */
  int64_t chunk;              /* CHUNK: C >= 1                                         */
  int64_t left, right;        /* WINDOW: reach to the left and to the right, >= 0      */
  const int64_t* head_left;   /* WINDOW, optional host [H]: per-head left reach (overrides left) */
  int64_t block;              /* BLOCK: token block size Bs >= 1                       */
  const uint8_t* block_mask;  /* BLOCK: host [Hb][Nb][Nb] row-major 0/1, Nb = ceil(L/Bs) */
  int32_t block_mask_heads;   /* BLOCK: Hb = 1 (shared by all heads) or H             */
  int64_t prefix;             /* FULL, CHUNK, WINDOW: keys 0 .. prefix-1 are added to every query's
                                 set before the causal cut (the StreamingLLM sink tokens kept beside a
                                 window, e.g. 572 + 4); 0 = none; must be 0 for BLOCK              */
} attn_mask_desc;

/* Launch context. */
typedef struct {
  void* stream;               /* hipStream_t; NULL = the default stream               */
  void* workspace;            /* device memory of at least workspace_bytes            */
  size_t workspace_bytes;
  float softmax_scale;        /* <= 0 selects 1/sqrt(D)                                */
  void* start_event;          /* optional hipEvent_t (created by the caller): records when the
                                 attention kernel starts (hipExtLaunchKernel); NULL = none   */
  void* stop_event;           /* optional hipEvent_t: records when the kernel ends          */
} attn_launch;

/* Opaque compiled mask: tile lists, schedule and the device image layout. */
typedef struct attn_plan attn_plan;

/*
 * One-shot forward.  Finds the plan for `mask` in an internal cache, or
 * compiles and caches it, makes sure launch->workspace holds its device image
 * and launches the kernel on launch->stream.
 *   q, k, v : bf16 [B, L, H, D] inputs (same B, L, H, D).
 *   mask    : host descriptor.
 *   sink    : NULL, or device float32 [H] sink logits.
 *   o       : bf16 [B, L, H, D] output (may not alias q, k or v).
 * Plan cache: a lookup hashes the descriptor's content (its fields, the
 * per-head left reaches and the block matrix, with L, H, D) a machine word at
 * a time, and a hit also compares that content with the cached entry's copy,
 * so descriptors that merely share a hash never share a plan.  At most 16
 * plans and about 2 GiB of host memory are kept, least recently used evicted
 * first.
 * Workspace: the library records which plan image each workspace holds (this
 * call, attn_plan_upload and attn_bwd_upload record their uploads) and copies
 * the image only when the workspace does not hold this plan's: repeated calls
 * with the same mask and workspace neither copy nor synchronise.  A caller
 * that frees the workspace or uses its memory for anything else must call
 * attn_workspace_release first (or upload another image into it through this
 * library).  Required size: attn_plan_workspace_bytes of the same plan (query
 * it with attn_workspace_bytes below).  Errors: ATTN_E_INVAL,
 * ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP, ATTN_E_NOMEM.
 */
attn_status attn_masked_fwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                            const attn_mask_desc* mask, const float* sink, attn_tensor* o,
                            const attn_launch* launch);

/* Workspace bytes attn_masked_fwd needs for this descriptor and shape. */
attn_status attn_workspace_bytes(const attn_mask_desc* mask, int64_t L, int64_t H, int64_t D,
                                 size_t* bytes);

/*
 * Allocation-free one-shot forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same computation, tensors and plan cache as
 * attn_masked_fwd, but the plan image and the split rows' partial states live
 * in a static device array of the library (32 MiB, one per GPU, held until
 * the process ends) instead of a caller workspace: launch->workspace must be
 * NULL and launch->workspace_bytes 0.  The call allocates no device memory
 * and calls no allocating library routine.  The image is copied (and the
 * stream synchronised once) only when the GPU's array does not hold this
 * plan's image already.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap in time on one GPU race
 * (serialise them, e.g. on one stream).  Errors: as attn_masked_fwd, plus
 * ATTN_E_WORKSPACE when the launch needs more than the 32 MiB (the message
 * gives the bytes needed) and ATTN_E_INVAL when a workspace is passed.
 */
attn_status attn_masked_fwd_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                    const attn_mask_desc* mask, const float* sink, attn_tensor* o,
                                    const attn_launch* launch);

/*
 * Forget whatever plan image `workspace` (a device address passed earlier as
 * a workspace) holds: the next attn_masked_fwd with it copies the image again,
 * and attn_masked_bwd refuses it until attn_bwd_upload.  Call it before
 * freeing that memory or reusing it for other data.  Never fails (an unknown
 * address is ignored); returns ATTN_OK.
 */
attn_status attn_workspace_release(const void* workspace);

/*
 * Mask-descriptor compiler.  Validates `mask` against (L, H, D) and builds, for
 * every (head, query tile), the ascending list of key tiles that hold at least
 * one allowed pair, each flagged FULL or PARTIAL, plus the work schedule.
 * Errors: ATTN_E_INVAL (bad descriptor; B violating Eq. 5), ATTN_E_UNSUPPORTED
 * (D not in {64, 80, 128, 256}), ATTN_E_NOMEM.  *out is set only on ATTN_OK.
 */
attn_status attn_plan_create(const attn_mask_desc* mask, int64_t L, int64_t H, int64_t D,
                             attn_plan** out);

/*
 * Canonical tile lists (host views owned by the plan, valid until destroy).
 * Rows are (head, query tile) in row-major order, n_rows = H * ceil(L/bm);
 * row_ptr[n_rows+1]; kv_tile[nnz] ascending within a row; flags[nnz]: 1 = FULL
 * (the whole bm x bn rectangle is inside the sequence and allowed), 0 = PARTIAL.
 */
attn_status attn_plan_tiles(const attn_plan* plan, int32_t* bm, int32_t* bn, int64_t* n_rows,
                            int64_t* nnz, const int32_t** row_ptr, const int32_t** kv_tile,
                            const uint8_t** flags);

/* Allowed (query, key) pairs: per head into pairs_per_head[H] (may be NULL) and in total. */
attn_status attn_plan_pairs(const attn_plan* plan, int64_t* pairs_per_head, int64_t* total);

/*
 * Work schedule of a batch-1 launch: n_items records of 8 int32 {head, query
 * tile, first list entry, one past the last list entry, partial slot, piece,
 * pieces, split row}, laid out as 8 equal-length queues (queue x = records
 * [x n_items/8, (x+1) n_items/8), run by the work-groups of XCD x in order).
 * Every (head, query tile) row is covered once: by one record (pieces = 1;
 * empty rows too: they write zeros) or, when its list is long compared with
 * the launch, by `pieces` records that cut the list into consecutive ranges;
 * each piece leaves its partial softmax state in partial slot (slot + piece)
 * of the workspace, and a second kernel of the same launch merges the pieces
 * of each split row in piece order.
 * Records with head = -1 pad the queues.  Launches with batch > 1 run an
 * unsplit schedule of the same layout.  Host view owned by the plan.
 */
attn_status attn_plan_schedule(const attn_plan* plan, int64_t* n_items, const int32_t** items);

/*
 * Forward kernel the plan's launches run (for profiling and tests):
 *   ATTN_KERNEL_SWIZZLED  head dims 64, 80: one wave group, XOR-swizzled LDS
 *                         tiles, two tiles in flight per iteration;
 *   ATTN_KERNEL_SINGLE    head dims 128 (rows of fewer than about 32 tiles on
 *                         average: two work-groups per CU) and 256;
 *   ATTN_KERNEL_PINGPONG  head dim 128 with long rows: two wave groups per
 *                         work-group taking alternate tiles, MFMA and softmax
 *                         phases alternating between the two waves of a SIMD.
 * A grouped launch runs the ping-pong kernel only when all its plans do.
 */
enum { ATTN_KERNEL_SWIZZLED = 0, ATTN_KERNEL_SINGLE = 1, ATTN_KERNEL_PINGPONG = 2 };
attn_status attn_plan_kernel(const attn_plan* plan, int32_t* kernel);

/*
 * Device bytes a launch needs in the workspace: the plan's image (tile lists,
 * schedules, the list of split rows) followed, for batch-1 launches, by the
 * partial states of split rows.  Launches that share a workspace must not
 * overlap in time (the partial states are per launch; launches on one stream
 * are ordered).
 */
attn_status attn_plan_workspace_bytes(const attn_plan* plan, size_t* bytes);

/* Copy the plan's device image into `workspace` on `stream` (returns once copied). */
attn_status attn_plan_upload(const attn_plan* plan, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Forward with a compiled plan whose image the caller has already uploaded
 * into launch->workspace with attn_plan_upload.  Same tensors and errors as
 * attn_masked_fwd; q/k/v/o must match the plan's L, H, D.
 */
attn_status attn_masked_fwd_plan(const attn_plan* plan, const attn_tensor* q, const attn_tensor* k,
                                 const attn_tensor* v, const float* sink, attn_tensor* o,
                                 const attn_launch* launch);

/*
 * Grouped forward: n (1..8) independent launches with the same head dim D and
 * batch B run as one kernel, whose work-groups take the items of every launch
 * (the per-XCD queues of launch 0, then of launch 1, ...).  It serves a layer
 * whose heads use different masks (the hybrid ViT of "Semantic Head
 * Specialization ...": full, chunk and sliding-window heads side by side) and
 * any set of masks applied together, with one dispatch instead of n.
 *   plans[j], q[j], k[j], v[j], sinks[j] (sinks may be NULL, or hold NULL
 *   entries), o[j]: as for attn_masked_fwd_plan; plans[j]'s image must have
 *   been uploaded into workspaces[j] (workspace_bytes[j] long, at least
 *   attn_plan_workspace_bytes).  Workspaces and outputs must be distinct
 *   (outputs must not overlap at all: that is not checked beyond the base
 *   pointers).  launch: stream, softmax_scale and the optional events; its
 *   workspace fields are ignored.
 * Errors: as attn_masked_fwd_plan for each launch (the message names it);
 * ATTN_E_INVAL for n < 1, NULL arrays, differing D or B, shared workspaces or
 * outputs; ATTN_E_UNSUPPORTED for n > 8.
 */
attn_status attn_masked_fwd_group(int32_t n, const attn_plan* const* plans, const attn_tensor* q,
                                  const attn_tensor* k, const attn_tensor* v, const float* const* sinks,
                                  attn_tensor* o, void* const* workspaces, const size_t* workspace_bytes,
                                  const attn_launch* launch);

/*
 * Forward that also writes the log-sum-exp of every row, which the backward
 * needs:  lse[b][h][i] = ln( sum over allowed j of exp(s_ij) + exp(s_aux[h]) )
 * with s_ij = softmax_scale q_i.k_j; -inf for a row with neither an allowed
 * key nor a sink.  lse: device float32 [B][H][L], contiguous, 4-byte aligned.
 * Everything else as attn_masked_fwd_plan (a backward workspace prepared by
 * attn_bwd_upload serves as the forward workspace too).
 */
attn_status attn_masked_fwd_lse(const attn_plan* plan, const attn_tensor* q, const attn_tensor* k,
                                const attn_tensor* v, const float* sink, attn_tensor* o, float* lse,
                                const attn_launch* launch);

/*
 * Backward pass.  For a loss with upstream gradient dO = dL/dO, the chain rule
 * through O = P V and the masked row softmax P (the same definition as the
 * forward; s_aux enters the denominator only) gives, per (batch, head), with
 * sigma = softmax_scale and p_ij = exp(s_ij - lse_i) on allowed pairs (0 elsewhere):
 *   D_i = dO_i . O_i,   dS_ij = p_ij (dO_i . v_j - D_i),
 *   dQ_i = sigma sum_j dS_ij k_j,   dK_j = sigma sum_i dS_ij q_i,   dV_j = sum_i p_ij dO_i,
 *   d s_aux[h] = - sum over b, i of exp(s_aux[h] - lse_i) D_i.
 * With grouped-query heads, dK and dV of a K/V head sum over its query heads.
 * The masks are those the pages train ("Semantic Head Specialization ...":
 * the ViT variants with full / chunk / sliding-window heads; "Asymmetric
 * Attention Heads": per-head causal windows); masked-out tiles are skipped,
 * as in the forward.
 *
 * Workspace: attn_bwd_workspace_bytes(plan, B, kv_heads) bytes, prepared once
 * by attn_bwd_upload(plan, kv_heads, ...) (it holds the plan's forward image,
 * the transposed tile lists and dK/dV schedules for kv_heads K/V heads, then
 * per-row statistics written by every backward launch and, for batch 1, the
 * partial sums of the long query rows and key blocks that the launch splits
 * over several work-groups and merges in a fixed order).  Launches sharing a
 * workspace must not overlap in time.  Plans of head dim 256 are refused with
 * ATTN_E_UNSUPPORTED by every backward entry point.
 */
attn_status attn_bwd_workspace_bytes(const attn_plan* plan, int64_t B, int64_t kv_heads, size_t* bytes);

/*
 * Transposed tile lists of the backward for kv_heads K/V heads (host views
 * owned by the plan, valid until destroy).  Key blocks are 128 keys (two key
 * tiles), n_blocks = ceil(L/128); rows are (K/V head, key block) in row-major
 * order, col_ptr[kv_heads * n_blocks + 1].  An entry is
 * (g << 24) | (query tile << 1) | full: query tile (of bm rows) of query head
 * kv_head * (H / kv_heads) + g lists at least one of the block's key tiles;
 * full = the whole 128-row x 128-key rectangle (clipped to the key tiles that
 * exist) lies inside the sequence and is allowed.  Entries are ordered by g,
 * then query tile.  items: the dK/dV work schedule, n_items records of 8 int32
 * {kv head, key block, first entry, one past the last, 0, 0, 1, 0} in 8 equal
 * queues like attn_plan_schedule (kv head -1 pads).
 */
attn_status attn_bwd_lists(const attn_plan* plan, int64_t kv_heads, int64_t* n_blocks, const int32_t** col_ptr,
                           int64_t* n_entries, const int32_t** entries, int64_t* n_items, const int32_t** items);

/* Copy the forward and backward images into `workspace` on `stream` (returns
 * once copied); kv_heads must divide the plan's H (at most 127 query heads per
 * K/V head). */
attn_status attn_bwd_upload(const attn_plan* plan, int64_t kv_heads, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Gradients of the forward with the same plan, inputs, sink and softmax_scale.
 *   q, k, v, o : the forward's bf16 inputs and output ([B, L, H, D]; k, v with
 *                kv_heads heads); dout: bf16 dL/dO [B, L, H, D].
 *   lse        : device float32 [B][H][L] written by attn_masked_fwd_lse.
 *   sink       : NULL or device float32 [H] (as in the forward).
 *   dq         : bf16 [B, L, H, D] output; dk, dv: bf16 [B, L, kv_heads, D]
 *                outputs (written entirely; distinct, not aliasing any input).
 *   dsink      : NULL, or device float32 [H] output (zeros when sink is NULL).
 *   launch     : stream, workspace (prepared by attn_bwd_upload for k->H K/V
 *                heads), softmax_scale, optional events (start of the first
 *                and end of the last of the backward kernels).
 * Asynchronous.  Errors: ATTN_E_INVAL (shapes, strides, aliasing, NULL
 * arguments, a workspace not prepared for this plan and K/V head count),
 * ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP, ATTN_E_NOMEM.
 */
attn_status attn_masked_bwd(const attn_plan* plan, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                            const attn_tensor* o, const attn_tensor* dout, const float* lse, const float* sink,
                            attn_tensor* dq, attn_tensor* dk, attn_tensor* dv, float* dsink,
                            const attn_launch* launch);

/*
 * RRAttention block-pattern search ("RRAttention", section 3, Eq. 6-12): from
 * Q and K to the block matrix B consumed by the BLOCK mask kind.
 *   Eq. 6-7  head h samples query P(i,h) = iS + (S-1-(h mod S)) of every full
 *            stride i = 0 .. floor(L/S)-1;
 *   Eq. 8    I_ij = q_P(i,h) . (sum of the keys of stride j) / (S sqrt(D));
 *   Eq. 9    softmax of each row over the causal key strides j <= i (the
 *            attention it feeds is causal, Eq. 2 and 5);
 *   Eq. 10   S_mn = sum of those probabilities over the strides of query
 *            block m and key block n (stride i lies in block iS / block);
 *   Eq. 11   per query block, the shortest prefix of S_m,n (n <= m) sorted
 *            in descending order (ties: lower n first) whose mass reaches
 *            tau times the row's mass;
 *   Eq. 12   with protect_last, every causal block of the last query block.
 * The stride importance runs on bf16 MFMA with fp32 accumulation; each stride
 * sum of the keys is formed in fp32 and carried as a pair of bf16 values
 * (hi + lo, the fp32 sum to about 2^-16 relative), so the products see the
 * key aggregate at fp32 accuracy.  One pass over the key strides takes each
 * row's probabilities against a fixed reference above every score of the row
 * (|q| times the head's largest key-aggregate norm); rows whose sum against it
 * underflows are recomputed exactly by a two-pass kernel.  The selection
 * compares fp32 sums.  The workspace holds the per (key block, row) sums of
 * the pass: 4 bytes per row and key block, with a row for every stride of
 * every block (Nb * block / stride rows, padded to a multiple of 256; 2 GiB at
 * 128K tokens, 32 heads, stride 8, block 128).
 */
typedef struct {
  int64_t stride;             /* S >= 1                                                   */
  int64_t block;              /* block size Bs: a multiple of S with Bs / S in {8, 16, 32} */
  float tau;                  /* threshold in (0, 1]                                      */
  int32_t protect_last;       /* 1: keep every causal block of the last query block      */
} attn_rr_params;

/* Workspace bytes attn_rr_search needs for q's shape (B, L, H, D) and prm. */
attn_status attn_rr_workspace_bytes(const attn_tensor* q, const attn_rr_params* prm, size_t* bytes);

/*
 * Run the search on launch->stream (asynchronous; launch->workspace of at least
 * attn_rr_workspace_bytes; optional events bracket all of its kernels).
 *   q, k         : bf16 [B, L, H, D] device views (same shape; D in {64, 80, 128}).
 *   block_mask   : device uint8 [B][H][Nb][Nb], Nb = ceil(L / block): written
 *                  entirely (1 = compute the block pair; zero above the diagonal).
 *   block_score  : device float [B][H][Nb][Nb]: the block scores S_mn (zero
 *                  above the diagonal).
 * Errors: ATTN_E_INVAL (shapes, strides, NULL pointers, stride/block/tau out of
 * range, L < stride), ATTN_E_UNSUPPORTED (D, block / stride not in {8, 16, 32},
 * Nb > 4096), ATTN_E_WORKSPACE, ATTN_E_HIP.
 */
attn_status attn_rr_search(const attn_tensor* q, const attn_tensor* k, const attn_rr_params* prm,
                           void* block_mask, void* block_score, const attn_launch* launch);

/*
 * Token serialisation orders of a grid_h x grid_w patch grid ("Semantic Head
 * Specialization ...", the Factor-2 slides and the Ariadne design):
 *   RASTER      row by row, position r * grid_w + c;
 *   BLOCK_ROW   (c) 2 x 2 blocks left to right, then top to bottom, the 4
 *               patches of a block row by row;
 *   BLOCK_COL   (d) the BLOCK_ROW order of the transposed grid: blocks top to
 *               bottom, then left to right, a block's patches column by column.
 * The block orders need even grid sides.
 */
typedef enum { ATTN_ORDER_RASTER = 0, ATTN_ORDER_BLOCK_ROW = 1, ATTN_ORDER_BLOCK_COL = 2 } attn_token_order;

/*
 * Re-permute the tokens of `in` (in order `from`) into `out` (order `to`):
 * out[b, t, h, :] = in[b, s, h, :] where s is the position, in order `from`,
 * of the patch that order `to` puts at t (Ariadne's re-permutation where the
 * layer order changes).  in, out: bf16 [B, L, H, D] device views with
 * L = grid_h * grid_w, any D that is a multiple of 8 (16-byte rows), same
 * shape; they must not overlap.  Asynchronous on launch->stream; optional
 * events mark the kernel; launch->workspace is not used.
 * Errors: ATTN_E_INVAL (shapes, strides, orders, odd grid for a block order,
 * out == in), ATTN_E_HIP.
 */
attn_status attn_reorder_tokens(const attn_tensor* in, int32_t from, attn_tensor* out, int32_t to,
                                int64_t grid_h, int64_t grid_w, const attn_launch* launch);

/*
 * One-query (decode) attention over a key/value cache.  The sliding-window
 * vs linear attention article generates with a causal window of the last W
 * cached tokens ("comparison at equal memory": 576 tokens with a learned
 * per-head sink, or 572 plus 4 StreamingLLM sink tokens) on grouped-query
 * heads (32 query heads on 8 key/value heads at head dim 128; its speed test
 * 16 on 4 at head dim 256).  For sequence b with n = seq_lens[b] cached
 * tokens the query is token n - 1, and its allowed keys are
 *     the window  n - W <= j <= n - 1   (W <= 0: every cached key, j < n)
 *     the prefix  j < P                 (P = 0: none),
 * the same set that the WINDOW mask with causal = 1, left = W - 1 and
 * prefix = P gives that row in the prefill.  Softmax, sink and empty rows as
 * for attn_masked_fwd.
 */
typedef struct {
  int64_t window;             /* W: window length in keys (query included); <= 0 = every cached key */
  int64_t prefix;             /* P >= 0: leading keys always allowed                          */
} attn_decode_desc;

/* Workspace bytes attn_decode_fwd needs for these shapes (0 when the keys of
 * a sequence are not split over several work-groups). */
attn_status attn_decode_workspace_bytes(const attn_tensor* q, const attn_tensor* k_cache, int64_t max_len,
                                        const attn_decode_desc* desc, size_t* bytes);

/*
 * Decode step on launch->stream (asynchronous; optional events bracket its
 * one or two kernels).
 *   q        : bf16 [B, 1, H, D] device view, one query token per sequence; D in {64, 128, 256}.
 *   k_cache, v_cache : bf16 [B, Lmax, Hkv, D] device views; H a multiple of Hkv
 *              with H / Hkv <= 16 (query head h reads cache head h / (H / Hkv)).
 *   seq_lens : device int32 [B]: cached tokens of each sequence; values are
 *              clamped to [0, max_len] (0: the output row is zero).
 *   max_len  : host bound on seq_lens, 0 <= max_len <= Lmax; it sizes the
 *              split of the keys over work-groups.
 *   desc     : host descriptor (window, prefix).
 *   sink     : NULL, or device float32 [H] sink logits.
 *   o        : bf16 [B, 1, H, D] output (must not alias the inputs).
 * Workspace: attn_decode_workspace_bytes bytes (may be NULL when that is 0);
 * launches that share a workspace must not overlap in time.
 * Errors: ATTN_E_INVAL (shapes, strides, alignment, NULL pointers, negative
 * prefix, max_len out of range), ATTN_E_UNSUPPORTED (D, H / Hkv > 16, a cache
 * too large for 32-bit row offsets), ATTN_E_WORKSPACE, ATTN_E_HIP.
 */
attn_status attn_decode_fwd(const attn_tensor* q, const attn_tensor* k_cache, const attn_tensor* v_cache,
                            const int32_t* seq_lens, int64_t max_len, const attn_decode_desc* desc,
                            const float* sink, attn_tensor* o, const attn_launch* launch);

/* Free a plan (NULL is allowed). */
void attn_plan_destroy(attn_plan* plan);

/*
 * Range checks of the checked build (libbss_attn_checked.so, built from the
 * same sources with BSS_CHECKED): before a forward work-group or split-row
 * merge touches memory, it checks its work item (head, query tile, list range,
 * piece and partial slot), the key tiles the item lists and the pointers it
 * needs against the launch's sizes; on a violation it ORs these bits into the
 * device's check word and returns without computing:
 *   1 head, 2 query tile, 4 list range, 8 piece or slot, 16 listed key tile,
 *   32 split-row record, 64 NULL pointer.
 * *enabled (optional): 1 in the checked build, 0 otherwise (bits stay 0).
 * *bits (optional): the current device's check word; the caller synchronizes
 * the launches first.  clear != 0 zeroes the word after reading it.
 * Errors: ATTN_E_HIP.
 */
attn_status attn_checks(int32_t* enabled, uint32_t* bits, int32_t clear);

/* Message for the last non-OK status on this thread ("" if none). */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSS_ATTN_H */
