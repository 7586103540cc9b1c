// C ABI of the library: validation, the plan cache, uploads and launches.
// Every entry point returns an attn_status; nothing throws across the ABI.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <initializer_list>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "bss_attn.h"
#include "kernels.hpp"
#include "plan.hpp"
#include "plan_cache.hpp"

namespace bss {

namespace {
thread_local std::string g_last_error;

// Compiled plans of the one-shot entry point, by descriptor content: at most
// 16 plans and about 2 GiB of host memory, least recently used evicted first.
PlanCache g_cache(16, size_t(2) << 30);
// Which plan image each caller workspace holds.
UploadTags g_tags;

// Per device: the plan whose image the allocation-free scratch holds (kept
// alive, so its serial is not reused while it is recorded here).
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
std::shared_ptr<const attn_plan> g_scratch_plan[kScratchDevices];

attn_status hip_fail(hipError_t e, const char* what) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return ATTN_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

attn_status check_tensor(const attn_tensor* t, const char* name, int64_t B, int64_t L, int64_t H,
                         int64_t D) {
  if (!t) { set_error(std::string(name) + " is NULL"); return ATTN_E_INVAL; }
  if (!t->data) { set_error(std::string(name) + ".data is NULL"); return ATTN_E_INVAL; }
  if (t->B != B || t->L != L || t->H != H || t->D != D) {
    set_error(std::string(name) + " shape differs from q (or from the plan)");
    return ATTN_E_INVAL;
  }
  if (t->stride_b < 0 || t->stride_l < D || t->stride_h < 0) {
    set_error(std::string(name) + " has a negative or overlapping stride");
    return ATTN_E_INVAL;
  }
  if (!aligned16(t->data) || (t->stride_b % 8) || (t->stride_l % 8) || (t->stride_h % 8)) {
    set_error(std::string(name) + " rows must start on 16-byte boundaries (strides multiple of 8)");
    return ATTN_E_INVAL;
  }
  if (t->stride_l * 2 * 64 > INT32_MAX) {
    set_error(std::string(name) + " token stride too large");
    return ATTN_E_UNSUPPORTED;
  }
  return ATTN_OK;
}

// Validate one launch of plan p and fill its kernel parameters.  ws/ws_bytes:
// the workspace holding p's uploaded image (and the partial states).
attn_status make_job(const attn_plan& p, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                     const float* sink, attn_tensor* o, void* ws_ptr, size_t ws_bytes, float softmax_scale,
                     FwdParams* out, int32_t* queue_len) {
  if (!q) { set_error("q is NULL"); return ATTN_E_INVAL; }
  const int64_t B = q->B;
  if (B < 1 || B > 65535) { set_error("batch must be in [1, 65535]"); return ATTN_E_INVAL; }
  attn_status st;
  if ((st = check_tensor(q, "q", B, p.L, p.H, p.D)) != ATTN_OK) return st;
  // grouped-query attention: K and V may have fewer heads, a divisor of Q's
  if (!k || !v) { set_error("k or v is NULL"); return ATTN_E_INVAL; }
  const int64_t hkv = k->H;
  if (hkv < 1 || p.H % hkv != 0 || v->H != hkv) {
    set_error("k and v need the same number of heads, a divisor of q's (" + std::to_string(p.H) + ")");
    return ATTN_E_INVAL;
  }
  if ((st = check_tensor(k, "k", B, p.L, hkv, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(v, "v", B, p.L, hkv, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(o, "o", B, p.L, p.H, p.D)) != ATTN_OK) return st;
  if (o->data == q->data || o->data == k->data || o->data == v->data) {
    set_error("o must not alias q, k or v");
    return ATTN_E_INVAL;
  }
  if (p.kind == ATTN_MASK_BLOCK && !p.block_aligned) {
    set_error("block size must be a multiple of 128 for the GPU kernel");
    return ATTN_E_UNSUPPORTED;
  }
  // batch 1 runs the split schedule, whose partial states follow the image
  const bool split = (B == 1);
  const size_t need = split ? p.layout.total : p.layout.bytes;
  if (!ws_ptr || ws_bytes < need) {
    set_error("workspace smaller than attn_plan_workspace_bytes (" + std::to_string(p.layout.total) +
              " bytes)");
    return ATTN_E_WORKSPACE;
  }
  const size_t n_items = split ? p.items.size() : p.items_unsplit.size();
  if (n_items % 8 != 0 || n_items / 8 > static_cast<size_t>(INT32_MAX / 8)) {
    set_error("too many work items");
    return ATTN_E_UNSUPPORTED;
  }
  if (!aligned16(ws_ptr)) { set_error("workspace must be 16-byte aligned"); return ATTN_E_INVAL; }
  const uint8_t* ws = static_cast<const uint8_t*>(ws_ptr);
  FwdParams f{};
  f.q = static_cast<const uint16_t*>(q->data);
  f.k = static_cast<const uint16_t*>(k->data);
  f.v = static_cast<const uint16_t*>(v->data);
  f.o = static_cast<uint16_t*>(o->data);
  f.q_sb = q->stride_b; f.q_sl = q->stride_l; f.q_sh = q->stride_h;
  f.k_sb = k->stride_b; f.k_sl = k->stride_l; f.k_sh = k->stride_h;
  f.v_sb = v->stride_b; f.v_sl = v->stride_l; f.v_sh = v->stride_h;
  f.o_sb = o->stride_b; f.o_sl = o->stride_l; f.o_sh = o->stride_h;
  f.items = reinterpret_cast<const int32_t*>(ws + (split ? p.layout.off_items : p.layout.off_items_unsplit));
  f.kv = reinterpret_cast<const int32_t*>(ws + p.layout.off_kv);
  f.head_left = reinterpret_cast<const int32_t*>(ws + p.layout.off_head_left);
  f.block_bits = reinterpret_cast<const uint32_t*>(ws + p.layout.off_bits);
  f.partials = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + p.layout.off_partials);
  f.merge_rows = reinterpret_cast<const int32_t*>(ws + p.layout.off_merge);
  f.n_merge = split ? static_cast<int32_t>(p.merge_rows.size()) : 0;
  f.sink = sink;
  const float scale = softmax_scale > 0.f ? softmax_scale : static_cast<float>(1.0 / std::sqrt(double(p.D)));
  f.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  f.L = static_cast<int32_t>(p.L);
  f.H = static_cast<int32_t>(p.H);
  f.n_items = static_cast<int32_t>(n_items);
  f.kind = p.kind;
  f.causal = p.causal;
  f.chunk = static_cast<int32_t>(std::min<int64_t>(p.chunk, p.L));
  if (f.chunk < 1) f.chunk = 1;
  f.right = static_cast<int32_t>(p.right);
  f.prefix = static_cast<int32_t>(std::min<int64_t>(p.prefix, p.L));
  f.kv_group = static_cast<int32_t>(p.H / hkv);
  f.pingpong = p.pingpong ? 1 : 0;
  f.n_entries = static_cast<int32_t>(p.kv_entries.size());
  f.n_slots = split ? static_cast<int32_t>(p.n_partial_slots) : 0;
  *out = f;
  *queue_len = static_cast<int32_t>(n_items / 8);
  return ATTN_OK;
}

attn_status run_group(const GroupParams& g, int64_t D, int64_t B, const attn_launch* launch) {
  hipError_t e = launch_fwd(g, static_cast<int>(D), static_cast<int>(B), static_cast<hipStream_t>(launch->stream),
                            static_cast<hipEvent_t>(launch->start_event),
                            static_cast<hipEvent_t>(launch->stop_event));
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return ATTN_OK;
}

attn_status launch_with_plan(const attn_plan& p, const attn_tensor* q, const attn_tensor* k,
                             const attn_tensor* v, const float* sink, attn_tensor* o,
                             const attn_launch* launch) {
  if (!launch) { set_error("launch is NULL"); return ATTN_E_INVAL; }
  GroupParams g{};
  g.n_jobs = 1;
  attn_status st = make_job(p, q, k, v, sink, o, launch->workspace, launch->workspace_bytes,
                            launch->softmax_scale, &g.job[0], &g.queue_len[0]);
  if (st != ATTN_OK) return st;
  return run_group(g, p.D, q->B, launch);
}

attn_status upload(const attn_plan& p, void* workspace, size_t bytes, void* stream) {
  if (!workspace || bytes < p.layout.bytes) {
    set_error("workspace smaller than attn_plan_workspace_bytes (" + std::to_string(p.layout.bytes) +
              " bytes)");
    return ATTN_E_WORKSPACE;
  }
  std::vector<uint8_t> img;
  try {
    img.resize(p.layout.bytes);
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed for the plan image");
    return ATTN_E_NOMEM;
  }
  write_image(p, img.data());
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(workspace, img.data(), img.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan image)");
  // The staging buffer is pageable host memory that goes out of scope here.
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (plan image)");
  return ATTN_OK;
}

attn_status cached_plan(const attn_mask_desc* mask, int64_t L, int64_t H, int64_t D,
                        std::shared_ptr<const attn_plan>* out) {
  if (!mask) { set_error("mask descriptor is NULL"); return ATTN_E_INVAL; }
  // the arrays the content is read from must be there before the cache reads them
  if (mask->kind == ATTN_MASK_BLOCK && (!mask->block_mask || mask->block < 1 ||
                                        (mask->block_mask_heads != 1 && mask->block_mask_heads != H))) {
    set_error("BLOCK descriptor needs block >= 1, block_mask and block_mask_heads in {1, H}");
    return ATTN_E_INVAL;
  }
  if (H < 1 || L < 1) { set_error("L and H must be >= 1"); return ATTN_E_INVAL; }
  try {
    return g_cache.get(mask, L, H, D, out);
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed for the plan cache");
    return ATTN_E_NOMEM;
  }
}

}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }

}  // namespace bss

using namespace bss;

extern "C" {

attn_status attn_plan_create(const attn_mask_desc* mask, int64_t L, int64_t H, int64_t D,
                             attn_plan** out) {
  try {
    return compile_plan(mask, L, H, D, out);
  } catch (...) {
    set_error("unexpected exception while compiling the plan");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_plan_tiles(const attn_plan* p, int32_t* bm, int32_t* bn, int64_t* n_rows, int64_t* nnz,
                            const int32_t** row_ptr, const int32_t** kv_tile, const uint8_t** flags) {
  if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
  if (bm) *bm = p->bm;
  if (bn) *bn = p->bn;
  if (n_rows) *n_rows = static_cast<int64_t>(p->row_ptr.size()) - 1;
  if (nnz) *nnz = static_cast<int64_t>(p->kv_tile.size());
  if (row_ptr) *row_ptr = p->row_ptr.data();
  if (kv_tile) *kv_tile = p->kv_tile.data();
  if (flags) *flags = p->flags.data();
  return ATTN_OK;
}

attn_status attn_plan_pairs(const attn_plan* p, int64_t* pairs_per_head, int64_t* total) {
  if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
  if (pairs_per_head) std::memcpy(pairs_per_head, p->pairs.data(), p->pairs.size() * sizeof(int64_t));
  if (total) *total = p->pairs_total;
  return ATTN_OK;
}

attn_status attn_plan_schedule(const attn_plan* p, int64_t* n_items, const int32_t** items) {
  if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
  if (n_items) *n_items = static_cast<int64_t>(p->items.size());
  if (items) *items = reinterpret_cast<const int32_t*>(p->items.data());
  return ATTN_OK;
}

attn_status attn_checks(int32_t* enabled, uint32_t* bits, int32_t clear) {
  if (enabled) *enabled = checked_build() ? 1 : 0;
  if (!bits) return ATTN_OK;
  hipError_t e = check_bits(bits, clear != 0);
  if (e != hipSuccess) return hip_fail(e, "reading the check word");
  return ATTN_OK;
}

attn_status attn_plan_kernel(const attn_plan* p, int32_t* kernel) {
  if (!p || !kernel) { set_error("plan or kernel is NULL"); return ATTN_E_INVAL; }
  *kernel = p->D == 128 ? (p->pingpong ? ATTN_KERNEL_PINGPONG : ATTN_KERNEL_SINGLE)
                        : (p->D == 256 ? ATTN_KERNEL_SINGLE : ATTN_KERNEL_SWIZZLED);
  return ATTN_OK;
}

attn_status attn_plan_workspace_bytes(const attn_plan* p, size_t* bytes) {
  if (!p || !bytes) { set_error("plan or bytes is NULL"); return ATTN_E_INVAL; }
  *bytes = p->layout.total;
  return ATTN_OK;
}

attn_status attn_plan_upload(const attn_plan* p, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
  try {
    g_tags.forget(workspace);
    attn_status st = upload(*p, workspace, workspace_bytes, stream);
    if (st == ATTN_OK) g_tags.note(workspace, p->serial, 0);
    return st;
  } catch (...) {
    set_error("unexpected exception during upload");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_masked_fwd_plan(const attn_plan* p, const attn_tensor* q, const attn_tensor* k,
                                 const attn_tensor* v, const float* sink, attn_tensor* o,
                                 const attn_launch* launch) {
  if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
  try {
    return launch_with_plan(*p, q, k, v, sink, o, launch);
  } catch (...) {
    set_error("unexpected exception during launch");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_workspace_bytes(const attn_mask_desc* mask, int64_t L, int64_t H, int64_t D,
                                 size_t* bytes) {
  if (!bytes) { set_error("bytes is NULL"); return ATTN_E_INVAL; }
  try {
    std::shared_ptr<const attn_plan> p;
    attn_status st = cached_plan(mask, L, H, D, &p);
    if (st != ATTN_OK) return st;
    *bytes = p->layout.total;
    return ATTN_OK;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_masked_fwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                            const attn_mask_desc* mask, const float* sink, attn_tensor* o,
                            const attn_launch* launch) {
  try {
    if (!q) { set_error("q is NULL"); return ATTN_E_INVAL; }
    if (!launch) { set_error("launch is NULL"); return ATTN_E_INVAL; }
    std::shared_ptr<const attn_plan> p;
    attn_status st = cached_plan(mask, q->L, q->H, q->D, &p);
    if (st != ATTN_OK) return st;
    if ((st = check_tensor(q, "q", q->B, p->L, p->H, p->D)) != ATTN_OK) return st;
    // the image is copied only when the workspace does not hold this plan's already
    if (!g_tags.holds_forward(launch->workspace, p->serial)) {
      g_tags.forget(launch->workspace);
      st = upload(*p, launch->workspace, launch->workspace_bytes, launch->stream);
      if (st != ATTN_OK) return st;
      g_tags.note(launch->workspace, p->serial, 0);
    }
    return launch_with_plan(*p, q, k, v, sink, o, launch);
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_masked_fwd_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                    const attn_mask_desc* mask, const float* sink, attn_tensor* o,
                                    const attn_launch* launch) {
  try {
    if (!q) { set_error("q is NULL"); return ATTN_E_INVAL; }
    if (!launch) { set_error("launch is NULL"); return ATTN_E_INVAL; }
    if (launch->workspace != nullptr || launch->workspace_bytes != 0) {
      set_error("attn_masked_fwd_noalloc takes no workspace: launch->workspace must be NULL and workspace_bytes 0");
      return ATTN_E_INVAL;
    }
    std::shared_ptr<const attn_plan> p;
    attn_status st = cached_plan(mask, q->L, q->H, q->D, &p);
    if (st != ATTN_OK) return st;
    if ((st = check_tensor(q, "q", q->B, p->L, p->H, p->D)) != ATTN_OK) return st;
    void* scr = nullptr;
    size_t scr_bytes = 0;
    hipError_t e = fwd_scratch(&scr, &scr_bytes);
    if (e != hipSuccess) return hip_fail(e, "scratch address (hipGetSymbolAddress)");
    const size_t need = q->B == 1 ? p->layout.total : p->layout.bytes;
    if (need > scr_bytes) {
      set_error("this launch needs " + std::to_string(need) + " bytes of scratch (plan image and split-row states); "
                "attn_masked_fwd_noalloc has " + std::to_string(scr_bytes) +
                " per GPU: use attn_masked_fwd with a workspace");
      return ATTN_E_WORKSPACE;
    }
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices) { set_error("device index out of range"); return ATTN_E_UNSUPPORTED; }
    {
      // the image is copied only when this GPU's scratch does not hold it already
      std::lock_guard<std::mutex> lk(g_scratch_mu);
      if (!g_scratch_plan[dev] || g_scratch_plan[dev]->serial != p->serial) {
        g_scratch_plan[dev].reset();
        if ((st = upload(*p, scr, scr_bytes, launch->stream)) != ATTN_OK) return st;
        g_scratch_plan[dev] = p;
      }
    }
    attn_launch ln = *launch;
    ln.workspace = scr;
    ln.workspace_bytes = scr_bytes;
    return launch_with_plan(*p, q, k, v, sink, o, &ln);
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_workspace_release(const void* workspace) {
  try {
    g_tags.forget(workspace);
    return ATTN_OK;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_masked_fwd_group(int32_t n, const attn_plan* const* plans, const attn_tensor* q,
                                  const attn_tensor* k, const attn_tensor* v, const float* const* sinks,
                                  attn_tensor* o, void* const* workspaces, const size_t* workspace_bytes,
                                  const attn_launch* launch) {
  try {
    if (n < 1 || n > kMaxJobs) {
      set_error("a group holds 1 to " + std::to_string(kMaxJobs) + " launches");
      return n < 1 ? ATTN_E_INVAL : ATTN_E_UNSUPPORTED;
    }
    if (!plans || !q || !k || !v || !o || !workspaces || !workspace_bytes || !launch) {
      set_error("NULL array argument");
      return ATTN_E_INVAL;
    }
    GroupParams g{};
    g.n_jobs = n;
    for (int32_t j = 0; j < n; ++j) {
      if (!plans[j]) { set_error("plan " + std::to_string(j) + " is NULL"); return ATTN_E_INVAL; }
      if (plans[j]->D != plans[0]->D || q[j].B != q[0].B) {
        set_error("the launches of a group need the same head dim and batch");
        return ATTN_E_INVAL;
      }
      for (int32_t i = 0; i < j; ++i) {
        if (workspaces[i] == workspaces[j]) { set_error("the launches of a group need distinct workspaces"); return ATTN_E_INVAL; }
        if (o[i].data == o[j].data) { set_error("the launches of a group need distinct outputs"); return ATTN_E_INVAL; }
      }
      attn_status st = make_job(*plans[j], &q[j], &k[j], &v[j], sinks ? sinks[j] : nullptr, &o[j], workspaces[j],
                                workspace_bytes[j], launch->softmax_scale, &g.job[j], &g.queue_len[j]);
      if (st != ATTN_OK) {
        set_error("launch " + std::to_string(j) + " of the group: " + attn_last_error());
        return st;
      }
    }
    return run_group(g, plans[0]->D, q[0].B, launch);
  } catch (...) {
    set_error("unexpected exception during launch");
    return ATTN_E_NOMEM;
  }
}

namespace {

static bool overlaps_any(const void* x, std::initializer_list<const void*> others) {
  for (const void* o : others)
    if (o == x) return true;
  return false;
}

// Backward requests: the kernels cover head dims 64, 80 and 128.
static attn_status check_kv_heads(const attn_plan& p, int64_t kv_heads) {
  if (p.D > 128) {
    set_error("the backward supports head dims 64, 80 and 128 (plan has " + std::to_string(p.D) + ")");
    return ATTN_E_UNSUPPORTED;
  }
  if (kv_heads < 1 || p.H % kv_heads != 0) {
    set_error("kv_heads must divide the plan's head count (" + std::to_string(p.H) + ")");
    return ATTN_E_INVAL;
  }
  if (p.H / kv_heads > 127) { set_error("at most 127 query heads per K/V head"); return ATTN_E_UNSUPPORTED; }
  return ATTN_OK;
}

// Validate a backward launch and fill its kernel parameters.
static attn_status make_bwd(const attn_plan& p, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                     const attn_tensor* o, const attn_tensor* dout, const float* lse, const float* sink,
                     attn_tensor* dq, attn_tensor* dk, attn_tensor* dv, float* dsink, const attn_launch* launch,
                     BwdParams* out) {
  if (!launch) { set_error("launch is NULL"); return ATTN_E_INVAL; }
  if (!q || !k || !v || !o || !dout || !dq || !dk || !dv) {
    set_error("q, k, v, o, dout, dq, dk and dv are required");
    return ATTN_E_INVAL;
  }
  const int64_t B = q->B;
  if (B < 1 || B > 65535) { set_error("batch must be in [1, 65535]"); return ATTN_E_INVAL; }
  const int64_t hkv = k->H;
  if (hkv < 1 || p.H % hkv != 0 || v->H != hkv) {
    set_error("k and v need the same number of heads, a divisor of q's (" + std::to_string(p.H) + ")");
    return ATTN_E_INVAL;
  }
  if (p.H / hkv > 127) { set_error("at most 127 query heads per K/V head"); return ATTN_E_UNSUPPORTED; }
  attn_status st = check_kv_heads(p, hkv);
  if (st != ATTN_OK) return st;
  if ((st = check_tensor(q, "q", B, p.L, p.H, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(k, "k", B, p.L, hkv, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(v, "v", B, p.L, hkv, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(o, "o", B, p.L, p.H, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(dout, "dout", B, p.L, p.H, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(dq, "dq", B, p.L, p.H, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(dk, "dk", B, p.L, hkv, p.D)) != ATTN_OK) return st;
  if ((st = check_tensor(dv, "dv", B, p.L, hkv, p.D)) != ATTN_OK) return st;
  const std::initializer_list<const void*> ins = {q->data, k->data, v->data, o->data, dout->data};
  if (overlaps_any(dq->data, ins) || overlaps_any(dk->data, ins) || overlaps_any(dv->data, ins) ||
      dq->data == dk->data || dq->data == dv->data || dk->data == dv->data) {
    set_error("dq, dk and dv must be distinct and must not alias the inputs");
    return ATTN_E_INVAL;
  }
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) { set_error("lse is NULL or misaligned"); return ATTN_E_INVAL; }
  if (p.kind == ATTN_MASK_BLOCK && !p.block_aligned) {
    set_error("block size must be a multiple of 128 for the GPU kernel");
    return ATTN_E_UNSUPPORTED;
  }
  const BwdImage& img = bwd_image(p, hkv);
  const BwdLayout lay = bwd_layout(p, img, B);
  if (!launch->workspace || launch->workspace_bytes < lay.total) {
    set_error("workspace smaller than attn_bwd_workspace_bytes (" + std::to_string(lay.total) + " bytes)");
    return ATTN_E_WORKSPACE;
  }
  if (!aligned16(launch->workspace)) { set_error("workspace must be 16-byte aligned"); return ATTN_E_INVAL; }
  if (!g_tags.holds_backward(launch->workspace, p.serial, hkv)) {
    set_error("workspace was not prepared by attn_bwd_upload for this plan and " + std::to_string(hkv) +
              " K/V heads");
    return ATTN_E_INVAL;
  }
  // batch 1 runs the forward's split schedule for dQ (pieces of long rows add their dQ sums into the
  // forward's partial slots, merged after the dQ kernel); batch > 1 the unsplit one
  const bool split = (B == 1) && !p.merge_rows.empty();
  const bool kv_split = (B == 1) && !img.merge.empty();
  const size_t nq_items = split ? p.items.size() : p.items_unsplit.size();
  const size_t nkv_items = kv_split ? img.items_split.size() : img.items.size();
  if (nq_items % 8 || nkv_items % 8 || nq_items / 8 > static_cast<size_t>(INT32_MAX / 8) ||
      nkv_items / 8 > static_cast<size_t>(INT32_MAX / 8) || p.nq * kBM > INT32_MAX) {
    set_error("too many work items");
    return ATTN_E_UNSUPPORTED;
  }
  uint8_t* ws = static_cast<uint8_t*>(launch->workspace);
  BwdParams f{};
  f.q = static_cast<const uint16_t*>(q->data);
  f.k = static_cast<const uint16_t*>(k->data);
  f.v = static_cast<const uint16_t*>(v->data);
  f.o = static_cast<const uint16_t*>(o->data);
  f.dout = static_cast<const uint16_t*>(dout->data);
  f.dq = static_cast<uint16_t*>(dq->data);
  f.dk = static_cast<uint16_t*>(dk->data);
  f.dv = static_cast<uint16_t*>(dv->data);
  f.q_sb = q->stride_b; f.q_sl = q->stride_l; f.q_sh = q->stride_h;
  f.k_sb = k->stride_b; f.k_sl = k->stride_l; f.k_sh = k->stride_h;
  f.v_sb = v->stride_b; f.v_sl = v->stride_l; f.v_sh = v->stride_h;
  f.o_sb = o->stride_b; f.o_sl = o->stride_l; f.o_sh = o->stride_h;
  f.do_sb = dout->stride_b; f.do_sl = dout->stride_l; f.do_sh = dout->stride_h;
  f.dq_sb = dq->stride_b; f.dq_sl = dq->stride_l; f.dq_sh = dq->stride_h;
  f.dk_sb = dk->stride_b; f.dk_sl = dk->stride_l; f.dk_sh = dk->stride_h;
  f.dv_sb = dv->stride_b; f.dv_sl = dv->stride_l; f.dv_sh = dv->stride_h;
  f.lse = lse;
  f.sink = sink;
  f.dsink = dsink;
  f.stat = reinterpret_cast<float*>(ws + lay.off_stat);
  f.sinkpart = reinterpret_cast<float*>(ws + lay.off_sinkpart);
  f.qs = reinterpret_cast<uint16_t*>(ws + lay.off_qs);
  f.q_items = reinterpret_cast<const int32_t*>(ws + (split ? p.layout.off_items : p.layout.off_items_unsplit));
  f.partials = reinterpret_cast<float*>(ws + p.layout.off_partials);
  f.merge_rows = reinterpret_cast<const int32_t*>(ws + p.layout.off_merge);
  f.n_merge = split ? static_cast<int32_t>(p.merge_rows.size()) : 0;
  f.kv = reinterpret_cast<const int32_t*>(ws + p.layout.off_kv);
  f.kv_items = reinterpret_cast<const int32_t*>(ws + lay.off_image + (kv_split ? img.off_items_split : img.off_items));
  f.dkdv_partials = reinterpret_cast<float*>(ws + lay.off_dkdv);
  f.kv_merge = reinterpret_cast<const int32_t*>(ws + lay.off_image + img.off_merge);
  f.n_kv_merge = kv_split ? static_cast<int32_t>(img.merge.size()) : 0;
  f.col = reinterpret_cast<const int32_t*>(ws + lay.off_image + img.off_col);
  f.head_left = reinterpret_cast<const int32_t*>(ws + p.layout.off_head_left);
  const float scale = launch->softmax_scale > 0.f ? launch->softmax_scale
                                                  : static_cast<float>(1.0 / std::sqrt(double(p.D)));
  f.scale = scale;
  f.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  f.L = static_cast<int32_t>(p.L);
  f.H = static_cast<int32_t>(p.H);
  f.Lpad = static_cast<int32_t>(p.nq * kBM);
  f.nq = static_cast<int32_t>(p.nq);
  f.kind = p.kind;
  f.causal = p.causal;
  f.chunk = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(p.chunk, p.L)));
  f.right = static_cast<int32_t>(p.right);
  f.prefix = static_cast<int32_t>(std::min<int64_t>(p.prefix, p.L));
  f.kv_group = static_cast<int32_t>(p.H / hkv);
  f.q_queue = static_cast<int32_t>(nq_items / 8);
  f.kv_queue = static_cast<int32_t>(nkv_items / 8);
  *out = f;
  return ATTN_OK;
}

}  // namespace

attn_status attn_masked_fwd_lse(const attn_plan* p, const attn_tensor* q, const attn_tensor* k,
                                const attn_tensor* v, const float* sink, attn_tensor* o, float* lse,
                                const attn_launch* launch) {
  try {
    if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
    if (!launch) { set_error("launch is NULL"); return ATTN_E_INVAL; }
    if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) { set_error("lse is NULL or misaligned"); return ATTN_E_INVAL; }
    GroupParams g{};
    g.n_jobs = 1;
    attn_status st = make_job(*p, q, k, v, sink, o, launch->workspace, launch->workspace_bytes,
                              launch->softmax_scale, &g.job[0], &g.queue_len[0]);
    if (st != ATTN_OK) return st;
    g.job[0].lse = lse;
    return run_group(g, p->D, q->B, launch);
  } catch (...) {
    set_error("unexpected exception during launch");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_bwd_workspace_bytes(const attn_plan* p, int64_t B, int64_t kv_heads, size_t* bytes) {
  try {
    if (!p || !bytes) { set_error("plan or bytes is NULL"); return ATTN_E_INVAL; }
    if (B < 1 || B > 65535) { set_error("batch must be in [1, 65535]"); return ATTN_E_INVAL; }
    attn_status st = check_kv_heads(*p, kv_heads);
    if (st != ATTN_OK) return st;
    *bytes = bwd_layout(*p, bwd_image(*p, kv_heads), B).total;
    return ATTN_OK;
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed while building the backward lists");
    return ATTN_E_NOMEM;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_bwd_lists(const attn_plan* p, int64_t kv_heads, int64_t* n_blocks, const int32_t** col_ptr,
                           int64_t* n_entries, const int32_t** entries, int64_t* n_items, const int32_t** items) {
  try {
    if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
    attn_status st = check_kv_heads(*p, kv_heads);
    if (st != ATTN_OK) return st;
    const BwdImage& img = bwd_image(*p, kv_heads);
    if (n_blocks) *n_blocks = img.nkb;
    if (col_ptr) *col_ptr = img.col_ptr.data();
    if (n_entries) *n_entries = static_cast<int64_t>(img.col.size());
    if (entries) *entries = img.col.data();
    if (n_items) *n_items = static_cast<int64_t>(img.items.size());
    if (items) *items = reinterpret_cast<const int32_t*>(img.items.data());
    return ATTN_OK;
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed while building the backward lists");
    return ATTN_E_NOMEM;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_bwd_upload(const attn_plan* p, int64_t kv_heads, void* workspace, size_t workspace_bytes,
                            void* stream) {
  try {
    if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
    attn_status st = check_kv_heads(*p, kv_heads);
    if (st != ATTN_OK) return st;
    const BwdImage& img = bwd_image(*p, kv_heads);
    // the upload writes the forward and backward images (the statistics and
    // partial sums behind them depend on the batch and are checked per launch)
    const BwdLayout lay = bwd_layout(*p, img, 1);
    const size_t images = lay.off_image + img.bytes;
    if (!workspace || workspace_bytes < images) {
      set_error("workspace smaller than the plan's forward and backward images (" + std::to_string(images) +
                " bytes)");
      return ATTN_E_WORKSPACE;
    }
    if (!aligned16(workspace)) { set_error("workspace must be 16-byte aligned"); return ATTN_E_INVAL; }
    g_tags.forget(workspace);
    if ((st = upload(*p, workspace, workspace_bytes, stream)) != ATTN_OK) return st;
    std::vector<uint8_t> buf(img.bytes);
    write_bwd_image(img, buf.data());
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(static_cast<uint8_t*>(workspace) + lay.off_image, buf.data(), buf.size(),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (backward image)");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (backward image)");
    g_tags.note(workspace, p->serial, kv_heads);
    return ATTN_OK;
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed for the backward image");
    return ATTN_E_NOMEM;
  } catch (...) {
    set_error("unexpected exception during upload");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_masked_bwd(const attn_plan* p, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                            const attn_tensor* o, const attn_tensor* dout, const float* lse, const float* sink,
                            attn_tensor* dq, attn_tensor* dk, attn_tensor* dv, float* dsink,
                            const attn_launch* launch) {
  try {
    if (!p) { set_error("plan is NULL"); return ATTN_E_INVAL; }
    BwdParams f;
    attn_status st = make_bwd(*p, q, k, v, o, dout, lse, sink, dq, dk, dv, dsink, launch, &f);
    if (st != ATTN_OK) return st;
    hipError_t e = launch_bwd(f, static_cast<int>(p->D), static_cast<int>(q->B),
                              static_cast<hipStream_t>(launch->stream), static_cast<hipEvent_t>(launch->start_event),
                              static_cast<hipEvent_t>(launch->stop_event));
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return ATTN_OK;
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed while building the backward lists");
    return ATTN_E_NOMEM;
  } catch (...) {
    set_error("unexpected exception during launch");
    return ATTN_E_NOMEM;
  }
}

namespace {

constexpr int kRrTileQ = 128;    // sampled queries per work-group of the two-pass scores kernel (twice that for the single pass)

// Workspace of the search, 256-byte aligned parts: sampled queries (rows of
// D bf16), stride-summed keys (hi then lo: rows of 2 D bf16 + 16 bytes), the
// squared norms of the key aggregates (one per row), the heads' largest
// key-aggregate norm, the query tiles to recompute, and the per (key block,
// row) sums of the single pass.  Rows: nb R (every query block's strides,
// nb R >= floor(L / S)) rounded up to whole 256-row tiles.
struct RrLayout {
  size_t qs, ks, knorm2, kmax, flags, u, total;
};
static RrLayout rr_layout(int64_t B, int64_t H, int64_t ns_pad, int64_t D, int64_t nb) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bh = static_cast<size_t>(B) * static_cast<size_t>(H);
  const size_t rows = bh * static_cast<size_t>(ns_pad);
  RrLayout l{};
  size_t o = 0;
  l.qs = o; o = up(o + rows * static_cast<size_t>(D) * 2);
  l.ks = o; o = up(o + rows * static_cast<size_t>(4 * D + 16));
  l.knorm2 = o; o = up(o + rows * 4);
  l.kmax = o; o = up(o + bh * 4);
  l.flags = o; o = up(o + bh * static_cast<size_t>(ns_pad / kRrTileQ) * 4);
  l.u = o; o = up(o + rows * static_cast<size_t>(nb) * 4);
  l.total = o;
  return l;
}

// Validate a search request and fill the kernel parameters (pointers except the workspace).
static attn_status rr_prepare(const attn_tensor* q, const attn_tensor* k, const attn_rr_params* prm, RrParams* out,
                       size_t* ws_bytes) {
  if (!q || !k || !prm) { set_error("q, k or prm is NULL"); return ATTN_E_INVAL; }
  const int64_t B = q->B, L = q->L, H = q->H, D = q->D;
  if (D != 64 && D != 80 && D != 128) {
    set_error("head dim " + std::to_string(D) + " not supported (64, 80, 128)");
    return ATTN_E_UNSUPPORTED;
  }
  if (B < 1 || B > 65535 || H < 1 || H > 65535 || L < 1 || L > INT32_MAX / 2) {
    set_error("batch, heads or length out of range");
    return ATTN_E_INVAL;
  }
  attn_status st;
  if ((st = check_tensor(q, "q", B, L, H, D)) != ATTN_OK) return st;
  if (k->H < 1 || H % k->H != 0) {
    set_error("k needs a number of heads that divides q's (grouped-query attention)");
    return ATTN_E_INVAL;
  }
  if ((st = check_tensor(k, "k", B, L, k->H, D)) != ATTN_OK) return st;
  const int64_t S = prm->stride, Bs = prm->block;
  if (S < 1 || Bs < 1 || Bs % S != 0) { set_error("block must be a positive multiple of stride"); return ATTN_E_INVAL; }
  const int64_t R = Bs / S;
  if (R != 8 && R != 16 && R != 32) {
    set_error("block / stride must be 8, 16 or 32 on the GPU path");
    return ATTN_E_UNSUPPORTED;
  }
  if (!(prm->tau > 0.f && prm->tau <= 1.f)) { set_error("tau must be in (0, 1]"); return ATTN_E_INVAL; }
  if (L < S) { set_error("the sequence is shorter than one stride"); return ATTN_E_INVAL; }
  if (prm->protect_last != 0 && prm->protect_last != 1) { set_error("protect_last must be 0 or 1"); return ATTN_E_INVAL; }
  const int64_t nb = (L + Bs - 1) / Bs;
  if (nb > kRrMaxBlocks) {
    set_error("more than " + std::to_string(kRrMaxBlocks) + " blocks per row");
    return ATTN_E_UNSUPPORTED;
  }
  const int64_t ns = L / S;
  const int64_t ns_pad = (nb * R + 2 * kRrTileQ - 1) / (2 * kRrTileQ) * (2 * kRrTileQ);  // 256-row tiles
  RrParams p{};
  p.q = static_cast<const uint16_t*>(q->data);
  p.k = static_cast<const uint16_t*>(k->data);
  p.q_sb = q->stride_b; p.q_sl = q->stride_l; p.q_sh = q->stride_h;
  p.k_sb = k->stride_b; p.k_sl = k->stride_l; p.k_sh = k->stride_h;
  p.scale_log2 = static_cast<float>(1.4426950408889634 / (double(S) * std::sqrt(double(D))));
  p.tau = prm->tau;
  p.B = static_cast<int32_t>(B); p.H = static_cast<int32_t>(H); p.L = static_cast<int32_t>(L);
  p.D = static_cast<int32_t>(D); p.S = static_cast<int32_t>(S); p.Bs = static_cast<int32_t>(Bs);
  p.ns = static_cast<int32_t>(ns);
  p.ns_pad = static_cast<int32_t>(ns_pad);
  p.nb = static_cast<int32_t>(nb);
  p.protect_last = prm->protect_last;
  p.kv_group = static_cast<int32_t>(H / k->H);
  *out = p;
  *ws_bytes = rr_layout(B, H, ns_pad, D, nb).total;
  return ATTN_OK;
}

// Key split of a decode launch: enough work-groups to fill the chip at the
// kernel's LDS-bound occupancy (4, 2, 1 work-groups per CU at head dim 64,
// 128, 256), at least one 64-key tile per split.
struct DecodeSplit {
  int32_t nsplit, chunk;
};
static DecodeSplit decode_split(int64_t B, int64_t hkv, int64_t D, int64_t max_len, int64_t window, int64_t prefix) {
  const int64_t max_keys = window > 0 ? std::min<int64_t>(max_len, window + prefix) : max_len;
  const int64_t tiles = std::max<int64_t>(1, (max_keys + 63) / 64);
  const int64_t target = 256 * (D <= 64 ? 4 : D <= 128 ? 2 : 1);
  const int64_t want = std::max<int64_t>(1, (target + B * hkv - 1) / (B * hkv));
  const int64_t ns = std::min<int64_t>(std::min<int64_t>(want, tiles), 4096);
  const int64_t per = (tiles + ns - 1) / ns;
  return DecodeSplit{static_cast<int32_t>((tiles + per - 1) / per), static_cast<int32_t>(per * 64)};
}

// Window and prefix of a decode launch as the kernel takes them: a window of
// at least max_len keys is every cached key (0).
static void decode_reach(const attn_decode_desc* desc, int64_t max_len, int64_t* window, int64_t* prefix) {
  *window = (desc->window <= 0 || desc->window >= max_len) ? 0 : desc->window;
  *prefix = std::min<int64_t>(desc->prefix, max_len);
}

// Validate a decode launch and fill its parameters (workspace not checked).
static attn_status make_decode(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v, const attn_tensor* o,
                        int64_t max_len, const attn_decode_desc* desc, DecodeParams* out, int64_t* D_out) {
  if (!q || !k || !v || !desc) { set_error("q, k_cache, v_cache or desc is NULL"); return ATTN_E_INVAL; }
  const int64_t B = q->B, H = q->H, D = q->D;
  if (D != 64 && D != 128 && D != 256) {
    set_error("decode supports head dims 64, 128 and 256");
    return ATTN_E_UNSUPPORTED;
  }
  if (B < 1 || B > 65535 || H < 1 || q->L != 1) {
    set_error("q must be [B, 1, H, D] with 1 <= B <= 65535, H >= 1");
    return ATTN_E_INVAL;
  }
  attn_status st;
  if ((st = check_tensor(q, "q", B, 1, H, D)) != ATTN_OK) return st;
  const int64_t hkv = k->H, lmax = k->L;
  if (hkv < 1 || H % hkv != 0 || v->H != hkv) {
    set_error("k_cache and v_cache need the same number of heads, a divisor of q's");
    return ATTN_E_INVAL;
  }
  if (H / hkv > 16) { set_error("at most 16 query heads per cache head"); return ATTN_E_UNSUPPORTED; }
  if (lmax < 1 || hkv > 65535) { set_error("the caches need 1 <= Lmax and Hkv <= 65535"); return ATTN_E_INVAL; }
  if ((st = check_tensor(k, "k_cache", B, lmax, hkv, D)) != ATTN_OK) return st;
  if ((st = check_tensor(v, "v_cache", B, lmax, hkv, D)) != ATTN_OK) return st;
  if ((st = check_tensor(o, "o", B, 1, H, D)) != ATTN_OK) return st;
  if (o->data == q->data || o->data == k->data || o->data == v->data) {
    set_error("o must not alias q or the caches");
    return ATTN_E_INVAL;
  }
  if (max_len < 0 || max_len > lmax || max_len > INT32_MAX / 2) {
    set_error("max_len must be in [0, Lmax]");
    return ATTN_E_INVAL;
  }
  if (desc->prefix < 0) { set_error("prefix must be >= 0"); return ATTN_E_INVAL; }
  // row offsets inside one (sequence, head) are 32-bit
  if (lmax * std::max(k->stride_l, v->stride_l) * 2 + D * 2 > static_cast<int64_t>(UINT32_MAX)) {
    set_error("cache token stride * Lmax too large for 32-bit row offsets");
    return ATTN_E_UNSUPPORTED;
  }
  int64_t window, prefix;
  decode_reach(desc, max_len, &window, &prefix);
  const DecodeSplit sp = decode_split(B, hkv, D, max_len, window, prefix);
  DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q->data);
  p.k = static_cast<const uint16_t*>(k->data);
  p.v = static_cast<const uint16_t*>(v->data);
  p.o = static_cast<uint16_t*>(o->data);
  p.q_sb = q->stride_b; p.q_sh = q->stride_h;
  p.k_sb = k->stride_b; p.k_sl = k->stride_l; p.k_sh = k->stride_h;
  p.v_sb = v->stride_b; p.v_sl = v->stride_l; p.v_sh = v->stride_h;
  p.o_sb = o->stride_b; p.o_sh = o->stride_h;
  p.B = static_cast<int32_t>(B);
  p.H = static_cast<int32_t>(H);
  p.G = static_cast<int32_t>(H / hkv);
  p.max_len = static_cast<int32_t>(max_len);
  p.window = static_cast<int32_t>(window);
  p.prefix = static_cast<int32_t>(prefix);
  p.nsplit = sp.nsplit;
  p.chunk = sp.chunk;
  *out = p;
  *D_out = D;
  return ATTN_OK;
}

static size_t decode_ws_bytes(int64_t B, int64_t H, int64_t D, int32_t nsplit) {
  return nsplit > 1 ? static_cast<size_t>(B) * H * nsplit * (D + 2) * sizeof(float) : 0;
}

}  // namespace

attn_status attn_rr_workspace_bytes(const attn_tensor* q, const attn_rr_params* prm, size_t* bytes) {
  try {
    if (!bytes) { set_error("bytes is NULL"); return ATTN_E_INVAL; }
    RrParams p;
    return rr_prepare(q, q, prm, &p, bytes);
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_rr_search(const attn_tensor* q, const attn_tensor* k, const attn_rr_params* prm,
                           void* block_mask, void* block_score, const attn_launch* launch) {
  try {
    if (!launch) { set_error("launch is NULL"); return ATTN_E_INVAL; }
    RrParams p;
    size_t need = 0;
    attn_status st = rr_prepare(q, k, prm, &p, &need);
    if (st != ATTN_OK) return st;
    if (!block_mask || !block_score) { set_error("block_mask and block_score are required"); return ATTN_E_INVAL; }
    if (!launch->workspace || launch->workspace_bytes < need) {
      set_error("workspace smaller than attn_rr_workspace_bytes (" + std::to_string(need) + " bytes)");
      return ATTN_E_WORKSPACE;
    }
    if (!aligned16(launch->workspace)) { set_error("workspace must be 16-byte aligned"); return ATTN_E_INVAL; }
    const RrLayout lay = rr_layout(p.B, p.H, p.ns_pad, p.D, p.nb);
    uint8_t* ws = static_cast<uint8_t*>(launch->workspace);
    p.qs = reinterpret_cast<uint16_t*>(ws + lay.qs);
    p.ks = reinterpret_cast<uint16_t*>(ws + lay.ks);
    p.knorm2 = reinterpret_cast<float*>(ws + lay.knorm2);
    p.kmax = reinterpret_cast<uint32_t*>(ws + lay.kmax);
    p.flags = reinterpret_cast<int32_t*>(ws + lay.flags);
    p.u = reinterpret_cast<float*>(ws + lay.u);
    p.gate = 0;
    p.score = static_cast<float*>(block_score);
    p.bmask = static_cast<uint8_t*>(block_mask);
    hipError_t e = launch_rr_search(p, static_cast<hipStream_t>(launch->stream),
                                    static_cast<hipEvent_t>(launch->start_event),
                                    static_cast<hipEvent_t>(launch->stop_event));
    if (e != hipSuccess) return hip_fail(e, "search launch");
    return ATTN_OK;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_reorder_tokens(const attn_tensor* in, int32_t from, attn_tensor* out, int32_t to,
                                int64_t grid_h, int64_t grid_w, const attn_launch* launch) {
  try {
    if (!in || !out || !launch) { set_error("in, out or launch is NULL"); return ATTN_E_INVAL; }
    if (from < 0 || from > 2 || to < 0 || to > 2) { set_error("unknown token order"); return ATTN_E_INVAL; }
    if (grid_h < 1 || grid_w < 1 || grid_h * grid_w != in->L) {
      set_error("grid_h * grid_w must equal the token count");
      return ATTN_E_INVAL;
    }
    if ((from != ATTN_ORDER_RASTER || to != ATTN_ORDER_RASTER) && (grid_h % 2 || grid_w % 2)) {
      set_error("2 x 2-block orders need even grid sides");
      return ATTN_E_INVAL;
    }
    if (in->D < 8 || in->D % 8 || in->B < 1 || in->H < 1 || in->L > INT32_MAX / 2 || in->B > 65535) {
      set_error("D must be a positive multiple of 8; B, H >= 1");
      return ATTN_E_INVAL;
    }
    attn_status st;
    if ((st = check_tensor(in, "in", in->B, in->L, in->H, in->D)) != ATTN_OK) return st;
    if ((st = check_tensor(out, "out", in->B, in->L, in->H, in->D)) != ATTN_OK) return st;
    if (in->data == out->data) { set_error("out must not alias in"); return ATTN_E_INVAL; }
    ReorderParams p{};
    p.in = static_cast<const uint16_t*>(in->data);
    p.out = static_cast<uint16_t*>(out->data);
    p.in_sb = in->stride_b; p.in_sl = in->stride_l; p.in_sh = in->stride_h;
    p.out_sb = out->stride_b; p.out_sl = out->stride_l; p.out_sh = out->stride_h;
    p.B = static_cast<int32_t>(in->B); p.L = static_cast<int32_t>(in->L);
    p.H = static_cast<int32_t>(in->H); p.D = static_cast<int32_t>(in->D);
    p.gh = static_cast<int32_t>(grid_h); p.gw = static_cast<int32_t>(grid_w);
    p.from = from; p.to = to;
    hipError_t e = launch_reorder(p, static_cast<hipStream_t>(launch->stream),
                                  static_cast<hipEvent_t>(launch->start_event),
                                  static_cast<hipEvent_t>(launch->stop_event));
    if (e != hipSuccess) return hip_fail(e, "reorder launch");
    return ATTN_OK;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_decode_workspace_bytes(const attn_tensor* q, const attn_tensor* k_cache, int64_t max_len,
                                        const attn_decode_desc* desc, size_t* bytes) {
  try {
    if (!bytes) { set_error("bytes is NULL"); return ATTN_E_INVAL; }
    if (!q || !k_cache || !desc) { set_error("q, k_cache or desc is NULL"); return ATTN_E_INVAL; }
    if (q->D != 64 && q->D != 128 && q->D != 256) {
      set_error("decode supports head dims 64, 128 and 256");
      return ATTN_E_UNSUPPORTED;
    }
    if (q->B < 1 || q->H < 1 || k_cache->H < 1 || q->H % k_cache->H != 0 || max_len < 0 ||
        max_len > k_cache->L || desc->prefix < 0) {
      set_error("inconsistent q / k_cache shapes, max_len or prefix");
      return ATTN_E_INVAL;
    }
    int64_t window, prefix;
    decode_reach(desc, max_len, &window, &prefix);
    const DecodeSplit sp = decode_split(q->B, k_cache->H, q->D, max_len, window, prefix);
    *bytes = decode_ws_bytes(q->B, q->H, q->D, sp.nsplit);
    return ATTN_OK;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

attn_status attn_decode_fwd(const attn_tensor* q, const attn_tensor* k_cache, const attn_tensor* v_cache,
                            const int32_t* seq_lens, int64_t max_len, const attn_decode_desc* desc,
                            const float* sink, attn_tensor* o, const attn_launch* launch) {
  try {
    if (!launch) { set_error("launch is NULL"); return ATTN_E_INVAL; }
    if (!seq_lens) { set_error("seq_lens is NULL"); return ATTN_E_INVAL; }
    DecodeParams p{};
    int64_t D = 0;
    attn_status st = make_decode(q, k_cache, v_cache, o, max_len, desc, &p, &D);
    if (st != ATTN_OK) return st;
    const size_t need = decode_ws_bytes(p.B, p.H, D, p.nsplit);
    if (need > 0) {
      if (!launch->workspace || launch->workspace_bytes < need) {
        set_error("workspace smaller than attn_decode_workspace_bytes (" + std::to_string(need) + " bytes)");
        return ATTN_E_WORKSPACE;
      }
      if (!aligned16(launch->workspace)) { set_error("workspace must be 16-byte aligned"); return ATTN_E_INVAL; }
      p.partials = static_cast<float*>(launch->workspace);
    }
    p.seq_lens = seq_lens;
    p.sink = sink;
    const float scale = launch->softmax_scale > 0.f ? launch->softmax_scale
                                                    : static_cast<float>(1.0 / std::sqrt(double(D)));
    p.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
    hipError_t e = launch_decode(p, static_cast<int>(D), static_cast<hipStream_t>(launch->stream),
                                 static_cast<hipEvent_t>(launch->start_event),
                                 static_cast<hipEvent_t>(launch->stop_event));
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ATTN_OK;
  } catch (...) {
    set_error("unexpected exception");
    return ATTN_E_NOMEM;
  }
}

void attn_plan_destroy(attn_plan* p) { delete p; }

const char* attn_last_error(void) { return bss::g_last_error.c_str(); }

const char* attn_version(void) { return "bss_attn 0.1.0 gfx950"; }

}  // extern "C"
