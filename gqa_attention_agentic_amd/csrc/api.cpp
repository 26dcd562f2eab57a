// C ABI of the shared-prefix GQA attention library (declared in gqa_attn.h).
//
// A forward call validates its arguments on the host, builds (or reuses) the
// plan, makes sure its device buffers are large enough, copies the plan to
// the device with one async copy when it changed, and launches up to three
// kernels: the MFMA-bound (wide) attention kernel, the 32-row (narrow)
// attention kernel and the LSE merge, all ordered on the caller's stream.
// When a forward has items of both attention kernels, the narrow one runs on
// the handle's side stream, forked from and joined back into the caller's
// stream with events, so that the two run side by side on the compute units
// the plan gives each. It never synchronises the stream. Everything that can
// fail for a reason other than a launch (arguments, metadata, allocation) is
// settled before the first launch.
//
// The handle's device buffers: the plan, the arrival counters of the
// in-launch combination (zero between forwards: every forward leaves them
// so), and the partial workspace. A buffer that a forward under HIP graph
// capture referenced is never rewritten with other contents nor freed before
// the handle is destroyed, so a captured graph stays valid after later
// forwards with other metadata. The no-allocation variant keeps the same
// three regions in the library's static per-device scratch (scratch.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gqa_attn.h"
#include "../../include/gqa_probe.h"
#include "kernels.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

gqa_status fail(gqa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

gqa_status hip_fail(hipError_t e, const char* what) {
  return fail(GQA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Kernel-only timing of one forward: each launch records its own pair of
// events around the kernel's execution.
struct TimerSlot {
  hipEvent_t ev[6];   // wide start/end, narrow start/end, merge start/end
  bool wide, narrow, merged, concurrent;
};

// A device buffer of the handle. `captured`: a forward made under HIP graph
// capture references it, so it keeps its contents' meaning and its memory
// until the handle is destroyed.
struct DevBuf {
  char* p = nullptr;
  size_t cap = 0;
  bool captured = false;
};

// Byte offsets of the serialised plan: wide items | narrow items | wide bins
// | narrow bins | token records | combination records (each 256-B aligned).
struct PlanLayout {
  size_t wide = 0, narrow = 0, wide_bins = 0, narrow_bins = 0, tok_rec = 0, combs = 0, bytes = 0;
};

// Every plan a handle builds gets a process-unique id, so that the
// no-allocation scratch of a device knows whose plan it holds.
std::atomic<uint64_t> g_next_plan_id{1};
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint64_t g_scratch_plan[kMaxDevices];   // plan id whose serialisation the device's scratch holds (0: none)

}  // namespace

struct gqa_attn {
  gqa_attn_params p{};
  int device = 0;
  int n_cu = 256;
  int wide_per_cu = 1, narrow_per_cu = 1;   // resident workgroups per CU of each attention kernel
  // plan cache (host)
  std::vector<int32_t> key;
  gqa::Plan plan;
  bool have_plan = false;
  uint64_t plan_id = 0;
  // device copy of plan `d_plan_id`, its pinned staging, and a pageable
  // serialisation for the no-allocation path
  DevBuf d_plan;
  uint64_t d_plan_id = 0;
  char* h_staging = nullptr;
  size_t h_staging_cap = 0;
  hipEvent_t staging_free = nullptr;   // recorded after the last staging -> device copy
  std::vector<char> h_pageable;
  // arrival counters (one per query token and KV head) and partial workspace
  // ((m, l) rows, then O rows)
  DevBuf d_counters;
  DevBuf d_work;
  std::vector<char*> retired;          // buffers a captured graph may still read
  void* scratch = nullptr;             // this device's no-allocation scratch
  // K/V append: per-row (branch, position) list on the device, and a ring
  // of pinned staging slots, each with the event after which it may be
  // rewritten (the host waits only for the upload of four calls back)
  int2* d_rows = nullptr;
  size_t d_rows_cap = 0;
  struct RowSlot {
    int2* h = nullptr;
    size_t cap = 0;
    hipEvent_t free = nullptr;
  } row_slots[4];
  int row_next = 0;
  std::vector<int32_t> rows_key;   // (private_len, n_new) per branch of the list now on the device
  std::vector<std::pair<hipEvent_t, hipEvent_t>> append_timers;   // start/stop of timed appends
  size_t append_timed = 0;
  // side stream for the narrow kernel when both attention kernels run
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // timing
  bool timing = false;
  std::vector<TimerSlot> timers;
  size_t timers_used = 0;
};

namespace {

gqa_status check_params(const gqa_attn_params* p) {
  if (!p) return fail(GQA_ERR_INVALID_ARG, "params is NULL");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(GQA_ERR_INVALID_ARG, "num_q_heads and num_kv_heads must be > 0");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(GQA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(GQA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->page_size <= 0 || p->page_size > 4096)
    return fail(GQA_ERR_INVALID_ARG, "page_size must be in 1..4096");
  if (p->dtype != GQA_BF16 && p->dtype != GQA_FP32) return fail(GQA_ERR_INVALID_ARG, "unknown dtype");
  // An M-tile holds whole tokens: the G query heads of a KV head must fit one.
  const int max_g = (p->dtype == GQA_BF16) ? gqa::kWideRowsBf16 : gqa::kWideRows;
  if (p->num_q_heads / p->num_kv_heads > max_g)
    return fail(GQA_ERR_UNSUPPORTED, "more than " + std::to_string(max_g) + " query heads per KV head");
  if (p->workspace_bytes_cap < 0) return fail(GQA_ERR_INVALID_ARG, "workspace_bytes_cap < 0");
  if (!(std::isfinite(p->softmax_scale))) return fail(GQA_ERR_INVALID_ARG, "softmax_scale is not finite");
  return GQA_OK;
}

gqa_status make_input(const gqa_attn_params* p, int32_t n_groups, const int32_t* gs, const int32_t* gl,
                      int32_t n_branches, const int32_t* bg, const int32_t* bq, const int32_t* bp,
                      const int32_t* splits, int32_t causal, int n_cu, int wide_per_cu, int narrow_per_cu,
                      gqa::PlanInput* in) {
  if (n_groups < 0 || n_branches < 0) return fail(GQA_ERR_INVALID_ARG, "negative group or branch count");
  if (n_groups > 0 && (!gs || !gl)) return fail(GQA_ERR_INVALID_ARG, "group arrays are NULL");
  if (n_branches > 0 && (!bg || !bq || !bp)) return fail(GQA_ERR_INVALID_ARG, "branch arrays are NULL");
  if (causal != 0 && causal != 1) return fail(GQA_ERR_INVALID_ARG, "causal must be 0 or 1");
  in->H_q = p->num_q_heads;
  in->H_kv = p->num_kv_heads;
  in->D = p->head_dim;
  in->page_size = p->page_size;
  in->dtype = p->dtype;
  in->causal = causal;
  in->n_cu = n_cu;
  in->wide_per_cu = wide_per_cu;
  in->narrow_per_cu = narrow_per_cu;
  in->g_start.assign(gs, gs + n_groups);
  in->g_len.assign(gl, gl + n_groups);
  in->b_group.assign(bg, bg + n_branches);
  in->b_qlen.assign(bq, bq + n_branches);
  in->b_priv.assign(bp, bp + n_branches);
  if (splits) in->splits_override.assign(splits, splits + n_groups + n_branches);
  std::string err = gqa::validate_plan_input(*in);
  if (!err.empty()) return fail(GQA_ERR_INVALID_ARG, err);
  return GQA_OK;
}

void fill_stats(const gqa::Plan& P, int64_t D, gqa_plan_stats* s) {
  s->n_items_wide = (int64_t)P.wide.size();
  s->n_items_narrow = (int64_t)P.narrow.size();
  s->n_kv_tiles = P.n_kv_tiles;
  s->n_merge_rows = P.merge_rows;
  s->workspace_bytes = P.part_rows * (D + 2) * (int64_t)sizeof(float);
  s->n_units = (int64_t)P.units.size();
  s->max_splits = P.max_splits;
  s->merge_launch = P.merge_launch ? 1 : 0;
  s->wide_cus = P.wide_cus;
  s->narrow_cus = P.narrow_cus;
}

PlanLayout plan_layout(const gqa::Plan& P) {
  PlanLayout L;
  size_t off = 0;
  L.wide = off;
  off = align_up(off + P.wide.size() * sizeof(gqa::WorkItem), 256);
  L.narrow = off;
  off = align_up(off + P.narrow.size() * sizeof(gqa::WorkItem), 256);
  L.wide_bins = off;
  off = align_up(off + P.wide_bins.size() * sizeof(int32_t), 256);
  L.narrow_bins = off;
  off = align_up(off + P.narrow_bins.size() * sizeof(int32_t), 256);
  L.tok_rec = off;
  off = align_up(off + P.tok_rec.size() * sizeof(gqa::TokRec), 256);
  L.combs = off;
  off = align_up(off + P.combs.size() * sizeof(gqa::CombTok), 256);
  L.bytes = std::max<size_t>(off, 256);
  return L;
}

void serialise_plan(const gqa::Plan& P, const PlanLayout& L, char* dst) {
  auto put = [&](size_t off, const void* src, size_t n) {
    if (n) std::memcpy(dst + off, src, n);
  };
  put(L.wide, P.wide.data(), P.wide.size() * sizeof(gqa::WorkItem));
  put(L.narrow, P.narrow.data(), P.narrow.size() * sizeof(gqa::WorkItem));
  put(L.wide_bins, P.wide_bins.data(), P.wide_bins.size() * sizeof(int32_t));
  put(L.narrow_bins, P.narrow_bins.data(), P.narrow_bins.size() * sizeof(int32_t));
  put(L.tok_rec, P.tok_rec.data(), P.tok_rec.size() * sizeof(gqa::TokRec));
  put(L.combs, P.combs.data(), P.combs.size() * sizeof(gqa::CombTok));
}

// Bytes of the arrival counters (one per token combined in the narrow
// launch and KV head, a 128-byte line each) and of the partial workspace
// ((m, l) rows, then O rows) that a plan needs.
size_t counter_bytes(const gqa::Plan& P, int H_kv) {
  return align_up((size_t)P.n_counter_slots * H_kv * gqa::kCounterStride * sizeof(int32_t), 256);
}
size_t ml_bytes(const gqa::Plan& P) { return align_up((size_t)P.part_rows * sizeof(float2), 256); }
size_t work_bytes(const gqa::Plan& P, int D) {
  return P.part_rows ? ml_bytes(P) + (size_t)P.part_rows * D * sizeof(float) : 0;
}

// Makes `b` hold at least `need` bytes; a buffer that must keep its
// contents' meaning (captured, or `replace` for a plan that differs) is
// retired rather than reused or freed. *fresh tells whether a new buffer
// was allocated.
gqa_status ensure_buf(gqa_attn* h, DevBuf& b, size_t need, bool replace, const char* what, bool* fresh) {
  if (fresh) *fresh = false;
  if (need == 0) return GQA_OK;
  if (need <= b.cap && !(replace && b.captured)) return GQA_OK;
  if (b.p) {
    if (b.captured) {
      h->retired.push_back(b.p);
    } else {
      hipError_t e = hipFree(b.p);   // synchronises the device: no kernel still reads it
      if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
  }
  b = DevBuf();
  const size_t cap = std::max(need, (size_t)256);
  hipError_t e = hipMalloc((void**)&b.p, cap);
  if (e != hipSuccess) {
    b.p = nullptr;
    return fail(GQA_ERR_NO_MEMORY, std::string(what) + " allocation of " + std::to_string(cap) + " bytes failed");
  }
  b.cap = cap;
  if (fresh) *fresh = true;
  return GQA_OK;
}

TimerSlot* next_timer(gqa_attn* h) {
  if (h->timers_used == h->timers.size()) {
    TimerSlot t{};
    for (int k = 0; k < 6; ++k) {
      if (hipEventCreate(&t.ev[k]) != hipSuccess) {
        for (int j = 0; j < k; ++j) hipEventDestroy(t.ev[j]);
        return nullptr;   // this forward goes untimed
      }
    }
    h->timers.push_back(t);
  }
  return &h->timers[h->timers_used++];
}

struct ForwardArgs {
  const void *q, *k_shared, *v_shared;
  int32_t n_shared_tokens;
  const void *k_pages, *v_pages;
  const int32_t* page_table;
  int32_t max_pages_per_branch;
  int32_t n_groups;
  const int32_t *group_shared_start, *group_shared_len;
  int32_t n_branches;
  const int32_t *branch_group, *branch_q_len, *branch_private_len, *splits_override;
  int32_t causal;
  void* o;
  float* lse;
  void* stream;
};

// Where a forward's plan, counters and partials live on the device.
struct DevRegions {
  const char* plan;
  int32_t* counters;
  char* work;
};

// The kernel launches of one forward (the plan is on the device already).
gqa_status launch_forward(gqa_attn* h, const ForwardArgs& f, const gqa::Plan& Q, const PlanLayout& L,
                          const DevRegions& R, hipStream_t st, TimerSlot* tm, bool use_side) {
  gqa::AttnArgs a{};
  a.q = f.q;
  a.k_shared = f.k_shared;
  a.v_shared = f.v_shared;
  a.k_pages = f.k_pages;
  a.v_pages = f.v_pages;
  a.page_table = f.page_table;
  a.tok_rec = (const gqa::TokRec*)(R.plan + L.tok_rec);
  a.combs = (const gqa::CombTok*)(R.plan + L.combs);
  a.counters = R.counters;
  a.part_ml = (float2*)R.work;
  a.part_o = (float*)(R.work + ml_bytes(Q));
  a.o = f.o;
  a.lse = f.lse;
  a.max_pages = f.max_pages_per_branch;
  a.H_q = h->p.num_q_heads;
  a.H_kv = h->p.num_kv_heads;
  a.G = a.H_q / a.H_kv;
  a.n_shared = f.n_shared_tokens;
  a.page_size = h->p.page_size;
  a.page_shift = -1;
  for (int sft = 0; sft < 13; ++sft)
    if ((1 << sft) == h->p.page_size) a.page_shift = sft;
  a.causal = f.causal;
  a.n_q_tokens = Q.n_q_tokens;
  a.scale_log2 = h->p.softmax_scale * 1.4426950408889634f;
  // Device-scope partial stores without a release fence when every
  // workgroup of the bf16 narrow kernel runs a single item (see
  // combine_if_last in attention.hip).
  a.coherent_parts = (h->p.dtype == GQA_BF16 && !Q.narrow.empty() && Q.narrow.size() + 1 == Q.narrow_bins.size()) ? 1 : 0;

  auto ev = [&](int k) -> hipEvent_t { return tm ? tm->ev[k] : nullptr; };
  if (tm) {
    tm->wide = !Q.wide.empty();
    tm->narrow = !Q.narrow.empty();
    tm->merged = Q.merge_launch;
    tm->concurrent = Q.concurrent && use_side;
  }
  hipError_t e;
  const bool side_by_side = Q.concurrent && use_side;
  if (side_by_side) {
    // Narrow kernel on the side stream, after everything already queued on
    // the caller's stream (plan upload, counter clear); the caller's stream
    // waits for it before the merge. Both streams have the default priority.
    e = hipEventRecord(h->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork, 0);
    if (e != hipSuccess) return hip_fail(e, "fork to the side stream");
    a.items = (const gqa::WorkItem*)(R.plan + L.narrow);
    a.bins = (const int32_t*)(R.plan + L.narrow_bins);
    e = gqa::launch_attention(a, (int32_t)Q.narrow_bins.size() - 1, true, h->p.dtype, h->p.head_dim, h->side,
                              ev(2), ev(3));
    if (e != hipSuccess) return hip_fail(e, "attention (narrow) launch");
    e = hipEventRecord(h->join, h->side);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(join)");
    a.items = (const gqa::WorkItem*)(R.plan + L.wide);
    a.bins = (const int32_t*)(R.plan + L.wide_bins);
    e = gqa::launch_attention(a, (int32_t)Q.wide_bins.size() - 1, false, h->p.dtype, h->p.head_dim, st, ev(0),
                              ev(1));
    // The caller's stream waits for the narrow kernel even when the wide
    // launch failed, so that no later work on it overlaps a kernel still
    // writing the outputs.
    const hipError_t ej = hipStreamWaitEvent(st, h->join, 0);
    if (e != hipSuccess) return hip_fail(e, "attention (wide) launch");
    if (ej != hipSuccess) return hip_fail(ej, "join from the side stream");
  } else if (!Q.wide.empty()) {
    a.items = (const gqa::WorkItem*)(R.plan + L.wide);
    a.bins = (const int32_t*)(R.plan + L.wide_bins);
    e = gqa::launch_attention(a, (int32_t)Q.wide_bins.size() - 1, false, h->p.dtype, h->p.head_dim, st, ev(0),
                              ev(1));
    if (e != hipSuccess) return hip_fail(e, "attention (wide) launch");
  }
  if (!side_by_side && !Q.narrow.empty()) {
    a.items = (const gqa::WorkItem*)(R.plan + L.narrow);
    a.bins = (const int32_t*)(R.plan + L.narrow_bins);
    e = gqa::launch_attention(a, (int32_t)Q.narrow_bins.size() - 1, true, h->p.dtype, h->p.head_dim, st, ev(2),
                              ev(3));
    if (e != hipSuccess) return hip_fail(e, "attention (narrow) launch");
  }
  if (Q.merge_launch) {
    e = gqa::launch_merge(a, h->p.dtype, h->p.head_dim, Q.max_row_parts, st, ev(4), ev(5));
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return GQA_OK;
}

enum class Mode { kOwned, kScratch };

gqa_status forward_impl(gqa_attn* h, const ForwardArgs& f, Mode mode) {
  if (!h) return fail(GQA_ERR_INVALID_ARG, "handle is NULL");
  gqa::PlanInput in;
  gqa_status s = make_input(&h->p, f.n_groups, f.group_shared_start, f.group_shared_len, f.n_branches,
                            f.branch_group, f.branch_q_len, f.branch_private_len, f.splits_override, f.causal,
                            h->n_cu, h->wide_per_cu, h->narrow_per_cu, &in);
  if (s != GQA_OK) return s;

  // Plan cache key: every input of the planner.
  std::vector<int32_t> key;
  key.reserve(8 + 2 * f.n_groups + 4 * f.n_branches);
  key.push_back(f.n_groups);
  key.push_back(f.n_branches);
  key.push_back(f.causal);
  key.push_back(f.splits_override ? 1 : 0);
  key.insert(key.end(), in.g_start.begin(), in.g_start.end());
  key.insert(key.end(), in.g_len.begin(), in.g_len.end());
  key.insert(key.end(), in.b_group.begin(), in.b_group.end());
  key.insert(key.end(), in.b_qlen.begin(), in.b_qlen.end());
  key.insert(key.end(), in.b_priv.begin(), in.b_priv.end());
  key.insert(key.end(), in.splits_override.begin(), in.splits_override.end());
  const bool same = h->have_plan && key == h->key;
  gqa::Plan fresh;
  const gqa::Plan& P = same ? h->plan : fresh;
  if (!same) {
    std::string err = gqa::build_plan(in, &fresh);
    if (!err.empty()) return fail(GQA_ERR_INVALID_ARG, err);
  }

  // Pointer checks against the (new) plan's extents.
  const bool any_q = P.n_q_tokens > 0;
  bool any_priv = false;
  for (int32_t b = 0; b < f.n_branches; ++b) any_priv |= in.b_priv[b] > 0;
  if (any_q && (!f.q || !f.o || !f.lse)) return fail(GQA_ERR_INVALID_ARG, "q, o and lse must be non-NULL");
  if (P.n_shared_tokens > 0 && (!f.k_shared || !f.v_shared))
    return fail(GQA_ERR_INVALID_ARG, "k_shared and v_shared must be non-NULL");
  if (f.n_shared_tokens < P.n_shared_tokens)
    return fail(GQA_ERR_INVALID_ARG, "a group's shared range ends past n_shared_tokens");
  if (any_priv && (!f.k_pages || !f.v_pages || !f.page_table))
    return fail(GQA_ERR_INVALID_ARG, "k_pages, v_pages and page_table must be non-NULL");
  if (any_priv && f.max_pages_per_branch < P.max_branch_pages)
    return fail(GQA_ERR_INVALID_ARG, "max_pages_per_branch is smaller than a branch's page count");
  const void* ptrs[] = {f.q, f.k_shared, f.v_shared, f.k_pages, f.v_pages, f.o};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GQA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if ((f.page_table && (reinterpret_cast<uintptr_t>(f.page_table) & 3u)) ||
      (f.lse && (reinterpret_cast<uintptr_t>(f.lse) & 3u)))
    return fail(GQA_ERR_INVALID_ARG, "page_table and lse must be 4-byte aligned");
  if (!any_q) return GQA_OK;

  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  hipStream_t st = (hipStream_t)f.stream;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  const bool capturing = cs != hipStreamCaptureStatusNone;

  const PlanLayout L = plan_layout(P);
  const int H_kv = h->p.num_kv_heads, D = h->p.head_dim;
  const size_t cnt_need = counter_bytes(P, H_kv), work_need = work_bytes(P, D);
  const char* under_capture =
      "under HIP graph capture a forward must reuse the plan and buffers of an earlier forward with the "
      "same metadata: make one outside capture first";
  size_t plan_off = 0, work_off = 0;   // scratch mode: offsets of the plan and the partials
  if (mode == Mode::kOwned) {
    if (h->p.workspace_bytes_cap > 0 && cnt_need + work_need > (size_t)h->p.workspace_bytes_cap)
      return fail(GQA_ERR_NO_MEMORY, "partial workspace of " + std::to_string(cnt_need + work_need) +
                                         " bytes exceeds workspace_bytes_cap");
    if (capturing && (!same || h->d_plan_id != h->plan_id || cnt_need > h->d_counters.cap ||
                      work_need > h->d_work.cap || (P.concurrent && !h->side)))
      return fail(GQA_ERR_INVALID_ARG, under_capture);
  } else {
    if (!h->scratch) return fail(GQA_ERR_HIP, "the no-allocation scratch of this device is not set up");
    if (cnt_need > gqa::kScratchCounterBytes)
      return fail(GQA_ERR_NO_MEMORY, "arrival counters of " + std::to_string(cnt_need) +
                                         " bytes exceed the scratch's counter region of " +
                                         std::to_string(gqa::kScratchCounterBytes));
    plan_off = gqa::kScratchCounterBytes;
    work_off = plan_off + align_up(L.bytes, 256);
    if (work_off + work_need > gqa::kScratchBytes)
      return fail(GQA_ERR_NO_MEMORY, "this forward needs " + std::to_string(work_off + work_need) +
                                         " bytes of scratch (plan " + std::to_string(L.bytes) + ", partials " +
                                         std::to_string(work_need) + "); the no-allocation scratch holds " +
                                         std::to_string(gqa::kScratchBytes));
    if (capturing) {
      std::lock_guard<std::mutex> lock(g_scratch_mu);
      if (!same || g_scratch_plan[h->device] != h->plan_id) return fail(GQA_ERR_INVALID_ARG, under_capture);
    }
  }

  // The host plan is committed; from here on a failure leaves it cached
  // (it is valid) and the device copy marked stale.
  if (!same) {
    h->plan = std::move(fresh);
    h->key = std::move(key);
    h->have_plan = true;
    h->plan_id = g_next_plan_id.fetch_add(1);
  }
  const gqa::Plan& Q = h->plan;
  const bool upload = mode == Mode::kOwned ? h->d_plan_id != h->plan_id : false;

  DevRegions R{};
  bool clear_counters = false;
  if (mode == Mode::kOwned) {
    // Every allocation before the first launch.
    s = ensure_buf(h, h->d_counters, cnt_need, false, "counter", &clear_counters);
    if (s == GQA_OK) s = ensure_buf(h, h->d_work, work_need, false, "workspace", nullptr);
    if (s == GQA_OK && upload) s = ensure_buf(h, h->d_plan, L.bytes, true, "device plan", nullptr);
    if (s != GQA_OK) return s;
    if (upload) {
      if (h->staging_free) {   // the staging buffer may still feed the previous copy
        e = hipEventSynchronize(h->staging_free);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      } else {
        e = hipEventCreateWithFlags(&h->staging_free, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
      }
      if (L.bytes > h->h_staging_cap) {
        if (h->h_staging) hipHostFree(h->h_staging);
        h->h_staging = nullptr;
        h->h_staging_cap = 0;
        e = hipHostMalloc((void**)&h->h_staging, L.bytes, hipHostMallocDefault);
        if (e != hipSuccess) return fail(GQA_ERR_NO_MEMORY, "pinned plan staging allocation failed");
        h->h_staging_cap = L.bytes;
      }
    }
    if (Q.concurrent && !h->side) {
      e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&h->join, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "side stream creation");
    }
    // Launches.
    if (clear_counters) {
      e = gqa::launch_zero_i32((int32_t*)h->d_counters.p, (int64_t)(h->d_counters.cap / sizeof(int32_t)), st);
      if (e != hipSuccess) return hip_fail(e, "counter clear");
    }
    if (upload) {
      serialise_plan(Q, L, h->h_staging);
      e = hipMemcpyAsync(h->d_plan.p, h->h_staging, L.bytes, hipMemcpyHostToDevice, st);
      if (e == hipSuccess) e = hipEventRecord(h->staging_free, st);
      if (e != hipSuccess) return hip_fail(e, "plan upload");
      h->d_plan_id = h->plan_id;
    }
    if (capturing) h->d_plan.captured = h->d_counters.captured = h->d_work.captured = true;
    R.plan = h->d_plan.p;
    R.counters = (int32_t*)h->d_counters.p;
    R.work = h->d_work.p;
  } else {
    char* base = (char*)h->scratch;
    {
      std::lock_guard<std::mutex> lock(g_scratch_mu);
      if (g_scratch_plan[h->device] != h->plan_id) {
        // From pageable host memory: the copy is staged before the call
        // returns, and stays ordered on the stream.
        h->h_pageable.resize(L.bytes);
        serialise_plan(Q, L, h->h_pageable.data());
        e = hipMemcpyAsync(base + plan_off, h->h_pageable.data(), L.bytes, hipMemcpyHostToDevice, st);
        if (e != hipSuccess) {
          g_scratch_plan[h->device] = 0;
          return hip_fail(e, "plan upload to the scratch");
        }
        g_scratch_plan[h->device] = h->plan_id;
      }
    }
    R.plan = base + plan_off;
    R.counters = (int32_t*)base;
    R.work = base + work_off;
  }
  TimerSlot* tm = (h->timing && !capturing && mode == Mode::kOwned) ? next_timer(h) : nullptr;
  return launch_forward(h, f, Q, L, R, st, tm, h->side != nullptr);
}

}  // namespace

extern "C" {

const char* gqa_attn_last_error(void) { return g_last_error.c_str(); }

gqa_status gqa_attn_create(const gqa_attn_params* p, gqa_attn** out) {
  if (!out) return fail(GQA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  gqa_status s = check_params(p);
  if (s != GQA_OK) return s;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GQA_ERR_UNSUPPORTED, "device index out of range");
  int ncu = 0;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  gqa_attn* h = new gqa_attn();
  h->p = *p;
  if (h->p.softmax_scale <= 0.f) h->p.softmax_scale = 1.0f / std::sqrt((float)p->head_dim);
  h->device = dev;
  h->n_cu = ncu > 0 ? ncu : 256;
  e = gqa::attention_occupancy(h->p.dtype, h->p.head_dim, false, &h->wide_per_cu);
  if (e == hipSuccess) e = gqa::attention_occupancy(h->p.dtype, h->p.head_dim, true, &h->narrow_per_cu);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  }
  // The device's no-allocation scratch: its address, looked up once per
  // device with the device current (and its counters cleared).
  e = gqa::scratch_setup(dev, &h->scratch);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "scratch set-up");
  }
  *out = h;
  return GQA_OK;
}

gqa_status gqa_attn_destroy(gqa_attn* h) {
  if (!h) return GQA_OK;
  hipSetDevice(h->device);
  hipDeviceSynchronize();
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (h->plan_id && g_scratch_plan[h->device] == h->plan_id) g_scratch_plan[h->device] = 0;
  }
  for (DevBuf* b : {&h->d_plan, &h->d_counters, &h->d_work})
    if (b->p) hipFree(b->p);
  for (char* p : h->retired) hipFree(p);
  if (h->h_staging) hipHostFree(h->h_staging);
  if (h->staging_free) hipEventDestroy(h->staging_free);
  if (h->side) hipStreamDestroy(h->side);
  if (h->d_rows) hipFree(h->d_rows);
  for (auto& rs : h->row_slots) {
    if (rs.h) hipHostFree(rs.h);
    if (rs.free) hipEventDestroy(rs.free);
  }
  for (auto& t : h->append_timers) {
    hipEventDestroy(t.first);
    hipEventDestroy(t.second);
  }
  if (h->fork) hipEventDestroy(h->fork);
  if (h->join) hipEventDestroy(h->join);
  for (auto& t : h->timers)
    for (auto& ev : t.ev) hipEventDestroy(ev);
  delete h;
  return GQA_OK;
}

gqa_status gqa_attn_forward(gqa_attn* h, const void* q, const void* k_shared, const void* v_shared,
                            int32_t n_shared_tokens, const void* k_pages, const void* v_pages, const int32_t* page_table,
                            int32_t max_pages_per_branch, int32_t n_groups,
                            const int32_t* group_shared_start, const int32_t* group_shared_len,
                            int32_t n_branches, const int32_t* branch_group, const int32_t* branch_q_len,
                            const int32_t* branch_private_len, const int32_t* splits_override,
                            int32_t causal, void* o, float* lse, void* stream) {
  const ForwardArgs f{q, k_shared, v_shared, n_shared_tokens, k_pages, v_pages, page_table, max_pages_per_branch,
                      n_groups, group_shared_start, group_shared_len, n_branches, branch_group, branch_q_len,
                      branch_private_len, splits_override, causal, o, lse, stream};
  return forward_impl(h, f, Mode::kOwned);
}

gqa_status gqa_attn_forward_noalloc(gqa_attn* h, const void* q, const void* k_shared, const void* v_shared,
                                    int32_t n_shared_tokens, const void* k_pages, const void* v_pages,
                                    const int32_t* page_table, int32_t max_pages_per_branch, int32_t n_groups,
                                    const int32_t* group_shared_start, const int32_t* group_shared_len,
                                    int32_t n_branches, const int32_t* branch_group, const int32_t* branch_q_len,
                                    const int32_t* branch_private_len, const int32_t* splits_override,
                                    int32_t causal, void* o, float* lse, void* stream) {
  const ForwardArgs f{q, k_shared, v_shared, n_shared_tokens, k_pages, v_pages, page_table, max_pages_per_branch,
                      n_groups, group_shared_start, group_shared_len, n_branches, branch_group, branch_q_len,
                      branch_private_len, splits_override, causal, o, lse, stream};
  return forward_impl(h, f, Mode::kScratch);
}

namespace {

// Row list of an append -- (branch, position in its private suffix) per new
// row -- through the next pinned staging slot to the device.
gqa_status upload_rows(gqa_attn* h, int32_t n_branches, const int32_t* branch_private_len,
                       const int32_t* branch_n_new, int64_t n_rows, hipStream_t st) {
  hipError_t e;
  // This staging slot may still feed the copy of four calls back.
  auto& rs = h->row_slots[h->row_next];
  if (rs.free) {
    e = hipEventSynchronize(rs.free);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  } else {
    e = hipEventCreateWithFlags(&rs.free, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  if ((size_t)n_rows > rs.cap) {
    if (rs.h) hipHostFree(rs.h);
    rs.h = nullptr;
    rs.cap = 0;
    e = hipHostMalloc((void**)&rs.h, (size_t)n_rows * sizeof(int2), hipHostMallocDefault);
    if (e != hipSuccess) return fail(GQA_ERR_NO_MEMORY, "pinned row-list staging allocation failed");
    rs.cap = (size_t)n_rows;
  }
  if ((size_t)n_rows > h->d_rows_cap) {
    if (h->d_rows) {
      e = hipFree(h->d_rows);   // synchronises the device: no kernel still reads it
      if (e != hipSuccess) return hip_fail(e, "hipFree(rows)");
    }
    h->d_rows = nullptr;
    h->d_rows_cap = 0;
    e = hipMalloc((void**)&h->d_rows, (size_t)n_rows * sizeof(int2));
    if (e != hipSuccess) return fail(GQA_ERR_NO_MEMORY, "row-list allocation failed");
    h->d_rows_cap = (size_t)n_rows;
  }
  int64_t r = 0;
  for (int32_t b = 0; b < n_branches; ++b)
    for (int32_t i = 0; i < branch_n_new[b]; ++i) rs.h[r++] = make_int2(b, branch_private_len[b] + i);
  e = hipMemcpyAsync(h->d_rows, rs.h, (size_t)n_rows * sizeof(int2), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipEventRecord(rs.free, st);
  if (e != hipSuccess) return hip_fail(e, "row-list upload");
  h->row_next = (h->row_next + 1) % 4;
  return GQA_OK;
}

}  // namespace

gqa_status gqa_attn_append_kv(gqa_attn* h, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                              int32_t n_pages, const int32_t* page_table, int32_t max_pages_per_branch,
                              int32_t n_branches, const int32_t* branch_private_len, const int32_t* branch_n_new,
                              void* stream) {
  if (!h) return fail(GQA_ERR_INVALID_ARG, "handle is NULL");
  if (n_branches < 0 || n_pages < 0 || max_pages_per_branch < 0)
    return fail(GQA_ERR_INVALID_ARG, "negative branch, page or page-table size");
  if (n_branches > 0 && (!branch_private_len || !branch_n_new))
    return fail(GQA_ERR_INVALID_ARG, "branch arrays are NULL");
  const int64_t ps = h->p.page_size;
  int64_t n_rows = 0;
  for (int32_t b = 0; b < n_branches; ++b) {
    if (branch_private_len[b] < 0 || branch_n_new[b] < 0)
      return fail(GQA_ERR_INVALID_ARG, "branch " + std::to_string(b) + ": negative length");
    if ((int64_t)branch_private_len[b] + branch_n_new[b] > (int64_t)max_pages_per_branch * ps)
      return fail(GQA_ERR_INVALID_ARG, "branch " + std::to_string(b) + ": appended rows exceed its page table");
    n_rows += branch_n_new[b];
  }
  if (n_rows > std::numeric_limits<int32_t>::max()) return fail(GQA_ERR_INVALID_ARG, "too many rows");
  if (n_rows == 0) return GQA_OK;
  if (!k_new || !v_new || !k_pages || !v_pages || !page_table || n_pages == 0)
    return fail(GQA_ERR_INVALID_ARG, "NULL tensor or empty page pool");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages))
    return fail(GQA_ERR_INVALID_ARG, "K/V tensors must be 16-byte aligned");
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  // The row list is uploaded only when it differs from the one already on
  // the device (stream order keeps that one valid for this launch).
  std::vector<int32_t> key(2 * (size_t)n_branches);
  for (int32_t b = 0; b < n_branches; ++b) {
    key[2 * b] = branch_private_len[b];
    key[2 * b + 1] = branch_n_new[b];
  }
  if (key != h->rows_key) {
    h->rows_key.clear();
    gqa_status s = upload_rows(h, n_branches, branch_private_len, branch_n_new, n_rows, st);
    if (s != GQA_OK) return s;
    h->rows_key = std::move(key);
  }
  gqa::AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.page_table = page_table;
  a.rows = h->d_rows;
  a.max_pages = max_pages_per_branch;
  a.n_pages = n_pages;
  a.page_size = h->p.page_size;
  a.num_kv_heads = h->p.num_kv_heads;
  a.row_bytes = h->p.head_dim * (h->p.dtype == GQA_BF16 ? 2 : 4);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (h->timing) {
    if (h->append_timed == h->append_timers.size()) {
      hipEvent_t x = nullptr, y = nullptr;
      e = hipEventCreate(&x);
      if (e == hipSuccess) e = hipEventCreate(&y);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
      h->append_timers.emplace_back(x, y);
    }
    e0 = h->append_timers[h->append_timed].first;
    e1 = h->append_timers[h->append_timed].second;
    ++h->append_timed;
  }
  e = gqa::launch_append(a, (int32_t)n_rows, st, e0, e1);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return GQA_OK;
}

gqa_status gqa_attn_append_times(gqa_attn* h, double* ms, int64_t* n_calls) {
  if (!h || !ms || !n_calls) return fail(GQA_ERR_INVALID_ARG, "NULL argument");
  double t = 0.0;
  for (size_t k = 0; k < h->append_timed; ++k) {
    hipError_t e = hipEventSynchronize(h->append_timers[k].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float x = 0.f;
    e = hipEventElapsedTime(&x, h->append_timers[k].first, h->append_timers[k].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    t += x;
  }
  *ms = t;
  *n_calls = (int64_t)h->append_timed;
  h->append_timed = 0;
  return GQA_OK;
}

gqa_status gqa_attn_plan_stats(const gqa_attn* h, gqa_plan_stats* out) {
  if (!h || !out) return fail(GQA_ERR_INVALID_ARG, "NULL argument");
  if (!h->have_plan) return fail(GQA_ERR_INVALID_ARG, "no forward has been planned on this handle");
  fill_stats(h->plan, h->p.head_dim, out);
  return GQA_OK;
}

gqa_status gqa_attn_plan_splits(const gqa_attn* h, int32_t* out, int32_t n) {
  if (!h || !out) return fail(GQA_ERR_INVALID_ARG, "NULL argument");
  if (!h->have_plan) return fail(GQA_ERR_INVALID_ARG, "no forward has been planned on this handle");
  if (n != (int32_t)h->plan.api_splits.size())
    return fail(GQA_ERR_INVALID_ARG, "n must equal n_groups + n_branches of the last forward");
  std::memcpy(out, h->plan.api_splits.data(), sizeof(int32_t) * n);
  return GQA_OK;
}

gqa_status gqa_attn_enable_timing(gqa_attn* h, int32_t enable) {
  if (!h) return fail(GQA_ERR_INVALID_ARG, "handle is NULL");
  h->timing = enable != 0;
  h->timers_used = 0;
  h->append_timed = 0;
  return GQA_OK;
}

}  // extern "C"

namespace {

// Attention and merge milliseconds of the timed forward `t` (when the two
// attention kernels ran side by side: the span from the earlier start to
// the later end).
gqa_status forward_times(TimerSlot& t, double* attn, double* merge) {
  const bool used[3] = {t.wide, t.narrow, t.merged};
  for (int j = 0; j < 3; ++j) {
    if (!used[j]) continue;
    hipError_t e = hipEventSynchronize(t.ev[2 * j + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  }
  *attn = *merge = 0.0;
  for (int j = 0; j < 3; ++j) {
    if (!used[j] || (t.concurrent && j == 1)) continue;
    float ms = 0.f;
    hipError_t e;
    if (t.concurrent && j == 0) {
      float best = 0.f;
      for (int s0 : {0, 2})
        for (int s1 : {1, 3}) {
          e = hipEventElapsedTime(&ms, t.ev[s0], t.ev[s1]);
          if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
          best = std::max(best, ms);
        }
      ms = best;
    } else {
      e = hipEventElapsedTime(&ms, t.ev[2 * j], t.ev[2 * j + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    }
    (j < 2 ? *attn : *merge) += ms;
  }
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_attn_kernel_times(gqa_attn* h, double* attn_ms, double* merge_ms, int64_t* n_forwards) {
  if (!h || !attn_ms || !merge_ms || !n_forwards) return fail(GQA_ERR_INVALID_ARG, "NULL argument");
  double at = 0.0, mg = 0.0;
  for (size_t k = 0; k < h->timers_used; ++k) {
    double a = 0.0, m = 0.0;
    gqa_status s = forward_times(h->timers[k], &a, &m);
    if (s != GQA_OK) return s;
    at += a;
    mg += m;
  }
  *attn_ms = at;
  *merge_ms = mg;
  *n_forwards = (int64_t)h->timers_used;
  h->timers_used = 0;
  return GQA_OK;
}

gqa_status gqa_attn_kernel_times_list(gqa_attn* h, double* attn_ms, double* merge_ms, int64_t cap,
                                      int64_t* n_forwards) {
  if (!h || !n_forwards) return fail(GQA_ERR_INVALID_ARG, "NULL argument");
  const int64_t n = (int64_t)h->timers_used;
  if (cap < n || (n > 0 && (!attn_ms || !merge_ms))) {
    *n_forwards = n;
    return fail(GQA_ERR_INVALID_ARG, "the arrays hold fewer entries than there are timed forwards");
  }
  for (int64_t k = 0; k < n; ++k) {
    gqa_status s = forward_times(h->timers[k], &attn_ms[k], &merge_ms[k]);
    if (s != GQA_OK) return s;
  }
  *n_forwards = n;
  h->timers_used = 0;
  return GQA_OK;
}

gqa_status gqa_attn_plan_host(const gqa_attn_params* p, int32_t n_groups, const int32_t* group_shared_start,
                              const int32_t* group_shared_len, int32_t n_branches, const int32_t* branch_group,
                              const int32_t* branch_q_len, const int32_t* branch_private_len,
                              const int32_t* splits_override, int32_t causal, int32_t* items, int64_t cap,
                              int64_t* n_items, int32_t* splits, gqa_plan_stats* stats) {
  gqa_status s = check_params(p);
  if (s != GQA_OK) return s;
  gqa::PlanInput in;
  s = make_input(p, n_groups, group_shared_start, group_shared_len, n_branches, branch_group, branch_q_len,
                 branch_private_len, splits_override, causal, 256, 1, 1, &in);
  if (s != GQA_OK) return s;
  gqa::Plan P;
  std::string err = gqa::build_plan(in, &P);
  if (!err.empty()) return fail(GQA_ERR_INVALID_ARG, err);
  const int64_t n = (int64_t)(P.wide.size() + P.narrow.size());
  if (n_items) *n_items = n;
  if (items && cap >= n) {
    int64_t k = 0;
    for (int pass = 0; pass < 2; ++pass) {
      const std::vector<gqa::WorkItem>& list = (pass == 0) ? P.wide : P.narrow;
      const std::vector<int32_t>& bins = (pass == 0) ? P.wide_bins : P.narrow_bins;
      int32_t b = 0;
      for (size_t x = 0; x < list.size(); ++x) {
        while (bins[b + 1] <= (int32_t)x) ++b;
        const gqa::WorkItem& w = list[x];
        int32_t* r = items + 10 * k++;
        r[0] = P.unit_slot[w.unit]; r[1] = w.kv; r[2] = w.row_begin; r[3] = w.n_rows;
        r[4] = w.key_begin; r[5] = w.key_end; r[6] = w.split; r[7] = pass; r[8] = b; r[9] = w.chain;
      }
    }
  }
  if (splits) std::memcpy(splits, P.api_splits.data(), sizeof(int32_t) * P.api_splits.size());
  if (stats) fill_stats(P, p->head_dim, stats);
  return GQA_OK;
}

}  // extern "C"

namespace {

double median(std::vector<double> v) {
  if (v.empty()) return 0.0;
  std::sort(v.begin(), v.end());
  const size_t n = v.size();
  return n % 2 ? v[n / 2] : 0.5 * (v[n / 2 - 1] + v[n / 2]);
}

// Runs `launch(k, e0, e1)` reps times on a private stream, each launch
// bracketed by its own events; returns the per-launch milliseconds.
template <class F>
gqa_status time_launches(int32_t reps, F launch, std::vector<double>* ms) {
  hipStream_t st = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "hipStreamCreate");
  std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
  gqa_status s = GQA_OK;
  for (auto& x : ev)
    if (hipEventCreate(&x) != hipSuccess) s = fail(GQA_ERR_HIP, "hipEventCreate");
  for (int32_t k = 0; s == GQA_OK && k < reps; ++k) {
    e = launch(k, st, ev[2 * k], ev[2 * k + 1]);
    if (e != hipSuccess) s = hip_fail(e, "probe launch");
  }
  if (s == GQA_OK) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) s = hip_fail(e, "hipStreamSynchronize");
  }
  for (int32_t k = 0; s == GQA_OK && k < reps; ++k) {
    float x = 0.f;
    e = hipEventElapsedTime(&x, ev[2 * k], ev[2 * k + 1]);
    if (e != hipSuccess) s = hip_fail(e, "hipEventElapsedTime");
    ms->push_back(x);
  }
  for (auto& x : ev)
    if (x) hipEventDestroy(x);
  hipStreamDestroy(st);
  return s;
}

}  // namespace

extern "C" {

gqa_status gqa_probe_mfma_bf16(int32_t waves_per_simd, int32_t iters, int32_t reps, double* tflops, double* ms) {
  if (!tflops || !ms || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || reps < 1)
    return fail(GQA_ERR_INVALID_ARG, "bad probe arguments");
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  // 256-thread workgroups are 4 waves, one per SIMD of a CU.
  const int blocks = ncu * waves_per_simd;
  float* out = nullptr;
  e = hipMalloc((void**)&out, (size_t)blocks * 256 * sizeof(float));
  if (e != hipSuccess) return fail(GQA_ERR_NO_MEMORY, "probe output allocation failed");
  std::vector<double> t;
  gqa_status s = time_launches(reps, [&](int32_t, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    return gqa::launch_probe_mfma(out, blocks, iters, st, e0, e1);
  }, &t);
  (void)hipFree(out);
  if (s != GQA_OK) return s;
  const double med = median(t);
  const double flops = (double)blocks * 4 * iters * 4 * (32.0 * 32 * 16 * 2);
  *ms = med;
  *tflops = med > 0 ? flops / (med * 1e-3) / 1e12 : 0.0;
  return GQA_OK;
}

gqa_status gqa_probe_read(const void* buf, int64_t bytes, int32_t n_copies, int32_t reps, double* gbps, double* us) {
  if (!buf || !gbps || !us || bytes <= 0 || bytes % 16 || n_copies < 1 || reps < 1 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u))
    return fail(GQA_ERR_INVALID_ARG, "bad probe arguments (16-byte aligned buffer of n_copies x bytes, bytes % 16 == 0)");
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  const int blocks = ncu * 8;
  uint32_t* out = nullptr;
  e = hipMalloc((void**)&out, (size_t)blocks * 256 * sizeof(uint32_t));
  if (e != hipSuccess) return fail(GQA_ERR_NO_MEMORY, "probe output allocation failed");
  std::vector<double> t;
  gqa_status s = time_launches(reps, [&](int32_t k, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const char* src = (const char*)buf + (int64_t)(k % n_copies) * bytes;
    return gqa::launch_probe_read(src, bytes, out, blocks, st, e0, e1);
  }, &t);
  (void)hipFree(out);
  if (s != GQA_OK) return s;
  const double med = median(t);
  *us = med * 1e3;
  *gbps = med > 0 ? (double)bytes / (med * 1e-3) / 1e9 : 0.0;
  return GQA_OK;
}

}  // extern "C"
