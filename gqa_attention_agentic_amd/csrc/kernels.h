// Launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_types.h"

namespace gqa {

struct AttnArgs {
  const void* q;
  const void* k_shared;
  const void* v_shared;
  const void* k_pages;
  const void* v_pages;
  const int32_t* page_table;
  const WorkItem* items;
  const int32_t* bins;  // workgroup b runs items [bins[b], bins[b+1])
  const TokRec* tok_rec;    // per query token
  const CombTok* combs;     // per token whose rows have two or more partials
  int32_t* counters;        // [n_q_tokens, H_kv] arrival counters, zero between launches
  float* part_o;        // [part_rows, D] unnormalised partial O
  float2* part_ml;      // [part_rows] (m in log2 units, l)
  void* o;              // [n_q_tokens, H_q, D] storage dtype
  float* lse;           // [n_q_tokens, H_q]
  int32_t max_pages;
  int32_t H_q;
  int32_t H_kv;
  int32_t G;
  int32_t n_shared;     // tokens per KV head in k_shared / v_shared
  int32_t page_size;
  int32_t page_shift;   // log2(page_size) when a power of two, else -1
  int32_t causal;
  int32_t n_q_tokens;
  float scale_log2;     // softmax_scale * log2(e)
  // Narrow kernel, each workgroup runs one item: partials are written with
  // device-scope stores and the arrival needs no release fence (see
  // combine_if_last); otherwise ordinary stores and a release fence.
  int32_t coherent_parts;
};

// Attention over a work-item list: one workgroup per bin (a.bins holds
// n_bins + 1 offsets into a.items). narrow selects the 32-row kernel.
// ev_start / ev_stop (may be null) are recorded by the launch itself around
// the kernel's execution (hipExtLaunchKernelGGL), for kernel-only timing.
hipError_t launch_attention(const AttnArgs& a, int32_t n_bins, bool narrow, int dtype,
                            int head_dim, hipStream_t stream, hipEvent_t ev_start = nullptr,
                            hipEvent_t ev_stop = nullptr);

// Workgroups of the attention kernel for (dtype, head_dim, narrow) that stay
// resident on one CU at once (at least 1).
hipError_t attention_occupancy(int dtype, int head_dim, bool narrow, int* per_cu);

// Log-sum-exp merge of the partials of every output row with >= 2 of them
// that was not combined inside the narrow kernel. max_parts: the largest
// number of partials any output row has.
hipError_t launch_merge(const AttnArgs& a, int dtype, int head_dim, int max_parts, hipStream_t stream,
                        hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);


// Zero fill of n int32 values (fill.hip): the arrival counters.
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t stream);

// Static device scratch of the forwards that allocate nothing (scratch.hip):
// kScratchBytes per device, starting with kScratchCounterBytes of arrival
// counters (zero between forwards), then the plan and the partials.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr size_t kScratchCounterBytes = size_t(1) << 20;

// Device address of the scratch on `device` (which must be current): looked
// up once per device with hipGetSymbolAddress, its counter region cleared
// the first time (a synchronous fill on the null stream).
hipError_t scratch_setup(int device, void** ptr);

// Append of new K and V rows to branches' private pages (append.hip).
struct AppendArgs {
  const void* k_new;        // [n_rows, H_kv, d]
  const void* v_new;
  void* k_pages;            // [n_pages, H_kv, page_size, d]
  void* v_pages;
  const int32_t* page_table;  // [n_branches, max_pages]
  const int2* rows;         // per appended row: (branch, position in its private suffix)
  int32_t max_pages;
  int32_t n_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t row_bytes;        // d x element size (a multiple of 16)
  int32_t pad;
};

hipError_t launch_append(const AppendArgs& p, int32_t n_rows, hipStream_t stream, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr);

// Achievable-peak probes (probe.hip): `blocks` workgroups of 256 threads;
// out holds one value per thread.
hipError_t launch_probe_mfma(float* out, int blocks, int iters, hipStream_t st, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t st,
                             hipEvent_t e0, hipEvent_t e1);

}  // namespace gqa
