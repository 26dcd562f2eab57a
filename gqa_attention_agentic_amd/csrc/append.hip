// Paged K/V append for gfx950: the step before a forward.
//
// A branch's private suffix lives in pages reached through its page table
// and grows by appending (AHBM Agentic Runtime Architecture, §3.1: a
// branch's context is its group's shared prefix, referenced without
// copying, followed by its own pages). The attention kernel only reads the
// cache; the new post-RoPE K rows and V rows are written before it runs
// (ADR-0060 GQA fused attention, §0.5.1 and §2.1: tokens are appended to the
// cache contiguously, slot after slot).
//
// A workgroup moves kRows appended rows: each thread first loads its
// 16-byte chunks of the new K and V rows (all in flight together), then
// stores them to page table[b][p / ps], slot p % ps, where p is the row's
// position in the branch's private suffix; the destination rows are looked
// up once per workgroup. The copy is bit-exact. HBM-bound: bytes per row =
// 2 (K, V) x H_kv x d x element size, read once and written once.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace gqa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 8;        // appended rows per workgroup
constexpr int kThreads = 256;
constexpr int kBatch = 8;       // chunks a thread has in flight

__global__ void __launch_bounds__(kThreads) append_kv_rows(AppendArgs p, int n_rows) {
  __shared__ int64_t dst_row[kRows];   // byte offset of the row's (page, head 0, slot), or -1
  const int64_t row0 = (int64_t)blockIdx.x * kRows;
  const int nr = (int)min((int64_t)kRows, (int64_t)n_rows - row0);
  if ((int)threadIdx.x < nr) {
    const int2 bp = p.rows[row0 + threadIdx.x];   // (branch, position in its private suffix)
    const int lp = bp.y / p.page_size, slot = bp.y - lp * p.page_size;
    const int page = p.page_table[(int64_t)bp.x * p.max_pages + lp];
    // A page id outside the pool is a broken precondition: the row is not
    // written rather than written out of bounds.
    dst_row[threadIdx.x] = (page < 0 || page >= p.n_pages)
                               ? -1
                               : ((int64_t)page * p.num_kv_heads * p.page_size + slot) * p.row_bytes;
  }
  const int cpr = p.row_bytes / 16;                 // 16-byte chunks per head row
  const int per_tensor = p.num_kv_heads * cpr;      // chunks of one row's K (or V)
  const int per_row = 2 * per_tensor;
  const int total = nr * per_row;
  // The loop variable is the same for every thread, so every thread takes
  // the barrier of the first round (which publishes dst_row) after issuing
  // its first loads.
  for (int base = 0; base < total; base += kThreads * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      // Chunks past the end load the last chunk instead (in bounds, never stored).
      const int c = min(base + k * kThreads + (int)threadIdx.x, total - 1);
      const int rr = c / per_row, rem = c - rr * per_row;
      const int tensor = rem >= per_tensor ? 1 : 0;
      const int w = rem - tensor * per_tensor;      // head * cpr + chunk
      v[k] = *(const u32x4*)((const char*)(tensor ? p.v_new : p.k_new) +
                             ((row0 + rr) * p.num_kv_heads * cpr + w) * 16);
    }
    if (base == 0) __syncthreads();
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = base + k * kThreads + (int)threadIdx.x;
      if (c < total) {
        const int rr = c / per_row, rem = c - rr * per_row;
        const int tensor = rem >= per_tensor ? 1 : 0;
        const int w = rem - tensor * per_tensor;
        const int head = w / cpr, ch = w - head * cpr;
        const int64_t d0 = dst_row[rr];
        if (d0 >= 0)
          *(u32x4*)((char*)(tensor ? p.v_pages : p.k_pages) + d0 + (int64_t)head * p.page_size * p.row_bytes +
                    ch * 16) = v[k];
      }
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& p, int32_t n_rows, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
  if (n_rows <= 0) return hipSuccess;
  hipExtLaunchKernelGGL(append_kv_rows, dim3((n_rows + kRows - 1) / kRows), dim3(kThreads), 0, stream, ev_start,
                        ev_stop, 0, p, n_rows);
  return hipGetLastError();
}

}  // namespace gqa
