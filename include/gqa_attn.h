/*
 * gqa_attn.h -- C ABI of the MI355X (gfx950) shared-prefix GQA attention library.
 *
 * What one forward call computes
 * ------------------------------
 * Causal grouped-query attention with an online softmax over a shared-prefix
 * KV cache, for agentic fan-out (AHBM Agentic Runtime Architecture, §1.1-§1.3
 * and §3.1-§3.4; ADR-0060 GQA fused attention, TL;DR kernel and §3-§5):
 *
 *   - Branches are grouped; a group's branches share one prefix stored once.
 *     Branch b's context is  shared[group(b)] ++ private(b),  where the
 *     private suffix is read through the branch's page table (AHBM Agentic
 *     Runtime Architecture, §3.1).
 *   - Branch b brings q_len(b) new query tokens; they are the last q_len(b)
 *     positions of its context, and key j of the context has position j.
 *   - Query head h reads KV head floor(h / G), G = H_q / H_kv (ADR-0060, §0.5.3).
 *   - z = softmax_scale * q.k; with causal != 0 key j is visible to the query
 *     at position p iff j <= p (ADR-0060, §5.4), otherwise every key of the
 *     branch's context is visible (§5.2).
 *   - O = sum_j softmax(z)_j v_j in the storage dtype (round to nearest even),
 *     LSE = ln(sum_j exp(z_j)) in fp32 (natural log, scaled-score units).
 *
 * Internally the library folds the G query heads of a KV head and the query
 * tokens of all branches of a group into one M dimension (ADR-0060, §5.2;
 * AHBM Agentic Runtime Architecture, §3.2), splits each KV range into shards
 * whose (m, l, O) partials are combined by a log-sum-exp merge (ADR-0060,
 * §4: in a separate merge launch, or, for rows whose partials all come from
 * the decode-like kernel, by the last of their items to finish), and skips
 * KV tiles that lie entirely in the future of a query block
 * (ADR-0060, §5.4). None of that is visible in the result beyond rounding.
 *
 * Conventions
 * -----------
 * Pointers are DEVICE pointers unless the comment says (host). The caller owns
 * every buffer; the library reads inputs, writes only `o` and `lse`, and never
 * writes K/V (the cache is appended upstream before launch: ADR-0060, §0.5.1).
 * Calls are stream-ordered and asynchronous: gqa_attn_forward returns without
 * waiting for the GPU. Host arrays may be reused as soon as a call returns.
 * One handle serves one stream at a time; concurrent calls on one handle race.
 * A forward with both decode-like and MFMA-bound work runs part of it on a
 * side stream that the handle owns (default priority), forked from and
 * joined back into the caller's stream with events; the forward's work is
 * still complete when the caller's stream reaches the point after the call.
 * Every entry point returns a gqa_status; on a negative status nothing was
 * launched and gqa_attn_last_error() holds a message (thread-local).
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = -1,   /* a size, pointer, alignment or length is wrong */
  GQA_ERR_UNSUPPORTED = -2,   /* valid request the library does not implement */
  GQA_ERR_NO_MEMORY = -3,     /* workspace or plan buffers could not be allocated
                                 (or would exceed workspace_bytes_cap)          */
  GQA_ERR_HIP = -4            /* a HIP runtime call or kernel launch failed     */
} gqa_status;

typedef enum {
  GQA_BF16 = 0,               /* Q, K, V, O in bfloat16; bf16 MFMA, fp32 accumulate */
  GQA_FP32 = 1                /* Q, K, V, O in float32; fp32 MFMA                   */
} gqa_dtype;

typedef struct {
  int32_t num_q_heads;        /* H_q, > 0, a multiple of num_kv_heads              */
  int32_t num_kv_heads;       /* H_kv, > 0                                         */
  int32_t head_dim;           /* d: 64 or 128                                      */
  int32_t page_size;          /* tokens per private page, 1..4096                  */
  int32_t dtype;              /* gqa_dtype                                         */
  float softmax_scale;        /* <= 0 selects 1/sqrt(d) (ADR-0060, §0.5.3)         */
  int64_t workspace_bytes_cap;/* cap on the split-partial workspace; 0 = no cap    */
} gqa_attn_params;

typedef struct gqa_attn gqa_attn;   /* opaque: plan buffers, workspace, timers */

/* Create a handle for fixed head geometry and dtype. `p` (host) is copied.
 * Errors: GQA_ERR_INVALID_ARG for bad parameters, GQA_ERR_UNSUPPORTED for a
 * head_dim other than 64/128 or more than 256 (bf16) / 128 (fp32) query
 * heads per KV head (the rows of one token must fit one M-tile of the
 * MFMA kernel), GQA_ERR_HIP if no HIP device is usable. */
gqa_status gqa_attn_create(const gqa_attn_params* p, gqa_attn** out);

/* One attention forward over a set of groups and branches.
 *
 *  q          [n_q_tokens, H_q, d]      branch b's q_len tokens are contiguous,
 *                                       branches in order (n_q_tokens = sum q_len)
 *  k_shared   [H_kv, n_shared_tokens, d]  shared prefixes of all groups,
 *  v_shared                             concatenated along the token axis
 *  n_shared_tokens  token extent (stride) of k_shared / v_shared; every
 *             group's [start, start + len) must lie inside it
 *  k_pages    [n_pages, H_kv, page_size, d]  private-suffix page pool
 *  v_pages
 *  page_table [n_branches, max_pages_per_branch] int32 physical page ids;
 *             entries past a branch's last page are ignored (pad with -1)
 *  n_groups, group_shared_start (host), group_shared_len (host):
 *             group g's prefix is tokens [start, start + len) of k_shared
 *  n_branches, branch_group (host), branch_q_len (host),
 *  branch_private_len (host): per branch; the branches of one group must be
 *             consecutive, and 0 <= q_len <= shared_len + private_len
 *  splits_override (host) [n_groups + n_branches] or NULL: KV shards per
 *             unit -- one entry per group prefix, then one per branch suffix;
 *             0 lets the library's split heuristic choose
 *  causal     0 or 1
 *  o          out [n_q_tokens, H_q, d] storage dtype
 *  lse        out [n_q_tokens, H_q] float32, natural log
 *  stream     hipStream_t (NULL = default stream)
 *
 * The page table's contents are a precondition (every id of a page a branch
 * uses must be a page of the pool); they are not checked on the device.
 * q, k/v and o must be 16-byte aligned, page_table and lse 4-byte aligned;
 * a pointer whose extent is zero may be NULL. Errors: GQA_ERR_INVALID_ARG, GQA_ERR_NO_MEMORY (workspace growth),
 * GQA_ERR_HIP (launch failure). On GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED
 * and GQA_ERR_NO_MEMORY nothing was launched: arguments, metadata and every
 * allocation are settled before the first launch.
 *
 * Plan and buffers: the plan is rebuilt only when the metadata differs from
 * the previous call on this handle. The handle grows its device buffers (the
 * plan, the arrival counters, the partial workspace) when a plan needs more
 * than they hold. A call whose plan is cached (same metadata as the previous
 * call, buffers already large enough) issues only kernel launches and, when
 * its two attention kernels run side by side, the event fork / join of the
 * handle's side stream: it allocates nothing and uploads nothing.
 *
 * HIP graph capture: a forward made while `stream` is capturing must be such
 * a cached call; any other returns GQA_ERR_INVALID_ARG (make the same call
 * once outside capture first). Buffers that a captured forward references
 * are kept, unchanged in meaning, until the handle is destroyed: later
 * forwards with other metadata get new buffers, so the graph stays valid.
 * Its replays share the partial workspace and counters with the handle's
 * other calls, so they must be ordered with them on the device. Timing
 * events are not recorded under capture. */
gqa_status gqa_attn_forward(gqa_attn* h,
                            const void* q,
                            const void* k_shared, const void* v_shared,
                            int32_t n_shared_tokens,
                            const void* k_pages, const void* v_pages,
                            const int32_t* page_table, int32_t max_pages_per_branch,
                            int32_t n_groups, const int32_t* group_shared_start,
                            const int32_t* group_shared_len,
                            int32_t n_branches, const int32_t* branch_group,
                            const int32_t* branch_q_len, const int32_t* branch_private_len,
                            const int32_t* splits_override,
                            int32_t causal,
                            void* o, float* lse,
                            void* stream);

/* The same forward, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Arguments, semantics and errors are those of
 * gqa_attn_forward; the differences are where its scratch lives and what
 * that costs:
 *  - The plan, the arrival counters and the split-KV partials go to a
 *    static device array of the library (64 MiB per GPU, 1 MiB of it
 *    counters), one per GPU, held until the process ends; its address is
 *    looked up by gqa_attn_create. The call makes no hipMalloc / hipFree /
 *    hipHostMalloc and no allocating library call; the host planner uses
 *    ordinary heap memory when the metadata changes.
 *  - A forward whose plan and partials do not fit returns
 *    GQA_ERR_NO_MEMORY before any launch (a 128-byte counter per KV head for
 *    each token combined inside the decode-class launch -- 1024 such tokens
 *    at 8 KV heads -- must fit 1 MiB; plan + partial rows x (d + 2) x 4
 *    bytes the rest). The
 *    fan-out and decode workloads fit; a long prefill split into many
 *    shards does not -- use gqa_attn_forward for it.
 *  - Every call on one GPU, from any handle, shares that GPU's array, which
 *    keeps the last call's plan and partials: calls that overlap on one GPU
 *    (different streams, or different host threads without ordering) race.
 *    The counters are zero between calls. A plan is uploaded (a pageable
 *    host-to-device copy on `stream`) when the array holds another one.
 *  - Under HIP graph capture the call must find its own plan in the array
 *    (the same call made once outside capture, with nothing in between
 *    replacing it); a replay is valid only while no call with other
 *    metadata has replaced the array's plan since.
 *  - The two attention kernels run side by side only if the handle already
 *    has its side stream (made by an earlier gqa_attn_forward that needed
 *    it); otherwise one after the other on `stream`, with the same result.
 *  - No timing events are recorded. */
gqa_status gqa_attn_forward_noalloc(gqa_attn* h,
                                    const void* q,
                                    const void* k_shared, const void* v_shared,
                                    int32_t n_shared_tokens,
                                    const void* k_pages, const void* v_pages,
                                    const int32_t* page_table, int32_t max_pages_per_branch,
                                    int32_t n_groups, const int32_t* group_shared_start,
                                    const int32_t* group_shared_len,
                                    int32_t n_branches, const int32_t* branch_group,
                                    const int32_t* branch_q_len, const int32_t* branch_private_len,
                                    const int32_t* splits_override,
                                    int32_t causal,
                                    void* o, float* lse,
                                    void* stream);

/* Append new K and V rows to branches' private pages: the step before a
 * forward that attends to them. A branch's context is its group's shared
 * prefix (referenced, never copied) followed by its private pages, filled
 * slot after slot (AHBM Agentic Runtime Architecture, §3.1); the cache is
 * written before attention reads it, with K already rotated by RoPE
 * (ADR-0060 GQA fused attention, §0.5.1 and §2.1).
 *
 *  k_new, v_new [n_new_rows, H_kv, d] storage dtype: branch b's
 *             branch_n_new(b) rows contiguous, branches in order
 *  k_pages    [n_pages, H_kv, page_size, d]  the pool, written in place
 *  v_pages
 *  page_table [n_branches, max_pages_per_branch] int32 physical page ids
 *  branch_private_len (host) [n_branches]: private tokens each branch has
 *             before the call; branch_n_new (host) [n_branches]: rows added
 *  stream     hipStream_t (NULL = default stream)
 *
 * Row i of branch b becomes private token p = private_len(b) + i, stored at
 * page page_table[b][p / page_size], slot p % page_size; the copy is
 * bit-exact. private_len(b) + n_new(b) must fit the branch's table row. A
 * page id outside [0, n_pages) is a broken precondition: that row is not
 * written. Stream-ordered and asynchronous like gqa_attn_forward; the
 * per-row list is uploaded only when (private_len, n_new) differ from the
 * previous call's. Errors:
 * GQA_ERR_INVALID_ARG, GQA_ERR_NO_MEMORY (growth of the handle's row list),
 * GQA_ERR_HIP. */
gqa_status gqa_attn_append_kv(gqa_attn* h, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                              int32_t n_pages, const int32_t* page_table, int32_t max_pages_per_branch,
                              int32_t n_branches, const int32_t* branch_private_len,
                              const int32_t* branch_n_new, void* stream);

/* Release the handle (waits for its outstanding work). NULL is accepted. */
gqa_status gqa_attn_destroy(gqa_attn* h);

/* Thread-local message describing the last non-OK status ("" if none). */
const char* gqa_attn_last_error(void);

/* Summary of the plan used by the most recent forward on `h` (host). */
typedef struct {
  int64_t n_items_wide;       /* work items on the 128-row MFMA kernel            */
  int64_t n_items_narrow;     /* work items on the 32-row decode kernel           */
  int64_t n_kv_tiles;         /* (item, KV tile) pairs the kernels will process   */
  int64_t n_merge_rows;       /* output rows (token, head) combined by the merge  */
  int64_t workspace_bytes;    /* partial-state workspace in use                   */
  int64_t n_units;            /* group prefixes + branch suffixes with keys       */
  int32_t max_splits;         /* largest split count of any unit                  */
  int32_t merge_launch;       /* 1 if the forward makes a separate merge launch;
                                 0 when every row with several partials is
                                 combined inside the narrow attention launch */
  int32_t wide_cus;           /* compute units given to each attention kernel:  */
  int32_t narrow_cus;         /* both the device's count, unless the forward has
                                 items of both kernels, which then run side by
                                 side on disjoint CUs (wide + narrow = device) */
} gqa_plan_stats;
gqa_status gqa_attn_plan_stats(const gqa_attn* h, gqa_plan_stats* out);

/* Split count chosen for each unit by the last forward (host array of
 * n_groups + n_branches entries, same order as splits_override; 0 for a
 * unit without keys or without queries). */
gqa_status gqa_attn_plan_splits(const gqa_attn* h, int32_t* out, int32_t n);

/* Kernel timing with HIP events that each launch records around its own
 * kernel's execution on the forward's stream (hipExtLaunchKernelGGL start /
 * stop events). enable != 0 starts recording (and clears earlier records).
 * gqa_attn_kernel_times waits for the recorded events and returns the summed
 * milliseconds of every forward since timing was enabled -- attn_ms sums the
 * attention launches (wide and narrow; when the two run side by side, the
 * span from the earlier start to the later end), merge_ms the separate
 * merge launch --
 * and the number of forwards, then clears the records. Rows whose partials
 * all come from the narrow (decode-like) kernel are combined inside that
 * launch, so their merge time is part of attn_ms; a forward with no other
 * such rows makes no merge launch and adds 0 to merge_ms. The events are not
 * free: on MI355X consecutive launches that record them start ~9 us apart
 * instead of back to back, so timing is best left off outside measurement. */
gqa_status gqa_attn_enable_timing(gqa_attn* h, int32_t enable);
gqa_status gqa_attn_kernel_times(gqa_attn* h, double* attn_ms, double* merge_ms,
                                 int64_t* n_forwards);

/* The same records forward by forward: attn_ms[k] and merge_ms[k] (host
 * arrays of at least `cap` entries) for the k-th timed forward, in issue
 * order; *n_forwards is their number. Clears the records like
 * gqa_attn_kernel_times. GQA_ERR_INVALID_ARG (records kept, *n_forwards
 * set) when cap is smaller than that number. */
gqa_status gqa_attn_kernel_times_list(gqa_attn* h, double* attn_ms, double* merge_ms, int64_t cap,
                                      int64_t* n_forwards);

/* Kernel time of the appends made while timing is enabled (events that each
 * append launch records around its own kernel, like gqa_attn_kernel_times):
 * summed milliseconds and the number of appends, then cleared. */
gqa_status gqa_attn_append_times(gqa_attn* h, double* ms, int64_t* n_calls);

/* Host-only planner check (no device use): plans the given metadata with
 * the handle-free parameters `p` for a 256-CU device with one resident
 * workgroup per CU and writes, for every work item, the tuple
 * (unit, kv_head, row_begin, n_rows, key_begin, key_end, split, kernel, bin,
 *  chain)
 * into `items` (host, int32, 10 per item) when `items` is not NULL and `cap`
 * allows. Items are listed per kernel in launch order: workgroup `bin` of
 * that kernel runs its items one after another, in the order listed.
 * `chain` is 0 for an item on its own; otherwise bit 0 says the item starts
 * from the previous item's (m, l, O) state and bit 1 that it hands its state
 * to the next item instead of writing it (the shards of one M-tile and KV
 * head run back to back, merged in registers; in a group with a single
 * branch the prefix's chain continues into the same rows' suffix shards).
 * Returns the item count through *n_items and the per-unit split counts
 * through `splits` (host, n_groups + n_branches entries, may be NULL). */
gqa_status gqa_attn_plan_host(const gqa_attn_params* p,
                              int32_t n_groups, const int32_t* group_shared_start,
                              const int32_t* group_shared_len,
                              int32_t n_branches, const int32_t* branch_group,
                              const int32_t* branch_q_len, const int32_t* branch_private_len,
                              const int32_t* splits_override, int32_t causal,
                              int32_t* items, int64_t cap, int64_t* n_items,
                              int32_t* splits, gqa_plan_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
