/*
 * sarathi_attn.h -- C ABI of libsarathi_attn: the per-iteration data-plane step
 * of chunked prefills with stall-free batching, for one attention layer on one
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (their titles and sections):
 *   [S1] "Sarathi-Serve：以 chunked-prefills 与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡"
 *   [S2] "In-flight Batching"
 *   [S3] "Sarathi-Serve: Chunked Prefills for Stall-Free LLM Inference"
 *
 * Conventions shared by every call
 *   - Every call returns sa_status; SA_OK (0) is success.  On failure,
 *     sa_last_error() returns a thread-local text describing the last failure
 *     of the calling thread.  No C++ exception crosses this boundary.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are GPU
 *     memory (e.g. from hipMalloc or a PyTorch CUDA/HIP tensor).  The library
 *     never allocates device memory and never frees caller memory; the only
 *     heap it owns is the scheduler handle, and the only device memory of its
 *     own is the static workspace of sa_hybrid_attn_noalloc (part of its code
 *     object, one per GPU).
 *   - Device calls enqueue work on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and return without waiting.  Launch
 *     failures are reported as SA_ERR_HIP; faults inside a kernel surface at
 *     the caller's next synchronisation of that stream.
 *   - bf16 tensors are passed as raw 16-bit words (uint16 storage).
 *
 * Paged KV cache layout (owned by the caller, one pair per layer):
 *   page size is 16 tokens ([S2] KV Cache 管理的协同优化).  With P physical
 *   pages, Hkv kv heads and head_dim d:
 *     k_cache: bf16 [P][Hkv][16][d]   -- token-major within a page
 *     v_cache: bf16 [P][Hkv][d][16]   -- dim-major within a page (transposed)
 *   A logical slot is page*16 + offset.  V is stored transposed so that the
 *   matrix-core product P*V reads 8 consecutive keys of one dim as one
 *   16-byte load.
 */
#ifndef SARATHI_ATTN_H
#define SARATHI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1,     /* bad shape, null pointer, out-of-range value        */
  SA_ERR_BUDGET = 2,          /* running decodes exceed the token budget             */
  SA_ERR_NO_PAGES = 3,        /* the page pool cannot supply a required page         */
  SA_ERR_CAPACITY = 4,        /* caller buffer too small; required sizes written back */
  SA_ERR_UNKNOWN_REQUEST = 5, /* request id not known to the scheduler               */
  SA_ERR_HIP = 6,             /* a HIP runtime call or kernel launch failed          */
  SA_ERR_UNSUPPORTED = 7,     /* shape the kernels do not implement (e.g. head_dim)  */
  SA_ERR_STATE = 8            /* call out of order (e.g. commit of a stale batch)    */
} sa_status;

/* Text of the calling thread's last failure ("" if none).  Valid until the
 * thread's next failing call. */
const char* sa_last_error(void);

/* Library version string, e.g. "sarathi_attn 0.1 gfx950". */
const char* sa_version(void);

/* ======================================================================
 * Scheduler (host only).  The stall-free batch builder: [S1] 核心机制-2
 * (Algorithm 3: running decodes, then unfinished prefill chunks, then new
 * admissions, under the token budget B; decodes are always in the batch and
 * the batch never exceeds B), [S3] The mechanism (chunk ~ B - n_decode, one
 * or more chunks per iteration), [S2] 调度状态机 (waiting -> prefill, possibly
 * in several chunks -> decode -> completed).  Readings where the pages are
 * silent, all fixed here:
 *   - decodes in running (admission) order, one token each; a decode whose
 *     new token starts a page takes one page from the pool;
 *   - chunk = min(prompt tokens left, B - tokens so far), greedy;
 *   - admission FCFS, head-of-line blocking; a new request reserves
 *     ceil(prompt_len/16) pages for its whole prompt at admission;
 *   - the pool is a FIFO, initial order given at create; freed pages return
 *     to its tail in logical order; no preemption;
 *   - the iteration that runs a prompt's last chunk yields its first output
 *     token; a request finishes once it generated max_new_tokens tokens.
 * A handle is not thread-safe: one thread at a time per handle.
 * ==================================================================== */
typedef struct {
  int32_t token_budget;        /* B >= 1                                         */
  int32_t page_size;           /* must be 16                                     */
  int32_t max_blocks_per_seq;  /* W >= 1: block-table width; a request may span
                                  at most 16*W positions (prompt + outputs - 1)  */
  int32_t num_pages;           /* size of the physical page pool, >= 1           */
} sa_sched_config;

typedef struct sa_sched sa_sched;   /* opaque */

/* free_pages: host int32[num_pages], a permutation of 0..num_pages-1 giving
 * the initial FIFO order.  *out receives a new handle (free with destroy). */
sa_status sa_sched_create(const sa_sched_config* cfg, const int32_t* free_pages, sa_sched** out);
void sa_sched_destroy(sa_sched* s);

/* Deep copy of a scheduler state (for snapshots/restarts). */
sa_status sa_sched_clone(const sa_sched* src, sa_sched** out);

/* Batch-building policy.  SA_POLICY_STALL_FREE (the default) is the
 * stall-free builder described above.  The other two are the baselines the
 * pages set it against ("Sarathi-Serve：以 chunked-prefills 与 stall-free
 * batching 驯服 LLM 推理的吞吐—延迟权衡", 问题背景: prefill-prioritizing vLLM /
 * Orca and decode-prioritizing request-level batching): an iteration is either
 * whole prompts only -- unfinished prompts first, then admissions FCFS while
 * KV pages allow, each whole, while the iteration's tokens stay within
 * prefill_token_limit (the first prompt always) -- during which every running
 * decode waits, or, when no prompt can run, all running decodes (at most
 * prefill_token_limit of them, else SA_ERR_BUDGET).
 *   SA_POLICY_PREFILL_FIRST: admissions whenever pages allow;
 *   SA_POLICY_DECODE_FIRST:  admissions only while nothing is running, so a
 *                            cohort decodes to its end before the next starts.
 * token_budget is not used by the baselines.  Errors: SA_ERR_INVALID_ARG
 * (unknown policy, limit < 1 for a baseline). */
enum { SA_POLICY_STALL_FREE = 0, SA_POLICY_PREFILL_FIRST = 1, SA_POLICY_DECODE_FIRST = 2 };
sa_status sa_sched_set_policy(sa_sched* s, int32_t policy, int32_t prefill_token_limit);

/* Enqueue a new request (num_computed = num_generated = 0), or inject one
 * already in flight (resume hook):
 *   0 < num_computed < prompt_len, num_generated = 0: a prefill in progress,
 *       reserves ceil(prompt_len/16) pages now;
 *   num_computed = prompt_len, 1 <= num_generated < max_new_tokens: a decode,
 *       reserves ceil((prompt_len + num_generated - 1)/16) pages now.
 * Pages are popped from the pool head in call order.  Errors: duplicate id or
 * bad lengths -> SA_ERR_INVALID_ARG; pool too small -> SA_ERR_NO_PAGES (state
 * unchanged).  Any successful call invalidates a built-but-uncommitted batch. */
sa_status sa_sched_add_request(sa_sched* s, int64_t req_id, int32_t prompt_len, int32_t max_new_tokens,
                               int32_t num_computed, int32_t num_generated);

/* Counts of running requests, waiting requests and free pages. */
sa_status sa_sched_stats(const sa_sched* s, int32_t* num_running, int32_t* num_waiting, int32_t* num_free_pages);

/* One batch, in caller-owned HOST buffers.  cap_* are inputs; the rest are
 * outputs.  Sequence order: decodes [0, num_decodes), then prefill chunks. */
typedef struct {
  int32_t cap_seqs;            /* in: capacity of the per-sequence arrays        */
  int32_t cap_tokens;          /* in: capacity of slot_mapping                   */
  int32_t num_seqs;            /* out: S                                         */
  int32_t num_decodes;         /* out: D                                         */
  int32_t num_prefill_chunks;  /* out: S - D                                     */
  int32_t num_tokens;          /* out: T = cu_seqlens_q[S] <= B                  */
  int32_t max_blocks_per_seq;  /* out: W, the row stride of block_tables         */
  int32_t max_kv_len;          /* out: max over sequences of context + q_len     */
  int64_t* req_ids;            /* [cap_seqs]                                     */
  int32_t* cu_seqlens_q;       /* [cap_seqs + 1] prefix sums of q_len            */
  int32_t* context_lens;       /* [cap_seqs] tokens in the cache before the step */
  int32_t* block_tables;       /* [cap_seqs * W] physical pages, -1 padded       */
  int32_t* slot_mapping;       /* [cap_tokens] slot of each new token            */
} sa_batch;

/* Build this iteration's batch (see the scheduler notes above).  The batch
 * is recorded as pending; pages are taken and admissions happen here, and
 * progress advances at sa_sched_commit.  On any error the state is unchanged.
 * SA_ERR_CAPACITY: the required num_seqs / num_tokens are written to the
 * count fields.  Building again before commit replaces the pending batch; the
 * pages and admissions of the earlier build stay in effect, so the state
 * stays consistent and the new batch is the same one. */
sa_status sa_build_batch(sa_sched* s, sa_batch* out);

/* Advance progress for the pending batch after it ran: decodes generate one
 * token; chunks add their tokens (the last chunk yields the first output
 * token).  Finished requests leave and free their pages.  Their ids are
 * written to finished_ids (host int64[cap]) in batch order.  The batch must
 * be the one returned by the last sa_build_batch (same req_ids and q_lens),
 * else SA_ERR_STATE. */
sa_status sa_sched_commit(sa_sched* s, const sa_batch* b, int64_t* finished_ids, int32_t cap,
                          int32_t* num_finished);

/* Slots of every cached position 0..context_len-1 of every sequence of the
 * batch, in batch order (host int32[cap]; *count receives the total).  Used to
 * place history K/V into the paged cache with sa_kv_append. */
sa_status sa_history_slots(const sa_batch* b, int32_t* slots, int64_t cap, int64_t* count);

/* ======================================================================
 * Device metadata.  sa_batch_upload packs a host batch, plus the work plan of
 * the attention kernels for the given head shape, into one pinned host
 * staging buffer and enqueues ONE copy of it into a device buffer.  The
 * caller keeps both buffers alive and the staging buffer unmodified until
 * that copy has completed on `stream`.
 * ==================================================================== */
typedef struct {
  /* device pointers into dev_buf */
  const int32_t* cu_seqlens_q;   /* [S + 1]                 */
  const int32_t* context_lens;   /* [S]                     */
  const int32_t* slot_mapping;   /* [T]                     */
  const int32_t* block_table_offsets;  /* [S]: start of sequence s's pages in block_tables */
  const int32_t* block_tables;   /* ragged: sequence s's ceil((context+q_len)/16) pages
                                    in logical order, from block_table_offsets[s] */
  const int32_t* work;           /* opaque work plan        */
  const int32_t* combine;        /* opaque combine plan     */
  /* host scalars */
  int32_t num_seqs, num_decodes, num_tokens, bt_stride;  /* bt_stride: pages of the widest sequence */
  int32_t num_q_heads, num_kv_heads, head_dim, num_pages;
  int32_t num_work_items, num_combine_groups, num_partials;
  int32_t sliding_window;        /* 0: none; see sa_batch_pack */
  int32_t plan_flags;            /* set by sa_batch_pack, read by sa_hybrid_attn:
                                    SA_PLAN_STREAM_KV (decode items read >= 90% of the
                                    plan's key tiles and >= 320 MB of K/V: the decode
                                    path reads K/V with non-temporal loads) */
  int32_t reserved;
} sa_batch_dev;
enum { SA_PLAN_STREAM_KV = 1 };

/* Bytes of staging/device buffer that sa_batch_upload needs (the work plan,
 * and so the size, depends on the head shape and the window). */
sa_status sa_batch_upload_size(const sa_batch* b, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t sliding_window, size_t* bytes);

/* The host half of sa_batch_upload: checks the batch (monotone cu_seqlens,
 * decodes have q_len 1, every page a sequence uses is in [0, num_pages), head
 * shape supported: head_dim 64 or 128, Hq % Hkv == 0, sliding_window >= 0)
 * and packs metadata and work plan into host_staging (at least
 * sa_batch_upload_size bytes, 16-byte aligned).
 * sliding_window: w > 0 restricts the row at absolute position p to keys
 * p-w+1 .. p (sliding-window model variants, "Sarathi-Serve: Chunked
 * Prefills for Stall-Free LLM Inference", Results and evidence); the plan
 * then skips the 32-key tiles wholly before a block's window; 0 = no
 * window.  It is recorded in `out` and applied by sa_hybrid_attn.  `out` describes the layout as it will be once the packed bytes
 * are copied to dev_buf (16-byte aligned; only its address is used, nothing
 * is read or written there).  No device call is made: the caller copies
 * sa_batch_upload_size bytes from host_staging to dev_buf before a kernel
 * uses `out`.  Errors: SA_ERR_INVALID_ARG (batch or buffers),
 * SA_ERR_UNSUPPORTED (head_dim), SA_ERR_CAPACITY (bytes too small). */
sa_status sa_batch_pack(const sa_batch* b, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t sliding_window, int32_t num_pages, void* host_staging, const void* dev_buf,
                        size_t bytes, sa_batch_dev* out);

/* sa_batch_pack, then one copy of the packed bytes into dev_buf on `stream`:
 * when host_staging is pinned (hipHostMalloc; it then has a device address)
 * a small kernel reads it over PCIe, otherwise hipMemcpyAsync copies it
 * (synchronously for pageable memory).  SA_ERR_HIP if the copy cannot be
 * enqueued. */
sa_status sa_batch_upload(const sa_batch* b, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t sliding_window, int32_t num_pages, void* host_staging, void* dev_buf,
                          size_t bytes, void* stream, sa_batch_dev* out);

/* sa_batch_upload followed by sa_kv_append(k_new, v_new, k_cache, v_cache,
 * out->slot_mapping, T, num_kv_heads, head_dim, num_pages), enqueued on
 * `stream` as ONE kernel: part of its workgroups copy the packed bytes into
 * dev_buf while the others scatter the step's new K/V rows into their
 * pages, reading the slot mapping from host_staging (the append of "Sarathi-
 * Serve：以 chunked-prefills 与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡",
 * GPU/系统数据路径 ⑤).  The cache ends bit-identical to the two calls, and
 * dev_buf holds the same bytes.  host_staging must be pinned (hipHostMalloc):
 * SA_ERR_INVALID_ARG otherwise (and for null or unaligned tensors when the
 * batch has tokens); the other errors as sa_batch_pack, SA_ERR_HIP if the
 * launch fails.  Buffers and lifetimes as sa_batch_upload and sa_kv_append. */
sa_status sa_batch_upload_append(const sa_batch* b, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t sliding_window, int32_t num_pages, void* host_staging, void* dev_buf,
                                 size_t bytes, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 void* stream, sa_batch_dev* out);

/* ======================================================================
 * Paged KV append ([S1] GPU / 系统数据路径 step ⑤: a chunk appends its new
 * K/V, a decode writes its one new token; [S2] KV Cache 管理的协同优化).
 *   k_new, v_new: device bf16 [T][Hkv][d] (row-major);
 *   slot_mapping: device int32 [T]; slot < 0 means "skip"; slots must be
 *                 distinct (two writes to one slot race);
 *   k_cache, v_cache: device, layout above, num_pages pages.
 * Slots >= 16*num_pages are skipped (no write).  head_dim 64 or 128.
 * Enqueue before sa_hybrid_attn on the same stream. */
sa_status sa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim, int32_t num_pages, void* stream);

/* ======================================================================
 * Hybrid-batch attention ([S1] GPU / 系统数据路径 steps ③-⑤: D single-token
 * decodes plus one or more prefill chunks in one step; a chunk row at absolute
 * position p attends causally to keys 0..p of its own prompt -- the earlier
 * chunks re-read from the cache plus its own rows; a decode attends to its
 * whole history plus itself; [S2] 技术原理: decode reads the whole KV cache).
 *   q:   device bf16 [T][Hq][d]; rows of sequence s are cu_seqlens_q[s]..;
 *   out: device bf16 [T][Hq][d];
 *   q head h reads kv head h / (Hq/Hkv) (grouped-query attention);
 *   softmax_scale multiplies q.k (usually 1/sqrt(d));
 *   b->sliding_window > 0 (set by sa_batch_pack) limits the row at position
 *   p to keys p-w+1 .. p.
 * The cache must already hold every key 0..context+q_len-1 of each sequence
 * (this step's rows included, via sa_kv_append).  workspace: device memory of
 * at least sa_hybrid_attn_workspace_size bytes (fp32 partial results of
 * column blocks whose keys are split over several workgroups); its contents
 * need no initialisation and are dead after the call.  Two calls that share
 * a workspace must not overlap in time.  Accumulation is fp32; outputs are
 * rounded to bf16 (nearest-even).  One attention launch, plus one merge
 * launch when the plan splits a block (b->num_combine_groups > 0). */
sa_status sa_hybrid_attn_workspace_size(const sa_batch_dev* b, size_t* bytes);
sa_status sa_hybrid_attn(const void* q, const void* k_cache, const void* v_cache, const sa_batch_dev* b,
                         float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* sa_hybrid_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and result as sa_hybrid_attn (the same kernels
 * and plan: the output is identical bit for bit), but the workspace is the
 * library's own static device array of SA_NOALLOC_WORKSPACE_BYTES (64 MiB),
 * one per GPU, resolved on the first call on each device and held until the
 * process ends.  No allocation happens in this call.  A plan whose workspace
 * (sa_hybrid_attn_workspace_size) exceeds that size is rejected with
 * SA_ERR_CAPACITY before anything is enqueued.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams,
 * other threads) race; serialise them.  The device that runs the call is the
 * calling thread's current device, which must be the device of `stream`. */
#define SA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
sa_status sa_hybrid_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, const sa_batch_dev* b,
                                 float softmax_scale, void* out, void* stream);

/* ======================================================================
 * Token-batch linear layer ([S1] 端到端文字序列 step ④: each layer runs the
 * hybrid batch through linear-layer GEMMs beside the attention kernel;
 * 两阶段天然不对称: they take most of the time of prefill and decode; 3 ·
 * token 预算的三个约束: the batch's token count meets the GPU's tile
 * quantisation).  y = x w^T:
 *   x: device bf16 [M][K] row-major, M >= 0 token rows (M = B for a hybrid
 *      batch);
 *   w: device bf16 [N][K] row-major, one output feature per row;
 *   y: device bf16 [M][N] row-major, written (no accumulation into it).
 * K must be a multiple of 64 and N of 8 (SA_ERR_UNSUPPORTED otherwise);
 * x, w, y 16-byte aligned.  Accumulation is fp32 on the matrix cores; y is
 * rounded to bf16 (nearest-even).  The result does not depend on the
 * launch's timing: for given M, N, K it is the same bits on every call.
 * workspace: device memory of at least sa_linear_workspace_size bytes
 * (16-byte aligned; 0 bytes when no split is needed): fp32 partial products
 * when the K range of a tile is split over several workgroups.  It needs no
 * initialisation and is dead after the call; calls sharing a workspace must
 * not overlap in time.  One GEMM launch, plus one launch that adds the
 * partials when K is split; M = 0 is a no-op.
 * ==================================================================== */
sa_status sa_linear_workspace_size(int32_t M, int32_t N, int32_t K, size_t* bytes);
sa_status sa_linear(const void* x, const void* w, void* y, int32_t M, int32_t N, int32_t K, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SARATHI_ATTN_H */
