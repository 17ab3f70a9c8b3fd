/*
 * cb.h - C ABI of libcb.so: one forward step of ragged continuous-batching attention on
 * one AMD Instinct MI355X (gfx950).
 *
 * The operation (Hugging Face blog "Continuous batching from first principles", sections
 * "Attention", "KV-cache", "Chunked prefill" and "Continuous batching"; zhangchitc
 * "continuous-batching", sections "Ragged batching: attention in per-request blocks" and
 * "Inside the kernel: cu_seqlens splits six rows back into three"):
 *
 *   All scheduled requests are packed into one token stream with no batch axis and no
 *   padding. Request r owns packed rows cu_q_lens[r] .. cu_q_lens[r+1]-1. A decode request
 *   contributes one row and a prefill chunk contributes q_r rows. Request r has ctx_lens[r]
 *   tokens cached before the step. Its new tokens sit at positions ctx_lens[r] + i.
 *   Each query row at position p of request r attends to keys 0..p of request r only. The
 *   mask is block-diagonal over requests and causal within a request:
 *       O[t,h,:] = softmax_j( scale * Q[t,h,:] . K_r[j,g,:] ) V_r[j,g,:],   j = 0..p,
 *   with g = h / (Hq / Hkv). K_r and V_r are the request's keys and values: its cache
 *   followed by this step's new tokens, which cb_kv_append writes into the cache first.
 *
 * Conventions for every call:
 *   - Pointers are either device pointers (HBM, from hipMalloc or torch) or host pointers.
 *     Each argument below says which. The library never frees or takes ownership of caller
 *     memory and never allocates caller-visible device memory.
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the
 *     default stream). Inputs must stay valid until the work on the stream completes.
 *   - The return value is 0 (CB_OK) or a negative cb_status. On error nothing has been
 *     launched. cb_last_error() returns a message for the calling thread.
 *   - Integer metadata is int32. Float tensors are dense and row-major in the dtype of
 *     cb_shape.dtype (bf16 or fp32).
 */
#ifndef CB_H
#define CB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CB_OK = 0,
  CB_ERR_INVALID_ARG = -1,        /* malformed shape, metadata or pointer */
  CB_ERR_UNSUPPORTED = -2,        /* valid but not implemented (head_dim, group size...) */
  CB_ERR_HIP = -3,                /* a HIP runtime call failed */
  CB_ERR_OUT_OF_BLOCKS = -4,      /* the scheduler's free list cannot cover the step */
  CB_ERR_WORKSPACE_TOO_SMALL = -5,
  CB_ERR_STATE = -6               /* call out of order (e.g. build twice without commit) */
} cb_status;

typedef enum { CB_F32 = 0, CB_BF16 = 1 } cb_dtype;

/* Model-side sizes.
 * num_q_heads % num_kv_heads == 0; head_dim in {64, 128}; block_size == 16.
 * Hq / Hkv (the query group size G) must be 1, 2, 4, 8 or a multiple of 8.
 * Paged KV cache, num_blocks physical blocks; for block b and kv head g:
 *   k_cache[b][g][s][d]  : [num_blocks, Hkv, block_size, head_dim]   (slot-major, as K rows)
 *   v_cache[b][g][d][s]  : [num_blocks, Hkv, head_dim, block_size]   (V stored transposed)
 * Both are contiguous, and each (b, g) page is block_size*head_dim elements. Position p of
 * a request lives in block block_tables[r][p / block_size], slot p % block_size. */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t dtype;                  /* cb_dtype */
} cb_shape;

/* One ragged step (zhangchitc, "Inside the kernel": cu_seqlens is the prefix sum of the
 * per-request row counts, e.g. lengths [4,1,1] give [0,4,5,6]).
 *   cu_q_lens    device int32 [num_reqs+1], nondecreasing, cu[0]=0, cu[R]=num_tokens
 *   ctx_lens     device int32 [num_reqs], tokens cached before this step (>= 0)
 *   block_tables device int32 [num_reqs * max_blocks_per_req], row r lists the physical
 *                blocks of request r in position order; entries past
 *                ceil((ctx+q)/block_size) are ignored (-1 by convention)
 *   h_cu_q_lens, h_ctx_lens  host copies of the two arrays above (same values). They are
 *                used to validate and to plan the launch without a device sync.
 * A request with zero rows is allowed and produces nothing. */
typedef struct {
  int32_t num_reqs;
  int32_t num_tokens;
  int32_t max_blocks_per_req;
  const int32_t* cu_q_lens;
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  const int32_t* h_cu_q_lens;
  const int32_t* h_ctx_lens;
} cb_batch;

/* ---------------------------------------------------------------------------------------
 * KV append (zhangchitc "continuous-batching", section "Inside the kernel": a step's new
 * keys and values go into the cache slots of the request they belong to, and attention
 * then reads them back from there).
 *   k_new, v_new  device [num_tokens, Hkv, head_dim], packed like Q
 *   k_cache, v_cache  device, layout in cb_shape; updated in place
 * Row t of request r (position p = ctx_lens[r] + t - cu_q_lens[r]) is copied bit for bit
 * to k_cache[bt[r][p/bs]][g][p%bs][:] and v_cache[bt[r][p/bs]][g][:][p%bs].
 * Block ids outside [0, num_blocks) are skipped on the device (no write).
 * ------------------------------------------------------------------------------------- */
int cb_kv_append(const cb_shape* shape, const cb_batch* batch, const void* k_new,
                 const void* v_new, void* k_cache, void* v_cache, void* stream);

/* ---------------------------------------------------------------------------------------
 * Ragged attention (the operation at the top of this file).
 *   q        device [num_tokens, Hq, head_dim]
 *   k_cache, v_cache  device caches, already holding this step's keys/values
 *   scale    multiplies Q.K before the softmax (the pages show none; 1/sqrt(D) is usual);
 *            must be positive and finite
 *   o        device [num_tokens, Hq, head_dim], written in full (dtype of the shape)
 *   workspace  device scratch of at least cb_ragged_attention_workspace_size() bytes,
 *            256-byte aligned, owned by the caller. It must not be shared by two calls in
 *            flight at the same time.
 * Rows of a request with one row (decode) take a split-K bandwidth path. Rows of a request
 * with more than one row (prefill chunk) take an MFMA tile path (bf16) or the split-K path
 * (fp32). Block ids in the tables are not range-checked on the device beyond skipping ids
 * outside [0, num_blocks); stale or wrong tables give wrong results, never a fault.
 * ------------------------------------------------------------------------------------- */
size_t cb_ragged_attention_workspace_size(const cb_shape* shape, const cb_batch* batch);

/* What cb_ragged_attention would launch for `batch` (host-side planning only: reads the
 * host mirrors h_cu_q_lens and h_ctx_lens, touches no device memory, needs no GPU). For
 * tests and tools that check the planner's choices; the fields are counts of the launch
 * lists, with the tuning knobs in effect at the call. */
typedef struct {
  int32_t prefill_rows;          /* query rows per prefill work-group (32 per wave / heads), 0: none */
  int32_t prefill_items;         /* prefill work-groups, empty launch-order slots included */
  int32_t prefill_split_items;   /* of those, items covering one key range of a split tile */
  int32_t decode_splits;         /* row splits of the split-K path (decode rows; fp32 prefill rows) */
  int32_t decode_items;          /* decode waves: splits x kv heads x query-head groups */
  int32_t split_blocks;          /* split length the sizing chose (KV blocks) */
  int32_t split_min_blocks;      /* shortest and longest split, in blocks (0 if none) */
  int32_t split_max_blocks;
  int32_t longest_first;         /* 1: splits are listed in non-increasing length */
  int32_t matrix_core_decode;    /* 1: the split-K rows run on the matrix-core kernel */
  int32_t combine_rows;          /* rows merged by the combine pass */
  int32_t mixed;                 /* 1: prefill tiles and decode waves share one launch */
  int32_t prefill_heads;         /* query heads per prefill work-group (of one kv head), 0: none */
} cb_plan_info;
/* Returns CB_OK, or the error cb_ragged_attention would return for the shape and batch. */
int cb_plan_describe(const cb_shape* shape, const cb_batch* batch, cb_plan_info* out);

int cb_ragged_attention(const cb_shape* shape, const cb_batch* batch, const void* q,
                        const void* k_cache, const void* v_cache, float scale, void* o,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Ragged attention that allocates nothing, for callers that cannot allocate memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks and results as cb_ragged_attention (bit for bit), without the
 * workspace: the launch plan and the fp32 split-K partials live in a fixed device array of
 * CB_NOALLOC_SCRATCH_BYTES that the library keeps on every GPU it runs on until the process
 * ends (each GPU holds its own copy). The plan is copied into the array on `stream` from
 * ordinary host memory. The call allocates no device memory and no pinned host memory and
 * frees nothing (its host-side planning uses the C++ heap).
 * A batch whose workspace (cb_ragged_attention_workspace_size) is larger than the array is
 * rejected with CB_ERR_WORKSPACE_TOO_SMALL before anything is copied or launched. Nothing in
 * the array needs to start at zero: each partial is written before the combine pass reads
 * it, and a call keeps whatever the previous call left there.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time on one GPU (on
 * different streams, or on different threads without ordering between them) race and give
 * wrong results. Calls on one stream are ordered. The "overlap_prefill" knob does not apply
 * here (prefill tiles run on `stream`).
 * ------------------------------------------------------------------------------------- */
#define CB_NOALLOC_SCRATCH_BYTES (32u << 20)
int cb_ragged_attention_noalloc(const cb_shape* shape, const cb_batch* batch, const void* q,
                                const void* k_cache, const void* v_cache, float scale, void* o,
                                void* stream);

/* ---------------------------------------------------------------------------------------
 * One whole step from host metadata: KV append then ragged attention, with the metadata and
 * the launch plan sent to the device in a single copy. This is the same work as uploading
 * cu_q_lens / ctx_lens / block_tables, calling cb_kv_append and then cb_ragged_attention,
 * with fewer device operations per step.
 *   h_cu_q_lens [num_reqs+1], h_ctx_lens [num_reqs], h_block_tables [num_reqs *
 *       max_blocks_per_req]  host int32, as in cb_batch and cb_step (the step builder's
 *       arrays can be passed as they are). Every block id a row of the step touches must
 *       lie in [0, num_blocks); this is checked on the host (CB_ERR_INVALID_ARG).
 *   q, k_new, v_new, k_cache, v_cache, scale, o: as in cb_kv_append / cb_ragged_attention.
 *   workspace: device, 256-byte aligned, at least cb_step_workspace_size() bytes; it holds
 *       the step's metadata, plan and partials and must not be shared by calls in flight.
 * In a step of decode rows only, a block that receives exactly one row (see cb_step_slots)
 * has its whole V page rewritten, its other positions with the bits they already hold:
 * nothing else may write that block while the step runs (as for every block of a request
 * in the step).
 * ------------------------------------------------------------------------------------- */
size_t cb_step_workspace_size(const cb_shape* shape, int32_t num_reqs, int32_t num_tokens,
                              int32_t max_blocks_per_req, const int32_t* h_cu_q_lens,
                              const int32_t* h_ctx_lens);

int cb_step_forward(const cb_shape* shape, int32_t num_reqs, int32_t num_tokens,
                    int32_t max_blocks_per_req, const int32_t* h_cu_q_lens,
                    const int32_t* h_ctx_lens, const int32_t* h_block_tables, const void* q,
                    const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    float scale, void* o, void* workspace, size_t workspace_bytes, void* stream);

/* The cache slot of every packed row as cb_step_forward stages it for its KV append (host
 * only: no device memory, no GPU; for tests and tools). The slot rule is cb_kv_append's: row
 * i of request r, at position p = h_ctx_lens[r] + i, goes to slot
 * block_tables[r][p / block_size] * block_size + p % block_size.
 *   out_slots  host int32 [num_tokens], written in full.
 In a step of decode rows only (every request has at most one row) and when
 * num_blocks * block_size <= 2^30, a row that is the only row of the step writing into its
 * block (every row, unless two requests share a block) also carries bit 30
 * (CB_SLOT_SOLE_WRITER). For such rows cb_step_forward (with the default "stage_kernel") and
 * cb_graph_step rewrite the block's whole transposed V page, the other positions with the
 * bits they hold, so that the append writes whole cache lines. Steps with prefill rows and
 * the copy-engine upload stage slots without the bit and write one element per d-row.
 * Returns CB_OK; the argument errors of cb_step_forward's host checks (CB_ERR_INVALID_ARG,
 * out-of-range block ids included); CB_ERR_UNSUPPORTED for pools beyond 2^31 / block_size
 * blocks, whose steps look slots up on the device instead. */
#define CB_SLOT_SOLE_WRITER (1 << 30)
int cb_step_slots(const cb_shape* shape, int32_t num_reqs, int32_t num_tokens, int32_t max_blocks_per_req,
                  const int32_t* h_cu_q_lens, const int32_t* h_ctx_lens, const int32_t* h_block_tables,
                  int32_t* out_slots);

/* ---------------------------------------------------------------------------------------
 * Captured steps (HIP graphs). Hugging Face blog "Continuous batching from first
 * principles", section "Continuous batching": graph capture needs static tensor shapes,
 * which a batch axis meets only by padding every prompt to one length. A cb_graph is the
 * whole step of cb_step_forward (metadata copy, KV append, prefill tiles, split-K decode,
 * combine) captured once and replayed for every later step whose packed rows fit its
 * capacity (max_tokens: the caller's bucket of T). Its shapes are static capacities, not
 * padding: the live sizes and work lists travel in a header that the replayed copy moves to
 * the device, and work-groups past the live counts exit at once.
 *
 * cb_graph_create: binds the graph to fixed buffers (device pointers, 16-byte aligned):
 *   q [max_tokens, Hq, D], k_new / v_new [max_tokens, Hkv, D], o [max_tokens, Hq, D]
 *   and the caches, as in cb_step_forward. A step uses their first num_tokens rows. The
 *   caller owns them and keeps them alive until cb_graph_destroy. The graph owns a device
 *   workspace and two pinned staging buffers, sized at the first step and grown (with a
 *   new capture) when a later step needs more. Captures on the current device; later
 *   calls must run with the same device current. Returns CB_OK and *out, or an error
 *   (nothing created).
 * cb_graph_step: one step from host metadata, exactly as cb_step_forward takes it (the
 *   same checks, CB_ERR_INVALID_ARG for num_tokens > max_tokens). Writes the header,
 *   metadata and plan into a staging buffer, then launches the graph on `stream`. The two
 *   staging buffers alternate; a call waits (host side) for the replay two steps back
 *   before it reuses its buffer, so the host may build step n+1 while step n runs. Steps of
 *   one graph must be ordered on one stream; graphs must not be shared between threads
 *   without a lock. Results are bit-identical to cb_step_forward's on the same inputs.
 * cb_graph_stats: replays launched, captures made (the first, then one each time a step
 *   outgrows the capacities, which then at least double) and the workspace size in bytes;
 *   any pointer may be NULL.
 * cb_graph_destroy: waits for replays in flight and frees the graph (NULL is a no-op).
 * ------------------------------------------------------------------------------------- */
typedef struct cb_graph cb_graph;

int cb_graph_create(const cb_shape* shape, int32_t max_tokens, const void* q, const void* k_new,
                    const void* v_new, void* k_cache, void* v_cache, float scale, void* o,
                    cb_graph** out);
int cb_graph_step(cb_graph* graph, int32_t num_reqs, int32_t num_tokens, int32_t max_blocks_per_req,
                  const int32_t* h_cu_q_lens, const int32_t* h_ctx_lens,
                  const int32_t* h_block_tables, void* stream);
int cb_graph_stats(const cb_graph* graph, int64_t* replays, int64_t* captures,
                   size_t* workspace_bytes);
void cb_graph_destroy(cb_graph* graph);

/* ---------------------------------------------------------------------------------------
 * Token-wise layers around attention (Hugging Face blog, section "Attention": normalisation
 * and matrix multiplications are token-wise, so they run on the packed stream unchanged;
 * hassanahmed, selective batching batches these shape-agnostic operations).
 *
 * cb_linear: c[M, N] = a[M, K] w[N, K]^T. All bf16, row-major, device pointers, 16-byte
 * aligned; fp32 accumulation, outputs rounded to nearest even. w is laid out like a torch
 * Linear weight ([out features, in features]). N must be a multiple of 128 and K of 64, at
 * most 1,048,576 (CB_ERR_UNSUPPORTED otherwise); M is any count of packed rows (0 is a
 * no-op). NULL or unaligned pointers: CB_ERR_INVALID_ARG. Enqueued on `stream`; nothing is
 * allocated and the caller owns every buffer.
 *
 * cb_qkv_project: the QKV projection of the packed rows with the KV append fused in
 * (zhangchitc "continuous-batching", section "Inside the kernel": the new keys and values go
 * into each request's cache entry before attention reads it). x [T, d_model] bf16, w_qkv
 * [(Hq + 2 Hkv) * D, d_model] bf16 (rows: the Hq*D query features, then Hkv*D key features,
 * then Hkv*D value features, head-major). Writes q [T, Hq, D] and, for every packed row, its
 * key and value into the cache slot given by batch (as cb_kv_append does; rows whose block
 * id is outside the pool are not written). bf16 only; d_model a multiple of 64 up to
 * 1,048,576 and Hq*D, Hkv*D multiples of 128 (CB_ERR_UNSUPPORTED otherwise). Same stream
 * semantics and metadata checks as cb_kv_append.
 * ------------------------------------------------------------------------------------- */
int cb_linear(int32_t M, int32_t N, int32_t K, const void* a, const void* w, void* c, void* stream);
int cb_qkv_project(const cb_shape* shape, const cb_batch* batch, int32_t d_model, const void* x,
                   const void* w_qkv, void* q, void* k_cache, void* v_cache, void* stream);

/* Message describing the last error on this thread ("" if none). Owned by the library. */
const char* cb_last_error(void);

/* Library version string, e.g. "cb 0.1 gfx950". */
const char* cb_version(void);

/* Device checks of the debug copy of the library (python -m ragged_continuous_batching_amd.build
 * --device-checks, loaded in place of libcb.so). The host checks a step's block ids against
 * the pool from its host mirrors before it launches anything; the kernels read the device
 * block table (and, for cb_step_forward, the staged slots). A kernel that meets a block id
 * outside the pool (a device table that disagrees with its host mirror) reads block 0 in its
 * place or skips the write, in every build, so it never faults; the debug copy also counts
 * each such meeting (once per wave or work-group that meets it).
 *   count  out: the count since the last reset, summed over every kernel (waits for the device)
 *   reset  nonzero: zero the counters after reading them
 * Returns CB_OK, or CB_ERR_UNSUPPORTED in a copy built without the checks (count is then 0).
 * Not for use while other threads launch library work. */
int cb_debug_violations(uint32_t* count, int reset);

/* Tuning knobs (process-wide, host-side, read by every later call when it plans its launches;
 * a captured cb_graph keeps the kernels it was captured with). Set them before issuing work:
 * changing a knob while another thread is inside a library call is a data race. Keys:
 *   "split_blocks"   KV blocks per split of a decode row, at most 1024; 0 = automatic
 *                    (default)
 *   "target_waves"   automatic split sizing aims for at least this many wave items; 0
 *                    (default) = 4096 for the vector-ALU decode kernel, 2048 for the
 *                    matrix-core one
 *   "overlap_prefill" 1 = run prefill tiles on an internal side stream (forked from and
 *                    joined back to `stream`) concurrently with decode rows; 0 (default)
 *                    runs them one after the other on `stream`
 *   "xcds"           number of XCDs work-groups are dispatched over round-robin (8 on
 *                    MI355X); prefill tiles that share keys are placed on one XCD
 *   "decode_mfma"    1 (default) = decode rows of bf16 models with 4 or more query heads per
 *                    kv head use the matrix-core kernel; 0 = the vector-ALU kernel
 *   "decode_group"   most query heads of one kv head that a decode wave handles (1, 2, 4
 *                    or 8; default 8). Smaller groups use fewer registers per wave; the
 *                    waves of one kv head then read the same pages back to back.
 *   "stage_kernel"   1 (default) = metadata and work lists are copied into the workspace by
 *                    a kernel that reads the pinned staging buffer (same queue as the
 *                    attention kernels); 0 = by the copy engine (hipMemcpyAsync)
 *   "prefill_waves"  waves per bf16 prefill work-group: 4 (128 query rows, two work-groups
 *                    per CU), 8 (256 rows, one per CU), or 0 (default) = 8 when a step has at
 *                    least 2 x 256 such work-groups, else 4
 *   "prefill_snake"  1 (default): within each XCD's queue of prefill work-groups, every
 *                    other round of one work-group per CU is reversed, so a CU that got a
 *                    long work-group in one round gets a short one in the next; 0: the
 *                    queues stay longest first
 *   "prefill_split"  1 (default): when a bf16 step has fewer prefill work-groups than the
 *                    GPU has work-group slots, prefill tiles with long key walks are split
 *                    over key ranges (partials merged by the combine pass); 0: never
 *   "prefill_split_tiles"  key tiles (64 keys) per split range, forcing splits in any step;
 *                    0 (default) = automatic
 *   "decode_order"   1 (default): decode splits launched longest first; 0: in the order of
 *                    their rows (longest row first)
 *   "mixed_launch"   1: a bf16 step with both prefill rows and grouped-query decode rows
 *                    (Hq/Hkv >= 4) runs its prefill tiles (128-row work-groups) and decode
 *                    waves in one launch, interleaved so that both kinds share every CU;
 *                    0: two launches. Steps taken by cb_graph_step always use two launches.
 *   "prefill_heads"  query heads of one kv head that a bf16 prefill work-group takes side
 *                    by side (1, 2, 4 or 8, capped by the group size and the waves): its
 *                    waves split into heads x 32-row blocks and share every key/value tile,
 *                    so a work-group covers 32 x waves / heads rows; 0 (default) = 4
 *   "mixed_order"    order of the mixed launch: 0 (default) spreads prefill and decode
 *                    work-groups in proportion to their counts; 1 alternates them until one
 *                    kind runs out
 * Returns CB_ERR_INVALID_ARG for an unknown key or a negative value. */
int cb_set_tuning(const char* key, int32_t value);
/* Current value of one tuning key (as stored: boolean keys read 0 or 1) into *value.
 * Returns CB_ERR_INVALID_ARG for an unknown key or a NULL value pointer. */
int cb_get_tuning(const char* key, int32_t* value);

/* ---------------------------------------------------------------------------------------
 * Kernel timing (hipEvents recorded on the stream each kernel is launched on).
 * cb_profile_enable(1) starts recording a start/stop event pair around every kernel the
 * library launches. cb_profile_read() waits for the recorded events and returns the summed
 * duration and the launch count for one kernel id. cb_profile_reset() drops all records.
 * ------------------------------------------------------------------------------------- */
enum { CB_KERNEL_APPEND = 0, CB_KERNEL_DECODE = 1, CB_KERNEL_COMBINE = 2, CB_KERNEL_PREFILL = 3,
       CB_KERNEL_GEMM = 4, CB_KERNEL_MIXED = 5, CB_KERNEL_COUNT = 6 };
int cb_profile_enable(int on);
int cb_profile_read(int kernel_id, double* total_ms, int64_t* launches);
/* Per-launch durations of one kernel id, in launch order: writes min(capacity, launches)
 * values (ms) to host array ms_out and the number of recorded launches to *launches. */
int cb_profile_launches(int kernel_id, float* ms_out, int64_t capacity, int64_t* launches);
int cb_profile_reset(void);
/* Restricts timing to the kernel ids whose bit (1 << id) is set in mask; the default, and
 * mask = 0, time every kernel. Each event pair costs the stream about a microsecond or two,
 * so a caller that times a whole step can select only the kernel it needs. */
int cb_profile_select(uint32_t mask);
const char* cb_kernel_name(int kernel_id);

/* A measurement aid, not part of a step: reads n_pages 4 KiB pages of `pages` in the order
 * `order` the way the decode kernels read the cache (non-temporal 16-byte loads of whole
 * pages; each wave requests its 16 pages before it uses the first) and does nothing with them. Timed around its launch,
 * it gives the read rate this GPU attains on the cache's access pattern; bench.py reports
 * the decode kernels against it beside the vendor figure.
 *   pages  device, n_pages * 4096 bytes, 16-byte aligned
 *   order  device int32 [n_pages], page indices (entries outside [0, n_pages) are skipped)
 *   sink   device uint32 [cb_paged_read_probe_sink_words(n_pages)], practically never written
 * Asynchronous on `stream`. Returns CB_OK, or CB_ERR_INVALID_ARG for n_pages < 1, a NULL or
 * misaligned pointer. */
int32_t cb_paged_read_probe_sink_words(int32_t n_pages);
int cb_paged_read_probe(const void* pages, int32_t n_pages, const int32_t* order, uint32_t* sink,
                        void* stream);

/* ---------------------------------------------------------------------------------------
 * Host step builder (Hugging Face blog, section "Continuous batching": aim for m tokens per
 * step, add every decoding request first with one token each, fill the rest with prefill
 * chunks, remove finished requests at once and admit waiting ones; hassanahmed "How
 * continuous batching speeds up LLM serving": evict, admit while can_admit, run one step;
 * the cache lives in fixed-size blocks handed out and reclaimed on demand).
 *
 * Host memory only; no HIP calls. Each build():
 *   1. evicts requests marked done by the previous commit, returning their blocks to the
 *      tail of the FIFO free list in block-table order;
 *   2. takes every decode-phase request (admission order, at most m), one token each,
 *      allocating a block when its position starts a new one;
 *   3. gives the remaining budget to partly prefilled requests (admission order), each
 *      taking min(remaining prompt, budget, tokens its blocks plus the free list can hold);
 *   4. admits waiting requests (FIFO) while budget > 0, the free list holds the blocks of
 *      the first chunk (min(prompt, budget) tokens), and fewer than max_num_seqs
 *      requests are running (if max_num_seqs > 0). The first request that does not fit
 *      stops admission.
 * A request is done once it has produced out_len tokens (the last prefill chunk produces
 * the first) or when commit() flags EOS for a step in which it produced a token.
 * ------------------------------------------------------------------------------------- */
typedef struct cb_sched cb_sched;

/* The arrays of one built step. They are owned by the scheduler and valid until the next
 * build/commit/destroy. block_tables is [num_reqs * max_blocks_per_req], -1 padded. */
typedef struct {
  int32_t num_reqs;
  int32_t num_tokens;
  int32_t max_blocks_per_req;
  int32_t num_decode;             /* the first num_decode requests are decodes (1 row) */
  const int64_t* req_ids;         /* [num_reqs] */
  const int32_t* cu_q_lens;       /* [num_reqs+1] */
  const int32_t* ctx_lens;        /* [num_reqs] */
  const int32_t* block_tables;    /* [num_reqs * max_blocks_per_req] */
  const int32_t* slot_mapping;    /* [num_tokens]: block*block_size + offset of each row */
  const int32_t* token_to_req;    /* [num_tokens]: index into this step's requests */
  int32_t num_evicted;
  int32_t num_admitted;
  const int64_t* evicted;         /* request ids evicted at the start of this build */
  const int64_t* admitted;        /* request ids admitted by this build */
  int32_t num_preempted;
  const int64_t* preempted;       /* request ids preempted by this build (back to waiting) */
} cb_step;

/* initial_free_list: host int32 [num_blocks], a permutation of 0..num_blocks-1 giving the
 * allocation order, or NULL for 0,1,2,... Returns NULL on invalid arguments. */
cb_sched* cb_sched_create(int32_t token_budget, int32_t block_size, int32_t num_blocks,
                          int32_t max_num_seqs, const int32_t* initial_free_list);
/* Switches the builder to naive batching, the baseline the pages contrast continuous
 * batching with (zhangchitc "continuous-batching", section "Naive batching: the whole batch
 * finishes together"; hassanahmed "How continuous batching speeds up LLM serving", the batch
 * loop that returns results when the batch finishes; batch_size 1 is request-at-a-time).
 * From then on each build():
 *   1. if every running request is done, evicts them all (blocks to the free list tail);
 *   2. with nothing running, admits up to batch_size waiting requests (FIFO) while the free
 *      list holds ceil(P / block_size) blocks for each of them, P being the longest prompt
 *      among them, and emits one prefill step of P rows per request: the prompt, then
 *      P - prompt_len pad rows (causal attention keeps pads out of the prompt's rows);
 *      commit() then sets the context to prompt_len, so the first decode row overwrites the
 *      first pad slot;
 *   3. otherwise emits one decode row for every running request, done ones included.
 * m does not apply. Call before any request runs (CB_ERR_STATE otherwise). */
int cb_sched_set_static(cb_sched* s, int32_t batch_size);
/* Preemption by recompute (hassanahmed "How continuous batching speeds up LLM serving",
 * paged-memory section: when the card fills, a request is evicted for a while and brought
 * back later). enable = 1: when the decode tokens of a build need more blocks than the free
 * list holds, the most recently admitted running request gives back all its blocks and goes
 * to the head of the waiting queue, repeatedly, until they fit. Re-admitted, it prefills all
 * prompt_len + generated tokens it has (chunked like any prompt); the last of them yields its
 * next token. watermark_blocks: admission also requires that many blocks to stay free (0 =
 * admit while the first chunk fits). Not with naive batching (CB_ERR_STATE). */
int cb_sched_set_preemption(cb_sched* s, int32_t enable, int32_t watermark_blocks);
/* A new request enters the waiting queue. prompt_len >= 1, out_len >= 1. */
int cb_sched_add(cb_sched* s, int64_t req_id, int32_t prompt_len, int32_t out_len);
/* A request that is already running with `cached` positions in the cache: either still in
 * prefill (generated == 0, cached < prompt_len) or decoding (1 <= generated < out_len and
 * cached == prompt_len + generated - 1). Allocates ceil(cached / block_size) blocks. */
int cb_sched_add_cached(cb_sched* s, int64_t req_id, int32_t prompt_len, int32_t out_len,
                        int32_t cached, int32_t generated);
int cb_sched_build(cb_sched* s, cb_step* out);
/* eos: host uint8 [num_reqs of the last step] or NULL (finish by out_len only). */
int cb_sched_commit(cb_sched* s, const uint8_t* eos);
/* Deep copy (free list, queues and requests); the copy has no step pending. */
cb_sched* cb_sched_clone(const cb_sched* s);
void cb_sched_destroy(cb_sched* s);
int cb_sched_stats(const cb_sched* s, int32_t* num_running, int32_t* num_waiting,
                   int32_t* num_free_blocks);

#ifdef __cplusplus
}
#endif

#endif /* CB_H */
