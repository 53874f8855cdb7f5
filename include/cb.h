/*
 * cb.h -- C ABI of libcb.so: one chunked-prefill mixed step on an AMD Instinct MI355X (gfx950).
 *
 * A mixed step puts every running decode (one query token each) and chunks of waiting prompts
 * (queries at absolute positions [c, c + d) of a longer prompt) into one token budget, rotates
 * queries and keys at their absolute positions, appends the new keys and values to a paged cache
 * and runs causal attention in which a chunk row at position c + i sees keys 0..c + i.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Chunked Prefill: Ending the Great Stall" (manishklach.github.io), §02-§05.
 *   [P2] "Splitting Prefill From Decode Inside a Step" (mercemay.com).
 *   [P3] "Chunked Prefill 的 Token 预算" (zwjcode.cn), §02-§11.
 *   [P4] the sference.com post on prefill head-of-line blocking (by section heading).
 *
 * Conventions for every function:
 *   - The return value is a status code (CB_OK = 0, negative on error).  No C++ exception
 *     crosses this boundary.  cb_status_string() names a code.
 *   - The library owns only cb_sched objects.  The caller owns every other buffer: host step
 *     buffers, device activations, the paged K/V caches, the rotary table and the workspace.
 *   - Device functions take a HIP stream as `void* stream` (a hipStream_t; NULL = the default
 *     stream), enqueue their kernels on it and return without synchronising.  They allocate no
 *     memory.  Argument checks that can be done on the host fail with CB_ERR_INVALID before any
 *     launch; a failed launch returns CB_ERR_HIP.  Device pointers are plain addresses in the
 *     current HIP device's memory.
 *   - Element type codes: CB_F32 (float32) or CB_BF16 (bfloat16).  q, k, v, caches and out share
 *     one type.  Index arrays are int32.  All 2-D and 3-D arrays are dense row-major.
 */
#ifndef CB_H
#define CB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CB_OK = 0,
  CB_ERR_INVALID = -1,            /* bad argument or unsupported shape                         */
  CB_ERR_DECODE_OVER_BUDGET = -2, /* more running decodes than the token budget                */
  CB_ERR_OUT_OF_BLOCKS = -3,      /* the block pool cannot cover a request                     */
  CB_ERR_CAPACITY = -4,           /* a caller-provided buffer is too small                     */
  CB_ERR_HIP = -5                 /* a HIP runtime call or kernel launch failed                */
};

enum { CB_F32 = 0, CB_BF16 = 1 };

/* Static string naming a status code; never NULL. */
const char* cb_status_string(int status);

/* ---------------------------------------------------------------------------------------------
 * Host batch builder.  [P1] §03-§04: every running decode is placed first at one token each, then
 * waiting prompts are walked first-come-first-served and each takes the largest chunk that fits
 * the rest of the budget; a prompt whose last chunk ran decodes from the next step.  [P3] §04:
 * decode tokens plus chunk tokens never exceed the budget; §05: more decodes than the budget is an
 * error; §08: the plan and the request progress commit together; §11 and [P2] "The arithmetic of
 * chunk boundaries": the cache blocks of a whole prompt are reserved before its first chunk.
 *
 * Readings where the pages are silent: a decode with context L has L tokens cached, its query is
 * at position L and its emitted context length is L + 1; blocks leave the front of the free list
 * in order; a prompt reserves ceil(prompt_len / block_size) blocks (its cached prefix's blocks
 * included) when it first gets tokens, and when the head of the queue cannot be reserved the walk
 * stops there; a decode that needs a block when none is free fails with CB_ERR_OUT_OF_BLOCKS (no
 * preemption).  Request ids are assigned 0, 1, 2, ... in the order requests are added.
 * A cb_sched is not thread-safe; distinct objects are independent.
 *
 * Optional caps and priority policies (cb_sched_config; all off by default, and then the plan is
 * the decode-first one above):
 *   max_chunk            per-request cap on a step's take: [P2] "Chunked prefill as a rate
 *                        control"; also [P4]'s shipped long-prefill threshold, which is the same
 *                        ceiling ("The fix").
 *   prefill_floor        [P4]'s proposed floor (closing section).  Reading: a first FCFS pass
 *                        grants each admitted prompt min(remaining, floor, budget left); the budget
 *                        still left is then shared evenly among the admitted prompts that have
 *                        tokens to go (each bounded by its remaining tokens and max_chunk), an
 *                        indivisible rest going one token each in FCFS order.
 *   max_partial_prefills [P3] §10.  Reading: a prompt whose first-pass grant leaves it unfinished
 *                        is admitted only while fewer than this many admitted prompts stay
 *                        unfinished; otherwise it is skipped this step (prompts behind it that
 *                        finish within the step may still be admitted).
 *   max_num_seqs         [P3] §10: sequences per step; the prompt walk stops at the cap.
 *   policy               [P2] "Choosing the priority order": CB_POLICY_DECODE_FIRST, CB_POLICY_
 *                        PREFILL_FIRST (the prompt walk gets the whole budget, decodes run in what
 *                        is left), CB_POLICY_FAIR_SHARE (decodes get up to decode_share_pct of the
 *                        budget, prompts the rest; a class's unused share goes to the other).
 *   prefill_quota_pct    [P3] §08 and §16: under decode-first, while prompts wait, decodes use at
 *                        most the budget minus ceil(pct * budget / 100).
 * Under prefill-first, fair share, a quota, or a sequence cap with one of these, a decode that does
 * not fit waits for a later step instead of failing: the decodes that have waited longest run
 * first (running order breaks ties) and are emitted in running order; a decode deferred still
 * holds its blocks.  Under plain decode-first, more decodes than the budget or max_num_seqs fail
 * with CB_ERR_DECODE_OVER_BUDGET. 
 * ------------------------------------------------------------------------------------------- */
typedef struct cb_sched cb_sched;

typedef struct {
  int32_t block_size;        /* tokens per KV block, >= 1                                      */
  int32_t num_blocks;        /* physical blocks in the pool, >= 0                              */
  const int32_t* free_list;  /* optional allocation order (a permutation of 0..num_blocks-1,
                                copied at create); NULL = 0, 1, ..., num_blocks - 1            */
  int32_t max_chunk;         /* 0 = no per-prompt cap (default); > 0 caps every chunk
                                ([P2] "Chunked prefill as a rate control")                     */
  int32_t prefill_floor;     /* 0 = off; > 0: the floor described above                        */
  int32_t max_partial_prefills; /* 0 = no cap                                                  */
  int32_t max_num_seqs;      /* 0 = no cap                                                     */
  int32_t policy;            /* CB_POLICY_*; 0 = decode-first                                  */
  int32_t decode_share_pct;  /* fair share: decodes' share of the budget, 1..99; 0 = 50        */
  int32_t prefill_quota_pct; /* 0..100; 0 = off                                                */
} cb_sched_config;

enum { CB_POLICY_DECODE_FIRST = 0, CB_POLICY_PREFILL_FIRST = 1, CB_POLICY_FAIR_SHARE = 2 };

/* Create a builder; *out receives it.  CB_ERR_INVALID on bad geometry or free list. */
int cb_sched_create(const cb_sched_config* cfg, cb_sched** out);
/* Free a builder (NULL is ignored). */
void cb_sched_destroy(cb_sched* s);
/* Deep copy (for replaying a step).  The copy is independent of the original. */
int cb_sched_clone(const cb_sched* s, cb_sched** out);

/* Set-up: a request already decoding with context_len >= 1 tokens cached.  Takes
 * ceil(context_len / block_size) blocks now (CB_ERR_OUT_OF_BLOCKS if the pool is short). */
int cb_sched_add_running(cb_sched* s, int32_t context_len, int32_t* req_id);
/* Set-up: a prompt of prompt_len >= 1 tokens whose first cached_len (0 <= cached_len <
 * prompt_len) are already cached; joins the end of the FCFS queue.  Takes the cached prefix's
 * ceil(cached_len / block_size) blocks now.  [P1] §05: with a cached prefix only the rest of the
 * prompt is computed, and the builder tracks cached length and chunk offset per request. */
int cb_sched_add_prompt(cb_sched* s, int32_t prompt_len, int32_t cached_len, int32_t* req_id);
/* Copy the physical block list of a request into out[0..cap); *n receives its length.
 * CB_ERR_CAPACITY if cap is too small (then *n still holds the length). */
int cb_sched_get_blocks(const cb_sched* s, int32_t req_id, int32_t* out, int32_t cap, int32_t* n);
/* *n = number of prompts that still have tokens to compute. */
int cb_sched_pending_prompts(const cb_sched* s, int32_t* n);
/* *n = blocks left in the free pool. */
int cb_sched_free_blocks(const cb_sched* s, int32_t* n);
/* Retire a request that has produced its last token: a running decode, or a prompt whose last
 * chunk has run.  Its blocks are appended, in its block order, to the back of the free list.
 * CB_ERR_INVALID for an unknown id or a prompt with tokens still to compute.  (The pages' decodes
 * end when their output is complete; this call is how a caller, e.g. a step simulator, says so.) */
int cb_sched_finish(cb_sched* s, int32_t req_id);

/* One step's metadata.  The caller sets the capacities and the seven array pointers (host
 * memory; pinned memory lets the copy to the device run asynchronously); the library fills the
 * arrays and the scalars.  Rows are ordered decodes first (running order), then chunks (FCFS).
 * [P3] §06: each row carries its absolute position and its physical KV slot; each sequence its
 * context length after the round and a block table of ceil(context / block_size) entries. */
typedef struct {
  int32_t cap_seqs, cap_tokens, cap_blocks;  /* in: capacities of the arrays below              */
  int32_t* seq_ids;        /* [num_seqs]     request id of each sequence                        */
  int32_t* cu_seqlens_q;   /* [num_seqs + 1] query-row offsets; cu[0] = 0, cu[num_seqs] = T     */
  int32_t* context_lens;   /* [num_seqs]     keys visible to the sequence's last row           */
  int32_t* cu_blocks;      /* [num_seqs + 1] offsets into block_table                          */
  int32_t* block_table;    /* [num_blocks_emitted] ceil(context_len / block_size) per sequence  */
  int32_t* positions;      /* [T] absolute position of each row, never restarted at a chunk     */
  int32_t* slot_mapping;   /* [T] block * block_size + position % block_size                    */
  int32_t num_seqs, num_decodes, num_tokens, num_prefill_tokens, unused_tokens;
  int32_t max_q_len, max_context_len, max_decode_context_len, num_blocks_emitted;
} cb_step;

/* Plan and commit one step under token_budget >= 1.  On any error the builder is unchanged:
 * CB_ERR_DECODE_OVER_BUDGET, CB_ERR_OUT_OF_BLOCKS, CB_ERR_CAPACITY (an array too small; the
 * needed sizes are then stored in cap_seqs / cap_tokens / cap_blocks), CB_ERR_INVALID. */
int cb_build_step(cb_sched* s, int32_t token_budget, cb_step* out);

/* Step metadata to the device (device work on the stream).  [P3] §06: the round's rows and
 * sequences carry these arrays; the builder writes them into host memory once per step.  Copies
 * nbytes from src, pinned host memory (hipHostMalloc, e.g. a pinned torch tensor), to dst, device
 * memory, with a kernel on the stream -- no copy engine, so the consumers on the same stream need
 * no cross-queue wait.  The kernel reads src with system-scope loads (no GPU caching), so src may
 * be rewritten once the copy has completed (e.g. after an event recorded behind it).  src, dst
 * and nbytes must be multiples of 8; CB_ERR_INVALID when they are not or when src is not pinned
 * host memory; CB_ERR_HIP when the launch fails. */
int cb_copy_host_to_device(void* stream, const void* src, void* dst, size_t nbytes);

/* ---------------------------------------------------------------------------------------------
 * Linear layers (device).  [P1] §02: selective batching runs the linear layers of an iteration
 * over all its tokens, decode and prefill alike; [P1]'s piggyback roofline and [P2] "Two kernels
 * with different limiting resources": one step reads the weights once, so T tokens perform about
 * T FLOP per bf16 weight byte.  y[m, n] = sum_k x[m, k] * w[n, k]: x [M, K] (the step's token rows,
 * e.g. hidden states before the QKV projection or attention outputs before the output
 * projection), w [N, K] (out_features x in_features), y [M, N]; row-major bfloat16 device
 * memory, float32 accumulation, one rounding to bfloat16 per output.  dtype must be CB_BF16;
 * M >= 0 (0 = nothing to do), N a multiple of 128, K a multiple of 64 and at most 2^22; x, w and y
 * 16-byte aligned and y not overlapping x or w.  A shape with few output tiles and no tile width
 * that covers a wide layer's few rows (M <= 64) over all of K splits K over several workgroups:
 * their float32 partials go to the caller's device workspace (16-byte aligned, at least
 * cb_linear_workspace_bytes(M, N, K) bytes; NULL when that is 0) and are summed in a fixed order,
 * so results are bitwise reproducible and depend on the shape only.  Asynchronous on the stream;
 * CB_ERR_INVALID on a bad argument, CB_ERR_CAPACITY when the workspace is too small, CB_ERR_HIP
 * when a launch fails. */
size_t cb_linear_workspace_bytes(int32_t M, int32_t N, int32_t K);
int cb_linear(void* stream, int32_t dtype, int32_t M, int32_t N, int32_t K, const void* x,
              const void* w, void* y, void* workspace, size_t workspace_bytes);

/* ---------------------------------------------------------------------------------------------
 * Rotary table (host).  [P3] §07: the rotary phase follows the absolute position, so a chunk's
 * rows must not restart at 0.  The variant is this library's reading (the pages fix none):
 * rotate-half over the full head dimension, theta_i = base^(-2i/D) in double precision,
 * out[p * D + i] = (float)cos(p * theta_i) and out[p * D + D/2 + i] = (float)sin(p * theta_i)
 * for 0 <= i < D/2, the angle p * theta_i a double product and cos/sin evaluated in x87 extended
 * precision (long double with a 64-bit significand) before one rounding to float.  out holds
 * max_pos * D floats (host memory).  D must be even.  CB_ERR_INVALID on a host whose long double
 * is another type (the table's bits would differ).
 * ------------------------------------------------------------------------------------------- */
int cb_rope_cos_sin(float* out, int32_t max_pos, int32_t D, double base);

/* ---------------------------------------------------------------------------------------------
 * Rotary embedding + paged KV append (device).  [P3] §06: each new key/value lands in the slot
 * slot_mapping[t] of the paged cache; §07: rotation at positions[t]; [P1] §05: paged blocks are
 * filled token by token whatever chunk wrote them.
 *
 * For every row t < T with 0 <= positions[t] < max_pos (other rows are skipped entirely):
 *   q_out[t, h, :] = rot(q[t, h, :], positions[t])   for h < Hq       (only if q != NULL)
 *   if 0 <= slot_mapping[t] < num_blocks * block_size, with b = slot / block_size and
 *   o = slot % block_size:
 *     k_cache[b, g, o, :] = rot(k[t, g, :], positions[t]),  v_cache[b, g, o, :] = v[t, g, :]
 * where rot pairs element i with i + D/2:  x_i c - x_{i+D/2} s  and  x_{i+D/2} c + x_i s, each
 * product and sum rounded to float32 separately (no fused multiply-add), c = cos_sin[p, i],
 * s = cos_sin[p, D/2 + i], then rounded to nearest-even into the element type.
 *
 * Layouts (device): q, q_out [T, Hq, D]; k, v [T, Hkv, D]; positions, slot_mapping [T];
 * cos_sin [max_pos, D] float32; k_cache, v_cache [num_blocks, Hkv, block_size, D].
 * q_out may equal q (in place); otherwise they must not overlap.  D in {64, 128}.
 * ------------------------------------------------------------------------------------------- */
int cb_rope_kv_append(void* stream, int32_t dtype, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                      int32_t block_size, const void* q, const void* k, const void* v,
                      const int32_t* positions, const int32_t* slot_mapping,
                      const float* cos_sin, int32_t max_pos, void* q_out, void* k_cache,
                      void* v_cache, int64_t num_blocks);

/* ---------------------------------------------------------------------------------------------
 * Mixed paged attention over a step's varlen batch (device).  [P3] §02 and §07: a row of a chunk
 * that starts at offset c, at position c + i, attends keys {0, ..., c + i} -- the cached prefix
 * plus its own chunk up to itself; [P1] §05: the chunk's attention is ordinary causal attention
 * over the prefix and the chunk, and the attention matrix is never materialised; [P1] §01 and
 * [P2] "Two kernels with different limiting resources": decode rows stream the whole cache
 * (bandwidth-bound) while chunk rows are dense matrix work (compute-bound).
 *
 * Sequences 0..num_decodes-1 are decode rows (one query each; sequence s owns row s); sequences
 * num_decodes..num_seqs-1 are chunks.  For sequence s with rows [cu_seqlens_q[s],
 * cu_seqlens_q[s+1]) of length d and ctx = context_lens[s], row i sits at position ctx - d + i and
 * for each query head h, with g = h / (Hq / Hkv):
 *     out[row, h, :] = sum_{j <= ctx-d+i} softmax_j(scale * q[row, h, :] . K_j,g) V_j,g
 * where key j of the sequence is k_cache[block_table[cu_blocks[s] + j / bs], g, j % bs, :].
 * q must already be rotated (cb_rope_kv_append's q_out) and the step's own keys appended.
 * Arithmetic: products on the matrix cores from the element type, float32 accumulation and
 * softmax; out is rounded to the element type.
 *
 * Host scalars (from cb_build_step, so no device-to-host read is needed): T = total rows,
 * max_q_len = longest sequence in rows, max_decode_ctx = largest context_lens[s] over decodes
 * (0 if none), max_ctx = largest over all sequences.  These size the grids; device values
 * beyond them are not processed.  Requirements: Hq % Hkv == 0, D in {64, 128},
 * block_size in {8, 16, 32, 64, 128, 256}.
 *
 * workspace: device memory of at least cb_attn_workspace_bytes(...) bytes for the same
 * arguments (float32 partial results of split-context work and the decode work split),
 * 256-byte aligned; CB_ERR_CAPACITY if workspace_bytes is smaller.  Calls that share a
 * workspace must not overlap in time.  Its size does not grow with decode context lengths.
 * Execution: up to three kernels in order on the stream: the decode work split (one
 * workgroup, only with decode rows and no host-made plan, see cb_decode_plan in cb_ext.h), the attention
 * kernel (decode waves and chunk tiles in one launch) and the combine (only when some row's work
 * was split).
 * Layouts (device): q, out [T, Hq, D]; caches as above; cu_seqlens_q, cu_blocks [num_seqs + 1];
 * context_lens [num_seqs]; block_table [cu_blocks[num_seqs]].  out must not overlap q.
 * ------------------------------------------------------------------------------------------- */
size_t cb_attn_workspace_bytes(int32_t num_seqs, int32_t num_decodes, int32_t T,
                               int32_t max_q_len, int32_t max_decode_ctx, int32_t max_ctx,
                               int32_t Hq, int32_t Hkv, int32_t D);

int cb_mixed_paged_attention(void* stream, int32_t dtype, int32_t num_seqs, int32_t num_decodes,
                             int32_t T, int32_t max_q_len, int32_t max_decode_ctx,
                             int32_t max_ctx, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t block_size, float scale, const void* q,
                             const void* k_cache, const void* v_cache,
                             const int32_t* cu_seqlens_q, const int32_t* context_lens,
                             const int32_t* cu_blocks, const int32_t* block_table, void* out,
                             void* workspace, size_t workspace_bytes);

/* cb_mixed_paged_attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments and result,
 * without a workspace argument.  The workspace is a device array inside the library of
 * CB_ATTN_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held until the process ends; calls whose
 * cb_attn_workspace_bytes(...) exceeds it return CB_ERR_CAPACITY (every workload here needs at
 * most ~44 MiB).  The call allocates nothing and makes no allocating library call; the first call
 * on a device looks the array's address up once (hipGetSymbolAddress, with that device made
 * current for the lookup).  Every call on one GPU shares the array: calls that overlap in time on
 * the same GPU (different streams, or other host threads) race and must be serialised by the
 * caller.  Errors: CB_ERR_INVALID on bad shapes or pointers (as cb_mixed_paged_attention),
 * CB_ERR_CAPACITY as above, CB_ERR_HIP if the address lookup or a launch fails. */
#define CB_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int cb_mixed_paged_attention_noalloc(void* stream, int32_t dtype, int32_t num_seqs,
                                     int32_t num_decodes, int32_t T, int32_t max_q_len,
                                     int32_t max_decode_ctx, int32_t max_ctx, int32_t Hq,
                                     int32_t Hkv, int32_t D, int32_t block_size, float scale,
                                     const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                     const int32_t* cu_blocks, const int32_t* block_table,
                                     void* out);

#ifdef __cplusplus
}
#endif
#endif /* CB_H */
