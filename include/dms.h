/*
 * dms.h - C ABI of the Dynamic Memory Sparsification (DMS) decode path on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 *   A KV cache whose tokens carry a learned, per-KV-head binary eviction
 *   decision, with the decision's effect delayed by a window of w steps, and
 *   the grouped-query decode attention that reads only the tokens still
 *   visible.  Source: "Inference-Time Hyper-Scaling with KV Cache
 *   Compression", third-party paper summary page, sections "Key claims" and
 *   "Method" (the paper's section 3.2, section 5.3 and Fig. 5): per-head
 *   decision alpha_t in {0,1}; a token marked at step t is still attended up
 *   to step t + w and dropped afterwards; the decisions act as an additive
 *   attention mask that never has to be built; the sparsified cache works
 *   with paged attention and adds no KV read/write operations (section 3.2
 *   "Performance Considerations", section 3.3).
 *
 * Readings fixed by this interface (the pages leave them open)
 *   - alpha = 1 exactly when the fp32 eviction logit passed in is > 0.
 *     0, -0 and NaN give alpha = 0.  A NaN logit is not an error.
 *   - A token marked at position i is visible to the queries at positions
 *     i .. i + w (inclusive) and to none after.  Unmarked tokens stay.
 *   - Decisions are per KV head.  Query head hq reads KV head hq / G with
 *     G = num_q_heads / num_kv_heads.
 *   - dms_append_step appends position q (retiring q - w - 1 if it was
 *     marked); dms_decode_attention then attends with the query of q, which
 *     sees itself.
 *   - Attention scale 1/sqrt(head_dim) unless dms_config.scale != 0.
 *
 * Conventions
 *   - Pointers named d_* are device pointers, h_* host pointers.  All are
 *     owned by the caller.  The library never allocates device memory: the
 *     cache lives entirely in the caller's workspace (dms_workspace_bytes),
 *     which holds offsets and indices only, no pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls marked "async" only enqueue work on `stream`; inputs must stay
 *     valid until the stream reaches them.  One cache is used from one
 *     stream at a time.
 *   - Every call returns DMS_OK (0) or a negative dms_status.  Argument and
 *     state errors are detected on the host before anything is enqueued.
 *     Running out of pool blocks is detected on the device: it sets a sticky
 *     error reported by dms_cache_stats and cleared by dms_cache_reset; the
 *     token that found no block is not stored and all memory accesses stay
 *     in bounds.
 *   - Layouts are row-major, innermost index last.  B = batch,
 *     Hq = num_q_heads, Hkv = num_kv_heads, d = head_dim.
 */
#ifndef DMS_H
#define DMS_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DMS_API __attribute__((visibility("default")))
#else
#define DMS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dms_cache dms_cache; /* opaque host handle */

typedef enum { DMS_F32 = 0, DMS_BF16 = 1 } dms_dtype;

typedef enum {
  DMS_OK = 0,
  DMS_ERR_ARG = -1,           /* invalid argument (null pointer, shape, dtype, ...) */
  DMS_ERR_WORKSPACE = -2,     /* workspace too small or not 256-byte aligned */
  DMS_ERR_OUT_OF_BLOCKS = -3, /* block pool exhausted (sticky, device-detected) */
  DMS_ERR_CAPACITY = -4,      /* a sequence would exceed max_tokens */
  DMS_ERR_STATE = -5,         /* call not valid in the cache's current state */
  DMS_ERR_HIP = -6,           /* a HIP runtime call or kernel launch failed */
  DMS_ERR_DEVICE = -7,        /* current device is not gfx950 */
  DMS_ERR_TOO_LARGE = -8      /* the call needs more scratch than the built-in buffer holds */
} dms_status;

typedef struct {
  int32_t batch;        /* B >= 1 sequences (B <= 65535) */
  int32_t num_q_heads;  /* Hq, a multiple of num_kv_heads, Hq / Hkv <= 16 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* d, 64 or 128 */
  int32_t window;       /* w >= 0; values >= max_tokens behave like max_tokens */
  int32_t block_tokens; /* tokens per cache block; must be 16 */
  int32_t max_tokens;   /* per sequence, prompt plus decode steps, 1 .. 2^24 */
  int32_t split_wgs;    /* how the decode attention shares its work among work-groups:
                           0 automatic (see dms_cache_balance; a split goes over one
                           work-group per CU); 1 every (sequence, KV head) whole to
                           one work-group; n >= 2 always split the live blocks in
                           equal shares over min(n, resident) work-groups (requires
                           batch * num_kv_heads <= 4096) */
  int64_t pool_blocks;  /* blocks in the shared pool, 1 .. 2^31-1; one block holds
                           16 tokens of K and V of one (sequence, KV head) */
  dms_dtype dtype;      /* element type of Q, K, V; outputs are always fp32 */
  float scale;          /* attention scale; 0 -> 1/sqrt(head_dim) */
} dms_config;

typedef struct {
  int64_t live_tokens;      /* sum over (sequence, KV head) of visible tokens now */
  int64_t seen_tokens;      /* sum over (sequence, KV head) of tokens appended so far */
  int64_t allocated_blocks; /* pool blocks in use */
  int64_t live_token_steps; /* sum, over dms_append_step calls, of live_tokens right after
                               the call: the visible K/V rows the following attention reads */
  int32_t sticky_error;     /* 0, or the first device-detected dms_status */
  int32_t split_mode;       /* 1 when the decode attention currently splits the live blocks
                               in equal shares, 0 when it gives each (sequence, KV head)
                               whole to one work-group (see dms_cache_balance) */
} dms_stats;

/* Bytes of device workspace the cache needs for `cfg`, or 0 if cfg is invalid.
   The caller allocates it (256-byte aligned) and keeps it alive until
   dms_cache_destroy.  The size grows with pool_blocks (one block is
   2*16*d*sizeof(dtype) bytes of K/V plus 68 bytes of metadata) and with
   B*Hkv*(max_tokens/16 + window + 6) 32-bit words of per-head state. */
DMS_API size_t dms_workspace_bytes(const dms_config* cfg);

/* Creates a handle over d_workspace and enqueues its initialisation (empty
   cache) on `stream`.  The current HIP device must be a gfx950 and must stay
   current for every later call on the handle.  *out receives the handle. */
DMS_API int dms_cache_create(const dms_config* cfg, void* d_workspace, size_t workspace_bytes,
                     void* stream, dms_cache** out);

/* Frees the host handle only; the workspace stays the caller's.  NULL is a no-op. */
DMS_API int dms_cache_destroy(dms_cache* c);

/* Async.  Empties the cache (all sequences back to length 0, pool released,
   sticky error cleared). */
DMS_API int dms_cache_reset(dms_cache* c, void* stream);

/* Async.  Compresses a prompt into an empty cache: for every (b, h), the
   tokens of positions 0 .. len_b - 1 that are visible to the query at
   len_b - 1 are stored, and the marked ones among the last w + 1 positions
   are scheduled for eviction, exactly as len_b calls of dms_append_step
   would leave the cache.  Only visible rows are read from d_k / d_v.
     d_k, d_v : [B, Hkv, max_len, d] of dtype
     d_logit  : [B, Hkv, max_len] fp32 eviction logits
     h_lengths: [B] host array, 0 <= len_b <= min(max_len, max_tokens)
   Errors: DMS_ERR_STATE if any sequence is non-empty, DMS_ERR_CAPACITY if a
   length exceeds max_tokens, DMS_ERR_ARG for other bad arguments. */
DMS_API int dms_prefill_compress(dms_cache* c, const void* d_k, const void* d_v, const float* d_logit,
                         const int32_t* h_lengths, int32_t max_len, void* stream);

/* Async.  Appends one token to every sequence b at position q_b = len_b:
   decides alpha from its logit, retires position q_b - w - 1 if that token
   was marked (its slot is reused), stores the new K/V row.
     d_k, d_v : [B, Hkv, d] of dtype
     d_logit  : [B, Hkv] fp32
   Errors: DMS_ERR_CAPACITY if some len_b + 1 > max_tokens. */
DMS_API int dms_append_step(dms_cache* c, const void* d_k, const void* d_v, const float* d_logit,
                    void* stream);

/* Where the _channel variants read the eviction logit.  Source: "Inference-
   Time Hyper-Scaling with KV Cache Compression", third-party paper summary
   page, sections "Key claims" and "Method": no parameters are added; one
   neuron of each head's K or Q projection is repurposed to produce the
   eviction logit. */
typedef enum {
  DMS_LOGIT_FROM_K = 0, /* KV head h's logit is channel `channel` of its own key row */
  DMS_LOGIT_FROM_Q = 1  /* it is channel `channel` of query head h * G, the group's first
                           query head (the pages do not say which query head of a group
                           drives the group's shared decision) */
} dms_logit_source;

/* Async.  dms_append_step with the eviction logit read from a projection
   channel instead of a separate array:
     logit[b, h] = fp32(d_k[b, h, channel])      for DMS_LOGIT_FROM_K
     logit[b, h] = fp32(d_q[b, h * G, channel])  for DMS_LOGIT_FROM_Q
   (bf16 values are upcast exactly), then the same decision, retirement and
   store.  d_q: [B, Hq, d] of dtype, read only for DMS_LOGIT_FROM_Q (may be
   NULL otherwise).  zero_channel != 0 (DMS_LOGIT_FROM_K only) stores the key
   row with that channel set to 0, so that the repurposed neuron takes no part
   in the attention scores; d_k itself is not modified.
   Errors: DMS_ERR_ARG for a bad source or channel (not in 0 .. d-1), a NULL
   d_q with DMS_LOGIT_FROM_Q, or zero_channel with DMS_LOGIT_FROM_Q;
   DMS_ERR_CAPACITY as dms_append_step. */
DMS_API int dms_append_step_channel(dms_cache* c, const void* d_k, const void* d_v, const void* d_q,
                                    int32_t source, int32_t channel, int32_t zero_channel, void* stream);

/* Async.  dms_prefill_compress with the eviction logits read from a
   projection channel (as dms_append_step_channel, at every prompt position):
     logit[b, h, i] = fp32(d_k[b, h, i, channel])      for DMS_LOGIT_FROM_K
     logit[b, h, i] = fp32(d_q[b, h * G, i, channel])  for DMS_LOGIT_FROM_Q
   d_q: [B, Hq, max_len, d] of dtype, read only for DMS_LOGIT_FROM_Q.
   zero_channel as in dms_append_step_channel.  Errors: those of
   dms_prefill_compress and of dms_append_step_channel's arguments. */
DMS_API int dms_prefill_compress_channel(dms_cache* c, const void* d_k, const void* d_v, const void* d_q,
                                         int32_t source, int32_t channel, int32_t zero_channel,
                                         const int32_t* h_lengths, int32_t max_len, void* stream);

/* Async.  Attention of every prompt query under the same visibility rule,
   for the prompt that dms_prefill_compress (or _channel) has just stored:
     out[b, hq, i, :] = sum_j softmax_j(scale * <q[b,hq,i], k_j>) v_j,
   j over the tokens of (b, hq / G) visible to position i, for every
   0 <= i < len_b: the unmarked positions below i - w and every position of
   i - w .. i.  Sources: "Inference-Time Hyper-Scaling with KV Cache
   Compression", third-party paper summary page, section "Method" (the
   decisions act as an additive attention mask that is never built, the same
   at every position, and it suits FlashAttention-style kernels).  The
   positions below i - w are read from the cache (right after the prompt's
   compression it holds exactly the unmarked ones among them), the window from
   d_k / d_v; the decisions are not needed again.  After
   dms_prefill_compress_channel with zero_channel, that key channel is read
   as 0 from d_k as well, as the cache stores it.
     d_q         : [B, Hq, max_len, d] of dtype, the prompt's queries
     d_k, d_v    : [B, Hkv, max_len, d], the tensors the compression read
     d_out       : [B, Hq, max_len, d] fp32; rows i >= len_b are not written
   Errors: DMS_ERR_STATE unless the last call that changed the cache was a
   successful prefill (an append or a reset in between makes it invalid);
   DMS_ERR_ARG for NULL pointers or a max_len shorter than some prompt. */
DMS_API int dms_prefill_attention(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, int32_t max_len,
                                  float* d_out, void* stream);

/* Async.  Grouped-query decode attention of the query at each sequence's
   last position over that sequence's visible tokens:
     out[b, hq, :] = sum_i softmax_i(scale * <q[b,hq], k_i>) v_i,
   i over the visible tokens of (b, hq / G).
     d_q  : [B, Hq, d] of dtype
     d_out: [B, Hq, d] fp32; the rows of a (sequence, KV head) left with no
            live token by an exhausted pool (sticky DMS_ERR_OUT_OF_BLOCKS)
            are not written
   Errors: DMS_ERR_STATE if some sequence has no token yet. */
DMS_API int dms_decode_attention(dms_cache* c, const void* d_q, float* d_out, void* stream);

/* Async.  One decode step: dms_append_step followed by dms_decode_attention,
   with the same arguments, results and final cache, in fewer launches.  In
   whole-unit mode (see dms_cache_balance) it is a single kernel: the
   work-group that attends a (sequence, KV head) also appends its token, and
   the attention reads the cache as it stood before the step without the
   retiring token, plus the new token from d_k / d_v, which is exactly the
   visible set after the append.  In split mode it is two launches: that
   attention, split over work-groups, then the split merge, which also
   appends.  Unlike the two calls, a sequence may be
   empty before the step (its output is then the new token's value row).
   When the pool is exhausted (sticky DMS_ERR_OUT_OF_BLOCKS) the token that
   found no block is not stored but is still attended in this step.
     d_q : [B, Hq, d]; d_k, d_v: [B, Hkv, d] of dtype; d_logit: [B, Hkv] fp32
     d_out: [B, Hq, d] fp32
   Errors: DMS_ERR_CAPACITY if some len_b + 1 > max_tokens; DMS_ERR_ARG for
   NULL pointers. */
DMS_API int dms_decode_step(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, const float* d_logit,
                            float* d_out, void* stream);

/* Async.  dms_decode_step with its launches timed by the HIP runtime:
   start_event is stamped at the start of the step's first kernel and
   stop_event at the end of its last (as dms_decode_attention_timed).  For
   measurement.  Errors: as dms_decode_step; DMS_ERR_ARG for a NULL event. */
DMS_API int dms_decode_step_timed(dms_cache* c, const void* d_q, const void* d_k, const void* d_v,
                                  const float* d_logit, float* d_out, void* start_event, void* stop_event,
                                  void* stream);

/* Async.  dms_decode_step with the eviction logit read from a projection
   channel, as dms_append_step_channel (same sources, channel and zeroing;
   d_q is both the step's queries and, for DMS_LOGIT_FROM_Q, the logit
   source).  Errors: those of dms_decode_step and of
   dms_append_step_channel's arguments. */
DMS_API int dms_decode_step_channel(dms_cache* c, const void* d_q, const void* d_k, const void* d_v,
                                    int32_t source, int32_t channel, int32_t zero_channel, float* d_out,
                                    void* stream);

/* Synchronises `stream`, reads every (sequence, KV head)'s live count and
   re-plans how the decode attention shares its work.  Heads reach different
   compression ratios ("Inference-Time Hyper-Scaling with KV Cache
   Compression", third-party paper summary page, section "Method": each head
   can land at its own compression ratio), so the live blocks per (sequence,
   KV head) can differ several-fold.  Whole-unit mode deals the (sequence, KV
   head)s to the work-groups longest first by live blocks; when the heaviest
   work-group would still carry more than 1/16 above the mean, the attention
   switches to split mode, which gives every work-group an equal share of the
   live blocks and merges the pieces of a split (sequence, KV head) in a
   second launch.  With fewer (sequence, KV head)s than work-groups, each
   gets a work-group of its own unless the heaviest one, streamed by one
   work-group alone, is estimated to take longer than the split with its
   fixed costs (the estimate's rates are MI355X measurements).  The plan stays in force until the next dms_cache_balance, reset
   or prompt compression; calls stay correct whatever the plan, only their
   speed depends on it.  With split_wgs != 0 the mode is fixed (1: whole
   units, dealt as above; >= 2: split, nothing to do).  Call after a prompt's
   compression and from time to time as the live counts drift. */
DMS_API int dms_cache_balance(dms_cache* c, void* stream);

/* Async.  dms_decode_attention, with its kernels timed by the HIP runtime:
   start_event and stop_event (hipEvent_t, created by the caller with timing
   enabled) are stamped with the start of the attention kernel and the end of
   the call's last kernel (the split merge when one runs), not at marker
   packets around the call, so hipEventElapsedTime gives the call's own
   device time.  For measurement; the results are those of
   dms_decode_attention.
   Errors: as dms_decode_attention; DMS_ERR_ARG for a NULL event. */
DMS_API int dms_decode_attention_timed(dms_cache* c, const void* d_q, float* d_out, void* start_event,
                                       void* stop_event, void* stream);

/* Async.  `chunk` decode steps at once: for every sequence b and every
   0 <= j < chunk, position q_j = len_b + j is appended (decision,
   retirement, store, as dms_append_step does, in order) and its query
   attends the tokens visible to q_j:
     out[b, hq, j, :] = attention of q[b, hq, j] over Vis(b, hq / G, q_j).
   The same results as `chunk` calls of dms_append_step + dms_decode_attention
   with the j-th slices (up to the order of floating-point sums), and the same
   final cache.  Sources: as dms_append_step and dms_decode_attention; the
   rule gives every position its own visible set whatever the order of work.
   Every cached block is read once for all the chunk's queries.
     d_q   : [B, Hq, chunk, d] of dtype
     d_k, d_v: [B, Hkv, chunk, d] of dtype
     d_logit: [B, Hkv, chunk] fp32
     d_out : [B, Hq, chunk, d] fp32
   Errors: DMS_ERR_ARG for NULL pointers, chunk < 1, or a cache whose
   max_tokens exceeds 131072 (the pending-eviction bitmap of a sequence is
   kept in on-chip memory); DMS_ERR_CAPACITY if some len_b + chunk >
   max_tokens. */
DMS_API int dms_decode_chunk(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, const float* d_logit,
                             int32_t chunk, float* d_out, void* stream);

/* Async.  dms_decode_chunk with the eviction logits read from a projection
   channel (as dms_append_step_channel, at every chunk position j):
     logit[b, h, j] = fp32(d_k[b, h, j, channel])      for DMS_LOGIT_FROM_K
     logit[b, h, j] = fp32(d_q[b, h * G, j, channel])  for DMS_LOGIT_FROM_Q
   zero_channel (DMS_LOGIT_FROM_K only): the chunk's keys are stored with that
   channel at 0 and attended that way.  Errors: those of dms_decode_chunk and
   of dms_append_step_channel's arguments. */
DMS_API int dms_decode_chunk_channel(dms_cache* c, const void* d_q, const void* d_k, const void* d_v,
                                     int32_t source, int32_t channel, int32_t zero_channel, int32_t chunk,
                                     float* d_out, void* stream);

/* Training-time relaxed DMS attention: the decisions as a differentiable
   soft mask (Gumbel-sigmoid), for learning the eviction logits.  Source:
   "Inference-Time Hyper-Scaling with KV Cache Compression", third-party
   paper summary page, section "Method": during training the binary decision
   is relaxed through a Gumbel-sigmoid at low temperature with a logit
   offset, its effect is delayed by the window, and the decisions enter
   attention as an additive mask.  The page prints no formula for that mask;
   the form below is this library's reading of it (the additive term whose
   limits alpha -> 0 and alpha -> 1 give the hard rule's 0 and -inf).
   Readings fixed here:
     x_i     = (logit_i + gamma + noise_i) / tau, alpha_i = sigmoid(x_i), with
               noise_i the Gumbel (logistic) sample, supplied by the caller
     bias    = log(1 - alpha_i) = -softplus(x_i) for queries q with q - i > w,
               0 for i <= q <= i + w (the window), -inf for i > q (causal)
     out     = softmax(scale * q k^T + bias) v per query head (GQA: query head
               hq reads KV head hq / G), scale = 1/sqrt(d) when 0 is passed
     lse     = natural log of each row's softmax denominator (for backward)
   As tau -> 0 with the logit's sign fixed this is the hard rule of the
   decode path (alpha in {0, 1}).  Unlike that rule, a NaN logit or noise
   value is not read as unmarked here: it propagates to the outputs and
   gradients of the queries it reaches, as in any differentiable layer.
   Layouts: d_q [B, Hq, T, d], d_k, d_v [B, Hkv, T, d] bf16; d_logit,
   d_noise [B, Hkv, T] fp32; d_out [B, Hq, T, d] and d_lse [B, Hq, T] fp32.
   d = 64 or 128; 1 <= T <= 2^20; window >= 0; tau > 0.  d_workspace:
   256-byte aligned, at least dms_soft_attention_forward_workspace_bytes (a
   copy of v in a transposed operand layout and each key's bias).  Async.
   Errors: DMS_ERR_ARG for NULL pointers or bad shapes or parameters,
   DMS_ERR_WORKSPACE for a small or unaligned workspace, DMS_ERR_DEVICE if
   the current device is not gfx950. */
DMS_API int dms_soft_attention_forward(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d, int32_t window,
                                       float gamma, float tau, float scale, const void* d_q, const void* d_k,
                                       const void* d_v, const float* d_logit, const float* d_noise, float* d_out,
                                       float* d_lse, void* d_workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace dms_soft_attention_forward needs (0 for bad
   shapes). */
DMS_API size_t dms_soft_attention_forward_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                                                          int32_t d);

/* Async.  dms_soft_attention_forward for callers that cannot allocate
   device memory (code under HIP graph capture, serving loops, harnesses that
   forbid hipMalloc): the same computation and results, with its scratch (the
   forward's workspace) in a buffer built into the library instead of a
   caller workspace.  The buffer holds dms_soft_attention_forward_noalloc_max_bytes()
   = 64 MiB per GPU, kept from the first call on that GPU until the process
   ends; its address is looked up on that first call (the only setup, no
   allocation).  Calls on one GPU share it: calls that overlap in time on
   one GPU (different streams without ordering, or different host threads)
   race, and must be ordered by the caller.  Nothing in the buffer carries
   over from one call to the next.
   Errors: as dms_soft_attention_forward; DMS_ERR_TOO_LARGE when
   dms_soft_attention_forward_workspace_bytes of the shape exceeds the
   buffer (nothing is enqueued); DMS_ERR_HIP if the buffer's address cannot
   be found. */
DMS_API int dms_soft_attention_forward_noalloc(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d,
                                               int32_t window, float gamma, float tau, float scale, const void* d_q,
                                               const void* d_k, const void* d_v, const float* d_logit,
                                               const float* d_noise, float* d_out, float* d_lse, void* stream);

/* Bytes of the buffer built into dms_soft_attention_forward_noalloc. */
DMS_API size_t dms_soft_attention_forward_noalloc_max_bytes(void);

/* Bytes of device workspace dms_soft_attention_backward needs (0 for bad
   shapes): copies of q, dout and k in a transposed operand layout, the row
   dot products sum(dout * out) and each key's bias. */
DMS_API size_t dms_soft_attention_backward_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                                                           int32_t d);

/* Gradients of sum(dout * out) of dms_soft_attention_forward with respect to
   q, k, v and the logits (noise, gamma, tau and scale are constants), from
   the forward's d_out and d_lse (recomputation of the scores, no stored
   probabilities).  d_dout bf16 [B, Hq, T, d]; d_dq fp32 [B, Hq, T, d]; d_dk,
   d_dv fp32 [B, Hkv, T, d]; d_dlogit fp32 [B, Hkv, T] (all written, not
   accumulated).  dK, dV and dlogit sum over the G query heads of each KV
   head; dlogit_i = -sigmoid(x_i) / tau * (sum of dS over the far queries),
   dS = P (dP - rowsum(dout * out)).  d_workspace: 256-byte aligned, at least
   dms_soft_attention_backward_workspace_bytes.  Async.  Errors: as the
   forward, and DMS_ERR_WORKSPACE for a small or unaligned workspace. */
DMS_API int dms_soft_attention_backward(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d, int32_t window,
                                        float gamma, float tau, float scale, const void* d_q, const void* d_k,
                                        const void* d_v, const float* d_logit, const float* d_noise,
                                        const float* d_out, const float* d_lse, const void* d_dout, float* d_dq,
                                        float* d_dk, float* d_dv, float* d_dlogit, void* d_workspace,
                                        size_t workspace_bytes, void* stream);

/* Synchronises `stream`, then fills *out. */
DMS_API int dms_cache_stats(dms_cache* c, dms_stats* out, void* stream);

/* Synchronises `stream`, then copies the logical state of the units
   u = unit_begin .. unit_begin + unit_count - 1, where u = b * Hkv + h:
     h_slot_pos: [unit_count, max_tokens]  position stored in each slot, -1 if
                 the slot holds no visible token
     h_ring    : [unit_count, min(window, max_tokens) + 1]  pending-eviction
                 ring: entry q mod (w+1) holds the slot of a marked token at
                 position q that is still visible, else -1
     h_n       : [unit_count]  slots in use (visible tokens)
   Any of the three may be NULL to skip it.  For tests and checkpoints; not
   on the hot path. */
DMS_API int dms_cache_export(dms_cache* c, int32_t unit_begin, int32_t unit_count, int32_t* h_slot_pos,
                     int32_t* h_ring, int32_t* h_n, void* stream);

/* Static string naming a status code. */
DMS_API const char* dms_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DMS_H */
