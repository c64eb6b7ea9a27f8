/*
 * tls.h -- C ABI of the MI355X (gfx950) two-level sparse-attention decode
 * library (libtls.so).
 *
 * The operation is one decode step of AsyncTLS two-level sparse attention
 * (pages "AsyncTLS: Efficient Generative LLM Inference with Asynchronous
 * Two-level Sparse Attention", section 2 "Methodology"):
 *   stage 1 (section 2A, coarse block filtering): per-block key max/min
 *     summaries scored with the Quest upper bound, evaluated as the GEMM
 *     [q+, q-] . [Kmax; Kmin]; the top-Kb blocks are kept;
 *   stage 2 (section 2A, fine token selection): inside the kept blocks, tokens
 *     are scored on a few label channels of an INT4 key cache (Double-Sparsity
 *     style); the top-Kt tokens are kept;
 *   attention over only the kept tokens (section 2A);
 *   staggered offload (section 2B): block selection for the next step
 *     overlaps the current step, and only the blocks missing from the device
 *     (T_t = M_t minus the resident set) are copied from pinned host memory.
 *
 * Conventions shared by every call
 *   - bf16 tensors are passed as device pointers to 16-bit bf16 values.
 *   - Every pointer argument is a device pointer unless stated otherwise.
 *     All buffers belong to the caller; the library keeps no pointer after a
 *     call returns, except the offload context (documented there).
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *     and return without synchronising. A fault inside a kernel surfaces at
 *     the caller's next synchronisation, as usual for HIP.
 *   - Return value: TLS_OK (0) or a negative TLS_ERR_* code; tls_last_error()
 *     then returns a message for the calling thread. Argument errors are
 *     detected before anything is enqueued.
 *   - One selection is made per (batch b, kv head h) pair, shared by the
 *     G = num_q_heads / num_kv_heads query heads g = h*G .. h*G+G-1; the heads
 *     of a group are combined by taking the maximum of their scores.
 *   - Index outputs are sets, written in ascending order. Ties in a top-k go to
 *     the lower index.
 *   - Workspaces: `ws` must be at least tls_workspace_size(shape, which) bytes
 *     (256-byte aligned). Their contents on entry do not matter, except for
 *     the first 64 KiB of a TLS_WS_DECODE workspace and for TLS_WS_STEP
 *     (see tls_sparse_decode and tls_decode_step). Calls that share one
 *     workspace must not overlap in time.
 *
 * Layouts (row-major)
 *   q          [B, Hq, D]            bf16
 *   kv         [B, Hkv, N, row]      bf16; row = D + DV (K then V) or, when
 *                                    v_is_k_prefix, row = D and V[t] = K[t, 0:DV]
 *   label_ch   [Hkv, r]              int32, ascending channel numbers in [0, D)
 *   summ       [B, Hkv, NT, D/32, 2, 4, 16, 8]  bf16, NT = ceil(NBs / 16) with
 *                                    NBs = ceil(ctx_capacity / bs) (NB when the
 *                                    capacity is the length): the
 *                                    block summaries in tile-fragment order --
 *                                    element [b, h, T, c, m, kq, n, e] is channel
 *                                    32c + 8kq + e of block 16T + n, m = 0 its
 *                                    Kmax, m = 1 its Kmin (so every 16-block,
 *                                    32-channel MFMA operand is 1 KB contiguous);
 *                                    the entries of blocks 16T + n >= NB in the
 *                                    last tile are not used
 *   codes      [B, Hkv, N, r/2]      uint8; channel i in byte i/2, low nibble for
 *                                    even i, two's-complement 4-bit code in [-7, 7]
 *   scale      [B, Hkv, N]           float; dequantised key = code * scale
 *   block_idx  [B, Hkv, Kb']         int32, Kb' = min(Kb, NB)
 *   token_idx  [B, Hkv, Kt']         int32, Kt' = min(Kt, Kb' * bs); a pair with
 *                                    fewer valid candidates (partial last block)
 *                                    is padded with -1 after its ascending entries
 *   out        [B, Hq, DV]           float
 *   lse        [B, Hq]               float, natural-log log-sum-exp of the scaled
 *                                    logits over the kept tokens
 *   with NB = ceil(N / bs).
 */
#ifndef TLS_H
#define TLS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TLS_OK = 0,
  TLS_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shape      */
  TLS_ERR_UNSUPPORTED = -2, /* valid shape that no compiled kernel covers       */
  TLS_ERR_WORKSPACE = -3,   /* workspace smaller than tls_workspace_size()      */
  TLS_ERR_HIP = -4,         /* a HIP runtime call failed (message has the name) */
  TLS_ERR_STATE = -5        /* offload context used out of order                */
};

enum { TLS_WS_BLOCKS = 0, TLS_WS_TOKENS = 1, TLS_WS_DECODE = 2, TLS_WS_SELECT = 3, TLS_WS_STEP = 4 };

typedef struct tls_shape {
  int32_t batch;         /* B                                                    */
  int32_t num_q_heads;   /* Hq, a multiple of num_kv_heads                       */
  int32_t num_kv_heads;  /* Hkv                                                  */
  int32_t head_dim_qk;   /* D: 128 (GQA/MHA) or 576 (MLA latent + rope); any     */
                         /*    multiple of 32 up to 576                          */
  int32_t head_dim_v;    /* DV: a multiple of 8, at most 512                     */
  int32_t v_is_k_prefix; /* 1: no separate V, V[t] = K[t, 0:DV] (MLA)            */
  int64_t ctx_len;       /* N: cached tokens of every sequence, >= 1             */
  int32_t block_size;    /* bs: tokens per block, 1..64                          */
  int32_t num_label_ch;  /* r: label channels, even, 2..32                       */
  int32_t top_kb;        /* Kb >= 1; values above NB keep every block            */
  int32_t top_kt;        /* Kt >= 1; values above Kb'*bs keep every candidate    */
  float sm_scale;        /* softmax scale applied to q.k (e.g. 1/sqrt(D))        */
  int64_t ctx_capacity;  /* tokens allocated per sequence (>= ctx_len; 0 means   */
                         /*    ctx_len): the stride of every per-sequence array  */
} tls_shape_t;

/* Bytes of workspace needed by tls_select_blocks (TLS_WS_BLOCKS),
 * tls_select_tokens (TLS_WS_TOKENS), tls_select (TLS_WS_SELECT: the other
 * two together) or tls_sparse_decode (TLS_WS_DECODE) for this shape; 0 if
 * the shape is invalid for that call. tls_select_tokens
 * takes any Kt' up to 16384 candidates per pair (Kb' * bs); beyond that (up
 * to 2^20 candidates, e.g. Kb >= NB: token selection over the whole cache)
 * it selects in passes over chunks and needs Kt' <= 8192. The other calls
 * have no such limit (attention over every token is Kb >= NB, Kt >= N). */
size_t tls_workspace_size(const tls_shape_t *shape, int which);

/* Block summaries and the INT4 label cache (section 2A: the block-level index
 * and the token-level index; run once per cache, not per step).
 *   kv [B,Hkv,N,row] -> summ (tile-fragment order, above), codes [B,Hkv,N,r/2],
 *   scale [B,Hkv,N].
 * Kmax/Kmin are exact per-channel extremes over the valid tokens of a block.
 * Label cache per token: a = max |K[t, c_i]| over the label channels; a == 0
 * gives scale 0 and codes 0, otherwise scale = float(a/7) and
 * code_i = clamp(rint(K[t,c_i] / scale), -7, 7), both divisions in double. */
int tls_build_summaries(const tls_shape_t *shape, const void *kv, const int32_t *label_ch, void *summ,
                        uint8_t *codes, float *scale, void *stream);

/* Decode-time append (the cache grows by n_new tokens per sequence).
 *   shape->ctx_len is the length BEFORE the append; ctx_len + n_new must not
 *   exceed ctx_capacity, the allocated length (the stride of kv, summ, codes
 *   and scale).
 *   new_kv [B,Hkv,n_new,row] bf16 device: the new rows, K then V (K only when
 *   v_is_k_prefix), 16-byte aligned like kv.
 * Writes the rows to positions ctx_len .. ctx_len+n_new-1 of kv and rebuilds
 * the summaries of the blocks holding them, and the codes and scales of all
 * their tokens, from the grown cache, so that summ, codes and scale equal what
 * tls_build_summaries gives for length ctx_len + n_new. Later calls pass
 * ctx_len + n_new. Two launches on `stream`; errors as tls_build_summaries. */
int tls_append_kv(const tls_shape_t *shape, const void *new_kv, int32_t n_new, void *kv, const int32_t *label_ch,
                  void *summ, uint8_t *codes, float *scale, void *stream);

/* Stage 1 (section 2A, coarse block filtering).
 *   s[g, j] = sum_c max(q_gc Kmax_jc, q_gc Kmin_jc) = [q_g+, q_g-] . [Kmax_j; Kmin_j]
 *   S[j] = max over the G heads of the pair;  block_idx = top-Kb' of S.
 * block_score_opt: NULL, or [B,Hkv,NB] float receiving S. */
int tls_select_blocks(const tls_shape_t *shape, const void *q, const void *summ, int32_t *block_idx,
                      float *block_score_opt, void *ws, size_t ws_bytes, void *stream);

/* Stage 2 (section 2A, fine token selection) inside the blocks of block_idx
 * (ascending, Kb' per pair).
 *   a[g, t] = scale_t * sum_i q[g, c_i] * code[t, i]  (q is not quantised)
 *   A[t] = max over the G heads;  token_idx = top-Kt' of A over the valid
 *   tokens (t < N) of the kept blocks. */
int tls_select_tokens(const tls_shape_t *shape, const void *q, const int32_t *label_ch, const uint8_t *codes,
                      const float *scale, const int32_t *block_idx, int32_t *token_idx, void *ws,
                      size_t ws_bytes, void *stream);

/* Both stages (section 2A) in one call, with the results of
 * tls_select_blocks followed by tls_select_tokens: block_idx [B,Hkv,Kb'] and
 * token_idx [B,Hkv,Kt'], both ascending. Up to 4096 blocks per sequence the
 * block top-k runs inside the token-scoring kernel (each of a pair's scoring
 * workgroups selects the pair's blocks from the block scores; one of them
 * writes block_idx), which saves a launch; above that it runs as in
 * tls_select_blocks. ws: tls_workspace_size(shape, TLS_WS_SELECT) bytes.
 * Errors as the two calls. */
int tls_select(const tls_shape_t *shape, const void *q, const void *summ, const int32_t *label_ch,
               const uint8_t *codes, const float *scale, int32_t *block_idx, int32_t *token_idx, void *ws,
               size_t ws_bytes, void *stream);

/* Attention over the kept tokens only (section 2A), split over the token
 * list and merged with log-sum-exp.
 *   out[b, g] = sum_t softmax_t(sm_scale * q_g . K[t]) V[t] over t in token_idx
 * kv_cache: with slot_map == NULL, the full cache [B,Hkv,N,row]. Otherwise a
 *   resident cache [B,Hkv,slots_per_pair,bs,row] addressed through
 *   slot_map [B,Hkv,NBs] (int32 slot of each block, -1 = not resident; NBs =
 *   blocks of ctx_capacity, NB when the capacity is the length); every
 *   block holding a kept token must be resident.
 * Entries -1 in token_idx are skipped. lse_opt: NULL or [B,Hq] float.
 * ws: tls_workspace_size(shape, TLS_WS_DECODE) bytes: 64 KiB of counters,
 *   then the splits' partial results. The counters must be zero before the
 *   first call (zero-fill the workspace once, e.g. one hipMemset); every call
 *   that completes leaves them zero, so later calls need no clearing, and
 *   calls of different shapes may share the workspace. A workspace written
 *   by anything else in between must be cleared again. (With 128-channel K
 *   and V rows and at most 512 attention workgroups, the last workgroup of
 *   each (pair, head tile) merges the splits, counting the workgroups done in
 *   these counters; otherwise a merge kernel follows the attention.) */
int tls_sparse_decode(const tls_shape_t *shape, const void *q, const void *kv_cache, const int32_t *slot_map,
                      int32_t slots_per_pair, const int32_t *token_idx, float *out, float *lse_opt, void *ws,
                      size_t ws_bytes, void *stream);

/* tls_sparse_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same kernels, same results (bit for bit) as tls_sparse_decode,
 * but the split partials go to a device array of the library's own
 * (TLS_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead of
 * a caller workspace; the caller passes only inputs and outputs. A shape whose
 * partials need more (tls_workspace_size(shape, TLS_WS_DECODE) above
 * TLS_NOALLOC_SCRATCH_BYTES) returns TLS_ERR_WORKSPACE before anything is
 * launched. Nothing in the array needs clearing: it starts zeroed, and every
 * call that completes leaves its counters zero (every partial is written
 * before it is read). Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other threads)
 * race on it, and the caller must order them. The first call on each device
 * looks the array's device address up (hipGetSymbolAddress, which may load
 * the library's device code), so make it before a graph capture begins. No
 * call allocates. Other errors as tls_sparse_decode. */
#define TLS_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
int tls_sparse_decode_noalloc(const tls_shape_t *shape, const void *q, const void *kv_cache,
                              const int32_t *slot_map, int32_t slots_per_pair, const int32_t *token_idx,
                              float *out, float *lse_opt, void *stream);

/* One whole decode step (section 2A: both selection stages, then attention
 * over the kept tokens) in ONE launch: the results of tls_select followed by
 * tls_sparse_decode on the full cache (kv [B,Hkv,N,row], no slot map) --
 * block_idx [B,Hkv,Kb'] and token_idx [B,Hkv,Kt'] ascending, out [B,Hq,DV],
 * lse_opt [B,Hq] or NULL. The pairs' steps are interleaved on the device: one
 * pair's selection runs while others stream their block summaries or gather
 * their rows.
 * Covers D = DV = 128 with a separate V, G <= 8, block size 64, 8 or 16 label
 * channels, NB <= 4096 and Kb' <= 128; other shapes return
 * TLS_ERR_UNSUPPORTED (use the two calls).
 * ws: tls_workspace_size(shape, TLS_WS_STEP) bytes, 256-byte aligned. Unlike
 * the other workspaces, its contents matter: it must be zero-filled before its
 * first use by this call (e.g. one hipMemset), and every call that completes
 * leaves it in that state, so later calls need no clearing. A workspace
 * written by anything else in between must be cleared again. Calls sharing a
 * workspace must not overlap in time. Errors as tls_select and
 * tls_sparse_decode; a failure inside the launch (which no valid input
 * causes) is reported by tls_decode_step_status. */
int tls_decode_step(const tls_shape_t *shape, const void *q, const void *summ, const int32_t *label_ch,
                    const uint8_t *codes, const float *scale, const void *kv, int32_t *block_idx,
                    int32_t *token_idx, float *out, float *lse_opt, void *ws, size_t ws_bytes, void *stream);

/* Synchronises `stream` and reads the error word tls_decode_step keeps in its
 * workspace: TLS_OK, or TLS_ERR_STATE if a launch abandoned work (an item it
 * waited for was not published within its time limit, or an XCD's queue was
 * left undrained); the outputs of such a launch are not valid and the
 * workspace must be zero-filled again. */
int tls_decode_step_status(void *ws, void *stream);

/* ----------------------------------------------------------------------
 * Staggered offload (section 2B). The full cache stays in pinned host memory;
 * the device holds a resident cache of 2*Kb' block slots per pair plus a slot
 * map. At step t the token stage and the attention use the blocks chosen at
 * step t-1, while stage 1 for step t runs on a side stream; then only the
 * blocks of T_t = M_t \ C_t (C_t: resident blocks) are copied host -> device.
 * When slots run out, resident blocks outside M_{t-1} and M_t are evicted,
 * least recently selected first, lower block index first on equal steps.
 */
typedef struct tls_offload tls_offload_t;

/* Create an offload context.
 *   host_kv      [B,Hkv,Ns,row] bf16 in pinned host memory (hipHostMalloc),
 *                Ns = ctx_capacity (ctx_len when 0), a multiple of bs, its
 *                first ctx_len tokens filled; borrowed until
 *                tls_offload_destroy. A capacity above ctx_len lets the cache
 *                grow (tls_offload_append) and needs at least Kb blocks now.
 *   dev_cache    [B,Hkv,2*Kb',bs,row] bf16 device memory, borrowed.
 *   dev_slot_map two device buffers of [B,Hkv,NBs] int32 each (NBs = blocks
 *                of Ns), borrowed
 *                (dev_slot_map[0] and dev_slot_map[1]); step t reads buffer t%2
 *                and the prefetch of step t writes buffer (t+1)%2.
 *   initial_blocks [B,Hkv,Kb'] int32 host array: M_{-1}, ascending. These
 *                blocks are copied synchronously, slots assigned in order.
 * On success *out receives the context. The call synchronises the device. */
int tls_offload_create(const tls_shape_t *shape, const void *host_kv, void *dev_cache, int32_t *dev_slot_map0,
                       int32_t *dev_slot_map1, const int32_t *initial_blocks, tls_offload_t **out);

/* Slot map (device pointer) that step `step` must pass to tls_sparse_decode. */
const int32_t *tls_offload_slot_map(const tls_offload_t *ctx, int32_t step);

/* Incremental prefetch for step `step` (0, 1, 2, ... in order).
 *   dev_block_idx  M_t [B,Hkv,Kb'] int32 device buffer written by
 *                  tls_select_blocks on `side` (a hipStream_t) before this call.
 * With TLS_COPY_DEVICE (or TLS_COPY_FULL) the call only enqueues, on `side`, a planning kernel
 * (T_t, evictions, slot assignment, next slot map) and a copy kernel that
 * reads the blocks of T_t from host memory, and returns at once; M_t must stay
 * unchanged until they ran. With the host-planned modes it enqueues a copy of
 * M_t to host on `side`, waits for it on the calling thread (run it on a
 * helper thread to keep the main stream busy), computes T_t and the evictions,
 * and enqueues the block copies and the next slot map on `side`. Either way it
 * records `copies_done` (a hipEvent_t) on `side`; step step+1 must wait for
 * that event before reading the resident cache. n_copied_opt (host, may be
 * NULL) receives |T_t| summed over all pairs, or -1 when planned on the GPU
 * (read tls_offload_total_copied instead). The pinned staging buffers of the
 * context are reused by the next call, which first waits for `side`.
 * When planned on the GPU a run of calls may be captured into a HIP graph: the
 * planning kernel counts steps on the device, so the captured launches need
 * no host work; since the slot maps alternate by step parity, replaying the
 * graph repeatedly needs an even number of captured steps. */
int tls_prefetch_delta(tls_offload_t *ctx, int32_t step, const int32_t *dev_block_idx, void *side,
                       void *copies_done, int64_t *n_copied_opt);

/* Where tls_prefetch_delta plans the transfer of T_t and how it moves it.
 *   TLS_COPY_DEVICE (default when host_kv, allocated with hipHostMalloc, has a
 *     device mapping, 2*Kb' <= 1024 and NB <= 16384): planned and copied by
 *     kernels on the side stream, the calling thread never waits;
 *   TLS_COPY_GATHER (default when the device limits are exceeded): planned on
 *     the host, then one kernel on the side stream reads every block of T_t
 *     from host memory and applies the slot-map changes;
 *   TLS_COPY_MEMCPY (default without a device mapping): planned on the host,
 *     one hipMemcpyAsync per block plus a full slot-map upload.
 * All three give the same slots and maps.
 *   TLS_COPY_FULL (a baseline for comparison, not the method): planned on the
 *     GPU like TLS_COPY_DEVICE but without reuse: every block of M_t is copied
 *     at every step, into the half of the resident cache that the step
 *     reading M_{t-1} does not use (T_t = M_t; nothing is evicted).
 * Returns TLS_ERR_UNSUPPORTED for a mode the context cannot run, TLS_ERR_STATE
 * for a change to or from a GPU-planned mode after step 0 (GATHER <-> MEMCPY
 * may change at any step). */
enum { TLS_COPY_GATHER = 0, TLS_COPY_MEMCPY = 1, TLS_COPY_DEVICE = 2, TLS_COPY_FULL = 3 };
int tls_offload_set_copy_mode(tls_offload_t *ctx, int mode);

/* Decode-time append to an offloaded cache (section 1: the cache grows with
 * every generated token; section 2B: it lives in host memory).
 *   new_kv [B,Hkv,n_new,row] bf16 device, 16-byte aligned: the rows of the
 *   next n_new tokens. summ/codes/scale: the device index the steps read
 *   (capacity strides), label_ch as for tls_build_summaries.
 * Three launches on `stream`: the rows are written to host_kv after the
 * current length (through its device mapping); the summaries of the blocks
 * they fall in are updated from the new rows and the previous summaries (the
 * max / min of a block is exact either way), and their codes and scales
 * computed, so the index equals tls_build_summaries of the longer cache; and
 * where such a block is resident in the slot map that the next step's
 * attention reads, the rows are written into its slot too (a block that is
 * not resident is read from host_kv when it is next transferred). The steps
 * after it take a shape whose ctx_len includes the new tokens.
 * Ordering: `stream` must run after the copies of the last tls_prefetch_delta
 * (its copies_done event) and before the next step's calls. Errors:
 * TLS_ERR_INVALID_ARG (length beyond ctx_capacity, n_new < 1, NULL or
 * misaligned buffers), TLS_ERR_UNSUPPORTED (host_kv without a device
 * mapping), TLS_ERR_HIP. */
int tls_offload_append(tls_offload_t *ctx, const void *new_kv, int32_t n_new, const int32_t *label_ch, void *summ,
                       uint8_t *codes, float *scale, void *stream);
/* The current mode, or a negative error code for a NULL context. */
int tls_offload_get_copy_mode(const tls_offload_t *ctx);

/* Host view of the last transfer (for checking): per pair the count |T_t|
 * and the transferred blocks ascending (host arrays [B*Hkv] and [B*Hkv, Kb']).
 * With TLS_COPY_DEVICE or TLS_COPY_FULL the call synchronises the device and returns
 * TLS_ERR_STATE if a step could not be planned (M_t held a block number
 * outside [0, NB)); such a step changed no slot and no map entry. */
int tls_offload_last_delta(const tls_offload_t *ctx, int32_t *counts, int32_t *blocks);

/* Blocks copied since creation, summed over all steps and pairs (host int64).
 * Synchronises the device when planned on the GPU; errors as tls_offload_last_delta. */
int tls_offload_total_copied(const tls_offload_t *ctx, int64_t *total);

void tls_offload_destroy(tls_offload_t *ctx);

/* Measurement hook. From now on every call that launches kernel `which`
 * records start_event and end_event (hipEvent_t handles created and owned by
 * the caller) on its stream immediately before and after that kernel, so its
 * duration can be read with hipEventElapsedTime apart from the launches
 * around it:
 *   TLS_PROFILE_BLOCK_SCORES: the block-score GEMM of tls_select_blocks
 *     (not its top-k);
 *   TLS_PROFILE_ATTENTION: the attention kernel of tls_sparse_decode (not
 *     its split merge);
 *   TLS_PROFILE_HOST_COPY: the kernel of tls_prefetch_delta that reads the
 *     blocks of T_t from host memory (all modes but TLS_COPY_MEMCPY).
 * NULL, NULL turns it off. Process-wide; set it while no other thread is
 * calling the library. TLS_ERR_INVALID_ARG if exactly one event is NULL or
 * `which` is unknown. */
enum { TLS_PROFILE_BLOCK_SCORES = 0, TLS_PROFILE_ATTENTION = 1, TLS_PROFILE_HOST_COPY = 2 };
int tls_profile_events(int which, void *start_event, void *end_event);

/* Message for the last failed call on this thread ("" if none). */
const char *tls_last_error(void);

/* Library version string. */
const char *tls_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TLS_H */
