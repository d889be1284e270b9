/*
 * rswa.h - C ABI of the MI355X (gfx950) Reference Sliding Window Attention library.
 *
 * What is computed. Output token t of a sequence attends to the whole reference prefix P of
 * L_m = m tokens (visual tokens plus prompt, always visible) and to its last n output tokens, the
 * current one included: N(t) = P u D_n(t). The decode KV cache is therefore a constant
 * m + min(n, t) rows: a static prefix region plus an n-slot ring that overwrites the oldest output
 * on every append. Standard causal attention ("full causal" mode here) keeps all m + t rows.
 *   - deep dive "Unlimited-OCR" (ai-news-5min): the N(t) code block and the cache-size formula
 *     C(T) = L_m + min(n, T) <= L_m + n;
 *   - GeekNews "Unlimited OCR": R-SWA section (two-segment window of size m + n), KV cache
 *     management section (L_m + T vs L_m + min(n, T)), model architecture section (queue of
 *     capacity m + n that evicts the oldest output KV on every new token).
 *
 * Conventions shared by every entry point.
 *   - H = num_heads, D = head_dim. D must be 128 (RSWA_E_UNSUPPORTED otherwise).
 *   - Pointers named *_dev are device pointers on the current HIP device (e.g. a torch tensor's
 *     data_ptr()); pointers named *_host are host memory. The caller owns every buffer it passes
 *     and must keep it alive until the stream has passed the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call only
 *     enqueues work on that stream and returns; nothing blocks unless stated.
 *   - Arguments are validated on the host before anything is enqueued: an invalid call returns an
 *     error status and changes no state. No C++ exception crosses this ABI.
 *   - Element types: RSWA_BF16 is bfloat16 (16-bit patterns), RSWA_F32 is IEEE float32. All
 *     attention arithmetic is float32; a bf16 output is the round-to-nearest-even of the float32
 *     result.
 *   - Inputs are already position-encoded: the library does no position arithmetic, so the ring's
 *     slot order never matters (softmax attention is invariant under key permutation).
 *   - A cache is not thread-safe; distinct caches are independent.
 */
#ifndef RSWA_H
#define RSWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rswa_status {
  RSWA_OK = 0,
  RSWA_E_INVALID = -1,     /* bad argument or state; nothing was enqueued */
  RSWA_E_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim != 128) */
  RSWA_E_CAPACITY = -3,    /* full-causal append past max_steps, or storage too small */
  RSWA_E_OOM = -4,         /* device allocation failed */
  RSWA_E_HIP = -5,         /* a HIP runtime call or kernel launch failed */
  RSWA_E_INTERNAL = -6     /* unexpected internal failure */
} rswa_status;

typedef enum rswa_dtype { RSWA_BF16 = 0, RSWA_F32 = 1 } rswa_dtype;

/* RSWA_MODE_RSWA: prefix + n-slot ring (constant m + n rows).
 * RSWA_MODE_FULL_CAUSAL: prefix + every output (m + max_steps rows), the standard-attention
 * reference whose per-step cost grows with t. */
typedef enum rswa_mode { RSWA_MODE_RSWA = 0, RSWA_MODE_FULL_CAUSAL = 1 } rswa_mode;

/* Description of a batch of B decode sequences sharing one cache object. */
typedef struct rswa_cache_desc {
  int32_t batch;              /* B >= 1 */
  int32_t num_heads;          /* H >= 1 */
  int32_t head_dim;           /* D, must be 128 */
  int32_t kv_dtype;           /* rswa_dtype of the cache, of q and of appended k / v */
  int32_t mode;               /* rswa_mode */
  const int32_t* prefix_len;  /* host [B]: m_b >= 0 */
  const int32_t* window;      /* host [B]: n_b >= 1 (RSWA mode; ignored in FULL_CAUSAL) */
  const int32_t* max_steps;   /* host [B]: appends allowed per sequence in FULL_CAUSAL (>= 1);
                                 may be NULL in RSWA mode */
  void* storage_dev;          /* caller-owned device storage of at least rswa_cache_bytes()
                                 bytes, or NULL: the library allocates (and frees) it */
  uint64_t storage_bytes;     /* size of storage_dev; ignored when storage_dev is NULL */
  int32_t prefix_paged;       /* 0: the cache holds a copy of every prefix (rswa_cache_create);
                                 1: prefixes stay in a caller-owned token pool, looked up through
                                 a page table (rswa_cache_create_paged); the storage then holds
                                 only the output rows */
} rswa_cache_desc;

typedef struct rswa_cache rswa_cache; /* opaque; owned by the library */

/* Storage layout, for callers that inspect or snapshot the cache. Sequence b owns
 * R_b = m_b + cap_b rows per head (cap_b = n_b in RSWA mode, max_steps_b in FULL_CAUSAL mode),
 * or R_b = cap_b with prefix_paged = 1 (storage row r then holds cache row m_b + r):
 *   K[b][h][r][i] at element seq_offset[b] + (h * R_b + r) * D + i,
 *   V[b][h][r][i] at element seq_offset[b] + H * R_b * D + (h * R_b + r) * D + i,
 * elements of kv_dtype. Rows [0, m_b) hold the prefix; in RSWA mode output index j (0-based) lives
 * in row m_b + (j mod n_b); in FULL_CAUSAL mode in row m_b + j.
 * Pure host computation (no HIP call). Any output pointer may be NULL. */
rswa_status rswa_cache_plan(const rswa_cache_desc* desc, int64_t* seq_offset_host /* [B] */,
                            int32_t* rows_host /* [B] */, uint64_t* storage_bytes_host);

/* Bytes of storage the description needs (0 if the description is invalid). Host only. The size
 * ends with 4096 bytes after the last row that no row uses: the decode kernel loads whole row
 * tiles, so the last tile of the last range may read (never use) up to that many bytes past it. */
uint64_t rswa_cache_bytes(const rswa_cache_desc* desc);

/* Create a cache: take or allocate storage, copy every sequence's prefix K / V into rows
 * [0, m_b) (the static prefix region, written once and never updated; GeekNews "Unlimited OCR",
 * DeepEncoder section: visual tokens are encoded once and stay static), set every step counter
 * t_b to 0. prefix_k_dev / prefix_v_dev: packed token-major [sum_b m_b][H][D] of kv_dtype
 * (sequence b's rows follow sequence b-1's); may be NULL only if every m_b is 0. The prefix is
 * copied, not aliased. Rows beyond the prefix are not touched. Enqueued on `stream`; the call
 * BLOCKS until that stream has finished the copies (its metadata upload is staged in host memory).
 * Errors: RSWA_E_INVALID (desc, pointers), RSWA_E_UNSUPPORTED (head_dim), RSWA_E_CAPACITY
 * (storage_bytes too small), RSWA_E_OOM, RSWA_E_HIP. On error *out is NULL. */
rswa_status rswa_cache_create(const rswa_cache_desc* desc, const void* prefix_k_dev,
                              const void* prefix_v_dev, void* stream, rswa_cache** out);

/* Create a cache from a packed prefill batch, so that decoding continues where a prefill /
 * teacher-forced pass over the same sequences ended (the prefill-to-cache fill). Sequence b is
 * the segment [cu_seqlens_host[b], cu_seqlens_host[b + 1]) of k_dev / v_dev: its first m_b rows
 * are the prefix and the remaining t_b = S_b - m_b rows its outputs so far, in order (the layout
 * rswa_prefill_attn reads). The cache equals one made by rswa_cache_create from the prefixes
 * followed by t_b appends of those outputs, bit for bit: prefix rows [0, m_b); in RSWA mode the
 * last min(n_b, t_b) outputs in their ring slots (output j in row m_b + (j mod n_b); the cache
 * holds the prefix plus the previous n outputs: deep dive "Unlimited-OCR", N(t) code block); in
 * FULL_CAUSAL mode all t_b outputs in rows m_b + j; step counter t_b. Rows beyond those are not
 * touched. k_dev / v_dev: packed token-major [total][H][D] of kv_dtype, 16-byte aligned, holding
 * at least cu_seqlens_host[batch] rows (the call has no size to check this against);
 * cu_seqlens_host: host [batch + 1], cu_seqlens_host[0] >= 0, S_b >= m_b. desc->prefix_paged
 * must be 0. Enqueued on `stream`; the call BLOCKS until that stream has finished the copies.
 * Errors as rswa_cache_create, plus RSWA_E_INVALID (cu_seqlens, a segment shorter than its
 * prefix, prefix_paged) and RSWA_E_CAPACITY (FULL_CAUSAL: t_b > max_steps). On error *out is
 * NULL. */
rswa_status rswa_cache_create_from_prefill(const rswa_cache_desc* desc, const void* k_dev,
                                           const void* v_dev, const int32_t* cu_seqlens_host,
                                           void* stream, rswa_cache** out);

/* Create a cache whose prefixes live in a shared, token-granular page pool (paged / shared prefix
 * KV: the SGLang server that the deep dive "Unlimited-OCR" shows infer.py launching runs with a
 * page size of one token, and GeekNews "Unlimited OCR", limitations and future work, plans a pool
 * of prefill KV chunks that the model fetches). desc->prefix_paged
 * must be 1. pool_k_dev / pool_v_dev: caller-owned device arrays [pool_rows][H][D] of kv_dtype
 * (token-major: one row per token, 256 B per head in bf16), read during every decode, unchanged
 * and alive until rswa_cache_destroy. prefix_table_dev: device int32 [sum_b m_b]; prefix token j
 * of sequence b is pool row table[M_b + j], M_b = sum_{b' < b} m_b'. Several sequences may
 * point at the same pool rows (one document decoded by many sequences is stored once). Output rows
 * (the ring, or the full-causal rows) are per sequence in the cache storage as usual. Entries
 * outside [0, pool_rows) are rejected with RSWA_E_INVALID (checked on the device at creation; the
 * call blocks until the check is done). Decode results equal those of rswa_cache_create with the
 * gathered prefixes, bit for bit, when both cut the key ranges alike: always while a step's live
 * rows fit the last-level cache (256 MiB), and under the same rswa_cache_set_decode_split grid.
 * Beyond it the copying cache streams its rows with fewer workgroups per CU (see
 * rswa_cache_set_decode_split), and the two agree to float32 summation order. */
rswa_status rswa_cache_create_paged(const rswa_cache_desc* desc, const void* pool_k_dev,
                                    const void* pool_v_dev, int64_t pool_rows,
                                    const int32_t* prefix_table_dev, void* stream,
                                    rswa_cache** out);

/* K1, append / evict. For every sequence b with active_dev[b] != 0 (or every b when active_dev
 * is NULL): write k_dev[b] / v_dev[b] ([B][H][D], kv_dtype) to row m_b + (t_b mod n_b) of every
 * head (RSWA: overwriting output t_b - n_b once the ring is full, i.e. the oldest output is
 * evicted; deep dive N(t) code block, GeekNews model architecture section) or to row m_b + t_b
 * (FULL_CAUSAL), then t_b += 1. The counters live on the device, so calls need no host sync.
 * Errors: RSWA_E_INVALID; RSWA_E_CAPACITY when a FULL_CAUSAL sequence already holds max_steps
 * outputs, checked on the host before enqueuing as long as no call on this cache has used an
 * active mask. Once one has, the host no longer knows each t_b: a FULL_CAUSAL append past capacity
 * is then skipped on the device (that sequence's counter stays) and reported by rswa_cache_steps()
 * and rswa_cache_query(). */
rswa_status rswa_append_kv(rswa_cache* cache, const void* k_dev, const void* v_dev,
                           const uint8_t* active_dev /* [B] or NULL */, void* stream);

/* K2, decode attention (split-K flash decode + merge). For every active sequence b and head h:
 *   out[b][h] = softmax(scale * K_L q[b][h]) V_L
 * over the L_b = m_b + min(n_b, t_b) live rows (RSWA) or m_b + t_b rows (FULL_CAUSAL), i.e. the
 * prefix and the last min(n_b, t_b) appended outputs, the latest one included. This is attention
 * over the set N(t) = P u D_n(t) of the deep dive "Unlimited-OCR" (N(t) code block: the whole
 * prefix P plus the previous n outputs) and of GeekNews "Unlimited OCR", R-SWA section (every
 * token sees all reference tokens; output attention is limited to the previous n tokens, a
 * two-segment window of size m + n). q_dev: [B][H][D] of
 * kv_dtype; out_dev: [B][H][D] of out_dtype (rows of inactive sequences are left untouched).
 * softmax_scale <= 0 selects 1/sqrt(D). active_dev: [B] or NULL (all).
 * Errors: RSWA_E_INVALID (pointers, out_dtype, or a sequence with m_b = 0 that has had no append
 * yet: its key set is empty), RSWA_E_HIP. */
rswa_status rswa_decode_attn(rswa_cache* cache, const void* q_dev, void* out_dev, int32_t out_dtype,
                             float softmax_scale, const uint8_t* active_dev, void* stream);

/* K1 + K2 fused: one decode step in one launch. Equivalent to rswa_append_kv(k_dev, v_dev,
 * active_dev) followed by rswa_decode_attn(q_dev, ...), with the same results bit for bit: the
 * workgroup whose share of the key range holds the new row takes it from k_dev / v_dev and writes it
 * into the ring slot, so the evicted output is never read and no second launch is needed for the
 * append. Same arguments, layouts and errors as the two calls it replaces (RSWA_E_CAPACITY as in
 * rswa_append_kv). */
rswa_status rswa_decode_step(rswa_cache* cache, const void* q_dev, const void* k_dev,
                             const void* v_dev, void* out_dev, int32_t out_dtype,
                             float softmax_scale, const uint8_t* active_dev, void* stream);

/* K3, R-SWA-masked prefill / teacher-forced pass over packed sequences (bf16 MFMA, fp32 softmax).
 * The mask is R-SWA's during training: every token sees all reference (prefix) tokens and an
 * output token sees only its previous n output tokens (GeekNews "Unlimited OCR", R-SWA section;
 * deep dive "Unlimited-OCR", N(t) code block), over multi-page documents packed into 32K-token
 * sequences (GeekNews "Unlimited OCR", training section).
 * Sequence s occupies token rows [cu_seqlens[s], cu_seqlens[s+1]) of q/k/v/out (which must hold
 * cu_seqlens[nseq] rows: no row count is passed, so neither the host nor the kernels can check
 * it), its first m_s = prefix_len[s] tokens being the prefix. Query p (position within the
 * sequence) sees key k
 * iff   k < m_s  and (prefix_causal == 0 or p >= m_s or k <= p)          (the reference prefix)
 *    or m_s <= k <= p and p - k < n_s                                   (its own output window)
 * so prefix queries never see outputs; with n_s >= the sequence length this is causal attention
 * over the outputs (the full-causal comparison).
 * Numerics: scores and the softmax run in float32; P is rounded to bf16 for the P V product
 * (float32 accumulation) and each output row is divided by the sum of P as rounded, so its
 * weights sum to one. rswa_prefill_fwd writes the same output bit for bit.
 * q/k/v_dev: [total][H][D] bf16, token-major; out_dev: [total][H][D] of out_dtype.
 * cu_seqlens_dev: device int32 [nseq + 1], nondecreasing, cu_seqlens[0] = 0;
 * prefix_len_dev / window_dev: device int32 [nseq]; m_s in [0, S_s], n_s >= 1.
 * max_seqlen (host) must be >= every S_s; it sizes the launch grid.
 * Errors: RSWA_E_INVALID (host-checkable arguments), RSWA_E_UNSUPPORTED (head_dim), RSWA_E_HIP.
 * Device-side metadata cannot be checked before the launch. The kernels check it on the device:
 * a sequence longer than max_seqlen (its rows past max_seqlen are then not written), m_s > S_s,
 * S_s < 0 or n_s < 1 sets a per-device error word that rswa_prefill_check() reports.
 * No decode cache is written here: rswa_cache_create_from_prefill builds one from the same k / v
 * and cu_seqlens (host copy), so decoding can continue after the pass. */
rswa_status rswa_prefill_attn(const void* q_dev, const void* k_dev, const void* v_dev,
                              void* out_dev, int32_t out_dtype, const int32_t* cu_seqlens_dev,
                              const int32_t* prefix_len_dev, const int32_t* window_dev,
                              int32_t nseq, int32_t num_heads, int32_t head_dim, int32_t max_seqlen,
                              int32_t prefix_causal, float softmax_scale, void* stream);

/* K3 forward for training: rswa_prefill_attn plus the per-row log-sum-exp that the backward
 * needs. lse_dev: device float32 [total][H], written lse[p][h] = ln sum_{k visible} exp(scale q.k)
 * over the same visible set. Other arguments and errors as rswa_prefill_attn; lse_dev NULL is
 * RSWA_E_INVALID. */
rswa_status rswa_prefill_fwd(const void* q_dev, const void* k_dev, const void* v_dev,
                             void* out_dev, int32_t out_dtype, float* lse_dev,
                             const int32_t* cu_seqlens_dev, const int32_t* prefix_len_dev,
                             const int32_t* window_dev, int32_t nseq, int32_t num_heads,
                             int32_t head_dim, int32_t max_seqlen, int32_t prefix_causal,
                             float softmax_scale, void* stream);

/* Backward of the teacher-forced pass (the pages train the R-SWA decoder on packed 32K-token
 * sequences: GeekNews "Unlimited OCR", training section; deep dive "Unlimited-OCR", training
 * setup). With P the masked softmax of rswa_prefill_attn, O = P V and the output gradient dO:
 *   delta_p = sum_d dO[p][d] O[p][d],  dS = P * (dO V^T - delta),
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
 * Packed documents: each cu_seqlens segment is one prefix + output document with its own m and n;
 * no query sees a key of another segment.
 * q/k/v_dev, dout_dev: [total][H][D] bf16; out_dev: the forward output [total][H][D] of out_dtype;
 * lse_dev: float32 [total][H] from rswa_prefill_fwd with the same arguments.
 * work_dev: caller-owned float32 work array of 2 * total_tokens * H values, overwritten with
 * [0][h][token] = lse * log2(e) and [1][h][token] = -delta (delta = the row sum of dO * O).
 * dq/dk/dv_dev: [total][H][D] of grad_dtype, overwritten on every row of every segment (rows
 * beyond cu_seqlens[nseq] are not touched). total_tokens (host) = rows of these arrays, at least
 * cu_seqlens[nseq]; the work array covers all of them.
 * The library allocates nothing; all work is enqueued on `stream`.
 * Errors: as rswa_prefill_attn, plus RSWA_E_INVALID for NULL dout/lse/work/dq/dk/dv, a bad
 * grad_dtype or total_tokens < 0. Device-side metadata is checked on the device as in
 * rswa_prefill_attn (a sequence past max_seqlen leaves gradient rows unwritten) and reported by
 * rswa_prefill_check(). */
rswa_status rswa_prefill_bwd(const void* q_dev, const void* k_dev, const void* v_dev,
                             const void* out_dev, int32_t out_dtype, const void* dout_dev,
                             const float* lse_dev, float* work_dev, void* dq_dev, void* dk_dev,
                             void* dv_dev, int32_t grad_dtype, const int32_t* cu_seqlens_dev,
                             const int32_t* prefix_len_dev, const int32_t* window_dev,
                             int32_t nseq, int32_t total_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t max_seqlen, int32_t prefix_causal,
                             float softmax_scale, void* stream);

/* rswa_prefill_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid hipMalloc): the same computation, results and errors,
 * without the work array. Its work rows live in a device array inside the library (held by each
 * device the library runs on until the process ends; nothing is allocated or freed by the call),
 * so total_tokens * num_heads must not exceed 1048576 (RSWA_E_INVALID otherwise, checked before
 * anything is enqueued). Every call on one device uses that device's array: calls that overlap on
 * one device (other streams, other threads) race and must be ordered by the caller. */
rswa_status rswa_prefill_bwd_noalloc(const void* q_dev, const void* k_dev, const void* v_dev,
                                     const void* out_dev, int32_t out_dtype, const void* dout_dev,
                                     const float* lse_dev, void* dq_dev, void* dk_dev,
                                     void* dv_dev, int32_t grad_dtype,
                                     const int32_t* cu_seqlens_dev,
                                     const int32_t* prefix_len_dev, const int32_t* window_dev,
                                     int32_t nseq, int32_t total_tokens, int32_t num_heads,
                                     int32_t head_dim, int32_t max_seqlen,
                                     int32_t prefix_causal, float softmax_scale, void* stream);

/* Graph-captured step loop (fused append + decode steps replayed from a HIP graph). Capture
 * `steps` consecutive rswa_decode_step launches of `cache` (no active mask) into a HIP graph:
 * step i of a replay reads q / k / v from slot i of q_slots / k_slots / v_slots (each [steps][B][H]
 * [D] of kv_dtype, caller-owned) and writes slot i of out_slots ([steps][B][H][D] of out_dtype).
 * The caller fills the input slots before each replay. steps must be even (the step counters are
 * double-buffered, so an even count returns them to the same parity) and at most 4096. The work
 * split of each step is fixed at capture; the kernels still derive every row range from the
 * device-side step counters, so replays at any later step are correct. When all sequences share
 * m, capacity and step count and no active mask has been used, a second copy of the steps is
 * captured that reads the one shared count (steps_in[0]) instead of every sequence's and then
 * follows the plan an eager step takes (no work table); a replay uses it while that still holds,
 * the general copy after an active mask. Capture uses a private stream and enqueues nothing; the
 * graph may be launched on any stream of the cache's device.
 * Errors: RSWA_E_INVALID, RSWA_E_HIP (capture or instantiation), RSWA_E_INTERNAL. */
typedef struct rswa_step_graph rswa_step_graph; /* opaque; owned by the library */
rswa_status rswa_step_graph_create(rswa_cache* cache, int32_t steps, const void* q_slots_dev,
                                   const void* k_slots_dev, const void* v_slots_dev,
                                   void* out_slots_dev, int32_t out_dtype, float softmax_scale,
                                   rswa_step_graph** out);

/* Replay the captured steps on `stream` (appends `steps` outputs to every sequence). Eager calls
 * on the same cache may come between replays: when they leave the step counters in the other
 * of the two counter buffers, the launch first enqueues a 4*B-byte device copy into the buffer
 * the graph reads. In FULL_CAUSAL mode RSWA_E_CAPACITY if a replay would pass max_steps (checked
 * on the host while no active mask has been used on the cache, else on the device). */
rswa_status rswa_step_graph_launch(rswa_step_graph* graph, void* stream);

/* Release the graph (does not synchronize; the caller must not destroy it while a replay that
 * it enqueued may still be pending). NULL is accepted. Every graph of a cache must be destroyed
 * before the cache (rswa_cache_destroy refuses otherwise). */
rswa_status rswa_step_graph_destroy(rswa_step_graph* graph);

/* Copy the per-sequence step counters t_b to steps_host [B]. BLOCKS until `stream` has passed
 * all prior work. Returns RSWA_E_CAPACITY if a FULL_CAUSAL append past max_steps was skipped on
 * the device since creation (the counters are still copied). */
rswa_status rswa_cache_steps(rswa_cache* cache, int32_t* steps_host, void* stream);

/* Storage base pointer and layout of a live cache (host only; see rswa_cache_plan).
 * Any output pointer may be NULL. */
rswa_status rswa_cache_info(const rswa_cache* cache, void** storage_dev,
                            int64_t* seq_offset_host /* [B] */, int32_t* rows_host /* [B] */);

/* Decode work split. By default, when no active mask has been given and all sequences hold equal
 * key ranges: a batch whose ranges about fill one round of resident workgroups gets one workgroup
 * per (b, h) range; a smaller batch has every range cut into k = min(resident workgroups / ranges,
 * rows / 64) >= 2 equal pieces. Otherwise the concatenated key ranges are cut into equal
 * contiguous pieces, one per resident workgroup. A range split over pieces is merged inside the
 * same launch by its last piece to finish. A step whose live rows exceed the last-level cache
 * (256 MiB on MI355X; none of them would still be there at the next step) reads them with
 * non-temporal loads and counts at most three resident workgroups per CU, unless the cache has a
 * paged prefix (its shared pool rows are reused). chunk_rows (> 0) sets the fewest rows a piece
 * may hold and grid_blocks (> 0) the number of pieces; either one forces the contiguous-piece
 * layout. 0
 * restores the automatic choice. Results depend on these only through float32 summation order.
 * Host only. */
rswa_status rswa_cache_set_decode_split(rswa_cache* cache, int32_t chunk_rows, int32_t grid_blocks);

/* What the next decode launch on this cache does when no active mask is given (appending = 1 for
 * rswa_decode_step, 0 for rswa_decode_attn): the workgroups of the decode kernel and the number of
 * kernel launches (1; 0 when there is nothing to decode). Host only. */
rswa_status rswa_cache_decode_plan(const rswa_cache* cache, int32_t appending,
                                   int32_t* grid_blocks, int32_t* launches);

/* Release the cache: BLOCKS until the whole device is idle (the cache may have been used on any
 * stream, and freeing device memory waits for the device in any case), then frees library-owned
 * memory. NULL is accepted. Caller-owned storage is left as is. RSWA_E_INVALID (and nothing is
 * released) while a step graph of this cache still exists. */
rswa_status rswa_cache_destroy(rswa_cache* cache);

/* Inspection of a live cache in one call (for tests and snapshots): the storage base pointer and,
 * per sequence b, the element offsets of its K block and V block (K[b][h][r][i] at
 * k_offset[b] + (h * R_b + r) * D + i, V likewise from v_offset[b]), R_b, and the step counters
 * t_b. In a paged cache the storage holds output rows only: storage row r is cache row m_b + r
 * (R_b = n_b or max_steps_b), the prefix rows being in the caller's pool. Layout outputs are
 * host-only; when steps_host is not NULL the call BLOCKS until `stream`
 * has passed all prior work and returns RSWA_E_CAPACITY as rswa_cache_steps() does. Any output
 * pointer may be NULL. */
rswa_status rswa_cache_query(rswa_cache* cache, void** storage_dev,
                             int64_t* k_offset_host /* [B] */, int64_t* v_offset_host /* [B] */,
                             int32_t* rows_host /* [B] */, int32_t* steps_host /* [B] */,
                             void* stream);

/* Report the metadata errors that prefill and backward launches on the current device found on
 * the device (see rswa_prefill_attn) since the last call, and clear them. BLOCKS until `stream`
 * has passed all prior work (launches on other streams must be complete too). RSWA_E_INVALID if
 * any launch found an error, else RSWA_OK. One error word per device: concurrent prefill calls
 * on one device share it. */
rswa_status rswa_prefill_check(void* stream);

/* Human-readable name of a status code (static string). */
const char* rswa_status_str(int32_t status);

/* Detail message of the last error returned on the calling thread (static per thread; empty
 * string if none). */
const char* rswa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RSWA_H */
