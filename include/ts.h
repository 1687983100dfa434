/*
 * ts.h — C ABI of the TokenSelect decode-time hot path on MI355X (gfx950).
 *
 * What the library computes (TokenSelect README, "Key Takeaways"; GrooveSquid
 * summary of the TokenSelect paper, "Medium Difficulty Summary"):
 *   1. per-head criticality of every cached token: s[h,j] = scale * <q[h], K[j, kv(h)]>,
 *      with grouped-query attention, kv(h) = h / (Hq / Hkv);
 *   2. per-head soft voting: softmax of s[h,:] over all N cached tokens, summed
 *      over the Hq heads, v[j] = sum_h softmax_h(s)[j];
 *   3. top-k: the k_eff = min(k, N) tokens with the largest votes, ties to the
 *      lower index, returned ascending and padded with -1 up to k;
 *   4. sparse attention: every query head attends, with the same scale, over
 *      the selected rows only (softmax renormalised over them);
 *   5. Selection Cache: when the cosine of the flattened query with the stored
 *      query exceeds theta, the stored selection is reused and steps 1-3 skip.
 *   plus a chunked-prefill variant of 1-3 in which query i of a chunk sits at
 *   position q_pos0 + i and sees keys 0 .. q_pos0 + i only.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked [host]. The caller owns every
 *     input, output and workspace buffer; the library never frees them.
 *   - Calls are asynchronous on `stream` (a hipStream_t, NULL = default stream)
 *     and never synchronise, except ts_sel_cache_create/destroy/stats, which
 *     say so.
 *   - The library allocates nothing on these calls, except inside
 *     ts_sel_cache_create (freed by ts_sel_cache_destroy).
 *   - All argument checks run on the host before anything is enqueued. On an
 *     error nothing is enqueued, no output is touched, and ts_last_error()
 *     describes the problem. A failed kernel launch returns TS_ERR_HIP.
 *   - Per-sequence lengths live on the device and are not checked on the host:
 *     0 <= seq_lens[b] <= max_len is the caller's contract. A length of 0 gives
 *     zero outputs and an all -1 selection.
 *   - Entry points are re-entrant; calls that share a workspace or a
 *     ts_sel_cache must be ordered on one stream.
 *
 * Supported shapes: head_dim 64 or 128; dtype fp32 or bf16 (q, K and V share
 * it; accumulation is fp32); num_kv_heads divides num_q_heads; num_kv_heads <= 64 for
 * bf16, <= 32 for fp32 with head_dim 64 and <= 16 for fp32 with head_dim 128 (one scoring
 * work-group holds a token's rows of every KV head); other shapes return TS_ERR_UNSUPPORTED.
 * Size limits (TS_ERR_UNSUPPORTED beyond them, so that every size the planner
 * derives fits its integer type): max_len, n_ctx, chunk, k and row_stride
 * <= 2^30; batch and max_batch <= 2^20; top-k rows <= 2^24; num_q_heads <= 256.
 */
#ifndef TS_H
#define TS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TS_ABI_VERSION 1

typedef enum ts_status {
  TS_OK = 0,
  TS_ERR_INVALID_ARG = 1,   /* null pointer, bad size or inconsistent shape       */
  TS_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim, head counts)  */
  TS_ERR_WORKSPACE = 3,     /* workspace smaller than the matching *_workspace_size */
  TS_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed         */
} ts_status;

typedef enum ts_dtype { TS_F32 = 0, TS_BF16 = 1 } ts_dtype;

/* Shape and memory layout of one layer's KV cache.
 *   contiguous (page_size == 0): K and V are [batch][max_len][num_kv_heads][head_dim];
 *   paged      (page_size  > 0): K and V are pools [num_pages][page_size][num_kv_heads][head_dim]
 *     and token j of sequence b lives in pool page page_table[b * page_table_stride + j / page_size],
 *     slot j % page_size. page_size must be a power of two. Every page that holds a token
 *     below seq_lens[b] must map to a pool page that exists (0 <= entry < pool pages): the
 *     scoring and attention kernels read those entries unchecked, and a bad entry is an
 *     out-of-bounds device read. Entries past the sequence are never read by them.       */
typedef struct ts_kv_layout {
  int32_t num_q_heads;        /* Hq                                                  */
  int32_t num_kv_heads;       /* Hkv, divides Hq                                     */
  int32_t head_dim;           /* d: 64 or 128                                        */
  int32_t dtype;              /* ts_dtype of q, K and V                              */
  float   scale;              /* logit scale; <= 0 selects 1/sqrt(head_dim)          */
  int32_t page_size;          /* 0 = contiguous                                      */
  int32_t max_len;            /* token capacity of one sequence (> 0)                */
  int32_t page_table_stride;  /* int32 entries per page-table row (paged only)       */
} ts_kv_layout;

int32_t     ts_abi_version(void);
/* Static string for a ts_status value. */
const char* ts_status_string(int32_t status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char* ts_last_error(void);

/* ---------------------------------------------------------------------------
 * ts_score — steps 1-2 (scoring and per-head soft voting) for one query per
 * sequence.
 *   q        [batch][Hq][d] (dtype)
 *   k_cache  see ts_kv_layout; page_table [batch][page_table_stride] int32 or NULL
 *   seq_lens [batch] int32
 *   votes    [batch][max_len] fp32 out; entries j >= seq_lens[b] are left unwritten.
 *            Each row sums to Hq (up to fp32 rounding).
 *   ws       scratch of at least ts_score_workspace_size bytes (256-byte aligned)
 * ------------------------------------------------------------------------- */
ts_status ts_score_workspace_size(const ts_kv_layout* layout /*[host]*/, int32_t batch,
                                  size_t* bytes /*[host] out*/);
ts_status ts_score(const ts_kv_layout* layout /*[host]*/, int32_t batch, const void* q,
                   const void* k_cache, const int32_t* page_table, const int32_t* seq_lens,
                   float* votes, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ts_topk — step 3 on `rows` independent rows.
 *   votes    [rows][row_stride] fp32; only the first row_lens[r] entries of a row count
 *   row_lens [rows] int32 (device), 0 <= row_lens[r] <= row_stride
 *   idx      [rows][k] int32 out: the min(k, row_lens[r]) largest entries, ties to the
 *            lower index, ascending, then -1 padding. Exact (a radix select on the
 *            order-preserving integer image of the floats; -0.0 equals +0.0;
 *            subnormals are ordered; rows must not hold NaN).
 *   k >= 1.
 * ------------------------------------------------------------------------- */
ts_status ts_topk_workspace_size(int32_t rows, int32_t row_stride, int32_t k,
                                 size_t* bytes /*[host] out*/);
ts_status ts_topk(int32_t rows, int32_t row_stride, const float* votes, const int32_t* row_lens,
                  int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ts_sparse_attend — step 4: attention of every query head over the rows a
 * selection names.
 *   idx  [batch][k] int32: token indices < seq_lens[b]; negative entries are skipped
 *        (any order; duplicates count twice).
 *   out  [batch][Hq][d] fp32. A sequence with no valid index gets zeros.
 *   Numerics: scores, softmax and sums in fp32 (base 2). With bf16 rows both
 *   products run on the matrix cores: the softmax weights enter the second
 *   one as two bf16 parts (about 16 significant bits); outputs stay within
 *   2e-5 of the fp64 reference, relative to the head's largest output, in the
 *   parity tests. ts_dense_attend and the
 *   attention inside ts_decode_step, ts_sparse_attend_prefill and
 *   ts_quest_attend share this kernel.
 * ------------------------------------------------------------------------- */
ts_status ts_sparse_attend_workspace_size(const ts_kv_layout* layout /*[host]*/, int32_t batch,
                                          int32_t k, size_t* bytes /*[host] out*/);
ts_status ts_sparse_attend(const ts_kv_layout* layout /*[host]*/, int32_t batch, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* page_table,
                           const int32_t* seq_lens, const int32_t* idx, int32_t k, float* out,
                           void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ts_append_kv — the decode loop's cache growth: sequence b's new K and V rows
 * (k_new, v_new [batch][Hkv][d], the cache's dtype) are written at position
 * seq_lens[b], then seq_lens[b] is incremented on the device. Everything stays
 * on the stream, so "append, then ts_decode_step" can be captured once in a
 * HIP graph and replayed for every token.
 *   Contiguous caches: a position >= layout.max_len is skipped (length kept).
 *   Paged caches: the page holding the position must already be in
 *   page_table (a negative entry is skipped likewise).
 * ------------------------------------------------------------------------- */
ts_status ts_append_kv(const ts_kv_layout* layout /*[host]*/, int32_t batch, const void* k_new,
                       const void* v_new, void* k_cache, void* v_cache,
                       const int32_t* page_table, int32_t* seq_lens, void* stream);

/* ---------------------------------------------------------------------------
 * Quest-style page selection, an alternative selector on paged KV ("Quest:
 * Query-Aware Sparsity for Efficient Long-Context LLM Inference", arXiv
 * 2406.10774: abstract and "Method Overview" point 4). Each KV page keeps the
 * channel-wise min and max of its keys; a page's score for query head h is
 * scale * sum_c max(q_hc * min_c, q_hc * max_c), an upper bound of its logits;
 * a KV head scores a page by the largest bound over its group's query heads
 * and keeps its own top k_pages pages; attention then runs per KV head over
 * the tokens of its pages.
 * Paged layouts only; G = Hq/Hkv <= 8 and Hkv <= 16 * 128 / d, otherwise
 * TS_ERR_UNSUPPORTED.
 *
 * ts_quest_meta — per-page key extremes.
 *   meta [P][Hkv][2][d] in the cache dtype, indexed by pool page: row 0 the
 *        channel minima, row 1 the maxima, over the page's existing tokens
 *        (< seq_lens[b]); exact (min/max of stored values).
 *   last_page_only = 0: every page of every sequence; != 0: only the page
 *        holding token seq_lens[b]-1 (call after ts_append_kv).
 *   Pages outside a sequence and unmapped (negative) entries are left alone.
 * ------------------------------------------------------------------------- */
ts_status ts_quest_meta(const ts_kv_layout* layout /*[host]*/, int32_t batch, const void* k_cache,
                        const int32_t* page_table, const int32_t* seq_lens,
                        int32_t last_page_only, void* meta, void* stream);

/* ts_quest_select — page scores, then the top k_pages pages per (sequence, KV head).
 *   scores   optional out [batch][Hkv][n_pages] fp32, n_pages = ceil(max_len /
 *            page_size); entries past a sequence's pages are unspecified.
 *            NULL keeps them in the workspace.
 *   page_idx [batch][Hkv][k_pages] int32 out: logical page numbers, ascending,
 *            the min(k_pages, pages of b) best (ties to the lower page), -1 padded.
 * ------------------------------------------------------------------------- */
ts_status ts_quest_select_workspace_size(const ts_kv_layout* layout /*[host]*/, int32_t batch,
                                         int32_t k_pages, size_t* bytes /*[host] out*/);
ts_status ts_quest_select(const ts_kv_layout* layout /*[host]*/, int32_t batch, const void* q,
                          const void* meta, const int32_t* page_table, const int32_t* seq_lens,
                          int32_t k_pages, float* scores, int32_t* page_idx, void* ws,
                          size_t ws_bytes, void* stream);

/* ts_quest_attend — every query head attends over the existing tokens of its
 * KV head's pages (softmax renormalised over them); negative page entries are
 * skipped; a head with no token gets zeros.
 *   page_idx [batch][Hkv][k_pages] as from ts_quest_select; out [batch][Hq][d] fp32.
 * ------------------------------------------------------------------------- */
ts_status ts_quest_attend_workspace_size(const ts_kv_layout* layout /*[host]*/, int32_t batch,
                                         int32_t k_pages, size_t* bytes /*[host] out*/);
ts_status ts_quest_attend(const ts_kv_layout* layout /*[host]*/, int32_t batch, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* page_table,
                          const int32_t* seq_lens, const int32_t* page_idx, int32_t k_pages,
                          float* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ts_sparse_attend_prefill — step 4 for a prefill chunk: query i (position
 * q_pos0 + i) attends, with every head, over the rows its own selection names
 * (TokenSelect README, "Key Takeaways": attention over the selected tokens).
 *   q        [chunk][Hq][d], k_cache / v_cache [n_ctx][Hkv][d] contiguous
 *            (layout.page_size 0, layout.max_len >= n_ctx), same dtype
 *   idx      [chunk][k] int32: row i's indices, each < q_pos0 + i + 1 (others,
 *            and negative entries, are skipped), e.g. from ts_select_prefill
 *   out      [chunk][Hq][d] fp32; a row with no valid index gets zeros.
 *   Requires q_pos0 >= 0 and q_pos0 + chunk <= n_ctx.
 * ------------------------------------------------------------------------- */
ts_status ts_sparse_attend_prefill_workspace_size(const ts_kv_layout* layout /*[host]*/,
                                                  int32_t chunk, int32_t k,
                                                  size_t* bytes /*[host] out*/);
ts_status ts_sparse_attend_prefill(const ts_kv_layout* layout /*[host]*/, int32_t chunk,
                                   int32_t q_pos0, const void* q, const void* k_cache,
                                   const void* v_cache, int32_t n_ctx, const int32_t* idx,
                                   int32_t k, float* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ts_dense_attend — the comparison arm of the method: ordinary softmax
 * attention of every query head over all seq_lens[b] cached tokens (the
 * TokenSelect README's "Result" quotes its speedups against full attention).
 * Same split-K kernels as ts_sparse_attend with token j in position j, so the
 * output equals ts_sparse_attend over idx = 0 .. seq_lens[b]-1.
 *   out  [batch][Hq][d] fp32; an empty sequence gets zeros.
 * ------------------------------------------------------------------------- */
ts_status ts_dense_attend_workspace_size(const ts_kv_layout* layout /*[host]*/, int32_t batch,
                                         size_t* bytes /*[host] out*/);
ts_status ts_dense_attend(const ts_kv_layout* layout /*[host]*/, int32_t batch, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* page_table,
                          const int32_t* seq_lens, float* out, void* ws, size_t ws_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------
 * Selection Cache state for up to max_batch sequences of one layer (step 5).
 *   compare_mode 0: compare with the previous step's query (stored every step);
 *   compare_mode 1: compare with the query of the last miss (the anchor).
 * Per sequence it keeps the stored query (fp32, Hq*d), the last selection
 * ([k] int32), a valid flag and hit/miss counters, all in device memory,
 * plus per-head fp64 sums that a decode step's scoring kernel fills and its
 * last kernel clears (the softmax denominators of step 2), so one cache must
 * not serve two decode steps in flight at once.
 * A step hits when the state is valid and cos(q, stored) > theta (strict; the
 * cosine is accumulated in fp64 over the flattened Hq*d query; a zero norm
 * never hits). The first step, a step after reset and a step on an empty
 * sequence miss; an empty sequence leaves the state invalid.
 * ------------------------------------------------------------------------- */
typedef struct ts_sel_cache ts_sel_cache;

/* Allocates the device state (hipMalloc) and zeroes it; synchronises the device.
 * head_dim must be 64 or 128 (TS_ERR_UNSUPPORTED otherwise). */
ts_status ts_sel_cache_create(int32_t max_batch, int32_t num_q_heads, int32_t head_dim, int32_t k,
                              int32_t compare_mode, ts_sel_cache** out /*[host]*/);
/* Marks sequences invalid and clears their hit/miss counters, so that their
 * next step misses (TokenSelect README, "Key Takeaways", third point: the
 * Selection Cache is state of one sequence; a batch slot that a new sequence
 * takes over must not reuse the previous occupant's query or selection).
 *   seq_mask  [max_batch] int32 (device) or NULL: sequence b is reset where
 *             seq_mask[b] != 0; NULL resets every sequence.
 * One small kernel on `stream` (no memset and no allocation, so the call can
 * be captured in a HIP graph); asynchronous like a decode step. */
ts_status ts_sel_cache_reset(ts_sel_cache* cache, const int32_t* seq_mask, void* stream);
/* Frees the device state; synchronises the device. */
ts_status ts_sel_cache_destroy(ts_sel_cache* cache);
/* Copies hit and miss counts of sequences 0..n-1 to host arrays; synchronises `stream`. */
ts_status ts_sel_cache_stats(ts_sel_cache* cache, int32_t n, int64_t* hits /*[host]*/,
                             int64_t* misses /*[host]*/, void* stream);

/* ---------------------------------------------------------------------------
 * ts_decode_step — one decode step of one layer for `batch` sequences:
 * Selection-Cache check; on a miss steps 1-3 and a new stored selection; then
 * step 4 with the current selection; then the state update.
 *   q, k_cache, v_cache, page_table, seq_lens as in ts_score / ts_sparse_attend
 *   theta    cosine threshold (a hit needs cos > theta)
 *   out      [batch][Hq][d] fp32
 *   idx_out  [batch][k] int32 or NULL: the selection used this step
 *   hit_out  [batch] int32 or NULL: 1 where the stored selection was reused
 * The layout's num_q_heads and head_dim must match the cache; batch <= max_batch.
 * Each head's softmax denominator (step 2) is summed in fp64 by device
 * atomics in arrival order, so repeated calls on the same inputs agree up to
 * the last bits of that sum (an fp32 vote could move by one ulp, rarely).
 * ------------------------------------------------------------------------- */
ts_status ts_decode_step_workspace_size(const ts_kv_layout* layout /*[host]*/, int32_t batch,
                                        int32_t k, size_t* bytes /*[host] out*/);
ts_status ts_decode_step(ts_sel_cache* cache, const ts_kv_layout* layout /*[host]*/,
                         int32_t batch, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* page_table, const int32_t* seq_lens, double theta,
                         float* out, int32_t* idx_out, int32_t* hit_out, void* ws,
                         size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ts_decode_step_noalloc — ts_decode_step for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, kernels and
 * results as ts_decode_step, without ws/ws_bytes: the workspace is a static
 * device array of TS_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one
 * per GPU, held until the process ends; its address is looked up when a
 * ts_sel_cache is created on that GPU. The call allocates nothing.
 *   Steps whose ts_decode_step_workspace_size exceeds TS_NOALLOC_SCRATCH_BYTES
 *   return TS_ERR_WORKSPACE (e.g. one Qwen2-7B-shape layer of 131072 tokens
 *   needs about 17 MB and fits; batches of several such sequences do not).
 *   The calling thread's current device must be the cache's device.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (other streams, other threads) race and must be ordered by the
 *   caller. A call leaves the array holding its intermediates; each call
 *   clears what it needs cleared itself, in its kernels.
 * ------------------------------------------------------------------------- */
#define TS_NOALLOC_SCRATCH_BYTES (32u << 20)
ts_status ts_decode_step_noalloc(ts_sel_cache* cache, const ts_kv_layout* layout /*[host]*/,
                                 int32_t batch, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* page_table,
                                 const int32_t* seq_lens, double theta, float* out,
                                 int32_t* idx_out, int32_t* hit_out, void* stream);

/* ---------------------------------------------------------------------------
 * ts_score_prefill — steps 1-2 for a chunk of `chunk` consecutive queries
 * (bf16 MFMA for the query-key products; fp32 softmax and votes).
 *   q        [chunk][Hq][d] bf16, query i at absolute position q_pos0 + i
 *   k_cache  [n_ctx][Hkv][d] bf16 contiguous (layout.page_size must be 0,
 *            layout.dtype TS_BF16, layout.max_len >= n_ctx)
 *   votes    [chunk][n_ctx] fp32 out: row i holds the soft vote over keys
 *            0 .. q_pos0 + i; entries past that are written as 0.
 *   Requires q_pos0 >= 0 and q_pos0 + chunk <= n_ctx.
 *   Built for bf16, head_dim 64 or 128, 1 to 8 query heads per KV head (laid
 *   out as 1, 2, 4 or 8 slots; unused slots are masked) and at most 8 KV
 *   heads; other shapes return TS_ERR_UNSUPPORTED. The workspace size does
 *   not depend on q_pos0.
 * ts_select_prefill additionally runs step 3 on every row:
 *   idx      [chunk][k] int32 out (row i selects from its q_pos0 + i + 1 keys).
 * ------------------------------------------------------------------------- */
ts_status ts_score_prefill_workspace_size(const ts_kv_layout* layout /*[host]*/, int32_t chunk,
                                          int32_t n_ctx, int32_t k, size_t* bytes /*[host] out*/);
ts_status ts_score_prefill(const ts_kv_layout* layout /*[host]*/, int32_t chunk, int32_t q_pos0,
                           const void* q, const void* k_cache, int32_t n_ctx, float* votes,
                           void* ws, size_t ws_bytes, void* stream);
ts_status ts_select_prefill(const ts_kv_layout* layout /*[host]*/, int32_t chunk, int32_t q_pos0,
                            const void* q, const void* k_cache, int32_t n_ctx, int32_t k,
                            float* votes, int32_t* idx, void* ws, size_t ws_bytes, void* stream);


/* ---------------------------------------------------------------------------
 * Kernel-level timing for measurement harnesses. While enabled, every kernel
 * launch of every entry point is bracketed by two HIP events recorded on the
 * launch's own stream, so the device-side duration of each kernel can be read
 * back per kernel kind. Enabling/disabling is a process-wide host switch: do
 * not toggle it while another thread launches. Events add a little queue
 * overhead, so time throughput with it off.
 *   ts_profile_read synchronizes every pending event and returns the number of
 *   launches and their summed duration (ms) for kernel kind `id`
 *   (0 <= id < ts_profile_num_kernels(); names from ts_profile_kernel_name).
 * ------------------------------------------------------------------------- */
int32_t     ts_profile_num_kernels(void);
const char* ts_profile_kernel_name(int32_t id);
ts_status   ts_profile_enable(int32_t on);
ts_status   ts_profile_reset(void);
ts_status   ts_profile_read(int32_t id, int64_t* launches /*[host]*/, double* total_ms /*[host]*/);

#ifdef __cplusplus
}
#endif

#endif /* TS_H */
