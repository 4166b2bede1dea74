/*
 * adamas.h -- C ABI of the MI355X (gfx950) ADAMAS decode path.
 *
 * The method (ADAMAS article, www.lnwmold.com/news/826806): rotate queries
 * and keys by a Hadamard matrix over the head dimension (§2.1), bucket each
 * rotated vector into 2-bit codes at -0.5*absmax, 0, +0.5*absmax (§2.2), keep
 * the keys' codes packed four per byte in a compact cache (§3.1), score a
 * query against every cached key by Manhattan distance between codes (§2.3),
 * keep a per-head token budget of the closest keys (§5.2), and run exact
 * softmax attention over only those K/V rows (§6).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - All tensor arguments are DEVICE pointers, borrowed for the duration of
 *    the enqueued work; the library never allocates, frees or retains them.
 *    Tensors are dense, row-major, in the layouts given per call, and must be
 *    16-byte aligned.
 *  - Element types: ADAMAS_F32 (binary32) or ADAMAS_BF16 (bfloat16).
 *  - head_dim must be 64, 128 or 256.
 *  - Calls enqueue work on `stream` (0 = the null stream) and return without
 *    waiting; results are visible after a stream synchronisation or event.
 *    No call synchronises the device, so calls may be captured into a graph.
 *  - Errors: every argument is checked on the host BEFORE anything is
 *    enqueued; on any non-zero status nothing was enqueued.  A launch failure
 *    reported by the runtime after enqueueing returns ADAMAS_ERR_DEVICE.
 *  - Workspace: calls that take (ws, ws_bytes) need a device buffer of at
 *    least adamas_workspace_bytes(...) bytes whose first ADAMAS_WS_CTRL_BYTES
 *    bytes are zero before the first call that uses it (allocate it zeroed).
 *    Every call that completes leaves those bytes zero again, so one
 *    workspace can be reused by any sequence of calls ON ONE STREAM; calls
 *    that may overlap in time need separate workspaces.
 *  - Codes: a row of d dims is d/4 bytes; code i sits in byte i/4 at bits
 *    (7 - 2*(i%4)) .. (6 - 2*(i%4)), i.e. the first code of a byte in its top
 *    two bits.  Code values: 0 if y < -a/2, 1 if y < 0, 2 if y < a/2, else 3,
 *    with y the unnormalised Sylvester-order Hadamard transform of the vector
 *    in binary32 and a = max|y_i| over the vector's group of 128 dimensions
 *    (the article's grouped quantization, §2.2): the whole vector at
 *    head_dim <= 128, each half separately at head_dim 256.
 */
#ifndef ADAMAS_H
#define ADAMAS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADAMAS_VERSION 100 /* 1.0.0 */

/* Leading bytes of a workspace that must be zero before its first use:
 * arrival counters, then the status word. */
#define ADAMAS_WS_CTRL_BYTES 65792

/* Byte offset in a workspace of a u32 status word.  A decode step that ran
 * with group waits (ADAMAS_DECODE_GROUP_WAIT) and found a wait exceeding its
 * bound (adamas_set_wait_polls) sets it to a nonzero value; that call's
 * outputs are then invalid, while its control bytes are still left zero, so
 * the workspace stays usable.  The library never clears the word: a caller
 * that may run group waits reads it after synchronising the stream (the
 * Python binding's Workspace.status()) and writes zero to re-arm it. */
#define ADAMAS_WS_STATUS_OFFSET 65536

typedef enum {
    ADAMAS_OK = 0,
    ADAMAS_ERR_INVALID = 1,     /* null/misaligned pointer, bad size or range */
    ADAMAS_ERR_UNSUPPORTED = 2, /* head_dim not 64/128/256, unknown dtype, limits */
    ADAMAS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than needed */
    ADAMAS_ERR_DEVICE = 4       /* the HIP runtime reported a launch error */
} adamas_status;

typedef enum { ADAMAS_F32 = 0, ADAMAS_BF16 = 1 } adamas_dtype;

/* How adamas_decode_step coordinates the workgroups that scan the chunks of
 * one KV head (see adamas_set_decode_mode). */
typedef enum {
    ADAMAS_DECODE_AUTO = 0,
    ADAMAS_DECODE_LAST_ARRIVAL = 1,
    ADAMAS_DECODE_GROUP_WAIT = 2,
    ADAMAS_DECODE_SPLIT = 3
} adamas_decode_mode;

typedef enum {
    ADAMAS_OP_SELECT_TOPK = 0,
    ADAMAS_OP_SPARSE_ATTEND = 1,
    ADAMAS_OP_DECODE_STEP = 2
} adamas_op;

/*
 * Encode keys (or queries) into 2-bit codes: §2.1 rotation, §2.2 bucketing,
 * §3.1 packing (the article's CompressedKVCache.update).
 *
 *   x          [batch][heads][n][head_dim] elements of `dtype`.
 *   codes      [batch][heads][cap][head_dim/4] bytes; rows [pos, pos+n) of
 *              each (batch, head) are written, no other byte is touched.
 *   x_copy_dst nullable; if set, [batch][heads][cap][head_dim] elements of
 *              `dtype` receiving a verbatim copy of x at rows [pos, pos+n)
 *              (append the raw keys to a K cache in the same pass).
 * A query vector is encoded with n = 1, cap = 1, pos = 0.
 * Requires batch, heads >= 1, n >= 0, 0 <= pos, pos + n <= cap.
 * n = 0 is a no-op that returns ADAMAS_OK.
 */
int adamas_encode_keys(const void *x, int dtype, int batch, int heads, int64_t n,
                       int head_dim, uint8_t *codes, int64_t cap, int64_t pos,
                       void *x_copy_dst, hipStream_t stream);

/*
 * Manhattan distance between query codes and the first n_ctx cached key
 * codes (§2.3): dist[b][hq][t] = sum_i |qc_i - kc_i|, in 0 .. 3*head_dim.
 * Query head hq reads KV head hq / (Hq / Hkv).
 *
 *   q_codes [B][Hq][head_dim/4] bytes.
 *   k_codes [B][Hkv][cap][head_dim/4] bytes.
 *   dist    [B][Hq][n_ctx] uint16.
 * Requires Hq % Hkv == 0, 0 <= n_ctx <= cap; n_ctx = 0 is a no-op.
 */
int adamas_score(const uint8_t *q_codes, const uint8_t *k_codes, int B, int Hq,
                 int Hkv, int head_dim, int64_t cap, int64_t n_ctx,
                 uint16_t *dist, hipStream_t stream);

/*
 * Token budget (§5.2): per (b, hq) keep the min(budget, n_ctx) tokens with
 * the smallest (distance, token index) -- the lowest index wins a tie --
 * and write their indices in ascending order, padding with -1.
 *
 *   dist [B][Hq][n_ctx] uint16, values <= 3*head_dim.
 *   idx  [B][Hq][budget] int32.
 * Requires n_ctx >= 1, budget >= 1, workspace of
 * adamas_workspace_bytes(ADAMAS_OP_SELECT_TOPK, ...).
 */
int adamas_select_topk(const uint16_t *dist, int B, int Hq, int64_t n_ctx,
                       int head_dim, int budget, int32_t *idx, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * Exact softmax attention over the selected rows only (§6):
 * s_j = scale * q . k_j, p = softmax(s), out = sum_j p_j v_j, accumulated in
 * binary32 and rounded to `dtype`.  Rows with idx < 0 are skipped; a head
 * with no valid index gets zeros.  Uses the original (unrotated) q, K, V.
 *
 *   q    [B][Hq][head_dim]; k, v [B][Hkv][cap][head_dim]; out [B][Hq][head_dim]
 *   idx  [B][Hq][budget] int32, every entry < cap.
 *   scale: 0 selects 1/sqrt(head_dim); must be finite.
 * Requires Hq % Hkv == 0, budget >= 1, workspace of
 * adamas_workspace_bytes(ADAMAS_OP_SPARSE_ATTEND, ...).
 */
int adamas_sparse_attend(const void *q, const void *k, const void *v, int dtype,
                         const int32_t *idx, int B, int Hq, int Hkv, int head_dim,
                         int64_t cap, int budget, float scale, void *out, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * One decode step of one layer, fused: encode each query head (§2.1-§2.2),
 * score it against cached codes rows [0, n_ctx) (§2.3), keep the budget
 * (§5.2) and attend over those K/V rows (§6).  Same results as
 * adamas_encode_keys(q) -> adamas_score -> adamas_select_topk ->
 * adamas_sparse_attend.
 *
 *   q [B][Hq][head_dim]; k, v [B][Hkv][cap][head_dim]; k_codes
 *   [B][Hkv][cap][head_dim/4]; out [B][Hq][head_dim]; idx_out nullable
 *   [B][Hq][budget] int32 (the selection, as adamas_select_topk writes it).
 * Requires Hq % Hkv == 0, 1 <= n_ctx <= cap, budget >= 1, workspace of
 * adamas_workspace_bytes(ADAMAS_OP_DECODE_STEP, ...).
 */
int adamas_decode_step(const void *q, const void *k, const void *v,
                       const uint8_t *k_codes, int dtype, int B, int Hq, int Hkv,
                       int head_dim, int64_t cap, int64_t n_ctx, int budget,
                       float scale, void *out, int32_t *idx_out, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * Process-wide choice of how adamas_decode_step splits the work of one KV
 * head (results are identical; only the schedule differs):
 *  - ADAMAS_DECODE_LAST_ARRIVAL: each chunk workgroup hands its chunk's
 *    min(budget, chunk) best candidates to the last workgroup to finish, which
 *    selects the budget (§5.2) and attends (§6) alone.
 *  - ADAMAS_DECODE_GROUP_WAIT: each chunk workgroup publishes its chunk's
 *    distance histogram and waits for the others of its KV head; from the sum
 *    it selects its own share of the budget and attends over it, and the last
 *    one merges the partial results.  Needs every workgroup of the launch
 *    resident at once, i.e. B*Hkv*chunks <= the device's compute units;
 *    adamas_decode_step returns ADAMAS_ERR_UNSUPPORTED when it is forced and
 *    the shape does not fit.  Launches of this kind on several streams of one
 *    device at once rely on the hardware starting a launch's workgroups in
 *    order; each wait is bounded (see ADAMAS_WS_STATUS_OFFSET).
 *  - ADAMAS_DECODE_SPLIT: each chunk workgroup publishes its chunk's
 *    candidates and its key counts per query head; a second launch, a few
 *    workgroups per query head, sums the counts to the head's threshold,
 *    places every chunk's share of the budget in the ascending selection and
 *    copies it there; a third launch attends.  For heads with many chunks
 *    (long contexts with large budgets), where one workgroup selecting from
 *    all chunk candidates would be slow.  Needs at most 2048 chunks per head
 *    (ADAMAS_ERR_UNSUPPORTED when forced beyond).
 *  - ADAMAS_DECODE_AUTO (default): LAST_ARRIVAL while its last workgroup can
 *    attend over the whole selection itself (G * ceil(min(budget, n_ctx) /
 *    256) <= 2) from at most 4096 chunk candidates per head; otherwise
 *    GROUP_WAIT where the shape fits, else SPLIT beyond 4096 candidates, else
 *    LAST_ARRIVAL with a separate attention launch.
 * Returns ADAMAS_OK, or ADAMAS_ERR_INVALID for an unknown mode.
 */
int adamas_set_decode_mode(int mode);

/*
 * Process-wide bound on each group wait of the ADAMAS_DECODE_GROUP_WAIT
 * schedule, in polls of the arrival counter (each poll sleeps about 64
 * cycles first).  A workgroup still waiting after `polls` polls gives up,
 * sets the workspace status word (ADAMAS_WS_STATUS_OFFSET) and runs to its
 * end with incomplete data: that call's outputs are invalid, and nothing
 * hangs.  The default, 1 << 20 polls, is far above any wait of a launch
 * whose workgroups are all resident; a small value (0 gives up at once)
 * forces the give-up path, e.g. to test a caller's status check.  Affects
 * launches enqueued after the call.  Returns ADAMAS_OK.
 */
int adamas_set_wait_polls(uint32_t polls);

/* The current group-wait bound (adamas_set_wait_polls). */
uint32_t adamas_wait_polls(void);

/*
 * Process-wide switch of the §2.1 rotation for every later adamas_encode_keys
 * and decode step (1, the default: rotate in binary32; 0: bucket vectors as
 * they are, the "2-bit quantisation only" row of the article's §3.2
 * ablation; 2: rotate in binary16, the article's advice to keep the Hadamard
 * transform in FP16 (§6): inputs rounded to binary16, every butterfly sum and
 * difference one binary16 operation; values beyond 65504 overflow to
 * infinities, so this is for inputs known to stay in range).  The distances
 * are integers whatever the setting (the article's INT8 similarity is exact
 * here already).  Codes made with one setting must only be scored against
 * queries encoded with the same one.  Returns ADAMAS_OK, or
 * ADAMAS_ERR_INVALID unless on is 0, 1 or 2.
 */
int adamas_set_rotation(int on);

/*
 * Per-head-group bucketing thresholds (article §2.2 with the §3.2 tuning
 * list, which gives groups of attention heads their own thresholds).  §2.2
 * buckets a rotated vector at -a/2, 0 and +a/2, a its absolute maximum (per
 * 128-dimension group).  After this call the outer thresholds of KV head h
 * are -t and +t with t = alpha[h % n] * a, one binary32 product (the middle
 * one stays 0); every query head of that KV head's group buckets with the
 * same alpha, so queries and keys of a head share one rule.  alpha: n host
 * floats, each finite and >= 0 (0 gives sign codes; 1 and above leaves only
 * the maximum in code 3), copied by the call.  n == 0 restores the §2.2 rule
 * (alpha 0.5 for every head, which is also what a table of 0.5s gives, bit
 * for bit).  Process-wide like adamas_set_rotation: it applies to launches
 * enqueued after the call, each launch keeps the table it was made with, and
 * codes made under one table must only be scored against queries encoded
 * under the same one.  Returns ADAMAS_OK, or ADAMAS_ERR_INVALID if n is
 * outside [0, ADAMAS_MAX_ALPHA_GROUPS], alpha is null with n > 0, or an
 * entry is negative, infinite or NaN (the table is then left as it was).
 */
#define ADAMAS_MAX_ALPHA_GROUPS 64
int adamas_set_bucket_alpha(const float* alpha, int n);

/*
 * The current table: copies min(n, cap) entries to alpha_out (when not
 * null) and returns n (0: the §2.2 rule).
 */
int adamas_bucket_alpha(float* alpha_out, int cap);

/*
 * The schedule adamas_decode_step would use for this shape on the current
 * device under the current mode: ADAMAS_DECODE_LAST_ARRIVAL,
 * ADAMAS_DECODE_GROUP_WAIT or ADAMAS_DECODE_SPLIT, or a negated status
 * (-ADAMAS_ERR_INVALID for a bad shape, -ADAMAS_ERR_UNSUPPORTED if
 * GROUP_WAIT or SPLIT is forced and does not fit, -ADAMAS_ERR_DEVICE if no
 * device can be queried).
 */
int adamas_decode_path(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int head_dim);

/*
 * Bytes per chunk key the decode kernel of the schedule adamas_decode_path
 * reports keeps in LDS for this shape (host-side planning; without a device
 * the last-arrival and split kernel's): 2, or 1 where grouped heads
 * (head_dim 64 or 128) would otherwise need more than one round of
 * workgroups (last-arrival, split) or more workgroups than the device holds
 * at once (group wait); one-byte keys hold chunks twice as long.  Results do
 * not depend on it (one-byte keys saturate at 255, and a chunk whose
 * selection reaches 255 is re-scanned with exact keys).  The ragged and
 * paged steps always keep 2.  Negated status for a shape adamas_decode_step
 * rejects.
 */
int adamas_decode_key_bytes(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int head_dim);

/*
 * Tokens per chunk (the code rows one decode workgroup scans, §2.3) that
 * adamas_decode_step plans for this shape under the schedule
 * adamas_decode_path reports: at least 1024, at most 16384 with 16-bit keys,
 * 32768 with one-byte keys or for multi-headed (one query per KV head)
 * launches of more than one round of workgroups, which then run two
 * workgroups per compute unit and select from each chunk a half at a time.
 * Host-side planning only; results do not depend on it.  The ragged step
 * plans the same chunks with 16-bit keys, the paged step at most 16384.
 * Negated status for a shape adamas_decode_step rejects.
 */
int adamas_decode_chunk_tokens(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int head_dim);

/*
 * adamas_select_topk and adamas_decode_step with a set of tokens that is
 * always kept: the first n_sink and the last n_recent of the n_ctx tokens
 * (attention sinks such as [CLS]/BOS positions, and a recent window; the
 * article keeps full attention for special tokens, §3.2 and §6).  They rank
 * ahead of every other token inside the budget: with F that set, the kept
 * tokens are all of F plus the plain selection of budget - |F| among the
 * others, or the budget's lowest-index members of F when |F| >= budget.
 * n_sink = n_recent = 0 gives the plain calls.  Requires n_sink, n_recent
 * >= 0; same workspace as the plain calls.
 */
int adamas_select_topk_keep(const uint16_t *dist, int B, int Hq, int64_t n_ctx,
                            int head_dim, int budget, int n_sink, int n_recent,
                            int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream);
int adamas_decode_step_keep(const void *q, const void *k, const void *v,
                            const uint8_t *k_codes, int dtype, int B, int Hq, int Hkv,
                            int head_dim, int64_t cap, int64_t n_ctx, int budget,
                            int n_sink, int n_recent, float scale, void *out,
                            int32_t *idx_out, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * One decode step of a batch whose sequences differ in length, with the
 * step's new token written into the caches in the same launch.  The
 * article's compressed cache (§3.1) takes each new token's packed key code at
 * its position as it is generated; here that key is rotated and bucketed
 * (§2.1-§2.2) inside the step, scored with the rest (§2.3), and can be
 * selected (§5.2) and attended (§6) in the step that adds it.  The step never
 * allocates or reads host state that changes between steps, so it can be
 * replayed from a HIP graph (graph launch is the article's small-batch
 * latency measure, §5.1).
 *   lens   [B] int32 device memory: rows already cached per sequence (L_b).
 *          Read only; the caller advances it between steps (the library never
 *          writes it), so the call can be captured in a HIP graph and replayed.
 *   k_new, v_new  [B][Hkv][head_dim] of dtype, or both NULL.  When set, row
 *          L_b of k, v and k_codes (for every KV head) receives the new key,
 *          value and key code, and sequence b attends over its L_b + 1 rows,
 *          the new one included.  When NULL nothing is written and sequence b
 *          attends over its L_b rows.
 *   k, v, k_codes  the caches of adamas_decode_step ([B][Hkv][cap][...]),
 *          written only at row L_b and only when k_new is set.
 *   max_len  host bound on the rows any sequence attends over (L_b + 1 with
 *          k_new, L_b without); 1 <= max_len <= cap.  The launch is planned
 *          for it: L_b is clamped to [0, max_len - 1] with k_new, to
 *          [0, max_len] without.  The workspace is adamas_workspace_bytes(
 *          ADAMAS_OP_DECODE_STEP, B, Hq, Hkv, max_len, budget, head_dim).
 * Everything else is as adamas_decode_step_keep, with n_ctx = each
 * sequence's own row count (so the recent window ends at its last row, and
 * each sequence keeps min(budget, rows) tokens).  A sequence with no rows
 * gets a zero output and idx_out rows of -1.  Always the LAST_ARRIVAL
 * schedule, whatever adamas_set_decode_mode chose.  Errors are returned
 * before anything is enqueued: ADAMAS_ERR_INVALID for bad sizes, a NULL or
 * misaligned pointer (lens needs 4 bytes, the rest 16), or only one of
 * k_new, v_new; ADAMAS_ERR_WORKSPACE for a short workspace.
 */
int adamas_decode_append_step(const void *q, const void *k_new, const void *v_new, void *k,
                              void *v, uint8_t *k_codes, const int32_t *lens, int dtype, int B,
                              int Hq, int Hkv, int head_dim, int64_t cap, int64_t max_len,
                              int budget, int n_sink, int n_recent, float scale, void *out,
                              int32_t *idx_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * adamas_encode_keys into paged pools (the layout of adamas_decode_paged_step
 * below): §2.1 rotation, §2.2 bucketing and §3.1 packing of a block of keys,
 * each token's code row (and, with x_pool, its raw row) written to the pool
 * page that its sequence's page table names; the article builds its
 * compressed cache this way, a chunk of tokens at a time (§3.1).
 *   x          [batch][heads][n][head_dim] elements of `dtype`: tokens
 *              [pos, pos + n) of each of `batch` sequences.
 *   code_pool  [n_pages][heads][page_size][head_dim/4] bytes.
 *   x_pool     nullable; [n_pages][heads][page_size][head_dim] elements of
 *              `dtype` receiving a verbatim copy of each row (a K pool).
 *   page_table [batch][max_pages] int32 device memory; token t of sequence
 *              b, head h, goes to pool row
 *              (page_table[b][t / page_size] * heads + h) * page_size
 *              + t % page_size.  Only the entries of pages that [pos, pos+n)
 *              spans are read; a token whose entry lies outside [0, n_pages)
 *              is not stored.  No other byte of the pools is touched.
 *   page_size  a power of two in [1024, 16384].
 * Requires batch, heads >= 1, n >= 0, pos >= 0, pos + n <= max_pages *
 * page_size, n_pages, max_pages >= 1; x, code_pool, x_pool 16-byte aligned
 * and page_table 4-byte aligned (else ADAMAS_ERR_INVALID; a page_size
 * outside the range ADAMAS_ERR_UNSUPPORTED).  n = 0 is a no-op.  Codes are
 * bit-identical to adamas_encode_keys' for the same rows.
 */
int adamas_encode_keys_paged(const void *x, int dtype, int batch, int heads, int64_t n,
                             int head_dim, uint8_t *code_pool, void *x_pool,
                             const int32_t *page_table, int page_size, int n_pages,
                             int max_pages, int64_t pos, hipStream_t stream);

/*
 * adamas_decode_append_step over paged caches.  The article's compressed
 * cache is built in chunks of a fixed number of tokens (§3.1, chunk_size
 * 1024); here every cache is a pool of such pages shared by all sequences,
 * and a page table maps each sequence's logical pages to pool pages, so a
 * sequence grows one page at a time without moving its rows.
 *   k_pool, v_pool  [n_pages][Hkv][page_size][head_dim] of dtype
 *   code_pool       [n_pages][Hkv][page_size][head_dim/4] u8
 *          (one pool page holds page_size consecutive tokens of every KV head;
 *          a page of one head is contiguous, so adamas_encode_keys with
 *          batch 1, heads Hkv, cap page_size fills it, x_copy_dst the K page)
 *   page_table [B][max_pages] int32 device memory: pool page of logical page
 *          i of sequence b, i.e. of its tokens [i*page_size, (i+1)*page_size).
 *          Every entry of a row up to the pages max_len spans may be read
 *          (the scan issues its first loads before it knows a sequence's
 *          length); entries a sequence does not reach only have to be
 *          readable, their values are clamped into [0, n_pages) and the rows
 *          they map are not used.
 *   page_size  a power of two in [1024, 16384].
 *   max_len    <= max_pages * page_size (the logical capacity).
 * Token t of sequence b, KV head h, is pool row
 * (page_table[b][t / page_size] * Hkv + h) * page_size + t % page_size.
 * Everything else (lens, k_new/v_new and the row they are written to,
 * clamping, outputs, workspace, errors) is as adamas_decode_append_step, with
 * the logical capacity in place of cap.  Page table entries outside
 * [0, n_pages) give undefined results for the rows they map (reads stay
 * inside the pools; a new token whose entry is out of range is not stored).
 * ADAMAS_ERR_UNSUPPORTED for a page_size outside the range above,
 * ADAMAS_ERR_INVALID for n_pages or max_pages < 1 or a NULL or misaligned
 * page table (4 bytes).
 */
int adamas_decode_paged_step(const void *q, const void *k_new, const void *v_new, void *k_pool,
                             void *v_pool, uint8_t *code_pool, const int32_t *page_table,
                             const int32_t *lens, int dtype, int B, int Hq, int Hkv, int head_dim,
                             int page_size, int n_pages, int max_pages, int64_t max_len,
                             int budget, int n_sink, int n_recent, float scale, void *out,
                             int32_t *idx_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Measurement hooks, not steps of the method.  A library built with
 * -DADAMAS_PHASES=1 (libadamas_phases.so) records, for every workgroup of
 * the decode, selection and attention kernels, the device's constant-rate
 * wall clock (adamas_wall_clock_khz ticks per millisecond) at marked points,
 * into a caller-owned device buffer of adamas_phase_buffer_bytes() bytes:
 * u64 [3 kernel regions: decode, split selection, attention][8192
 * workgroups][24 slots], 0 where a slot was not reached; each launch
 * overwrites its region.  adamas_set_phase_buffer(NULL, 0) stops recording.
 * In the product build adamas_phase_stamps_built() is 0 and
 * adamas_set_phase_buffer returns ADAMAS_ERR_UNSUPPORTED; ADAMAS_ERR_INVALID
 * for a misaligned or short buffer.  The buffer is borrowed until it is
 * unset; launches that overlap in time overwrite each other's stamps.
 */
int adamas_phase_stamps_built(void);
size_t adamas_phase_buffer_bytes(void);
int adamas_set_phase_buffer(void *buf, size_t bytes);
int adamas_wall_clock_khz(void);

/*
 * adamas_decode_step for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument; the call allocates nothing and calls no allocating
 * routine.  Its scratch (candidate lists, arrival counters, partial results)
 * is a static device buffer of ADAMAS_STATIC_SCRATCH_BYTES inside the
 * library, one copy per device, held from the library's load until the
 * process ends; the first call on a device resolves its address and enqueues
 * a small kernel that zeroes its control bytes.  All calls on one device
 * share that buffer: calls that may overlap in time on one device (several
 * streams, several host threads) race and must not be made.  It never takes
 * the group-wait schedule (adamas_set_decode_mode's GROUP_WAIT is read as
 * AUTO), so there is no status word to check.  Arguments, layouts, results
 * and errors are those of adamas_decode_step; a shape whose scratch
 * (adamas_static_scratch_need) exceeds ADAMAS_STATIC_SCRATCH_BYTES returns
 * ADAMAS_ERR_WORKSPACE before anything is enqueued, and a failure to resolve
 * the buffer ADAMAS_ERR_DEVICE.
 */
#define ADAMAS_STATIC_SCRATCH_BYTES (16u << 20)
int adamas_decode_step_static(const void *q, const void *k, const void *v,
                              const uint8_t *k_codes, int dtype, int B, int Hq, int Hkv,
                              int head_dim, int64_t cap, int64_t n_ctx, int budget, float scale,
                              void *out, int32_t *idx_out, hipStream_t stream);

/* Scratch bytes adamas_decode_step_static needs for a shape (0 if invalid or
 * beyond the decode step's limits). */
size_t adamas_static_scratch_need(int B, int Hq, int Hkv, int64_t n_ctx, int budget,
                                  int head_dim);

/* Workspace bytes needed by `op` for the given shape (0 for invalid shapes and
 * for shapes beyond the entry points' limits: n_ctx > INT32_MAX, B or Hq >
 * 65535, B*Hq > 8192). */
size_t adamas_workspace_bytes(int op, int B, int Hq, int Hkv, int64_t n_ctx,
                              int budget, int head_dim);

/*
 * Reference streaming read, not a step of the method: reads `bytes` (a
 * multiple of 16) at `src` (16-byte aligned) once, with the 16-byte
 * non-temporal loads of the decode scan, each of
 * adamas_stream_read_blocks(bytes) workgroups taking one contiguous slice,
 * and writes one XOR word per workgroup to sink[] so the reads stay.  Timing
 * it gives the bandwidth plain reads reach on the device, the figure the
 * decode step's achieved bandwidth is read against.  Returns
 * ADAMAS_ERR_INVALID for a null sink, misaligned src or a bad size.
 */
int adamas_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Workgroups (sink words) adamas_stream_read uses for `bytes`. */
size_t adamas_stream_read_blocks(size_t bytes);

/* Static, human-readable text for a status code. */
const char *adamas_status_string(int status);

/* ADAMAS_VERSION of the built library. */
int adamas_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ADAMAS_H */
