/*
 * dsa_indexer.h -- C ABI of the DSA indexer decode step on MI355X (gfx950).
 *
 * One decode step of the DeepSeek sparse-attention (DSA) indexer, as described
 * on the pages "The O(Actual) Indexer: Validating 128K Context at 500 tok/s on
 * Blackwell" (sections "The Bottleneck That Was" and "The Benchmark Results")
 * and "The Moment of Breakthrough: Validating the Indexer Fix" (section "The
 * Context: A Long Hunt for the Hidden Wall"):
 *
 *   1. walk each request's page table over c4-compressed key pages of 64
 *      positions (a 256-token page, one key per 4 tokens);
 *   2. score every valid position s of request b as
 *        score[b][s] = sum_{h<32} w[b][h] * max(0, sum_{d<64} q[b][h][d] * k[s][d])
 *      with bfloat16 q and k, float32 w and float32 accumulation;
 *   3. write -inf at every position at or past the request's length, into a
 *      full-width output of max_pages * 64 positions, skipping the key reads
 *      and the products for pages past the length (so that the work follows
 *      the actual length, not the configured maximum);
 *   4. select the top-k positions of each request.
 *
 * Conventions shared by every entry point
 *   - All buffer pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees, synchronizes, or reads device memory on the host;
 *     a call validates its scalar arguments and pointers on the host, enqueues
 *     kernels on `stream` (NULL = the null stream) and returns. Every call can
 *     be captured into a hipGraph (launch shapes depend only on the scalar
 *     arguments, never on device data).
 *   - Errors detectable on the host return a negative dsa_status_t and enqueue
 *     nothing. A failed launch returns DSA_ERR_HIP; the HIP error code is then
 *     available from dsa_indexer_last_hip_error() on the same thread.
 *   - Conditions only the device can see are not errors (reporting them would
 *     need a synchronization) and are defined instead:
 *       * seq_lens[b] is clamped to [0, max_pages * 64];
 *       * a page id outside [0, num_pages) in a slot that holds valid
 *         positions is never dereferenced; those valid positions score NaN;
 *       * slots at or past ceil(seq_lens[b] / 64) are never read, so they may
 *         hold anything (e.g. -1);
 *       * non-finite q, k or w give unspecified scores.
 *   - Shapes are fixed by the method: 32 heads, head dim 64, 64 positions per
 *     page. All arrays are dense, row-major, innermost index last.
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_INDEXER_ABI_VERSION 7
#define DSA_INDEXER_HEADS 32 /* indexer heads */
#define DSA_INDEXER_DIM 64   /* head dimension */
#define DSA_INDEXER_PAGE 64  /* c4 positions per page */
#define DSA_INDEXER_HIST_BINS 2048 /* bins of the first-digit histogram (score_hist / topk_hist) */
#define DSA_INDEXER_NOALLOC_SCRATCH_BYTES (64u << 20) /* fixed workspace of dsa_indexer_topk_noalloc, per GPU */

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,      /* a required pointer is NULL */
  DSA_ERR_SHAPE = -2,     /* batch, max_pages, num_pages or max_c4 out of range */
  DSA_ERR_ALIGN = -3,     /* a pointer misses its required alignment */
  DSA_ERR_K = -4,         /* k out of [1, max_c4] */
  DSA_ERR_WORKSPACE = -5, /* workspace too small for the call */
  DSA_ERR_HIP = -6,       /* the HIP runtime reported an error for a launch */
  DSA_ERR_SCRATCH = -7    /* sizes beyond the fixed scratch of dsa_indexer_topk_noalloc */
} dsa_status_t;

/* DSA_INDEXER_ABI_VERSION of the loaded library. */
int dsa_indexer_abi_version(void);

/* Static text for a dsa_status_t value ("unknown status" otherwise). */
const char *dsa_indexer_status_string(int status);

/* hipError_t of the last DSA_ERR_HIP on the calling thread (0 if none). */
int dsa_indexer_last_hip_error(void);

/*
 * Score step (steps 1-3 above): fills logits[b][0 : max_pages*64] for every
 * request.
 *
 *   q          bf16  [batch][32][64], 16-byte aligned
 *   w          fp32  [batch][32], 16-byte aligned (each request's 32 weights
 *              are read as eight 16-byte vectors)
 *   k_pool     bf16  [num_pages][64][64], 16-byte aligned: page p, row i is the
 *              key of the position that maps to (p, i); dims contiguous
 *   num_pages  pages in k_pool (> 0)
 *   page_table int32 [batch][max_pages]: physical page of each slot; position
 *              s of request b lives in page page_table[b][s / 64], row s % 64
 *   seq_lens   int32 [batch]: valid c4 positions per request
 *   batch      1 .. 65535
 *   max_pages  1 .. 2^22 (row width max_pages * 64 at most 2^28 positions),
 *              with batch * max_pages at most 2^26 (at most 2^32 logits)
 *   logits     fp32  [batch][max_pages*64], 16-byte aligned; on return of the
 *              enqueued work: the score for s < seq_lens[b], -inf otherwise
 *              (bit pattern 0xFF800000)
 *   row_hwm    NULL, or int32 [batch] high-water marks for the incremental
 *              tail. With NULL every call writes the whole -inf tail. With a
 *              buffer, the caller keeps `logits` and `row_hwm` across calls and
 *              guarantees that on entry logits[b][s] == -inf for every
 *              s >= row_hwm[b] (e.g. logits all -inf and row_hwm all 0 before
 *              the first call); the call then rewrites -inf only on pages in
 *              [seq_lens[b], row_hwm[b]) and sets row_hwm[b] = seq_lens[b]
 *              (clamped). The result is identical in both modes.
 *   stream     HIP stream to enqueue on
 */
int dsa_indexer_score(const void *q, const float *w, const void *k_pool, int64_t num_pages,
                      const int32_t *page_table, const int32_t *seq_lens, int32_t batch,
                      int32_t max_pages, float *logits, int32_t *row_hwm, hipStream_t stream);

/*
 * Score step that also counts what the top-k needs first (the fused pair
 * dsa_indexer_score_hist + dsa_indexer_topk_hist; the top-k over the
 * indexer's logits is the step page "The O(Actual) Indexer", section "The
 * Benchmark Results", names as the remaining cost). Everything
 * dsa_indexer_score does, argument for argument, and in addition:
 *
 *   hist       uint32 [batch][2048], 16-byte aligned. For every valid
 *              position s < seq_lens[b] (clamped) the call adds one count to
 *              hist[b][key(logits[b][s]) >> 21], where key() is the
 *              order-preserving map of a float to 32 bits (non-negative x:
 *              bits(x) | 0x80000000; negative x: ~bits(x); -0 counts as +0;
 *              NaN as key 1, i.e. bin 0). The counts are added to what hist
 *              holds: it must be all zero on entry (zero it once when it is
 *              allocated; dsa_indexer_topk_hist sets it back to zero).
 *
 * Errors as for dsa_indexer_score (DSA_ERR_NULL also for a NULL hist,
 * DSA_ERR_ALIGN for a misaligned one); q, w, k_pool and logits are 16-byte
 * aligned as there.
 */
int dsa_indexer_score_hist(const void *q, const float *w, const void *k_pool, int64_t num_pages,
                           const int32_t *page_table, const int32_t *seq_lens, int32_t batch,
                           int32_t max_pages, float *logits, int32_t *row_hwm, uint32_t *hist,
                           hipStream_t stream);

/*
 * Score step with fp8 keys (page "The Indexer O(max_context) Breakthrough"
 * mentions an fp8 KV cache; the pages do not say how the indexer's keys are
 * stored, so this format is a reading, not a page fact): each key is 64 OCP
 * FP8 E4M3 codes (e4m3fn: bias 7, no infinities, largest value 448; code
 * 0x7F/0xFF is NaN) and one float32 scale, and the key that enters the
 * formula is scale * decode(codes). Everything else is as for
 * dsa_indexer_score, which this mirrors argument for argument:
 *
 *   k_pool_fp8 uint8 [num_pages][64][64], 16-byte aligned: codes of page p,
 *              row i (the key of the position that maps to (p, i)), dims
 *              contiguous; 4 KiB per page
 *   k_scale    fp32  [num_pages][64], 4-byte aligned: the scale of each key
 *
 * q, w and logits are 16-byte aligned as for dsa_indexer_score. Errors as for
 * dsa_indexer_score (DSA_ERR_NULL also for a NULL k_scale).
 */
int dsa_indexer_score_fp8(const void *q, const float *w, const void *k_pool_fp8, const float *k_scale,
                          int64_t num_pages, const int32_t *page_table, const int32_t *seq_lens,
                          int32_t batch, int32_t max_pages, float *logits, int32_t *row_hwm,
                          hipStream_t stream);

/*
 * Several query tokens per request (the current token and draft tokens of a
 * multi-token-prediction or speculative step; page "The Indexer
 * O(max_context) Breakthrough", section "MTP/EAGLE Integration (Phase 2)"):
 * steps 1-3 for `tokens` query tokens per request, each token t with its own
 * causal length seq_lens[b][t] (clamped to [0, max_pages * 64]):
 *   logits[b][t][s] = sum_h w[b][t][h] * max(0, q[b][t][h] . k[s])   for s < seq_lens[b][t]
 * and -inf for s >= seq_lens[b][t]. Each key page below the longest of a
 * request's lengths is read once for all its tokens. The logits rows are
 * [batch * tokens][max_pages * 64], so dsa_indexer_topk with batch * tokens
 * rows and the same seq_lens selects per token.
 *
 *   q          bf16  [batch][tokens][32][64], 16-byte aligned
 *   w          fp32  [batch][tokens][32], 16-byte aligned
 *   k_pool, num_pages, page_table, max_pages: as for dsa_indexer_score
 *   seq_lens   int32 [batch][tokens]
 *   batch      1 .. 65535;  tokens 1 .. 4;  batch * tokens * max_pages <= 2^26
 *   logits     fp32  [batch][tokens][max_pages * 64], 16-byte aligned
 *   row_hwm    NULL (every call writes the whole -inf tail of every token's
 *              row), or int32 [batch] high-water marks for the incremental
 *              tail, one per request for all its tokens: as for
 *              dsa_indexer_score with L_b = the longest of the request's
 *              clamped lengths. The caller guarantees on entry that
 *              logits[b][t][s] == -inf for every t and every s >= row_hwm[b];
 *              the call rewrites -inf only on pages in [L_b, row_hwm[b]) of
 *              every token's row and sets row_hwm[b] = L_b. The result is
 *              identical in both modes.
 *
 * Errors and device-side conventions as for dsa_indexer_score.
 */
int dsa_indexer_score_mtp(const void *q, const float *w, const void *k_pool, int64_t num_pages,
                          const int32_t *page_table, const int32_t *seq_lens, int32_t batch, int32_t tokens,
                          int32_t max_pages, float *logits, int32_t *row_hwm, hipStream_t stream);

/* Bytes of device workspace dsa_indexer_topk needs for these sizes: 0 when
 * max_c4 <= 32768 (the workspace may then be NULL) or the sizes are out of
 * range, else batch * ceil(max_c4 / 4096) * (32 + 32768) bytes, about twice the
 * logits' own size. */
size_t dsa_indexer_topk_workspace_bytes(int32_t batch, int32_t max_c4, int32_t k);

/*
 * Top-k step (step 4 above; page "The O(Actual) Indexer", section "The
 * Benchmark Results", on the top-k that follows the indexer): for every
 * request b with L = clamp(seq_lens[b], 0, max_c4), picks the min(k, L)
 * positions of logits[b][0:L] with the largest scores. Ranking: larger score
 * first; among equal scores the lower position first (-0 and +0 are equal);
 * NaN ranks below every number. Positions at or past L are never read.
 *
 *   logits     fp32  [batch][max_c4] (as written by dsa_indexer_score)
 *   seq_lens   int32 [batch]
 *   batch      1 .. 65535
 *   max_c4     row width, 1 .. 2^28
 *   k          1 .. max_c4
 *   out_idx    int32 [batch][k]: the chosen positions in ascending order,
 *              then -1 in the remaining k - min(k, L) slots
 *   out_vals   NULL, or fp32 [batch][k]: logits at out_idx, NaN in padding
 *   workspace  device buffer, 16-byte aligned, of ws_bytes >=
 *              dsa_indexer_topk_workspace_bytes() (may be NULL when that is
 *              0); its contents on entry do not matter and are overwritten.
 *              Calls that may overlap (other streams) need workspaces of
 *              their own
 *   stream     HIP stream to enqueue on
 *
 * One workgroup per request selects its row's top k. With max_c4 <= 32768 it
 * is the only kernel: a row longer than 4096 positions is held in registers,
 * cut at a key sampled from 64 runs of 32 positions, and the keys at or
 * above the cut become the candidates. With a wider row width, a segment kernel is
 * enqueued first: it splits each row longer than 4096 positions into
 * segments of 4096 (up to 8 workgroups per request, each taking every 8th
 * segment from its own) and writes each segment's keys at or above a cut
 * sampled from that segment, with their positions, to the workspace, which
 * the row's workgroup then gathers. Either way the row's workgroup falls back
 * to a select over the whole row whenever the candidates cannot be shown to
 * hold the whole top k, so the result never depends on the sampling.
 */
int dsa_indexer_topk(const float *logits, const int32_t *seq_lens, int32_t batch, int32_t max_c4,
                     int32_t k, int32_t *out_idx, float *out_vals, void *workspace,
                     size_t ws_bytes, hipStream_t stream);

/*
 * Top-k for callers that cannot allocate device memory (code under hipGraph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the result
 * of dsa_indexer_topk, argument for argument, without the workspace
 * arguments. The workspace lives in a fixed device array of
 * DSA_INDEXER_NOALLOC_SCRATCH_BYTES per GPU, part of the library's code object
 * (held from load until the process ends); the call allocates nothing.
 *
 *   - Sizes whose dsa_indexer_topk_workspace_bytes(batch, max_c4, k) exceeds
 *     DSA_INDEXER_NOALLOC_SCRATCH_BYTES are refused with DSA_ERR_SCRATCH
 *     (64 MiB: batch * ceil(max_c4 / 4096) up to 2046, e.g. 64 requests of a
 *     row width up to 126976 positions; a row width of at most 32768
 *     positions needs none).
 *   - The first call on a device that needs the array resolves its address
 *     there (hipGetSymbolAddress, no allocation); make that first call
 *     outside graph capture.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     (other streams, other threads) race and give unspecified positions.
 *     Calls in stream order are safe; the array needs no clearing between
 *     them.
 *
 * Errors as for dsa_indexer_topk, plus DSA_ERR_SCRATCH.
 */
int dsa_indexer_topk_noalloc(const float *logits, const int32_t *seq_lens, int32_t batch, int32_t max_c4,
                             int32_t k, int32_t *out_idx, float *out_vals, hipStream_t stream);

/*
 * Top-k step over logits written by dsa_indexer_score_hist, with its
 * histogram: the same result as dsa_indexer_topk, argument for argument, plus
 *
 *   hist       uint32 [batch][2048], 16-byte aligned: the histogram that
 *              dsa_indexer_score_hist accumulated for exactly these logits
 *              and seq_lens. The call reads it and sets it back to all zero
 *              (ready for the next dsa_indexer_score_hist).
 *
 * The histogram gives every row's first radix digit of the k-th largest
 * score exactly, so no cut is sampled and the first radix pass is skipped:
 * the candidates are the keys in or above that bin. Counts that do not
 * belong to these logits give unspecified positions (never accesses outside
 * the buffers). Errors as for dsa_indexer_topk (DSA_ERR_NULL also for a NULL
 * hist, DSA_ERR_ALIGN for a misaligned one); the workspace is sized by
 * dsa_indexer_topk_workspace_bytes.
 */
int dsa_indexer_topk_hist(const float *logits, const int32_t *seq_lens, int32_t batch, int32_t max_c4,
                          int32_t k, int32_t *out_idx, float *out_vals, uint32_t *hist, void *workspace,
                          size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse attention over the selected positions (the step after the indexer;
 * page "The Indexer O(max_context) Breakthrough", sections "Phase 1: The MMA
 * Sparse-MLA Decode Kernel" and "Phase 2: Split-K Parallelization").
 *
 * For every request b and head h < 32, with the list entries s = idx[b][j]
 * that are >= 0:
 *   score_s  = scale * sum_{d<576} q[b][h][d] * kv[s][d]
 *   out[b][h][v] = sum_s softmax(score)_s * kv[s][v]     for v < 512
 *   lse[b][h]    = log(sum_s exp(score_s))               (natural log)
 * where kv[s] is the latent of position s: row s % 64 of page
 * page_table[b][s / 64]. Each latent (576 bfloat16: the first 512 are the
 * value, the last 64 only enter the score) is read once per request and
 * shared by the 32 heads. Products are exact, sums are float32, and the
 * softmax weights enter the weighted sum of values as bfloat16.
 *
 *   q          bf16  [batch][32][576], 16-byte aligned
 *   kv_pool    bf16  [num_pages][64][576], 16-byte aligned
 *   num_pages  1 .. 2^26 - 1
 *   page_table int32 [batch][max_pages] (the indexer's table)
 *   batch      1 .. 65535;  max_pages 1 .. 2^22
 *   idx        int32 [batch][k]: positions in any order; negative entries are
 *              skipped (the -1 padding of dsa_indexer_topk's out_idx)
 *   k          1 .. 2048
 *   scale      softmax scale (finite)
 *   out        fp32 [batch][32][512], 16-byte aligned
 *   lse        fp32 [batch][32]
 *   workspace  device buffer, 16-byte aligned, of ws_bytes >=
 *              dsa_indexer_sparse_attention_workspace_bytes() (may be NULL when
 *              that is 0); contents on entry do not matter. Overlapping calls
 *              (other streams) need workspaces of their own
 *   stream     HIP stream to enqueue on
 *
 * Defined outcomes that only the device can see: a request with no entry >= 0
 * gets out = 0 and lse = -inf; a request with an entry at or past
 * max_pages * 64, or on a page id outside [0, num_pages), gets NaN in all of
 * its out and lse (no memory outside the pool is read).
 *
 * Each request's list is cut into splits of equal length, planned from
 * (batch, k) alone; one workgroup per (request, split) computes that split's
 * softmax-normalised output and log-sum-exp, and with more than one split a
 * second kernel merges them by their log-sum-exps.
 */
size_t dsa_indexer_sparse_attention_workspace_bytes(int32_t batch, int32_t k);

int dsa_indexer_sparse_attention(const void *q, const void *kv_pool, int64_t num_pages,
                                 const int32_t *page_table, int32_t batch, int32_t max_pages,
                                 const int32_t *idx, int32_t k, float scale, float *out, float *lse,
                                 void *workspace, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_H */
