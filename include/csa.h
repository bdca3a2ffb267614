/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed-attention library (libcsa.so).
 *
 * The library computes the attention hot path of a CSA/HCA hybrid-attention
 * transformer layer:
 *
 *   csa_compress    block KV compressor (CSA block m = 4, HCA block m' = 128)
 *   csa_append      decode-time state cache: ring of raw rows + compression of
 *                   the blocks each new token completes
 *   csa_index_topk  Lightning-Indexer scores of compressed entries + per-query top-k
 *   csa_index_topk_bf16  the same selection on scores rounded to bf16 (approximate)
 *   csa_index_topk_fp8   the same selection with fp8 x fp8 dot products (query
 *                   quantised to e4m3 like the keys)
 *   csa_attend      attention over the selected compressed entries and the raw
 *                   sliding window, under one softmax
 *   hca_attend      dense attention over every visible heavy entry and the window
 *
 * Method sources (pages on the web, cited by section):
 *   [digest]  V4 report digest, https://gitcode.csdn.net/69eb1ea054b52172bc6fc291.html
 *             section 三 (CSA / HCA / window), section 七 (low-precision indexer QK
 *             path, compressed cache vs. state cache)
 *   [book]    "Evolution map", https://igloomatics.github.io/DeepSeek-V4-book/chapters/ch01.html
 *             section 4 (m = 4 super-KV, top-k = 1024, m' = 128, n/m' dense entries)
 *   [summary] https://www.10100.com/article/149217299 sections 2.1, 2.2, 五
 *
 * Conventions for every call
 *   - Tensor arguments are DEVICE pointers to row-major arrays whose innermost
 *     dimension is contiguous, with the shapes given below; base addresses must
 *     be 16-byte aligned.  Sizes are element counts.  A pointer to an array
 *     with no elements (T = 0, N_alloc = 0, T_new = 0, ...) may be NULL.
 *   - B sequences in a call share the context length and query positions.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL means the null
 *     stream) and is asynchronous: a call never synchronises and never allocates
 *     device memory.  The caller owns every buffer.
 *   - Every argument is validated before any HIP call; a non-OK status means
 *     nothing was enqueued.  csa_last_error() then returns a thread-local
 *     description.  CSA_E_HIP reports a failed launch (with the HIP error text).
 *   - Workspaces: the *_workspace() functions return the bytes a call needs for
 *     the given shape (0: none needed, NULL allowed).  A workspace must be
 *     zero-filled before its first use with this library.  Its first 2 MiB hold
 *     control words (arrival counters, histograms) at offsets that do not depend
 *     on the shape, and every call returns them to zero when its last kernel
 *     finishes; the rest is scratch that a call writes before it reads.  One
 *     zero fill at allocation therefore serves any sequence of calls, of any
 *     function and shape, that share the workspace, provided the calls are
 *     ordered (same stream, or synchronised); concurrent calls on one
 *     workspace race.
 *   - Numerics: compressor sums are accumulated in fp64 and rounded once to the
 *     output type; dot products accumulate in fp32 (bf16 x bf16 products are
 *     exact in fp32); softmax statistics are fp32; the softmax weights enter the
 *     value product as a bf16 hi + lo pair (about 16 significant bits).
 *   - Non-finite inputs (NaN, +-inf) never change how long a call runs (every
 *     loop is bounded by the sizes alone) and follow IEEE arithmetic:
 *       * indexer: the rectifier max(0, x) keeps a NaN of either sign, so a
 *         NaN in a key row, in a query head or in a weight makes the affected
 *         scores NaN; an infinity gives +-inf, or NaN through inf - inf or
 *         0 * inf.  A NaN score ranks above every number (+inf included),
 *         NaN ties going to the lower index as any tie does, and out_score
 *         reports it as NaN.  -inf is an ordinary (lowest) score: visibility
 *         depends on positions only, never on a score's value.
 *       * attention: a NaN or infinity in q[b,i,h,:] or in a K or V row that
 *         takes part in query i's softmax makes outputs of that query
 *         non-finite: a NaN in q[b,i,h,:] the row (i, h); in a K row, every
 *         head of query i; in column c of a V row, column c of every head of
 *         query i.  A skipped slot (invalid, invisible or padding index) reads
 *         nothing.  An infinity may give NaN where exact arithmetic would give
 *         an infinity.  One exception: in hca_attend over at least 16
 *         consecutive query tokens per sequence, a non-finite heavy-entry or
 *         window row also reaches the tokens of the same group of up to 4
 *         consecutive tokens that share its tile without seeing it (a zero
 *         weight times NaN is NaN).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 7

typedef enum {
  CSA_F32 = 0,      /* IEEE binary32 */
  CSA_BF16 = 1,     /* bfloat16 (upper half of a binary32) */
  CSA_FP8_E4M3 = 2  /* OCP fp8 e4m3fn, one byte per value, with a per-row fp32 scale */
} csa_dtype_t;

typedef enum {
  CSA_OK = 0,
  CSA_E_NULL = 1,        /* a required pointer is NULL */
  CSA_E_SHAPE = 2,       /* a size is out of range or inconsistent */
  CSA_E_DTYPE = 3,       /* unsupported dtype or dtype combination */
  CSA_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  CSA_E_WORKSPACE = 5,   /* workspace NULL or smaller than *_workspace() */
  CSA_E_UNSUPPORTED = 6, /* valid request the library does not implement */
  CSA_E_HIP = 7          /* a HIP runtime call failed */
} csa_status_t;

typedef void* csa_stream_t; /* hipStream_t */

/* Version of this header's ABI (CSA_ABI_VERSION of the built library). */
int csa_abi_version(void);
/* Static name of a status code. */
const char* csa_status_string(int status);
/* Thread-local description of the last non-OK status returned on this thread. */
const char* csa_last_error(void);

/*
 * csa_compress -- fold every m consecutive raw rows into one compressed entry.
 *
 * [digest] 三 and [book] 4: CSA folds each block of m = 4 tokens into one
 * entry, HCA each block of m' = 128.  Here entry j of a sequence is
 *     out[b, j, :] = sum_{s<m} alpha_s * x[position j*m + s, :],
 *     alpha = softmax(logits)      (one learned logit per slot)
 * over non-overlapping blocks; a trailing partial block is never emitted.
 *
 *   x          [B, n_raw, d] of x_dt (CSA_F32 | CSA_BF16): raw rows for the
 *              positions raw_base .. raw_base + n_raw - 1.
 *   logits     [m + overlap] fp32, device.  1 <= m, m + overlap <= 128.
 *   overlap    0 for the blocks above.  overlap = o > 0 is a method variant
 *              ([summary] 2.1: position weighting and overlapping blocks, no
 *              formula): entry j folds the m + o rows of positions
 *              j*m - o .. j*m + m - 1 with alpha = softmax(logits) over the
 *              m + o slots; slots before position 0 are left out and the
 *              first entries renormalise over the rest.  An entry still ends
 *              at position j*m + m - 1 (its visibility is unchanged).
 *   entries    [entry_begin, entry_end) of each sequence are written; every
 *              covered position must lie inside x:
 *              raw_base <= max(0, entry_begin*m - overlap) and
 *              entry_end*m <= raw_base + n_raw, 0 <= entry_begin <= entry_end <= N_alloc.
 *   out        [B, N_alloc, d] of out_dt: CSA_F32 | CSA_BF16 (sum rounded once,
 *              nearest-even), or CSA_FP8_E4M3 (bytes) with out_scale.
 *   out_scale  [B, N_alloc] fp32, required iff out_dt == CSA_FP8_E4M3, else
 *              must be NULL.  The fp32 image r of the sum is stored as
 *              scale = f32(max_i |r_i| / 448) (1 for an all-zero row) and
 *              code_i = e4m3(f32(r_i / scale)), nearest-even.
 *   d          8 <= d <= 512, d % 8 == 0 (a power of two >= 16 for CSA_FP8_E4M3).
 * An empty entry range is a no-op.  No workspace.
 */
csa_status_t csa_compress(const void* x, csa_dtype_t x_dt, int B, int64_t n_raw, int d,
                          int64_t raw_base, const float* logits, int m, int overlap,
                          int64_t entry_begin, int64_t entry_end, int64_t N_alloc, void* out,
                          csa_dtype_t out_dt, float* out_scale, csa_stream_t stream);

/*
 * csa_append -- decode-time state cache: append raw rows and compress the
 * blocks they complete.
 *
 * [digest] 七: besides the compressed cache there is a state cache for the
 * sliding-window rows and for the tokens of a block that is not complete yet.
 * Here it is a ring of R rows per sequence kept twice ("mirrored"): position p
 * lives in rows p % R and p % R + R of ring, so the newest R positions are
 * always R consecutive rows.  Readers take the ring as ordinary raw rows:
 * positions s .. s + L - 1 (L <= R, all among the newest R) are the rows
 * starting at s % R, i.e. pass x / k_raw / v_raw = ring, n_raw = 2R and
 * raw_base = s - s % R to csa_compress, csa_attend or hca_attend.
 *
 *   x_new   [B, T_new, d] of dt (CSA_F32 | CSA_BF16): the rows of positions
 *           t0 .. t0 + T_new - 1 (0 <= T_new <= 4096; 0 is a no-op).
 *   ring    [B, 2R, d] of dt, updated in place.  It must already hold the
 *           positions t0 - R + T_new .. t0 - 1 (those >= 0) from earlier calls.
 *   R       ring rows, 1 <= R <= 2^24 and R >= m + overlap + T_new - 1 (so
 *           that the rows of every completed block are still in the ring);
 *           R >= W + T_new keeps a window of W rows readable after the call.
 *   logits, m, overlap, out, out_dt, out_scale, N_alloc: as in csa_compress.  Every
 *           block j < N_alloc that the new rows complete, t0 <= (j+1) m - 1 <=
 *           t0 + T_new - 1, is written to out[b, j] with the same arithmetic
 *           (and hence the same bits) as csa_compress over the full history.
 *   d       as in csa_compress.
 * Calls for one ring must be ordered on one stream.  No workspace.
 */
csa_status_t csa_append(const void* x_new, csa_dtype_t dt, int B, int T_new, int d, int64_t t0,
                        void* ring, int64_t R, const float* logits, int m, int overlap,
                        int64_t N_alloc, void* out, csa_dtype_t out_dt, float* out_scale,
                        csa_stream_t stream);

/*
 * csa_index_topk -- Lightning-Indexer scores and per-query top-k selection.
 *
 * [digest] 三: an indexer scores the compressed entries and only the top-k take
 * part in the core attention; [digest] 七: its cached keys are kept in low
 * precision.  Query i of every sequence sits at position t = t0 + i and sees
 * the entries whose block ends at or before t:  j < c(t) = min(N_alloc, (t+1)/m).
 * Its score of entry j is
 *     I(t, j) = sum_{h<H_I} w[b,i,h] * max(0, q_idx[b,i,h,:] . k_idx[b,j,:])
 * computed in fp32, and the selected set is the min(top_k, c(t)) entries with
 * the highest I (ties to the lower j), shared by all attention heads.
 *
 *   q_idx     [B, T, H_I, d_I] of q_dt
 *   w         [B, T, H_I] fp32, or NULL for all ones
 *   k_idx     [B, N_alloc, d_I] of k_dt; CSA_FP8_E4M3 keys need k_scale
 *             [B, N_alloc] fp32 (the key row is code * scale), else k_scale NULL.
 *   dtypes    (q_dt, k_dt) = (CSA_F32, CSA_F32), (CSA_BF16, CSA_BF16) or
 *             (CSA_BF16, CSA_FP8_E4M3).
 *   out_idx   [B, T, top_k] int32: the selected entries in no particular order,
 *             then -1 in unused slots.
 *   out_score [B, T, top_k] fp32 or NULL: the fp32 score of each listed entry
 *             (-inf in unused slots).
 *   limits    1 <= H_I <= 16, d_I in {32, 64}, 1 <= top_k <= 2048, m >= 1,
 *             T >= 0, t0 >= 0, N_alloc >= 0, B >= 1.
 */
size_t csa_index_topk_workspace(int B, int64_t T, int H_I, int d_I, int64_t N_alloc, int top_k,
                                csa_dtype_t k_dt);
csa_status_t csa_index_topk(const void* q_idx, csa_dtype_t q_dt, const float* w, const void* k_idx,
                            csa_dtype_t k_dt, const float* k_scale, int B, int64_t T, int H_I,
                            int d_I, int64_t N_alloc, int64_t t0, int m, int top_k,
                            int32_t* out_idx, float* out_score, void* workspace,
                            size_t workspace_bytes, csa_stream_t stream);

/*
 * csa_index_topk_bf16 -- the approximate selector: csa_index_topk on scores
 * rounded to bf16.
 *
 * [digest] 七: the indexer's selector may rank bf16 scores, for speed, at a
 * small loss of recall against the exact selection.  Here each fp32 score
 * I(t, j) is rounded to the nearest bf16 value (ties to even) and the
 * selection is the exact top min(top_k, c(t)) of the rounded scores, ties to
 * the lower j (rounding makes ties common).  out_score holds the rounded
 * scores.  Arguments, limits, workspace (csa_index_topk_workspace) and errors
 * are those of csa_index_topk.
 */
csa_status_t csa_index_topk_bf16(const void* q_idx, csa_dtype_t q_dt, const float* w,
                                 const void* k_idx, csa_dtype_t k_dt, const float* k_scale, int B,
                                 int64_t T, int H_I, int d_I, int64_t N_alloc, int64_t t0, int m,
                                 int top_k, int32_t* out_idx, float* out_score, void* workspace,
                                 size_t workspace_bytes, csa_stream_t stream);

/*
 * csa_index_topk_fp8 -- csa_index_topk with fp8 x fp8 dot products.
 *
 * [digest] 七: the indexer's QK path runs in low precision, since its
 * activations are cached, loaded and multiplied there; [summary] 五: fp8
 * caches.  With keys already cached as e4m3 codes + one fp32 scale per entry,
 * the query is quantised the same way, one scale per (token, head) row:
 *     s[b,i,h] = max_d |q_idx[b,i,h,d]| / 448 in fp32 (NaN elements ignored;
 *                1 where the quotient is 0),
 *     code[d]  = e4m3 nearest-even of the fp32 quotient q_idx[b,i,h,d] / s,
 * and I(t, j) is computed on the quantised rows code * s.  The code dot
 * products run on the fp8 matrix cores, whose sums are not rounded like fp32
 * ones: within each group of 8 consecutive dims the products are aligned to
 * the largest one and the bits of the others below 2^-13 of its power of two
 * are dropped (the group sums then add in fp32), so each dot product may be
 * off by up to 7 * 2^-13 of its group's largest product per group, before the
 * scales apply.  The selection, ties, outputs, limits, workspace
 * (csa_index_topk_workspace with k_dt = CSA_FP8_E4M3) and errors are those of
 * csa_index_topk, on the scores so computed.
 *
 *   q_idx     [B, T, H_I, d_I] bf16;  k_idx [B, N_alloc, d_I] e4m3 codes;
 *   k_scale   [B, N_alloc] fp32 (required when N_alloc > 0).
 */
csa_status_t csa_index_topk_fp8(const void* q_idx, const float* w, const void* k_idx, const float* k_scale,
                                int B, int64_t T, int H_I, int d_I, int64_t N_alloc, int64_t t0, int m,
                                int top_k, int32_t* out_idx, float* out_score, void* workspace,
                                size_t workspace_bytes, csa_stream_t stream);

/*
 * csa_attend -- CSA core attention: selected compressed entries + raw window.
 *
 * [digest] 三: attention runs over the top-k compressed entries, and the newest
 * window tokens are added uncompressed.  For query i at t = t0 + i and head h,
 * over the multiset E(t) = {k_cmp/v_cmp rows idx[b,i,:] with 0 <= j < c(t)}
 * plus {k_raw/v_raw rows of positions max(0, t-window+1) .. t}:
 *     o[b,i,h,:] = sum_e softmax_e(scale * q[b,i,h,:] . K_e) * V_e
 *     lse[b,i,h] = ln sum_e exp(scale * q . K_e)
 * one softmax over both kinds of entry; an empty E gives o = 0, lse = -inf.
 * Listed indices that are negative, >= N_alloc or not yet visible
 * (j >= (t+1)/m) are skipped; a repeated index counts once per listing.
 *
 *   q        [B, T, H, d] of dt;  k_cmp, v_cmp [B, N_alloc, d] of kv_dt
 *   kv_dt    dt, or CSA_FP8_E4M3 (dt == CSA_BF16 only) for compressed caches of
 *            e4m3 codes with one fp32 scale per entry, as csa_compress writes
 *            them ([summary] 五: low-precision KV caches): the entry is
 *            code * scale.  k_scale, v_scale [B, N_alloc] fp32, 16-byte
 *            aligned, required iff kv_dt == CSA_FP8_E4M3 (else NULL).  The raw
 *            window rows stay of dt.
 *   idx      [B, T, top_k] int32 (top_k may be 0: window only)
 *   k_raw, v_raw [B, n_raw, d] of dt for positions raw_base ..; every window
 *            position of every query must be inside (else CSA_E_SHAPE).
 *   v may alias k (models with K = V).
 *   out      [B, T, H, d] of out_dt (CSA_F32 | CSA_BF16);  lse [B, T, H] fp32 or NULL
 *   dtypes   dt = CSA_BF16: d in {64, 128}, H % 16 == 0, H <= 128;
 *            dt = CSA_F32:  d in {32, 64, 128}, 1 <= H <= 32.
 *   limits   0 <= window <= 1024, 0 <= top_k <= 2048, m >= 1.
 */
size_t csa_attend_workspace(int B, int64_t T, int H, int d, int top_k, int window);
csa_status_t csa_attend(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                        csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                        int64_t N_alloc, int m, const int32_t* idx, int top_k, const void* k_raw,
                        const void* v_raw, int64_t raw_base, int64_t n_raw, int B, int64_t T,
                        int H, int d, int64_t t0, int window, float scale, void* out,
                        csa_dtype_t out_dt, float* lse, void* workspace, size_t workspace_bytes,
                        csa_stream_t stream);

/*
 * csa_attend_noalloc -- csa_attend on scratch that the library holds itself.
 *
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments, layouts,
 * numerics and errors are those of csa_attend, without the workspace pair:
 * the scratch is a static device array of CSA_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends, whose address is looked up on the first call
 * on each device (that call also enqueues one small fill kernel on `stream`
 * to clear its control words).  A shape whose csa_attend_workspace() exceeds
 * the scratch is rejected with CSA_E_WORKSPACE before anything is enqueued.
 * The call never allocates.  All calls on one GPU share its scratch, and each
 * call leaves the control words at zero for the next: calls that overlap on
 * one GPU (concurrent streams or threads) race and must be ordered.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (16u << 20)
csa_status_t csa_attend_noalloc(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                                csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                                int64_t N_alloc, int m, const int32_t* idx, int top_k, const void* k_raw,
                                const void* v_raw, int64_t raw_base, int64_t n_raw, int B, int64_t T,
                                int H, int d, int64_t t0, int window, float scale, void* out,
                                csa_dtype_t out_dt, float* lse, csa_stream_t stream);

/*
 * hca_attend -- HCA attention: every visible heavy entry + raw window, one softmax.
 *
 * [digest] 三 and [book] 4: HCA folds every m' tokens and attends densely to all
 * n/m' heavy entries (no top-k), plus the window.  E(t) = {heavy entries
 * j < min(N_alloc, (t+1)/m_heavy)} plus the raw window; the formulas, layouts,
 * dtypes (kv_dt, k_scale, v_scale included) and limits are those of csa_attend.
 */
size_t hca_attend_workspace(int B, int64_t T, int H, int d, int64_t N_alloc, int m_heavy,
                            int window);
csa_status_t hca_attend(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                        csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                        int64_t N_alloc, int m_heavy, const void* k_raw, const void* v_raw,
                        int64_t raw_base, int64_t n_raw, int B, int64_t T, int H, int d,
                        int64_t t0, int window, float scale, void* out, csa_dtype_t out_dt,
                        float* lse, void* workspace, size_t workspace_bytes, csa_stream_t stream);

/*
 * Per-kernel timing (diagnostics, not part of the method).  While enabled on the
 * calling thread, every kernel the library enqueues from that thread is
 * bracketed by two HIP events on its stream; the work itself is unchanged.
 * csa_profile_report waits for the recorded events, writes a JSON object
 * {"<kernel>": {"launches": n, "total_ms": t}, ...} into buf (truncated to n
 * bytes, NUL-terminated), forgets the records, and returns the JSON length
 * (-1 if an event query failed).  Do not enable it while capturing a graph.
 * csa_profile_enable returns the previous setting.
 */
int csa_profile_enable(int on);
int csa_profile_report(char* buf, size_t n);

/*
 * Diagnostics: the bandwidth a plain read reaches on the device (not part of
 * the method; the benchmark quotes it beside the kernels' rooflines).  Reads
 * `bytes` (a multiple of 16) from the device buffer `buf` (16-byte aligned)
 * with a streaming kernel of 8192 workgroups, each reading one contiguous
 * chunk with 16-byte loads, and writes to `sink` ([8192] uint32, device) only
 * when a checksum hits one fixed value, so that the loads are kept.
 */
csa_status_t csa_diag_stream_read(const void* buf, size_t bytes, uint32_t* sink, csa_stream_t stream);

/*
 * Diagnostics: the rate at which workgroups gather scattered rows, the access
 * pattern of the decode attention's selected entries (not part of the method;
 * the benchmark quotes it for the choice between split and whole decode rows).
 * `groups` workgroups of 512 threads; workgroup g reads, for each s <
 * per_group, row idx[g * per_group + s] of `k` and of `v` (n_rows rows of 256
 * bytes each: d = 128 in bf16; both 16-byte aligned, device), 16 lanes per
 * row and four rows of each per 16 lanes in flight, and writes to `sink`
 * ([groups] uint32, device) only when a checksum hits one fixed value, so that
 * the loads are kept.  idx: [groups * per_group] int32 (device); an index
 * outside [0, n_rows) is clamped into it, so no read leaves the buffers.
 * Errors: CSA_E_NULL (a NULL pointer), CSA_E_ALIGN, CSA_E_SHAPE (groups not
 * in [1, 65536], per_group not in [1, 4096], n_rows not in [1, 2^31)).
 */
csa_status_t csa_diag_gather_read(const void* k, const void* v, int64_t n_rows, const int32_t* idx,
                                  int64_t groups, int64_t per_group, uint32_t* sink, csa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
