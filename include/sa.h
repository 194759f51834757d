/*
 * sa.h -- C ABI of libsa.so: structured sparse prefill attention on AMD MI355X (gfx950).
 *
 * The method: causal prefill attention in which a per-head structured mask is
 * applied to the logits before softmax, so that only the retained (query i,
 * key j) pairs are computed.  Sources, cited by page title and section:
 *   [DAM]    Pith review of "DAM: Dynamic Attention Mask for Long-Context Large
 *            Language Model Inference Acceleration": "What carries the argument"
 *            (pattern pool, Box-Cox lambda = 0.5, tau = 0.3, overlap score gamma,
 *            mu = 0.8, extension to S x S, mask before softmax), "Referee Report"
 *            (Summary: A' = (Q K^T / sqrt(d_k)) (.) M; minor comment 1: epsilon),
 *            "Circularity Check" (step 1: extended mask = union of matched
 *            patterns; step 2: cost O(sL) with s retained keys per query).
 *   [Seer]   "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
 *            abstract: block-level (64 x 64) attention sparsity.
 *   [Anchor] "AnchorAttention: Difference-Aware Sparse Attention with Stripe
 *            Granularity", abstract: stripe-granularity sparsity for prefill.
 *   [SampleAttention] "SampleAttention: Near-Lossless Acceleration of Long Context
 *            LLM Inference with Adaptive Structured Sparse Attention", abstract:
 *            head-specific sparse patterns captured at runtime, per input.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  Structs are passed by
 *     host pointer; the device pointers inside them are read by the kernels.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on `stream` and returns, except where a call is documented to
 *     synchronise `stream`.
 *   - The library never allocates or frees device memory: the caller owns every
 *     buffer.  It keeps no state between calls; calls are thread-safe.
 *   - q, k, v, o and maps base addresses are 16-byte aligned (hipMalloc's are);
 *     a misaligned one is SA_ERR_INVALID_ARG.
 *   - Arguments are validated on the host before anything is enqueued: a negative
 *     return value means nothing was launched, except SA_ERR_HIP, which reports a
 *     failed launch.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sa_status;
#define SA_OK 0
#define SA_ERR_INVALID_ARG (-1)  /* null pointer, bad shape or size, inconsistent sizes */
#define SA_ERR_UNSUPPORTED (-2)  /* valid request outside what the library implements */
#define SA_ERR_DESC_INVALID (-3) /* descriptor contents not sorted/unique/in range */
#define SA_ERR_CAPACITY (-4)     /* an output array is smaller than the result */
#define SA_ERR_HIP (-5)          /* a HIP runtime call or kernel launch failed */

#define SA_DTYPE_F32 0
#define SA_DTYPE_BF16 1

/* Bits of sa_index.status (device int32). */
#define SA_STATUS_OVERFLOW 1     /* a fill stopped at an array's capacity */
#define SA_STATUS_DESC_INVALID 2 /* a descriptor list was unsorted, repeated or out of range */

/* Flags of sa_build_index. */
#define SA_BUILD_VALIDATE 1 /* check descriptor contents on the device (reported via sizes query) */

/* Text for a status code (host; static string, never NULL). */
const char* sa_status_string(sa_status s);
/* Library version string (host; static string). */
const char* sa_version(void);

/*
 * Pattern descriptor, one mask per QUERY head h in [0, n_heads), shared by every
 * batch element.  Pair (i, j) is retained iff j <= i < S and at least one holds:
 *   (i - j) in D_h          diagonal patterns  j = i - r        [DAM, pattern pool]
 *   j in C_h                vertical patterns  j = c, i >= c    [DAM, pattern pool]
 *   block_mask[h][i/bs][j/bs] != 0   bs = block_size           [Seer, block sparsity]
 *   j in stripe list (h, i / stripe_rows)                       [Anchor, stripes]
 * (the extended mask is the union of the patterns [DAM, Circularity Check 1]).
 *   diag_ptr  int32 [n_heads+1]  CSR row pointers into diag_off (diag_ptr[0] = 0)
 *   diag_off  int32 [diag_ptr[n_heads]]  per head strictly increasing, in [0, S)
 *   vert_ptr  int32 [n_heads+1]; vert_col int32 [...]: strictly increasing, in [0, S)
 *   block_mask  NULL, or uint8 [n_heads][nbq][nbq], nbq = ceil(S / block_size);
 *               entries above the block diagonal are ignored (causality).
 *   block_size  multiple of the index row block (64 or 128) when block_mask != NULL.
 *   stripe_ptr  NULL, or int64 [n_heads * nst + 1], nst = ceil(S / stripe_rows);
 *               list (h, t) = stripe_col[stripe_ptr[h*nst+t] .. stripe_ptr[h*nst+t+1])
 *   stripe_col  int32, strictly increasing within each list, in [0, S).
 *   stripe_rows multiple of the index row block when stripe_ptr != NULL.
 * The ptr arrays must be consistent with the allocation sizes of the arrays they
 * index (the library reads diag_off[diag_ptr[h] .. diag_ptr[h+1]) and so on).
 */
typedef struct sa_pattern_desc {
  int32_t S;
  int32_t n_heads;
  const int32_t* diag_ptr;
  const int32_t* diag_off;
  const int32_t* vert_ptr;
  const int32_t* vert_col;
  const uint8_t* block_mask;
  int32_t block_size;
  const int64_t* stripe_ptr;
  const int32_t* stripe_col;
  int32_t stripe_rows;
} sa_pattern_desc;

/* Element counts of the variable-length index arrays. */
typedef struct sa_index_sizes {
  int64_t n_runs;  /* run_lo / run_hi */
  int64_t n_segs;  /* seg_lo / seg_hi */
  int64_t n_bcols; /* bcol_idx */
  int64_t n_cols;  /* col_idx */
} sa_index_sizes;

/*
 * Canonical sparse index for one descriptor and one row block BM (the pages give
 * no index format; this is the layout the attention kernel consumes).  Row block
 * rb covers query rows [b0, b1] = [rb*BM, min(S, (rb+1)*BM) - 1]; item it = h*nb + rb.
 *   run_ptr [n_heads+1], run_lo/run_hi [n_runs]: maximal runs [lo, hi] of D_h.
 *   U(h, rb) = { j >= 0 : i - j in D_h for some i in [b0, b1] }: the key columns
 *              the diagonals touch inside the row block.
 *   seg_ptr [n_items+1] (int64), seg_lo/seg_hi [n_segs]: maximal intervals of U, ascending.
 *   X(h, rb) = verticals <= b1, columns of the blocks in block row b0/bs (<= b1),
 *              columns of stripe list (h, b0/stripe_rows) (<= b1).
 *   bcol_ptr [n_items+1] (int64), bcol_idx: X intersect U, ascending.
 *   col_ptr  [n_items+1] (int64), col_idx:  X minus U, ascending.
 *   pair_count [n_heads] (int64): exact number of retained pairs per head
 *              (the retained keys s per query, summed [DAM, Circularity Check 2]).
 *   dbits    uint32 [n_heads][ceil(S/32)]: bit r of head h (word r/32, bit r%32) is set
 *              iff r is in D_h (the diagonal offsets as a bitmap).
 *   status   int32 [1]: SA_STATUS_* bits raised by the last build (0 = clean).
 * Every retained pair is computed exactly once by the attention kernel: pairs with
 * j in U in the segment phase (retained iff (i-j) in D_h or j in bcols), the others
 * in the gathered phase (j in cols).  S, n_heads, row_block and n_row_blocks are
 * host values; `capacity` holds the host-side element capacities of run_lo/run_hi,
 * seg_lo/seg_hi, bcol_idx and col_idx.
 */
typedef struct sa_index {
  int32_t S;
  int32_t n_heads;
  int32_t row_block;
  int32_t n_row_blocks;
  int32_t* run_ptr;
  int32_t* run_lo;
  int32_t* run_hi;
  int64_t* seg_ptr;
  int32_t* seg_lo;
  int32_t* seg_hi;
  int64_t* bcol_ptr;
  int32_t* bcol_idx;
  int64_t* col_ptr;
  int32_t* col_idx;
  int64_t* pair_count;
  uint32_t* dbits;
  int32_t* status;
  sa_index_sizes capacity;
} sa_index;

/*
 * sa_build_index: descriptor -> canonical index (count, exclusive scan, fill; all on
 * the device).  idx->S, n_heads, row_block (64 or 128), n_row_blocks = ceil(S/BM) and
 * the fixed-size arrays run_ptr, seg_ptr, bcol_ptr, col_ptr, pair_count, dbits and
 * status must be set.
 * Size query: if `sizes` (host) is non-NULL, the call synchronises `stream` after the
 *   counting pass, writes the totals to *sizes and returns SA_ERR_DESC_INVALID if
 *   validation (flags & SA_BUILD_VALIDATE) found a bad descriptor.  If any of run_lo,
 *   run_hi, seg_lo, seg_hi, bcol_idx, col_idx is NULL the call stops after the counts
 *   (sizes must then be non-NULL); pair_count and dbits are then not yet valid (the
 *   counting pass uses dbits as scratch; the fill writes both).
 * Fill: with every array present the call recounts and fills; it stays asynchronous
 *   when sizes == NULL.  A fill that would exceed a capacity stops at the capacity and
 *   raises SA_STATUS_OVERFLOW in idx->status (SA_ERR_CAPACITY is returned directly
 *   when `sizes` was requested and shows the shortfall).
 * Limits: 1 <= S <= 262144 (the per-block bitmap lives in LDS), n_heads >= 1.
 * Errors: SA_ERR_INVALID_ARG (nulls, shapes, row_block not dividing block_size or
 *   stripe_rows), SA_ERR_UNSUPPORTED (S above the limit), SA_ERR_DESC_INVALID,
 *   SA_ERR_CAPACITY, SA_ERR_HIP.
 */
sa_status sa_build_index(const sa_pattern_desc* desc, sa_index* idx, sa_index_sizes* sizes, int32_t flags,
                         void* stream);

/*
 * sa_build_index_workspace_bytes (host): bytes of device scratch a build of `desc` at
 * row block `row_block` needs beyond the index arrays.  Always 0 here: the counting
 * pass keeps its per-item counts in the index's own pointer arrays and scans them in
 * place, and the per-item kinds ride in the dbits array until the fill writes it, so
 * sa_build_index takes no workspace argument.  Provided so that a caller written
 * against a workspace-taking build can size (and skip) its allocation.  desc may be NULL.
 */
size_t sa_build_index_workspace_bytes(const sa_pattern_desc* desc, int32_t row_block);

/*
 * sa_sparse_attn_prefill: O = softmax(mask(Q K^T * scale)) V over retained pairs
 * only [DAM, Referee Report Summary; What carries the argument: masked pairs get
 * zero weight, read as logit -inf].
 *   q, o  [batch][hq][S][head_dim], k, v [batch][hkv][S][head_dim], contiguous,
 *         element type `dtype` (SA_DTYPE_BF16 or SA_DTYPE_F32); o has q's type.
 *   lse   NULL or float [batch][hq][S]: natural-log log-sum-exp of the scaled
 *         retained logits; -inf for a row without retained keys (whose o row is 0).
 *   query head h reads kv head h / (hq / hkv) (hq % hkv == 0).
 *   softmax_scale <= 0 selects 1 / sqrt(head_dim).
 *   head_dim in {64, 128}.  idx: built for this S with n_heads == hq.
 * bf16: bf16 MFMA products with fp32 accumulation, fp32 online softmax, probabilities
 * rounded to bf16 for the P.V product, output rounded to bf16 (nearest even).
 * f32: fp32 MFMA throughout.
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_HIP.
 */
sa_status sa_sparse_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int32_t batch, int32_t hq, int32_t hkv, int32_t S, int32_t head_dim,
                                 int32_t dtype, float softmax_scale, const sa_index* idx, void* stream);

/*
 * sa_sparse_attn_decode: one new query row per sequence against a K/V cache
 * [DAM, Referee Report Summary; What carries the argument], i.e. row pos[b] of the
 * prefill output when Q[b][h][pos[b]] is q[b][h]: the keys are the cache rows
 * j <= pos[b] that the mask retains for row pos[b], masked logits get no weight.
 *   q, o  [batch][hq][head_dim], element type `dtype`; o has q's type.
 *   k, v  [batch][hkv][S][head_dim] (the cache; rows > pos[b] are never read).
 *   pos   int32 [batch] (device): the query position of each sequence,
 *         0 <= pos[b] < S; a position outside that range gives o = 0, lse = -inf.
 *   lse   NULL or float [batch][hq] (natural log; -inf without retained keys).
 *   softmax_scale, head_dim, GQA mapping and idx as for sa_sparse_attn_prefill
 *   (the index is the prefill index of the same patterns and S).
 * Arithmetic: fp32 dot products and online softmax (exp2 domain), fp32 P.V.
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_HIP.
 */
sa_status sa_sparse_attn_decode(const void* q, const void* k, const void* v, const int32_t* pos, void* o, float* lse,
                                int32_t batch, int32_t hq, int32_t hkv, int32_t S, int32_t head_dim, int32_t dtype,
                                float softmax_scale, const sa_index* idx, void* stream);

/*
 * sa_attention_maps [DAM, What carries the argument: average attention maps of the
 * first L (pattern capture length) positions, accumulated over the inputs;
 * Assumptions & free parameters: the batch mean stands in for each sequence]:
 *   maps[h][i][j] = (1/batch) sum_b softmax_j( q[b][h][i] . k[b][g][j] * scale ),
 *                   the softmax over j <= i;  maps[h][i][j] = 0 for j > i,
 *   g = h / (hq / hkv); softmax_scale <= 0 selects 1 / sqrt(head_dim).
 *   q [batch][hq][L][head_dim], k [batch][hkv][L][head_dim]: element type `dtype`.
 *   maps  float [hq][L][L] (every element written): the input of sa_pattern_capture.
 * Arithmetic: fp32 MFMA scores, fp32 softmax (exp2 domain), batch mean accumulated
 * in element order b = 0, 1, ...
 * Limits: 1 <= L <= 4096, head_dim 64 or 128.
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_HIP.
 */
sa_status sa_attention_maps(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t L,
                            int32_t head_dim, int32_t dtype, float softmax_scale, float* maps, void* stream);

/*
 * sa_pattern_capture [DAM, What carries the argument; Referee Report major comment 4
 * for lambda, tau and mu other than the pages' values]: for each averaged attention
 * map A (float [n_maps][L][L], row-major; entries with j > i are ignored):
 *   y = Box-Cox(A + eps): (x^lambda - 1) / lambda, log x at lambda = 0; the
 *       pages' lambda = 0.5 is computed as (sqrt(x) - 1) / 0.5
 *   t = (y - ymin) / (ymax - ymin)      min/max over the causal row (norm_scope 0)
 *                                       or over the causal map (norm_scope 1);
 *                                       a constant row/map gives t = 1
 *   M = (t >= tau)                      the binary true mask (t = 1 on a constant row)
 *   diag_hits[r] = sum_i M[i][i-r], vert_hits[c] = sum_i M[i][c]
 *   keep_diag[r] = hits / (L - r) >= mu, keep_vert[c] = hits / (L - c) >= mu
 * All of it in fp64.  At lambda = 0.5 sqrt and division are correctly rounded, so
 * the keep flags, hit counts and mask are exact; other lambdas use the device pow /
 * log (a few ulp), so a cell whose t lies within about 1e-15 of tau may differ
 * from a correctly rounded evaluation.  eps: 1e-8 in one section of the paper,
 * 1e-10 in its appendix [DAM, Referee Report minor comment 1] -- a parameter here.
 * Requires every causal entry finite with A + eps >= 0 (attention probabilities).
 *   keep_diag, keep_vert  uint8 [n_maps][L];  diag_hits, vert_hits NULL or int32
 *   [n_maps][L];  true_mask NULL or uint8 [n_maps][L][L] (zeros above the diagonal).
 * Limits: 1 <= L <= 4096; lambda finite, and eps > 0 when lambda <= 0 (else
 * SA_ERR_INVALID_ARG); norm_scope 0 or 1.
 */
sa_status sa_pattern_capture(const float* maps, int32_t n_maps, int32_t L, double lambda, double eps, double tau,
                             double mu, int32_t norm_scope, uint8_t* keep_diag, uint8_t* keep_vert,
                             int32_t* diag_hits, int32_t* vert_hits, uint8_t* true_mask, void* stream);

/*
 * sa_pattern_coverage [DAM, Referee Report major comments 2 and 4: agreement of the
 * kept masks with the attention maps, and their sparsity]: per map m,
 *   cells[m] = #{ (i, j) : j <= i < L, keep_diag[m][i - j] or keep_vert[m][j] }
 *   mass[m]  = sum of A over those cells / sum of A over j <= i  (0 if that is 0)
 *   maps  float [n_maps][L][L] as for sa_pattern_capture;  keep_* uint8 [n_maps][L]
 *   mass  double [n_maps];  cells  NULL or int64 [n_maps]
 * fp64 sums in a fixed order (deterministic; the order differs from a plain
 * row-major sum, so mass agrees with one to rounding).
 * Limits: 1 <= L <= 4096.  Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_HIP.
 */
sa_status sa_pattern_coverage(const float* maps, int32_t n_maps, int32_t L, const uint8_t* keep_diag,
                              const uint8_t* keep_vert, double* mass, int64_t* cells, void* stream);

/*
 * sa_sample_scores [SampleAttention, abstract: head-specific sparse patterns captured
 * at runtime, per input, at low cost; DAM, What carries the argument: the pattern
 * pool of diagonals j = i - r and verticals j = c]: the query rows
 * i = row0 .. row0 + n_rows - 1 of every sequence take their causal softmax over
 * the keys j <= i (scores q_i . k_j * scale, kv head h / (hq / hkv)), and each
 * row's probabilities on the pairs not covered yet -- outside the local window
 * (i - j >= band) and off the columns marked in skip_cols -- are ADDED onto its
 * head's pattern scores:
 *   diag_score[h][r] += sum of p_i(i - r), rounded to units of 2^-32 per partial sum
 *   vert_score[h][c] += sum of p_i(c), rounded to units of 2^-32 per partial sum
 * (partial sums: fp32, in a fixed order, over the rows of a 32-row chunk and the
 * sequences of the batch for a column, over a 32-row, 32-key block for a diagonal);
 * int64 fixed point, so the sums are exact integer sums whatever the order of the
 * atomics (deterministic); the caller zeroes both arrays first and may call again
 * with other row blocks to accumulate.  Each sampled row holds 2^32 units in all
 * (its probabilities sum to 1), the window and skipped columns included.
 *   q [batch][hq][S][head_dim], k [batch][hkv][S][head_dim]: element type `dtype`.
 *   skip_cols  NULL or uint8 [hq][S] (nonzero: column already kept).
 *   row_lse  float [batch][hq][n_rows]: natural-log LSE of each sampled row over all
 *            its keys; written, or read when lse_given is nonzero (a second call
 *            over the same rows skips that pass).
 *   workspace  device scratch of at least sa_sample_scores_workspace(...) bytes,
 *            8-byte aligned, used when lse_given is 0 (partial row statistics per
 *            256-key split); may be NULL when lse_given is nonzero.
 *   diag_score, vert_score  int64 [hq][S], 8-byte aligned; either may be NULL to skip
 *            that family (not both), e.g. verticals only for the first stage.
 * Arithmetic: fp32 MFMA scores, fp32 softmax (exp2 domain), as for attention.
 * Limits: 0 <= row0, 1 <= n_rows <= 2048, row0 + n_rows <= S, batch * n_rows <= 2^20,
 * band >= 0; head_dim 64 or 128.  softmax_scale <= 0 selects 1 / sqrt(head_dim).
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_CAPACITY (workspace too
 * small), SA_ERR_HIP.
 */
sa_status sa_sample_scores(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                           int32_t head_dim, int32_t dtype, float softmax_scale, int32_t row0, int32_t n_rows,
                           int32_t band, const uint8_t* skip_cols, int32_t lse_given, float* row_lse,
                           void* workspace, size_t workspace_bytes, int64_t* diag_score, int64_t* vert_score,
                           void* stream);

/* Bytes of workspace sa_sample_scores needs (host; 0 for invalid sizes):
 * batch * hq * n_rows * ceil((row0 + n_rows) / 256) * 8. */
size_t sa_sample_scores_workspace(int32_t batch, int32_t hq, int32_t row0, int32_t n_rows);

/*
 * sa_sample_scores_noalloc: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Computes
 * exactly what sa_sample_scores computes, with the same arguments minus the workspace,
 * and the same kernels: the LSE pass keeps its per-split row statistics in a static
 * device array of the library, 16 MiB (16777216 bytes) per GPU, which each GPU the
 * library runs on holds until the process ends.  The call allocates nothing and calls
 * no allocating routine; the caller still owns q, k, skip_cols, row_lse and the scores.
 * Its first call on a device (with that device current) looks up the array's address
 * on that device once.
 *   The scratch need, batch * hq * n_rows * ceil((row0 + n_rows) / 256) * 8 bytes (as
 *   sa_sample_scores_workspace reports), must not exceed 16 MiB: else SA_ERR_CAPACITY
 *   and nothing is launched (e.g. 32 heads, 128 sampled rows, S up to 131072 fit).
 *   With lse_given nonzero no scratch is used.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on two
 * streams, or from two host threads) race and may corrupt each other's row LSE; order
 * them.  The array needs no clearing (every slot a call reads, that call writes first).
 * Errors: as sa_sample_scores (SA_ERR_CAPACITY: the scratch need is above 16 MiB).
 */
sa_status sa_sample_scores_noalloc(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                                   int32_t head_dim, int32_t dtype, float softmax_scale, int32_t row0, int32_t n_rows,
                                   int32_t band, const uint8_t* skip_cols, int32_t lse_given, float* row_lse,
                                   int64_t* diag_score, int64_t* vert_score, void* stream);

/*
 * sa_select_patterns [SampleAttention, abstract: adaptive, head-specific selection,
 * near-lossless; the rule is this library's reading]: for one pattern family, per
 * head h, scores v[0..S) as sa_sample_scores makes them over `rows` sampled row
 * sequences (batch * n_rows):
 *   T_all = rows * 2^32 (all sampled mass);  T = sum v (the mass not covered yet);
 *   need = ceil(alpha * (double)T_all) - (T_all - T): what this family must add so
 *          that the covered mass reaches alpha of T_all;
 *   need <= 0: nothing is kept;  need > T: every pattern with v > 0 is kept;
 *   else theta = the largest score value with sum of { v : v >= theta } >= need,
 *        keep[x] = (v[x] >= theta and v[x] > 0): the fewest top-scoring patterns,
 *        ties at theta all kept.
 *   Patterns x < band are always kept (the local window, for the diagonal family).
 * The two-stage use: columns first (scores with skip_cols = NULL, band = the
 * window), then diagonals (scores with skip_cols = the kept columns); the window,
 * the columns and the diagonals then hold at least alpha of the sampled mass.
 * Exact integer arithmetic (the product alpha * T_all is one IEEE double rounding).
 *   scores  int64 [n_heads][S] (>= 0, 8-byte aligned);  keep  uint8 [n_heads][S].
 * Limits: 0 < alpha <= 1, 1 <= rows <= 2^30, band >= 0.
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_HIP.
 */
sa_status sa_select_patterns(const int64_t* scores, int32_t n_heads, int32_t S, double alpha, int64_t rows,
                             int32_t band, uint8_t* keep, void* stream);

/*
 * sa_patterns_to_desc [DAM, What carries the argument; Circularity Check 1]: the kept
 * patterns of each map are pasted into an S x S mask, i.e. the per-head descriptor
 * lists at length S are D_h = { r : keep_diag[h][r], r < S } and
 * C_h = { c : keep_vert[h][c], c < S }.
 *   keep_diag, keep_vert  uint8 [n_maps][L]   (one map per query head)
 *   diag_ptr, vert_ptr    int32 [n_maps + 1]
 *   diag_off, vert_col    int32, capacity n_maps * min(L, S) each (always enough)
 */
sa_status sa_patterns_to_desc(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t n_maps, int32_t L,
                              int32_t S, int32_t* diag_ptr, int32_t* diag_off, int32_t* vert_ptr,
                              int32_t* vert_col, void* stream);

/*
 * Calibration (measurement support; computes nothing of the method).
 *
 * sa_calib_mfma_bf16: n_workgroups workgroups of 256 threads each run `iters` rounds of
 *   four independent 32x32x16 bf16 MFMAs per wave from registers, i.e.
 *   n_workgroups * 4 waves * iters * 4 * 32768 flops; the caller times the launch.
 *   sink float [n_workgroups * 256] receives one value per thread.
 * sa_calib_gather: n_workgroups workgroups of 256 threads each read reads_per_workgroup
 *   chunks of chunk_bytes at pseudo-random chunk-aligned offsets (splitmix64 of seed,
 *   workgroup and read index) of buf[0 .. region_bytes), with 16-byte loads:
 *   n_workgroups * reads_per_workgroup * chunk_bytes bytes requested.  buf 16-byte
 *   aligned; chunk_bytes a multiple of 16, at most region_bytes; sink as above.
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_HIP.
 */
sa_status sa_calib_mfma_bf16(int32_t n_workgroups, int32_t iters, float* sink, void* stream);
sa_status sa_calib_gather(const void* buf, int64_t region_bytes, int32_t chunk_bytes, int32_t n_workgroups,
                          int32_t reads_per_workgroup, uint64_t seed, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
