/*
 * kalm.h -- C ABI of the KaLM-Reranker-V1 hot-path library (libkalm.so), gfx950.
 *
 * The library computes the data-parallel hot path of the "fast but not late
 * interaction" reranker: chunk pooling of passage encoder states, the cross
 * K/V projection of the pooled vectors, the merged self+cross attention of
 * the decoder and the yes/no relevance score, plus the linear layers and row
 * layout that chain them into a decoder stack, the ranking of the scores, the
 * split forms of the merged attention (self part once, cross part resumed or
 * in split-KV shares) and the optional parts of a model-shaped layer (RMSNorm,
 * RoPE, gated GELU).
 *
 * Page citations (by page title and section):
 *   [MLX]  "KaLM-Reranker-V1-Nano -- MLX (Apple Silicon)": What this is, Speed.
 *   [Q4KM] "KaLM-Reranker-V1-Small Q4_K_M GGUF": Score a pair, Runtime boundaries,
 *          Troubleshooting.
 *   [Q80]  "KaLM-Reranker-V1-Large Q8_0 GGUF": Frozen inference contract,
 *          Score one query-passage pair, Runtime limitations.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or keeps them.  Layouts are row-major and contiguous unless a
 *    leading dimension (ld, in elements) is given.  Data pointers must be 16-byte
 *    aligned.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream).  The caller synchronises.
 *  - Arguments are validated on the host before anything is launched; a bad
 *    argument returns KALM_ERR_INVALID_ARG, an unsupported shape or dtype
 *    KALM_ERR_UNSUPPORTED, a failed launch KALM_ERR_LAUNCH.  kalm_last_error()
 *    then returns a thread-local message.
 *  - There is no CPU fallback.  Without a usable GPU every call returns
 *    KALM_ERR_NO_DEVICE (the same stance as the --require-gpu guard in [Q4KM]
 *    Troubleshooting and [Q80] Score one query-passage pair).
 *  - Every output element is written, padded positions included (except the rows
 *    of pairs an entry point documents as skipped), so results are
 *    deterministic run to run (no atomics in any reduction).
 *  - Calls keep no state between them and may be made from several host threads.
 */
#ifndef KALM_H
#define KALM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KALM_OK = 0,
  KALM_ERR_INVALID_ARG = 1,
  KALM_ERR_UNSUPPORTED = 2,
  KALM_ERR_NO_DEVICE = 3,
  KALM_ERR_LAUNCH = 4,
  KALM_ERR_BOUNDS = 5 /* debug build only: a kernel's index guard fired (see kalm_debug_build) */
} kalm_status;

typedef enum { KALM_F32 = 0, KALM_BF16 = 1 } kalm_dtype;

/* Library version, major*10000 + minor*100 + patch (0.2.0: split attention,
 * one-layer final rows, layer parts; 0.3.0: fused gate/up projection and
 * activation; 0.4.0: every layer's cross K/V in one call, 64-bit pair layout). */
int32_t kalm_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* kalm_last_error(void);

/* 1 in the debug build of the library (libkalm_debug.so, compiled with
 * -DKALM_DEBUG), 0 in the release build (libkalm.so).  Both export the same
 * entry points and run the same kernels.  Every kernel guards its
 * data-dependent indexes in both builds: a pair whose rows fall outside the
 * given row counts is skipped, a passage index outside [0, D), a residual
 * source row, gathered row or final row outside its array gives NaN outputs, a
 * RoPE row outside X is left alone, and a pair layout past INT32_MAX gives -1
 * offsets.  In the debug build each guard that fires is also recorded, and
 * every entry point synchronises its stream after its launches and returns
 * KALM_ERR_BOUNDS (with kalm_last_error naming the guard) instead of KALM_OK;
 * a kernel fault is reported as KALM_ERR_LAUNCH against the call that ran it.
 * Because it synchronises, the debug build cannot be captured into a HIP graph,
 * and concurrent calls on one device share its guard record. */
int32_t kalm_debug_build(void);

/* KALM_OK when a gfx950 device is visible, KALM_ERR_NO_DEVICE otherwise. */
kalm_status kalm_device_check(void);

/*
 * a0 -- ragged batch layout.  Every query is paired with every one of n_docs
 * passages ([MLX] Speed: one document set reranked against many queries);
 * pair p joins query p / n_docs with doc p % n_docs; its decoder rows are packed
 * after those of pair p-1, and its score is read at its last row ([MLX] What
 * this is: the decoder's final position).
 *
 *   lq        [n_queries] int32   decoder length of each query, 1..max (device)
 *   cu_q      [P+1] int32 out     row offsets, cu_q[0] = 0, P = n_queries*n_docs
 *   doc_of_pair, final_row [P] int32 out
 *   h0_row    [rows] int32 out, nullable: row of the query's first-layer hidden
 *             state (queries packed in order) that pair row r starts from
 *   rows      capacity of h0_row; must equal n_docs * sum(lq) when h0_row is given
 *   h0_final  [P] int32 out, nullable: that row for the pair's final position
 *             (the query's last row in the per-query packing)
 *   cu_u      [n_queries+1] int32 out, nullable: row offsets of the per-query
 *             packing itself (cu_u[0] = 0; the layout with n_docs = 1)
 * Row offsets are computed in 64 bits on the device (the lengths live there).
 * A pair whose rows would extend past INT32_MAX gets cu_q = final_row =
 * h0_final = -1, and cu_q[P] (cu_u[n_queries]) is -1 when the total does not
 * fit: the attention entry points skip such pairs and kalm_yesno_score gives
 * them NaN, so an oversized batch never wraps into valid-looking rows.
 */
kalm_status kalm_pair_layout(const int32_t* lq, int32_t n_queries, int32_t n_docs,
                             int32_t* cu_q, int32_t* doc_of_pair, int32_t* final_row,
                             int32_t* h0_row, int64_t rows, int32_t* h0_final, int32_t* cu_u,
                             void* stream);

/*
 * a1 -- chunk pooling ([Q80] Frozen inference contract: masked mean over
 * consecutive groups of 4 encoder tokens under right padding; [MLX] What this
 * is: chunk size 4, masked mean per chunk; [Q4KM] Runtime boundaries: encoder
 * chunk size 4, at most 1024 tokens).
 *
 *   x           [D, T, H] dtype dt (F32 or BF16); padded tokens are never read
 *   token_mask  [D, T] uint8, nonzero = valid token (any 0/1 pattern is allowed)
 *   chunk       tokens per chunk, 1..64 (4 in the model)
 *   pooled      [D, Cmax, H] dtype dt out, Cmax = ceil(T / chunk); chunk c of doc d
 *               is the mean of the valid tokens among [c*chunk, (c+1)*chunk): fp32
 *               sum, one IEEE division by the count, one round to dt; a chunk with
 *               no valid token is written as 0
 *   chunk_mask  [D, Cmax] uint8 out, 1 iff the chunk has a valid token
 *   n_chunks    [D] int32 out, number of chunks with chunk_mask = 1
 * Requires H % 8 == 0 (BF16) or H % 4 == 0 (F32), T >= 1.
 */
kalm_status kalm_chunk_pool(const void* x, const uint8_t* token_mask, int32_t D, int32_t T,
                            int32_t H, int32_t chunk, kalm_dtype dt, void* pooled,
                            uint8_t* chunk_mask, int32_t* n_chunks, void* stream);

/*
 * a2 -- cross K/V projection of the cached pooled passage vectors ([MLX] What
 * this is: cross-attention KV computed over the cached passage encodings).
 * One bias-free linear map with both projections stacked:
 *   KVc[r, 0:kv_dim]        = pooled[r] . Wkv[0:kv_dim]^T          (keys)
 *   KVc[r, kv_dim:2*kv_dim] = pooled[r] . Wkv[kv_dim:2*kv_dim]^T   (values)
 *
 *   pooled    [D*Cmax, H] dtype dt
 *   chunk_mask [D*Cmax] uint8, nullable: rows whose mask byte is 0 are written as
 *             0 without being computed (padded chunks of right-padded passages)
 *   Wkv       [2*kv_dim, H] dtype dt ([out, in] layout)
 *   KVc       [D*Cmax, 2*kv_dim] dtype dt out (fp32 accumulation, one rounding)
 * Requires H % 8 == 0 and kv_dim % 4 == 0.
 */
kalm_status kalm_cross_kv(const void* pooled, const uint8_t* chunk_mask, int32_t D, int32_t Cmax,
                          int32_t H, const void* Wkv, int32_t kv_dim, kalm_dtype dt, void* KVc,
                          void* stream);

/*
 * a2 for every layer of a stack at once ([MLX] What this is: the cross K/V of
 * the cached passage encodings; each layer has its own projection and the
 * pooled vectors are shared by all layers): one GEMM over the layers' stacked
 * weights, the same arithmetic as n_layers calls of kalm_cross_kv.
 *   KVc[r, l, 0:kv_dim]        = pooled[r] . Wkv[l, 0:kv_dim]^T          (keys)
 *   KVc[r, l, kv_dim:2*kv_dim] = pooled[r] . Wkv[l, kv_dim:2*kv_dim]^T   (values)
 *
 *   pooled    [D*Cmax, H] dtype dt
 *   chunk_mask [D*Cmax] uint8, nullable: rows whose mask byte is 0 are written as
 *             0 for every layer (whole tiles of such rows are not computed)
 *   Wkv       [n_layers, 2*kv_dim, H] dtype dt (each layer in [out, in] layout)
 *   KVc       [D*Cmax, n_layers, 2*kv_dim] dtype dt out: layer l's keys of row r
 *             start at element (r*n_layers + l)*2*kv_dim, so a layer's K (or V)
 *             is a view with row stride n_layers*2*kv_dim elements (the c_ld of
 *             kalm_merged_attn)
 * Requires H % 8 == 0 (bf16) or H % 4 == 0 (f32), kv_dim % 4 == 0, n_layers >= 1,
 * 2*kv_dim*n_layers < 2^31.
 */
kalm_status kalm_cross_kv_layers(const void* pooled, const uint8_t* chunk_mask, int32_t D, int32_t Cmax,
                                 int32_t H, const void* Wkv, int32_t kv_dim, int32_t n_layers, kalm_dtype dt,
                                 void* KVc, void* stream);

/*
 * a3 -- merged self+cross attention ([MLX] What this is: one scaled-dot-product
 * attention whose KV is the decoder's self KV concatenated with the cross KV of
 * the cached passage).  For pair p, query head h and pair-local row i:
 *   o = softmax( [q.k_self_j * scale]_{j<=i}  U  [q.k_cross_c * scale]_{chunk_mask[doc,c]} )
 *       . [v_self ; v_cross]
 * in one softmax (single pass, online rescaling across the self/cross boundary).
 * Query head h reads KV head h / (nq / nkv).
 *
 *   Q         [rows, *] dtype dt, row stride q_ld; head h at columns h*d .. h*d+d-1
 *   Ks, Vs    [rows, *] dtype dt, row stride kv_ld; KV head g at columns g*d ..
 *   cu_q      [P+1] int32 row offsets (non-decreasing, cu_q[P] <= rows; a pair
 *             whose rows fall outside [0, rows) is skipped, its outputs not written)
 *   max_lq    >= every pair's length cu_q[p+1]-cu_q[p]; rows of a pair beyond
 *             max_lq are not computed (the caller's contract)
 *   Kc, Vc    [D*Cmax, *] dtype dt, row stride c_ld; doc d's chunk c is row d*Cmax+c
 *   chunk_mask[D, Cmax] uint8; doc_of_pair [P] int32 in [0, D) (a pair with an
 *             out-of-range doc gets NaN outputs)
 *   O         [rows, *] dtype dt out, row stride o_ld, same head columns as Q
 *   lse       [rows, nq] float out, nullable: natural-log log-sum-exp of the
 *             scaled logits of each row
 * Requires nq % nkv == 0; BF16: d == 256 (the model's head dim); F32: d <= 256,
 * d % 32 == 0; ld values multiples of 8.
 */
kalm_status kalm_merged_attn(const void* Q, int64_t q_ld, const void* Ks, const void* Vs,
                             int64_t kv_ld, const int32_t* cu_q, int32_t P, int64_t rows,
                             int32_t max_lq, const void* Kc, const void* Vc, int64_t c_ld,
                             const uint8_t* chunk_mask, const int32_t* doc_of_pair, int32_t D,
                             int32_t Cmax, int32_t nq, int32_t nkv, int32_t d, float scale,
                             kalm_dtype dt, void* O, int64_t o_ld, float* lse, void* stream);

/*
 * a3 with a choice of query rows (the same operation as kalm_merged_attn).
 * The pair's self keys are its Lq = cu_q[p+1] - cu_q[p] decoder positions;
 * row_mode selects which query rows are computed and where the rows live:
 *   0  every position of every pair; Q, Ks/Vs and O rows of pair p start at
 *      cu_q[p] (exactly kalm_merged_attn; q_rows = kv_rows = o_rows = rows).
 *   1  only the final position Lq-1 of each pair (it sees all Lq self keys):
 *      Q row p and O/lse row p; Ks/Vs rows start at cu_q[p].  The score is read
 *      at the decoder's final position only ([MLX] What this is), so the last
 *      layer needs no other row.
 *   2  rows shared by the D passages of a query: with the kalm_pair_layout
 *      layout (pair p = query p / D, passage p % D), Q and Ks/Vs rows are the
 *      query's rows in a per-query packing, starting at cu_q[(p/D)*D] / D;
 *      O/lse rows start at cu_q[p].  While every passage of a query still
 *      holds the query's own hidden states (the decoder models the query,
 *      [MLX] What this is; one passage set reranked against many queries,
 *      [MLX] Speed), their Q/K/V projections are one set of rows.
 *   3  the final position of the shared rows: Q row cu_q[(p/D)*D] / D + Lq-1
 *      (the query's last row in the per-query packing), Ks/Vs rows as mode 2,
 *      O/lse row p.  A one-layer stack needs nothing else: its only layer is
 *      both the first and the last.
 *   q_rows, kv_rows, o_rows  rows in Q, in Ks/Vs and in O (and lse); a pair
 *      whose rows fall outside them is skipped (its outputs are not written).
 * Other arguments as kalm_merged_attn; row_mode outside 0..3 is
 * KALM_ERR_INVALID_ARG.
 */
kalm_status kalm_merged_attn_rows(const void* Q, int64_t q_ld, int64_t q_rows, const void* Ks,
                                  const void* Vs, int64_t kv_ld, int64_t kv_rows, const int32_t* cu_q,
                                  int32_t P, int32_t max_lq, const void* Kc, const void* Vc,
                                  int64_t c_ld, const uint8_t* chunk_mask, const int32_t* doc_of_pair,
                                  int32_t D, int32_t Cmax, int32_t nq, int32_t nkv, int32_t d,
                                  float scale, kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows,
                                  float* lse, int32_t row_mode, void* stream);

/*
 * a3 split at the self/cross boundary.  The merged softmax over [self keys ;
 * cross keys] equals the log-sum-exp merge of a softmax over the self keys
 * alone and one over the cross keys alone ([MLX] What this is: one attention
 * over the concatenated KV; the merge is the usual online-softmax identity).
 * While every passage of a query still holds the query's own hidden states
 * (the first decoder layer; one passage set reranked against many queries,
 * [MLX] Speed), the self part is the same for all of the query's passages:
 * kalm_self_attn_partial computes it once per query and
 * kalm_merged_attn_resume finishes each pair from it with the passage's cross
 * keys.
 *
 * kalm_self_attn_partial -- plain causal self-attention of n_seq packed
 * sequences (the merged attention with no visible cross key):
 *   Q, Ks, Vs   as kalm_merged_attn, rows cu_s[i] .. cu_s[i+1]-1 of sequence i
 *   cu_s        [n_seq+1] int32 row offsets (kalm_pair_layout's cu_u gives the
 *               per-query packing); max_len >= every length
 *   O           [rows, *] float out, row stride o_ld (elements): the normalised
 *               self output of each row and head, fp32 for both dtypes
 *   lse         [rows, nq] float out, required: log-sum-exp of the scaled self
 *               logits (natural log)
 * Requires what kalm_merged_attn requires (bf16: d == 256, o_ld % 8 == 0,
 * 16-byte aligned pointers).
 */
kalm_status kalm_self_attn_partial(const void* Q, int64_t q_ld, const void* Ks, const void* Vs,
                                   int64_t kv_ld, int64_t rows, const int32_t* cu_s, int32_t n_seq,
                                   int32_t max_len, int32_t nq, int32_t nkv, int32_t d, float scale,
                                   kalm_dtype dt, float* O, int64_t o_ld, float* lse, void* stream);

/*
 * kalm_merged_attn_resume -- the merged attention of every pair given the self
 * partial of its query rows: only the pair's valid cross keys are read, and
 * the online softmax starts from (o_self, lse_self) of the Q row, so that
 *   O = (e^lse_self o_self + sum_c e^s_c v_c) / (e^lse_self + sum_c e^s_c)
 * and lse (nullable) is the log-sum-exp of all of the row's logits.
 * Rows follow kalm_merged_attn_rows with the same row_mode (0..3); o_self
 * [q_rows, *] float (row stride s_ld, elements, s_ld % 4 == 0 and 16-byte
 * aligned for bf16) and lse_self [q_rows, nq] are indexed like Q.  With the
 * partial of kalm_self_attn_partial on the same Q/K/V rows the result is that
 * of kalm_merged_attn_rows up to rounding.  Other arguments as
 * kalm_merged_attn_rows (there are no self-key arguments).
 */
kalm_status kalm_merged_attn_resume(const void* Q, int64_t q_ld, int64_t q_rows, const float* o_self,
                                    int64_t s_ld, const float* lse_self, const int32_t* cu_q, int32_t P,
                                    int32_t max_lq, const void* Kc, const void* Vc, int64_t c_ld,
                                    const uint8_t* chunk_mask, const int32_t* doc_of_pair, int32_t D,
                                    int32_t Cmax, int32_t nq, int32_t nkv, int32_t d, float scale,
                                    kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows, float* lse,
                                    int32_t row_mode, void* stream);

/*
 * kalm_merged_attn_split -- kalm_merged_attn_resume with the cross keys split
 * into n_split shares that run as separate workgroups (split-KV, for batches
 * whose pairs alone cannot fill the GPU, such as one query against 100
 * passages at the final row): share s walks cross tiles of 32 chunks
 * [s T, s T + T), T = ceil(ceil(Cmax / 32) / n_split), and writes an fp32
 * partial (o, lse) to the workspace; a second kernel merges the self partial
 * and the shares with log-sum-exp weights ([MLX] What this is: the one softmax
 * over the concatenated KV, regrouped).  Same result as
 * kalm_merged_attn_resume up to rounding.
 *   workspace        device memory of at least n_split * o_rows * nq * (d + 1)
 *                    * 4 bytes, 16-byte aligned, owned by the caller; its
 *                    contents on entry do not matter and are overwritten
 *   n_split          1..64
 * BF16 only (KALM_ERR_UNSUPPORTED for F32).  Other arguments as
 * kalm_merged_attn_resume.
 */
kalm_status kalm_merged_attn_split(const void* Q, int64_t q_ld, int64_t q_rows, const float* o_self,
                                   int64_t s_ld, const float* lse_self, const int32_t* cu_q, int32_t P,
                                   int32_t max_lq, const void* Kc, const void* Vc, int64_t c_ld,
                                   const uint8_t* chunk_mask, const int32_t* doc_of_pair, int32_t D,
                                   int32_t Cmax, int32_t nq, int32_t nkv, int32_t d, float scale,
                                   kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows, float* lse,
                                   int32_t row_mode, int32_t n_split, void* workspace,
                                   int64_t workspace_bytes, void* stream);

/*
 * kalm_merged_attn_split_noalloc -- kalm_merged_attn_split for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the split partials live in a
 * static 16 MiB device array inside the library instead of a caller
 * workspace, and the call allocates and frees nothing.  Each GPU the library
 * runs on holds its own copy of the array from library load until the process
 * ends; its address is looked up once per device, on the first call made with
 * that device current.
 *   Limit: n_split * o_rows * nq * (d + 1) * 4 <= 16 MiB (16777216 bytes);
 *          a larger request returns KALM_ERR_INVALID_ARG before anything is
 *          launched.
 *   Every scratch slot the merge reads is written by the same call first, so
 *   the array needs no clearing; it keeps the last call's partials.
 *   Calls that overlap in time on one GPU (different streams or host threads
 *   without ordering between them) share the array and race: order them.
 * Other arguments, results and errors as kalm_merged_attn_split.
 */
kalm_status kalm_merged_attn_split_noalloc(const void* Q, int64_t q_ld, int64_t q_rows, const float* o_self,
                                           int64_t s_ld, const float* lse_self, const int32_t* cu_q, int32_t P,
                                           int32_t max_lq, const void* Kc, const void* Vc, int64_t c_ld,
                                           const uint8_t* chunk_mask, const int32_t* doc_of_pair, int32_t D,
                                           int32_t Cmax, int32_t nq, int32_t nkv, int32_t d, float scale,
                                           kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows, float* lse,
                                           int32_t row_mode, int32_t n_split, void* stream);

/*
 * Decoder-layer completion (a model-shaped layer around a3).  The pages say the
 * forward pass reads every dim, head count, layer count and RoPE parameter from
 * the model's config, RoPE inverse frequencies computed from it ("KaLM-Reranker
 * -V1-Nano -- MLX (Apple Silicon)", What this is / Derivation); no other layer
 * internal is given, so these are the standard forms.
 *
 * kalm_rms_norm -- y[m] = x[m] / sqrt(mean_j x[m,j]^2 + eps) * w, fp32 sum of
 * squares, one rounding to y's dtype.  x [M, H] (row stride x_ld), w [H],
 * y [M, H] (row stride y_ld); dtypes F32 or BF16 each.  Requires H % 4 == 0,
 * ld values multiples of 4, 16-byte aligned pointers; x and y may not overlap.
 */
kalm_status kalm_rms_norm(const void* x, kalm_dtype x_dt, int64_t x_ld, int64_t M, int32_t H,
                          const void* w, kalm_dtype w_dt, float eps, void* y, kalm_dtype y_dt,
                          int64_t y_ld, void* stream);

/*
 * kalm_rope -- rotary position embedding, in place, on n_heads heads of d
 * columns starting at column col0 of X [rows, *] (row stride ld): for each head
 * and i < d/2 the pair (x_i, x_{i+d/2}) at position t turns by the angle
 * t * theta^(-2i/d) ("rotate half" pairing), fp32 arithmetic, one rounding.
 *   row_mode 0  sequence s owns rows cu[s] .. cu[s+1]-1 at positions 0, 1, ...
 *               (max_len >= every length; rows past max_len are not touched)
 *   row_mode 1  one row per sequence: row s at position cu[s+1]-cu[s]-1 (the
 *               final position)
 * Rows outside [0, rows) are skipped.  Requires d % 8 == 0, col0 and ld
 * multiples of 4, theta > 1, X 16-byte aligned.
 */
kalm_status kalm_rope(void* X, kalm_dtype dt, int64_t ld, int64_t rows, int32_t col0, int32_t n_heads,
                      int32_t d, const int32_t* cu, int32_t n_seq, int32_t max_len, int32_t row_mode,
                      float theta, void* stream);

/*
 * kalm_gated_gelu -- the gated MLP's activation: A[m, j] = gelu(Y[m, j]) *
 * Y[m, I + j] for j < I, gelu in its tanh form 0.5 x (1 + tanh(sqrt(2/pi)
 * (x + 0.044715 x^3))); Y [M, 2I] holds the gate projection then the up
 * projection.  Requires I % 4 == 0, ld values multiples of 4, 16-byte aligned
 * pointers.
 */
kalm_status kalm_gated_gelu(const void* Y, kalm_dtype dt, int64_t y_ld, int64_t M, int32_t I, void* A,
                            int64_t a_ld, void* stream);

/*
 * kalm_linear_gated_gelu -- the gated MLP's gate and up projections fused with
 * its activation: A[m, j] = gelu(X[m] . Wg[j]) * (X[m] . Wu[j]), the same
 * tanh-form gelu as kalm_gated_gelu, fp32 products (not rounded to bf16
 * between the projection and the activation), one rounding to bf16.
 *   X   [M, K] bf16, row-major (K contiguous)
 *   Wg  [I, K] bf16 gate rows, Wu [I, K] bf16 up rows (PyTorch [out, in])
 *   A   [M, I] bf16 out, row-major
 * BF16 only.  Requires K % 8 == 0, I % 128 == 0 (an output tile holds 128 gate
 * and the matching 128 up units), 16-byte aligned pointers; X, Wg, Wu and A
 * must not overlap.
 */
kalm_status kalm_linear_gated_gelu(const void* X, const void* Wg, const void* Wu, int32_t M, int32_t K, int32_t I,
                                   void* A, void* stream);

/*
 * a4 -- yes/no readout ([MLX] What this is: score = softmax([logit_yes,
 * logit_no])[yes] at the decoder's final position; [Q4KM] Score a pair and [Q80]
 * Frozen inference contract: margin = yes - no, score = sigmoid(margin)).
 *
 *   h          [rows, H] dtype h_dt (F32 or BF16), row stride h_ld
 *   final_row  [P] int32 row of each pair's final position (outside [0, rows):
 *              NaN outputs for that pair)
 *   w_yesno    [2, H] dtype w_dt: row 0 the "yes" LM-head row, row 1 the "no" row
 *   yes, no, score [P] float out; margin [P] float out, nullable
 * score uses the overflow-free logistic form (equal to the two-way softmax).
 */
kalm_status kalm_yesno_score(const void* h, kalm_dtype h_dt, int64_t h_ld, int64_t rows,
                             const int32_t* final_row, int32_t P, int32_t H, const void* w_yesno,
                             kalm_dtype w_dt, float* yes, float* no, float* margin, float* score,
                             void* stream);

/*
 * a5 -- linear layer of the decoder stack glue (the pages give the layer counts,
 * [MLX] What this is: Nano 18 layers at H=640, Small 26 at H=1152; the layer
 * internals besides the merged attention are a reading: projections in
 * [out, in] layout with fp32 accumulation and an fp32 residual).
 *   Y = X . W^T              (accumulate == 0)
 *   Y = Y + X . W^T          (accumulate != 0; Y must be F32: the residual stream)
 *   Y_bf16 = bf16(Y_final)   (optional second output, F32 Y only)
 *
 *   X  [M, K] dtype dt;  W [N, K] dtype dt;  Y [M, N] dtype y_dt
 * dt == BF16: y_dt BF16 or F32, K % 8 == 0, N % 8 == 0.  dt == F32: y_dt F32,
 * K % 4 == 0, N % 4 == 0.
 */
kalm_status kalm_linear(const void* X, const void* W, int32_t M, int32_t K, int32_t N,
                        kalm_dtype dt, void* Y, kalm_dtype y_dt, int32_t accumulate, void* Y_bf16,
                        void* stream);

/*
 * kalm_linear_residual -- the residual update of a layer whose residual stream
 * starts from gathered rows: Y[m] = R[r_row[m]] + X[m] . W^T (fp32; R[m] when
 * r_row is NULL), with the optional bf16 copy Y_bf16 of Y.  The first decoder
 * layer of a batch in which every passage of a query starts from the query's
 * own first hidden states ([MLX] What this is: the decoder models the query;
 * [MLX] Speed: one passage set, many queries) adds its output projection to
 * those rows directly, with no materialised copy of them per pair.
 *   R      [r_rows, N] float, contiguous; r_row [M] int32 (nullable; without
 *          it R needs M rows); an index outside [0, r_rows) gives NaN in that
 *          row of Y
 *   Y      [M, N] float out; must not overlap R unless r_row is NULL and R == Y
 * Other arguments as kalm_linear (accumulate into an F32 Y).
 */
kalm_status kalm_linear_residual(const void* X, const void* W, int32_t M, int32_t K, int32_t N,
                                 kalm_dtype dt, const float* R, const int32_t* r_row, int64_t r_rows,
                                 float* Y, void* Y_bf16, void* stream);

/*
 * a5 -- row gather that starts the residual stream of every pair from its
 * query's first-layer hidden state (all passages of a query share it).
 *   dst[m] = src[idx[m]]   for m < M   (float rows of length H)
 *   dst_bf16[m] = bf16(dst[m])   (nullable second output)
 * idx values outside [0, n_src) give NaN rows.  Requires H % 4 == 0.
 */
kalm_status kalm_gather_rows(const float* src, const int32_t* idx, int64_t M, int32_t H,
                             int64_t n_src, float* dst, void* dst_bf16, void* stream);

/*
 * Ranking of each query's passages by relevance score, the step above the
 * score: rerank(query, docs, top_n) returns the top_n passages highest score
 * first as (index, relevance_score) ([MLX] What this is / Files: the
 * rerank(query, docs, top_n) call; [Q4KM] Score a pair: rank larger margins
 * first -- the score is monotone in the margin).
 *   score      [n_queries, n_docs] float: row q holds query q's passage scores
 *              (the kalm_yesno_score output in pair order q * n_docs + d)
 *   out_index  [n_queries, top_n] int32 out: passage indices, best first
 *   out_score  [n_queries, top_n] float out: their scores
 * Order: higher score first; equal scores by lower index; NaN scores last (by
 * index).  Requires 0 <= top_n <= n_docs <= 4096.
 */
kalm_status kalm_rank_topn(const float* score, int32_t n_queries, int32_t n_docs, int32_t top_n,
                           int32_t* out_index, float* out_score, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KALM_H */
