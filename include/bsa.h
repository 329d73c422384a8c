/*
 * bsa.h -- selector-driven block-sparse landmark attention for AMD Instinct MI355X (gfx950).
 *
 * The method (from the pages this library implements):
 *  1. keys are pooled into one landmark per 64-token block (LSA page, "Latent Sparse
 *     Attention", section "The index stops scanning the whole context", paragraph 3:
 *     neighbouring keys are merged before indexing; the HiLS page calls such per-chunk
 *     vectors landmarks);
 *  2. each query block scores the landmarks with a light selector and keeps the hard top-K
 *     blocks (SAS page, "Scientists taught transformers to select context directly...",
 *     summary paragraph 1 and "How to apply");
 *  3. attention runs only over the chosen blocks plus the start of the context and a recent
 *     window (LSA page, first section, paragraph 4), the current block always kept (SAS
 *     page, summary paragraph 3);
 *  4. variants: SAS adds a log-form gate inside the softmax, normalised against the current
 *     block (SAS page, summary paragraph 3, "Key facts" item 3); HiLS attends to each chunk
 *     separately and merges the chunk results by the chunks' retrieval scores (HiLS page,
 *     "HiLS-Attention: hierarchical sparse attention...", summary paragraph 2).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, contiguous, in the layouts
 *    given below, 16-byte aligned.  The library never allocates, frees, synchronises or keeps
 *    a pointer after a call returns.  Work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream) and completes asynchronously.
 *  - Layouts are head-major: q [B,Hq,Tq,D]; k, v [B,Hkv,Tk,D]; landmarks [B,Hkv,NB,D] with
 *    NB = ceil(Tk/64); selection rows [B,Hkv,R,NA] with R = ceil(Tq/64) for prefill and 1 for
 *    decode and NA = n_sink + n_local + topk.  Query head h uses kv head h / (Hq/Hkv).
 *  - Element type of q, k, v, landmarks and outputs is params->dtype (float32 or bf16);
 *    idx is int32, sc and lse are float32.
 *  - Arguments are checked before anything is launched: on an invalid argument the call
 *    returns a non-zero status, launches nothing and leaves every buffer untouched;
 *    bsa_last_error() then describes the failure (thread-local).  A failed kernel launch
 *    returns BSA_ERR_HIP.  No call aborts, exits or throws.
 *  - The library holds no state: calls on different streams may run concurrently.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsa_status {
  BSA_OK = 0,
  BSA_ERR_NULL = 1,        /* a required pointer is NULL */
  BSA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  BSA_ERR_UNSUPPORTED = 3, /* a value outside what the kernels implement (D, block, dtype, mode) */
  BSA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  BSA_ERR_WORKSPACE = 5,   /* workspace pointer NULL or smaller than required */
  BSA_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} bsa_status_t;

typedef enum bsa_dtype { BSA_DTYPE_F32 = 0, BSA_DTYPE_BF16 = 1 } bsa_dtype_t;

typedef enum bsa_mode {
  BSA_MODE_PLAIN = 0, /* softmax over the attended keys */
  BSA_MODE_SAS = 1,   /* + gate log sigmoid(S_j - S_c) on every logit of attended block j != c */
  BSA_MODE_HILS = 2   /* per-chunk softmax, chunks merged by softmax_j(q . L_j * scale) */
} bsa_mode_t;

typedef struct bsa_params {
  int32_t batch;    /* B >= 1 (prefill: sequences; decode: sequences, one query token each) */
  int32_t heads_q;  /* Hq >= 1, a multiple of heads_kv */
  int32_t heads_kv; /* Hkv >= 1 */
  int32_t head_dim; /* D: 64 or 128 */
  int32_t seq_q;    /* prefill: == seq_k; decode: 1 (the query is the token at seq_k - 1) */
  int32_t seq_k;    /* Tk >= 1 tokens in k, v (a decode cache includes the query's own k, v) */
  int32_t block;    /* must be 64 */
  int32_t topk;     /* K >= 0 blocks chosen beyond the sink and the local window */
  int32_t n_sink;   /* >= 0 leading blocks always attended (the start of the context) */
  int32_t n_local;  /* >= 1 blocks ending at the current one always attended */
  float scale;      /* softmax scale; 0 selects 1/sqrt(head_dim) */
  int32_t dtype;    /* bsa_dtype_t */
  int32_t mode;     /* bsa_mode_t (used by the attend calls) */
} bsa_params_t;

/*
 * Landmarks (LSA page, "The index stops scanning the whole context", paragraph 3: neighbouring
 * keys are pooled before indexing; HiLS page, summary paragraph 2: per-chunk landmarks).
 * lm[b,g,j,:] = mean of k[b,g,t,:] over the tokens t of block j (a partial last
 * block averages the tokens present), accumulated in float64 and rounded once, to nearest
 * even, to the dtype.
 *   k  [B,Hkv,Tk,D] (input)      lm [B,Hkv,NB,D] (output)
 */
bsa_status_t bsa_pool_landmarks(const bsa_params_t* params, const void* k, void* lm,
                                void* stream);

/* Bytes of workspace bsa_select_topk needs for these params (0 if params are invalid). */
size_t bsa_select_workspace_bytes(const bsa_params_t* params);

/*
 * Selection (SAS page, summary paragraph 1 and "How to apply": a light selector scores the
 * units of context and inference keeps the hard top-K; LSA page, first section, paragraphs 2
 * and 4: each contiguous block is scored, the start of the context and a recent window are
 * always attended; SAS page, summary paragraph 3: the current block is always kept).
 * Selector vector qbar = sum over the query heads of each kv group of the mean
 * query of each 64-token query block (decode: of the one query token), kept in float32.
 * Scores S[c][j] = qbar_c . L_j for j <= c (no softmax scale).  Candidates are the blocks
 * n_sink <= j <= c - n_local; the K = min(topk, #candidates) highest scores are chosen, the
 * lower block index first among equal scores.  Row c of idx lists, ascending: blocks
 * 0..min(n_sink, c+1)-1, the chosen candidates, then blocks max(n_sink, c-n_local+1)..c,
 * padded with -1; sc holds S[c][j] for each listed block (0 in the padding).  The current
 * block c is therefore always the last valid entry.
 *   q    [B,Hq,Tq,D]  (prefill: Tq == Tk; decode: Tq == 1)
 *   lm   [B,Hkv,NB,D] landmarks of the Tk keys (bsa_pool_landmarks)
 *   idx  [B,Hkv,R,NA] int32 output, sc [B,Hkv,R,NA] float32 output
 *   ws   device workspace of at least bsa_select_workspace_bytes(params) bytes (the selector
 *        vectors and the float32 score rows; none where the one-pass selection below runs: bf16
 *        prefill rows with topk <= 32 and more than 4096 blocks; then ws may be NULL); contents
 *        on entry are ignored.
 */
bsa_status_t bsa_select_topk(const bsa_params_t* params, const void* q, const void* lm,
                             int32_t* idx, float* sc, void* ws, size_t ws_bytes, void* stream);

/*
 * The same selection as bsa_select_topk (same idx and sc, bit for bit) by one kernel that
 * scores each tile row of the lower triangle and keeps, per row, only candidates that can still
 * be among the K best, so no score rows are written (LSA page, "The index stops scanning the
 * whole context", paragraph 2: the candidate search is what grows with the context; SAS page,
 * summary paragraph 1: hard top-K).  bsa_select_topk uses it by itself for rows of more than
 * 4096 blocks; this entry point takes it at any length.
 *   Applies to prefill (seq_q == seq_k) with dtype BSA_BF16, topk <= 32 and at most 65536
 *   blocks; otherwise BSA_ERR_UNSUPPORTED.  The kernel forms the selector vectors itself.
 *   ws, ws_bytes  unused (no workspace; may be NULL, 0).
 */
bsa_status_t bsa_select_topk_fused(const bsa_params_t* params, const void* q, const void* lm,
                                   int32_t* idx, float* sc, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * Prefill attention (SAS page, summary paragraph 4: blockwise, FlashAttention-style, without
 * the full square matrix; summary paragraph 3 and "Key facts" item 3: the SAS gate sits inside
 * the softmax in log form, normalised against the current block; HiLS page, summary paragraph
 * 2: per-chunk attention merged by the chunks' retrieval scores).
 * seq_q == seq_k == T.  For query token t of head h in block c = t/64 and
 * the attended set A_c = row c of idx (entries must be ascending, <= c, end with c and be
 * followed only by -1 padding):
 *   PLAIN: o = sum_u softmax_u(scale * q.k_u) v_u over keys u in the blocks of A_c, u <= t;
 *   SAS:   the logit of each key of block j != c gets + log sigmoid(sc_j - sc_c);
 *   HILS:  o = sum_{j in A_c} w_j o_j, o_j = softmax attention over the keys u <= t of block
 *          j alone, w = softmax_j(scale * q.L_j); needs lm.
 *   q [B,Hq,T,D], k/v [B,Hkv,T,D], lm [B,Hkv,NB,D] (HILS only, else may be NULL),
 *   idx/sc [B,Hkv,R,NA] from bsa_select_topk (sc may be NULL for PLAIN and HILS),
 *   out [B,Hq,T,D] output, lse [B,Hq,T] float32 output = log of the softmax denominator
 *   (PLAIN/SAS; may be NULL; must be NULL for HILS).
 */
bsa_status_t bsa_attend_prefill(const bsa_params_t* params, const void* q, const void* k,
                                const void* v, const void* lm, const int32_t* idx,
                                const float* sc, void* out, float* lse, void* stream);

/* Bytes of workspace bsa_attend_decode needs for these params (0 if params are invalid). */
size_t bsa_decode_workspace_bytes(const bsa_params_t* params);

/*
 * Decode attention (LSA page, "The index stops scanning the whole context", paragraph 1: per
 * generated token the work is the attention over the selected blocks only; the passages of
 * bsa_attend_prefill define the three modes).
 * seq_q == 1: the query of each sequence is the token at position Tk - 1
 * and sees every key of its attended blocks; same PLAIN / SAS / HILS rules as prefill.  The
 * attended blocks are split over workgroups and the partial softmax states merged through
 * their log-sum-exp.
 *   q [B,Hq,1,D], kc/vc [B,Hkv,Tk,D] cache, lm [B,Hkv,NB,D] (HILS only), idx/sc [B,Hkv,1,NA],
 *   out [B,Hq,1,D] output, lse [B,Hq] (PLAIN/SAS, may be NULL; NULL for HILS),
 *   ws device workspace of bsa_decode_workspace_bytes(params) bytes (may be NULL if that is 0).
 *   The bf16 path needs Hq/Hkv <= 32.
 */
bsa_status_t bsa_attend_decode(const bsa_params_t* params, const void* q, const void* kc,
                               const void* vc, const void* lm, const int32_t* idx,
                               const float* sc, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): bsa_attend_decode without a workspace argument.  The
 * split partial states that bsa_attend_decode keeps in the caller's workspace live instead in a
 * static device array of 4 MiB (4194304 bytes) inside the library; each device that runs it
 * holds its own copy until the process ends, and its address is looked up on the first call on
 * that device (the device of `stream`).  The call allocates and frees nothing.  Shapes whose
 * partial states need more than 4 MiB (bsa_decode_workspace_bytes(params) > 4194304) are
 * rejected with BSA_ERR_WORKSPACE before anything is launched.  Every call on one device shares
 * that array: calls that overlap on one device race (serialise them, e.g. on one stream).
 * Arguments, results and errors otherwise as bsa_attend_decode.
 */
bsa_status_t bsa_attend_decode_noalloc(const bsa_params_t* params, const void* q, const void* kc,
                                       const void* vc, const void* lm, const int32_t* idx,
                                       const float* sc, void* out, float* lse, void* stream);

/*
 * Paged, ragged decode: the serving layout, where sequences of different lengths share one pool
 * of 64-token pages (one page = one block, so a block never straddles two pages).
 *   k_pool, v_pool [n_pages, Hkv, 64, D]: page p of kv head g is the contiguous 64 x D tile at
 *       (p * Hkv + g) * 64 * D;
 *   page_table [B, NB] int32 (NB = params->seq_k / 64, seq_k a multiple of 64: the capacity of
 *       a sequence): logical block j of sequence b is page page_table[b * NB + j];
 *   seq_lens [B] int32: sequence b holds seq_lens[b] tokens (1 <= seq_lens[b] <= seq_k), its
 *       query is the token seq_lens[b] - 1, and its K / V include that token.
 * Per sequence, every rule of the contiguous calls holds with Tk = seq_lens[b] (landmark means,
 * candidates, sink / local window, gates, HiLS merge).  Page indices and lengths are device
 * data and are not checked by the host: out-of-range values are clamped into range (results
 * then unspecified, but nothing outside the pools, the table or the outputs is accessed).
 * params: batch = B, seq_q = 1, seq_k = NB * 64; the other fields as for the contiguous calls.
 *
 * Landmarks of the paged cache: lm [B, Hkv, NB, D], block j of sequence b the mean of its
 * min(64, seq_lens[b] - 64 j) tokens (float64 accumulation, one rounding); blocks past the end
 * of a sequence are written as zeros.  float32 and bf16.
 */
bsa_status_t bsa_pool_landmarks_paged(const bsa_params_t* params, const void* k_pool,
                                      int32_t n_pages, const int32_t* page_table,
                                      const int32_t* seq_lens, void* lm, void* stream);

/*
 * Selection for a paged batch: as bsa_select_topk for a decode step, sequence b's query block
 * being (seq_lens[b] - 1) / 64.  q [B,Hq,1,D], lm from bsa_pool_landmarks_paged, idx / sc
 * [B,Hkv,1,NA] outputs.  bf16 only, NB <= 16384; needs no workspace.
 */
bsa_status_t bsa_select_topk_paged(const bsa_params_t* params, const void* q, const void* lm,
                                   const int32_t* seq_lens, int32_t* idx, float* sc,
                                   void* stream);

/*
 * Decode attention over a paged batch: as bsa_attend_decode with the cache read through the
 * page table; ws of bsa_decode_workspace_bytes(params) bytes.  bf16 only.
 */
bsa_status_t bsa_attend_decode_paged(const bsa_params_t* params, const void* q,
                                     const void* k_pool, const void* v_pool, int32_t n_pages,
                                     const int32_t* page_table, const int32_t* seq_lens,
                                     const void* lm, const int32_t* idx, const float* sc,
                                     void* out, float* lse, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * One decode step: the selection of bsa_select_topk followed by the attention of
 * bsa_attend_decode (method steps 2-4 for the query token of each sequence), in one call.
 * For bf16 with at least one workgroup's worth of (sequence, kv head) pairs per compute unit
 * (B * Hkv >= 256), NB <= 4096 and NA <= 256, both run in a single kernel: each (sequence, kv
 * head) workgroup scores its landmarks, takes its top-K and streams the attended blocks, the
 * sink and local blocks' copies starting while the top-K is decided.  Otherwise the two are
 * launched one after the other.  idx and sc follow bsa_select_topk's rule and layout; the fused
 * kernel sums each score in another float32 order, so sc may differ from that call's in the last
 * bits and the chosen set only where two scores agree to that precision.  out and lse are those
 * of bsa_attend_decode on the written idx / sc, up to float32 summation order.
 *   q [B,Hq,1,D], kc/vc [B,Hkv,Tk,D], lm [B,Hkv,NB,D] (inputs); idx/sc [B,Hkv,1,NA],
 *   out [B,Hq,1,D], lse [B,Hq] (outputs; lse may be NULL and must be NULL for HILS);
 *   ws of bsa_decode_step_workspace_bytes(params) bytes, 256-byte aligned (NULL if that is 0).
 */
size_t bsa_decode_step_workspace_bytes(const bsa_params_t* params);
bsa_status_t bsa_decode_step(const bsa_params_t* params, const void* q, const void* kc,
                             const void* vc, const void* lm, int32_t* idx, float* sc, void* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * The same step over a paged, ragged batch (k_pool, v_pool, n_pages, page_table, seq_lens as
 * for bsa_attend_decode_paged; lm from bsa_pool_landmarks_paged).  bf16 only, NB <= 16384;
 * ws of bsa_decode_step_workspace_bytes(params) bytes.
 */
bsa_status_t bsa_decode_step_paged(const bsa_params_t* params, const void* q,
                                   const void* k_pool, const void* v_pool, int32_t n_pages,
                                   const int32_t* page_table, const int32_t* seq_lens,
                                   const void* lm, int32_t* idx, float* sc, void* out,
                                   float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Landmark refresh after tokens are appended (decode-time cache maintenance).  A block's pooled
 * key depends only on its own tokens (LSA page, "The index stops scanning the whole context",
 * paragraph 3: keys are pooled per block, and a block's index entry is fixed once the block is
 * complete), so after n_new tokens are appended only the blocks holding them change: this call
 * recomputes, for every (sequence, kv head), the landmarks of blocks (seq_k - n_new) / 64 ..
 * NB - 1 of k [B,Hkv,seq_k,D] exactly as bsa_pool_landmarks computes them, and writes no other
 * element of lm [B,Hkv,NB,D].  n_new >= 1 (n_new >= seq_k refreshes every block).
 */
bsa_status_t bsa_update_landmarks(const bsa_params_t* params, const void* k, int32_t n_new,
                                  void* lm, void* stream);

/*
 * The same refresh for a paged, ragged batch (layouts of bsa_pool_landmarks_paged): sequence b,
 * holding seq_lens[b] tokens of which the last n_new were appended since its landmarks were
 * last computed, gets the landmarks of blocks (seq_lens[b] - n_new) / 64 .. (seq_lens[b]-1) / 64
 * recomputed as bsa_pool_landmarks_paged computes them; blocks before them and past its last
 * block are not written.  A decode loop that appends one token per sequence and step calls it
 * with n_new = 1 (one block per sequence and kv head) instead of re-pooling the whole cache.
 */
bsa_status_t bsa_update_landmarks_paged(const bsa_params_t* params, const void* k_pool,
                                        int32_t n_pages, const int32_t* page_table,
                                        const int32_t* seq_lens, int32_t n_new, void* lm,
                                        void* stream);

/*
 * Flat clustered index over the landmarks (LSA page, "The index stops scanning the whole
 * context", paragraphs 3-5: similar pooled keys are grouped by Ward's algorithm once a block of
 * the context is complete, and kept as each cluster's centre plus the table of its positions).
 * Every completed segment s of seg_blocks landmarks (blocks s*seg_blocks .. +seg_blocks, for
 * s < NS = floor(NB / seg_blocks); NB = ceil(seq_k / 64)) is clustered into n_clusters clusters:
 * starting from single landmarks, the two clusters A, B with the smallest
 * |A||B| / (|A|+|B|) * ||mean_A - mean_B||^2 are merged (equal costs: the smallest pair of ids,
 * a cluster's id being its lowest block; float32 arithmetic) until n_clusters remain.
 *   lm       [B,Hkv,NB,D] landmarks (params->dtype) from bsa_pool_landmarks
 *   centres  [B,Hkv,NS*n_clusters,D] float32 output: the mean of each cluster's landmarks
 *   members  [B,Hkv,NS,seg_blocks] int32 output: each segment's blocks grouped by cluster
 *            (clusters in id order, blocks ascending), absolute block indices
 *   offsets  [B,Hkv,NS,n_clusters+1] int32 output: cluster r of a segment is members[o_r .. o_r+1)
 *   merges   [B,Hkv,NS,seg_blocks-n_clusters,2] int32 output: the merged pairs of ids, in order
 *            (may be NULL when seg_blocks == n_clusters)
 * Limits: 1 <= n_clusters <= seg_blocks <= 64.  With NS = 0 nothing is launched.
 */
bsa_status_t bsa_lsa_build_index(const bsa_params_t* params, const void* lm, int32_t seg_blocks,
                                 int32_t n_clusters, float* centres, int32_t* members,
                                 int32_t* offsets, int32_t* merges, void* stream);

/*
 * Index maintenance (LSA page, "The index stops scanning the whole context", paragraph 3: once a
 * block of the context is complete its clusters are computed and then kept): clusters only the
 * completed segments first_segment .. NS-1 into the arrays of bsa_lsa_build_index (same layouts,
 * same arithmetic) and writes nothing of the segments below first_segment, whose clusters stay
 * as they were.  first_segment = 0 is bsa_lsa_build_index; first_segment >= NS writes nothing.
 */
bsa_status_t bsa_lsa_update_index(const bsa_params_t* params, const void* lm, int32_t seg_blocks,
                                  int32_t n_clusters, int32_t first_segment, float* centres,
                                  int32_t* members, int32_t* offsets, int32_t* merges,
                                  void* stream);

/*
 * Workspace bytes of bsa_lsa_select and bsa_lsa_tree_select (decode: 0).  Prefill: the selector
 * vectors (B*Hkv*R*D float32, rounded up to 256 bytes), then, used by bsa_lsa_select alone, a
 * table of the clusters' candidate counts and a buffer of at most 256 MiB for precomputed
 * cluster scores.  Both selections accept any workspace of at least the selector vectors'
 * bytes; bsa_lsa_select uses the rest when given all of it.
 */
size_t bsa_lsa_select_workspace_bytes(const bsa_params_t* params);

/*
 * Attended block sets from the flat clustered index (prefill: one row per 64-token query
 * block; decode: seq_q == 1, one row for the query at position seq_k - 1), same layout as
 * bsa_select_topk's.  The selector vector qbar is that of bsa_select_topk.  With
 * last = c - n_local the last candidate block, the units are: the clusters of the completed
 * segments lying wholly at or before block last (first NE = min(NS, (last+1)/seg_blocks)
 * segments), scored qbar . centre, and every other candidate block j (max(n_sink, NE*seg_blocks)
 * <= j <= last) on its own, scored qbar . L_j (float32).  Units are taken by score, descending
 * (equal scores: the lower id first), and expanded into their candidate blocks (blocks >= n_sink,
 * ascending) until min(topk, candidates) blocks are chosen, the last unit cut short if needed.
 * Row c lists the sink blocks, the chosen blocks ascending, the local window, then -1; sc holds
 * a chosen block's unit score and qbar . L_j for sink and local blocks (0 in the padding).
 *   q, lm: as for bsa_select_topk; centres, members, offsets: from bsa_lsa_build_index with the
 *   same seg_blocks and n_clusters (may be NULL when NS = 0); ws: device workspace, 256-byte
 *   aligned, of at least the selector vectors' bytes (see bsa_lsa_select_workspace_bytes).
 *   With more than 1024 clusters per row and room for at least 64 rows of cluster scores after
 *   the selector vectors and the count table, the cluster scores are first formed for tiles of
 *   rows on MFMA (the selector vector and the centres each split into three bf16 terms; the six
 *   leading products summed in float32), chunk by chunk; otherwise each row computes them as
 *   float32 dot products.  The two differ only in the last bits of a score.
 * Limits: as bsa_lsa_build_index, plus NS * n_clusters + seg_blocks <= 8192 and topk <= 2048.
 */
bsa_status_t bsa_lsa_select(const bsa_params_t* params, const void* q, const void* lm,
                            int32_t seg_blocks, int32_t n_clusters, const float* centres,
                            const int32_t* members, const int32_t* offsets, int32_t* idx,
                            float* sc, void* ws, size_t ws_bytes, void* stream);

/*
 * Tree over the flat index (LSA page, the same section, paragraph 5: the tree variant joins the
 * clusters into a hierarchy and walks it by beam search, keeping a few branches per level, so a
 * query makes a logarithmic number of comparisons).  Above the clusters of a segment sits the
 * segment, above segments groups of `fanout` consecutive segments; a node's centre is the mean
 * of the landmarks under it.
 *   seg_centres [B,Hkv,NS,D] float32 output; grp_centres [B,Hkv,NG,D] float32 output,
 *   NG = floor(NS / fanout) (may be NULL when NG = 0).  lm as for bsa_lsa_build_index.
 */
bsa_status_t bsa_lsa_tree_centres(const bsa_params_t* params, const void* lm,
                                  int32_t seg_blocks, int32_t fanout, float* seg_centres,
                                  float* grp_centres, void* stream);

/*
 * Attended block sets by beam search over the tree.  For query block c (decode: the query at
 * seq_k - 1), with NE the eligible segments of bsa_lsa_select: the top level holds the whole
 * groups among them and the eligible segments left over; at each level the `beam` best nodes
 * (by qbar . centre, descending; equal scores: the node whose first block is lower) pass their
 * children on -- groups their segments, segments their clusters -- and the `beam` best clusters
 * become units, expanded with the not yet clustered candidate blocks exactly as in
 * bsa_lsa_select (same row layout and scores).  Arguments as bsa_lsa_select plus the tree
 * centres; ws: bsa_lsa_select_workspace_bytes.
 * Limits: those of bsa_lsa_build_index, topk <= 2048, 1 <= beam <= 64, fanout >= 1, and
 * NS / fanout + fanout, beam * fanout, beam * n_clusters and beam + seg_blocks each at most
 * 1024 (no limit on NS * n_clusters: one level's nodes are sorted at a time).
 */
bsa_status_t bsa_lsa_tree_select(const bsa_params_t* params, const void* q, const void* lm,
                                 int32_t seg_blocks, int32_t n_clusters, int32_t fanout,
                                 int32_t beam, const float* centres, const int32_t* members,
                                 const int32_t* offsets, const float* seg_centres,
                                 const float* grp_centres, int32_t* idx, float* sc, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Workspace bytes of bsa_attend_prefill_backward for these params (0 if the params are
 * rejected by that call).
 */
size_t bsa_backward_workspace_bytes(const bsa_params_t* params);

/*
 * Backward of prefill attention (bf16 only).  PLAIN / SAS: the selector is trained end to end
 * through the SAS gates (SAS page, summary paragraphs 2-3: the top-K choice itself is hard, but
 * the continuous scores enter the softmax through the gates and carry gradient).  HILS: the
 * chunk results are merged by the chunks' retrieval scores (HiLS page, summary paragraph 2), so
 * the gradient also reaches the landmarks through those scores.
 * PLAIN / SAS, with the forward's logits x_tu = scale * q_t.k_u + g_j(u) over the keys u of A_c
 * (u <= t), P = exp(x - lse), dP_tu = dout_t.v_u and dx = P * (dP - dout_t.out_t):
 *   dq_t = scale * sum_u dx_tu k_u;  dk_u = scale * sum_t dx_tu q_t;  dv_u = sum_t P_tu dout_t
 *   (sums over every query head of the kv group and every query block that attends u);
 *   SAS: dg_j = sum of dx over the rows of block c (all heads of the group) and the keys of
 *   block j; d sc_j = dg_j * sigmoid(sc_c - sc_j) for j != c and d sc_c = -(sum of those).
 * HILS, with P_j the softmax of row t over the visible keys of chunk j alone, o_j = P_j V,
 * w = softmax_j(scale * q_t.L_j), dw_j = dout_t.o_j and dr_j = w_j (dw_j - sum_i w_i dw_i):
 *   chunk j is a softmax attention with output gradient w_j dout (giving dq, dk, dv as above
 *   with dx = w_j P_j (dP - dw_j)); dq_t += scale * sum_j dr_j L_j; dlm_j = scale * sum of
 *   dr_j q_t over every row and query head that attends chunk j.  dk does not include the
 *   pooling that produced the landmarks (a caller training through it adds dlm_j / n_j to
 *   each of the n_j keys of block j).
 *   q, k, v, idx: the forward's inputs; sc (SAS: required; else ignored); lm [B,Hkv,NB,D] bf16
 *   (HILS: the landmarks the forward used, required; else ignored);
 *   out [B,Hq,T,D] bf16 and lse [B,Hq,T] float32: the forward's output and lse (PLAIN / SAS:
 *   required; HILS: ignored, may be NULL -- the sum over chunks is formed exactly instead);
 *   dout [B,Hq,T,D] bf16: gradient of the loss with respect to out;
 *   dq [B,Hq,T,D], dk, dv [B,Hkv,T,D] bf16 outputs (every element written);
 *   dsc [B,Hkv,R,NA] float32 output, zero in the padding and for PLAIN / HILS (may be NULL
 *   unless SAS); dlm [B,Hkv,NB,D] float32 output (HILS: required, every element written; else
 *   ignored);
 *   ws: device workspace of bsa_backward_workspace_bytes(params) bytes, 256-byte aligned;
 *       contents on entry are ignored.
 * Limits: at most 65535 key blocks; R * NA < 2^31.  Sums over many query blocks (dk, dv,
 * dlm) are taken in a fixed order when a key block is attended by at most 4096 query blocks;
 * beyond that their float32 rounding may differ between runs.  dsc accumulates with float32
 * atomics and its rounding may differ between runs.
 */
bsa_status_t bsa_attend_prefill_backward(const bsa_params_t* params, const void* q,
                                         const void* k, const void* v, const void* lm,
                                         const int32_t* idx, const float* sc, const void* out,
                                         const float* lse, const void* dout, void* dq, void* dk,
                                         void* dv, float* dsc, float* dlm, void* ws,
                                         size_t ws_bytes, void* stream);

/*
 * One query for every call that takes a workspace: which = BSA_WS_SELECT (bsa_select_topk),
 * BSA_WS_DECODE (bsa_attend_decode, bsa_attend_decode_paged), BSA_WS_DECODE_STEP
 * (bsa_decode_step, bsa_decode_step_paged), BSA_WS_BACKWARD (bsa_attend_prefill_backward) or
 * BSA_WS_LSA_SELECT (bsa_lsa_select, bsa_lsa_tree_select).  Returns the same number as that
 * call's own *_workspace_bytes function: 0 when the params are rejected, when `which` is
 * unknown, or when the call needs no workspace for these params.
 */
typedef enum bsa_workspace_call {
  BSA_WS_SELECT = 0,
  BSA_WS_DECODE = 1,
  BSA_WS_DECODE_STEP = 2,
  BSA_WS_BACKWARD = 3,
  BSA_WS_LSA_SELECT = 4
} bsa_workspace_call_t;
size_t bsa_workspace_bytes(const bsa_params_t* params, int which);

/* Static description of a status code. */
const char* bsa_status_string(int status);
/* Detail of the last failed call on this thread ("" if none). */
const char* bsa_last_error(void);
/* Library version, e.g. 100 for 1.0.0. */
int bsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
