/*
 * fastar.h -- C ABI of the TempCache compressed-KV attention step on gfx950.
 *
 * The operation (FAST-AR technical summary, gist.science, Portuguese page and
 * its French twin, section "2. Componentes Principais / A. TempCache"): each
 * new token's key is matched top-1 against the cached keys through a
 * locality-sensitive hash instead of full attention matrices; a match above a
 * similarity threshold is merged into the cached slot, which keeps the mean of
 * the merged values and the group size; attention then shifts each slot's logit
 * by the log of its group size, which Lemma 5.1 shows is exact for identical
 * keys; the cache is bounded so memory and latency stay constant.  AnnCA
 * (section "2. Componentes Principais / B. AnnCA") keeps, per frame, only the
 * prompt tokens that share a hash bucket with at least one query of the frame.
 *
 * Readings of what the pages leave open, fixed by this library:
 *   - hash: SimHash, L tables of b random hyperplanes; bit j of table t is
 *     [<r_tj, x> > 0], stored as (1u << j) of one uint32 per table;
 *   - candidates: live slots whose code equals the token's code in any table;
 *     top-1 by cosine against the slot's stored key, ties to the lowest slot;
 *   - merge iff cosine >= cos_threshold; merged key and value are running means
 *     kept in binary32 (m += (x - m) / (count + 1), one rounded op at a time,
 *     tokens of a frame in ascending order), mirrored in the storage dtype;
 *   - eviction when a frame's inserts exceed the free slots: exactly the missing
 *     number of slots not merged into in this frame, smallest
 *     (last updated frame, slot id) first; inserts take the freed and then the
 *     never-used ids in ascending order, so the live slots are always
 *     [0, n_live);
 *   - merged slots are re-hashed from their new stored key after each frame;
 *   - attention: logit = <q, k_s> * scale + ln(count_s), softmax over the live
 *     slots, output = sum_s p_s v_s.
 *
 * Conventions for every call:
 *   - Pointers named *_dev are device memory owned by the caller; pointers
 *     named *_host are host memory owned by the caller.  The library never
 *     frees caller memory and never allocates device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; pointers must stay valid until
 *     that work has completed.  Calls that read results back to the host say
 *     so and synchronise the stream.
 *   - Tensors are row-major with the last (feature) dimension contiguous;
 *     strides are in elements.  Storage dtype FASTAR_BF16 means raw bfloat16
 *     (16-bit) elements, FASTAR_F32 binary32.
 *   - Every call returns a status.  Argument errors are detected on the host
 *     before anything is enqueued and leave all state unchanged.  A HIP launch
 *     error returns FASTAR_ERR_HIP; a device fault surfaces at the next
 *     synchronising call.  fastar_last_error() gives a thread-local message.
 *   - One cache handle must not be used from two streams at once.
 */
#ifndef FASTAR_H
#define FASTAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FASTAR_OK = 0,
  FASTAR_ERR_INVALID_ARGUMENT = 1,
  FASTAR_ERR_WORKSPACE_TOO_SMALL = 2,
  FASTAR_ERR_CAPACITY = 3,
  FASTAR_ERR_HIP = 4,
  FASTAR_ERR_UNSUPPORTED = 5
} fastar_status;

typedef enum { FASTAR_F32 = 0, FASTAR_BF16 = 1 } fastar_dtype;

/* Limits checked by every call. */
#define FASTAR_MAX_TABLES 8
#define FASTAR_MAX_BITS 32
#define FASTAR_MAX_BUDGET 32768
#define FASTAR_MAX_TOKENS_PER_FRAME 8192
#define FASTAR_MAX_ANNCA_QUERIES_PER_FRAME 4096
#define FASTAR_MAX_ANNCA_PROMPT 16384

typedef struct {
  int32_t num_heads;     /* H >= 1; heads never interact                      */
  int32_t head_dim;      /* d: 64 or 128                                       */
  int32_t budget_slots;  /* B: slots per head, 1..FASTAR_MAX_BUDGET            */
  int32_t num_tables;    /* L: 1..FASTAR_MAX_TABLES                            */
  int32_t num_bits;      /* b: 0..FASTAR_MAX_BITS (0 = one bucket per table)    */
  float cos_threshold;   /* merge iff cosine >= this (any finite value)         */
  fastar_dtype dtype;    /* storage dtype of keys, values, queries, outputs    */
  int32_t pq_subspaces;  /* 0: SimHash codes, planes [L][b][d]; M in {1, 2, 4,
                          * 8 (d = 128 only)}: product-quantization codes,
                          * codebooks [L][M][2^(b/M)][d/M], b = M x (1..8)    */
  int32_t rope_members;  /* 0..4: frames of each slot's most recent members kept
                          * for fastar_attend_rope (its largest m)           */
} fastar_config;

typedef struct fastar_cache_s* fastar_cache_t;

/* Totals over all heads since create/reset (or as imported). */
typedef struct {
  int64_t frame;           /* frames merged so far                            */
  int64_t tokens_seen;     /* tokens passed to fastar_match_merge             */
  int64_t live_slots;      /* sum of n_live                                   */
  int64_t merged_tokens;   /* tokens merged into an existing slot             */
  int64_t inserted_tokens; /* tokens that took a new slot                     */
  int64_t evicted_slots;   /* slots evicted to make room                      */
  int64_t evicted_tokens;  /* tokens those slots held (sum of their counts)   */
  int32_t max_live;        /* largest n_live over heads                       */
  int32_t refused_frames;  /* (head, frame) pairs the merge refused because
                            * fewer slots were evictable than its inserts
                            * needed; such a frame changes nothing.  Stays 0
                            * for states built by the library or accepted by
                            * fastar_cache_import.                           */
} fastar_stats;

/* Host-side image of a cache's state; any pointer may be NULL to skip it, and
 * frame = -1 skips the frame counter (next frame to merge).
 * Shapes: k/v_master float [H][B][d]; k/v_mirror dtype [H][B][d];
 * count, last int32 [H][B]; codes uint32 [H][L][B]; n_live int32 [H];
 * evicted_tokens int64 [H]; member_frames int32 [H][B][rope_members]: the
 * frames of each slot's most recent members, most recent first (entries past
 * the slot's count unspecified). */
typedef struct {
  float* k_master;
  float* v_master;
  void* k_mirror;
  void* v_mirror;
  int32_t* count;
  int32_t* last;
  uint32_t* codes;
  int32_t* n_live;
  int64_t* evicted_tokens;
  int64_t frame;
  int32_t* member_frames;
} fastar_cache_state;

/* Thread-local text of the last error (empty string if none). */
const char* fastar_last_error(void);

/* Bytes of device workspace a cache with this configuration needs (host only).
 * The size depends only on the configuration, never on how many frames are
 * merged: the cache is bounded so memory stays constant over a rollout
 * (section 2A "Benefício"). */
fastar_status fastar_cache_workspace_bytes(const fastar_config* cfg, size_t* bytes);

/* Create a cache in caller-provided device memory (section 2A "Benefício": a
 * fixed budget of slots per head holds the merged groups, so this one
 * workspace serves a rollout of any length; "Mecanismo": the LSH hyperplanes
 * the cache hashes with are fixed at creation).
 * planes_host: the SimHash hyperplanes, [L][b][d] in cfg->dtype, or with
 * pq_subspaces = M > 0 the product-quantization codebooks [L][M][2^(b/M)][d/M];
 * copied into the workspace.  workspace_dev: at least fastar_cache_workspace_bytes bytes,
 * 256-byte aligned, kept alive by the caller until fastar_cache_destroy.
 * The cache starts empty (n_live = 0, frame = 0).  Returns
 * FASTAR_ERR_UNSUPPORTED if the current device is not gfx950.  On success
 * *out is a host handle owned by the library. */
fastar_status fastar_cache_create(const fastar_config* cfg, const void* planes_host,
                                  void* workspace_dev, size_t workspace_bytes, void* stream,
                                  fastar_cache_t* out);

/* Free the host handle (the workspace stays the caller's).  Library plumbing:
 * the pages describe no API. */
fastar_status fastar_cache_destroy(fastar_cache_t cache);

/* Empty the cache (state zeroed, frame = 0) on `stream`: the start of a new
 * rollout, whose first frame has no earlier frames to match (section 2A
 * "Mecanismo").  Changes the cache, so an AnnSA index built before it is
 * refused afterwards. */
fastar_status fastar_cache_reset(fastar_cache_t cache, void* stream);

/* Device pointer of the cache's hyperplanes ([L][b][d], cfg dtype), or of its
 * product-quantization codebooks ([L][M][2^(b/M)][d/M]) when pq_subspaces > 0
 * (section 2A "Mecanismo": the same LSH family hashes the new keys, e.g. with
 * fastar_hash, and the cached ones).  The pointer stays owned by the cache and
 * valid until its workspace is freed. */
fastar_status fastar_cache_planes(fastar_cache_t cache, const void** planes_dev);

/* SimHash codes of H x N vectors (section 2A "Mecanismo": LSH as the ANN).
 * x_dev: element (h, n, k) at x_dev[h*stride_h + n*stride_n + k], d in {64,128}.
 * planes_dev: [L][b][d], same dtype as x.  codes_dev: uint32 [H][L][N]
 * (bits above b are 0; b = 0 gives all-zero codes).  Stateless. */
fastar_status fastar_hash(const void* x_dev, fastar_dtype dtype, int32_t H, int32_t N, int32_t d,
                          int64_t stride_h, int64_t stride_n, const void* planes_dev, int32_t L,
                          int32_t b, uint32_t* codes_dev, void* stream);

/* Product-quantization codes of H x N vectors (section 2: the nearest-
 * neighbour search uses LSH or quantization; read as product quantization).
 * Table t splits the d features into M equal slices; slice m takes the index
 * of its nearest centroid (Euclidean, ties to the lowest index) among
 * 2^(b/M) in codebooks_dev[t][m] ([L][M][2^(b/M)][d/M], same dtype as x),
 * and the code holds slice m's index at bits [m*b/M, (m+1)*b/M).  x_dev,
 * strides and codes_dev ([H][L][N]) as for fastar_hash.  M in {1, 2, 4, 8},
 * d/M a multiple of 16, b = M x (1..8).  Stateless. */
fastar_status fastar_pq_codes(const void* x_dev, fastar_dtype dtype, int32_t H, int32_t N,
                              int32_t d, int64_t stride_h, int64_t stride_n,
                              const void* codebooks_dev, int32_t L, int32_t M, int32_t b,
                              uint32_t* codes_dev, void* stream);

/* Match, merge, evict, insert and re-hash `num_frames` frames of new tokens
 * (section 2A: top-1 match against previous frames, merge above a threshold,
 * bounded cache).  Frames are processed in order; frame f sees the state left
 * by frame f-1 (including earlier frames of the same call), never its own
 * tokens.  Token i of frame f of head h is k_dev/v_dev[h*stride_h +
 * (f*tokens_per_frame + i)*stride_n + k] (cfg dtype).  codes_dev: uint32
 * [H][L][num_frames*tokens_per_frame] codes of those keys, or NULL to hash them
 * here with the cache's hyperplanes.  Optional outputs, [H][num_frames *
 * tokens_per_frame]: slot_out_dev (slot each token ended in), merged_out_dev (1
 * if merged into an existing slot).  Requires tokens_per_frame <= budget and
 * <= FASTAR_MAX_TOKENS_PER_FRAME (then eviction always finds room). */
fastar_status fastar_match_merge(fastar_cache_t cache, const void* k_dev, const void* v_dev,
                                 int64_t stride_h, int64_t stride_n, const uint32_t* codes_dev,
                                 int32_t tokens_per_frame, int32_t num_frames,
                                 int32_t* slot_out_dev, uint8_t* merged_out_dev, void* stream);

/* Key projection with the SimHash codes taken in its epilogue (section 2A,
 * "Mecanismo": the keys TempCache hashes are the attention layer's keys).
 * For n_tok tokens x (row n at x_dev + n*x_stride, d_in bf16) and the layer's
 * key weight w (nn.Linear layout: out feature r at w_dev + r*w_stride, d_in
 * bf16; head h owns rows [h*d, (h+1)*d)), writes the bf16 keys k = x w^T,
 * rounded to nearest even once from fp32 accumulation, to (h, n, k) at
 * k_out_dev[h*k_stride_h + n*k_stride_n + k], and their codes under the
 * cache's hyperplanes to codes_dev[(h*L + t)*codes_ld + n] (uint32, the layout
 * fastar_match_merge takes).  No bias, normalisation or rotation.  Requires a
 * bf16 cache with SimHash codes (else FASTAR_ERR_UNSUPPORTED), d_in a
 * positive multiple of 32, 16-byte aligned x, w, k_out and row strides that
 * are multiples of 16 bytes, codes_ld >= n_tok.  Reads the cache's
 * hyperplanes only; all buffers stay the caller's.  Measured on MI355X at the
 * 1.3B-layer chunk (4680 tokens, d_in 1536, 12 heads) it is slower than a
 * library GEMM followed by fastar_hash (40 us against 27 + 9 us): it saves the
 * keys' second read, not time, at that shape. */
fastar_status fastar_project_keys(fastar_cache_t cache, const void* x_dev, int64_t x_stride,
                                  int32_t n_tok, int32_t d_in, const void* w_dev, int64_t w_stride,
                                  void* k_out_dev, int64_t k_stride_h, int64_t k_stride_n,
                                  uint32_t* codes_dev, int64_t codes_ld, void* stream);

/* Attention of Nq queries per head over the live slots (section 2A, Lemma 5.1:
 * logits shifted by the group size).  q_dev: (h, n, k) at q_dev[h*stride_h +
 * n*stride_n + k]; o_dev likewise with o_stride_h, o_stride_n (cfg dtype);
 * scale: logit scale, > 0, or 0 for 1/sqrt(d) (negative values are refused);
 * lse_dev: optional float [H][Nq],
 * natural-log partition function.  An empty cache gives zero outputs and
 * lse = -inf.  The call writes the slots' log-count shifts divided by the
 * scale into the cache's workspace before attending (a few bytes per slot),
 * and, on bf16 caches when the last round of workgroups would leave a
 * quarter or more of the GPU idle, the partial results of (head, query tile)
 * pairs whose key tiles it splits in four; so attention calls on one cache
 * must not overlap.  A split pair's outputs differ from the unsplit ones by
 * summation order only (within bf16 rounding). */
fastar_status fastar_attend(fastar_cache_t cache, const void* q_dev, int64_t stride_h,
                            int64_t stride_n, int32_t Nq, float scale, void* o_dev,
                            int64_t o_stride_h, int64_t o_stride_n, float* lse_dev, void* stream);

/* Attention of one denoising step of a chunk (the problem statement: frames
 * are streamed by an autoregressive diffusion model over a KV cache of the
 * frames already generated; section 2A, Lemma 5.1): each of Nq queries per
 * head attends, in one softmax, over the live slots (logit + ln count) and
 * n_new raw tokens of the chunk being denoised (count 1, no shift).  The
 * cache is read only; merging the chunk's final tokens is a separate
 * fastar_match_merge.  k_new_dev, v_new_dev: (h, j, k) at
 * k_new_dev[h*kv_stride_h + j*kv_stride_n + k] for j < n_new, cfg dtype,
 * 16-byte aligned, strides multiples of 16 bytes; the buffers stay the
 * caller's.  n_new = 0 is fastar_attend.  Other arguments and outputs as
 * fastar_attend; no slots and n_new = 0 give zero outputs and lse = -inf. */
fastar_status fastar_attend_with_chunk(fastar_cache_t cache, const void* q_dev, int64_t stride_h,
                                       int64_t stride_n, int32_t Nq, const void* k_new_dev,
                                       const void* v_new_dev, int64_t kv_stride_h,
                                       int64_t kv_stride_n, int32_t n_new, float scale, void* o_dev,
                                       int64_t o_stride_h, int64_t o_stride_n, float* lse_dev,
                                       void* stream);

/* Attention with the rotation-corrected M-degree approximation (LIPAR summary,
 * section 2B "Recuperação de Atenção", 1. "Aproximação de Grau-M": a group's
 * exponential sum from its m most recent tokens, corrected for the rotary
 * embedding; applied to the TempCache groups of section 2A).  The cache holds
 * keys without their temporal rotation; each live slot of count c contributes
 * the keys R(t_i) k_hat of its m' = min(m, c) most recent members' frames
 * t_i, each with logit shift ln(c / m'), and its value v_hat; queries arrive
 * rotated at their own frame.  R(t) turns features (2p, 2p+1),
 * p < rope_dims / 2, by t * rope_base^(-2p / rope_dims); frames are the
 * cache's frame counter at each member's merge.  Requires a bf16 cache made
 * with rope_members >= m >= 1 (else FASTAR_ERR_UNSUPPORTED / invalid
 * argument), rope_dims even in [0, d], rope_base > 0.  Other arguments and
 * outputs as fastar_attend.  The rotated keys are built in the cache's
 * workspace, so calls on one cache must not overlap. */
fastar_status fastar_attend_rope(fastar_cache_t cache, const void* q_dev, int64_t stride_h,
                                 int64_t stride_n, int32_t Nq, int32_t m, int32_t rope_dims,
                                 float rope_base, float scale, void* o_dev, int64_t o_stride_h,
                                 int64_t o_stride_n, float* lse_dev, void* stream);

/* AnnSA set-up (section 2C: the buckets of the cached keys): SimHash codes of
 * the cache's slot keys (its mirrors) under any hyperplanes, and a bucket
 * index of them kept in the cache, which fastar_annsa_attend reads.  Call it
 * after the last change of the cache (match_merge, import, reset) and before
 * fastar_annsa_attend.  planes_dev: [L][b][d] in the cfg dtype, 1 <= L <= 4.
 * codes_dev: optional copy of the codes, slot s of table t of head h at
 * codes_dev[(h*L + t)*codes_ld + s] for s < budget (codes_ld >= budget); only
 * the first n_live columns of a head are meaningful. */
fastar_status fastar_cache_hash_slots(fastar_cache_t cache, const void* planes_dev, int32_t L,
                                      int32_t b, uint32_t* codes_dev, int64_t codes_ld,
                                      void* stream);

/* AnnSA: attention of Nq queries per head over only those live slots that
 * share a bucket with the query (section 2C: each query attends only to the
 * keys of its own bucket(s); read as equal codes in at least one of L tables
 * of one LSH family).  Logits are shifted by the group size as in
 * fastar_attend.  q_codes_dev: uint32 [H][L][Nq] codes of the queries under
 * the hyperplanes of the latest fastar_cache_hash_slots (fastar_hash), which
 * must have been called with the same L after the last change of the cache
 * (else FASTAR_ERR_INVALID_ARGUMENT).  The candidates come from the bucket
 * index, so the work follows the number of shared (query, slot) pairs.  A
 * query that shares no bucket gets a zero output and lse = -inf.  Other
 * arguments as fastar_attend. */
fastar_status fastar_annsa_attend(fastar_cache_t cache, const void* q_dev, int64_t stride_h,
                                  int64_t stride_n, int32_t Nq, const uint32_t* q_codes_dev,
                                  int32_t L, float scale, void* o_dev, int64_t o_stride_h,
                                  int64_t o_stride_n, float* lse_dev, void* stream);

/* Totals over heads (section 2A "Benefício": the live-slot and eviction counts
 * show the cache staying within its budget).  Library plumbing for tests and
 * monitoring; synchronises `stream`. */
fastar_status fastar_cache_stats(fastar_cache_t cache, void* stream, fastar_stats* out);

/* Copy the state to host buffers (library plumbing for checkpoints and tests;
 * the pages describe no API).  Buffers are the caller's, shaped as in
 * fastar_cache_state; NULL members are skipped.  Synchronises `stream`. */
fastar_status fastar_cache_export(fastar_cache_t cache, void* stream, fastar_cache_state* out);

/* Overwrite the state from host buffers, for resume and tests (library
 * plumbing; the pages describe no API).  NULL members and frame = -1 keep the
 * current contents; then the bucket index is rebuilt.  The state it would leave
 * is checked first (members not given are read back from the device): n_live
 * in [0, budget], and every live slot s < n_live with count >= 1 and last in
 * [0, frame).  A state that fails returns FASTAR_ERR_INVALID_ARGUMENT and
 * leaves the cache unchanged.  Synchronises `stream`. */
fastar_status fastar_cache_import(fastar_cache_t cache, const fastar_cache_state* in, void* stream);

/* AnnCA selection (section 2B: keep the prompt tokens that share a bucket with
 * at least one query of the frame).  q_codes_dev: uint32 [H][L][F*Nf] codes of
 * the queries, frame g = columns [g*Nf, (g+1)*Nf); p_codes_dev: uint32
 * [H][L][Np] codes of the prompt keys.  Outputs: sel_idx_dev int32
 * [H][F][Np], the kept prompt ids of (h, g) in ascending order in the first
 * sel_count_dev[h*F + g] entries (the rest unspecified).  Requires
 * Nf <= FASTAR_MAX_ANNCA_QUERIES_PER_FRAME, Np <= FASTAR_MAX_ANNCA_PROMPT. */
fastar_status fastar_annca_select(const uint32_t* q_codes_dev, int32_t Nf, int32_t F,
                                  const uint32_t* p_codes_dev, int32_t Np, int32_t H, int32_t L,
                                  int32_t* sel_idx_dev, int32_t* sel_count_dev, void* stream);

/* Softmax attention of each frame's queries over a per-frame subset of keys
 * (section 2B: attention over the kept prompt tokens only; no logit bias).
 * q_dev (h, g*Nf + i, k); k_dev, v_dev (h, j, k) for j < Np with strides
 * kv_stride_h, kv_stride_n; sel_idx_dev / sel_count_dev as produced by
 * fastar_annca_select, or both NULL to attend over all Np keys (dense);
 * o_dev like q_dev with o strides.  A frame with an empty subset gets zero
 * outputs.  scale > 0, or 0 for 1/sqrt(d). */
fastar_status fastar_attend_subset(const void* q_dev, int64_t q_stride_h, int64_t q_stride_n,
                                   const void* k_dev, const void* v_dev, int64_t kv_stride_h,
                                   int64_t kv_stride_n, const int32_t* sel_idx_dev,
                                   const int32_t* sel_count_dev, int32_t Nf, int32_t F, int32_t Np,
                                   int32_t H, int32_t d, fastar_dtype dtype, float scale,
                                   void* o_dev, int64_t o_stride_h, int64_t o_stride_n,
                                   void* stream);

/* The AnnCA step in two launches (section 2B "Mecanismo": latent queries and
 * prompt keys share one hashed space; per frame, only the prompt tokens that
 * share a bucket with at least one of the frame's queries are attended).
 * First the queries are hashed into q_codes_dev (uint32 [H][L][F*Nf], written
 * exactly as fastar_hash writes them, under q_planes_dev [L][b][128] bf16);
 * then one attention launch has every workgroup build its frame's bucket
 * bitmaps from those codes, keep prompt row j iff p_codes_dev[(h*L + t)*Np + j]
 * (uint32, e.g. from fastar_hash of the prompt keys) equals a query's code of
 * table t for some t, and attend each query of the frame over the kept rows
 * only (no logit bias); a frame that keeps nothing gets zero outputs.  The
 * outputs equal fastar_hash of the queries, fastar_annca_select and
 * fastar_attend_subset, without the selection buffers and the select launch.
 * bf16 only, d = 128, 1 <= L <= 4, 0 <= b <= 16, Np <= 4096; q_dev, k_dev,
 * v_dev, o_dev and strides as fastar_attend_subset (frame g's queries are rows
 * [g*Nf, (g+1)*Nf) of head h); scale > 0, or 0 for 1/sqrt(d).  q_codes_dev is
 * caller-owned and holds the query codes on return. */
fastar_status fastar_annca_attend(const void* q_dev, int64_t q_stride_h, int64_t q_stride_n,
                                  const void* q_planes_dev, int32_t L, int32_t b,
                                  uint32_t* q_codes_dev, const uint32_t* p_codes_dev,
                                  const void* k_dev, const void* v_dev,
                                  int64_t kv_stride_h, int64_t kv_stride_n, int32_t Nf, int32_t F,
                                  int32_t Np, int32_t H, int32_t d, float scale, void* o_dev,
                                  int64_t o_stride_h, int64_t o_stride_n, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the AnnCA
 * step of fastar_annca_select followed by fastar_attend_subset, with the
 * per-frame selection (the kept prompt ids and their counts) held in a device
 * array inside the library instead of caller buffers.  It allocates nothing:
 * the array is a static device object of
 * (FASTAR_ANNCA_STATIC_MAX_SELECTED + FASTAR_ANNCA_STATIC_MAX_SEGMENTS) int32
 * (4 MiB + 16 KiB) that each GPU the library runs on holds until the process
 * ends.  Requires H*F <= FASTAR_ANNCA_STATIC_MAX_SEGMENTS and
 * H*F*Np <= FASTAR_ANNCA_STATIC_MAX_SELECTED (else FASTAR_ERR_CAPACITY).
 * Every call on one GPU shares that GPU's array and leaves its selection
 * there; calls that overlap on one GPU (other streams, other threads) race and
 * must be ordered by the caller.  Arguments as fastar_annca_select (q_codes_dev
 * [H][L][F*Nf], p_codes_dev [H][L][Np]) and fastar_attend_subset (q, k, v, o and
 * their strides, d, dtype, scale); the output equals that pair's. */
#define FASTAR_ANNCA_STATIC_MAX_SELECTED (1 << 20)
#define FASTAR_ANNCA_STATIC_MAX_SEGMENTS 4096
fastar_status fastar_annca_attend_static(const void* q_dev, int64_t q_stride_h, int64_t q_stride_n,
                                         const uint32_t* q_codes_dev, const void* k_dev,
                                         const void* v_dev, int64_t kv_stride_h,
                                         int64_t kv_stride_n, const uint32_t* p_codes_dev,
                                         int32_t Nf, int32_t F, int32_t Np, int32_t H, int32_t d,
                                         int32_t L, fastar_dtype dtype, float scale, void* o_dev,
                                         int64_t o_stride_h, int64_t o_stride_n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FASTAR_H */
