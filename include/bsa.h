/*
 * bsa.h - block-sparse spatiotemporal attention for MI355X (gfx950), C ABI.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps no state and allocates no device memory.  Calls that need scratch
 *     take a caller-owned workspace whose size comes from a *_workspace query.
 *   - Every call validates its arguments on the host first.  A failed check
 *     returns a non-zero bsa_status, writes a message readable through
 *     bsa_last_error() (per host thread), launches nothing and leaves every
 *     output untouched.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream).  No call synchronises.  A launch failure returns
 *     BSA_ERR_HIP with the HIP error text in bsa_last_error().
 *   - Results are deterministic: no floating-point atomics anywhere.
 *   - Q, K, V, O tensors are [B, H, N, D] with element strides (stride_b,
 *     stride_h, stride_n) and a contiguous D axis; all four share one shape.
 *     Token t of a video latent of F frames x P patches is frame t / P,
 *     in-frame raster position t % P (frame-major flattening).
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsa_status {
  BSA_OK = 0,
  BSA_ERR_ARG = 1,          /* invalid argument (null pointer, bad size, bad enum)   */
  BSA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. a head_dim)           */
  BSA_ERR_CAPACITY = 3,     /* an output buffer is too small                         */
  BSA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the query returned  */
  BSA_ERR_HIP = 5,          /* a HIP runtime call or kernel launch failed            */
  BSA_ERR_CHECK = 6,        /* a BSA_DEBUG invariant check of an output failed       */
  BSA_STATUS_MAX = 0x7fffffff  /* range sentinel: any 32-bit value is representable  */
} bsa_status;

/* The *_MAX enumerators are not values to pass: they make every 32-bit value
 * representable in the enum type, so the library can receive an unknown value
 * from a C caller and reject it without undefined behaviour. */
typedef enum bsa_dtype { BSA_DT_BF16 = 0, BSA_DT_F32 = 1, BSA_DT_MAX = 0x7fffffff } bsa_dtype;

typedef enum bsa_mask_kind {
  BSA_MASK_ALL = 0,            /* every block pair kept (dense attention)            */
  BSA_MASK_WINDOW_ANCHOR = 1,  /* local frame window + rotating global anchor frames */
  BSA_MASK_RADIAL = 2,         /* window shrinking with temporal distance            */
  BSA_MASK_KIND_MAX = 0x7fffffff
} bsa_mask_kind;

/* Block-mask description.
 *
 * Token rule (a real token pair q, k with frames fq, fk and positions pq, pk):
 *  WINDOW_ANCHOR - "[논문리뷰] LVSA: Training-Free Sparse Attention for Long Video
 *    Diffusion", section 3 Method & Key Results, Figures 1 and 2: kept when
 *    |fq - fk| <= window, or fk is an anchor frame, or (anchor_rows != 0 and fq
 *    is an anchor frame).  Anchor frames are {f < frames : f % anchor_period ==
 *    anchor_step % anchor_period}; anchor_step is the denoising step, so the
 *    anchor set rotates by one frame per step.  anchor_period 0 = no anchors.
 *  RADIAL - Radial Attention headline page (static mask, window shrinking
 *    exponentially with temporal distance, O(n log n)): kept when fq == fk, or
 *    |pq - pk| * 2^floor(log2 |fq - fk|) <= radial_w.
 *  ALL - every pair kept.
 * Block rule: blocks of `block` consecutive tokens; block pair (i, j) is kept
 * when any real token pair (q in block i, k in block j) is kept.  The sequence
 * has N = frames * frame_tokens real tokens and nb = ceil(N / block) blocks;
 * the last block may be partial (tokens past N do not exist).
 * Limits: frames, frame_tokens, block >= 1; block <= 4096; nb <= 46340;
 * window, anchor_period, anchor_step, radial_w >= 0. */
typedef struct bsa_mask_desc {
  int32_t kind;
  int32_t frames;
  int32_t frame_tokens;
  int32_t block;
  int32_t window;
  int32_t anchor_period;
  int32_t anchor_step;
  int32_t anchor_rows;
  int32_t radial_w;
} bsa_mask_desc;

typedef struct bsa_shape {
  int32_t B, H, N, D;
  int64_t stride_b, stride_h, stride_n; /* element strides; D is contiguous */
} bsa_shape;

/* Number of blocks nb = ceil(N / block) of a valid description, else -1. */
int32_t bsa_mask_num_blocks(const bsa_mask_desc* desc);

/* Build the block mask of `desc` as CSR on the device.
 * Operation: the block rule above (LVSA review page section 3; Radial Attention
 * headline page).  Integer-only, bit-exact.
 * row_ptr: int32[nb + 1] device, written with row offsets (row_ptr[0] = 0).
 * col_idx: int32[col_capacity] device, written with the kept key-block indices
 *          of each row in ascending order.  col_capacity must be >= nb * nb
 *          (the largest possible count), else BSA_ERR_CAPACITY.
 * row_order: nullable int32[nb + 1] device output, a launch schedule for
 *          bsa_block_sparse_attn_fwd: entries 0..nb-1 are a permutation of the
 *          rows, entry nb is the number nh of "long" rows (kept-block count at
 *          least 1.5 times the mean).  The nh long rows come first, by
 *          descending count (ties by ascending index), then the other rows in
 *          ascending index order.
 * The mask is shared by every batch and head. */
bsa_status bsa_build_block_mask(const bsa_mask_desc* desc, int32_t* row_ptr, int32_t* col_idx,
                                int64_t col_capacity, int32_t* row_order, void* stream);

/* Block-sparse softmax attention forward.
 * Operation (LVSA review page section 1 Key Terms and section 3; SVG-EAR page,
 * technical summary section 1: compute the kept blocks, skip the rest): for a
 * real query row q in block i, over the real keys t of kept blocks (i, j):
 *   l_t = scale * q . k_t,  out = sum_t exp(l_t - m) v_t / sum_t exp(l_t - m),
 *   lse = m + ln sum_t exp(l_t - m)  (m = max l_t).
 * Skipped blocks are never read.  A row with no kept block gets out = 0 and
 * lse = -inf.
 * q, k, v, o: device tensors of `dtype` with `shape`.  BSA_DT_BF16: bf16
 *   inputs, fp32 accumulation, o written in bf16 (round to nearest even);
 *   D in {64, 128}, block in {64, 128}.  BSA_DT_F32: fp32 end to end; D in
 *   {32, 64, 128}, block in {16, 32, 64, 128}.
 * lse: nullable fp32 [B, H, N] contiguous device array.
 * row_ptr, col_idx: the CSR from bsa_build_block_mask for the same N and block
 *   (nb = ceil(N / block) rows, ascending columns < nb).
 * row_order: nullable int32[nb + 1]; the schedule written by
 *   bsa_build_block_mask (any permutation of the nb rows followed by a count
 *   nh in [0, nb] is valid).  The first nh listed rows run first, for every
 *   batch and head, which keeps long rows out of the tail of the launch; the
 *   rest run in list order with each XCD taking a contiguous range of (batch,
 *   head, row).  Without it every row is in the second group, in index order.
 *   Results are bitwise identical with or without it.  Ignored by the fp32
 *   path.  Like col_idx, its device contents are trusted.
 * scale: the softmax scale (1/sqrt(D) for standard attention); must be finite
 *   and > 0 (BSA_ERR_ARG otherwise). */
bsa_status bsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                     float* lse, bsa_dtype dtype, const bsa_shape* shape,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     const int32_t* row_order, int32_t block, float scale,
                                     void* stream);

/* Transposed block mask: for every key block j the query blocks i with
 * (i, j) kept, ascending, as CSR (col_ptr int32 [nb + 1], row_idx int32, at
 * least nb * nb entries of capacity or BSA_ERR_CAPACITY).  row_ptr / col_idx
 * as bsa_build_block_mask writes them (device contents trusted: columns
 * ascending and in [0, nb)).  Deterministic; meant to be run once per mask. */
bsa_status bsa_transpose_block_mask(const int32_t* row_ptr, const int32_t* col_idx, int32_t nb, int32_t* col_ptr,
                                    int32_t* row_idx, int64_t capacity, void* stream);

/* Workspace bytes required by bsa_block_sparse_attn_bwd (Delta, fp32 per query
 * row, and the launch schedules of the mask's rows and columns); 0 if the
 * shape is invalid. */
size_t bsa_block_sparse_attn_bwd_workspace(const bsa_shape* shape);

/* Gradients of block-sparse attention (the backward pass of
 * bsa_block_sparse_attn_fwd).  Needed by the training uses on the pages: the
 * LoRA fine-tuning of Radial Attention for longer videos (hyper.ai headline)
 * and LinVideo's post-training (technical summary sections 1-2).  With
 * P = softmax(scale * Q K^T) over each row's kept keys (recomputed from lse):
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),  dQ = scale * dS K,
 *   dK = scale * dS^T Q.
 * q, k, v, o (the forward output), dO: bf16 device tensors with `shape`,
 *   D = 128; dq, dk, dv: bf16 outputs with the same layout.
 * lse: fp32 [B, H, N], natural log, as the forward writes it.
 * row_ptr, col_idx: the forward's block CSR for block = 128; col_ptr, row_idx:
 *   its transpose (bsa_transpose_block_mask).  Device contents trusted.
 * Precision: fp32 accumulation; P and dS enter the MFMA as bf16; Delta uses the
 *   bf16 forward output.  Deterministic (no atomics).  Rows without kept keys
 *   get zero dq; keys no row keeps get zero dk and dv.
 * scale: as in the forward, finite and > 0.
 * workspace: at least bsa_block_sparse_attn_bwd_workspace(shape) bytes,
 *   256-byte aligned.  Only bf16, D = 128, block = 128 (BSA_ERR_UNSUPPORTED). */
bsa_status bsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                     const float* lse, bsa_dtype dtype, const bsa_shape* shape,
                                     const int32_t* row_ptr, const int32_t* col_idx, const int32_t* col_ptr,
                                     const int32_t* row_idx, int32_t block, float scale, void* dq, void* dk,
                                     void* dv, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes required by bsa_linear_attn_fwd for `shape` (0 if the shape
 * is invalid).  The workspace holds per-chunk partial states (fp32), the
 * reduced S^T in bf16 and z. */
size_t bsa_linear_attn_workspace(const bsa_shape* shape);

/* Non-causal linear attention with the elu+1 feature map.
 * Operation (LinVideo page, technical summary sections 1-2: O(n) linear
 * attention replacing quadratic softmax attention), with phi(x) = x + 1 for
 * x > 0 and exp(x) otherwise:
 *   S = sum_n phi(k_n) v_n^T,  z = sum_n phi(k_n),
 *   o_n = phi(q_n)^T S / (phi(q_n)^T z)        (no softmax scale).
 * q, k, v, o: bf16 device tensors with `shape`; D in {64, 128}.  phi is taken in
 *   fp32; the MFMA operands phi(K), V, phi(Q) and S are bf16; S and z
 *   accumulate in fp32; the denominator is fp32.
 * S: nullable fp32 [B, H, D, D] device output (row d of S is phi-dimension d).
 * z: nullable fp32 [B, H, D] device output.
 * workspace: device buffer of at least bsa_linear_attn_workspace(shape) bytes,
 *   256-byte aligned, owned by the caller; contents need not be initialised.
 * Only dtype BSA_DT_BF16 is implemented (BSA_ERR_UNSUPPORTED otherwise). */
bsa_status bsa_linear_attn_fwd(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                               const bsa_shape* shape, float* S, float* z, void* workspace,
                               size_t ws_bytes, void* stream);

/* bsa_linear_attn_fwd without a workspace argument and without allocating, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same operation,
 * arguments (minus the workspace), kernels and launch plan as
 * bsa_linear_attn_fwd, so results are bitwise identical to it.  The scratch is
 * a file-scope device array of bsa_linear_attn_noalloc_max_scratch() bytes
 * (40 MiB) in the library, one per GPU, held until the process ends; its
 * address is looked up once per device on the first call there (no
 * hipMalloc, hipFree or allocating routine is called).  Every call on a GPU
 * shares that GPU's array and it keeps the last call's contents, so calls
 * that overlap on one GPU (concurrent streams or threads) race: serialise
 * them.  A shape whose workspace (bsa_linear_attn_workspace) exceeds the
 * array returns BSA_ERR_UNSUPPORTED before any launch (at D = 128 that is
 * beyond about 220 (batch, head) pairs). */
bsa_status bsa_linear_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                                       const bsa_shape* shape, float* S, float* z, void* stream);

/* Size in bytes of the scratch array of bsa_linear_attn_fwd_noalloc. */
size_t bsa_linear_attn_noalloc_max_scratch(void);

/* Workspace bytes required by bsa_causal_linear_attn_fwd for `shape` (0 if
 * the shape is invalid or not supported): the fp32 state partials of every
 * token split, B * H * splits * (D * D + D) * 4 bytes, splits being about
 * 512 / (B * H) (at least 1, at most the number of 32-token tiles). */
size_t bsa_causal_linear_attn_workspace(const bsa_shape* shape);

/* Causal (chunked) linear attention with the elu+1 feature map.
 * Operation: the linear attention of the LinVideo page (technical summary
 * sections 1-2) restricted to earlier tokens, the form used by causal
 * (autoregressive) video generators such as the Self-Forcing model of the
 * LIPAR page (sections 3 Key Contributions and 4 Results: causal as well as
 * bidirectional attention):
 *   S_n = S0 + sum_{m <= n} phi(k_m) v_m^T,  z_n = z0 + sum_{m <= n} phi(k_m),
 *   o_n = phi(q_n)^T S_n / (phi(q_n)^T z_n).
 * (S0, z0) is the state carried in from earlier tokens, so a long sequence can
 * be processed in pieces: passing the S_out, z_out of one call as S_in, z_in of
 * the next gives the same result as one call over the concatenation (up to
 * fp32 rounding of the carried state).
 * q, k, v, o: bf16 device tensors with `shape`, D = 128, 16-byte aligned rows.
 * S_in, z_in: nullable fp32 device inputs [B, H, D, D] (row d = phi dimension
 *   d) and [B, H, D]; both NULL (zero state) or both given.
 * S_out, z_out: nullable fp32 device outputs, the state after the last token;
 *   may be the same buffers as S_in, z_in.  All four 16-byte aligned.
 * Precision: phi is taken in fp32; phi(Q), phi(K), V, the step scores and S^T
 *   enter the MFMA as bf16; S, z, the scores and the denominator are fp32.
 * workspace: at least bsa_causal_linear_attn_workspace(shape) bytes, 256-byte
 *   aligned, owned by the caller; contents need not be initialised.
 * Only dtype BSA_DT_BF16 is implemented (BSA_ERR_UNSUPPORTED otherwise). */
bsa_status bsa_causal_linear_attn_fwd(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                                      const bsa_shape* shape, const float* S_in, const float* z_in,
                                      float* S_out, float* z_out, void* workspace, size_t ws_bytes,
                                      void* stream);

/* Mixed attention.  Source: "LinVideo: A Post-Training Framework towards O(n)
 * Attention in Efficient Video Generation", technical summary section 2 A.
 * Selective Transfer: a per-layer scalar r in [0, 1] blends quadratic
 * attention (r = 1) and linear attention (r = 0):
 *   o = r * block_sparse_attn(q, k, v; row_ptr, col_idx, block, scale)
 *       + (1 - r) * linear_attn(q, k, v)
 * (the quadratic branch is the block-sparse call above; an all-blocks mask is
 * dense attention).  bf16, D = 128.  With r = 1 only the quadratic branch runs
 * (workspace may be NULL), with r = 0 only the linear one (row_ptr, col_idx may
 * be NULL).  Otherwise the quadratic output is written to o first and the
 * linear pass blends into it row by row: each branch is rounded to bf16 once
 * before the blend (two roundings in all).
 * workspace: at least bsa_linear_attn_workspace bytes, 256-byte aligned.
 * r outside [0, 1] or NaN is rejected; with r > 0, scale must be finite and
 * > 0. */
bsa_status bsa_mixed_attn_fwd(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                              const bsa_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                              const int32_t* row_order, int32_t block, float scale, float r,
                              void* workspace, size_t ws_bytes, void* stream);

/* ---- token clustering ------------------------------------------------------
 * Source: "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video
 * Generation via Error-aware Routing", technical summary section 2 Method:
 * query and key tokens are grouped by similarity into clusters before the
 * cluster-block calls below, which take their rows in cluster order. */

/* Workspace bytes required by bsa_kmeans for `shape` and C clusters (0 if the
 * shape or C is invalid or not supported). */
size_t bsa_kmeans_workspace(const bsa_shape* shape, int32_t C);

/* k-means of the N token rows of every (batch, head): from the given centres,
 * `iters` Lloyd steps (assign each row to its nearest centre, move each centre
 * to the mean of its rows; a centre without rows stays), then a final
 * assignment to the final centres.  Ties go to the lowest centre index.
 * x: bf16 [B, H, N, D] device tensor with `shape`, D = 128.
 * C: clusters per (batch, head), 1 <= C <= 1024.
 * centroids: fp32 [B*H][C][D] device buffer; in: the initial centres, out: the
 *   final ones (the centres the returned labels refer to).
 * labels: int32 [B*H][N] device output, the cluster of every row.
 * perm, offsets: nullable int32 device outputs [B*H][N] and [B*H][C + 1]: the
 *   stable cluster order of the final labels (cluster a is rows
 *   [offsets[a], offsets[a+1]) of the permuted sequence, tokens in their
 *   original order; perm[i] is the original row of permuted row i), the
 *   q_off / k_off form the calls below take.
 * Precision: the assignment compares |c_b|^2 - 2 x.c_b with c_b the centre
 *   rounded to bf16 (fp32 MFMA accumulation of exact bf16 products); means are
 *   fp32 sums in a fixed order divided by the count.  Deterministic.
 * workspace: at least bsa_kmeans_workspace(shape, C) bytes, 256-byte aligned.
 * All pointers 16-byte aligned.  Only BSA_DT_BF16 (BSA_ERR_UNSUPPORTED). */
bsa_status bsa_kmeans(const void* x, bsa_dtype dtype, const bsa_shape* shape, int32_t C, int32_t iters,
                      float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* workspace,
                      size_t ws_bytes, void* stream);

/* Rows into cluster order: out[b, h, i] = x[b, h, perm[b*H + h][i]] for every
 * i < N.  x and out: device tensors of `dtype` (bf16 or fp32) with the layout
 * of `shape` (rows of a multiple of 16 bytes), distinct buffers.  perm: int32
 * [B*H][N] device array; an entry outside [0, N) leaves that output row
 * untouched.  Bit-exact copies. */
bsa_status bsa_gather_rows(const void* x, bsa_dtype dtype, const bsa_shape* shape, const int32_t* perm, void* out,
                           void* stream);

/* Rows back to token order: out[b, h, perm[b*H + h][i]] = y[b, h, i] (the
 * inverse of bsa_gather_rows for a permutation).  Same conventions. */
bsa_status bsa_scatter_rows(const void* y, bsa_dtype dtype, const bsa_shape* shape, const int32_t* perm, void* out,
                            void* stream);

/* ---- clustered sparse attention with centroid compensation ---------------
 * Source: "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video
 * Generation via Error-aware Routing", technical summary section 2 Method.
 * Inputs common to these calls:
 *   q, k, v: bf16 [B, H, N, D] device tensors (D in {64, 128}) whose rows are
 *     already ordered by cluster, per (batch, head): query cluster a is rows
 *     [q_off[a], q_off[a+1]) of q, key cluster b is rows [k_off[b], k_off[b+1])
 *     of k and v.
 *   q_off: int32 [B*H][Cq + 1], k_off: int32 [B*H][Ck + 1] device arrays,
 *     non-decreasing from 0 to N (not checked on the host: offsets outside
 *     [0, N] are undefined behaviour).  Empty clusters are allowed.
 *   A block is a (query cluster a, key cluster b) pair with cost n_a * n_b.
 *   Centroid arrays are fp32 row-major: q_cent [B*H][Cq][D], k_cent and
 *   v_cent [B*H][Ck][D].  Scores are fp32 [B*H][Cq][Ck]. */

/* Step 1 (idea 1, cluster centroids): q_cent[a] = mean of the q rows of cluster
 * a; k_cent[b], v_cent[b] = means of the k and v rows of key cluster b (fp32
 * accumulation; an empty cluster gets zeros).  q_cent may be NULL (then q is
 * not read), or k_cent and v_cent both NULL (then k and v are not read); the
 * route-score call computes the key and value centroids itself, so the
 * routing path asks for the query centroids only. */
bsa_status bsa_cluster_centroids(const void* q, const void* k, const void* v, bsa_dtype dtype,
                                 const bsa_shape* shape, const int32_t* q_off, int32_t Cq,
                                 const int32_t* k_off, int32_t Ck, float* q_cent, float* k_cent,
                                 float* v_cent, void* stream);

/* Workspace bytes of bsa_route_scores (0 for an invalid shape). */
size_t bsa_route_scores_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck);

/* Step 2 (idea 2, error estimation by probing with query-cluster centroids as
 * proxies, streamed without storing logits): with l_aj = scale * c^_a . k_j over
 * all keys j, m_a = max_j l_aj, Z_a = sum_j exp(l_aj - m_a),
 *   e_ab = (sum_{j in b} exp(l_aj - m_a) v_j - n_b exp(scale c^_a . c_b - m_a) vbar_b) / Z_a,
 *   score[a][b] = |e_ab|^2 / n_b  (squared output error per unit cost),
 * and 0 when cluster a or b is empty.  q_cent (input) holds the query
 * centroids c^_a (bsa_cluster_centroids); the key and value centroids c_b,
 * vbar_b (idea 1) are computed in the same pass over k and v and written to
 * k_cent and v_cent (outputs, as bsa_cluster_centroids would give them up to
 * fp32 rounding order), so k and v are read once.  Head_dim 128: the pass
 * accumulates U_ab = sum_{j in b} exp(l_aj - m_a) v_j with the proxies and the
 * weights split into two bf16 MFMA operands each (about 16 significant bits),
 * takes scale c^_a . c_b as the mean of the keys' logits, and forms
 * U_ab - n_b exp(scale c^_a . c_b - m_a) vbar_b in fp32; head_dim 64 takes the
 * centroids first and accumulates the difference directly.
 * workspace: at least bsa_route_scores_workspace bytes, 256-byte aligned. */
bsa_status bsa_route_scores(const void* k, const void* v, bsa_dtype dtype, const bsa_shape* shape,
                            const int32_t* q_off, int32_t Cq, const int32_t* k_off, int32_t Ck,
                            const float* q_cent, float* k_cent, float* v_cent, float scale, float* score,
                            void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of bsa_route_select (0 for an invalid shape). */
size_t bsa_route_select_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck);

/* Step 3 (idea 2, error-to-cost routing under a density budget): per (batch,
 * head), order the non-empty blocks by (score descending, a * Ck + b
 * ascending) and keep the longest prefix whose total cost is <=
 * floor(N * N * density_ppm / 10^6) (integer arithmetic, bsa_route_budget).  Bit-exact for a given
 * score array.  Output CSR per (batch, head): route_row_ptr int32 [B*H][Cq + 1]
 * (offsets relative to that head's route_col segment), route_col int32
 * [B*H][Cq * Ck] with the kept key clusters of each query cluster ascending.
 * density_ppm in [0, 10^6].  Scores must be non-negative and not NaN (the
 * order is taken on their bit patterns).  workspace: at least
 * bsa_route_select_workspace bytes, 256-byte aligned (keep flags and the cost
 * histograms of the first selection level). */
bsa_status bsa_route_select(const float* score, const bsa_shape* shape, const int32_t* q_off,
                            int32_t Cq, const int32_t* k_off, int32_t Ck, int32_t density_ppm,
                            int32_t* route_row_ptr, int32_t* route_col, void* workspace,
                            size_t ws_bytes, void* stream);

/* The density budget of bsa_route_select, in scores per (batch, head):
 * floor(N * N * density_ppm / 10^6), computed exactly (128-bit intermediate);
 * -1 for N < 0 or density_ppm outside [0, 10^6].  Host only. */
int64_t bsa_route_budget(int32_t N, int32_t density_ppm);

/* Step 4 (idea 1, parameter-free linear compensation): for a query q of
 * cluster a, one softmax over the exact keys of the kept clusters of route row
 * a and one virtual key per skipped non-empty cluster b (key k_cent[b], value
 * v_cent[b], logit scale * q . k_cent[b] + ln n_b), i.e. the n_b keys of a
 * skipped cluster are replaced by n_b copies of their centroid.  o (bf16) and
 * lse (nullable fp32 [B, H, N]) are in the cluster order of q.  Ck <= 512.
 * The centroids enter the dot products rounded to bf16, like any key.
 * workspace: at least bsa_compensated_attn_workspace bytes, 256-byte aligned
 * (may be NULL when that is 0). */
bsa_status bsa_compensated_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                    bsa_dtype dtype, const bsa_shape* shape, const int32_t* q_off,
                                    int32_t Cq, const int32_t* k_off, int32_t Ck,
                                    const int32_t* route_row_ptr, const int32_t* route_col,
                                    const float* k_cent, const float* v_cent, float scale,
                                    void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of bsa_compensated_attn_fwd: for head_dim 128, bf16 copies of
 * the key and value centroids (the virtual keys and values) and the launch's
 * tile schedule (per-cluster work, and the 128-row query tiles ordered longest
 * first); 0 otherwise (then workspace may be NULL).  0 for an invalid shape as
 * well. */
size_t bsa_compensated_attn_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck);

/* Workspace bytes of bsa_centroid_compensate (0 for an invalid shape). */
size_t bsa_centroid_compensate_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck);

/* Steps 1-4 in one call.  use_given_route = 0: query centroids, route scores
 * (with the key and value centroids from the same pass), route selection at
 * density_ppm, compensated attention; route_row_ptr / route_col receive the
 * route and score (nullable) the scores.  use_given_route = 1: route_row_ptr
 * / route_col are inputs (a route from an earlier call, or any route of the
 * form bsa_route_select writes); the call takes the centroids and runs the
 * compensated attention on that route (density_ppm and score are ignored).
 * workspace: at least bsa_centroid_compensate_workspace bytes, 256-byte
 * aligned. */
bsa_status bsa_centroid_compensate(const void* q, const void* k, const void* v, void* o, float* lse,
                                   bsa_dtype dtype, const bsa_shape* shape, const int32_t* q_off,
                                   int32_t Cq, const int32_t* k_off, int32_t Ck, int32_t density_ppm,
                                   int32_t use_given_route, float scale, int32_t* route_row_ptr,
                                   int32_t* route_col, float* score, void* workspace, size_t ws_bytes,
                                   void* stream);

/* ---- latent inter-frame pruning and restoration --------------------------
 * Source: "LIPAR: 비디오 생성 AI 를 위한 '스마트 스킵' 기술" (summary of the
 * LIPAR paper), section 2 Methodology, B. LIPAR pipeline: latent inter-frame
 * pruning (patches whose difference to the adjacent frame is at most tau are
 * dropped) and restoration (the pruned sequence is expanded back by copying the
 * previous frame's patches).
 * Each (batch, head) slice of x [B, H, N, D] (bf16, D a multiple of 8, at most
 * 4096) is one token sequence of `frames` frames of P = N / frames patches,
 * token n = f * P + p.  Token (f, p), f >= 1, is kept iff
 *   sum_c |x[f, p, c] - x[f - 1, p, c]| > tau * D
 * (mean absolute difference to the same patch of the previous input frame
 * above tau), the differences and their sum taken in float64 from the bf16
 * values (exact for values within a normal exponent range), compared with the
 * float64 product of the float tau and D; frame 0 is always kept.  tau may be
 * negative (keep all) or +inf (keep frame 0 only); NaN is rejected.
 * The motion-detection refinement the page mentions is not specified there and
 * is not applied. */

/* Outputs, all caller-owned device arrays, per sequence r = b * H + h:
 *   keep     uint8 [B*H][N]  1 if kept
 *   cpos     int32 [B*H][N]  number of kept tokens before token n (the position
 *                            of a kept token in the pruned sequence)
 *   kept_idx int32 [B*H][N]  entries 0 .. n_kept[r] - 1: the kept tokens, ascending
 *   n_kept   int32 [B*H]
 *   x_pruned bf16 dense [B*H][N][D]: rows 0 .. n_kept[r] - 1 are the kept rows in
 *            token order (row j of sequence r at ((r * N) + j) * D); the other
 *            rows are left untouched. */
bsa_status bsa_lipar_prune(const void* x, bsa_dtype dtype, const bsa_shape* shape, int32_t frames,
                           float tau, uint8_t* keep, int32_t* cpos, int32_t* kept_idx,
                           int32_t* n_kept, void* x_pruned, void* stream);

/* Restoration: out [B, H, N, D] (bf16, strides of shape) gets, for a kept token
 * n, row cpos[n] of y_pruned (dense [B*H][N][D] like x_pruned above), and for a
 * pruned token (f, p) the restored row of (f - 1, p): the row of the latest kept
 * frame of patch p.  keep and cpos as written by bsa_lipar_prune. */
bsa_status bsa_lipar_restore(const void* y_pruned, bsa_dtype dtype, const bsa_shape* shape,
                             int32_t frames, const uint8_t* keep, const int32_t* cpos, void* out,
                             void* stream);

/* Measurement reference (not part of the attention path): streams `bytes` of
 * the device buffer `buf` once with 16-byte loads and writes nothing but, at
 * most, one word of `sink` (device, 4 bytes).  Timed over a buffer larger than
 * the last-level cache it gives the read-only HBM rate that the HBM-bound
 * kernels are compared with.  buf 16-byte aligned, bytes a multiple of 16. */
bsa_status bsa_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Host-side check of a block CSR held in HOST memory: row_ptr [nrows + 1]
 * starts at 0 and never decreases, row_ptr[nrows] <= capacity, and every row's
 * columns lie in [0, ncols) in strictly ascending order.  Returns BSA_OK, or
 * BSA_ERR_ARG / BSA_ERR_CAPACITY naming the first violation in
 * bsa_last_error().  Reads nothing past row_ptr[nrows] entries of col_idx.
 *
 * Debug mode: while the environment variable BSA_DEBUG holds a non-empty value
 * other than "0" (read at each call), bsa_build_block_mask,
 * bsa_route_select and bsa_centroid_compensate (routing mode) synchronise
 * their stream after the launch, copy the CSR they wrote to the host and run
 * this check on it, returning BSA_ERR_CHECK on a violation.  That costs a
 * synchronisation and a copy per call; it is meant for debugging, not for
 * stream capture. */
bsa_status bsa_check_csr(const int32_t* row_ptr, const int32_t* col_idx, int32_t nrows, int32_t ncols,
                         int64_t capacity);

/* Text of a status code (static storage). */
const char* bsa_status_string(bsa_status status);

/* Detail of the last failure on the calling host thread ("" if none). */
const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
