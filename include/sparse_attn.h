/*
 * sparse_attn.h -- C-ABI of the MI355X (gfx950) dynamic block-sparse
 * self-attention library (libsparse_attn.so).
 *
 * What the library computes follows the NABLA summary page ("NABLA:
 * Neighborhood Adaptive Block-Level Attention", section "Methodologie :
 * NABLA"): tokens of a latent video grid T x H x W arrive in tile-major order
 * (item "Reordonnancement des Jetons", fractal flattening: one 1 x 8 x 8 tile
 * of 64 tokens per block), Q and K are mean-pooled per block
 * ("Sous-echantillonnage"), a softmax attention map is taken over the pooled
 * blocks ("Attention Reduite"), each of its rows is cut by the CDF threshold
 * ("Seuil CDF"), optionally united with a static sliding-tile window
 * ("Integration Hybride avec STA", M = M_nabla OR M_STA), and exact softmax
 * attention is then run over the kept 64 x 64 tiles only ("Expansion").
 *
 * Conventions shared by every entry point
 *   - Tensors are dense row-major [B, H, N, d].  The blocks are the
 *     nT x nTy x nTx = ceil(grid / tile) tiles of the token grid, frame-block
 *     outermost, and a tile-major tensor has N = 64 nB slots: block b of a head
 *     is slots [64 b, 64 b + 64), row-major inside its tile.  On a grid that is
 *     not a whole number of tiles (item "Fractal Flattening": patches whatever the
 *     global size of the video), the last tile along an axis is partial and its
 *     slots beyond the grid are padding: their contents must be finite but do not
 *     matter (sparse_attn_to_tiles writes zeros); pooling leaves them out, the
 *     attention gives them no weight as keys, and as queries they get O = 0 and
 *     LSE = -inf.  Raster tensors (sparse_attn_to_tiles and friends) have
 *     N = grid_t*grid_h*grid_w.  Element type is given by shape->dtype (fp32 or
 *     bf16); q, k, v and out share it.
 *   - All pointers named as device pointers must point to device memory (or
 *     memory the device can address) and be 16-byte aligned.  Host pointers
 *     are read during the call only and are not retained.
 *   - The caller owns every buffer.  The library allocates and frees nothing
 *     and keeps no state between calls; scratch space comes in through
 *     `workspace` (see sparse_attn_workspace_size).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously: no call synchronises the host, except the
 *     debugging check sparse_attn_select_check.  Concurrent
 *     calls are safe as long as they do not share output or workspace
 *     buffers.
 *   - Return value: SPARSE_ATTN_OK (0) or a negative status.  Every argument
 *     is checked on the host before anything is enqueued, so a call that
 *     fails a check launches nothing and writes nothing.  SPARSE_ATTN_HIP_ERROR
 *     reports a launch failure (work enqueued before it may have run).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_VERSION 10000 /* 1.0.0 */

/* element types */
#define SPARSE_ATTN_F32 0
#define SPARSE_ATTN_BF16 1

/* status codes */
#define SPARSE_ATTN_OK 0
#define SPARSE_ATTN_INVALID_ARGUMENT (-1) /* null/misaligned pointer, bad size, bad threshold   */
#define SPARSE_ATTN_UNSUPPORTED (-2)      /* dtype, head_dim, tile or size not implemented      */
#define SPARSE_ATTN_CAPACITY (-3)         /* col_idx shorter than the worst case B*H*nB*nB      */
#define SPARSE_ATTN_WORKSPACE (-4)        /* workspace smaller than sparse_attn_workspace_size  */
#define SPARSE_ATTN_HIP_ERROR (-5)        /* a kernel launch failed                             */
#define SPARSE_ATTN_LOOKBACK_FAULT (-6)   /* a selection gave up in its CSR look-back (see
                                             sparse_attn_select_check)                          */
#define SPARSE_ATTN_SCRATCH (-7)          /* shape too large for sparse_attn_select_noalloc      */

/* Size of the static device scratch of sparse_attn_select_noalloc (96 MiB). */
#define SPARSE_ATTN_SCRATCH_BYTES (96ll << 20)

/*
 * Problem shape.  head_dim must be 64 or 128; the tile must hold 64 tokens
 * (1 x 8 x 8 in the video workloads; any tile_t x tile_h x tile_w of volume 64
 * works) and need not divide the grid (see partial tiles above; the clustering
 * selector takes whole tiles only).  scale is the
 * softmax scale of both the pooled scores and the attention; it must be
 * finite and >= 0, and 0 means 1/sqrt(head_dim).  The worst-case block
 * count B*H*nB*nB (nB = blocks per head) must fit in int32.
 */
typedef struct sparse_attn_shape {
    int32_t batch, heads, head_dim;
    int32_t grid_t, grid_h, grid_w;
    int32_t tile_t, tile_h, tile_w;
    int32_t dtype;
    float scale;
} sparse_attn_shape;

/*
 * Selection parameters.
 *   threshold        CDF mass to keep per query block, in (0, 1]; values >= 1
 *                    keep every block.  NaN or <= 0 is rejected.
 *   head_thresholds  optional HOST array [heads] overriding `threshold` per
 *                    head (same rules), or NULL.  At most 1024 heads.
 *   win_t/h/w        radii, in blocks, of the static window united with the
 *                    CDF mask: key block j is also kept when |dt| <= win_t,
 *                    |dy| <= win_h and |dx| <= win_w between the block
 *                    coordinates of query and key (clipped at the grid edges,
 *                    no wrap).  Any negative radius turns the window off.
 */
typedef struct sparse_attn_select_params {
    float threshold;
    const float *head_thresholds;
    int32_t win_t, win_h, win_w;
} sparse_attn_select_params;

/* Library version (SPARSE_ATTN_VERSION of the build). */
int32_t sparse_attn_version(void);

/* Static text for a status code (never NULL). */
const char *sparse_attn_status_string(int32_t status);

/*
 * Worst-case number of kept blocks, B*H*nB*nB, i.e. the col_idx length
 * sparse_attn_select and sparse_attn_mask_to_csr require.  Negative status
 * if the shape is invalid or the worst case does not fit in int32.
 */
int64_t sparse_attn_csr_capacity(const sparse_attn_shape *shape);

/*
 * Bytes of device workspace needed by every entry point for this shape
 * (one size serves select, forward and mask_to_csr).  Negative status if
 * the shape is invalid.
 */
int64_t sparse_attn_workspace_size(const sparse_attn_shape *shape);

/*
 * Outcome of the last selection (sparse_attn_select, _select_raster, _select_sip or
 * _select_ibcs) that used `workspace`, for callers that want to confirm a block
 * list before using it.  The selections chain the CSR offsets of their row groups
 * through a look-back whose waits are bounded; a group that runs out of polls
 * writes -1 as the row_ptr entry of each of its rows (so the block list fails any
 * validity check) and sets a fault word in the workspace.  This call reads that
 * word: it enqueues a 4-byte device-to-host copy on `stream` and, unlike every
 * other entry point, waits for the stream to finish.
 *   Returns SPARSE_ATTN_OK, SPARSE_ATTN_LOOKBACK_FAULT, or an argument status
 *   (checked on the host first, as everywhere).
 * The wait is 2^22 polls.  The environment variable SPARSE_ATTN_LOOKBACK_SPIN_CAP
 * (a decimal count, at most 2^22, read by each selection call) lowers it, so that
 * tests can drive the give-up path without hanging anything; 0 gives up at the
 * first unpublished word.
 */
int32_t sparse_attn_select_check(const sparse_attn_shape *shape, const void *workspace, int64_t workspace_bytes,
                                 void *stream);

/*
 * Dynamic block selection (pooling, reduced attention map, CDF cut, window
 * union) emitted as a CSR block list.
 *
 *   q, k        device, [B, H, N, d] in shape->dtype, tile-major tokens.
 *   row_ptr     device, int32 [B*H*nB + 1], written: row r = (b*H + h)*nB + i
 *               owns col_idx[row_ptr[r] .. row_ptr[r+1]); row_ptr[0] = 0 and
 *               row_ptr[B*H*nB] = nnz (left on the device, not returned).
 *   col_idx     device, int32 [col_capacity]; entries [0, nnz) are written,
 *               strictly ascending key-block indices within each row.
 *   col_capacity  must be >= sparse_attn_csr_capacity(shape).
 *   workspace   device, >= sparse_attn_workspace_size(shape) bytes; its
 *               contents on entry do not matter.
 * Ties in the CDF order go to the lower key-block index.  A row of pooled
 * scores is held in registers, so nB <= 4096 blocks per head (262,144
 * tokens); larger grids return SPARSE_ATTN_UNSUPPORTED.
 */
int32_t sparse_attn_select(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                           const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                           int64_t col_capacity, void *workspace, int64_t workspace_bytes,
                           void *stream);

/* Parameters of sparse_attn_select_sip. */
typedef struct {
    float budget;    /* expected kept key blocks per row, > 0 (>= nB keeps every block) */
    uint64_t seed;   /* seed of the SplitMix64 stream the draws come from */
} sparse_attn_sip_params;

/*
 * Block selection by sampling with inclusion-probability weighting, the second
 * technique of AB-Attention (AB-Attention page, section "Les trois techniques
 * d'AB-Attention"), on NABLA's pooled scores: for each row, p_j is the softmax of
 * the pooled scores over all key blocks (as in sparse_attn_select), the
 * inclusion probabilities are pi_j = min(1, c p_j) with c such that
 * sum_j pi_j = budget (the blocks whose c p_j reaches 1 are always kept), and
 * block j of row r is kept when u < pi_j, where u is the top 24 bits of output
 * r*nB + j + 1 of the SplitMix64 stream seeded with params->seed, times 2^-24.
 * Every kept block gets the logit offset -ln(pi_j), for
 * sparse_attn_forward_biased: the Horvitz-Thompson weight 1/pi_j.
 *
 *   q, k, row_ptr, col_idx, col_capacity, workspace: as in sparse_attn_select.
 *   col_bias    device, fp32 [col_capacity]; entries [0, nnz) are written,
 *               aligned with col_idx.
 * bf16 or fp32, nB <= 4096 (SPARSE_ATTN_UNSUPPORTED otherwise); a budget that is
 * not a finite positive number is SPARSE_ATTN_INVALID_ARGUMENT.
 */
int32_t sparse_attn_select_sip(const sparse_attn_shape *shape, const sparse_attn_sip_params *params,
                               const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                               float *col_bias, int64_t col_capacity, void *workspace,
                               int64_t workspace_bytes, void *stream);

/*
 * Block selection with the intra-block clustering selector, the first technique
 * of AB-Attention (AB-Attention page, section "Les trois techniques
 * d'AB-Attention"), cut by NABLA's CDF rule.  Each pair of query blocks
 * (2p, 2p+1: 128 tokens; an odd last block alone) is clustered by Lloyd's
 * k-means, 8 clusters and 4 rounds, started from the queries at positions n*c/8
 * (ties to the lower cluster; an empty cluster keeps its centroid), with weights
 * equal to the last assignment's shares.  Key block j scores
 * p~_j = sum_c w_c softmax_j(mu_c . Kbar_j * scale) over all key blocks, and both
 * blocks of the pair keep the blocks NABLA's CDF rule keeps on p~ (threshold,
 * per-head thresholds and window as in sparse_attn_select).
 *
 *   Arguments as in sparse_attn_select.  bf16 or fp32, nB <= 4096, whole tiles
 *   (SPARSE_ATTN_UNSUPPORTED otherwise).
 */
int32_t sparse_attn_select_ibcs(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                                int64_t col_capacity, void *workspace, int64_t workspace_bytes,
                                void *stream);

/*
 * Block-sparse attention forward over a CSR block list (from
 * sparse_attn_select, sparse_attn_mask_to_csr or the caller).
 *
 *   q, k, v     device, [B, H, N, d] in shape->dtype.
 *   row_ptr     device, int32 [B*H*nB + 1], non-decreasing, row_ptr[0] = 0.
 *   col_idx     device, int32 [col_count]; each row's entries are strictly
 *               ascending key-block indices in [0, nB) (the order
 *               sparse_attn_select and sparse_attn_mask_to_csr produce).  An
 *               entry outside [0, nB) or not above the row's previous accepted
 *               entry is skipped; row ends beyond col_count are clipped to
 *               col_count.
 *   out         device, [B, H, N, d] in shape->dtype: for each query token,
 *               softmax(scale * q k^T) v over the tokens of the row's key
 *               blocks.  A row with no block gives zeros.
 *   lse         optional device fp32 [B, H, N] (natural-log log-sum-exp of
 *               the scaled logits; -inf for an empty row), or NULL.
 *   workspace   device, >= sparse_attn_workspace_size(shape) bytes; its
 *               contents on entry do not matter.  In bf16 the call plans the
 *               work first: pairs of query blocks whose rows are much longer
 *               than the average share are cut into pieces that are merged by
 *               their log-sum-exp, so that no single row holds the GPU up.
 * Calls that share one workspace must not overlap on different streams.
 */
int32_t sparse_attn_forward(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                            const int32_t *row_ptr, const int32_t *col_idx, int64_t col_count,
                            void *out, float *lse, void *workspace, int64_t workspace_bytes,
                            void *stream);

/*
 * sparse_attn_forward with a logit offset per block-list entry: the keys of
 * entry e's block get col_bias[e] added to their scaled logits before the
 * softmax (numerator and normaliser alike).  This is how AB-Attention's
 * sampling with inclusion-probability weighting ("SIP", AB-Attention page,
 * section "Les trois techniques d'AB-Attention") applies its Horvitz-Thompson
 * weights: offset -ln(pi) makes a block count 1/pi times.
 *
 *   col_bias    device, fp32 [col_count], finite values in natural-log units,
 *               aligned with col_idx (skipped entries' offsets are ignored).
 *               NULL is allowed only when col_count == 0.
 *   lse         as in sparse_attn_forward, including the offsets.
 * Everything else as in sparse_attn_forward (bf16 or fp32; the fp32 kernel adds the
 * offsets to a tile's scaled scores before taking its max).
 */
int32_t sparse_attn_forward_biased(const sparse_attn_shape *shape, const void *q, const void *k,
                                   const void *v, const int32_t *row_ptr, const int32_t *col_idx,
                                   const float *col_bias, int64_t col_count, void *out, float *lse,
                                   void *workspace, int64_t workspace_bytes, void *stream);

/*
 * sparse_attn_forward over a list of 4-token key blocks: AB-Attention's fine
 * selection on coarse hardware (AB-Attention page, section "Les trois techniques
 * d'AB-Attention", third technique): key and value blocks of 4 tokens, and the kernel
 * gathers the kept ones by index into full 64-key tiles for the matrix cores, with no
 * copy or permutation of the tokens.
 *
 *   row_ptr     as in sparse_attn_forward: one row per 64-token query block.
 *   col_idx     device, int32 [col_count]: 4-token key-block indices in [0, 16 nB)
 *               (key block j is tile-major tokens [4 j, 4 j + 4), half a row of an
 *               8 x 8 tile), ascending per row; out-of-range, repeated or descending
 *               entries are skipped as in sparse_attn_forward.
 *   Everything else as in sparse_attn_forward: for each query token, the softmax over
 *   the tokens of its row's 4-token blocks, applied to V.
 * bf16 and whole tiles only (SPARSE_ATTN_UNSUPPORTED otherwise).
 */
int32_t sparse_attn_forward_gather(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                                   const int32_t *row_ptr, const int32_t *col_idx, int64_t col_count, void *out,
                                   float *lse, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Selection of 4-token key blocks for each 64-token query block: AB-Attention's
 * fine key/value blocks (AB-Attention page, section "Les trois techniques
 * d'AB-Attention", third technique), chosen with NABLA's rule (NABLA summary page,
 * section "Methodologie : NABLA": "Sous-echantillonnage", "Attention Reduite",
 * "Seuil CDF").  For query block i of head h: qbar_i = mean of its 64 tokens,
 * kbar_j = mean of tile-major key tokens [4 j, 4 j + 4) for j in [0, 16 nB), scores
 * qbar_i . kbar_j * scale, softmax over all 16 nB key blocks of the head, and the
 * blocks kept in descending probability while the mass before them is below the
 * threshold (ties to the lower index; threshold >= 1 keeps every block).  The
 * near-ties at the cut are ordered by their exact scores, as in sparse_attn_select.
 * The list feeds sparse_attn_forward_gather.
 *
 *   q, k         device bf16 [B, H, N, head_dim], tile-major, 16-byte aligned.
 *   params       threshold / head_thresholds as in sparse_attn_select; the window
 *                must be off (it is a box of 64-token blocks): UNSUPPORTED otherwise.
 *   row_ptr      device int32 [B*H*nB + 1]; col_idx device int32 [col_capacity], with
 *                col_capacity >= sparse_attn_fine_csr_capacity (B*H*nB*16nB);
 *                4-token key-block indices, ascending per row.
 *   workspace    device, >= sparse_attn_fine_workspace_size bytes.
 * bf16, whole tiles and nB <= 512 only (SPARSE_ATTN_UNSUPPORTED otherwise).  A
 * selection that gives up in its look-back writes -1 into the row_ptr entries of
 * the rows it could not place, so that the list fails every validity check.
 */
int32_t sparse_attn_select_fine(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                                int64_t col_capacity, void *workspace, int64_t workspace_bytes, void *stream);

/* Worst-case col_idx entries of sparse_attn_select_fine (B*H*nB*16nB), or a negative
   status when the shape is unsupported. */
int64_t sparse_attn_fine_csr_capacity(const sparse_attn_shape *shape);

/* Workspace bytes of sparse_attn_select_fine, or a negative status. */
int64_t sparse_attn_fine_workspace_size(const sparse_attn_shape *shape);

/*
 * External block mask to CSR (the path that accepts a caller's mask, e.g. a
 * static window or a mask reused from an earlier step).
 *
 *   block_mask  device, uint8 [B, H, nB, nB]; nonzero = keep key block j for
 *               query block i.
 *   row_ptr, col_idx, col_capacity, workspace: as in sparse_attn_select.
 */
int32_t sparse_attn_mask_to_csr(const sparse_attn_shape *shape, const uint8_t *block_mask,
                                int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                                void *workspace, int64_t workspace_bytes, void *stream);

/* Parameters of sparse_attn_radial_csr (block-grid units). */
typedef struct {
    float r0;        /* window width at frame distance 0, finite, >= 0 */
    float gamma;     /* width decay per frame of distance, in (0, 1] */
    int32_t lambda;  /* every lambda-th frame of distance keeps its co-located block; 0 = off */
} sparse_attn_radial_params;

/*
 * DynamicRad's radial window (DynamicRad page, section "Methodologie :
 * DynamicRad", items A and B: a shared candidate set from the decay of
 * attention with spatial and temporal distance, a decay factor and a long-range
 * factor) as a CSR block list, the same for every (batch, head).  Width at
 * frame distance dt: r0 * gamma^dt (dt successive fp64 multiplications);
 * radius floor(width) while the width is >= 1; a frame whose width is below 1 is
 * skipped unless lambda >= 1 divides dt, which keeps the co-located block; the
 * own frame always keeps radius max(floor(r0), 0).  Key block j is kept for
 * query block i iff max(|dy|, |dx|) in tiles is within the radius of |dt|.
 *
 *   row_ptr, col_idx, col_capacity, workspace: as in sparse_attn_mask_to_csr.
 * nB <= 4096 (SPARSE_ATTN_UNSUPPORTED otherwise).
 */
int32_t sparse_attn_radial_csr(const sparse_attn_shape *shape, const sparse_attn_radial_params *params,
                               int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                               void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Backward of sparse_attn_forward (bf16 or fp32, nB <= 4096; SPARSE_ATTN_UNSUPPORTED
 * otherwise):
 * the gradients for training (NABLA summary page, "Methodologie : NABLA" and its
 * training results).  With P the forward's softmax weights (recovered from lse)
 * and dO the upstream gradient:
 *   dV = P^T dO,  dS = P o (dO V^T - rowsum(dO o O)),  dQ = scale dS K,
 *   dK = scale dS^T Q.
 *
 *   q, k, v, out  device, [B, H, N, d] in shape->dtype: the forward's inputs and output.
 *   lse         device fp32 [B, H, N]: the forward's log-sum-exp (required).
 *   dout        device, [B, H, N, d] in shape->dtype: dL/dout.
 *   row_ptr, col_idx, col_count: the block list the forward used (same rules).
 *   dq, dk, dv  device, [B, H, N, d] in shape->dtype, fully written (zeros where no tile
 *               reaches a row, and at the padding slots of partial tiles, which
 *               take no part in any other token's gradient).
 *   t_idx       device int32 [col_count], caller-owned scratch: receives the
 *               transposed block list (for each key block, the query blocks
 *               that keep it, ascending).
 *   workspace   as in sparse_attn_forward.
 * The result is deterministic (no atomics; fixed summation order).  bf16 rounds P
 * and dS to bf16 for its MFMA products; fp32 keeps them fp32 (fp32 MFMA), with one
 * workgroup per block and no splitting of long rows.
 */
int32_t sparse_attn_backward(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                             const void *out, const float *lse, const void *dout, const int32_t *row_ptr,
                             const int32_t *col_idx, int64_t col_count, void *dq, void *dk, void *dv,
                             int32_t *t_idx, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The dense block list: every query block keeps every key block (row r holds
 * 0 .. nB-1 at col_idx[r * nB ...]).  For dense warm-up steps or layers in a
 * denoising loop, where the selection is skipped or its block list is reused
 * for several steps (the pages' schedules that keep the first steps or blocks
 * dense and amortise the selection over later steps).
 *   row_ptr, col_idx, col_capacity: as in sparse_attn_select.
 */
int32_t sparse_attn_full_csr(const sparse_attn_shape *shape, int32_t *row_ptr, int32_t *col_idx,
                             int64_t col_capacity, void *stream);

/*
 * Token reordering between raster order and the tile-major order the calls above
 * take (the "Fractal Flattening" item of the NABLA summary page, section
 * "Methodologie : NABLA": the tokens of each spatial patch are made contiguous;
 * with 64-token tiles this is one level of tiling).
 *
 *   src, dst    device, [B, H, N, d] in shape->dtype; distinct, not overlapping.
 *   raster      token (t, y, x) at index (t * grid_h + y) * grid_w + x.
 *   tile-major  block b = (bt * nTy + by) * nTx + bx holds tokens [64 b, 64 b + 64):
 *               the tile_t x tile_h x tile_w tile at (bt, by, bx), row-major inside.
 * sparse_attn_to_tiles: raster [B, H, grid_t*grid_h*grid_w, d] -> tile-major
 * [B, H, 64 nB, d], padding slots of partial tiles written as zeros;
 * sparse_attn_from_tiles: the inverse (padding slots dropped).
 */
int32_t sparse_attn_to_tiles(const sparse_attn_shape *shape, const void *src, void *dst, void *stream);
int32_t sparse_attn_from_tiles(const sparse_attn_shape *shape, const void *src, void *dst, void *stream);

/*
 * sparse_attn_select on raster-order inputs, with the reorder fused into the
 * pooling: Q and K are copied to tile-major order exactly as sparse_attn_to_tiles
 * does, and each tile's mean (the "Sous-echantillonnage" step of the NABLA summary
 * page, section "Methodologie : NABLA") is formed by that copy, so the selection
 * reads Q and K once in all.  The block list equals the one sparse_attn_select
 * gives on the tile-major copies, up to fp32 summation order in the means (which
 * moves only blocks whose cumulative mass lies at the threshold).
 *
 *   q, k          device, [B, H, grid_t*grid_h*grid_w, d] in shape->dtype, raster order.
 *   q_tiles, k_tiles  device, [B, H, 64 nB, d], written: the tile-major copies, ready for
 *               sparse_attn_forward.  Four distinct, non-overlapping buffers.
 *   params, row_ptr, col_idx, col_capacity, workspace: as in sparse_attn_select.
 * Errors as in sparse_attn_select and sparse_attn_to_tiles.
 */
int32_t sparse_attn_select_raster(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                  const void *q, const void *k, void *q_tiles, void *k_tiles,
                                  int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                                  void *workspace, int64_t workspace_bytes, void *stream);

/*
 * sparse_attn_select without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It computes exactly what sparse_attn_select computes, with the same
 * kernels; their scratch (per-head thresholds, key block means, look-back words,
 * ticket, and the exact fp64 key means with their norms) lives in a static device
 * array of SPARSE_ATTN_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends.  The call allocates
 * and frees nothing.
 *
 *   Arguments as in sparse_attn_select, minus the workspace.  The current device's
 *   array is used, so `stream` must belong to the current device.
 *   Returns SPARSE_ATTN_SCRATCH when the shape needs more scratch than the array
 *   holds (sparse_attn_select_noalloc_bytes > SPARSE_ATTN_SCRATCH_BYTES; the
 *   workloads of up to 12 heads x 3,840 blocks or 40 heads x 1,260 blocks at
 *   d = 128 fit), and otherwise the statuses of sparse_attn_select.
 *   All calls on one GPU share its array, which keeps the last call's contents:
 *   calls that overlap on one GPU (different streams or threads without ordering
 *   between them) race and must not be issued.  sparse_attn_select_check does not
 *   apply (it reads a workspace).
 */
int32_t sparse_attn_select_noalloc(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                   const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                                   int64_t col_capacity, void *stream);

/* Bytes of the static scratch sparse_attn_select_noalloc needs for this shape, or a
   negative status for an invalid shape. */
int64_t sparse_attn_select_noalloc_bytes(const sparse_attn_shape *shape);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
