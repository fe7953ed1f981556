// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sattn {

// Geometry of the tile-major slots.  Blocks are the ceil(grid / tile) tiles of the
// token grid, frame-block outermost; slot u of a block is (u / (th tw), (u / tw) % th,
// u % tw) inside its tile, and it holds a grid token iff those coordinates fall inside
// the grid.  Only the last tile along an axis can be partial; when no tile is
// (`partial` == 0) every slot is a token.
struct SlotGeo {
    int32_t nTy, nTx;         // tiles along y and x
    int32_t tt, th, tw;       // tile
    int32_t gt, gh, gw;       // token grid
    int32_t partial;          // some tile is cut by the grid edge
};
// Whether slot u of block b holds a grid token.
__host__ __device__ inline bool slot_valid(const SlotGeo &g, int32_t b, int32_t u) {
    const int32_t bt = b / (g.nTy * g.nTx), by = (b / g.nTx) % g.nTy, bx = b % g.nTx;
    const int32_t ut = u / (g.th * g.tw), uy = (u / g.tw) % g.th, ux = u % g.tw;
    return bt * g.tt + ut < g.gt && by * g.th + uy < g.gh && bx * g.tw + ux < g.gw;
}

struct ThrChunk {
    static constexpr int kMax = 256;
    float v[kMax];
};

// Row groups: 16 consecutive query blocks of one (batch, head), the unit of the
// selection workgroup; group G of head bh covers rows bh*nB + 16g .. (g = G mod
// ceil(nB/16)).  Each group's kept-block total feeds the CSR prefix.
constexpr int kGroupRows = 16;

// Key block means are stored in the B-operand order of v_mfma_f32_16x16x32_bf16, 16
// key blocks to a group, groups padded per (batch, head): group g of head bh starts at
// element (bh * ceil(nB / 16) + g) * 32 D; inside it, part p (0: hi = bf16(x), 1: lo =
// bf16(x - hi)), k-block kb and lane L = ii + 16 kq hold the 8 elements 32 kb + 8 kq ..
// 32 kb + 8 kq + 7 of key block 16 g + ii, at element p * 16 D + 512 kb + 8 L.  Every
// operand load of a wave is then one contiguous 1 KiB run.
__host__ __device__ constexpr int64_t kbar_group(int64_t bh, int64_t groups_per_head, int64_t g, int D) {
    return (bh * groups_per_head + g) * 32 * D;
}

// Side job done by the pooling kernel for the selection that follows.
struct PoolSide {
    ThrChunk thr;             // first thresholds, by value
    float *thr_dst;           // [H] (workspace)
    int32_t n_thr;            // thresholds in `thr` (<= ThrChunk::kMax)
    uint64_t *status;         // look-back words of the selection that follows, zeroed here
    int64_t n_status;
    uint32_t *ticket;         // its ticket counter ([0]) and look-back fault word ([1]), zeroed here
};

// Look-back word of a row group: 0 until published, then kStatAgg | the group's
// kept-block total, finally kStatPre | the inclusive prefix of the totals up to and
// including the group.  Waits on these words give up after spin_cap polls (kSpinCap
// unless the caller lowers it; they end in microseconds when every earlier group
// runs, which the ticket order ensures).  A group that gives up sets the fault word
// (ticket[1] = 1) and writes -1 as the row_ptr entry of each of its rows, so that the
// block list it leaves fails every validity check instead of looking plausible.
constexpr uint64_t kStatAgg = 1ull << 62, kStatPre = 2ull << 62, kStatFlags = 3ull << 62;
constexpr uint32_t kSpinCap = 1u << 22;

// Longest row the selection holds in registers (64 words of 64 key blocks).
constexpr int kSelectMaxBlocks = 4096;

// Exact rescoring of near-ties at the cut: the scores' error bound is
// kScoreEps * scale * log2(e) * |qbar| * max_j |kbar_j| (split-bf16 products and fp32
// accumulation: 3 * 2^-16 per product plus 384 * 2^-24 of accumulation, below 2^-13);
// the blocks whose probability lies within that bound of the crossing value are
// ordered again by their exact fp64 scores, when there are at most kRefineMax of them.
constexpr float kScoreEps = 0x1p-13f;
constexpr int kRefineMax = 64;

struct SelectArgs {
    const void *q;            // [BH*N][D] queries in the input dtype (tile-major)
    const __bf16 *kbar;       // key block means as bf16 pairs, in fragment order (kbar_group)
    const double *kbar64;     // [BH*nB][D] exact key block means
    const float *knorm;       // [BH*nB] Euclidean norms of the key block means
    SlotGeo geo;              // which slots of the query blocks are tokens
    const __bf16 *qbar;       // null: the selection pools Q itself; else [BH*nB][2][D] query
                              // block means as bf16 pairs (hi, then lo), formed by the reorder
    const double *qbar64;     // with qbar: [BH*nB][D] exact query block means
    const float *thr;         // [H] thresholds (device)
    uint64_t *status;         // [n_groups] look-back words (zeroed by the pooling kernel)
    uint32_t *ticket;         // group ticket counter (zeroed by the pooling kernel)
    uint32_t *fault;          // look-back fault word (ticket + 1, zeroed with it)
    uint32_t spin_cap;        // polls of one look-back before it gives up
    int32_t *row_ptr;         // [rows + 1]
    int32_t *col_idx;         // [nnz]
    int64_t rows;             // BH * nB
    int64_t n_groups;         // workgroups = BH * groups_per_head
    int32_t groups_per_head;  // ceil(nB / 16)
    int32_t H, nB, nBp;       // heads, blocks, nB rounded up to 64
    int32_t nTy, nTx;         // block grid (t is implied)
    int32_t window, wt, wh, ww;
    float scale_log2;         // softmax scale * log2(e)
    // sampling with inclusion probabilities (the SIP selection): expected kept blocks
    // per row, the uniforms' seed, and the offsets written beside col_idx
    float budget;
    uint64_t seed;
    float *col_bias;
    // the clustering selector (IBCS): log2 of the mixture rows of the heads
    // [head0, head0 + heads), one row per query-block pair
    const float *mix_rows;
    int64_t head0;
};
// Selection of 4-token key blocks (nK = 16 nB per head) for each 64-token query
// block: a workgroup of kFineWaves waves takes R query blocks of one head by ticket;
// wave w holds the scores of keys [w S, w S + S) of all R rows (W words of 64 a lane).
constexpr int kFineWaves = 16;
struct FineArgs {
    const __bf16 *q;          // [BH*N][D] queries (bf16, tile-major)
    const __bf16 *k;          // [BH*N][D] keys (bf16, tile-major): the exact rescoring
    const float *kf;          // [BH][D/4][nK][4] fp32 means of the 4-token key blocks
    const float *knorm;       // [BH*nK] their Euclidean norms
    const float *thr;         // [H] thresholds (device)
    uint64_t *status;         // [n_groups] look-back words (zeroed by the pooling kernel)
    uint32_t *ticket;         // group ticket counter (zeroed by the pooling kernel)
    uint32_t *fault;          // look-back fault word (ticket + 1)
    uint32_t spin_cap;
    int32_t *row_ptr;         // [rows + 1]
    int32_t *col_idx;         // [nnz]: key-block indices in [0, nK)
    int64_t rows;             // BH * nB
    int64_t n_groups;         // BH * groups_per_head
    int32_t groups_per_head;  // ceil(nB / R)
    int32_t H, nB, nK, S;     // heads, query blocks, key blocks, keys per wave slice
    float scale_log2;
};
int fine_words(int64_t nK);   // W
int fine_rows(int W);         // R
int launch_fine_pool(const __bf16 *k, float *kf, float *knorm, int64_t nK, int64_t nkeys, int d, const PoolSide &side,
                     hipStream_t s);
int launch_fine_select(const FineArgs &a, int d, hipStream_t s);

constexpr int kIbcsClusters = 8, kIbcsIters = 4;
struct IbcsArgs {
    const void *q;            // [BH*N][D] queries (bf16 or fp32, tile-major)
    const __bf16 *kbar;       // key block means (hi | lo), in fragment order (kbar_group)
    float *rows;              // [heads][pairs][nBp]: log2 of the mixture row of each pair
    int64_t head0;            // first (batch, head) of this launch
    int32_t nB, nBp, pairs_per_head;
    float scale_log2;
};
int launch_ibcs_mix(const IbcsArgs &a, int64_t heads, int d, int dtype, hipStream_t s);

// Row splitting of the bf16 attention.  Pairs of query blocks whose rows hold more
// than L tiles are cut into pieces of at most about L tiles (by position in each
// row); pieces run first, write normalised partial outputs and their log-sum-exp
// to partial slots, and a merge kernel combines them.  L follows the total work
// over the workgroups resident at once, so that no work item outlasts the rest.
// With at least two rounds of pairs, the pairs dispatched last (the last round)
// are cut into kTailPieces pieces as well, which run after every whole pair: the
// launch then ends on short items instead of a part-filled round of whole pairs.
struct SplitItem {
    int32_t pair, slot;          // query-block pair, partial slot
    int32_t a0, a1, ra;          // row A entries [a0, a1); the row's first entry ra
    int32_t b0, b1, rb;          // row B likewise (b0 == b1 when the pair has no row B)
};
constexpr int kResidentPairs = 512;   // attention workgroups resident at once (256 CUs x 2)
constexpr int kMinPiece = 64;         // shortest piece (tiles)
constexpr int kLongSlots = 512;       // partial slots of long-row pieces at most
constexpr int kTailPairs = 384;       // pairs of the last round cut into pieces (3/4 of the resident pairs)
constexpr int kTailPieces = 4;        // pieces per such pair (a pair needs 16 tiles per piece)
constexpr int kMaxSlots = kLongSlots + kTailPairs * kTailPieces;   // partial slots at most
struct SplitPlan {
    SplitItem *items;        // [max_slots] pieces: long-row pieces from 0, last-round pieces from long_slots
    int32_t *counts;         // [0] long-row pieces, [1] split pairs, [2] piece length L, [3] last-round pieces
    int32_t *pair_flag;      // [n_pairs] 0: not split, else first slot + 1
    int32_t *merge;          // [max_slots][3] pair, first slot, pieces (one entry per split pair)
    float *part_o;           // [max_slots][2 blocks][D][64 queries] normalised partial outputs
    float *part_lse;         // [max_slots][2 blocks][64] partial log2-sum-exp (scaled-score units)
    int32_t max_slots;       // partial slots
    int32_t long_slots;      // of which the first long_slots serve long-row pieces
};

// Query-block pairs of the bf16 forward.  Blocks are frame-major (b = t S + s with
// S blocks per frame), and neighbouring frames keep nearly the same key blocks, so
// a pair is two frame-neighbours: pair p < (nT / 2) S of a head is
// (2u S + s, (2u + 1) S + s), u = p / S, s = p mod S; an odd last frame pairs its
// own blocks side by side ((nT - 1) S + 2 s', + 1; the last one alone when S is
// odd).  Either way a head has ceil(nB / 2) pairs.  S = 1 gives (2p, 2p + 1).
__host__ __device__ inline void pair_blocks(int32_t p, int32_t S, int32_t nB, int32_t &blk_a, int32_t &blk_b) {
    const int32_t nT = nB / S, full = (nT / 2) * S;
    if (p < full) {
        const int32_t u = p / S, s = p - u * S;
        blk_a = 2 * u * S + s;
        blk_b = blk_a + S;
    } else {
        const int32_t s2 = p - full;
        blk_a = (nT - 1) * S + 2 * s2;
        blk_b = 2 * s2 + 1 < S ? blk_a + 1 : -1;
    }
}

struct AttnArgs {
    const void *q, *k, *v;
    const int32_t *row_ptr, *col_idx;
    const float *col_bias;    // nullable: logit offset per col_idx entry (bf16 path)
    int64_t col_count;
    void *out;
    float *lse;               // nullable
    int64_t rows;             // B*H*nB
    int64_t n_pairs;          // B*H*pairs_per_head (query-block pairs of the bf16 kernel)
    int32_t pairs_per_head;   // ceil(nB / 2)
    int32_t nB;
    int32_t nK;               // key blocks per head that col_idx may name: nB, or 16 nB for 4-token blocks
    int32_t kpt;              // key blocks per 64-key tile: 1, or 16 (4-token blocks gathered into tiles)
    int32_t pair_stride;      // S of pair_blocks: blocks per frame, or 1
    float scale_log2;         // softmax scale * log2(e)
    SlotGeo geo;              // padding slots of partial tiles: no weight as keys, zero output as queries
    // bf16 path with partial tiles: per-block masks of the slots that are grid tokens,
    // written by the plan kernel (slot_mask_w) and read by the attention (slot_mask);
    // null when every tile is whole
    const uint64_t *slot_mask;
    uint64_t *slot_mask_w;
    SplitPlan plan;           // bf16 path only
};

struct ReorderArgs {
    int32_t nB, nTy, nTx;          // blocks per head, block grid (t implied)
    int32_t tt, th, tw;            // tile
    int32_t gt, gh, gw;            // token grid
    int64_t nr;                    // raster tokens per head, gt * gh * gw (<= 64 nB: partial tiles pad)
    int32_t row_log2;              // log2 of the 16-byte pieces per token row
    int32_t inverse;               // 0: raster -> tile-major, 1: tile-major -> raster
};
int launch_reorder(const void *src, void *dst, const ReorderArgs &a, int64_t tiles, hipStream_t s);
// Raster -> tile-major copies of K and Q plus their block means (keys in fragment
// order, kbar_group with gph groups a head; queries as [hi | lo] rows), and the
// selection's side jobs.  One launch of 2 * tiles workgroups.
struct ReorderPoolArgs {
    ReorderArgs a;
    const void *k_src, *q_src;
    void *k_dst, *q_dst;
    __bf16 *kbar, *qbar;
    double *kbar64, *qbar64;  // [BH*nB][D] exact means
    float *knorm;             // [BH*nB] norms of the key means
    int64_t tiles;            // B * H * nB
    int32_t gph;
    PoolSide side;
};
int launch_reorder_pool(const ReorderPoolArgs &p, int dtype, int d, hipStream_t s);

int launch_pool_keys(const void *k, __bf16 *kbar, double *kbar64, float *knorm, int64_t nblocks, int32_t nB, int dtype,
                     int d, const PoolSide &side, const SlotGeo &geo, hipStream_t s);
int launch_fill_thresholds(const float *host_thr, int n, float *dst, hipStream_t s);
int launch_select(const SelectArgs &a, int d, int dtype, hipStream_t s);
int launch_select_sip(const SelectArgs &a, int d, int dtype, hipStream_t s);
int launch_select_rows(const SelectArgs &a, int64_t groups, hipStream_t s);
int launch_mask_bits(const uint8_t *mask, int64_t bh, int32_t nB, int32_t nW, uint64_t *bits, int32_t *counts,
                     int32_t *group_sums, hipStream_t s);
int launch_full_csr(int64_t rows, int32_t nB, int32_t *row_ptr, int32_t *col_idx, hipStream_t s);
struct RadialArgs {
    int32_t nT, nTy, nTx;     // block grid
    float r0, gamma;          // width at frame distance 0, decay per frame
    int32_t lambda;           // long-range sampling period (0: off)
};
int launch_radial_bits(const RadialArgs &a, int64_t bh, int32_t nB, int32_t nW, uint64_t *bits, int32_t *counts,
                       int32_t *group_sums, hipStream_t s);
int launch_emit(const uint64_t *bits, const int32_t *counts, const int32_t *group_sums, int64_t rows, int32_t nB,
                int32_t nW, int32_t *row_ptr, int32_t *col_idx, hipStream_t s);
// Backward (bf16).
struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *lse2, *dn;       // [B*H*N]: the forward's log-sum-exp in log2 units, dO . O
    const int32_t *ptr, *idx;     // block list walked: CSR (dQ) or its transpose (dV, dK)
    int64_t idx_count;            // entries of idx
    void *grad;                   // the gradient this pass writes, bf16 [B, H, N, d]
    void *grad2;                  // second gradient of the fused dV + dK pass (dK; grad is dV)
    int64_t n_pairs;              // B*H*ceil(nB/2) pairs of blocks
    int32_t pairs_per_head, nB;
    int32_t pair_stride;          // S of pair_blocks (blocks per frame, or 1)
    float scale_log2, scale;
    // pieces of long pairs and of the last round (the forward's plan over the list
    // walked): each piece writes its partial gradient rows, fp32 and scaled, to
    // part[slot][block of the pair][64][d] (and the dK part to part2); a merge adds them
    SplitPlan plan;
    float *part, *part2;
    // partial tiles: per-block masks of the slots that are grid tokens (written by the
    // plan of the first pass), or null when every tile is whole
    const uint64_t *slot_mask;
    SlotGeo geo;                  // the same slots from the grid (fp32 passes)
};
struct BwdLaunch {
    BwdArgs args;                 // fields common to the gradient passes
    SlotGeo geo;                  // partial tiles: which slots are grid tokens
    uint64_t *slot_mask_w;        // workspace [nB] for their masks, or null (whole tiles)
    const void *out;
    const float *lse;
    float *lse2, *dn;             // workspace
    const int32_t *row_ptr, *col_idx;
    int64_t col_count;
    uint64_t *bits;               // workspace [rows][nW]
    int32_t *colcount, *col_ptr;  // workspace [rows], [rows + 1]
    int32_t *t_idx;               // caller's [col_count]: the transposed list
    void *dq, *dk, *dv;
    int64_t rows, BH;
    int32_t nB, nW, d;
    bool f32;                     // fp32 tensors (else bf16)
};
int launch_backward(const BwdLaunch &L, hipStream_t s);

int launch_attention(const AttnArgs &a, int dtype, int d, hipStream_t s);   // bf16: plan, attention, merge
// The work plan of the bf16 forward (long-row and last-round pieces) over the CSR view
// in a (row_ptr, col_idx, col_count, pair fields, plan); also used by the backward.
int launch_plan(const AttnArgs &a, hipStream_t s);

}  // namespace sattn
