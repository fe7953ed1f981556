// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sattn {

struct ThrChunk {
    static constexpr int kMax = 256;
    float v[kMax];
};

// Rows per chunk of the kept-count prefix (emit workgroup size in rows).
constexpr int kEmitRowsLog2 = 6;
constexpr int kEmitRows = 1 << kEmitRowsLog2;

// Side jobs done by the pooling kernel for the selection that follows.
struct PoolSide {
    ThrChunk thr;             // first thresholds, by value
    float *thr_dst;           // [H] (workspace)
    int32_t n_thr;            // thresholds in `thr` (<= ThrChunk::kMax)
    int32_t *chunk_sums;      // [n_chunks] kept blocks per chunk of kEmitRows rows, cleared here
    int64_t n_chunks;
};

struct SelectArgs {
    const float *qbar;        // [BH][nB][D] fp32 block means
    const float *kbar;
    const float *thr;         // [H] thresholds (device)
    uint64_t *bits;           // [BH*nB][nBp/64] kept-block bitmask
    int32_t *counts;          // [BH*nB] kept blocks per row
    int32_t *chunk_sums;      // [ceil(BH*nB / kEmitRows)] kept blocks per chunk of rows
    int64_t n_groups;         // workgroups = BH * groups_per_head
    int32_t groups_per_head;  // ceil(nB / R)
    int32_t H, nB, nBp, R;    // heads, blocks, nB rounded up to 64, rows per workgroup
    int32_t nTy, nTx;         // block grid (t is implied)
    int32_t window, wt, wh, ww;
    float scale_log2;         // softmax scale * log2(e)
};

struct AttnArgs {
    const void *q, *k, *v;
    const int32_t *row_ptr, *col_idx;
    int64_t col_count;
    void *out;
    float *lse;               // nullable
    int64_t rows;             // B*H*nB
    int64_t n_pairs;          // B*H*pairs_per_head (query-block pairs of the bf16 kernel)
    int32_t pairs_per_head;   // ceil(nB / 2)
    int32_t nB;
    float scale_log2;         // softmax scale * log2(e)
};

int launch_pool(const void *q, const void *k, float *qbar, float *kbar, int64_t nblocks, int dtype, int d,
                const PoolSide &side, hipStream_t s);
int launch_fill_thresholds(const float *host_thr, int n, float *dst, hipStream_t s);
int launch_select(const SelectArgs &a, int d, hipStream_t s);
// Large block counts: scores through HBM (a.n_groups = rows, one row per wave).
int launch_select_big(const SelectArgs &a, int d, float *scores, hipStream_t s);
int launch_mask_bits(const uint8_t *mask, int64_t rows, int32_t nB, int32_t nW, uint64_t *bits,
                     int32_t *counts, int32_t *chunk_sums, hipStream_t s);
int launch_clear(int32_t *p, int64_t n, hipStream_t s);
int launch_emit(const uint64_t *bits, const int32_t *counts, const int32_t *chunk_sums, int64_t rows, int32_t nW,
                int32_t *row_ptr, int32_t *col_idx, hipStream_t s);
int launch_attention(const AttnArgs &a, int dtype, int d, hipStream_t s);

}  // namespace sattn
