// CSR construction from per-row kept-block bitmasks (gfx950).
//
// The block mask is turned into the list of 64x64 tiles to compute (the
// "Expansion" item of the NABLA summary page, section "Methodologie :
// NABLA") without materialising a token mask: row_ptr is the exclusive scan
// of the per-row counts and col_idx lists each row's kept key blocks in
// ascending order.
#include "common.h"
#include "kernels.h"

namespace sattn {

// External dense uint8 mask [rows][nB] -> bitmask rows + counts.  Workgroup G owns row
// group G (16 waves, one row each) and writes the group's total.
__global__ __launch_bounds__(1024) void mask_bits_kernel(const uint8_t *__restrict__ mask, int32_t nB, int32_t nW,
                                                         int32_t groups_per_head, uint64_t *__restrict__ bits,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ group_sums) {
    __shared__ int32_t wave_count[kGroupRows];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t G = blockIdx.x;
    const int64_t bh = G / groups_per_head;
    const int i = (int)(G % groups_per_head) * kGroupRows + wave;
    int count = 0;
    if (i < nB) {
        const int64_t row = bh * nB + i;
        const uint8_t *m = mask + row * (int64_t)nB;
        for (int e = 0; e < nW; ++e) {
            const int j = 64 * e + lane;
            const uint64_t b = __ballot(j < nB && m[j] != 0);
            count += __popcll(b);
            if (lane == 0) bits[row * nW + e] = b;
        }
        if (lane == 0) counts[row] = count;
    }
    if (lane == 0) wave_count[wave] = count;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t t = 0;
#pragma unroll
        for (int w = 0; w < kGroupRows; ++w) t += wave_count[w];
        group_sums[G] = t;
    }
}

// DynamicRad's radial window (DynamicRad page, section "Methodologie : DynamicRad",
// items A and B) as row bitmasks + counts, in the layout of mask_bits_kernel.  The
// width of frame distance dt is r0 * gamma^dt, formed by dt successive fp64
// multiplications; radius floor(width) while the width is at least 1; a frame below
// that is skipped unless lambda >= 1 divides dt, which keeps its co-located block;
// the own frame keeps radius max(floor(r0), 0).  Key block j is kept iff the
// Chebyshev distance in tiles is within the radius of |t_i - t_j|.
__global__ __launch_bounds__(1024) void radial_bits_kernel(RadialArgs a, int32_t nB, int32_t nW,
                                                           int32_t groups_per_head, uint64_t *__restrict__ bits,
                                                           int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ group_sums) {
    __shared__ int32_t wave_count[kGroupRows];
    __shared__ int32_t radius[kSelectMaxBlocks];      // per frame distance (frames <= blocks)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int dt = threadIdx.x; dt < a.nT; dt += blockDim.x) {
        double w = (double)a.r0;
        for (int u = 0; u < dt; ++u) w = w * (double)a.gamma;
        int r;
        if (dt == 0) r = w >= 1.0 ? (int)floor(fmin(w, 1e6)) : 0;
        else if (w >= 1.0) r = (int)floor(fmin(w, 1e6));
        else r = (a.lambda >= 1 && dt % a.lambda == 0) ? 0 : -1;
        radius[dt] = r;
    }
    __syncthreads();
    const int64_t G = blockIdx.x;
    const int64_t bh = G / groups_per_head;
    const int i = (int)(G % groups_per_head) * kGroupRows + wave;
    const int nTyx = a.nTy * a.nTx;
    int count = 0;
    if (i < nB) {
        const int64_t row = bh * nB + i;
        const int ti = i / nTyx, yi = (i / a.nTx) % a.nTy, xi = i % a.nTx;
        for (int e = 0; e < nW; ++e) {
            const int j = 64 * e + lane;
            bool keep = false;
            if (j < nB) {
                const int tj = j / nTyx, yj = (j / a.nTx) % a.nTy, xj = j % a.nTx;
                const int ds = max(abs(yj - yi), abs(xj - xi));
                keep = ds <= radius[abs(tj - ti)];
            }
            const uint64_t b = __ballot(keep);
            count += __popcll(b);
            if (lane == 0) bits[row * nW + e] = b;
        }
        if (lane == 0) counts[row] = count;
    }
    if (lane == 0) wave_count[wave] = count;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t t = 0;
#pragma unroll
        for (int w = 0; w < kGroupRows; ++w) t += wave_count[w];
        group_sums[G] = t;
    }
}

// Prefix and compaction in one pass, one wave per row; workgroup b owns rows
// 4b .. 4b+3.  The offset of a row is the sum of the totals of the row groups before
// its own plus the counts of the rows of its group before it: the workgroup sums the
// totals before the group of its first row once, each wave adds what lies between
// that and its row, writes row_ptr and expands its row's bitmask into ascending
// col_idx.
__global__ __launch_bounds__(256) void emit_kernel(const uint64_t *__restrict__ bits,
                                                   const int32_t *__restrict__ counts,
                                                   const int32_t *__restrict__ group_sums, int64_t rows, int32_t nB,
                                                   int32_t nW, int32_t *__restrict__ row_ptr,
                                                   int32_t *__restrict__ col_idx) {
    __shared__ int32_t part[4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t gph = (nB + kGroupRows - 1) / kGroupRows;
    auto group_of = [&](int64_t r) { return (r / nB) * gph + (r % nB) / kGroupRows; };
    const int64_t r0 = (int64_t)blockIdx.x * 4;
    const int64_t G0 = group_of(r0);
    int32_t s = 0;
    for (int64_t g = t; g < G0; g += 256) s += group_sums[g];
    const int32_t ws = wave_sum_i(s);
    if (lane == 0) part[wave] = ws;
    __syncthreads();
    const int64_t row = r0 + wave;
    if (row >= rows) return;
    const int64_t G = group_of(row);
    const int64_t first = (row / nB) * nB + ((row % nB) / kGroupRows) * kGroupRows;   // first row of G
    int32_t mine = 0;
    if (lane < G - G0) mine += group_sums[G0 + lane];          // at most 3 groups lie between
    if (lane < row - first) mine += counts[first + lane];      // at most 15 rows
    int32_t pos = part[0] + part[1] + part[2] + part[3] + wave_sum_i(mine);
    if (lane == 0) {
        row_ptr[row] = pos;
        if (row == rows - 1) row_ptr[rows] = pos + counts[row];
    }
    // per word, the lanes whose bit is set (the word as the execution mask) store their
    // column at the running offset plus the set bits below them
    const uint64_t *b = bits + row * nW;
    int32_t *const dst = col_idx + __builtin_amdgcn_readfirstlane(pos);
    uint32_t off = 0;
    for (int w0 = 0; w0 < nW; w0 += 64) {
        const uint64_t mine_w = (w0 + lane < nW) ? b[w0 + lane] : 0ull;
        const int nw = min(64, nW - w0);
        for (int e = 0; e < nw; ++e) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine_w, e);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine_w >> 32), e);
            const uint64_t m = ((uint64_t)hi << 32) | lo;
            if (__builtin_amdgcn_inverse_ballot_w64(m))
                dst[__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, off))] = (w0 + e) * 64 + lane;
            off += (uint32_t)__popcll(m);
        }
    }
}

// Every row keeps every key block: row_ptr[r] = r * nB, col_idx = 0 .. nB-1 per row.
__global__ void full_csr_kernel(int64_t rows, int32_t nB, int32_t *__restrict__ row_ptr,
                                int32_t *__restrict__ col_idx) {
    const int64_t n = rows * nB;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        col_idx[i] = (int32_t)(i % nB);
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r <= rows; r += (int64_t)gridDim.x * blockDim.x)
        row_ptr[r] = (int32_t)(r * nB);
}

int launch_full_csr(int64_t rows, int32_t nB, int32_t *row_ptr, int32_t *col_idx, hipStream_t s) {
    const int64_t n = rows * nB;
    int64_t blocks = (n + 255) / 256;
    blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
    full_csr_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(rows, nB, row_ptr, col_idx);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mask_bits(const uint8_t *mask, int64_t bh, int32_t nB, int32_t nW, uint64_t *bits, int32_t *counts,
                     int32_t *group_sums, hipStream_t s) {
    const int32_t gph = (nB + kGroupRows - 1) / kGroupRows;
    mask_bits_kernel<<<dim3((unsigned)(bh * gph)), dim3(64 * kGroupRows), 0, s>>>(mask, nB, nW, gph, bits, counts,
                                                                                 group_sums);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_radial_bits(const RadialArgs &a, int64_t bh, int32_t nB, int32_t nW, uint64_t *bits, int32_t *counts,
                       int32_t *group_sums, hipStream_t s) {
    const int32_t gph = (nB + kGroupRows - 1) / kGroupRows;
    radial_bits_kernel<<<dim3((unsigned)(bh * gph)), dim3(64 * kGroupRows), 0, s>>>(a, nB, nW, gph, bits, counts,
                                                                                   group_sums);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_emit(const uint64_t *bits, const int32_t *counts, const int32_t *group_sums, int64_t rows, int32_t nB,
                int32_t nW, int32_t *row_ptr, int32_t *col_idx, hipStream_t s) {
    emit_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(bits, counts, group_sums, rows, nB, nW, row_ptr,
                                                                       col_idx);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
