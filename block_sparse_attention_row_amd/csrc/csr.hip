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

// External dense uint8 mask [rows][nB] -> bitmask rows + counts; one wave per row.
__global__ __launch_bounds__(256) void mask_bits_kernel(const uint8_t *__restrict__ mask, int64_t rows, int32_t nB,
                                                        int32_t nW, uint64_t *__restrict__ bits,
                                                        int32_t *__restrict__ counts, int32_t *__restrict__ chunk_sums) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint8_t *m = mask + row * (int64_t)nB;
    int count = 0;
    for (int e = 0; e < nW; ++e) {
        const int j = 64 * e + lane;
        const bool k = j < nB && m[j] != 0;
        const uint64_t b = __ballot(k);
        count += __popcll(b);
        if (lane == 0) bits[row * nW + e] = b;
    }
    if (lane == 0) {
        counts[row] = count;
        atomicAdd(chunk_sums + (row >> kEmitRowsLog2), count);
    }
}

__global__ void clear_kernel(int32_t *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// Prefix and compaction in one pass, one wave per row.  Workgroup b owns rows
// 4b .. 4b+3.  The offset of row 4b is the sum of the per-chunk kept counts of the
// 64-row chunks before its chunk (the selection accumulated those) plus the counts
// of the rows of its own chunk before it; each wave adds the counts of the rows
// of the workgroup before its own, writes row_ptr and expands its row's bitmask
// into ascending col_idx.
template <int CTRL> __device__ __forceinline__ int dppi(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int s) {
    s += dppi<0xB1>(s);
    s += dppi<0x4E>(s);
    s += dppi<0x141>(s);
    s += dppi<0x140>(s);
    return __builtin_amdgcn_readlane(s, 0) + __builtin_amdgcn_readlane(s, 16) + __builtin_amdgcn_readlane(s, 32) +
           __builtin_amdgcn_readlane(s, 48);
}

__global__ __launch_bounds__(256) void emit_kernel(const uint64_t *__restrict__ bits,
                                                   const int32_t *__restrict__ counts,
                                                   const int32_t *__restrict__ chunk_sums, int64_t rows, int32_t nW,
                                                   int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx) {
    __shared__ int32_t part[4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * 4;
    const int64_t c = r0 >> kEmitRowsLog2;
    const int64_t c0 = c << kEmitRowsLog2;
    int32_t s = 0;
    for (int64_t i = t; i < c; i += 256) s += chunk_sums[i];
    if (t < r0 - c0) s += counts[c0 + t];
    const int32_t ws = wave_sum_i(s);
    if (lane == 0) part[wave] = ws;
    __syncthreads();
    const int64_t row = r0 + wave;
    if (row >= rows) return;
    int32_t pos = part[0] + part[1] + part[2] + part[3];
    for (int w = 0; w < wave; ++w) pos += counts[r0 + w];
    if (lane == 0) {
        row_ptr[row] = pos;
        if (row == rows - 1) row_ptr[rows] = pos + counts[row];
    }
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t *b = bits + row * nW;
    for (int w0 = 0; w0 < nW; w0 += 64) {
        const uint64_t mine = (w0 + lane < nW) ? b[w0 + lane] : 0ull;
        const int cnt = __popcll(mine);
        int incl = cnt;
        incl += dppi<0x111>(incl);
        incl += dppi<0x112>(incl);
        incl += dppi<0x114>(incl);
        incl += dppi<0x118>(incl);
        {
            const int q0 = __builtin_amdgcn_readlane(incl, 15), q1 = __builtin_amdgcn_readlane(incl, 31),
                      q2 = __builtin_amdgcn_readlane(incl, 47);
            const int row16 = lane >> 4;
            incl += (row16 >= 1 ? q0 : 0) + (row16 >= 2 ? q1 : 0) + (row16 >= 3 ? q2 : 0);
        }
        const int excl = incl - cnt;
        const int nw = min(64, nW - w0);
        for (int e = 0; e < nw; ++e) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, e);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), e);
            const uint64_t m = ((uint64_t)hi << 32) | lo;
            const int off = __builtin_amdgcn_readlane(excl, e);
            if ((m >> lane) & 1ull) col_idx[pos + off + __popcll(m & lt_mask)] = (w0 + e) * 64 + lane;
        }
        pos += __builtin_amdgcn_readlane(incl, 63);
    }
}

int launch_mask_bits(const uint8_t *mask, int64_t rows, int32_t nB, int32_t nW, uint64_t *bits, int32_t *counts,
                     int32_t *chunk_sums, hipStream_t s) {
    mask_bits_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(mask, rows, nB, nW, bits, counts,
                                                                            chunk_sums);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_clear(int32_t *p, int64_t n, hipStream_t s) {
    const int64_t blocks = (n + 255) / 256;
    clear_kernel<<<dim3((unsigned)(blocks < 1024 ? (blocks > 0 ? blocks : 1) : 1024)), dim3(256), 0, s>>>(p, n);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_emit(const uint64_t *bits, const int32_t *counts, const int32_t *chunk_sums, int64_t rows, int32_t nW,
                int32_t *row_ptr, int32_t *col_idx, hipStream_t s) {
    emit_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(bits, counts, chunk_sums, rows, nW, row_ptr,
                                                                       col_idx);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
