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
                                                        int32_t *__restrict__ counts) {
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
    if (lane == 0) counts[row] = count;
}

// row_ptr[r] = sum of counts[0 .. r), row_ptr[rows] = total.  One workgroup:
// each thread sums a contiguous chunk, the chunk sums are scanned in LDS,
// then each thread writes its chunk.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t *__restrict__ counts, int64_t rows,
                                                    int32_t *__restrict__ row_ptr) {
    __shared__ int32_t wave_tot[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t per = (rows + 1023) / 1024;
    const int64_t beg = min(rows, (int64_t)t * per), end = min(rows, beg + per);
    int32_t s = 0;
    for (int64_t i = beg; i < end; ++i) s += counts[i];
    int32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t carry = 0;
    for (int w = 0; w < wave; ++w) carry += wave_tot[w];
    int32_t run = carry + incl - s;
    for (int64_t i = beg; i < end; ++i) {
        row_ptr[i] = run;
        run += counts[i];
    }
    if (t == 1023) row_ptr[rows] = run;
}

// Bitmask rows -> col_idx (ascending within a row); one wave per row.
__global__ __launch_bounds__(256) void emit_kernel(const uint64_t *__restrict__ bits,
                                                   const int32_t *__restrict__ row_ptr, int64_t rows, int32_t nW,
                                                   int32_t *__restrict__ col_idx) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint64_t *b = bits + row * nW;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t base = row_ptr[row];
    for (int w0 = 0; w0 < nW; w0 += 64) {
        const uint64_t mine = (w0 + lane < nW) ? b[w0 + lane] : 0ull;
        const int cnt = __popcll(mine);
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        const int excl = incl - cnt;
        const int nw = min(64, nW - w0);
        for (int e = 0; e < nw; ++e) {
            const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)mine, e, 64);
            const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(mine >> 32), e, 64);
            const uint64_t m = ((uint64_t)hi << 32) | lo;
            const int off = __shfl(excl, e, 64);
            if ((m >> lane) & 1ull) col_idx[base + off + __popcll(m & lt_mask)] = (w0 + e) * 64 + lane;
        }
        base += __shfl(incl, 63, 64);
    }
}

int launch_mask_bits(const uint8_t *mask, int64_t rows, int32_t nB, int32_t nW, uint64_t *bits, int32_t *counts,
                     hipStream_t s) {
    mask_bits_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(mask, rows, nB, nW, bits, counts);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_scan(const int32_t *counts, int64_t rows, int32_t *row_ptr, hipStream_t s) {
    scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(counts, rows, row_ptr);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_emit(const uint64_t *bits, const int32_t *row_ptr, int64_t rows, int32_t nW, int32_t *col_idx,
                hipStream_t s) {
    emit_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(bits, row_ptr, rows, nW, col_idx);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
