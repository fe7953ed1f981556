// Block pooling and dynamic block selection (gfx950).
//
// Follows the NABLA summary page ("NABLA: Neighborhood Adaptive Block-Level
// Attention", section "Methodologie : NABLA"):
//   pool_kernel   -- "Sous-echantillonnage": mean of each 64-token block of Q and K;
//   select_kernel -- "Attention Reduite": softmax over the pooled scores of a
//                    row; "Seuil CDF": keep blocks in descending probability
//                    while the mass before them is below thr; "Integration
//                    Hybride avec STA": OR with a static box window.
// The selection result of a row is a bitmask over key blocks plus its
// popcount; csr.hip turns those into row_ptr / col_idx.
#include "common.h"
#include "kernels.h"

namespace sattn {

// ---------------------------------------------------------------------------
// Pooling.  One wave per (tensor, block): the block is 64*D contiguous
// elements; each lane streams 16-byte chunks, accumulates in fp32, and the
// lanes that share a column slice are combined with xor-shuffles.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                   float *__restrict__ qbar, float *__restrict__ kbar,
                                                   int64_t nblocks, PoolSide side) {
    // side jobs for the selection that follows: the first ThrChunk::kMax thresholds and
    // clearing the per-chunk kept counts
    if (blockIdx.x == 0 && (int)threadIdx.x < side.n_thr) side.thr_dst[threadIdx.x] = side.thr.v[threadIdx.x];
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < side.n_chunks;
         c += (int64_t)gridDim.x * blockDim.x)
        side.chunk_sums[c] = 0;
    constexpr int VEC = 16 / sizeof(T);
    constexpr int LPR = D / VEC;               // lanes covering one token row
    constexpr int RPW = kWave / LPR;           // token rows per wave-wide load
    constexpr int ITER = kTokensPerBlock / RPW;
    constexpr int BATCH = ITER < 16 ? ITER : 16;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
    if (w >= 2 * nblocks) return;
    const int64_t blk = w >> 1;
    const T *src = (w & 1) ? k : q;
    float *dst = (w & 1) ? kbar : qbar;
    const int col = (lane % LPR) * VEC, row0 = lane / LPR;
    const u32x4 *p = reinterpret_cast<const u32x4 *>(src + (blk * kTokensPerBlock + row0) * D + col);
    constexpr int STEP = RPW * D * (int)sizeof(T) / 16;   // u32x4 units between iterations

    float acc[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = 0.f;
#pragma unroll
    for (int b0 = 0; b0 < ITER; b0 += BATCH) {
        u32x4 buf[BATCH];
#pragma unroll
        for (int it = 0; it < BATCH; ++it) buf[it] = p[(b0 + it) * STEP];
#pragma unroll
        for (int it = 0; it < BATCH; ++it) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if constexpr (sizeof(T) == 2) {
                    acc[2 * c] += bf16_lo(buf[it][c]);
                    acc[2 * c + 1] += bf16_hi(buf[it][c]);
                } else {
                    acc[c] += __uint_as_float(buf[it][c]);
                }
            }
        }
    }
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] += __shfl_xor(acc[c], o, 64);
    }
    if (lane < LPR) {
        f32x4 *o = reinterpret_cast<f32x4 *>(dst + blk * D + col);
#pragma unroll
        for (int c = 0; c < VEC / 4; ++c) {
            f32x4 v;
            v[0] = acc[4 * c] * (1.f / 64.f);
            v[1] = acc[4 * c + 1] * (1.f / 64.f);
            v[2] = acc[4 * c + 2] * (1.f / 64.f);
            v[3] = acc[4 * c + 3] * (1.f / 64.f);
            o[c] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Thresholds are copied to the workspace by value (no host memcpy).
__global__ void fill_thresholds_kernel(ThrChunk c, float *__restrict__ dst, int n) {
    const int i = threadIdx.x;
    if (i < n) dst[i] = c.v[i];
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Phase 2 for one row, run by one wave: sr holds the row's nB scores (already
// multiplied by scale*log2(e)) in LDS and is overwritten with e_j; writes the row's
// kept-block bitmask, its count, and adds the count to its chunk.
__device__ __forceinline__ void select_row(const SelectArgs &a, float *sr, float *hist, int64_t bh, int i) {
    const int lane = threadIdx.x & 63;
    const int64_t row = bh * a.nB + i;
    const int ne = a.nBp / 64;
    const int h = (int)(bh % a.H);
    const float thr = a.thr[h];
    const bool keep_all = !(thr < 1.f);
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nTyx = a.nTy * a.nTx;

    float mx = -INFINITY;
    for (int e = 0; e < ne; ++e) {
        const int j = lane + 64 * e;
        if (j < a.nB) mx = fmaxf(mx, sr[j]);
    }
    mx = wave_max_u(mx);
    float z = 0.f;
    for (int e = 0; e < ne; ++e) {
        const int j = lane + 64 * e;
        if (j < a.nB) {
            const float pe = __builtin_amdgcn_exp2f(sr[j] - mx);
            sr[j] = pe;
            z += pe;
        }
    }
    const float thrz = thr * wave_sum_u(z);

    // Radix digits start at the highest bit where the row's keys differ (the bits
    // above it are common to all keys), so the first histogram spreads over the
    // row's actual range instead of piling onto one exponent bucket.
    uint32_t vstar = 0;
    float M = 0.f;
    if (!keep_all) {
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        for (int e = 0; e < ne; ++e) {
            const int j = lane + 64 * e;
            if (j < a.nB) {
                const uint32_t u = __float_as_uint(sr[j]);
                kmin = min(kmin, u);
                kmax = max(kmax, u);
            }
        }
        kmin = wave_min_u32(kmin);
        kmax = wave_max_u32_u(kmax);
        const uint32_t diff = kmin ^ kmax;
        uint32_t prefix = kmax;            // all keys equal: v* is that key, M = 0
        if (diff) {
            int hi = 31 - __builtin_clz(diff);                 // highest differing bit
            prefix = hi == 31 ? 0u : kmax >> (hi + 1);          // the common upper bits
#pragma unroll 1
            while (hi >= 0) {
                const int lo = hi >= 7 ? hi - 7 : 0, w = hi - lo + 1;
                const uint32_t dmask = (1u << w) - 1u;
                reinterpret_cast<f32x4 *>(hist)[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
                wave_lds_sync();
                for (int e = 0; e < ne; ++e) {
                    const int j = lane + 64 * e;
                    if (j < a.nB) {
                        const float pe = sr[j];
                        const uint32_t u = __float_as_uint(pe);
                        const bool match = hi == 31 || (u >> (hi + 1)) == prefix;
                        if (match) atomicAdd(&hist[(u >> lo) & dmask], pe);
                    }
                }
                wave_lds_sync();
                // lane l takes buckets 4(63-l)+3 .. 4(63-l): lane order is descending bucket order
                const f32x4 hv = reinterpret_cast<const f32x4 *>(hist)[63 - lane];
                const float T = (hv[0] + hv[1]) + (hv[2] + hv[3]);
                const float above = M + (wave_prefix_sum(T, lane) - T);   // mass of the higher buckets
                // the last lane whose higher buckets stay below thr*Z holds the crossing bucket
                const uint64_t bal = __ballot(above < thrz);
                const int L = 63 - __builtin_clzll(bal);   // lane 0 always qualifies: above == M < thr*Z
                const float c3 = above + hv[3];
                const float c2 = c3 + hv[2];
                const float c1 = c2 + hv[1];
                int sub;
                float mnew;
                if (c3 >= thrz) { sub = 3; mnew = above; }
                else if (c2 >= thrz) { sub = 2; mnew = c3; }
                else if (c1 >= thrz) { sub = 1; mnew = c2; }
                else { sub = 0; mnew = c1; }
                sub = __builtin_amdgcn_readlane(sub, L);
                mnew = lane_value(mnew, L);
                prefix = (prefix << w) | (uint32_t)(4 * (63 - L) + sub);
                M = mnew;
                wave_lds_sync();
                hi = lo - 1;
            }
        }
        vstar = prefix;
    }

    // ---- emit: kept = above v*, or tie within thr*Z, or in the window
    const int ti = i / nTyx, yi = (i / a.nTx) % a.nTy, xi = i % a.nTx;
    const float vstar_f = __uint_as_float(vstar);
    int ties_before = 0;
    int count = 0;
    uint64_t *brow = a.bits + row * (int64_t)ne;
    for (int e = 0; e < ne; ++e) {
        const int j = lane + 64 * e;
        const bool valid = j < a.nB;
        bool kept = valid && keep_all;
        if (!keep_all) {
            const uint32_t u = valid ? __float_as_uint(sr[j]) : 0u;
            const bool tie = valid && u == vstar;
            const uint64_t tb = __ballot(tie);
            kept = valid && u > vstar;
            if (tie) {
                const int rank = ties_before + __popcll(tb & lt_mask);
                kept = M + (float)rank * vstar_f < thrz;
            }
            ties_before += __popcll(tb);
        }
        if (a.window && valid) {
            const int tj = j / nTyx, yj = (j / a.nTx) % a.nTy, xj = j % a.nTx;
            if (abs(tj - ti) <= a.wt && abs(yj - yi) <= a.wh && abs(xj - xi) <= a.ww) kept = true;
        }
        const uint64_t m = __ballot(kept);
        count += __popcll(m);
        if (lane == 0) brow[e] = m;
    }
    if (lane == 0) {
        a.counts[row] = count;
        atomicAdd(a.chunk_sums + (row >> kEmitRowsLog2), count);   // integer adds: order does not matter
    }
}

// ---------------------------------------------------------------------------
// Selection.  A workgroup (8 waves) owns R <= 16 consecutive query blocks of one
// (batch, head).  Phase 1 computes the R x nB pooled scores with fp32 MFMA
// (v_mfma_f32_16x16x4_f32; each wave sweeps every eighth 16-column tile) and parks
// them in LDS, pre-multiplied by scale*log2(e).  Phase 2 gives each wave whole rows:
// e_j = 2^(s_j - max) in place and their sum Z; then an exact mass-weighted radix
// select over the fp32 bit patterns of the e_j (positive floats order like their
// bit patterns) finds the crossing value v* and the mass M strictly above it, in
// four 8-bit passes whose histograms live in LDS.  A block is kept when e_j > v*,
// or e_j == v* and M plus the mass of the equal blocks with lower index is below
// thr * Z.  That is the CDF rule with ties going to the lower index, without
// normalising the row.  Wave-wide sums and scans use DPP and v_readlane.
template <int D>
__global__ __launch_bounds__(512) void select_kernel(SelectArgs a) {
    extern __shared__ float smem[];
    float *scores = smem;                                 // [R][nBp]
    float *hist_all = smem + (size_t)a.R * a.nBp;         // [8][256]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t g = xcd_remap(blockIdx.x, a.n_groups);
    const int64_t bh = g / a.groups_per_head;
    const int i0 = (int)(g % a.groups_per_head) * a.R;
    const int nrows = min(a.R, a.nB - i0);
    const float *qb = a.qbar + (bh * a.nB) * (int64_t)D;
    const float *kb = a.kbar + (bh * a.nB) * (int64_t)D;

    // ---- phase 1: scores -------------------------------------------------
    {
        const int ii = lane & 15, gq = lane >> 4;
        f32x4 aq[D / 16];
        const bool qok = ii < nrows;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
            aq[m] = qok ? *reinterpret_cast<const f32x4 *>(qb + (int64_t)(i0 + ii) * D + 16 * m + 4 * gq)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int ntiles = a.nBp / 16;
        for (int ct = wave; ct < ntiles; ct += 8) {
            const int jj = 16 * ct + ii;
            const bool kok = jj < a.nB;
            f32x4 bk[D / 16];
#pragma unroll
            for (int m = 0; m < D / 16; ++m) {
                bk[m] = kok ? *reinterpret_cast<const f32x4 *>(kb + (int64_t)jj * D + 16 * m + 4 * gq)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < D / 16; ++m) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[m][s4], bk[m][s4], acc, 0, 0, 0);
            }
            // acc[e] = S[row 4*gq + e][col 16*ct + ii]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * gq + e;
                if (r < a.R) scores[(size_t)r * a.nBp + jj] = acc[e] * a.scale_log2;
            }
        }
    }
    __syncthreads();

    // ---- phase 2: per-row softmax mass, CDF cut, window, bitmask -----------
    float *hist = hist_all + wave * 256;
    for (int r = wave; r < nrows; r += 8) select_row(a, scores + (size_t)r * a.nBp, hist, bh, i0 + r);
}

// ---------------------------------------------------------------------------
// Large block counts: the R x nB score rows no longer fit LDS in useful numbers, so
// the scores take a trip through HBM.  score_gemm_kernel forms S = (Qbar Kbar^T) *
// scale * log2(e) for a whole head in 64 x 64 tiles per wave, each fp32 operand
// split into a bf16 high part and a bf16 remainder, with the three products
// hi*hi + hi*lo + lo*hi on v_mfma_f32_32x32x16_bf16 (relative error near 2^-16 per
// product, fp32 accumulation); select_scores_kernel then copies one score row per
// wave into LDS and runs the same per-row cut.
__device__ __forceinline__ void split_bf16x8(const f32x4 &x0, const f32x4 &x1, bf16x8 &hi, bf16x8 &lo) {
    f32x8 v = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    hi = __builtin_convertvector(v, bf16x8);
    f32x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = v[e] - (float)hi[e];
    lo = __builtin_convertvector(r, bf16x8);
}

template <int D>
__global__ __launch_bounds__(256) void score_gemm_kernel(const float *__restrict__ qbar, const float *__restrict__ kbar,
                                                         float *__restrict__ S, int32_t nB, int32_t tiles,
                                                         int64_t n_wtiles, float scale_log2) {
    const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
    const int64_t wt = xcd_remap((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), n_wtiles);
    if (wt >= n_wtiles) return;
    const int64_t per_head = (int64_t)tiles * tiles;
    const int64_t bh = wt / per_head;
    const int ti = (int)((wt % per_head) / tiles), tj = (int)(wt % tiles);
    const float *qb = qbar + bh * nB * (int64_t)D;
    const float *kb = kbar + bh * nB * (int64_t)D;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
    int ri[2], cj[2];
    bool rok[2], cok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        ri[u] = 64 * ti + 32 * u + l32;
        cj[u] = 64 * tj + 32 * u + l32;
        rok[u] = ri[u] < nB;
        cok[u] = cj[u] < nB;
    }
#pragma unroll 2
    for (int c = 0; c < D / 16; ++c) {
        bf16x8 ahi[2], alo[2], bhi[2], blo[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const float *qa = qb + (int64_t)ri[u] * D + 16 * c + 8 * h;
            const float *kk = kb + (int64_t)cj[u] * D + 16 * c + 8 * h;
            const f32x4 a0 = rok[u] ? *reinterpret_cast<const f32x4 *>(qa) : z;
            const f32x4 a1 = rok[u] ? *reinterpret_cast<const f32x4 *>(qa + 4) : z;
            const f32x4 b0 = cok[u] ? *reinterpret_cast<const f32x4 *>(kk) : z;
            const f32x4 b1 = cok[u] ? *reinterpret_cast<const f32x4 *>(kk + 4) : z;
            split_bf16x8(a0, a1, ahi[u], alo[u]);
            split_bf16x8(b0, b1, bhi[u], blo[u]);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[a], bhi[b], acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[a], blo[b], acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[a], bhi[b], acc[a][b], 0, 0, 0);
            }
    }
    // acc[a][b][v] = S[row 64 ti + 32 a + 8 (v/4) + 4 h + v%4][col 64 tj + 32 b + l32]
    float *Sh = S + bh * nB * (int64_t)nB;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (!cok[b]) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 64 * ti + 32 * a + 8 * (v >> 2) + 4 * h + (v & 3);
                if (r < nB) Sh[(int64_t)r * nB + cj[b]] = acc[a][b][v] * scale_log2;
            }
        }
}

__global__ __launch_bounds__(256) void select_scores_kernel(SelectArgs a, const float *__restrict__ S) {
    extern __shared__ float smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t rows = a.n_groups;                 // one row per wave here
    const int64_t row = xcd_remap((int64_t)blockIdx.x * (blockDim.x >> 6) + wave, rows);
    if (row >= rows) return;
    float *sr = smem + (size_t)wave * (a.nBp + 256);
    float *hist = sr + a.nBp;
    const float *src = S + row * (int64_t)a.nB;
    for (int j = lane; j < a.nB; j += 64) sr[j] = src[j];
    wave_lds_sync();
    select_row(a, sr, hist, row / a.nB, (int)(row % a.nB));
}

// ---------------------------------------------------------------------------
int launch_pool(const void *q, const void *k, float *qbar, float *kbar, int64_t nblocks, int dtype, int d,
                const PoolSide &side, hipStream_t s) {
    const int64_t waves = 2 * nblocks;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (dtype == 1 && d == 128)
        pool_kernel<__bf16, 128><<<grid, block, 0, s>>>((const __bf16 *)q, (const __bf16 *)k, qbar, kbar, nblocks, side);
    else if (dtype == 1 && d == 64)
        pool_kernel<__bf16, 64><<<grid, block, 0, s>>>((const __bf16 *)q, (const __bf16 *)k, qbar, kbar, nblocks, side);
    else if (dtype == 0 && d == 128)
        pool_kernel<float, 128><<<grid, block, 0, s>>>((const float *)q, (const float *)k, qbar, kbar, nblocks, side);
    else
        pool_kernel<float, 64><<<grid, block, 0, s>>>((const float *)q, (const float *)k, qbar, kbar, nblocks, side);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fill_thresholds(const float *host_thr, int n, float *dst, hipStream_t s) {
    for (int off = 0; off < n; off += ThrChunk::kMax) {
        ThrChunk c;
        const int m = n - off < ThrChunk::kMax ? n - off : ThrChunk::kMax;
        for (int i = 0; i < m; ++i) c.v[i] = host_thr[off + i];
        fill_thresholds_kernel<<<1, ThrChunk::kMax, 0, s>>>(c, dst + off, m);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

int launch_select_big(const SelectArgs &a, int d, float *scores, hipStream_t s) {
    const int tiles = (a.nB + 63) / 64;
    const int64_t bh = a.n_groups / a.nB;
    const int64_t n_wtiles = bh * tiles * tiles;
    const dim3 g1((unsigned)((n_wtiles + 3) / 4)), b1(256);
    if (d == 128)
        score_gemm_kernel<128><<<g1, b1, 0, s>>>(a.qbar, a.kbar, scores, a.nB, tiles, n_wtiles, a.scale_log2);
    else
        score_gemm_kernel<64><<<g1, b1, 0, s>>>(a.qbar, a.kbar, scores, a.nB, tiles, n_wtiles, a.scale_log2);
    if (hipGetLastError() != hipSuccess) return -1;
    // as many rows (waves) per workgroup as 64 KB of LDS holds, up to 4
    const size_t per_wave = (size_t)(a.nBp + 256) * sizeof(float);
    int wpg = (int)(65536 / per_wave);
    wpg = wpg > 4 ? 4 : (wpg < 1 ? 1 : wpg);
    select_scores_kernel<<<dim3((unsigned)((a.n_groups + wpg - 1) / wpg)), dim3(64 * wpg), wpg * per_wave, s>>>(a,
                                                                                                          scores);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_select(const SelectArgs &a, int d, hipStream_t s) {
    const size_t lds = ((size_t)a.R * a.nBp + 8 * 256) * sizeof(float);
    const dim3 grid((unsigned)a.n_groups), block(512);
    if (d == 128)
        select_kernel<128><<<grid, block, lds, s>>>(a);
    else
        select_kernel<64><<<grid, block, lds, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
