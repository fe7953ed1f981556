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
                                                   int64_t nblocks) {
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

// ---------------------------------------------------------------------------
// Selection.  A workgroup (4 waves) owns R consecutive query blocks of one
// (batch, head).  Phase 1 computes the R x nB pooled scores with fp32 MFMA
// (v_mfma_f32_16x16x4_f32; each wave sweeps every fourth 16-column tile) and
// parks them in LDS, pre-multiplied by scale*log2(e).  Phase 2 gives each
// wave whole rows: softmax in place, then an exact mass-weighted radix
// select over the fp32 bit patterns of the probabilities (positive floats
// order like their bit patterns) finds the crossing value v* and the mass M
// strictly above it; a block is kept when its probability is above v*, or
// equal to v* and M plus the mass of the equal blocks with lower index is
// below thr.  That is the CDF rule with ties going to the lower index.
template <int D>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
    extern __shared__ float smem[];
    float *scores = smem;                                 // [R][nBp]
    float *hist_all = smem + (size_t)a.R * a.nBp;         // [4][256]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
        for (int ct = wave; ct < ntiles; ct += 4) {
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
                for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[m][s], bk[m][s], acc, 0, 0, 0);
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

    // ---- phase 2: per-row softmax, CDF cut, window, bitmask ----------------
    float *hist = hist_all + wave * 256;
    const int ne = a.nBp / 64;
    const int h = (int)(bh % a.H);
    const float thr = a.thr[h];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r = wave; r < nrows; r += 4) {
        const int i = i0 + r;
        const int64_t row = bh * a.nB + i;
        float *sr = scores + (size_t)r * a.nBp;

        float mx = -INFINITY;
        for (int e = 0; e < ne; ++e) {
            const int j = lane + 64 * e;
            if (j < a.nB) mx = fmaxf(mx, sr[j]);
        }
        mx = wave_max(mx);
        float z = 0.f;
        for (int e = 0; e < ne; ++e) {
            const int j = lane + 64 * e;
            if (j < a.nB) {
                const float pe = exp2f(sr[j] - mx);
                sr[j] = pe;
                z += pe;
            }
        }
        z = wave_sum(z);
        const float rz = 1.f / z;
        for (int e = 0; e < ne; ++e) {
            const int j = lane + 64 * e;
            if (j < a.nB) sr[j] *= rz;
        }

        uint32_t vstar = 0;
        float M = 0.f;
        const bool keep_all = !(thr < 1.f);
        if (!keep_all) {
            uint32_t prefix = 0;
#pragma unroll 1
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                reinterpret_cast<f32x4 *>(hist)[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
                wave_lds_sync();
                for (int e = 0; e < ne; ++e) {
                    const int j = lane + 64 * e;
                    if (j < a.nB) {
                        const float pe = sr[j];
                        const uint32_t u = __float_as_uint(pe);
                        const bool match = pass == 0 || (u >> (shift + 8)) == prefix;
                        if (match) atomicAdd(&hist[(u >> shift) & 255u], pe);
                    }
                }
                wave_lds_sync();
                const f32x4 hv = reinterpret_cast<const f32x4 *>(hist)[lane];   // buckets 4l .. 4l+3
                const float T = (hv[0] + hv[1]) + (hv[2] + hv[3]);
                // inclusive suffix sum over lanes (higher lanes hold higher buckets)
                float S = T;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const float t = __shfl_down(S, o, 64);
                    if (lane + o < 64) S += t;
                }
                float X = __shfl_down(S, 1, 64);      // mass of the buckets above this lane
                if (lane == 63) X = 0.f;
                const float above = M + X;
                // lowest lane whose upper neighbours stay below thr holds the crossing bucket
                const uint64_t bal = __ballot(above < thr);
                const int L = __builtin_ctzll(bal);   // bal is never 0: lane 63 has above == M < thr
                const float c3 = above + hv[3];
                const float c2 = c3 + hv[2];
                const float c1 = c2 + hv[1];
                int sub;
                float mnew;
                if (c3 >= thr) { sub = 3; mnew = above; }
                else if (c2 >= thr) { sub = 2; mnew = c3; }
                else if (c1 >= thr) { sub = 1; mnew = c2; }
                else { sub = 0; mnew = c1; }
                sub = __shfl(sub, L, 64);
                mnew = __shfl(mnew, L, 64);
                prefix = (prefix << 8) | (uint32_t)(4 * L + sub);
                M = mnew;
                wave_lds_sync();
            }
            vstar = prefix;
        }

        // ---- emit: kept = above v*, or tie within thr, or in the window
        const int nTyx = a.nTy * a.nTx;
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
                    kept = M + (float)rank * vstar_f < thr;
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
        if (lane == 0) a.counts[row] = count;
    }
}

// ---------------------------------------------------------------------------
int launch_pool(const void *q, const void *k, float *qbar, float *kbar, int64_t nblocks, int dtype, int d,
                hipStream_t s) {
    const int64_t waves = 2 * nblocks;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (dtype == 1 && d == 128)
        pool_kernel<__bf16, 128><<<grid, block, 0, s>>>((const __bf16 *)q, (const __bf16 *)k, qbar, kbar, nblocks);
    else if (dtype == 1 && d == 64)
        pool_kernel<__bf16, 64><<<grid, block, 0, s>>>((const __bf16 *)q, (const __bf16 *)k, qbar, kbar, nblocks);
    else if (dtype == 0 && d == 128)
        pool_kernel<float, 128><<<grid, block, 0, s>>>((const float *)q, (const float *)k, qbar, kbar, nblocks);
    else
        pool_kernel<float, 64><<<grid, block, 0, s>>>((const float *)q, (const float *)k, qbar, kbar, nblocks);
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

int launch_select(const SelectArgs &a, int d, hipStream_t s) {
    const size_t lds = ((size_t)a.R * a.nBp + 4 * 256) * sizeof(float);
    const dim3 grid((unsigned)a.n_groups), block(256);
    if (d == 128)
        select_kernel<128><<<grid, block, lds, s>>>(a);
    else
        select_kernel<64><<<grid, block, lds, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
