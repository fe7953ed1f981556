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
// lanes that share a column slice are combined with xor-shuffles.  The fp32
// mean x is stored as a pair of bf16 values, hi = bf16(x) and lo = bf16(x - hi)
// (row layout [hi: D][lo: D]), the operand form of the split-bf16 score products.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                   __bf16 *__restrict__ qbar, __bf16 *__restrict__ kbar,
                                                   int64_t nblocks, PoolSide side) {
    // side job for the selection that follows: the first ThrChunk::kMax thresholds
    if (blockIdx.x == 0 && (int)threadIdx.x < side.n_thr) side.thr_dst[threadIdx.x] = side.thr.v[threadIdx.x];
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
    __bf16 *dst = (w & 1) ? kbar : qbar;
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
        typedef __attribute__((ext_vector_type(VEC))) float fv;
        typedef __attribute__((ext_vector_type(VEC))) __bf16 bv;
        fv x;
#pragma unroll
        for (int c = 0; c < VEC; ++c) x[c] = acc[c] * (1.f / 64.f);
        const bv hi = __builtin_convertvector(x, bv);
        fv r;
#pragma unroll
        for (int c = 0; c < VEC; ++c) r[c] = x[c] - (float)hi[c];
        const bv lo = __builtin_convertvector(r, bv);
        __bf16 *o = dst + blk * (2 * D) + col;
        *reinterpret_cast<bv *>(o) = hi;
        *reinterpret_cast<bv *>(o + D) = lo;
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
// Selection.  A workgroup of 16 waves owns 16 consecutive query blocks (rows) of
// one (batch, head); wave w ends up holding row w in registers, key block
// j = 64c + lane in s[c].
//
// Scores ("Attention Reduite"): S = Qbar Kbar^T * scale * log2(e), in chunks of
// 256 key blocks.  Per chunk each wave forms a 16 x 16 tile (the 16 rows x its 16
// keys) with v_mfma_f32_16x16x32_bf16 on the split operands, hi*hi + hi*lo + lo*hi
// (relative error near 2^-16, fp32 accumulation), and parks it in a double-buffered
// LDS stage; after one barrier every wave reads its own row's 256 scores back.
//
// Cut ("Seuil CDF"), per wave on its register row: e_j = 2^(s_j - max) and their sum
// Z; then an exact mass-weighted radix select over the fp32 bit patterns of the e_j
// (positive floats order like their bit patterns) finds the crossing value v* and
// the mass M strictly above it; the digits start at the highest bit where the row's
// e_j differ, 8 bits per pass, with the pass histogram in LDS.  A block is kept when
// e_j > v*, or e_j == v* and M plus the mass of the equal blocks with lower index is
// below thr * Z: the CDF rule with ties going to the lower index, without
// normalising the row.  Then the optional box window ("Integration Hybride avec
// STA"), the row's bitmask, its count and the count of its 64-row chunk.
constexpr int kSelRows = kGroupRows;    // rows (and waves) per workgroup
constexpr int kSelChunk = 256;          // key blocks per score chunk (16 waves x 16)
constexpr int kStageStride = kSelChunk + 4;   // padded: the 16x16 tile stores are conflict-free

template <int D> constexpr int qf_stride() { return 2 * D + 8; }   // bf16; 16 B pad per row
template <int D> constexpr size_t select_lds_bytes() {
    return (size_t)kSelRows * qf_stride<D>() * 2 + (size_t)2 * kSelRows * kStageStride * 4 +
           (size_t)kSelRows * 256 * 4;
}

// The cut of row i of head bh (threshold thr), run by one wave on its register row s
// (scaled scores, -inf for padding keys); writes the row's bitmask and count, and
// its count to `out`.
template <int NE>
__device__ __forceinline__ void select_cut(const SelectArgs &a, float (&s)[NE], float *hist_all, int64_t bh, int i,
                                           float thr, int lane, int32_t &out) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = bh * a.nB + i;
    const int nvc = a.nBp >> 6;
    const bool keep_all = !(thr < 1.f);
    uint32_t *list = reinterpret_cast<uint32_t *>(hist_all + wave * 256);   // up to 64 keys of the bracket

    // e_j = 2^(s_j - max) in place (0 for padding), Z, the smallest positive key and
    // how many keys are positive
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < NE; ++c) mx = fmaxf(mx, s[c]);
    mx = wave_max_u(mx);
    float z = 0.f;
    uint32_t kmin = 0xffffffffu, npos = 0;
#pragma unroll
    for (int c = 0; c < NE; ++c) {
        const float pe = __builtin_amdgcn_exp2f(s[c] - mx);
        s[c] = pe;
        z += pe;
        kmin = min(kmin, __float_as_uint(pe) - 1u);         // padding (0) wraps to the top
        npos += (uint32_t)__popcll(__ballot(pe > 0.f));
    }
    const float Z = wave_sum_u(z);
    const float thrz = thr * Z;

    // Crossing value v* and the mass M strictly above it.  Keys are the fp32 bit
    // patterns of the e_j (order-preserving for e >= 0).  The key bracket (lo, hi]
    // keeps  Mhi = mass(key > hi) < thr*Z <= Mlo = mass(key > lo);  each step splits it
    // at a pivot and costs one compare/select/add per element plus a wave sum; the
    // compare masks' popcounts track how many elements the bracket holds.  Pivots
    // alternate between regula falsi on the values (the mass above a value is linear
    // in the value when the e_j are spread evenly in log scale) and halving the key
    // range, which bounds the steps.  Once at most 64 elements remain they are
    // compacted to LDS, sorted across the lanes, and the crossing is read off their
    // prefix sums.
    uint32_t vstar = 0x3f800000u;
    float M = 0.f;
    if (!keep_all) {
        uint32_t lo = wave_min_u32(kmin), hi = 0x3f800000u;   // every e_j <= 1, the row max is exactly 1
        float Mhi = 0.f, Mlo = Z;
        uint32_t clo = npos, chi = 0;                         // counts of key > lo, key > hi
#pragma unroll 1
        for (int step = 0; clo - chi > 64 && hi - lo > 1; ++step) {
            uint32_t p;
            if (step < 2 || (step & 1) == 0) {
                const float vlo = __uint_as_float(lo), vhi = __uint_as_float(hi);
                const float f = (thrz - Mhi) / (Mlo - Mhi);
                p = __float_as_uint(vhi - f * (vhi - vlo));
                p = min(max(p, lo + 1u), hi - 1u);
            } else {
                p = lo + ((hi - lo) >> 1);
            }
            float acc = 0.f;
            uint32_t cnt = 0;
#pragma unroll
            for (int c = 0; c < NE; ++c) {
                const bool gt = __float_as_uint(s[c]) > p;
                acc += gt ? s[c] : 0.f;
                cnt += (uint32_t)__popcll(__ballot(gt));
            }
            const float A = wave_sum_u(acc);
            if (A < thrz) {
                hi = p;
                Mhi = A;
                chi = cnt;
            } else {
                lo = p;
                Mlo = A;
                clo = cnt;
            }
        }
        vstar = hi;       // a single key left in the bracket: v* = hi, M = Mhi
        M = Mhi;
        if (clo - chi <= 64 && clo > chi) {
            uint32_t base = 0;
#pragma unroll
            for (int c = 0; c < NE; ++c) {
                const uint32_t u = __float_as_uint(s[c]);
                const bool in = u > lo && u <= hi;
                const uint64_t m = __ballot(in);
                if (in)
                    list[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = u;
                base += (uint32_t)__popcll(m);
            }
            wave_lds_sync();
            const uint32_t n = clo - chi;
            uint32_t u = (uint32_t)lane < n ? list[lane] : 0u;
            wave_lds_sync();
            // bitonic sort of the bracket's keys, descending across the lanes
#pragma unroll
            for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
                for (int j = k >> 1; j > 0; j >>= 1) {
                    const uint32_t o = (uint32_t)__shfl_xor((int)u, j, 64);
                    const bool desc = (lane & k) == 0 || k == 64;
                    const bool low = (lane & j) == 0;
                    u = (low == desc) ? max(u, o) : min(u, o);
                }
            }
            const float e = __uint_as_float(u);
            const float incl = wave_prefix_sum(e, lane);
            const uint64_t reach = __ballot((uint32_t)lane < n && Mhi + incl >= thrz);
            const int L = reach ? __builtin_ctzll(reach) : (int)n - 1;   // rounding may leave thr*Z unreached
            vstar = (uint32_t)__builtin_amdgcn_readlane((int)u, L);
            M = Mhi + wave_sum_u(u > vstar ? e : 0.f);
        }
    }

    // ---- kept = key above v*, or equal to v* with M + (its rank among the equal
    //      keys, by index) * v* below thr*Z, or inside the window
    const int nTyx = a.nTy * a.nTx;
    const int ti = i / nTyx, yi = (i / a.nTx) % a.nTy, xi = i % a.nTx;
    const float vstar_f = __uint_as_float(vstar);
    uint32_t ties_before = 0, count = 0, wlo = 0, whi = 0;
#pragma unroll
    for (int c = 0; c < NE; ++c) {
        const int j = 64 * c + lane;
        uint64_t m;
        if (keep_all) {
            m = __ballot(j < a.nB);
        } else {
            const uint32_t u = __float_as_uint(s[c]);
            m = __ballot(u > vstar);
            const uint64_t tb = __ballot(u == vstar);      // padding (0) never equals v* > 0
            if (tb) {
                const uint32_t rank =
                    ties_before + __builtin_amdgcn_mbcnt_hi((uint32_t)(tb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)tb, 0u));
                m |= __ballot(u == vstar && M + (float)rank * vstar_f < thrz);
                ties_before += (uint32_t)__popcll(tb);
            }
        }
        if (a.window) {
            const int tj = j / nTyx, yj = (j / a.nTx) % a.nTy, xj = j % a.nTx;
            m |= __ballot(j < a.nB && abs(tj - ti) <= a.wt && abs(yj - yi) <= a.wh && abs(xj - xi) <= a.ww);
        }
        count += (uint32_t)__popcll(m);
        if (lane == c) {
            wlo = (uint32_t)m;
            whi = (uint32_t)(m >> 32);
        }
    }
    if (lane < nvc) a.bits[row * (int64_t)nvc + lane] = ((uint64_t)whi << 32) | wlo;
    if (lane == 0) {
        a.counts[row] = (int32_t)count;
        out = (int32_t)count;
    }
}

// NE = 4 * ceil(nB / 256): the register row length in 64-key words (chunks of 256 keys).
template <int D, int NE>
__global__ __launch_bounds__(1024) void select_kernel(SelectArgs a) {
    static_assert(NE % 4 == 0 && NE <= 64, "NE: register row length in 64-key words");
    constexpr int KB = D / 32;                     // k-blocks of one 16x16x32 product
    constexpr int NCH = NE / 4;                    // score chunks
    // registers for the next chunk's operands where they fit; at NE <= 8 two
    // workgroups share a CU instead
    constexpr bool kPrefetch = NE > 8 && NE <= 32;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __bf16 *qf = reinterpret_cast<__bf16 *>(smem_raw);                              // [16][2D+8]
    float *stage = reinterpret_cast<float *>(smem_raw + (size_t)kSelRows * qf_stride<D>() * 2);  // [2][16][260]
    float *hist_all = stage + 2 * kSelRows * kStageStride;                          // [16][256]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t g = (uint32_t)xcd_remap(blockIdx.x, a.n_groups);
    const uint32_t bh = g / (uint32_t)a.groups_per_head;
    const int i0 = (int)(g - bh * (uint32_t)a.groups_per_head) * kSelRows;
    const int nrows = min(kSelRows, a.nB - i0);
    const __bf16 *qs = a.qbar + ((int64_t)bh * a.nB + i0) * (2 * D);
    const __bf16 *ks = a.kbar + ((int64_t)bh * a.nB) * (2 * D);
    const float thr = a.thr[bh % (uint32_t)a.H];

    // ---- the group's pooled queries (hi | lo) and chunk 0's keys, loads issued together
    constexpr int PER_ROW = 2 * D / 4;             // 8-byte pieces per query row
    const int qr = threadIdx.x / PER_ROW, qc = threadIdx.x % PER_ROW;
    uint2 qv = {0u, 0u};
    if (qr < nrows) qv = reinterpret_cast<const uint2 *>(qs + (int64_t)qr * 2 * D)[qc];

    const int ii = lane & 15, kq = lane >> 4;
    float s[NE];
    bf16x8 kh[2][KB], kl[2][KB];
    // keys past nB read row 0 (in bounds); their scores land on padding columns
    auto load_k = [&](int cc, int slot) {
        const int jj = kSelChunk * cc + 16 * wave + ii;
        const __bf16 *kr = ks + (int64_t)(jj < a.nB ? jj : 0) * (2 * D) + 8 * kq;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            kh[slot][kb] = *reinterpret_cast<const bf16x8 *>(kr + 32 * kb);
            kl[slot][kb] = *reinterpret_cast<const bf16x8 *>(kr + D + 32 * kb);
        }
    };
    load_k(0, 0);
    if (qr < kSelRows) reinterpret_cast<uint2 *>(qf + qr * qf_stride<D>())[qc] = qv;
    __syncthreads();

    // ---- scores, chunk by chunk, into the register row
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
        const int cur = kPrefetch ? (cc & 1) : 0;
        if (kPrefetch && cc + 1 < NCH) load_k(cc + 1, cur ^ 1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const __bf16 *qrow = qf + ii * qf_stride<D>() + 8 * kq;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 qh = *reinterpret_cast<const bf16x8 *>(qrow + 32 * kb);
            const bf16x8 ql = *reinterpret_cast<const bf16x8 *>(qrow + D + 32 * kb);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kh[cur][kb], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kl[cur][kb], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kh[cur][kb], acc, 0, 0, 0);
        }
        if (!kPrefetch && cc + 1 < NCH) load_k(cc + 1, 0);
        // acc[e] = S[row 4*kq + e][key 256*cc + 16*wave + ii]
        float *st = stage + (cc & 1) * kSelRows * kStageStride;
#pragma unroll
        for (int e = 0; e < 4; ++e) st[(4 * kq + e) * kStageStride + 16 * wave + ii] = acc[e] * a.scale_log2;
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float v = st[wave * kStageStride + 64 * t + lane];
            s[4 * cc + t] = kSelChunk * cc + 64 * t + lane < a.nB ? v : -INFINITY;   // padding keys
        }
    }
    __shared__ int32_t wave_count[kSelRows];
    if (wave < nrows) select_cut<NE>(a, s, hist_all, bh, i0 + wave, thr, lane, wave_count[wave]);
    else if (lane == 0) wave_count[wave] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t t = 0;
#pragma unroll
        for (int w = 0; w < kSelRows; ++w) t += wave_count[w];
        a.group_sums[g] = t;
    }
}

// ---------------------------------------------------------------------------
int launch_pool(const void *q, const void *k, __bf16 *qbar, __bf16 *kbar, int64_t nblocks, int dtype, int d,
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

template <int D, int NCH> static void launch_select_nch(const SelectArgs &a, int nch, hipStream_t s) {
    if constexpr (NCH <= kSelectMaxBlocks / kSelChunk) {
        if (nch == NCH) {
            select_kernel<D, 4 * NCH><<<dim3((unsigned)a.n_groups), dim3(64 * kSelRows), select_lds_bytes<D>(), s>>>(a);
            return;
        }
        launch_select_nch<D, NCH + 1>(a, nch, s);
    }
}

int launch_select(const SelectArgs &a, int d, hipStream_t s) {
    if (a.nBp > kSelectMaxBlocks) return -1;
    const int nch = (a.nB + kSelChunk - 1) / kSelChunk;
    if (d == 128)
        launch_select_nch<128, 1>(a, nch, s);
    else
        launch_select_nch<64, 1>(a, nch, s);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
