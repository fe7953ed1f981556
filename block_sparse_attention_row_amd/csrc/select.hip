// Block pooling, dynamic block selection and the CSR of the kept blocks (gfx950).
//
// Follows the NABLA summary page ("NABLA: Neighborhood Adaptive Block-Level
// Attention", section "Methodologie : NABLA"):
//   pool_kernel        -- "Sous-echantillonnage": mean of each 64-token block of K;
//   select_emit_kernel -- the same mean for the workgroup's own query blocks, then
//                         "Attention Reduite": softmax over the pooled scores of a
//                         row; "Seuil CDF": keep blocks in descending probability
//                         while the mass before them is below thr; "Integration
//                         Hybride avec STA": OR with a static box window; and the
//                         "Expansion" into row_ptr / col_idx, whose offsets come
//                         from a look-back over the groups' totals.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lookback.h"

namespace sattn {

// ---------------------------------------------------------------------------
// Pooling of one 64-token block by one wave: the block is 64*D contiguous elements;
// each lane streams 16-byte chunks (BATCH loads in flight), accumulates in Acc, and
// the lanes that share a column slice are combined with xor-shuffles.  Lanes
// 0 .. LPR-1 end up with the VEC means of columns col .. col+VEC-1.  With Acc =
// double the means are exact (a sum of 64 bf16 values, or of 64 fp32 values of
// moderate spread, is exact in fp64, and the division by 64 is a power of two).
template <typename T, int D, int BATCH> struct BlockPool {
    static constexpr int VEC = 16 / sizeof(T);
    static constexpr int LPR = D / VEC;               // lanes covering one token row
    static constexpr int RPW = kWave / LPR;           // token rows per wave-wide load
    static constexpr int ITER = kTokensPerBlock / RPW;
    static constexpr int B = ITER < BATCH ? ITER : BATCH;
    static __device__ __forceinline__ int col(int lane) { return (lane % LPR) * VEC; }
    // `valid`: bit u set when slot u of the block is a grid token (a partial tile's
    // padding slots are skipped and the mean divides by the token count)
    template <typename Acc>
    static __device__ __forceinline__ void mean(const T *blk, int lane, Acc (&x)[VEC], uint64_t valid = ~0ull) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(blk + (lane / LPR) * D + col(lane));
        constexpr int STEP = RPW * D * (int)sizeof(T) / 16;   // u32x4 units between iterations
        Acc acc[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c] = 0;
#pragma unroll
        for (int b0 = 0; b0 < ITER; b0 += B) {
            u32x4 buf[B];
#pragma unroll
            for (int it = 0; it < B; ++it) buf[it] = p[(b0 + it) * STEP];
            if (valid != ~0ull) {
#pragma unroll
                for (int it = 0; it < B; ++it)
                    if (!((valid >> (lane / LPR + RPW * (b0 + it))) & 1ull)) buf[it] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int it = 0; it < B; ++it) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if constexpr (sizeof(T) == 2) {
                        acc[2 * c] += (Acc)bf16_lo(buf[it][c]);
                        acc[2 * c + 1] += (Acc)bf16_hi(buf[it][c]);
                    } else {
                        acc[c] += (Acc)__uint_as_float(buf[it][c]);
                    }
                }
                // one load's conversions at a time: the fp64 temporaries of all loads
                // at once would not fit the register budget
                if constexpr (sizeof(Acc) == 8) __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] += __shfl_xor(acc[c], o, 64);
        }
        if (valid == ~0ull) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) x[c] = acc[c] * (Acc)(1.0 / 64.0);
        } else {
            const Acc n = (Acc)__popcll(valid);
#pragma unroll
            for (int c = 0; c < VEC; ++c) x[c] = acc[c] / n;
        }
    }
    // the exact means, for the selection's exact rescoring of near-ties
    static __device__ __forceinline__ void store64(const double (&x)[VEC], double *row, int lane) {
#pragma unroll
        for (int c = 0; c < VEC; c += 2)
            *reinterpret_cast<double2 *>(row + col(lane) + c) = double2{x[c], x[c + 1]};
    }
    static __device__ __forceinline__ void to_f32(const double (&x)[VEC], float (&y)[VEC]) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) y[c] = (float)x[c];
    }
    // the fp32 means as bf16 pairs, hi = bf16(x) and lo = bf16(x - hi): the operand
    // form of the split-bf16 score products ([hi: D][lo: D] per block)
    static __device__ __forceinline__ void store_split(const float (&x)[VEC], __bf16 *row, int lane) {
        typedef __attribute__((ext_vector_type(VEC))) float fv;
        typedef __attribute__((ext_vector_type(VEC))) __bf16 bv;
        fv xv, r;
#pragma unroll
        for (int c = 0; c < VEC; ++c) xv[c] = x[c];
        const bv hi = __builtin_convertvector(xv, bv);
#pragma unroll
        for (int c = 0; c < VEC; ++c) r[c] = xv[c] - (float)hi[c];
        const bv lo = __builtin_convertvector(r, bv);
        *reinterpret_cast<bv *>(row + col(lane)) = hi;
        *reinterpret_cast<bv *>(row + D + col(lane)) = lo;
    }
    // the same pair in the key means' fragment order (kbar_group): lane's columns
    // col .. col+VEC-1 share one k-block kb and one 8-column slice kq
    static __device__ __forceinline__ void store_frag(const float (&x)[VEC], __bf16 *group, int ii, int lane) {
        typedef __attribute__((ext_vector_type(VEC))) float fv;
        typedef __attribute__((ext_vector_type(VEC))) __bf16 bv;
        fv xv, r;
#pragma unroll
        for (int c = 0; c < VEC; ++c) xv[c] = x[c];
        const bv hi = __builtin_convertvector(xv, bv);
#pragma unroll
        for (int c = 0; c < VEC; ++c) r[c] = xv[c] - (float)hi[c];
        const bv lo = __builtin_convertvector(r, bv);
        const int d0 = col(lane), kb = d0 / 32, kq = (d0 % 32) / 8;
        __bf16 *at = group + 512 * kb + 8 * (ii + 16 * kq) + d0 % 8;
        *reinterpret_cast<bv *>(at) = hi;
        *reinterpret_cast<bv *>(at + 16 * D) = lo;
    }
};

// Key block means, one wave per block, stored in fragment order (kbar_group).  Side jobs for the selection that follows:
// the first ThrChunk::kMax thresholds, and zeroing its ticket and look-back words.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ k, __bf16 *__restrict__ kbar,
                                                   double *__restrict__ kbar64, float *__restrict__ knorm,
                                                   int64_t nblocks, int32_t nB, PoolSide side, SlotGeo geo) {
    const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blockIdx.x == 0 && (int)threadIdx.x < side.n_thr) side.thr_dst[threadIdx.x] = side.thr.v[threadIdx.x];
    for (int64_t i = gt; i < side.n_status; i += (int64_t)gridDim.x * blockDim.x) side.status[i] = 0;
    if (gt == 0) {
        side.ticket[0] = 0u;
        side.ticket[1] = 0u;
    }
    using P = BlockPool<T, D, 16>;
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const int64_t bh = blk / nB;
    const int j = (int)(blk - bh * nB);
    const uint64_t valid = geo.partial ? __ballot(slot_valid(geo, j, lane)) : ~0ull;
    double x64[P::VEC];
    float x[P::VEC];
    P::mean(k + blk * kTokensPerBlock * D, lane, x64, valid);
    P::to_f32(x64, x);
    // the mean's Euclidean norm (for the scores' error bound)
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < P::VEC; ++c) ss += lane < P::LPR ? x[c] * x[c] : 0.f;
    ss = wave_sum_u(ss);
    if (lane < P::LPR) {
        P::store_frag(x, kbar + kbar_group(bh, (nB + 15) / 16, j / 16, D), j % 16, lane);
        P::store64(x64, kbar64 + blk * D, lane);
    }
    if (lane == 0) knorm[blk] = sqrtf(ss);
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
// Z; a pivot search over the fp32 bit patterns of the e_j (positive floats order
// like their bit patterns) narrows the crossing value v* and the mass M strictly
// above it, and the last <= 64 candidates are sorted across the lanes.  A block is
// kept when e_j > v*, or e_j == v* and M plus the mass of the equal blocks with
// lower index is below thr * Z: the CDF rule with ties going to the lower index,
// without normalising the row.  Then the optional box window ("Integration Hybride
// avec STA"), the row's bitmask and its count.
constexpr int kSelRows = kGroupRows;    // rows (and waves) per workgroup
constexpr int kSelChunk = 256;          // key blocks per score chunk (16 waves x 16)
constexpr int kStageStride = kSelChunk + 4;   // padded: the 16x16 tile stores are conflict-free

template <int D> constexpr int qf_stride() { return 2 * D + 8; }   // bf16; 16 B pad per row
template <int D> constexpr size_t select_lds_bytes() {
    return (size_t)kSelRows * qf_stride<D>() * 2 + (size_t)2 * kSelRows * kStageStride * 4 +
           (size_t)kSelRows * 256 * 4 + (size_t)kSelRows * D * 8;
}

// Exact order of the near-ties at the cut.  The band is the set of blocks whose
// probability lies within the scores' error bound of the crossing value: `list` holds
// its nb block indices in ascending order, `cdf` (word c in lane c) the blocks the cut
// keeps, m of them in the band, with 2 <= nb <= kRefineMax and 0 < m < nb (otherwise
// nothing is ambiguous).  The band's blocks
// are scored again in fp64 from the exact means (qrow: this row's query mean in LDS;
// k64: the head's key means) and the m best of them by exact score (ties to the lower
// index) replace the cut's choice among them.  Every block outside the band is
// ordered correctly against every block inside it, so this is the cut of the exact
// scores wherever the kept count m is itself settled (it can change only when the
// threshold lies within the band's spread of mass, i.e. at the boundary).
template <int D>
__device__ __forceinline__ void refine_band(uint64_t *cdf_bits, int nb, int m, const double *qrow, const double *k64,
                                            const uint32_t *list, int lane) {
    static_assert(D % 16 == 0, "whole double2 loads");
    const int my_j = lane < nb ? (int)list[lane] : 0x7fffffff;
    // lane n scores band block list[n]: its whole key-mean row at once (independent
    // loads, so the band costs one memory latency, not nb), against the query row in
    // LDS (broadcast reads)
    double my_s = 0.0;
    if (lane < nb) {
        const double2 *kr = reinterpret_cast<const double2 *>(k64 + (int64_t)my_j * D);
        const double2 *qr = reinterpret_cast<const double2 *>(qrow);
        double acc0 = 0.0, acc1 = 0.0;
#pragma unroll 16
        for (int u = 0; u < D / 2; ++u) {
            const double2 kv = kr[u], qv = qr[u];
            acc0 = __builtin_fma(qv.x, kv.x, acc0);
            acc1 = __builtin_fma(qv.y, kv.y, acc1);
        }
        my_s = acc0 + acc1;
    }
    // rank by (exact score descending, index ascending); the m best are kept, and
    // lane n sets or clears its block's bit in the row's LDS mask words
    int rank = 0;
    for (int n = 0; n < nb; ++n) {
        const double sn = __shfl(my_s, n, 64);
        const int jn = __shfl(my_j, n, 64);
        rank += (sn > my_s || (sn == my_s && jn < my_j)) ? 1 : 0;
    }
    if (lane < nb) {
        const unsigned long long bit = 1ull << (my_j & 63);
        if (rank < m)
            atomicOr(reinterpret_cast<unsigned long long *>(cdf_bits + (my_j >> 6)), bit);
        else
            atomicAnd(reinterpret_cast<unsigned long long *>(cdf_bits + (my_j >> 6)), ~bit);
    }
}

// Pivot steps of the cut over an array of keys v (the register row, or the bracket
// compacted out of it; zeros are inert).  The key bracket (lo, hi] keeps
//   Mhi = mass(key > hi) < thr*Z <= Mlo = mass(key > lo),
// with clo, chi the counts of keys above lo and hi; mass and count of the keys above
// the array's own range come in as m0, c0.  Each step splits the bracket at a pivot,
// at one compare/select/add per element plus a wave sum; the compare masks'
// popcounts count the keys.  Pivots alternate between regula falsi on the values
// (the mass above a value is linear in the value when the e_j are spread evenly in
// log scale) and halving the key range, which bounds the steps.  Steps run while the
// bracket holds more than `stop` keys and more than one key value.
template <int N>
__device__ __forceinline__ void pivot_steps(const float (&v)[N], float thrz, float m0, uint32_t c0, uint32_t stop,
                                            uint32_t &lo, uint32_t &hi, float &Mlo, float &Mhi, uint32_t &clo,
                                            uint32_t &chi, int &step) {
#pragma unroll 1
    for (; clo - chi > stop && hi - lo > 1; ++step) {
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
        uint32_t cnt = c0;
#pragma unroll
        for (int c = 0; c < N; ++c) {
            const bool gt = __float_as_uint(v[c]) > p;
            acc += gt ? v[c] : 0.f;
            cnt += (uint32_t)__popcll(__ballot(gt));
        }
        const float A = m0 + wave_sum_u(acc);
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
}

// The keys of v inside (lo, hi], in index order, to dst (LDS); returns how many.
template <int N>
__device__ __forceinline__ uint32_t compact_bracket(const float (&v)[N], uint32_t lo, uint32_t hi, uint32_t *dst) {
    uint32_t base = 0;
#pragma unroll
    for (int c = 0; c < N; ++c) {
        const uint32_t u = __float_as_uint(v[c]);
        // the mask straight from the two compares (no per-lane bool in between), and the
        // stores under it
        const uint64_t m = __ballot(u > lo) & __ballot(u <= hi);
        if (__builtin_amdgcn_inverse_ballot_w64(m))
            dst[__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, base))] = u;
        base += (uint32_t)__popcll(m);
    }
    return base;
}

// Quotient of j by d for j, d <= 4096: j * ceil(2^24 / d) / 2^24 is exact while
// j (d - 1) < 2^24.  m24 = ceil(2^24 / d) is formed once per wave.
__device__ __forceinline__ uint32_t div_small(uint32_t j, uint32_t m24) { return __umulhi(j << 8, m24); }

// f(std::integral_constant<int, I>) for I = B .. E-1, in order, at compile time.
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// The cut of row i (threshold thr), run by one wave on its register row s (scaled
// scores, -inf for padding keys).  Returns the row's bitmask (lane c holds the word
// of key blocks 64c .. 64c+63) and its count.  `bracket` is 512 words of LDS for this
// wave (the compacted bracket, then the band's block list); `hist_all` holds 256
// words per wave: the row's 64-bit mask words while the band's exact order sets or
// clears their bits.
template <int NE, int D>
__device__ __forceinline__ void select_cut(const SelectArgs &a, float (&s)[NE], float *hist_all, uint32_t *bracket,
                                           int i, float thr, int lane, uint64_t &word, int32_t &count_out,
                                           const double *qrow, const double *k64, float band_rel) {
    constexpr int NC = 8;                  // compacted bracket: 8 words a lane, 512 keys
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool keep_all = !(thr < 1.f);
    uint32_t *list = bracket;                                                // up to 64 keys of the bracket
    uint64_t *cdf_bits = reinterpret_cast<uint64_t *>(hist_all + wave * 256);   // [NE] words (band rescoring)

    // e_j = 2^(s_j - max) in place (0 for padding), Z, the smallest positive key and
    // how many keys are positive
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < NE; ++c) mx = fmaxf(mx, s[c]);
    mx = wave_max_u(mx);
    float z = 0.f;
    uint32_t kmin = 0xffffffffu;
    int npos_l = 0;                                          // this lane's positive keys
#pragma unroll
    for (int c = 0; c < NE; ++c) {
        const float pe = __builtin_amdgcn_exp2f(s[c] - mx);
        s[c] = pe;
        z += pe;
        kmin = min(kmin, __float_as_uint(pe) - 1u);         // padding (0) wraps to the top
        npos_l += pe > 0.f ? 1 : 0;
    }
    const float Z = wave_sum_u(z);
    const float thrz = thr * Z;

    // Crossing value v* and the mass M strictly above it.  Keys are the fp32 bit
    // patterns of the e_j (order-preserving for e >= 0).  Pivot steps over the row
    // until the bracket holds at most 512 keys; on long rows those are then compacted
    // (through LDS) into NC words a lane and the steps go on over them.  Once at most
    // 64 keys remain they are compacted to LDS, sorted across the lanes, and the
    // crossing is read off their prefix sums.
    uint32_t vstar = 0x3f800000u;
    float M = 0.f;
    if (!keep_all) {
        uint32_t lo = wave_min_u32(kmin), hi = 0x3f800000u;   // every e_j <= 1, the row max is exactly 1
        float Mhi = 0.f, Mlo = Z;
        uint32_t clo = (uint32_t)wave_sum_i(npos_l), chi = 0; // counts of key > lo, key > hi
        int step = 0;
        bool packed = false;
        float t[NC];
        if constexpr (NE > NC) {
            pivot_steps(s, thrz, 0.f, 0u, 64u * NC, lo, hi, Mlo, Mhi, clo, chi, step);
            if (clo - chi > 64 && hi - lo > 1) {
                const float m0 = Mhi;
                const uint32_t c0 = chi, n = compact_bracket(s, lo, hi, bracket);
                wave_lds_sync();
#pragma unroll
                for (int w = 0; w < NC; ++w)
                    t[w] = (uint32_t)(64 * w + lane) < n ? __uint_as_float(bracket[64 * w + lane]) : 0.f;
                wave_lds_sync();
                pivot_steps(t, thrz, m0, c0, 64u, lo, hi, Mlo, Mhi, clo, chi, step);
                packed = true;
            }
        } else {
            pivot_steps(s, thrz, 0.f, 0u, 64u, lo, hi, Mlo, Mhi, clo, chi, step);
        }
        vstar = hi;       // a single key left in the bracket: v* = hi, M = Mhi
        M = Mhi;
        if (clo - chi <= 64 && clo > chi) {
            if (packed)
                compact_bracket(t, lo, hi, list);
            else
                compact_bracket(s, lo, hi, list);
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
    //      keys, by index) * v* below thr*Z.  Each 64-block word goes to LDS from
    //      one lane as it is formed, so that no per-word mask stays live in scalar
    //      registers; lane c reads word c back at the end.
    const float vstar_f = __uint_as_float(vstar);
    // the band of near-ties around v* (band_rel < 0: no exact rescoring); the main pass
    // only counts the band and the kept blocks in it, by popcounts of wave masks
    const bool refine = !keep_all && band_rel >= 0.f && qrow != nullptr;
    const float blo = vstar_f * (1.f - band_rel), bhi = vstar_f * (1.f + band_rel);
    // as bit patterns (blo_u >= 1 leaves out the padding, whose e is 0)
    const uint32_t blo_u = blo > 0.f ? max(__float_as_uint(blo), 1u) : 1u, bhi_u = __float_as_uint(bhi);
    uint32_t ties_before = 0, nb = 0, mb = 0;
    static_for<0, NE>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        uint64_t m;
        if (keep_all) {
            m = __ballot(64 * c + lane < a.nB);
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
            if (refine) {
                const uint64_t bm = __ballot(u >= blo_u) & __ballot(u <= bhi_u);
                nb += (uint32_t)__popcll(bm);
                mb += (uint32_t)__popcll(bm & m);
            }
        }
        if (lane == 0) cdf_bits[c] = m;
    });
    if (refine && nb >= 2 && nb <= (uint32_t)kRefineMax && mb > 0 && mb < nb) {
        // the band's indices, ascending, into this wave's LDS list; the row's words to
        // LDS, where the exact order of the band sets or clears their bits
        uint32_t base = 0;
#pragma unroll
        for (int c = 0; c < NE; ++c) {
            const uint32_t u = __float_as_uint(s[c]);
            const uint64_t bm = __ballot(u >= blo_u) & __ballot(u <= bhi_u);
            if (__builtin_amdgcn_inverse_ballot_w64(bm))
                list[__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, base))] =
                    (uint32_t)(64 * c + lane);
            base += (uint32_t)__popcll(bm);
        }
        wave_lds_sync();
        refine_band<D>(cdf_bits, (int)nb, (int)mb, qrow, k64, list, lane);
    }
    wave_lds_sync();
    // word c of the row to lane c
    uint64_t cdf_word = lane < NE ? cdf_bits[lane] : 0ull;
    // ---- the window, ORed in: frames form a contiguous range of j, rows and columns
    //      come from exact small quotients
    if (a.window) {
        const int nTyx = a.nTy * a.nTx;
        const int ti = i / nTyx, yi = (i / a.nTx) % a.nTy, xi = i % a.nTx;
        const int nT = a.nB / nTyx;
        const int jlo = max(ti - a.wt, 0) * nTyx;                                  // frames in reach
        const int jhi = ((a.wt >= nT - ti ? nT - 1 : ti + a.wt) + 1) * nTyx;
        const uint32_t m_x = (0x1000000u + (uint32_t)a.nTx - 1u) / (uint32_t)a.nTx;
        const uint32_t m_y = (0x1000000u + (uint32_t)a.nTy - 1u) / (uint32_t)a.nTy;
        wave_lds_sync();      // every lane has read its word: the window's words reuse the array
        static_for<0, NE>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            const int j = 64 * c + lane;
            const uint32_t row = div_small((uint32_t)j, m_x);                 // j / nTx
            const int xj = j - (int)row * a.nTx;
            const int yj = (int)row - (int)div_small(row, m_y) * a.nTy;      // (j / nTx) % nTy
            const uint64_t mw = __ballot(j >= jlo && j < jhi && abs(yj - yi) <= a.wh && abs(xj - xi) <= a.ww);
            if (lane == 0) cdf_bits[c] = mw;
        });
        wave_lds_sync();
        if (lane < NE) cdf_word |= cdf_bits[lane];
    }
    word = cdf_word;
    count_out = (int32_t)wave_sum_i(__popcll(word));
}

// Uniform in [0, 1) for block j of row r: the top 24 bits of output r * nB + j + 1
// of the SplitMix64 stream seeded with `seed` (state advanced by the golden gamma,
// output through the variant-13 murmur3 finaliser), times 2^-24.
constexpr uint64_t kSplitmixGamma = 0x9E3779B97F4A7C15ull;
// the output function applied to the state z = seed + counter * gamma
__device__ __forceinline__ float splitmix_out(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (float)(uint32_t)(z >> 40) * 0x1p-24f;
}

// Sampling with inclusion probabilities ("SIP", AB-Attention page, section "Les
// trois techniques d'AB-Attention") on row i, run by one wave on its register row s
// (pooled scores in log2 units, -inf for padding): pi_j = min(1, c p_j) with
// sum pi = budget, p the row softmax.  The capped blocks are those with s_j >= sigma;
// with mR the largest uncapped score and E = sum over the uncapped of 2^(s - mR), an
// uncapped block gets (budget - #capped) 2^(s_j - mR) / E = 2^(s_j - t) with
// t = mR + log2(E / (budget - #capped)), taken relative to mR so that no
// probability underflows.  Starting with nothing capped, every block with s_j >= t is
// capped (sigma = t) and t recomputed, until t lies above every uncapped score (the
// capped set only grows).  A budget of at least the number of real blocks keeps all
// of them.  Block j is kept when its uniform is below pi_j.  Returns this lane's
// bitmask word (as select_cut), the count, sigma and t (sigma = -inf: keep all).
template <int NE>
__device__ __forceinline__ void sip_cut(const SelectArgs &a, const float (&s)[NE], int64_t row, int lane,
                                        uint64_t *wbits, uint64_t &word, int32_t &count_out, float &sigma_out,
                                        float &t_out) {
    float sigma = INFINITY, t = INFINITY;
    if (a.budget < (float)a.nB) {
        uint32_t ncap = 0;
        for (int it = 0; it < 64; ++it) {
            float mr = -INFINITY;
#pragma unroll
            for (int c = 0; c < NE; ++c) mr = fmaxf(mr, s[c] < sigma ? s[c] : -INFINITY);
            mr = wave_max_u(mr);
            float e = 0.f;
#pragma unroll
            for (int c = 0; c < NE; ++c) e += s[c] < sigma ? __builtin_amdgcn_exp2f(s[c] - mr) : 0.f;
            const float E = wave_sum_u(e);
            t = mr + __log2f(E / (a.budget - (float)ncap));
            if (!(t <= mr)) break;                    // the largest uncapped block stays below 1
            uint32_t cnt = 0;
#pragma unroll
            for (int c = 0; c < NE; ++c) cnt += (uint32_t)__popcll(__ballot(s[c] >= t));
            sigma = t;
            ncap = cnt;
        }
    } else {
        sigma = -INFINITY;
    }
    // the generator's state for key j = 64c + lane, seed + (row nB + j + 1) gamma, steps
    // by 64 gamma from one word to the next (the same value mod 2^64).  Each word goes
    // to LDS from one lane as it is formed (no mask stays live in scalar registers),
    // and lane c reads word c back.
    uint64_t z = a.seed + ((uint64_t)row * (uint64_t)a.nB + (uint64_t)lane + 1ull) * kSplitmixGamma;
    uint32_t count = 0;
#pragma unroll
    for (int c = 0; c < NE; ++c) {
        const int j = 64 * c + lane;
        const float pi = s[c] >= sigma ? 1.f : __builtin_amdgcn_exp2f(s[c] - t);
        const uint64_t m = __ballot(j < a.nB) & __ballot(splitmix_out(z) < pi);
        z += 64ull * kSplitmixGamma;
        count += (uint32_t)__popcll(m);
        if (lane == 0) wbits[c] = m;
    }
    wave_lds_sync();
    word = lane < NE ? wbits[lane] : 0ull;
    count_out = (int32_t)count;
    sigma_out = sigma;
    t_out = t;
}


// NE = 4 * ceil(nB / 256): the register row length in 64-key words (chunks of 256 keys).
// Workgroup = row group taken by ticket (groups start in order).  Wave w pools query
// block i0 + w into LDS while the first key chunk loads, the waves form the scores
// chunk by chunk, each cuts its row, wave 0 finds the group's offset by look-back,
// and each wave writes its row's row_ptr entry and kept columns.
//
// MODE 0: NABLA's CDF cut; MODE 1: sampling with inclusion probabilities, which also
// writes the offset -ln(pi) of every kept block to col_bias; MODE 2: NABLA's CDF cut
// on rows given in log2 units (mix_rows, one per pair of query blocks: the
// clustering selector), with no pooling or scores of its own.
template <typename T, int D, int NE, int MODE>
__device__ __forceinline__ void select_emit_body(const SelectArgs &a) {
    static_assert(NE % 4 == 0 && NE <= 64, "NE: register row length in 64-key words");
    constexpr int KB = D / 32;                     // k-blocks of one 16x16x32 product
    constexpr int NCH = NE / 4;                    // score chunks
    // registers for the next chunk's operands where they fit (at NE <= 8 the chunks are
    // few and the prefetch measured no faster)
    constexpr bool kPrefetch = NE > 8 && NE <= 32;
    // the CDF selection pools its queries in fp64 (exact means for the near-tie
    // rescoring); rows of up to 512 blocks keep 4 loads a lane in flight, longer rows
    // (registers free while the scores do not exist yet) all 16
    using QP = BlockPool<T, D, MODE == 0 ? (NE <= 8 ? 4 : 16) : 8>;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __bf16 *qf = reinterpret_cast<__bf16 *>(smem_raw);                              // [16][2D+8]
    float *stage = reinterpret_cast<float *>(smem_raw + (size_t)kSelRows * qf_stride<D>() * 2);  // [2][16][260]
    float *hist_all = stage + 2 * kSelRows * kStageStride;                          // [16][256]
    double *q64 = reinterpret_cast<double *>(hist_all + kSelRows * 256);            // [16][D] exact query means
    __shared__ uint32_t s_ticket;
    __shared__ int32_t wave_count[kSelRows];
    __shared__ int64_t s_base;
    __shared__ int32_t s_gave_up;
    __shared__ float s_kmax[kSelRows];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (threadIdx.x == 0) s_ticket = atomicAdd(a.ticket, 1u);
    __syncthreads();
    const uint32_t g = __builtin_amdgcn_readfirstlane(s_ticket);
    const uint32_t bh = g / (uint32_t)a.groups_per_head;
    const int i0 = (int)(g - bh * (uint32_t)a.groups_per_head) * kSelRows;
    const int nrows = min(kSelRows, a.nB - i0);
    const __bf16 *ks = a.kbar + kbar_group(bh, a.groups_per_head, 0, D);
    const float thr = a.thr[bh % (uint32_t)a.H];

    const int ii = lane & 15, kq = lane >> 4;
    float s[NE];
    if constexpr (MODE == 2) {
        const int64_t pr = ((int64_t)bh - a.head0) * ((a.nB + 1) / 2) + (i0 + wave) / 2;
        const float *src = a.mix_rows + pr * a.nBp;
#pragma unroll
        for (int c = 0; c < NE; ++c) {
            const int j = 64 * c + lane;
            s[c] = (wave < nrows && j < a.nB) ? src[j] : -INFINITY;
        }
    } else {
    bf16x8 kh[2][KB], kl[2][KB];
    // the 16 keys of group 16 cc + wave, one contiguous 1 KiB run per load; groups past
    // the head's last read its first (in bounds), and keys past nB inside the last
    // group read its padding: their scores land on padding columns
    auto load_k = [&](int cc, int slot) {
        const int gg = (kSelChunk / 16) * cc + wave;
        const __bf16 *kr = ks + (int64_t)(gg < a.groups_per_head ? gg : 0) * (32 * D) + 8 * lane;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            kh[slot][kb] = *reinterpret_cast<const bf16x8 *>(kr + 512 * kb);
            kl[slot][kb] = *reinterpret_cast<const bf16x8 *>(kr + 16 * D + 512 * kb);
        }
    };
    // one part of the group: the hi parts (lo = false) or the lo parts
    auto load_k_part = [&](int cc, int slot, bool lo) {
        const int gg = (kSelChunk / 16) * cc + wave;
        const __bf16 *kr = ks + (int64_t)(gg < a.groups_per_head ? gg : 0) * (32 * D) + 8 * lane;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if (lo)
                kl[slot][kb] = *reinterpret_cast<const bf16x8 *>(kr + 16 * D + 512 * kb);
            else
                kh[slot][kb] = *reinterpret_cast<const bf16x8 *>(kr + 512 * kb);
        }
    };
    // ---- the largest key-mean norm of the head (for the scores' error bound), each
    //      wave over a slice of the head's key blocks
    if constexpr (MODE == 0) {
        const int per = (a.nB + kSelRows - 1) / kSelRows;
        float mx = 0.f;
        for (int j = wave * per + lane; j < min(a.nB, (wave + 1) * per); j += 64)
            mx = fmaxf(mx, a.knorm[(int64_t)bh * a.nB + j]);
        mx = wave_max_u(mx);
        if (lane == 0) s_kmax[wave] = mx;
    }
    // ---- the group's pooled queries (hi | lo), one query block per wave: pooled here,
    //      or copied from the means the reorder formed
    {
        __bf16 *qrow = qf + wave * qf_stride<D>();
        if (a.qbar != nullptr) {
            using QV = std::conditional_t<D == 128, uint2, uint32_t>;   // 2D bf16 over the 64 lanes
            const QV v =
                wave < nrows ? reinterpret_cast<const QV *>(a.qbar + ((int64_t)bh * a.nB + i0 + wave) * (2 * D))[lane]
                             : QV{};
            reinterpret_cast<QV *>(qrow)[lane] = v;
            if constexpr (MODE == 0) {
                if (wave < nrows) {
                    const double *src = a.qbar64 + ((int64_t)bh * a.nB + i0 + wave) * D;
#pragma unroll
                    for (int u = 0; u < D / 64; ++u) q64[wave * D + (D / 64) * lane + u] = src[(D / 64) * lane + u];
                }
            }
        } else if (wave < nrows) {
            float x[QP::VEC];
            const T *qb = reinterpret_cast<const T *>(a.q) + (((int64_t)bh * a.nB + i0 + wave) * kTokensPerBlock) * D;
            const uint64_t valid = a.geo.partial ? __ballot(slot_valid(a.geo, i0 + wave, lane)) : ~0ull;
            if constexpr (MODE == 0) {
                double x64[QP::VEC];
                QP::mean(qb, lane, x64, valid);
                QP::to_f32(x64, x);
                if (lane < QP::LPR) QP::store64(x64, q64 + wave * D, lane);
            } else {
                QP::mean(qb, lane, x, valid);
            }
            if (lane < QP::LPR) QP::store_split(x, qrow, lane);
        } else if (lane < 2 * D / 8) {
            reinterpret_cast<uint4 *>(qrow)[lane] = uint4{0u, 0u, 0u, 0u};
        }
    }
    load_k(0, 0);
    __syncthreads();

    // ---- scores, chunk by chunk, into the register row
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
        const int cur = kPrefetch ? (cc & 1) : 0;
        if (kPrefetch && cc + 1 < NCH) load_k(cc + 1, cur ^ 1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const __bf16 *qrow = qf + ii * qf_stride<D>() + 8 * kq;
        if constexpr (kPrefetch) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 qh = *reinterpret_cast<const bf16x8 *>(qrow + 32 * kb);
                const bf16x8 ql = *reinterpret_cast<const bf16x8 *>(qrow + D + 32 * kb);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kh[cur][kb], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kl[cur][kb], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kh[cur][kb], acc, 0, 0, 0);
            }
        } else {
            // the products with the K hi parts first: those registers then take the next
            // chunk's hi parts while the products with the lo parts run, and the lo parts
            // follow; the loads get the lo products, the stage and the barrier ahead of use
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 qh = *reinterpret_cast<const bf16x8 *>(qrow + 32 * kb);
                const bf16x8 ql = *reinterpret_cast<const bf16x8 *>(qrow + D + 32 * kb);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kh[0][kb], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kh[0][kb], acc, 0, 0, 0);
            }
            if (cc + 1 < NCH) load_k_part(cc + 1, 0, false);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 qh = *reinterpret_cast<const bf16x8 *>(qrow + 32 * kb);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kl[0][kb], acc, 0, 0, 0);
            }
            if (cc + 1 < NCH) load_k_part(cc + 1, 0, true);
        }
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
    __syncthreads();   // every wave has its row: the cut reuses the stage
    }
    uint64_t word = 0;
    int32_t count = 0;
    float sigma = 0.f, tcap = 0.f;
    if (wave < nrows) {
        if constexpr (MODE == 0) {
            // half-width of the near-tie band, relative: twice the score bound (the row
            // max carries one too) in log2 units, plus the exponential's own rounding
            float kmax = 0.f;
#pragma unroll
            for (int w = 0; w < kSelRows; ++w) kmax = fmaxf(kmax, s_kmax[w]);
            const double *qrow = q64 + wave * D;
            float qq = 0.f;
#pragma unroll
            for (int u = 0; u < D / 64; ++u) {
                const float x = (float)qrow[(D / 64) * lane + u];
                qq += x * x;
            }
            const float qn = sqrtf(wave_sum_u(qq));
            const float band_rel =
                __builtin_amdgcn_exp2f(2.f * kScoreEps * a.scale_log2 * qn * kmax * 1.01f) - 1.f + 0x1p-20f;
            select_cut<NE, D>(a, s, hist_all, reinterpret_cast<uint32_t *>(stage) + 512 * wave, i0 + wave, thr, lane,
                              word, count, qrow, a.kbar64 + (int64_t)bh * a.nB * D, band_rel);
        } else if constexpr (MODE == 2) {
            select_cut<NE, D>(a, s, hist_all, reinterpret_cast<uint32_t *>(stage) + 512 * wave, i0 + wave, thr, lane,
                              word, count, nullptr, nullptr, -1.f);
        } else {
            sip_cut<NE>(a, s, (int64_t)bh * a.nB + i0 + wave, lane,
                        reinterpret_cast<uint64_t *>(hist_all + wave * 256), word, count, sigma, tcap);
        }
    }
    if (lane == 0) wave_count[wave] = count;
    __syncthreads();

    // ---- offsets: the group's by look-back, then the rows' within the group
    if (wave == 0) {
        const int32_t total = wave_sum_i(lane < kSelRows ? wave_count[lane] : 0);
        bool gave_up;
        const int64_t base = group_lookback(a.status, g, total, lane, a.spin_cap, gave_up);
        if (lane == 0) {
            s_base = base;
            s_gave_up = gave_up;
            if (gave_up) __hip_atomic_store(a.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (wave >= nrows) return;
    const int64_t row = (int64_t)bh * a.nB + i0 + wave;
    if (s_gave_up) {
        // the offset is unknown: poison the group's rows and write no columns
        if (lane == 0) {
            a.row_ptr[row] = -1;
            if (row == a.rows - 1) a.row_ptr[a.rows] = -1;
        }
        return;
    }
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_count[w];
    int32_t pos = (int32_t)s_base + before;
    if (lane == 0) {
        a.row_ptr[row] = pos;
        if (row == a.rows - 1) a.row_ptr[a.rows] = pos + count;
    }
    // ---- kept columns, ascending: word e of the row sits in lane e.  Per word the
    //      lanes whose bit is set (the word itself as the execution mask) store their
    //      column at the word's offset plus the set bits below them; the offset runs
    //      on in a scalar register.
    const int nvc = a.nBp >> 6;
    const int32_t pos_s = __builtin_amdgcn_readfirstlane(pos);
    int32_t *const dst = a.col_idx + pos_s;
    uint32_t off = 0;
    if constexpr (MODE != 1) {
        for (int e = 0; e < nvc; ++e) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)word, e);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(word >> 32), e);
            const uint64_t m = ((uint64_t)hi << 32) | lo;
            if (__builtin_amdgcn_inverse_ballot_w64(m))
                dst[__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, off))] = 64 * e + lane;
            off += (uint32_t)__popcll(m);
        }
    } else {
        // the register row is indexed by the word, so the loop runs at compile time (a
        // test rather than an exit keeps it unrolled, and the row in registers)
        float *const bdst = a.col_bias + pos_s;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            if (e >= nvc) continue;
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)word, e);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(word >> 32), e);
            const uint64_t m = ((uint64_t)hi << 32) | lo;
            if (__builtin_amdgcn_inverse_ballot_w64(m)) {
                const uint32_t at = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, off));
                dst[at] = 64 * e + lane;
                bdst[at] = s[e] >= sigma ? 0.f : (tcap - s[e]) * kLn2;   // -ln(pi)
            }
            off += (uint32_t)__popcll(m);
        }
    }
}

// One workgroup a CU (up to 128 VGPRs a wave).  Rows of up to 512 key blocks would fit
// two workgroups a CU at 64 VGPRs, but the fp64 pooling then spills (88 B of scratch a
// lane), and one unspilled workgroup a CU measured faster (480p: 84 -> 75 us).
template <typename T, int D, int NE, int MODE>
__global__ __launch_bounds__(1024, 4) void select_emit_kernel(SelectArgs a) {
    select_emit_body<T, D, NE, MODE>(a);
}

// ---------------------------------------------------------------------------
int launch_pool_keys(const void *k, __bf16 *kbar, double *kbar64, float *knorm, int64_t nblocks, int32_t nB, int dtype,
                     int d, const PoolSide &side, const SlotGeo &geo, hipStream_t s) {
    const dim3 grid((unsigned)((nblocks + 3) / 4)), block(256);
    if (dtype == 1 && d == 128)
        pool_kernel<__bf16, 128><<<grid, block, 0, s>>>((const __bf16 *)k, kbar, kbar64, knorm, nblocks, nB, side, geo);
    else if (dtype == 1 && d == 64)
        pool_kernel<__bf16, 64><<<grid, block, 0, s>>>((const __bf16 *)k, kbar, kbar64, knorm, nblocks, nB, side, geo);
    else if (dtype == 0 && d == 128)
        pool_kernel<float, 128><<<grid, block, 0, s>>>((const float *)k, kbar, kbar64, knorm, nblocks, nB, side, geo);
    else
        pool_kernel<float, 64><<<grid, block, 0, s>>>((const float *)k, kbar, kbar64, knorm, nblocks, nB, side, geo);
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

template <typename T, int D, int NCH, int MODE = 0>
static void launch_select_nch(const SelectArgs &a, int nch, hipStream_t s) {
    if constexpr (NCH <= kSelectMaxBlocks / kSelChunk) {
        if (nch == NCH) {
            select_emit_kernel<T, D, 4 * NCH, MODE>
                <<<dim3((unsigned)a.n_groups), dim3(64 * kSelRows), select_lds_bytes<D>(), s>>>(a);
            return;
        }
        launch_select_nch<T, D, NCH + 1, MODE>(a, nch, s);
    }
}

int launch_select(const SelectArgs &a, int d, int dtype, hipStream_t s) {
    if (a.nBp > kSelectMaxBlocks) return -1;
    const int nch = (a.nB + kSelChunk - 1) / kSelChunk;
    if (dtype == 1 && d == 128)
        launch_select_nch<__bf16, 128, 1>(a, nch, s);
    else if (dtype == 1 && d == 64)
        launch_select_nch<__bf16, 64, 1>(a, nch, s);
    else if (dtype == 0 && d == 128)
        launch_select_nch<float, 128, 1>(a, nch, s);
    else
        launch_select_nch<float, 64, 1>(a, nch, s);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------
// The clustering selector's rows (AB-Attention page, section "Les trois techniques
// d'AB-Attention", first item).  A workgroup of 16 waves serves two pairs of query
// blocks of one (batch, head) (128 queries a pair; an odd last block alone); waves
// 8P .. 8P + 7 serve pair P.
//  - Lloyd's k-means with 8 clusters and 4 rounds, started from the queries at
//    positions n*c/8.  Assignment: each query is split over 4 lanes (D/4
//    dimensions each, in registers); the squared distances to the 8 centroids, fp32
//    sums of (x - mu)^2 over the lane's dimensions and then over the 4 lanes, pick
//    the nearest, ties to the lower cluster.  Update: the cluster sums are the
//    product onehot^T X on v_mfma_f32_16x16x32_bf16 (0/1 and the bf16 queries are
//    exact operands, fp32 accumulation); a centroid becomes its cluster's sum over
//    its count, and an empty cluster keeps its centroid.  The weights are the last
//    assignment's shares.
//  - Scores of the 16 centroids on every key block mean, S = mu . Kbar * scale, on
//    the same MFMA with each centroid split into three bf16 parts (hi, mid, lo) and
//    the key means in their two (hi, lo): the five products that reach 2^-24.
//  - Wave 8P + c: softmax of centroid c on its register row (max, then the sum),
//    weighted by w_c.  The pair's row is the sum of its 8 weighted rows, added in
//    cluster order through LDS 256 keys at a time, and stored in log2 units for the
//    cut.
// QT = float (fp32 queries): they are staged in fp32, the k-means runs on their exact
// values, and the cluster sums take each value as three bf16 parts (hi, mid, lo),
// which hold an fp32 value exactly (away from the bottom of the exponent range), in
// three one-hot products.
template <typename QT, int D, int NE>
__global__ __launch_bounds__(1024) void ibcs_mix_kernel(IbcsArgs a) {
    constexpr int K = kIbcsClusters, DP = D / 4, KB = D / 32, NCH = NE / 4;
    constexpr int QW = 3 * D + 8;                                   // bf16 per centroid row: hi | mid | lo, pad
    constexpr int QBYTES = 2 * 128 * D * (int)sizeof(QT);            // the two pairs' queries
    constexpr int SBYTES = 16 * QW * 2 + 2 * kSelRows * kStageStride * 4;
    constexpr int BIG = QBYTES > SBYTES ? QBYTES : SBYTES;
    constexpr int V16 = 16 / (int)sizeof(QT);                        // elements per 16-byte load
    static_assert(K == 8 && D % 32 == 0 && (2 * 128 * D / V16) % 1024 == 0, "layout");
    __shared__ __attribute__((aligned(16))) unsigned char big[BIG];
    __shared__ float mu[2][K][D];
    __shared__ int32_t asg[2][128];
    __shared__ int32_t cnt[2][K];
    QT *qs = reinterpret_cast<QT *>(big);                             // [2][128][D], during the k-means
    __bf16 *qf = reinterpret_cast<__bf16 *>(big);                   // [16][QW], afterwards
    float *stage = reinterpret_cast<float *>(big + 16 * QW * 2);    // [2][16][kStageStride]

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int P = wave >> 3, w8 = wave & 7;
    const int gph = (a.pairs_per_head + 1) / 2;
    const int64_t bh = a.head0 + blockIdx.x / gph;
    const int p0 = 2 * (int)(blockIdx.x % gph);
    const int np = p0 + 1 < a.pairs_per_head ? 2 : 1;               // pairs in this workgroup
    const int64_t N = (int64_t)a.nB * 64;
    auto pair_n = [&](int pp) { return 2 * (p0 + pp) + 1 < a.nB ? 128 : 64; };
    {
        // the pairs' queries, a batch of this thread's loads in flight before its stores
        // (fp32: two batches, so that the staging registers stay those of bf16)
        constexpr int PER = 2 * 128 * D / V16 / 1024, PP = 128 * D / V16;
        constexpr int BAT = PER < 4 ? PER : 4;
        const QT *qg = reinterpret_cast<const QT *>(a.q);
#pragma unroll
        for (int u0 = 0; u0 < PER; u0 += BAT) {
            uint4 tmp[BAT];
#pragma unroll
            for (int u = 0; u < BAT; ++u) {
                const int e = t + 1024 * (u0 + u), pp = e / PP, r = e % PP;
                const bool ok = pp < np && r < pair_n(pp) * D / V16;
                tmp[u] = ok ? reinterpret_cast<const uint4 *>(qg + (bh * N + (int64_t)128 * (p0 + pp)) * D)[r]
                            : uint4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < BAT; ++u) reinterpret_cast<uint4 *>(qs)[t + 1024 * (u0 + u)] = tmp[u];
        }
    }
    __syncthreads();

    // ---- k-means of pair P: lane (q, part) holds query q's dimensions part*DP ..
    const int tp = t & 511, q = tp >> 2, part = tp & 3;
    const int n = pair_n(P);
    float x[DP];
    if constexpr (sizeof(QT) == 2) {
        const uint4 *src = reinterpret_cast<const uint4 *>(qs + (P * 128 + q) * D + part * DP);
#pragma unroll
        for (int u = 0; u < DP / 8; ++u) {
            const uint4 w = src[u];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[8 * u + 2 * k] = bf16_lo(ws[k]);
                x[8 * u + 2 * k + 1] = bf16_hi(ws[k]);
            }
        }
    } else {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(qs + (P * 128 + q) * D + part * DP);
#pragma unroll
        for (int u = 0; u < DP / 4; ++u) {
            const f32x4 w = src[u];
#pragma unroll
            for (int k = 0; k < 4; ++k) x[4 * u + k] = w[k];
        }
    }
    for (int e = tp; e < K * D; e += 512) {
        const int c = e / D, dd = e % D;
        mu[P][c][dd] = (float)qs[(P * 128 + (n * c) / K) * D + dd];
    }
    __syncthreads();
#pragma unroll 1
    for (int it = 0; it < kIbcsIters; ++it) {
        float dist[K];
#pragma unroll
        for (int c = 0; c < K; ++c) {
            const float *m = &mu[P][c][part * DP];
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < DP; ++i) {
                const float df = x[i] - m[i];
                acc = __builtin_fmaf(df, df, acc);
            }
            dist[c] = acc;
        }
#pragma unroll
        for (int c = 0; c < K; ++c) {
            dist[c] += __shfl_xor(dist[c], 1, 64);
            dist[c] += __shfl_xor(dist[c], 2, 64);
        }
        int best = 0;
        float bd = dist[0];
#pragma unroll
        for (int c = 1; c < K; ++c)
            if (dist[c] < bd) {
                bd = dist[c];
                best = c;
            }
        if (part == 0) asg[P][q] = q < n ? best : -1;
        __syncthreads();
        if (w8 == 0) {
#pragma unroll
            for (int c = 0; c < K; ++c) {
                const int m = __popcll(__ballot(asg[P][lane] == c)) + __popcll(__ballot(asg[P][64 + lane] == c));
                if (lane == 0) cnt[P][c] = m;
            }
        }
        // cluster sums of dimensions 16 w8 .. 16 w8 + 15: row = cluster (0 .. 15, 8 .. 15
        // empty), k = query, column = dimension
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        const int cl = lane & 15, kq = lane >> 4, dim = 16 * w8 + (lane & 15);
        if (16 * w8 < D) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int qb = 32 * ks + 8 * kq;
                bf16x8 oh;
#pragma unroll
                for (int i = 0; i < 8; ++i) oh[i] = asg[P][qb + i] == cl ? (__bf16)1.f : (__bf16)0.f;
                if constexpr (sizeof(QT) == 2) {
                    bf16x8 xb;
#pragma unroll
                    for (int i = 0; i < 8; ++i) xb[i] = qs[(P * 128 + qb + i) * D + dim];
                    sum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, xb, sum, 0, 0, 0);
                } else {
                    bf16x8 xh, xm, xl;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float v = qs[(P * 128 + qb + i) * D + dim];
                        xh[i] = (__bf16)v;
                        const float r1 = v - (float)xh[i];
                        xm[i] = (__bf16)r1;
                        xl[i] = (__bf16)(r1 - (float)xm[i]);
                    }
                    sum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, xh, sum, 0, 0, 0);
                    sum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, xm, sum, 0, 0, 0);
                    sum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, xl, sum, 0, 0, 0);
                }
            }
        }
        __syncthreads();            // counts written; every read of the old centroids done
        if (16 * w8 < D) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 4 * kq + i;
                if (c < K && cnt[P][c] > 0) mu[P][c][dim] = sum[i] / (float)cnt[P][c];
            }
        }
        __syncthreads();
    }
    const float wgt = (float)cnt[P][w8] / (float)n;                  // this wave's centroid weight

    // ---- centroid rows as three bf16 parts (the query buffer is free)
    for (int e = t; e < 16 * D; e += 1024) {
        const int r = e / D, dd = e % D;
        const float v = (r >> 3) < np ? mu[r >> 3][r & 7][dd] : 0.f;
        const __bf16 h = (__bf16)v;
        const float r1 = v - (float)h;
        const __bf16 m = (__bf16)r1;
        qf[r * QW + dd] = h;
        qf[r * QW + D + dd] = m;
        qf[r * QW + 2 * D + dd] = (__bf16)(r1 - (float)m);
    }
    __syncthreads();

    // ---- scores, chunk by chunk, into the register row of wave 8P + c (as in the
    //      selection: 16 rows x 16 keys per wave and chunk, parked in the LDS stage)
    const int ii = lane & 15, kq = lane >> 4;
    const int32_t kgph = (a.nB + 15) / 16;   // key groups per head
    const __bf16 *ks = a.kbar + kbar_group(bh, kgph, 0, D);
    float s[NE];
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
        bf16x8 kh[KB], kl[KB];
        const int gg = (kSelChunk / 16) * cc + wave;   // key group (padding groups read the first)
        const __bf16 *kr = ks + (int64_t)(gg < kgph ? gg : 0) * (32 * D) + 8 * lane;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            kh[kb] = *reinterpret_cast<const bf16x8 *>(kr + 512 * kb);
            kl[kb] = *reinterpret_cast<const bf16x8 *>(kr + 16 * D + 512 * kb);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const __bf16 *qrow = qf + ii * QW + 8 * kq;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 qh = *reinterpret_cast<const bf16x8 *>(qrow + 32 * kb);
            const bf16x8 qm = *reinterpret_cast<const bf16x8 *>(qrow + D + 32 * kb);
            const bf16x8 ql = *reinterpret_cast<const bf16x8 *>(qrow + 2 * D + 32 * kb);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kh[kb], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qm, kl[kb], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qm, kh[kb], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kl[kb], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kh[kb], acc, 0, 0, 0);
        }
        // acc[e] = S[row 4 kq + e][key 256 cc + 16 wave + ii]
        float *st = stage + (cc & 1) * kSelRows * kStageStride;
#pragma unroll
        for (int e = 0; e < 4; ++e) st[(4 * kq + e) * kStageStride + 16 * wave + ii] = acc[e] * a.scale_log2;
        __syncthreads();
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const float v = st[wave * kStageStride + 64 * t4 + lane];
            s[4 * cc + t4] = kSelChunk * cc + 64 * t4 + lane < a.nB ? v : -INFINITY;
        }
    }

    // ---- softmax of this wave's centroid, weighted; the pair's row in cluster order
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < NE; ++c) mx = fmaxf(mx, s[c]);
    const float gmx = wave_max_u(mx);
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < NE; ++c) z += __builtin_amdgcn_exp2f(s[c] - gmx);
    const float f = wgt / wave_sum_u(z);
    float *T = stage;                                               // [16][kStageStride]
    __syncthreads();                                                // every wave has read its last stage
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
            T[wave * kStageStride + 64 * t4 + lane] = f * __builtin_amdgcn_exp2f(s[4 * e + t4] - gmx);
        __syncthreads();
        if (t < 512) {
            const int pp = t >> 8, k = t & 255, j = kSelChunk * e + k;
            if (pp < np && j < a.nB) {
                float sum = 0.f;
#pragma unroll
                for (int c = 0; c < K; ++c) sum += T[(8 * pp + c) * kStageStride + k];
                a.rows[((bh - a.head0) * a.pairs_per_head + p0 + pp) * a.nBp + j] =
                    sum > 0.f ? __log2f(sum) : -INFINITY;
            }
        }
        __syncthreads();
    }
}

template <typename T, int D, int NCH>
static void launch_ibcs_nch(const IbcsArgs &a, dim3 g, int nch, hipStream_t s) {
    if constexpr (NCH <= kSelectMaxBlocks / kSelChunk) {
        if (nch == NCH) {
            ibcs_mix_kernel<T, D, 4 * NCH><<<g, dim3(1024), 0, s>>>(a);
            return;
        }
        launch_ibcs_nch<T, D, NCH + 1>(a, g, nch, s);
    }
}

int launch_ibcs_mix(const IbcsArgs &a, int64_t heads, int d, int dtype, hipStream_t s) {
    if (a.nBp > kSelectMaxBlocks) return -1;
    const dim3 g((unsigned)(heads * ((a.pairs_per_head + 1) / 2)));
    const int nch = (a.nB + kSelChunk - 1) / kSelChunk;
    if (dtype == 1 && d == 128)
        launch_ibcs_nch<__bf16, 128, 1>(a, g, nch, s);
    else if (dtype == 1)
        launch_ibcs_nch<__bf16, 64, 1>(a, g, nch, s);
    else if (d == 128)
        launch_ibcs_nch<float, 128, 1>(a, g, nch, s);
    else
        launch_ibcs_nch<float, 64, 1>(a, g, nch, s);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int NCH> static void launch_rows_nch(const SelectArgs &a, int64_t groups, int nch, hipStream_t s) {
    if constexpr (NCH <= kSelectMaxBlocks / kSelChunk) {
        if (nch == NCH) {
            select_emit_kernel<__bf16, 128, 4 * NCH, 2>
                <<<dim3((unsigned)groups), dim3(64 * kSelRows), select_lds_bytes<128>(), s>>>(a);
            return;
        }
        launch_rows_nch<NCH + 1>(a, groups, nch, s);
    }
}

int launch_select_rows(const SelectArgs &a, int64_t groups, hipStream_t s) {
    if (a.nBp > kSelectMaxBlocks) return -1;
    launch_rows_nch<1>(a, groups, (a.nB + kSelChunk - 1) / kSelChunk, s);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_select_sip(const SelectArgs &a, int d, int dtype, hipStream_t s) {
    if (a.nBp > kSelectMaxBlocks) return -1;
    const int nch = (a.nB + kSelChunk - 1) / kSelChunk;
    if (dtype == 1 && d == 128)
        launch_select_nch<__bf16, 128, 1, 1>(a, nch, s);
    else if (dtype == 1)
        launch_select_nch<__bf16, 64, 1, 1>(a, nch, s);
    else if (d == 128)
        launch_select_nch<float, 128, 1, 1>(a, nch, s);
    else
        launch_select_nch<float, 64, 1, 1>(a, nch, s);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
