// Selection of 4-token key blocks for each 64-token query block (gfx950).
//
// AB-Attention page, section "Les trois techniques d'AB-Attention", third technique:
// key/value blocks of 4 tokens, which the attention kernel gathers by index into full
// tiles.  They are scored and cut with NABLA's rule (NABLA summary page, section
// "Methodologie : NABLA": "Sous-echantillonnage" -- means of the blocks; "Attention
// Reduite" -- softmax over the pooled scores of a row; "Seuil CDF" -- keep blocks in
// descending probability while the mass before them is below thr).
//
//   fine_pool_kernel   -- the 4-token key means (fp32 from an fp64 sum, in planes of 4
//                         columns so that the lanes of a wave read consecutive keys),
//                         their norms, and the selection's side jobs;
//   fine_select_kernel -- R query blocks of one head per workgroup: their means (fp64,
//                         exact), fp32 scores against all nK = 16 nB key means of the
//                         head, spread over the 16 waves (a slice of S keys each, W
//                         words of 64 a lane, R rows at once), the row softmax, the CDF
//                         cut by a pivot search whose partial sums meet in LDS, the
//                         exact fp64 order of the near-ties at the cut, and the CSR by
//                         look-back over the groups' totals.
#include "common.h"
#include "kernels.h"
#include "lookback.h"

namespace sattn {

// One thread per (4-token key block, 8 columns): the mean of tokens 4j .. 4j+3 summed in
// fp64 (exact for bf16 tokens) and rounded once to fp32, stored in plane d/4 of the head
// ([BH][D/4][nK][4]); the key's D/8 threads then combine its squared norm.
template <int D>
__global__ __launch_bounds__(256) void fine_pool_kernel(const __bf16 *__restrict__ k, float *__restrict__ kf,
                                                        float *__restrict__ knorm, int64_t nK, int64_t nkeys,
                                                        PoolSide side) {
    constexpr int CPK = D / 8;   // threads per key
    const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blockIdx.x == 0 && (int)threadIdx.x < side.n_thr) side.thr_dst[threadIdx.x] = side.thr.v[threadIdx.x];
    for (int64_t i = gt; i < side.n_status; i += (int64_t)gridDim.x * blockDim.x) side.status[i] = 0;
    if (gt == 0) {
        side.ticket[0] = 0u;
        side.ticket[1] = 0u;
    }
    const int64_t jg = gt / CPK;   // key block over all heads
    const int c = (int)(gt % CPK);
    const bool ok = jg < nkeys;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ok) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(k + (4 * jg + u) * D + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += (double)bf16_lo(w[e]);
                acc[2 * e + 1] += (double)bf16_hi(w[e]);
            }
        }
    }
    float m[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        m[e] = (float)(acc[e] * 0.25);
        ss = __builtin_fmaf(m[e], m[e], ss);
    }
    if (ok) {
        const int64_t bh = jg / nK, j = jg - bh * nK;
        float *plane = kf + (bh * (D / 4) + 2 * c) * nK * 4;
        *reinterpret_cast<f32x4 *>(plane + j * 4) = f32x4{m[0], m[1], m[2], m[3]};
        *reinterpret_cast<f32x4 *>(plane + nK * 4 + j * 4) = f32x4{m[4], m[5], m[6], m[7]};
    }
#pragma unroll
    for (int o = 1; o < CPK; o <<= 1) ss += __shfl_xor(ss, o, 64);
    if (ok && c == 0) knorm[jg] = sqrtf(ss);
}

namespace {

// Exact mean of one 64-token bf16 block by one wave (fp64; the sum of 64 bf16 values
// is exact and 1/64 is a power of two).  Lane l covers token rows l / LPR + RPW * it
// and columns 8 (l % LPR) .. +8; lanes 0 .. LPR-1 return the means of their columns.
template <int D> __device__ __forceinline__ void block_mean64(const __bf16 *blk, int lane, double (&x)[8]) {
    constexpr int LPR = D / 8, RPW = 64 / LPR;
    const __bf16 *p = blk + (lane / LPR) * D + 8 * (lane % LPR);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.0;
#pragma unroll 4
    for (int it = 0; it < 64 / RPW; ++it) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p + it * RPW * D);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] += (double)bf16_lo(w[e]);
            x[2 * e + 1] += (double)bf16_hi(w[e]);
        }
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += __shfl_xor(x[e], o, 64);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= 1.0 / 64.0;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

}  // namespace

// Row state in LDS, per row of the group (all threads read it; thread r < R writes row r).
struct FineRow {
    float Z, thrZ, Mlo, Mhi;   // row mass; its thr share; masses above lo and above hi
    float vstar, M, band;      // crossing value, mass strictly above it, relative band half-width
    uint32_t lo, hi;           // bracket (fp32 bit patterns of e): v* lies in (lo, hi]
    uint32_t clo, chi;         // keys above lo, above hi
    uint32_t done;             // no cut: padding row, or keep every block
    uint32_t ncand;            // compaction counter
    uint32_t tkeep;            // ties at v* that are kept (lowest indices first)
    uint32_t nband, mband;     // near-tie band: blocks, of which kept by the fp32 cut
    uint32_t refine;           // the band is ordered again exactly
};

template <int D, int W, int R>
__global__ __launch_bounds__(1024) void fine_select_kernel(FineArgs a) {
    static_assert(W * R <= 64 && R <= 16, "register row budget");
    constexpr int NW = kFineWaves;
    __shared__ __align__(16) float qf[R][D];   // query means, fp32 (scores)
    __shared__ double q64[R][D];               // query means, fp64 (exact rescoring)
    __shared__ float red_f[R][NW];
    __shared__ float red_g[R][NW];
    __shared__ uint32_t red_u[R][NW];
    __shared__ FineRow row[R];
    __shared__ uint32_t cand[R][64];
    __shared__ uint32_t band[R][64];           // band blocks; bit 31 = kept after the exact order
    __shared__ int32_t cnt_rw[R][NW];          // kept blocks per (row, wave)
    __shared__ int32_t tie_rw[R][NW];          // blocks equal to v* per (row, wave)
    __shared__ float s_kmax[NW];
    __shared__ uint32_t s_ticket;
    __shared__ int64_t s_base;
    __shared__ int32_t s_gave_up;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (threadIdx.x == 0) s_ticket = atomicAdd(a.ticket, 1u);
    __syncthreads();
    const uint32_t g = __builtin_amdgcn_readfirstlane(s_ticket);
    const uint32_t bh = g / (uint32_t)a.groups_per_head;
    const int i0 = (int)(g - bh * (uint32_t)a.groups_per_head) * R;
    const int nrows = min(R, a.nB - i0);
    const float thr = a.thr[bh % (uint32_t)a.H];
    const bool keep_all = !(thr < 1.f);
    const int kbase = wave * a.S;          // this wave's key slice: kbase .. kbase + S - 1
    const int slice = min(a.S, a.nK - kbase);   // keys of the slice that exist (may be <= 0)

    // ---- the group's query means, one wave per row
    if (wave < R) {
        if (wave < nrows) {
            double x[8];
            block_mean64<D>(a.q + (((int64_t)bh * a.nB + i0 + wave) * 64) * D, lane, x);
            if (lane < D / 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    q64[wave][8 * lane + e] = x[e];
                    qf[wave][8 * lane + e] = (float)x[e];
                }
            }
        } else {
            for (int e = lane; e < D; e += 64) {
                q64[wave][e] = 0.0;
                qf[wave][e] = 0.f;
            }
        }
    }
    // ---- the largest key-mean norm of the slice (for the scores' error bound)
    {
        float mx = 0.f;
        for (int t = lane; t < slice; t += 64) mx = fmaxf(mx, a.knorm[(int64_t)bh * a.nK + kbase + t]);
        mx = wave_max_u(mx);
        if (lane == 0) s_kmax[wave] = mx;
    }
    __syncthreads();

    // ---- scores: fp32 FMAs of the query means (LDS, broadcast) with this lane's keys
    //      kbase + 64 w + lane (planes of 4 columns: a wave reads 1 KiB runs)
    float s[R][W];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int w = 0; w < W; ++w) s[r][w] = 0.f;
    {
        // four words at a time (their operands in registers), all d for each
        constexpr int WC = W < 4 ? W : 4;
        const float *kp = a.kf + (int64_t)bh * (D / 4) * a.nK * 4 + (int64_t)(kbase + lane) * 4;
#pragma unroll
        for (int w0 = 0; w0 < W; w0 += WC) {
#pragma unroll 2
            for (int d4 = 0; d4 < D / 4; ++d4) {
                f32x4 kv[WC];
#pragma unroll
                for (int w = 0; w < WC; ++w)
                    kv[w] = 64 * (w0 + w) + lane < slice
                                ? *reinterpret_cast<const f32x4 *>(kp + ((int64_t)d4 * a.nK + 64 * (w0 + w)) * 4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const f32x4 qv = *reinterpret_cast<const f32x4 *>(&qf[r][4 * d4]);
#pragma unroll
                    for (int w = 0; w < WC; ++w) {
                        float t = s[r][w0 + w];
                        t = __builtin_fmaf(qv[0], kv[w][0], t);
                        t = __builtin_fmaf(qv[1], kv[w][1], t);
                        t = __builtin_fmaf(qv[2], kv[w][2], t);
                        s[r][w0 + w] = __builtin_fmaf(qv[3], kv[w][3], t);
                    }
                }
            }
        }
        // log2 units; keys outside the slice are -inf
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                s[r][w] = 64 * w + lane < slice ? s[r][w] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, s[r][w]);
            }
            mx = wave_max_u(mx);
            if (lane == 0) red_f[r][wave] = mx;
        }
    }
    __syncthreads();
    // ---- e = 2^(s - row max) in place (the row max becomes exactly 1), Z and the count
    //      of positive e
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red_f[r][w]);
        float z = 0.f;
        uint32_t n = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            s[r][w] = __builtin_amdgcn_exp2f(s[r][w] - mx);
            z += s[r][w];
            n += (uint32_t)__popcll(__ballot(s[r][w] > 0.f));
        }
        z = wave_sum_u(z);
        if (lane == 0) {
            red_g[r][wave] = z;
            red_u[r][wave] = n;
        }
    }
    __syncthreads();
    if (threadIdx.x < R) {
        const int r = threadIdx.x;
        float Z = 0.f;
        uint32_t n = 0;
        for (int w = 0; w < NW; ++w) {
            Z += red_g[r][w];
            n += red_u[r][w];
        }
        FineRow &o = row[r];
        o.Z = Z;
        o.thrZ = thr * Z;
        o.Mlo = Z;              // every positive key is above lo = +0
        o.Mhi = 0.f;            // no key is above hi = 1 (the row max)
        o.lo = 0u;
        o.hi = 0x3f800000u;
        o.clo = n;
        o.chi = 0u;
        o.done = (r >= nrows || keep_all) ? 1u : 0u;
        o.ncand = 0u;
    }
    __syncthreads();

    // ---- pivot search on the fp32 bit patterns of e (they order like the values):
    //      each step splits the bracket (lo, hi] of every unfinished row at a pivot
    //      (interpolated on the masses at even steps and the first two, else the middle
    //      of the bit range), the waves' masses and counts above it meet in LDS, and
    //      thread r moves row r's bracket.  A row is finished once its bracket holds at
    //      most 64 keys, or a single value.  The pivot stays strictly inside the bracket,
    //      so the bracket shrinks every step and 64 steps end every row.
    auto active = [&](int r) {
        const FineRow &o = row[r];
        return !o.done && o.clo - o.chi > 64u && o.hi - o.lo > 1u;
    };
#pragma unroll 1
    for (int step = 0; step < 80; ++step) {
        uint32_t pv[R];
        bool any = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const FineRow &o = row[r];
            uint32_t p = 0xffffffffu;   // a finished row: no key is above it
            if (active(r)) {
                any = true;
                if (step < 2 || (step & 1) == 0) {
                    const float vlo = __uint_as_float(o.lo), vhi = __uint_as_float(o.hi);
                    const float f = (o.thrZ - o.Mhi) / (o.Mlo - o.Mhi);
                    p = __float_as_uint(vhi - f * (vhi - vlo));
                } else {
                    p = o.lo + ((o.hi - o.lo) >> 1);
                }
                p = min(max(p, o.lo + 1u), o.hi - 1u);
            }
            pv[r] = p;
        }
        if (!any) break;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc = 0.f;
            uint32_t cnt = 0;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const bool gt = __float_as_uint(s[r][w]) > pv[r];
                acc += gt ? s[r][w] : 0.f;
                cnt += (uint32_t)__popcll(__ballot(gt));
            }
            acc = wave_sum_u(acc);
            if (lane == 0) {
                red_f[r][wave] = acc;
                red_u[r][wave] = cnt;
            }
        }
        __syncthreads();
        if (threadIdx.x < R) {
            const int r = threadIdx.x;
            if (active(r)) {
                float A = 0.f;
                uint32_t c = 0;
                for (int w = 0; w < NW; ++w) {
                    A += red_f[r][w];
                    c += red_u[r][w];
                }
                FineRow &o = row[r];
                if (A < o.thrZ) {
                    o.hi = pv[r];
                    o.Mhi = A;
                    o.chi = c;
                } else {
                    o.lo = pv[r];
                    o.Mlo = A;
                    o.clo = c;
                }
            }
        }
        __syncthreads();
    }

    // ---- the <= 64 keys of a finished bracket to LDS; one wave per row sorts them
    //      (descending) and finds the crossing value v* and the mass M above it.  A
    //      bracket of one value (or of more than 64 keys) crosses at hi.
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const FineRow &o = row[r];
        if (!o.done && o.clo - o.chi <= 64u) {
            const uint32_t lo = o.lo, hi = o.hi;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const uint32_t u = __float_as_uint(s[r][w]);
                if (u > lo && u <= hi) cand[r][atomicAdd(&row[r].ncand, 1u)] = u;
            }
        }
    }
    __syncthreads();
    if (wave < R) {
        const int r = wave;
        const FineRow &o = row[r];
        float vstar = __uint_as_float(o.hi), M = o.Mhi;
        if (!o.done && o.clo - o.chi <= 64u && o.clo > o.chi) {
            const uint32_t n = o.ncand;
            uint32_t u = (uint32_t)lane < n ? cand[r][lane] : 0u;
            // bitonic sort, descending over the 64 lanes
#pragma unroll
            for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
                for (int j = kk >> 1; j > 0; j >>= 1) {
                    const uint32_t v = (uint32_t)__shfl_xor((int)u, j, 64);
                    const bool desc = (lane & kk) == 0;
                    const bool low = (lane & j) == 0;
                    u = (low == desc) ? max(u, v) : min(u, v);
                }
            }
            const float e = __uint_as_float(u);
            const float incl = wave_prefix_sum(e, lane);
            const uint64_t reach = __ballot((uint32_t)lane < n && o.Mhi + incl >= o.thrZ);
            const int L = reach ? __builtin_ctzll(reach) : (int)n - 1;
            const uint32_t vs = (uint32_t)__builtin_amdgcn_readlane((int)u, L);
            vstar = __uint_as_float(vs);
            M = o.Mhi + wave_sum_u(u > vs ? e : 0.f);
        }
        // half-width of the near-tie band, relative to v*: the scores' fp32 error bound
        // for two keys of the row (dot products of D terms of fp32 means, the means'
        // own rounding and the scaling), in log2 units, plus the exponential's rounding
        float qq = 0.f;
        for (int e = lane; e < D; e += 64) qq += qf[r][e] * qf[r][e];
        const float qn = sqrtf(wave_sum_u(qq));
        float kmax = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) kmax = fmaxf(kmax, s_kmax[w]);
        const float ds = 2.f * (float)(D + 4) * 0x1p-24f * a.scale_log2 * qn * kmax * 1.01f;
        if (lane == 0) {
            row[r].vstar = vstar;
            row[r].M = M;
            row[r].band = __builtin_amdgcn_exp2f(ds) - 1.f + 0x1p-20f;
        }
    }
    __syncthreads();

    // ---- ties at v*: counted per wave; thread r keeps them in index order while the
    //      mass before each stays below thr Z
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float vs = row[r].vstar;
        uint32_t n = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) n += (uint32_t)__popcll(__ballot(s[r][w] == vs && vs > 0.f));
        if (lane == 0) tie_rw[r][wave] = (int32_t)n;
    }
    __syncthreads();
    if (threadIdx.x < R) {
        const int r = threadIdx.x;
        FineRow &o = row[r];
        uint32_t neq = 0;
        for (int w = 0; w < NW; ++w) neq += (uint32_t)tie_rw[r][w];
        uint32_t t = 0;
        while (t < neq && o.M + (float)t * o.vstar < o.thrZ) ++t;
        o.tkeep = t;
        o.ncand = 0u;
    }
    __syncthreads();

    // The fp32 cut of word w of row r: above v*, or a tie within the kept ranks (tb: ties
    // of the row before this word, advanced here).  inb: in the near-tie band.
    auto cut_word = [&](float sv, bool real, const FineRow &o, uint32_t &tb, bool &inb) -> bool {
        const bool eq = sv == o.vstar && o.vstar > 0.f;
        const uint64_t eqm = __ballot(eq);
        const uint32_t rank = tb + lanes_below(eqm);
        tb += (uint32_t)__popcll(eqm);
        inb = !o.done && sv > 0.f && sv >= o.vstar * (1.f - o.band) && sv <= o.vstar * (1.f + o.band);
        return real && (keep_all || sv > o.vstar || (eq && rank < o.tkeep));
    };
    int32_t tie_before[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        tie_before[r] = 0;
        for (int w = 0; w < wave; ++w) tie_before[r] += tie_rw[r][w];
    }

    // ---- the near-tie band of each row: its blocks, and how many the fp32 cut keeps
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const FineRow &o = row[r];
        uint32_t tb = (uint32_t)tie_before[r], nb = 0, mb = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            bool inb;
            const bool k = cut_word(s[r][w], 64 * w + lane < slice, o, tb, inb);
            nb += (uint32_t)__popcll(__ballot(inb));
            mb += (uint32_t)__popcll(__ballot(inb && k));
        }
        if (lane == 0) {
            red_u[r][wave] = nb;
            cnt_rw[r][wave] = (int32_t)mb;
        }
    }
    __syncthreads();
    if (threadIdx.x < R) {
        const int r = threadIdx.x;
        FineRow &o = row[r];
        uint32_t nb = 0, mb = 0;
        for (int w = 0; w < NW; ++w) {
            nb += red_u[r][w];
            mb += (uint32_t)cnt_rw[r][w];
        }
        o.nband = nb;
        o.mband = mb;
        o.refine = (!o.done && nb >= 2u && nb <= 64u && mb > 0u && mb < nb) ? 1u : 0u;
    }
    __syncthreads();
    // ---- rows whose band holds kept and dropped blocks: the band's blocks to LDS, then
    //      one wave per row scores them exactly (the fp64 query mean against the exact
    //      mean of the 4 key tokens) and keeps the mband best (lower index on a tie)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const FineRow &o = row[r];
        if (!o.refine) continue;
        uint32_t tb = (uint32_t)tie_before[r];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            bool inb;
            (void)cut_word(s[r][w], 64 * w + lane < slice, o, tb, inb);
            if (inb) band[r][atomicAdd(&row[r].ncand, 1u)] = (uint32_t)(kbase + 64 * w + lane);
        }
    }
    __syncthreads();
    if (wave < R && row[wave].refine) {
        const int r = wave, nb = (int)row[r].nband, m = (int)row[r].mband;
        const int my_j = lane < nb ? (int)band[r][lane] : 0x7fffffff;
        double my_s = 0.0;
        constexpr int DPL = D / 64;
        for (int n = 0; n < nb; ++n) {
            const int j = __builtin_amdgcn_readfirstlane((int)band[r][n]);
            const __bf16 *kt = a.k + ((int64_t)bh * a.nK + j) * 4 * D;
            double part = 0.0;
#pragma unroll
            for (int u = 0; u < DPL; ++u) {
                const int dd = DPL * lane + u;
                const double km = (((double)(float)kt[dd] + (double)(float)kt[D + dd]) +
                                   ((double)(float)kt[2 * D + dd] + (double)(float)kt[3 * D + dd])) * 0.25;
                part = __builtin_fma(q64[r][dd], km, part);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
            if (lane == n) my_s = part;
        }
        int rank = 0;
        for (int n = 0; n < nb; ++n) {
            const double sn = __shfl(my_s, n, 64);
            const int jn = __shfl(my_j, n, 64);
            rank += (sn > my_s || (sn == my_s && jn < my_j)) ? 1 : 0;
        }
        if (lane < nb) band[r][lane] = (uint32_t)my_j | (rank < m ? 0x80000000u : 0u);
    }
    __syncthreads();

    // The final decision of word w of row r: the fp32 cut, or the exact order in the band.
    auto keep_word = [&](int r, float sv, bool real, const FineRow &o, uint32_t &tb, int j) -> bool {
        bool inb;
        bool k = cut_word(sv, real, o, tb, inb);
        if (o.refine && inb) {
            for (uint32_t n = 0; n < o.nband; ++n) {
                const uint32_t bw = band[r][n];
                if ((int)(bw & 0x7fffffffu) == j) k = (bw >> 31) != 0u;
            }
        }
        return k;
    };

    // ---- counts per (row, wave), the group's offset by look-back, and the columns
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const FineRow &o = row[r];
        uint32_t tb = (uint32_t)tie_before[r];
        int c = 0;
#pragma unroll
        for (int w = 0; w < W; ++w)
            c += __popcll(__ballot(keep_word(r, s[r][w], 64 * w + lane < slice, o, tb, kbase + 64 * w + lane)));
        if (lane == 0) cnt_rw[r][wave] = c;
    }
    __syncthreads();
    if (wave == 0) {
        int v = 0;
        for (int t = lane; t < nrows * NW; t += 64) v += cnt_rw[t / NW][t % NW];
        const int total = wave_sum_i(v);
        bool gave_up;
        const int64_t base = group_lookback(a.status, g, total, lane, a.spin_cap, gave_up);
        if (lane == 0) {
            s_base = base;
            s_gave_up = gave_up;
            if (gave_up) __hip_atomic_store(a.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    int64_t pos = s_base;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r >= nrows) break;
        const FineRow &o = row[r];
        const int64_t grow = (int64_t)bh * a.nB + i0 + r;
        int before = 0, total = 0;
        for (int w = 0; w < NW; ++w) {
            before += w < wave ? cnt_rw[r][w] : 0;
            total += cnt_rw[r][w];
        }
        if (wave == 0 && lane == 0) {
            a.row_ptr[grow] = s_gave_up ? -1 : (int32_t)pos;
            if (grow == a.rows - 1) a.row_ptr[a.rows] = s_gave_up ? -1 : (int32_t)(pos + total);
        }
        if (!s_gave_up) {
            int64_t at = pos + before;
            uint32_t tb = (uint32_t)tie_before[r];
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const int j = kbase + 64 * w + lane;
                const bool k = keep_word(r, s[r][w], 64 * w + lane < slice, o, tb, j);
                const uint64_t m = __ballot(k);
                if (k) a.col_idx[at + lanes_below(m)] = j;
                at += __popcll(m);
            }
        }
        pos += total;
    }
}

int launch_fine_pool(const __bf16 *k, float *kf, float *knorm, int64_t nK, int64_t nkeys, int d, const PoolSide &side,
                     hipStream_t s) {
    const int64_t threads = nkeys * (d / 8);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (d == 128)
        fine_pool_kernel<128><<<grid, block, 0, s>>>(k, kf, knorm, nK, nkeys, side);
    else
        fine_pool_kernel<64><<<grid, block, 0, s>>>(k, kf, knorm, nK, nkeys, side);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Words per lane W (keys of a wave's slice / 64, a power of two; up to 8, i.e. nB <=
// 512) and rows per workgroup R (R W <= 64 registers for the scores).
int fine_words(int64_t nK) {
    const int64_t per = (nK + kFineWaves - 1) / kFineWaves;
    int w = 1;
    while (64 * (int64_t)w < per) w *= 2;
    return w;
}
int fine_rows(int W) { return W >= 8 ? 64 / W : 8; }

template <int D> static int launch_fine_d(const FineArgs &a, int W, hipStream_t s) {
    const dim3 g((unsigned)a.n_groups), b(64 * kFineWaves);
    switch (W) {
    case 1: fine_select_kernel<D, 1, 8><<<g, b, 0, s>>>(a); break;
    case 2: fine_select_kernel<D, 2, 8><<<g, b, 0, s>>>(a); break;
    case 4: fine_select_kernel<D, 4, 8><<<g, b, 0, s>>>(a); break;
    case 8: fine_select_kernel<D, 8, 8><<<g, b, 0, s>>>(a); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fine_select(const FineArgs &a, int d, hipStream_t s) {
    const int W = fine_words(a.nK);
    return d == 128 ? launch_fine_d<128>(a, W, s) : launch_fine_d<64>(a, W, s);
}

}  // namespace sattn
