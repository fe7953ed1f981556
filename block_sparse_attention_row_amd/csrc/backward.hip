// Block-sparse attention backward (gfx950, bf16 inputs, bf16 MFMA, fp32 accumulation).
//
// Gradients of the forward in attention.hip, for the training use of the NABLA
// summary page ("NABLA: Neighborhood Adaptive Block-Level Attention", sections
// "Methodologie : NABLA" and the training results).  With P the softmax weights
// recovered from the forward's log-sum-exp, P_nm = exp(scale q_n.k_m - lse_n), and an
// upstream gradient dO:
//   dV = P^T dO,  dP = dO V^T,  D_n = dO_n . O_n,  dS = P o (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Two passes, each writing whole output rows from one workgroup (no atomics, a
// fixed summation order):
//   dQ      a pair of query blocks walks its CSR rows (key tiles streamed into LDS):
//           S^T = K Q^T, dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T;
//   dV, dK  a pair of key blocks walks the transposed list (query tiles streamed):
//           S = Q K^T, P, dP = dO V^T, dS, then dV^T += dO^T P and dK^T += Q^T dS.
// Pairs are neighbours in time, as in the forward (pair_blocks).  Partial tiles
// (MASKED): padding queries carry lse2 = +inf from the prep kernel, so every P of
// theirs is 0 and they neither receive nor pass on gradient; the dQ pass masks the
// padding keys of the key tiles it streams, and the dV/dK pass writes zero rows for
// the padding keys it owns.  Each pass is the
// forward's tile machinery with other operands: the streamed tile is
// the A operand of the scores and, read transposed, of the output product; the
// pair's own rows sit in registers as the B operand.  The transposed list (for
// every key block, the query blocks that keep it, ascending) is built from row
// bitmasks, so it is deterministic and applies the forward's skip rule.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace sattn {

// ---------------------------------------------------------------------------
// D_n = dO_n . O_n and lse_n in log2 units, one token per D/8 lanes.  A token whose
// LSE is -inf (a padding query, or a query block that keeps no tile) gets lse2 = +inf,
// so that every softmax weight recovered for it in the passes is 0.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16 *__restrict__ o, const __bf16 *__restrict__ dout,
                                                       const float *__restrict__ lse, float *__restrict__ lse2,
                                                       float *__restrict__ dn, int64_t ntok) {
    constexpr int LPT = D / 8, TPW = 64 / LPT;
    const int lane = threadIdx.x & 63;
    const int64_t tok = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW + lane / LPT;
    float acc = 0.f;
    if (tok < ntok) {
        const bf16x8 x = *reinterpret_cast<const bf16x8 *>(o + tok * D + 8 * (lane % LPT));
        const bf16x8 g = *reinterpret_cast<const bf16x8 *>(dout + tok * D + 8 * (lane % LPT));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)g[e];
    }
#pragma unroll
    for (int off = 1; off < LPT; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (tok < ntok && lane % LPT == 0) {
        dn[tok] = acc;
        const float l = lse[tok];
        lse2[tok] = l == -INFINITY ? INFINITY : l * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// Transposed block list.
//
// Row bitmasks with the forward's skip rule: an entry counts when it lies in [0, nB)
// and above every entry the row accepted before it (a prefix max over the lanes).
__global__ __launch_bounds__(256) void csr_bits_kernel(const int32_t *__restrict__ row_ptr,
                                                       const int32_t *__restrict__ col_idx, int64_t col_count,
                                                       int64_t rows, int32_t nB, int32_t nW,
                                                       uint64_t *__restrict__ bits) {
    __shared__ unsigned long long wb[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= rows) return;
    if (lane < nW) wb[wave][lane] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int64_t beg = row_ptr[row], end = row_ptr[row + 1];
    end = end < col_count ? end : col_count;
    beg = beg < 0 ? 0 : beg;
    int carry = -1;
    for (int64_t base = beg; base < end; base += 64) {
        const int c = base + lane < end ? col_idx[base + lane] : -1;
        const bool valid = c >= 0 && c < nB;
        int incl = valid ? c : -1;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o, 64);
            if (lane >= o) incl = max(incl, u);
        }
        int excl = __shfl_up(incl, 1, 64);
        excl = max(carry, lane == 0 ? -1 : excl);
        if (valid && c > excl) atomicOr(&wb[wave][c >> 6], 1ull << (c & 63));
        carry = max(carry, __shfl(incl, 63, 64));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < nW) bits[row * nW + lane] = wb[wave][lane];
}

// One wave per (head, 64-column word): lane b owns column 64 w + b.  The rows are
// taken 64 at a time (lane l loads row r0 + l's word); per bit, a ballot over the
// lanes gives the rows that keep that column.  COUNT: columns' totals; else the
// rows are written to their column's list in ascending order.
template <bool COUNT>
__global__ __launch_bounds__(256) void csc_pass_kernel(const uint64_t *__restrict__ bits, int64_t BH, int32_t nB,
                                                       int32_t nW, int32_t *__restrict__ colcount,
                                                       const int32_t *__restrict__ col_ptr,
                                                       int32_t *__restrict__ row_idx) {
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= BH * nW) return;
    const int64_t bh = wv / nW;
    const int w = (int)(wv % nW);
    const int col = 64 * w + lane;
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int run = 0;                                          // rows found so far for column 64 w + lane
    const int cp = (!COUNT && col < nB) ? col_ptr[bh * nB + col] : 0;
    for (int r0 = 0; r0 < nB; r0 += 64) {
        const uint64_t word = r0 + lane < nB ? bits[(bh * nB + r0 + lane) * nW + w] : 0ull;
        for (int b = 0; b < 64; ++b) {
            const bool set = (word >> b) & 1ull;
            const uint64_t m = __ballot(set);
            if (!COUNT && set) {
                const int pos = __builtin_amdgcn_readlane(cp, b) + __builtin_amdgcn_readlane(run, b) +
                                __popcll(m & lt_mask);
                row_idx[pos] = r0 + lane;
            }
            if (lane == b) run += __popcll(m);
        }
    }
    if (COUNT && col < nB) colcount[bh * nB + col] = run;
}

// Exclusive prefix of n counts into out[0 .. n] (one workgroup).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t *__restrict__ in, int64_t n,
                                                    int32_t *__restrict__ out) {
    __shared__ int32_t part[16];
    int32_t carry = 0;
    for (int64_t b0 = 0; b0 < n; b0 += 1024) {
        const int64_t i = b0 + threadIdx.x;
        int32_t total;
        const int32_t ex = block_scan32(i < n ? in[i] : 0, part, total);
        if (i < n) out[i] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) out[n] = carry;
}

// ---------------------------------------------------------------------------
// The gradient passes: dQ over the block rows, dV and dK together over the transposed list.
enum BwdMode { kDQ = 0, kDKV = 1 };

// kDKV: dV and dK in one walk of the transposed list (S and dP once per tile, four
// products; 8% faster at d = 128 than a dV pass and a dK pass that each form S);
// at d = 128 its two d-wide accumulators take one wave per SIMD, so there its tile
// runs in phases with the softmax work beside the MFMAs and the fragment reads
// kDkvAhead MFMAs ahead of use (dkv_tile below); at d = 64 (two waves per SIMD) the
// other wave covers that work.
constexpr int kDkvAhead = 6;
template <int D, int MODE, bool MASKED>
__global__ __launch_bounds__(256, MODE == kDKV && D == 128 ? 1 : 2) void bwd_kernel(BwdArgs a) {
    using G = TileGeo<D>;
    constexpr int ROWB = G::ROWB, SLOTS = G::SLOTS, RPI = G::RPI, IPW = G::IPW, NDT = G::NDT, TILEB = G::TILEB;
    __shared__ __attribute__((aligned(1024))) char T1s[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char T2s[2 * TILEB];
    __shared__ __attribute__((aligned(16))) float aux[2][256];   // per buffer: lse2 [64], D [64] of the streamed block

    const int t = threadIdx.x, lane = t & 63, hh = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 1, half = wave & 1;   // block of the pair, 32-row half of the block
    // work item, as in the forward: long-row pieces, then whole pairs that were not
    // split, then the last round's pieces
    const int64_t ls = a.plan.long_slots, bid = blockIdx.x;
    int64_t pair;
    SplitItem it = {};
    bool split = true;
    if (bid < ls) {
        if (bid >= a.plan.counts[0]) return;
        it = a.plan.items[bid];
        pair = it.pair;
    } else if (bid < ls + a.n_pairs) {
        split = false;
        pair = xcd_chunk_remap<256>(bid - ls, a.n_pairs);
        if (a.plan.pair_flag[pair]) return;
    } else {
        if (bid - ls - a.n_pairs >= a.plan.counts[3]) return;
        it = a.plan.items[bid - a.n_pairs];
        if (it.pair < 0) return;      // a last-round pair that was not cut
        pair = it.pair;
    }
    const int64_t bh = pair / a.pairs_per_head;
    int32_t blk_a, blk_b;   // the pair's two blocks, neighbours in time (pair_blocks)
    pair_blocks((int32_t)(pair % a.pairs_per_head), a.pair_stride, a.nB, blk_a, blk_b);
    const int64_t N = (int64_t)a.nB * 64;
    // streamed tiles: key tiles K, V for dQ; query tiles Q, dO for dV and dK
    const char *t1g = (const char *)(MODE == kDQ ? a.k : a.q) + bh * N * ROWB + 16 * wave * ROWB;
    const char *t2g = (const char *)(MODE == kDQ ? a.v : a.dout) + bh * N * ROWB + 16 * wave * ROWB;
    const float c = a.scale_log2;

    const int64_t rowA = bh * a.nB + blk_a, rowB = bh * a.nB + blk_b;
    const bool hasB = blk_b >= 0;
    auto clamp_range = [&](int64_t r, int64_t &b, int64_t &e) {
        b = a.ptr[r];
        e = a.ptr[r + 1];
        e = e < a.idx_count ? e : a.idx_count;
        b = b < 0 ? 0 : b;
        if (e < b) e = b;
    };
    int64_t begA, endA, begB = 0, endB = 0;
    int lastA = -1, lastB = -1;
    if (split) {
        begA = it.a0;
        endA = it.a1;
        begB = it.b0;
        endB = it.b1;
        // the whole-list walk would arrive at the piece with the largest valid block
        // of the entries before it as its last one
        auto prefix_max = [&](int64_t from, int64_t to) {
            int m = -1;
            for (int64_t i = from + lane; i < to; i += 64) {
                const int cc = a.idx[i];
                if (cc >= 0 && cc < a.nB) m = cc > m ? cc : m;
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const int u = __shfl_xor(m, o, 64);
                m = u > m ? u : m;
            }
            return __builtin_amdgcn_readfirstlane(m);
        };
        lastA = prefix_max(it.ra, begA);
        lastB = prefix_max(it.rb, begB);
    } else {
        clamp_range(rowA, begA, endA);
        if (hasB) clamp_range(rowB, begB, endB);
    }
    const bool has_row = grp == 0 || hasB;

    // the pair's own rows, B operands of the score products: queries and dO (dQ), keys
    // (dV), keys and V (dK); row 32 half + l32 of the pair's block grp, d = 16 cq + 8 hh ..
    const int64_t own = bh * N + (int64_t)(grp && hasB ? blk_b : blk_a) * 64 + 32 * half + l32;
    const __bf16 *o1 = (const __bf16 *)(MODE == kDQ ? a.q : a.k) + own * D;
    const __bf16 *o2 = (const __bf16 *)(MODE == kDQ ? a.dout : a.v) + own * D;
    bf16x8 f1[D / 16], f2[D / 16];
#pragma unroll
    for (int cq = 0; cq < D / 16; ++cq) {
        f1[cq] = has_row ? *reinterpret_cast<const bf16x8 *>(o1 + 16 * cq + 8 * hh) : bf16x8{};
        f2[cq] = has_row ? *reinterpret_cast<const bf16x8 *>(o2 + 16 * cq + 8 * hh) : bf16x8{};
    }
    const float lse2_q = (MODE == kDQ && has_row) ? a.lse2[own] : 0.f;
    const float d_q = (MODE == kDQ && has_row) ? a.dn[own] : 0.f;

    // merged walk over the two lists (as in the forward)
    constexpr int kNone = 0x7fffffff;
    const int32_t *cv = a.idx;
    auto window = [&](int64_t base, int64_t e) { return base + lane < e ? cv[base + lane] : kNone; };
    int64_t baseA = begA, baseB = begB;
    int posA = 0, posB = 0;
    int winA = window(baseA, endA), nxtA = window(baseA + 64, endA);
    int winB = window(baseB, endB), nxtB = window(baseB + 64, endB);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    auto peek = [&](int64_t &base, int &pos, int &win, int &nxt, int64_t e, int last) {
        while (base + pos < e) {
            if (pos == 64) {
                base += 64;
                pos = 0;
                win = nxt;
                nxt = window(base + 64, e);
            }
            const int cc = __builtin_amdgcn_readlane(win, pos);
            if (cc > last && cc < a.nB) return cc;
            ++pos;
        }
        return kNone;
    };
    auto next_union = [&](int &col, bool &mine) {
        const int cA = peek(baseA, posA, winA, nxtA, endA, lastA);
        const int cB = peek(baseB, posB, winB, nxtB, endB, lastB);
        col = cA < cB ? cA : cB;
        const bool inA = cA == col && col != kNone, inB = cB == col && col != kNone;
        if (inA) { lastA = cA; ++posA; }
        if (inB) { lastB = cB; ++posB; }
        mine = grp ? inB : inA;
    };

    // direct loads: this wave covers rows 16 w .. 16 w + 15 of each streamed tile;
    // for dV and dK wave 0 also brings the block's lse2 and D (lanes 0-15 and 16-31;
    // lanes 32-63 repeat them into the unused half of the buffer)
    uint32_t voff[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
        const int r = RPI * j + lane / SLOTS, sl = lane % SLOTS;
        voff[j] = r * ROWB + 16 * (sl ^ swz_key<SLOTS>(r));
    }
    const uint32_t t1s0 = (uint32_t)(uintptr_t)(lds_char *)T1s + 16 * wave * ROWB;
    const uint32_t t2s0 = (uint32_t)(uintptr_t)(lds_char *)T2s + 16 * wave * ROWB;
    const uint32_t ax0 = (uint32_t)(uintptr_t)(lds_char *)&aux[0][0];
    const uint32_t aux_voff = (uint32_t)((lane & 31) < 16 ? 16 * (lane & 15)
                                                           : (uint32_t)((const char *)a.dn - (const char *)a.lse2) +
                                                                 16 * (lane & 15));
    auto issue = [&](int64_t col, int buf) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) dma16(t1s0 + buf * TILEB + RPI * i * ROWB, voff[i], t1g + col * TILEB);
#pragma unroll
        for (int i = 0; i < IPW; ++i) dma16(t2s0 + buf * TILEB + RPI * i * ROWB, voff[i], t2g + col * TILEB);
        if (MODE != kDQ && wave == 0)
            dma16(ax0 + buf * 1024, aux_voff, (const char *)a.lse2 + (bh * N + col * 64) * 4);
    };

    FragOffsets<D> fo;
    fo.init(lane);
    f32x16 acc[NDT], acc2[NDT];     // acc2: dK of the fused pass
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            acc[i][v] = 0.f;
            acc2[i][v] = 0.f;
        }

    int col0, col1;
    bool mine0, mine1;
    next_union(col0, mine0);
    if (col0 != kNone) issue(col0, 0);

    // One tile of the fused dV/dK pass, as three MFMA phases with the softmax work
    // spread over them (the wave has its SIMD to itself, so VALU work beside no MFMA
    // leaves the matrix unit idle): S; then dP beside P (S complete), two of P's
    // elements after each MFMA; then dV^T += dO^T P beside dS (dP complete); then
    // dK^T += Q^T dS.  Fragment reads run kDkvAhead MFMAs ahead and consecutive MFMAs
    // use different accumulators.  Formulas and summation orders are those of the
    // unphased form, so the gradients are the same bit for bit.
    auto dkv_tile = [&](const char *T1, const char *T2, const float *ax, f32x16 *s, f32x16 *dp, bf16x8 *pf,
                        bf16x8 *pf2) {
        constexpr int NC = D / 16, NM = 2 * NC, PER = 32 / NM, AH = kDkvAhead, RR = 2 * AH;
        constexpr int NDT2 = TileGeo<D>::NDT, NV = 4 * NDT2, PERV = 32 / NV;
        // lse2 and D of the 64 streamed rows this lane's elements belong to
        float l2v[32], ddv[32];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const f32x4 lo_l = *reinterpret_cast<const f32x4 *>(ax + 16 * kc + 4 * hh);
            const f32x4 hi_l = *reinterpret_cast<const f32x4 *>(ax + 16 * kc + 8 + 4 * hh);
            const f32x4 lo_d = *reinterpret_cast<const f32x4 *>(ax + 64 + 16 * kc + 4 * hh);
            const f32x4 hi_d = *reinterpret_cast<const f32x4 *>(ax + 64 + 16 * kc + 8 + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                l2v[8 * kc + e] = lo_l[e];
                l2v[8 * kc + 4 + e] = hi_l[e];
                ddv[8 * kc + e] = lo_d[e];
                ddv[8 * kc + 4 + e] = hi_d[e];
            }
        }
        // S (alternating key halves)
        {
            auto frag = [&](int i) { return fo.kfrag(T1, i & 1, i >> 1); };
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s[0][v] = 0.f;
                s[1][v] = 0.f;
            }
            bf16x8 kf[RR];
#pragma unroll
            for (int j = 0; j < AH; ++j) kf[j] = frag(j);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                if (i + AH < NM) kf[(i + AH) % RR] = frag(i + AH);
                s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % RR], f1[i >> 1], s[i & 1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // dP beside P (fp32 P kept in s for dS)
        {
            auto frag = [&](int i) { return fo.kfrag(T2, i & 1, i >> 1); };
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                dp[0][v] = 0.f;
                dp[1][v] = 0.f;
            }
            bf16x8 kf[RR];
#pragma unroll
            for (int j = 0; j < AH; ++j) kf[j] = frag(j);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                if (i + AH < NM) kf[(i + AH) % RR] = frag(i + AH);
                dp[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % RR], f2[i >> 1], dp[i & 1], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int e = PER * i + u, kc = e >> 3;
                    const int q = 8 * (kc & 1) + (e & 7);
                    s[kc >> 1][q] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kc >> 1][q], c, -l2v[e]));
                    if ((e & 7) == 7) {
                        f32x8 pv;
#pragma unroll
                        for (int w = 0; w < 8; ++w) pv[w] = s[kc >> 1][8 * (kc & 1) + w];
                        pf[kc] = __builtin_convertvector(pv, bf16x8);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // dV^T += dO^T P beside dS, then dK^T += Q^T dS
        {
            auto frag = [&](const char *T, int i) { return fo.vfrag(T, i / NDT2, i % NDT2); };
            bf16x8 vf[RR];
#pragma unroll
            for (int j = 0; j < AH; ++j) vf[j] = frag(T2, j);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (i + AH < NV) vf[(i + AH) % RR] = frag(T2, i + AH);
                acc[i % NDT2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % RR], pf[i / NDT2], acc[i % NDT2], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < PERV; ++u) {
                    const int e = PERV * i + u, kc = e >> 3;
                    const int q = 8 * (kc & 1) + (e & 7);
                    s[kc >> 1][q] = s[kc >> 1][q] * (dp[kc >> 1][q] - ddv[e]);
                    if ((e & 7) == 7) {
                        f32x8 pv;
#pragma unroll
                        for (int w = 0; w < 8; ++w) pv[w] = s[kc >> 1][8 * (kc & 1) + w];
                        pf2[kc] = __builtin_convertvector(pv, bf16x8);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < AH; ++j) vf[j] = frag(T1, j);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (i + AH < NV) vf[(i + AH) % RR] = frag(T1, i + AH);
                acc2[i % NDT2] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % RR], pf2[i / NDT2], acc2[i % NDT2], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    auto step = [&](auto bj_tag) {
        constexpr int BJ = decltype(bj_tag)::value;
        wait_vmcnt<0>();            // this wave's part of tile j has landed
        next_union(col1, mine1);
        __syncthreads();            // ... and everyone's; the buffers of tile j-1 are free
        if (col1 != kNone) issue(col1, BJ ^ 1);
        if (!mine0) return;
        const char *T1 = T1s + BJ * TILEB, *T2 = T2s + BJ * TILEB;
        const float *ax = aux[BJ];
        f32x16 s[2], dp[2];
        bf16x8 pf[4], pf2[4];           // pf2: dS of the fused pass (pf holds P there)
        if constexpr (MODE == kDKV && D == 128) {
            dkv_tile(T1, T2, ax, s, dp, pf, pf2);
            return;
        }
        tile_scores<D>(T1, f1, fo, s);
        if constexpr (MASKED && MODE == kDQ) {
            // padding keys of a partial key tile: no weight (dP needs no mask, P = 0 there)
            const uint64_t km = a.slot_mask[__builtin_amdgcn_readfirstlane(col0)];
            if (km != ~0ull) mask_keys(s, km, hh);
        }
        tile_scores<D>(T2, f2, fo, dp);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            f32x4 lo_l, hi_l, lo_d, hi_d;   // lse2, D of the 8 streamed rows of this chunk (dV, dK)
            if (MODE != kDQ) {
                lo_l = *reinterpret_cast<const f32x4 *>(ax + 16 * kc + 4 * hh);
                hi_l = *reinterpret_cast<const f32x4 *>(ax + 16 * kc + 8 + 4 * hh);
                lo_d = *reinterpret_cast<const f32x4 *>(ax + 64 + 16 * kc + 4 * hh);
                hi_d = *reinterpret_cast<const f32x4 *>(ax + 64 + 16 * kc + 8 + 4 * hh);
            }
            f32x8 pv, pv2;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = s[kc >> 1][8 * (kc & 1) + e];
                const float l2 = MODE == kDQ ? lse2_q : (e < 4 ? lo_l[e] : hi_l[e - 4]);
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -l2));
                const float dd = MODE == kDQ ? d_q : (e < 4 ? lo_d[e] : hi_d[e - 4]);
                const float ds = p * (dp[kc >> 1][8 * (kc & 1) + e] - dd);
                if (MODE == kDKV) {
                    pv[e] = p;
                    pv2[e] = ds;
                } else {
                    pv[e] = ds;
                }
            }
            pf[kc] = __builtin_convertvector(pv, bf16x8);
            if (MODE == kDKV) pf2[kc] = __builtin_convertvector(pv2, bf16x8);
        }
        // dQ^T += K^T dS^T (K tile read transposed); dV^T += dO^T P; dK^T += Q^T dS
        tile_pv<D>(MODE == kDKV ? T2 : T1, pf, fo, acc);
        if (MODE == kDKV) tile_pv<D>(T1, pf2, fo, acc2);
    };
    while (col0 != kNone) {
        step(std::integral_constant<int, 0>{});
        col0 = col1;
        mine0 = mine1;
        if (col0 == kNone) break;
        step(std::integral_constant<int, 1>{});
        col0 = col1;
        mine0 = mine1;
    }

    if (!has_row) return;
    // lane owns row 32 half + l32 of its block, d = 32 dt + 8 rr + 4 hh + {0..3}
    const float mult = MODE == kDKV ? 1.f : a.scale;
    if constexpr (MASKED && MODE == kDKV) {
        // a padding key of the pair's own block: zero dV and dK rows
        if (!((a.slot_mask[grp && hasB ? blk_b : blk_a] >> (32 * half + l32)) & 1ull)) {
#pragma unroll
            for (int i = 0; i < NDT; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    acc[i][v] = 0.f;
                    acc2[i][v] = 0.f;
                }
        }
    }
    if (split) {
        // piece of a split pair: its scaled fp32 partial rows, summed by bwd_merge_kernel
        const int64_t at = ((int64_t)it.slot * 2 + grp) * (64 * D) + (32 * half + l32) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                f32x4 w, w2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w[e] = acc[dt][4 * rr + e] * mult;
                    w2[e] = acc2[dt][4 * rr + e] * a.scale;
                }
                *reinterpret_cast<f32x4 *>(a.part + at + 32 * dt + 8 * rr + 4 * hh) = w;
                if constexpr (MODE == kDKV) *reinterpret_cast<f32x4 *>(a.part2 + at + 32 * dt + 8 * rr + 4 * hh) = w2;
            }
        return;
    }
    __bf16 *og = (__bf16 *)a.grad + own * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = acc[dt][4 * rr + e] * mult;
            *reinterpret_cast<bf16x4 *>(og + 32 * dt + 8 * rr + 4 * hh) = __builtin_convertvector(w, bf16x4);
        }
    if constexpr (MODE == kDKV) {
        __bf16 *og2 = (__bf16 *)a.grad2 + own * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = acc2[dt][4 * rr + e] * a.scale;
                *reinterpret_cast<bf16x4 *>(og2 + 32 * dt + 8 * rr + 4 * hh) = __builtin_convertvector(w, bf16x4);
            }
    }
}

// Gradient rows of the split pairs: the sum of their pieces' partial rows, in piece
// order (deterministic), to bf16; grad2 from part2 when `two`.
template <int D>
__global__ __launch_bounds__(256) void bwd_merge_kernel(BwdArgs a, int two) {
    const int m = blockIdx.x;
    if (m >= a.plan.counts[1]) return;
    const int32_t *me = a.plan.merge + 3 * (int64_t)m;
    const int64_t pair = me[0];
    const int first = me[1], ns = me[2];
    const int64_t bh = pair / a.pairs_per_head;
    int32_t blk_a, blk_b;
    pair_blocks((int32_t)(pair % a.pairs_per_head), a.pair_stride, a.nB, blk_a, blk_b);
    const int64_t N = (int64_t)a.nB * 64;
    for (int g = 0; g < 2; ++g) {
        const int32_t blk = g ? blk_b : blk_a;
        if (blk < 0) continue;
        const int64_t orow = (bh * N + (int64_t)blk * 64) * D;
        for (int i = threadIdx.x; i < 64 * D / 4; i += blockDim.x) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
            for (int p = 0; p < ns; ++p) {
                const int64_t src = ((int64_t)(first + p) * 2 + g) * (64 * D) + 4 * i;
                s += *reinterpret_cast<const f32x4 *>(a.part + src);
                if (two) s2 += *reinterpret_cast<const f32x4 *>(a.part2 + src);
            }
            *reinterpret_cast<bf16x4 *>((__bf16 *)a.grad + orow + 4 * i) = __builtin_convertvector(s, bf16x4);
            if (two) *reinterpret_cast<bf16x4 *>((__bf16 *)a.grad2 + orow + 4 * i) = __builtin_convertvector(s2, bf16x4);
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: the same gradients with fp32 MFMA (v_mfma_f32_32x32x2_f32), in the plain
// form of the fp32 forward: one workgroup of 2 waves per block (32 rows a wave), one
// tile at a time through LDS, no pieces.  As in that forward, the k = 2 of each MFMA
// makes the score accumulators the operand of the next product element by element:
// accumulator v of half h of a lane holds tile row 32 h + 8 (v / 4) + 4 hh + v % 4
// against the lane's own row l32, which is the k = hh slot of that product.

// D_n = dO_n . O_n and lse2 (lse in log2 units, -inf turned to +inf), one token a thread.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_f32_kernel(const float *__restrict__ o, const float *__restrict__ dout,
                                                           const float *__restrict__ lse, float *__restrict__ lse2,
                                                           float *__restrict__ dn, int64_t ntok) {
    const int64_t tok = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tok >= ntok) return;
    const f32x4 *x = reinterpret_cast<const f32x4 *>(o + tok * D);
    const f32x4 *g = reinterpret_cast<const f32x4 *>(dout + tok * D);
    float acc = 0.f;
#pragma unroll 4
    for (int c = 0; c < D / 4; ++c) {
        const f32x4 a = x[c], b = g[c];
        acc += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
    }
    dn[tok] = acc;
    const float l = lse[tok];
    lse2[tok] = l == -INFINITY ? INFINITY : l * kLog2e;
}

// dQ: block row `row` walks its kept key tiles (the forward's skip rule).
//   S^T = K Q^T, dP^T = V dO^T, P = 2^(S c - lse2), dS = P (dP - D), dQ^T += K^T dS^T.
template <int D>
__global__ __launch_bounds__(128) void bwd_dq_f32_kernel(BwdArgs a, int64_t rows) {
    constexpr int KS = D + 1, NDT = D / 32;
    __shared__ float Ks[64 * KS];
    __shared__ float Vs[64 * KS];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, hh = lane >> 5, l32 = lane & 31;
    const int64_t row = xcd_remap(blockIdx.x, rows);
    const int64_t bh = row / a.nB;
    const int64_t N = (int64_t)a.nB * 64;
    const int64_t qrow = bh * N + (row % a.nB) * 64 + 32 * wave + l32;
    const float *kg = (const float *)a.k + bh * N * D;
    const float *vg = (const float *)a.v + bh * N * D;
    float qf[D / 2], gf[D / 2];
#pragma unroll
    for (int c = 0; c < D / 2; ++c) {
        qf[c] = ((const float *)a.q)[qrow * D + 2 * c + hh];
        gf[c] = ((const float *)a.dout)[qrow * D + 2 * c + hh];
    }
    const float l2 = a.lse2[qrow], dq = a.dn[qrow];
    f32x16 acc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

    int64_t beg = a.ptr[row], end = a.ptr[row + 1];
    end = end < a.idx_count ? end : a.idx_count;
    beg = beg < 0 ? 0 : beg;
    const bool partial = a.geo.partial != 0;
    int last = -1;
    for (int64_t e = beg; e < end; ++e) {
        const int col = a.idx[e];
        if (col <= last || col >= a.nB) continue;
        last = col;
        const uint64_t km = partial ? __ballot(slot_valid(a.geo, col, lane)) : ~0ull;
        __syncthreads();
        const float *kt = kg + (int64_t)col * 64 * D, *vt = vg + (int64_t)col * 64 * D;
        for (int c = t; c < 64 * D / 4; c += 128) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(kt + 4 * c);
            const f32x4 vv = *reinterpret_cast<const f32x4 *>(vt + 4 * c);
            const int key = (4 * c) / D, d4 = (4 * c) % D;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                Ks[key * KS + d4 + u] = kv[u];
                Vs[key * KS + d4 + u] = vv[u];
            }
        }
        __syncthreads();
        f32x16 sc[2], dp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                sc[h][v] = 0.f;
                dp[h][v] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < D / 2; ++c) {
                sc[h] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[(32 * h + l32) * KS + 2 * c + hh], qf[c], sc[h], 0, 0, 0);
                dp[h] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[(32 * h + l32) * KS + 2 * c + hh], gf[c], dp[h], 0, 0, 0);
            }
        }
        if (km != ~0ull) mask_keys(sc, km, hh);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[h][v], a.scale_log2, -l2));
                sc[h][v] = p * (dp[h][v] - dq);
            }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = 32 * h + 8 * (v >> 2) + 4 * hh + (v & 3);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[key * KS + 32 * dt + l32], sc[h][v], acc[dt], 0, 0, 0);
            }
    }
    float *og = (float *)a.grad + qrow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 w;
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = acc[dt][4 * rr + u] * a.scale;
            *reinterpret_cast<f32x4 *>(og + 32 * dt + 8 * rr + 4 * hh) = w;
        }
}

// dV and dK: key block `row` walks the query blocks that keep it (the transposed list).
//   S = Q K^T, dP = dO V^T, P, dS as above; dV^T += dO^T P, dK^T += Q^T dS.
template <int D>
__global__ __launch_bounds__(128) void bwd_dkv_f32_kernel(BwdArgs a, int64_t rows) {
    constexpr int KS = D + 1, NDT = D / 32;
    __shared__ float Qs[64 * KS];
    __shared__ float Gs[64 * KS];
    __shared__ float Ls[64], Dd[64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, hh = lane >> 5, l32 = lane & 31;
    const int64_t row = xcd_remap(blockIdx.x, rows);
    const int64_t bh = row / a.nB;
    const int64_t N = (int64_t)a.nB * 64;
    const int32_t kb = (int32_t)(row % a.nB);
    const int64_t krow = bh * N + (int64_t)kb * 64 + 32 * wave + l32;
    const float *qg = (const float *)a.q + bh * N * D;
    const float *gg = (const float *)a.dout + bh * N * D;
    float kf[D / 2], vf[D / 2];
#pragma unroll
    for (int c = 0; c < D / 2; ++c) {
        kf[c] = ((const float *)a.k)[krow * D + 2 * c + hh];
        vf[c] = ((const float *)a.v)[krow * D + 2 * c + hh];
    }
    f32x16 adv[NDT], adk[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            adv[i][v] = 0.f;
            adk[i][v] = 0.f;
        }
    int64_t beg = a.ptr[row], end = a.ptr[row + 1];
    end = end < a.idx_count ? end : a.idx_count;
    beg = beg < 0 ? 0 : beg;
    for (int64_t e = beg; e < end; ++e) {
        const int qb = a.idx[e];          // the transposed list holds valid, ascending blocks
        __syncthreads();
        const int64_t q0 = (int64_t)qb * 64;
        const float *qt = qg + q0 * D, *gt = gg + q0 * D;
        for (int c = t; c < 64 * D / 4; c += 128) {
            const f32x4 qv = *reinterpret_cast<const f32x4 *>(qt + 4 * c);
            const f32x4 gv = *reinterpret_cast<const f32x4 *>(gt + 4 * c);
            const int r = (4 * c) / D, d4 = (4 * c) % D;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                Qs[r * KS + d4 + u] = qv[u];
                Gs[r * KS + d4 + u] = gv[u];
            }
        }
        if (t < 64) {
            Ls[t] = a.lse2[bh * N + q0 + t];
            Dd[t] = a.dn[bh * N + q0 + t];
        }
        __syncthreads();
        f32x16 sc[2], dp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                sc[h][v] = 0.f;
                dp[h][v] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < D / 2; ++c) {
                sc[h] = __builtin_amdgcn_mfma_f32_32x32x2f32(Qs[(32 * h + l32) * KS + 2 * c + hh], kf[c], sc[h], 0, 0, 0);
                dp[h] = __builtin_amdgcn_mfma_f32_32x32x2f32(Gs[(32 * h + l32) * KS + 2 * c + hh], vf[c], dp[h], 0, 0, 0);
            }
        }
        // P and dS of query 32 h + 8 (v / 4) + 4 hh + v % 4 against this lane's key
        // (padding queries carry lse2 = +inf: P = 0)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int qi = 32 * h + 8 * (v >> 2) + 4 * hh + (v & 3);
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[h][v], a.scale_log2, -Ls[qi]));
                sc[h][v] = p;
                dp[h][v] = p * (dp[h][v] - Dd[qi]);
            }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int qi = 32 * h + 8 * (v >> 2) + 4 * hh + (v & 3);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    adv[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Gs[qi * KS + 32 * dt + l32], sc[h][v], adv[dt], 0, 0, 0);
                    adk[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Qs[qi * KS + 32 * dt + l32], dp[h][v], adk[dt], 0, 0, 0);
                }
            }
    }
    // a padding key of a partial tile: zero rows
    const bool valid = !a.geo.partial || slot_valid(a.geo, kb, 32 * wave + l32);
    float *ov = (float *)a.grad + krow * D, *ok = (float *)a.grad2 + krow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 wv, wk;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                wv[u] = valid ? adv[dt][4 * rr + u] : 0.f;
                wk[u] = valid ? adk[dt][4 * rr + u] * a.scale : 0.f;
            }
            *reinterpret_cast<f32x4 *>(ov + 32 * dt + 8 * rr + 4 * hh) = wv;
            *reinterpret_cast<f32x4 *>(ok + 32 * dt + 8 * rr + 4 * hh) = wk;
        }
}

// ---------------------------------------------------------------------------
int launch_backward(const BwdLaunch &L, hipStream_t s) {
    const int64_t ntok = L.rows * 64;
    const int tpw = 64 / (L.d / 8);
    const dim3 pg((unsigned)((ntok + 4 * tpw - 1) / (4 * tpw))), pb(256);
    const bool f32 = L.f32;
    if (f32) {
        const dim3 fg((unsigned)((ntok + 255) / 256));
        if (L.d == 128)
            bwd_prep_f32_kernel<128><<<fg, pb, 0, s>>>((const float *)L.out, (const float *)L.args.dout, L.lse, L.lse2, L.dn, ntok);
        else
            bwd_prep_f32_kernel<64><<<fg, pb, 0, s>>>((const float *)L.out, (const float *)L.args.dout, L.lse, L.lse2, L.dn, ntok);
    } else if (L.d == 128)
        bwd_prep_kernel<128><<<pg, pb, 0, s>>>((const __bf16 *)L.out, (const __bf16 *)L.args.dout, L.lse, L.lse2, L.dn, ntok);
    else
        bwd_prep_kernel<64><<<pg, pb, 0, s>>>((const __bf16 *)L.out, (const __bf16 *)L.args.dout, L.lse, L.lse2, L.dn, ntok);
    csr_bits_kernel<<<dim3((unsigned)((L.rows + 3) / 4)), dim3(256), 0, s>>>(L.row_ptr, L.col_idx, L.col_count, L.rows,
                                                                            L.nB, L.nW, L.bits);
    const int64_t words = L.BH * L.nW;
    const dim3 wg((unsigned)((words + 3) / 4)), wb(256);
    csc_pass_kernel<true><<<wg, wb, 0, s>>>(L.bits, L.BH, L.nB, L.nW, L.colcount, nullptr, nullptr);
    scan_kernel<<<1, 1024, 0, s>>>(L.colcount, L.rows, L.col_ptr);
    csc_pass_kernel<false><<<wg, wb, 0, s>>>(L.bits, L.BH, L.nB, L.nW, nullptr, L.col_ptr, L.t_idx);
    BwdArgs csr = L.args, csc = L.args;
    csr.ptr = L.row_ptr;
    csr.idx = L.col_idx;
    csr.idx_count = L.col_count;
    csr.grad = L.dq;
    csc.ptr = L.col_ptr;
    csc.idx = L.t_idx;
    csc.idx_count = L.col_count;
    const dim3 g((unsigned)(L.args.plan.max_slots + L.args.n_pairs)), b(256), mg((unsigned)L.args.plan.max_slots);
    BwdArgs cdkv = csc;
    cdkv.grad = L.dv;
    cdkv.grad2 = L.dk;
    if (f32) {
        // one workgroup per block, no pieces
        const dim3 rg((unsigned)L.rows), rb(128);
        if (L.d == 128) {
            bwd_dq_f32_kernel<128><<<rg, rb, 0, s>>>(csr, L.rows);
            bwd_dkv_f32_kernel<128><<<rg, rb, 0, s>>>(cdkv, L.rows);
        } else {
            bwd_dq_f32_kernel<64><<<rg, rb, 0, s>>>(csr, L.rows);
            bwd_dkv_f32_kernel<64><<<rg, rb, 0, s>>>(cdkv, L.rows);
        }
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    // each pass: the forward's plan over the list it walks, the pass, the merge of its pieces
    auto plan = [&](const BwdArgs &w, bool masks) {
        AttnArgs pa = {};
        if (masks && L.slot_mask_w != nullptr) {
            // the first plan also writes the slot masks of partial tiles
            pa.geo = L.geo;
            pa.slot_mask_w = L.slot_mask_w;
            pa.slot_mask = L.slot_mask_w;
        }
        pa.row_ptr = w.ptr;
        pa.col_idx = w.idx;
        pa.col_count = w.idx_count;
        pa.n_pairs = w.n_pairs;
        pa.pairs_per_head = w.pairs_per_head;
        pa.nB = w.nB;
        pa.nK = w.nB;
        pa.kpt = 1;
        pa.pair_stride = w.pair_stride;
        pa.plan = w.plan;
        return launch_plan(pa, s);
    };
    const bool masked = L.args.slot_mask != nullptr;
    if (plan(csr, true)) return -1;
    if (L.d == 128) {
        if (masked) bwd_kernel<128, kDQ, true><<<g, b, 0, s>>>(csr);
        else bwd_kernel<128, kDQ, false><<<g, b, 0, s>>>(csr);
        bwd_merge_kernel<128><<<mg, b, 0, s>>>(csr, 0);
    } else {
        if (masked) bwd_kernel<64, kDQ, true><<<g, b, 0, s>>>(csr);
        else bwd_kernel<64, kDQ, false><<<g, b, 0, s>>>(csr);
        bwd_merge_kernel<64><<<mg, b, 0, s>>>(csr, 0);
    }
    if (plan(cdkv, false)) return -1;
    if (L.d == 128) {
        if (masked) bwd_kernel<128, kDKV, true><<<g, b, 0, s>>>(cdkv);
        else bwd_kernel<128, kDKV, false><<<g, b, 0, s>>>(cdkv);
        bwd_merge_kernel<128><<<mg, b, 0, s>>>(cdkv, 1);
    } else {
        if (masked) bwd_kernel<64, kDKV, true><<<g, b, 0, s>>>(cdkv);
        else bwd_kernel<64, kDKV, false><<<g, b, 0, s>>>(cdkv);
        bwd_merge_kernel<64><<<mg, b, 0, s>>>(cdkv, 1);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
