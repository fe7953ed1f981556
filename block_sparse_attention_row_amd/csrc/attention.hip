// Block-sparse flash-attention forward over a CSR list of kept 64x64 tiles (gfx950).
//
// For every query block the kernel walks the key blocks of its CSR row and
// runs exact attention with an online softmax, so only the kept tiles are
// computed (the "Expansion" item of the NABLA summary page, "NABLA:
// Neighborhood Adaptive Block-Level Attention", section "Methodologie :
// NABLA").  The result equals a dense softmax over the tokens of the kept
// blocks.
//
// Layout of the work (bf16): a workgroup of 4 waves serves a pair of neighbouring
// query blocks, 32 queries per wave, and walks the union of the two CSR rows;
//   * the transposed score tile S^T = K Q^T is formed on MFMA with K as the
//     A operand (from LDS) and Q as the B operand (kept in registers), so that
//     each lane's accumulators belong to one query: the softmax row max needs
//     one exchange with the partner lane (l ^ 32) and the rescale of the
//     output is a per-lane scalar;
//   * O^T += V^T P^T reuses the S^T accumulators directly as the B operand:
//     the eight accumulators a lane holds for a 16-key chunk are exactly the
//     eight keys it must supply, once V is read transposed from LDS in the key
//     order {0-3, 8-11, 4-7, 12-15} of each 16-key chunk;
//   * K and V tiles stream from global memory straight into double-buffered LDS
//     (K two tiles ahead of use, V one), and the scores of tile j+1 are formed
//     while the softmax of tile j runs on the VALU.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace sattn {

// Online-softmax bookkeeping of the kernel with a logit offset beta (log2 units) on
// each tile: scores are s*c + beta, this lane owns one query, and the running max M
// (log2 units) only moves when a tile's max exceeds it by more than kLazy: in
// between, P = 2^(s*c + beta - M) stays below 2^kLazy and the output needs no
// rescaling.  The result is the same softmax.
template <int NDT>
__device__ __forceinline__ void tile_rescale_biased(const f32x16 *acc_s, float c, float beta, float &M,
                                                    float &l_run, f32x16 *acc_o) {
    float mt = fmaxf(acc_s[0][0], acc_s[0][1]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = (kt == 0 ? 2 : 0); v < 16; v += 2) mt = fmaxf(mt, fmaxf(acc_s[kt][v], acc_s[kt][v + 1]));
    mt = __builtin_fmaf(pair_max(mt), c, beta);
    const bool grow = mt - M > kLazy;
    if (__ballot(grow)) {
        const float m_new = grow ? mt : M;
        const float alpha = __builtin_amdgcn_exp2f(M - m_new);
        M = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc_o[i][v] *= alpha;
    }
}

// P = 2^(s*c - m*c) as bf16 B operands; the row sum takes the same bf16-rounded P.
__device__ __forceinline__ void tile_probs(const f32x16 *acc_s, float c, float mc, float &l_run, bf16x8 *pf) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[kc >> 1][8 * (kc & 1) + e], c, -mc));
        pf[kc] = __builtin_convertvector(pv, bf16x8);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            l_run = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf[kc][2 * e], pf[kc][2 * e + 1]}, kOnes2, l_run, false);
    }
}

// The plain kernel forms a tile's P with the running max as it stands and checks
// the lane's share of the tile's row sum: above 2^16, or not finite (the row's first
// tile), the max moves to the tile's and the tile's P is formed again.  P stays
// below 2^16 and the accumulators far from overflow, and the max scan of every
// tile drops out of the common path.  Returns the share to add to the row sum.
constexpr float kTileSumCap = 65536.f;
template <int NDT>
__device__ __forceinline__ float tile_commit(const f32x16 *acc_s, float c, float &m_run, float &l_run, float lt,
                                             f32x16 *acc_o, bf16x8 *pf) {
    if (__ballot(!(lt <= kTileSumCap))) {
        float mt = fmaxf(acc_s[0][0], acc_s[0][1]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = (kt == 0 ? 2 : 0); v < 16; v += 2) mt = fmaxf(mt, fmaxf(acc_s[kt][v], acc_s[kt][v + 1]));
        const float m_new = fmaxf(m_run, pair_max(mt));
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc_o[i][v] *= alpha;
        lt = 0.f;
        tile_probs(acc_s, c, m_run * c, lt, pf);
    }
    return lt;
}

// One compare-exchange stage of a bitonic merge over lanes 0-31 (ascending): lane l
// and lane l ^ J exchange through a swizzle, the lower lane keeps the smaller key.
template <int J> __device__ __forceinline__ uint32_t merge_stage(uint32_t key, int lane) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)key, (J << 10) | 0x1f);
    return (lane & J) ? max(key, o) : min(key, o);
}

// Inclusive prefix max over lanes 0 .. 31 of values >= -1 (lanes 32-63: unspecified),
// by row shifts within each 16-lane row and lane 15 carried into the second row.
__device__ __forceinline__ int prefix_max32(int v, int lane) {
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppShr1, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppShr2, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppShr4, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppShr8, 0xF, 0xF, false));
    const int r15 = __builtin_amdgcn_readlane(v, 15);
    return (lane >= 16 && lane < 32) ? max(v, r15) : v;
}

// Scores of the next tile (MFMA) interleaved with the probabilities of the current
// one (VALU): each score MFMA is grouped with an equal share of the softmax work, and the K reads run two MFMAs ahead.
template <int D>
__device__ __forceinline__ void tile_scores_probs(const char *K, const bf16x8 *qf, const FragOffsets<D> &fo,
                                                  f32x16 *sn, const f32x16 *sc, float c, float mc, float &l_run,
                                                  bf16x8 *pf) {
    constexpr int NC = D / 16, NM = 2 * NC;       // score MFMAs per tile
    constexpr int PER = 32 / NM;                  // probabilities per MFMA group
    // MFMA i works on key half i & 1 and d chunk i >> 1, so consecutive MFMAs feed
    // different accumulators and never wait on each other
    auto kfrag = [&](int i) { return fo.kfrag(K, i & 1, i >> 1); };
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        sn[0][v] = 0.f;
        sn[1][v] = 0.f;
    }
    bf16x8 kf[4];                                 // four-slot ring, as in tile_pv
    kf[0] = kfrag(0);
    kf[1] = kfrag(1);
    f32x8 pv;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        if (i + 2 < NM) kf[(i + 2) % 4] = kfrag(i + 2);
        sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % 4], qf[i >> 1], sn[i & 1], 0, 0, 0);
        // probabilities PER*i .. PER*i + PER - 1 of the current tile (8 per 16-key chunk)
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = PER * i + u, kc = e >> 3;
            pv[e & 7] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kc >> 1][8 * (kc & 1) + (e & 7)], c, -mc));
            if ((e & 7) == 7) {
                pf[kc] = __builtin_convertvector(pv, bf16x8);
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    l_run = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf[kc][2 * w], pf[kc][2 * w + 1]}, kOnes2,
                                                            l_run, false);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Workgroup of 4 waves = a pair of query blocks of one (batch, head), neighbours in
// time (pair_blocks); waves 2g and 2g+1 own queries 0-31 and 32-63 of block g of
// the pair.  The pair walks the
// union of its two ascending CSR rows; each union tile is loaded once and computed
// by the waves whose row keeps it.  The walk is software-pipelined one tile deep:
// while the scores of tile j+1 are formed on MFMA, the softmax of tile j runs on
// the VALU, then P V of tile j follows.  K runs two tiles ahead of use and V one,
// in two LDS buffers each.
//
// BIAS: every block-list entry carries a logit offset (col_bias, natural-log units)
// that is added to the scores of its tile; the running max is then tracked in log2
// units, including the offset.
//
// GATHER: the block list names 4-token key blocks (AB-Attention page, section "Les
// trois techniques d'AB-Attention", third technique).  The pair walks the union of its
// two rows 16 entries at a time, and the 16 blocks of a step are gathered by index
// into one 64-key tile: each wave's direct loads cover 4 consecutive tile rows per
// 16-row group, exactly one block, so a block's address is the load's scalar base
// (no copy, no permutation of the tokens).  A wave masks the keys of entries its own
// row does not keep, and those past the list's end.
//
// MASKED: the grid ends in partial tiles; the keys of their padding slots are masked
// and padding queries get O = 0, LSE = -inf (a separate instantiation, so that the
// plain walk carries none of it).
template <int D, bool BIAS, bool GATHER, bool MASKED>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
    static_assert(!(BIAS && GATHER) && !(GATHER && MASKED), "combinations that are not built");
    using G = TileGeo<D>;
    constexpr int ROWB = G::ROWB, SLOTS = G::SLOTS, RPI = G::RPI, IPW = G::IPW, NDT = G::NDT, TILEB = G::TILEB;
    __shared__ __attribute__((aligned(1024))) char Ks[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char Vs[2 * TILEB];

    const int t = threadIdx.x, lane = t & 63, hh = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 1;                    // 0: first query block of the pair, 1: second
    // work item: the first long_slots workgroups take the pieces of long rows (so that
    // long work starts first), the next n_pairs take whole pairs that were not split,
    // and the last ones the pieces of the last round's pairs (so that the launch ends
    // on short items)
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
    int32_t blk_a, blk_b;
    pair_blocks((int32_t)(pair % a.pairs_per_head), a.pair_stride, a.nB, blk_a, blk_b);
    const int64_t N = (int64_t)a.nB * 64;
    const char *kgh = (const char *)a.k + bh * N * ROWB, *vgh = (const char *)a.v + bh * N * ROWB;
    const char *kg = kgh + 16 * wave * ROWB;
    const char *vg = vgh + 16 * wave * ROWB;
    const_i32 *rp = (const_i32 *)a.row_ptr;
    const float c = a.scale_log2;

    // CSR ranges of the two rows (the second may not exist when nB is odd)
    const int64_t rowA = bh * a.nB + blk_a, rowB = bh * a.nB + blk_b;
    const bool hasB = blk_b >= 0;
    const int blk = grp && hasB ? blk_b : blk_a;   // this wave's query block
    auto clamp_range = [&](int64_t r, int64_t &b, int64_t &e) {
        b = rp[r];
        e = rp[r + 1];
        e = e < a.col_count ? e : a.col_count;
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
        // the whole-row walk would arrive at the piece with the largest valid column
        // of the entries before it as its last column
        auto prefix_max = [&](int64_t from, int64_t to) {
            int m = -1;
            for (int64_t i = from + lane; i < to; i += 64) {
                const int cc = a.col_idx[i];
                if (cc >= 0 && cc < a.nK) m = cc > m ? cc : m;
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

    // Q fragments (B operand of S^T): query 32*(wave&1) + l32 of this wave's block, d = 16c + 8hh .. +7
    const __bf16 *qg = (const __bf16 *)a.q + (bh * N + (int64_t)blk * 64) * D;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int cq = 0; cq < D / 16; ++cq)
        qf[cq] = has_row ? *reinterpret_cast<const bf16x8 *>(qg + (32 * (wave & 1) + l32) * D + 16 * cq + 8 * hh)
                         : bf16x8{};
    // settle the Q loads here (vmcnt(0) through the builtin, which the compiler's own
    // wait tracking sees), so that no wait for them lands inside the tile loop
    __builtin_amdgcn_s_waitcnt(0x0f70);

    // per-lane source offsets of the direct loads (this wave covers rows 16 w .. 16 w + 15)
    uint32_t voff[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
        const int r = RPI * j + lane / SLOTS, sl = lane % SLOTS;   // row within the wave's 16 (== row mod 16)
        voff[j] = r * ROWB + 16 * (sl ^ swz_key<SLOTS>(r));
    }
    const uint32_t ks0 = (uint32_t)(uintptr_t)(lds_char *)Ks + 16 * wave * ROWB;
    const uint32_t vs0 = (uint32_t)(uintptr_t)(lds_char *)Vs + 16 * wave * ROWB;
    // merged walk over the two rows' ascending lists (entries out of range or not
    // ascending are skipped).  Each row's upcoming entries sit in a VGPR window (lane
    // l holds entry base + l) read with v_readlane; the following window is loaded
    // one window ahead, so the walk never waits on memory.
    constexpr int kNone = 0x7fffffff;
    const int32_t *cv = a.col_idx;
    auto window = [&](int64_t base, int64_t e) { return base + lane < e ? cv[base + lane] : kNone; };
    // (BIAS) the entries' offsets travel in windows of their own, in step with the columns
    auto bwindow = [&](int64_t base, int64_t e) {
        if constexpr (BIAS) return base + lane < e ? a.col_bias[base + lane] : 0.f;
        else return 0.f;
    };
    int64_t baseA = begA, baseB = begB;
    int posA = 0, posB = 0;
    int winA = window(baseA, endA), nxtA = window(baseA + 64, endA);
    int winB = window(baseB, endB), nxtB = window(baseB + 64, endB);
    float bwinA = bwindow(baseA, endA), bnxtA = bwindow(baseA + 64, endA);
    float bwinB = bwindow(baseB, endB), bnxtB = bwindow(baseB + 64, endB);
    auto peek = [&](int64_t &base, int &pos, int &win, int &nxt, float &bwin, float &bnxt, int64_t e, int last) {
        while (base + pos < e) {
            if (pos == 64) {
                base += 64;
                pos = 0;
                win = nxt;
                nxt = window(base + 64, e);
                if constexpr (BIAS) {
                    bwin = bnxt;
                    bnxt = bwindow(base + 64, e);
                }
            }
            const int cc = __builtin_amdgcn_readlane(win, pos);
            if (cc > last && cc < a.nK) return cc;
            ++pos;
        }
        return kNone;
    };
    // next union tile: its column, whether this wave's row keeps it, and (BIAS) the
    // offset of this wave's entry in log2 units
    auto next_union = [&](int &col, bool &mine, float &beta) {
        const int cA = peek(baseA, posA, winA, nxtA, bwinA, bnxtA, endA, lastA);
        const int cB = peek(baseB, posB, winB, nxtB, bwinB, bnxtB, endB, lastB);
        col = cA < cB ? cA : cB;
        const bool inA = cA == col && col != kNone, inB = cB == col && col != kNone;
        if constexpr (BIAS) {
            const float bA = inA ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bwinA), posA)) : 0.f;
            const float bB = inB ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bwinB), posB)) : 0.f;
            beta = (grp ? bB : bA) * kLog2e;
        } else {
            beta = 0.f;
        }
        if (inA) { lastA = cA; ++posA; }
        if (inB) { lastB = cB; ++posB; }
        mine = grp ? inB : inA;
    };

    f32x16 acc_o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[i][v] = 0.f;
    // running max: raw score units, or (BIAS) log2 units including the offsets
    float m_run = -INFINITY, l_run = 0.f;
    FragOffsets<D> fo;
    fo.init(lane);
    // partial tiles: the per-block slot masks the plan wrote
    auto mask_tile = [&](f32x16 *sc, int col) {
        if constexpr (MASKED) {
            const uint64_t km = a.slot_mask[__builtin_amdgcn_readfirstlane(col)];
            if (km != ~0ull) mask_keys(sc, km, hh);
        }
    };

    if constexpr (!GATHER) {
    auto issue_k = [&](int col, int buf) {
        const int64_t cu = __builtin_amdgcn_readfirstlane(col);
#pragma unroll
        for (int i = 0; i < IPW; ++i) dma16(ks0 + buf * TILEB + RPI * i * ROWB, voff[i], kg + cu * TILEB);
    };
    auto issue_v = [&](int col, int buf) {
        const int64_t cu = __builtin_amdgcn_readfirstlane(col);
#pragma unroll
        for (int i = 0; i < IPW; ++i) dma16(vs0 + buf * TILEB + RPI * i * ROWB, voff[i], vg + cu * TILEB);
    };
    // tiles j (scores pending), j+1 (K resident), j+2 (lookahead)
    int col0, col1, col2;
    bool mine0, mine1, mine2;
    float beta0, beta1, beta2;
    next_union(col0, mine0, beta0);
    next_union(col1, mine1, beta1);
    f32x16 sa[2], sb[2];
    if (col0 != kNone) {
        issue_k(col0, 0);
        issue_v(col0, 0);
        if (col1 != kNone) issue_k(col1, 1);
        wait_vmcnt<0>();
        __syncthreads();
        if (mine0) {
            tile_scores<D>(Ks, qf, fo, sa);
            mask_tile(sa, col0);
        }
    }
    // One pipeline step for tile j with j & 1 == BJ: the scores of tile j are in sc,
    // those of tile j+1 go to sn; buffer offsets are compile-time constants.
    auto step = [&](auto bj_tag, f32x16 *sc, f32x16 *sn) {
        constexpr int BJ = decltype(bj_tag)::value;
        wait_vmcnt<0>();            // this wave's part of K(j+1) and V(j) has landed
        next_union(col2, mine2, beta2);   // (after the wait: a window load never waits on tile loads)
        __syncthreads();            // ... and everyone's; K(j) and V(j-1) are free
        if (col2 != kNone) issue_k(col2, BJ);
        if (col1 != kNone) issue_v(col1, BJ ^ 1);

        // (BIAS: the offset moves the scores tile by tile, so the max is checked first)
        float mc = 0.f, lt = 0.f;
        if (mine0) {
            if constexpr (BIAS) {
                tile_rescale_biased<NDT>(sc, c, beta0, m_run, l_run, acc_o);
                mc = m_run - beta0;
            } else {
                mc = m_run * c;
            }
        }
        bf16x8 pf[4];
        float &lacc = BIAS ? l_run : lt;
        if (mine0 && mine1) {
            tile_scores_probs<D>(Ks + (BJ ^ 1) * TILEB, qf, fo, sn, sc, c, mc, lacc, pf);
        } else if (mine1) {
            tile_scores<D>(Ks + (BJ ^ 1) * TILEB, qf, fo, sn);
        } else if (mine0) {
            tile_probs(sc, c, mc, lacc, pf);
        }
        if (mine1) mask_tile(sn, col1);
        if constexpr (!BIAS) {
            if (mine0) l_run += tile_commit<NDT>(sc, c, m_run, l_run, lt, acc_o, pf);
        }
        // P V is MFMA work only: the wave runs it at raised priority, so that the
        // SIMD's other wave fills the matrix unit's gaps with its softmax instead of
        // delaying these MFMAs
        __builtin_amdgcn_s_setprio(1);
        if (mine0) tile_pv<D>(Vs + BJ * TILEB, pf, fo, acc_o);
        __builtin_amdgcn_s_setprio(0);
        col0 = col1;
        mine0 = mine1;
        beta0 = beta1;
        col1 = col2;
        mine1 = mine2;
        beta1 = beta2;
    };
    while (col0 != kNone) {
        step(std::integral_constant<int, 0>{}, sa, sb);
        if (col0 == kNone) break;
        step(std::integral_constant<int, 1>{}, sb, sa);
    }

    } else {
    // The units of the gathered walk: the next up-to-16 entries of the union of the
    // pair's two rows, gathered into one tile each.  Each row keeps a buffer of its next
    // valid entries in a VGPR (lane l: the l-th next one, kNone past them), topped up 32
    // raw entries at a time from a window loaded one top-up ahead; the skip rule of the
    // tile walk (an entry counts if it is in range and above every earlier counted
    // entry) applies to a whole window at once through a prefix max.  A unit is then
    // the 16 smallest distinct entries of the two rows' first 16 candidates, merged
    // across the lanes (a bitonic merge), an entry both rows hold taken once.  Unseen
    // entries of either row are larger than every placed one, since each buffer holds
    // at least 16 entries or the whole rest of its row.
    // above every 4-token column (nK <= 16 * 4096); twice it plus one fits 32 bits
    constexpr int kGatherSentinel = 0x3fffffff;
    struct Unit {
        int cols;         // lane e holds entry e's block (padded with the last one)
        bool mine;        // this wave's row keeps some entry of the unit
        int n;            // entries in the unit (0 past the end)
        uint32_t em;      // this wave's entries (bit e: entry e)
    };
    struct RowBuf {
        int buf;          // lane l: the l-th next counted entry, kNone past cnt
        int cnt;
        int raw;          // lanes 0-31: raw entries next .. next + 31 (kNone past end)
        int64_t next, end;
        int last;         // the last counted entry (the skip rule's running max)
    };
    auto raw_window = [&](int64_t base, int64_t e) { return lane < 32 && base + lane < e ? cv[base + lane] : kNone; };
    auto topup = [&](RowBuf &r) {
        while (r.cnt <= 32 && r.next < r.end) {
            const int v = lane < 32 ? r.raw : kNone;
            const bool inr = v >= 0 && v < a.nK;
            const int incl = prefix_max32(inr ? v : -1, lane);
            const int r15 = __builtin_amdgcn_readlane(incl, 15);
            int ex = __builtin_amdgcn_update_dpp(-1, incl, kDppShr1, 0xF, 0xF, false);
            ex = lane == 16 ? r15 : ex;
            ex = max(ex, r.last);
            const bool ok = lane < 32 && inr && v > ex;
            const uint64_t om = __ballot(ok);
            const int k = __popcll(om);
            // the counted entries to lanes cnt .. cnt + k - 1 in order, the others to the
            // remaining lanes (a permutation of the 64 lanes)
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(om >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)om, 0u));
            const int to = ok ? r.cnt + below : (r.cnt + k + (lane - below)) & 63;
            const int pushed = __builtin_amdgcn_ds_permute(to * 4, v);
            r.buf = (lane >= r.cnt && lane < r.cnt + k) ? pushed : r.buf;
            r.cnt += k;
            r.last = max(r.last, __builtin_amdgcn_readlane(incl, 31));
            r.next += 32;
            r.raw = raw_window(r.next, r.end);
        }
    };
    auto consume = [&](RowBuf &r, int t) {
        const int sh = __builtin_amdgcn_ds_bpermute(((lane + t) & 63) * 4, r.buf);
        r.buf = lane + t < 64 ? sh : kNone;
        r.cnt -= t;
    };
    RowBuf RA{kNone, 0, raw_window(begA, endA), begA, endA, lastA};
    RowBuf RB{kNone, 0, raw_window(begB, endB), begB, endB, lastB};
    auto next_unit = [&](Unit &u) {
        topup(RA);
        topup(RB);
        const int xa = RA.buf, xbv = RB.buf;
        // lanes 0-15 take row A's first 16 candidates, lanes 16-31 row B's
        const bool isA = lane < 16, isB = lane >= 16 && lane < 32;
        // the 32 candidates in merged order: row B's reversed behind row A's form one
        // bitonic sequence over lanes 0-31, which five compare-exchange stages sort.  The
        // keys are 2 x value + row (kNone as a value above every column), so that of an
        // entry both rows hold, row A's copy comes first.
        // (the lane exchanges are swizzles and wave shifts with immediate patterns, so
        // that no per-lane address vector stays live across the walk)
        const int xrev = __builtin_amdgcn_ds_swizzle(xbv, kSwizzleXor31);   // lane 16 + i: B[15 - i]
        const int xv = isA ? xa : (isB ? xrev : kNone);
        uint32_t key = ((uint32_t)min(xv, kGatherSentinel) << 1) | (isB ? 1u : 0u);
        key = merge_stage<16>(key, lane);
        key = merge_stage<8>(key, lane);
        key = merge_stage<4>(key, lane);
        key = merge_stage<2>(key, lane);
        key = merge_stage<1>(key, lane);
        const int val = (int)(key >> 1);
        const bool fromB = key & 1u;
        // an entry both rows hold: row A's copy is followed by row B's, which is dropped
        const uint32_t kprev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, kDppWaveShr1, 0xF, 0xF, false);
        const uint32_t knext = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, kDppWaveShl1, 0xF, 0xF, false);
        const bool dupB = fromB && lane > 0 && (kprev >> 1) == (uint32_t)val;
        const bool dupA = !fromB && lane < 31 && (knext >> 1) == (uint32_t)val;
        const bool keep = lane < 32 && val < kGatherSentinel && !dupB;
        const uint64_t km = __ballot(keep);
        const int nk = __popcll(km);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
        // the kept entries to lanes 0 .. nk-1 in order, the others to the remaining lanes
        // (a permutation of the 64 lanes); lane e < 16 then holds entry e (value, row flags)
        const int to = keep ? below : (nk + (lane - below)) & 63;
        const int flag = fromB ? 2 : (dupA ? 3 : 1);
        const int packed = __builtin_amdgcn_ds_permute(to * 4, (int)((uint32_t)val * 4u + (uint32_t)flag));
        const int col = lane < 16 && lane < nk ? packed >> 2 : 0;
        const int fl = lane < 16 && lane < nk ? (packed & 3) : 0;
        const uint64_t present = __ballot(fl != 0);
        u.n = __popcll(present);
        const int lastc = u.n ? __builtin_amdgcn_readlane(col, u.n - 1) : 0;
        u.cols = lane < u.n ? col : lastc;
        const uint32_t my = (uint32_t)__ballot(lane < 16 && (fl & (grp ? 2 : 1)));
        u.mine = my != 0;
        u.em = my;
        // both rows move past the unit's last entry
        const int tA = __popcll(__ballot(lane < 16 && xa != kNone && u.n && xa <= lastc));
        const int tB = __popcll(__ballot(lane < 16 && xbv != kNone && u.n && xbv <= lastc));
        consume(RA, tA);
        consume(RB, tB);
    };
    // direct loads of a unit into tile buffer buf
    auto issue_u = [&](const char *gw, const char *gh, uint32_t lds0, const Unit &u, int buf) {
        (void)gw;
        if constexpr (RPI == 4) {
            // load i of wave w covers tile rows 16 w + 4 i .. + 3: entry 4 w + i
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int j = __builtin_amdgcn_readlane(u.cols, 4 * wave + i);
                dma16(lds0 + buf * TILEB + RPI * i * ROWB, voff[i], gh + (int64_t)(4 * (j - i)) * ROWB);
            }
        } else {
            // RPI == 8: load i covers entries 4 w + 2 i (lanes 0-31) and 4 w + 2 i + 1 (32-63)
            static_assert(RPI == 8, "4-token entries per direct load");
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int jlo = __builtin_amdgcn_readlane(u.cols, 4 * wave + 2 * i);
                const int jhi = __builtin_amdgcn_readlane(u.cols, 4 * wave + 2 * i + 1);
                const uint32_t v = voff[i] + (hh ? (uint32_t)(4 * (jhi - jlo - 1) * ROWB) : 0u);
                dma16(lds0 + buf * TILEB + RPI * i * ROWB, v, gh + (int64_t)(4 * (jlo - 2 * i)) * ROWB);
            }
        }
    };
    auto live = [&](const Unit &u) { return u.n != 0; };
    auto mask_u = [&](f32x16 *sc, const Unit &u) {
        if (u.em != 0xffffu) mask_entries(sc, u.em);
    };

    // units j (scores pending), j+1 (K resident), j+2 (lookahead)
    Unit u0, u1, u2;
    next_unit(u0);
    next_unit(u1);
    f32x16 sa[2], sb[2];
    if (live(u0)) {
        issue_u(kg, kgh, ks0, u0, 0);
        issue_u(vg, vgh, vs0, u0, 0);
        if (live(u1)) issue_u(kg, kgh, ks0, u1, 1);
        wait_vmcnt<0>();
        __syncthreads();
        if (u0.mine) {
            tile_scores<D>(Ks, qf, fo, sa);
            mask_u(sa, u0);
        }
    }
    // One pipeline step for unit j with j & 1 == BJ: the scores of unit j are in sc,
    // those of unit j+1 go to sn; buffer offsets are compile-time constants.
    auto step = [&](auto bj_tag, f32x16 *sc, f32x16 *sn) {
        constexpr int BJ = decltype(bj_tag)::value;
        wait_vmcnt<0>();            // this wave's part of K(j+1) and V(j) has landed
        next_unit(u2);              // (after the wait: a window load never waits on tile loads)
        __syncthreads();            // ... and everyone's; K(j) and V(j-1) are free
        if (live(u2)) issue_u(kg, kgh, ks0, u2, BJ);
        if (live(u1)) issue_u(vg, vgh, vs0, u1, BJ ^ 1);

        const bool mine0 = u0.mine, mine1 = u1.mine;
        float lt = 0.f;
        const float mc = mine0 ? m_run * c : 0.f;
        bf16x8 pf[4];
        float &lacc = lt;
        if (mine0 && mine1) {
            tile_scores_probs<D>(Ks + (BJ ^ 1) * TILEB, qf, fo, sn, sc, c, mc, lacc, pf);
        } else if (mine1) {
            tile_scores<D>(Ks + (BJ ^ 1) * TILEB, qf, fo, sn);
        } else if (mine0) {
            tile_probs(sc, c, mc, lacc, pf);
        }
        if (mine1) mask_u(sn, u1);
        if (mine0) l_run += tile_commit<NDT>(sc, c, m_run, l_run, lt, acc_o, pf);
        // P V is MFMA work only: the wave runs it at raised priority, so that the
        // SIMD's other wave fills the matrix unit's gaps with its softmax instead of
        // delaying these MFMAs
        __builtin_amdgcn_s_setprio(1);
        if (mine0) tile_pv<D>(Vs + BJ * TILEB, pf, fo, acc_o);
        __builtin_amdgcn_s_setprio(0);
        u0 = u1;
        u1 = u2;
    };
    while (live(u0)) {
        step(std::integral_constant<int, 0>{}, sa, sb);
        if (!live(u0)) break;
        step(std::integral_constant<int, 1>{}, sb, sa);
    }

    }
    if (!has_row) return;
    // epilogue: normalise and store; lane owns query l32, d = 32 dt + 8 rr + 4 hh + {0..3}.
    // A padding slot of a partial tile gets O = 0 and LSE = -inf.
    const float l_tot = pair_sum(l_run);
    bool qvalid = true;
    if constexpr (MASKED) qvalid = (a.slot_mask[blk] >> (32 * (wave & 1) + l32)) & 1ull;
    const float inv = (l_tot > 0.f && qvalid) ? 1.f / l_tot : 0.f;
    if (split) {
        // piece of a split pair: the normalised partial output and its log2-sum-exp
        const int q = 32 * (wave & 1) + l32;
        float *po = a.plan.part_o + ((int64_t)it.slot * 2 + grp) * (D * 64);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    po[(32 * dt + 8 * rr + 4 * hh + e) * 64 + q] = qvalid ? acc_o[dt][4 * rr + e] * inv : 0.f;
        if (hh == 0)
            a.plan.part_lse[((int64_t)it.slot * 2 + grp) * 64 + q] =
                (l_tot > 0.f && qvalid) ? (BIAS ? m_run : m_run * c) + __log2f(l_tot) : -INFINITY;
        return;
    }
    const int64_t qrow = bh * N + (int64_t)blk * 64 + 32 * (wave & 1) + l32;
    __bf16 *og = (__bf16 *)a.out + qrow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = qvalid ? acc_o[dt][4 * rr + e] * inv : 0.f;
            *reinterpret_cast<bf16x4 *>(og + 32 * dt + 8 * rr + 4 * hh) = __builtin_convertvector(w, bf16x4);
        }
    if (a.lse && hh == 0)
        a.lse[qrow] = (l_tot > 0.f && qvalid) ? ((BIAS ? m_run : m_run * c) + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Row splitting: the plan (one workgroup) and the merge of the pieces.

// CSR range of row r, clamped as the attention kernel clamps it.
__device__ __forceinline__ void row_range(const AttnArgs &a, int64_t r, int64_t &b, int64_t &e) {
    b = a.row_ptr[r];
    e = a.row_ptr[r + 1];
    e = e < a.col_count ? e : a.col_count;
    b = b < 0 ? 0 : b;
    if (e < b) e = b;
}
__device__ __forceinline__ void pair_ranges(const AttnArgs &a, int64_t p, int64_t &bA, int64_t &eA, int64_t &bB,
                                            int64_t &eB) {
    const int64_t bh = p / a.pairs_per_head;
    int32_t blk_a, blk_b;
    pair_blocks((int32_t)(p % a.pairs_per_head), a.pair_stride, a.nB, blk_a, blk_b);
    row_range(a, bh * a.nB + blk_a, bA, eA);
    bB = eB = 0;
    if (blk_b >= 0) row_range(a, bh * a.nB + blk_b, bB, eB);
}

// Sum over the 1024 threads of the workgroup, returned to every thread.
__device__ __forceinline__ int64_t block_sum64(int64_t v, int64_t *lds16) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds16[threadIdx.x >> 6] = v;
    __syncthreads();
    int64_t t = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += lds16[w];
    return t;
}
// Piece length L = max(kMinPiece, total work / resident workgroups), doubled until
// the pieces fit the partial slots; a pair whose longer row holds est > L tiles is cut
// into ceil(est / L) pieces, each row split evenly by position.  A piece also records
// where its rows begin, from which its workgroup recovers the last column the
// whole-row walk would have taken before the piece (so that both skip the same entries).
__global__ __launch_bounds__(1024) void plan_kernel(AttnArgs a) {
    __shared__ int64_t red[16];
    __shared__ int32_t scan[16];
    const SplitPlan &P = a.plan;
    const int t = threadIdx.x;
    // which slots of each block are grid tokens, for grids that end in partial tiles
    if (a.slot_mask != nullptr) {
        for (int b = t; b < a.nB; b += 1024) {
            uint64_t m = 0;
            for (int u = 0; u < 64; ++u) m |= (uint64_t)slot_valid(a.geo, b, u) << u;
            a.slot_mask_w[b] = m;
        }
    }
    auto est_of = [&](int64_t p) {
        int64_t bA, eA, bB, eB;
        pair_ranges(a, p, bA, eA, bB, eB);
        return (max(eA - bA, eB - bB) + a.kpt - 1) / a.kpt;   // tiles (gathered chunks of kpt entries)
    };
    int64_t tot = 0;
    for (int64_t p = t; p < a.n_pairs; p += 1024) tot += est_of(p);
    tot = block_sum64(tot, red);
    int64_t L = (tot + kResidentPairs - 1) / kResidentPairs;
    L = L > kMinPiece ? L : kMinPiece;
    for (int iter = 0; iter < 48; ++iter) {
        int64_t need = 0;
        for (int64_t p = t; p < a.n_pairs; p += 1024) {
            const int64_t e = est_of(p);
            if (e > L) need += (e + L - 1) / L;
        }
        need = block_sum64(need, red);
        if (need <= P.long_slots) break;
        L *= 2;
    }
    int32_t base = 0, mbase = 0;
    for (int64_t p0 = 0; p0 < a.n_pairs; p0 += 1024) {
        const int64_t p = p0 + t;
        int64_t bA = 0, eA = 0, bB = 0, eB = 0;
        int32_t ns = 0;
        if (p < a.n_pairs) {
            pair_ranges(a, p, bA, eA, bB, eB);
            const int64_t e = (max(eA - bA, eB - bB) + a.kpt - 1) / a.kpt;
            ns = e > L ? (int32_t)((e + L - 1) / L) : 0;
        }
        int32_t tot_ns, tot_sp;
        const int32_t excl = block_scan32(ns, scan, tot_ns);
        const int32_t mex = block_scan32(ns > 0 ? 1 : 0, scan, tot_sp);
        if (p < a.n_pairs) {
            P.pair_flag[p] = ns ? base + excl + 1 : 0;
            if (ns) {
                const int32_t first = base + excl;
                int32_t *me = P.merge + 3 * (int64_t)(mbase + mex);
                me[0] = (int32_t)p;
                me[1] = first;
                me[2] = ns;
                for (int32_t sI = 0; sI < ns; ++sI) {
                    SplitItem it;
                    it.pair = (int32_t)p;
                    it.slot = first + sI;
                    it.a0 = (int32_t)(bA + (eA - bA) * sI / ns);
                    it.a1 = (int32_t)(bA + (eA - bA) * (sI + 1) / ns);
                    it.ra = (int32_t)bA;
                    it.b0 = (int32_t)(bB + (eB - bB) * sI / ns);
                    it.b1 = (int32_t)(bB + (eB - bB) * (sI + 1) / ns);
                    it.rb = (int32_t)bB;
                    P.items[first + sI] = it;
                }
            }
        }
        base += tot_ns;
        mbase += tot_sp;
    }
    // the last round's pairs (the last T in dispatch order, unless already cut), in
    // kTailPieces pieces each when every piece keeps 16 tiles.  Their items are laid
    // out by dispatch position: piece s of tail pair t sits at position
    // 8 (s (T / 8) + t / 8) + t % 8, so that it runs on the XCD that would have run
    // its whole pair (workgroups are dealt to the XCDs round-robin), and an XCD runs
    // the first pieces of its pairs, then the second ones, and so on: pieces that
    // run together walk the same part of the key range and share the L2, as whole
    // pairs do.  An uncut pair leaves empty items; the partial slots stay
    // consecutive per pair.
    __syncthreads();   // every pair_flag above is written
    static_assert(kTailPairs <= 1024 && kTailPairs % 8 == 0, "one pass, whole rounds of XCDs");
    const int64_t T = a.n_pairs >= 2 * kResidentPairs
                          ? min((int64_t)kTailPairs, (int64_t)(P.max_slots - P.long_slots) / kTailPieces) / 8 * 8
                          : 0;
    int32_t tail = 0;
    {
        int64_t p = 0, bA = 0, eA = 0, bB = 0, eB = 0;
        int32_t ns = 0;
        if (t < T) {
            p = xcd_chunk_remap<256>(a.n_pairs - T + t, a.n_pairs);
            if (P.pair_flag[p] == 0) {
                pair_ranges(a, p, bA, eA, bB, eB);
                ns = max(eA - bA, eB - bB) >= (int64_t)16 * kTailPieces * a.kpt ? kTailPieces : 0;
            }
        }
        int32_t tot_ns, tot_sp;
        const int32_t excl = block_scan32(ns, scan, tot_ns);
        const int32_t mex = block_scan32(ns > 0 ? 1 : 0, scan, tot_sp);
        if (t < T) {
            const int32_t first = P.long_slots + excl;
            if (ns) {
                P.pair_flag[p] = first + 1;
                int32_t *me = P.merge + 3 * (int64_t)(mbase + mex);
                me[0] = (int32_t)p;
                me[1] = first;
                me[2] = ns;
            }
            for (int32_t sI = 0; sI < kTailPieces; ++sI) {
                SplitItem it = {};
                it.pair = -1;
                if (sI < ns) {
                    it.pair = (int32_t)p;
                    it.slot = first + sI;
                    it.a0 = (int32_t)(bA + (eA - bA) * sI / ns);
                    it.a1 = (int32_t)(bA + (eA - bA) * (sI + 1) / ns);
                    it.ra = (int32_t)bA;
                    it.b0 = (int32_t)(bB + (eB - bB) * sI / ns);
                    it.b1 = (int32_t)(bB + (eB - bB) * (sI + 1) / ns);
                    it.rb = (int32_t)bB;
                }
                P.items[P.long_slots + 8 * (sI * (T / 8) + t / 8) + t % 8] = it;
            }
        }
        tail = (int32_t)(T * kTailPieces);
        mbase += tot_sp;
    }
    if (t == 0) {
        P.counts[0] = base;
        P.counts[1] = mbase;
        P.counts[2] = (int32_t)L;
        P.counts[3] = tail;
    }
}

// One workgroup per split pair; thread (g, dq, q) combines the pieces of query q of
// block g for d in quarter dq: O = sum_s 2^(lse_s - lse) O_s with
// lse = log2 sum_s 2^(lse_s).
template <int D>
__global__ __launch_bounds__(512) void merge_kernel(AttnArgs a) {
    constexpr int DQ = D / 4;
    const int m = blockIdx.x;
    if (m >= a.plan.counts[1]) return;
    const int32_t *me = a.plan.merge + 3 * (int64_t)m;
    const int64_t pair = me[0];
    const int first = me[1], ns = me[2];
    const int t = threadIdx.x, q = t & 63, dq = (t >> 6) & 3, g = t >> 8;
    const int64_t bh = pair / a.pairs_per_head;
    int32_t blk_a, blk_b;
    pair_blocks((int32_t)(pair % a.pairs_per_head), a.pair_stride, a.nB, blk_a, blk_b);
    const int32_t blk = g ? blk_b : blk_a;
    if (blk < 0) return;
    const int64_t N = (int64_t)a.nB * 64;
    const int64_t qrow = bh * N + (int64_t)blk * 64 + q;
    const float *pl = a.plan.part_lse + ((int64_t)first * 2 + g) * 64 + q;   // piece s at pl[128 s]
    float mx = -INFINITY;
    for (int sI = 0; sI < ns; ++sI) mx = fmaxf(mx, pl[128 * sI]);
    float acc[DQ];
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
    float ltot = -INFINITY;
    if (mx != -INFINITY) {              // else no kept tile in any piece: O = 0
        float sum = 0.f;
        for (int sI = 0; sI < ns; ++sI) sum += __builtin_amdgcn_exp2f(pl[128 * sI] - mx);
        ltot = mx + __log2f(sum);
        for (int sI = 0; sI < ns; ++sI) {
            const float w = __builtin_amdgcn_exp2f(pl[128 * sI] - ltot);
            const float *po = a.plan.part_o + (((int64_t)(first + sI) * 2 + g) * D + dq * DQ) * 64 + q;
#pragma unroll
            for (int e = 0; e < DQ; ++e) acc[e] += w * po[64 * e];
        }
    }
    bf16x8 *og = reinterpret_cast<bf16x8 *>((__bf16 *)a.out + qrow * D + dq * DQ);
#pragma unroll
    for (int e8 = 0; e8 < DQ / 8; ++e8) {
        f32x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[8 * e8 + e];
        og[e8] = __builtin_convertvector(v, bf16x8);
    }
    if (a.lse && dq == 0) a.lse[qrow] = mx == -INFINITY ? -INFINITY : ltot * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 inputs, fp32 MFMA (v_mfma_f32_32x32x2_f32).  Same structure; with
// k = 2 per instruction the S^T accumulators map one-to-one onto the P^T
// operand, so V stays row-major in LDS.  BIAS: each list entry's logit offset
// (col_bias, natural-log units) is added to the scaled scores of its tile before the
// tile's max, so the online softmax takes it in exactly.
template <int D, bool BIAS>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs a) {
    constexpr int KS = D + 1;
    constexpr int VS = D;
    constexpr int NDT = D / 32;
    __shared__ float Ks[64 * KS];
    __shared__ __attribute__((aligned(16))) float Vs[64 * VS];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, hh = lane >> 5, l32 = lane & 31;
    const int64_t row = xcd_remap(blockIdx.x, a.rows);
    const int64_t bh = row / a.nB;
    const int64_t N = (int64_t)a.nB * 64;
    const float *qg = (const float *)a.q + (bh * N + (row % a.nB) * 64) * D;
    const float *kg = (const float *)a.k + bh * N * D;
    const float *vg = (const float *)a.v + bh * N * D;

    int64_t beg = a.row_ptr[row], end = a.row_ptr[row + 1];
    end = end < a.col_count ? end : a.col_count;
    beg = beg < 0 ? 0 : beg;
    const int ntile = end > beg ? (int)(end - beg) : 0;

    float qf[D / 2];
#pragma unroll
    for (int c = 0; c < D / 2; ++c) qf[c] = qg[(32 * wave + l32) * D + 2 * c + hh];

    f32x16 acc_o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[i][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // entries out of range, repeated or below the last accepted column are skipped,
    // exactly as in the bf16 walk
    int last = -1;
    const bool partial = a.geo.partial != 0;
    for (int e = 0; e < ntile; ++e) {
        const int col = a.col_idx[beg + e];
        if (col <= last || col >= a.nB) continue;
        last = col;
        // padding slots of a partial key tile take no weight
        const uint64_t km = partial ? __ballot(slot_valid(a.geo, col, lane)) : ~0ull;
        __syncthreads();
        const float *kt = kg + (int64_t)col * 64 * D;
        const float *vt = vg + (int64_t)col * 64 * D;
        for (int c = t; c < 64 * D / 4; c += 128) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(kt + 4 * c);
            const f32x4 vv = *reinterpret_cast<const f32x4 *>(vt + 4 * c);
            const int key = (4 * c) / D, col4 = (4 * c) % D;
#pragma unroll
            for (int u = 0; u < 4; ++u) Ks[key * KS + col4 + u] = kv[u];
            *reinterpret_cast<f32x4 *>(&Vs[key * VS + col4]) = vv;
        }
        __syncthreads();

        f32x16 acc_s[2];
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc_s[kt2][v] = 0.f;
#pragma unroll
            for (int c = 0; c < D / 2; ++c)
                acc_s[kt2] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[(32 * kt2 + l32) * KS + 2 * c + hh], qf[c],
                                                                  acc_s[kt2], 0, 0, 0);
        }
        if (km != ~0ull) mask_keys(acc_s, km, hh);
        const float beta = BIAS ? a.col_bias[beg + e] * kLog2e : 0.f;
        float mt = -INFINITY;
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc_s[kt2][v] = BIAS ? __builtin_fmaf(acc_s[kt2][v], a.scale_log2, beta) : acc_s[kt2][v] * a.scale_log2;
                mt = fmaxf(mt, acc_s[kt2][v]);
            }
        mt = pair_max(mt);
        const float m_new = fmaxf(m_run, mt);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = exp2f(acc_s[kt2][v] - m_new);
                acc_s[kt2][v] = p;
                ls += p;
            }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc_o[i][v] *= alpha;
        // key of accumulator v of half kt2 for this lane: 32 kt2 + 8 (v/4) + 4 hh + v%4
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = 32 * kt2 + 8 * (v >> 2) + 4 * hh + (v & 3);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VS + 32 * dt + l32], acc_s[kt2][v],
                                                                     acc_o[dt], 0, 0, 0);
            }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const bool qvalid = !partial || slot_valid(a.geo, (int32_t)(row % a.nB), 32 * wave + l32);
    const float inv = (l_tot > 0.f && qvalid) ? 1.f / l_tot : 0.f;
    const int64_t qrow = bh * N + (row % a.nB) * 64 + 32 * wave + l32;
    float *og = (float *)a.out + qrow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 w;
#pragma unroll
            for (int s = 0; s < 4; ++s) w[s] = qvalid ? acc_o[dt][4 * rr + s] * inv : 0.f;
            *reinterpret_cast<f32x4 *>(og + 32 * dt + 8 * rr + 4 * hh) = w;
        }
    if (a.lse && hh == 0)
        a.lse[qrow] = (l_tot > 0.f && qvalid) ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

int launch_plan(const AttnArgs &a, hipStream_t s) {
    plan_kernel<<<1, 1024, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_attention(const AttnArgs &a, int dtype, int d, hipStream_t s) {
    const dim3 pgrid((unsigned)(a.plan.max_slots + a.n_pairs)), pblock(256), grid((unsigned)a.rows), block(128);
    // (long_slots workgroups of long-row pieces, n_pairs of whole pairs, then max_slots -
    // long_slots of last-round pieces)
    const dim3 mgrid((unsigned)a.plan.max_slots), mblock(512);
    if (dtype == 1) {
        plan_kernel<<<1, 1024, 0, s>>>(a);
        const bool bias = a.col_bias != nullptr, gather = a.kpt > 1, masked = a.slot_mask != nullptr;
        if (d == 128) {
            if (gather) attn_bf16_kernel<128, false, true, false><<<pgrid, pblock, 0, s>>>(a);
            else if (bias && masked) attn_bf16_kernel<128, true, false, true><<<pgrid, pblock, 0, s>>>(a);
            else if (bias) attn_bf16_kernel<128, true, false, false><<<pgrid, pblock, 0, s>>>(a);
            else if (masked) attn_bf16_kernel<128, false, false, true><<<pgrid, pblock, 0, s>>>(a);
            else attn_bf16_kernel<128, false, false, false><<<pgrid, pblock, 0, s>>>(a);
            merge_kernel<128><<<mgrid, mblock, 0, s>>>(a);
        } else {
            if (gather) attn_bf16_kernel<64, false, true, false><<<pgrid, pblock, 0, s>>>(a);
            else if (bias && masked) attn_bf16_kernel<64, true, false, true><<<pgrid, pblock, 0, s>>>(a);
            else if (bias) attn_bf16_kernel<64, true, false, false><<<pgrid, pblock, 0, s>>>(a);
            else if (masked) attn_bf16_kernel<64, false, false, true><<<pgrid, pblock, 0, s>>>(a);
            else attn_bf16_kernel<64, false, false, false><<<pgrid, pblock, 0, s>>>(a);
            merge_kernel<64><<<mgrid, mblock, 0, s>>>(a);
        }
    } else if (dtype == 0 && d == 128 && a.col_bias != nullptr)
        attn_f32_kernel<128, true><<<grid, block, 0, s>>>(a);
    else if (dtype == 0 && d == 64 && a.col_bias != nullptr)
        attn_f32_kernel<64, true><<<grid, block, 0, s>>>(a);
    else if (dtype == 0 && d == 128)
        attn_f32_kernel<128, false><<<grid, block, 0, s>>>(a);
    else
        attn_f32_kernel<64, false><<<grid, block, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
