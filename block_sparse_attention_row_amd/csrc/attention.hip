// Block-sparse flash-attention forward over a CSR list of kept 64x64 tiles (gfx950).
//
// For every query block the kernel walks the key blocks of its CSR row and
// runs exact attention with an online softmax, so only the kept tiles are
// computed (the "Expansion" item of the NABLA summary page, "NABLA:
// Neighborhood Adaptive Block-Level Attention", section "Methodologie :
// NABLA").  The result equals a dense softmax over the tokens of the kept
// blocks.
//
// Layout of the work (one workgroup of 2 waves per query block, 32 queries
// per wave):
//   * the transposed score tile S^T = K Q^T is formed on MFMA with K as the
//     A operand (from LDS) and Q as the B operand (kept in registers), so that
//     each lane's accumulators belong to one query: the softmax row max needs
//     one exchange with the partner lane (l ^ 32) and the rescale of the
//     output is a per-lane scalar;
//   * O^T += V^T P^T reuses the S^T accumulators directly as the B operand:
//     the eight accumulators a lane holds for a 16-key chunk are exactly the
//     eight keys it must supply, provided V^T is stored in LDS with the keys
//     of each 16-key chunk in the order {0-3, 8-11, 4-7, 12-15} (the
//     transpose is done in registers while the tile is copied to LDS);
//   * the next tile's K and V are fetched into registers while the current
//     tile is computed.
#include "common.h"
#include "kernels.h"

namespace sattn {

// ---------------------------------------------------------------------------
// bf16 inputs, bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
template <int D>
__global__ __launch_bounds__(128) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KS = D + 8;        // K row stride in LDS (elements)
    constexpr int VS = 64 + 8;       // V^T row stride in LDS (elements)
    constexpr int NDG = D / 8;       // 16-byte column groups per token row
    constexpr int KCH = 64 * NDG / 128;   // K chunks per thread
    constexpr int NDT = D / 32;      // 32-wide d tiles of the output
    __shared__ __attribute__((aligned(16))) __bf16 Ks[64 * KS];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VS];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, hh = lane >> 5, l32 = lane & 31;
    const int64_t row = xcd_remap(blockIdx.x, a.rows);
    const int64_t bh = row / a.nB;
    const int64_t N = (int64_t)a.nB * 64;
    const __bf16 *qg = (const __bf16 *)a.q + (bh * N + (row % a.nB) * 64) * D;
    const __bf16 *kg = (const __bf16 *)a.k + bh * N * D;
    const __bf16 *vg = (const __bf16 *)a.v + bh * N * D;

    int64_t beg = a.row_ptr[row], end = a.row_ptr[row + 1];
    end = end < a.col_count ? end : a.col_count;
    beg = beg < 0 ? 0 : beg;
    const int ntile = end > beg ? (int)(end - beg) : 0;

    // Q fragments (B operand of S^T): query 32*wave + l32, d = 16c + 8hh .. +7
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = *reinterpret_cast<const bf16x8 *>(qg + (32 * wave + l32) * D + 16 * c + 8 * hh);

    // per-thread roles in the tile copy
    const bool vrole = t < 8 * NDG;
    const int vdg = t % NDG, vh = (t / NDG) & 1, vkc = t / (2 * NDG);

    u32x4 kreg[KCH], vreg[8];
    auto fetch = [&](int col) {
        const __bf16 *kt = kg + (int64_t)col * 64 * D;
        const __bf16 *vt = vg + (int64_t)col * 64 * D;
#pragma unroll
        for (int it = 0; it < KCH; ++it) {
            const int c = t + 128 * it;
            kreg[it] = *reinterpret_cast<const u32x4 *>(kt + (c / NDG) * D + (c % NDG) * 8);
        }
        if (vrole) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = 16 * vkc + (e < 4 ? 4 * vh + e : 8 + 4 * vh + (e - 4));
                vreg[e] = *reinterpret_cast<const u32x4 *>(vt + key * D + vdg * 8);
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int it = 0; it < KCH; ++it) {
            const int c = t + 128 * it;
            *reinterpret_cast<u32x4 *>(&Ks[(c / NDG) * KS + (c % NDG) * 8]) = kreg[it];
        }
        if (vrole) {
            // 8 keys x 8 d (16-bit) -> 8 d-rows x 8 keys
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                u32x4 lo, hi;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    lo[m] = __builtin_amdgcn_perm(vreg[2 * m + 1][w], vreg[2 * m][w], 0x05040100u);
                    hi[m] = __builtin_amdgcn_perm(vreg[2 * m + 1][w], vreg[2 * m][w], 0x07060302u);
                }
                const int d0 = vdg * 8 + 2 * w;
                *reinterpret_cast<u32x4 *>(&Vt[d0 * VS + 16 * vkc + 8 * vh]) = lo;
                *reinterpret_cast<u32x4 *>(&Vt[(d0 + 1) * VS + 16 * vkc + 8 * vh]) = hi;
            }
        }
    };

    f32x16 acc_o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[i][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    int e_next = 0;
    auto next_valid = [&](int from) {
        while (from < ntile && (unsigned)a.col_idx[beg + from] >= (unsigned)a.nB) ++from;
        return from;
    };
    e_next = next_valid(0);
    if (e_next < ntile) fetch(a.col_idx[beg + e_next]);

    while (e_next < ntile) {
        __syncthreads();
        stash();
        __syncthreads();
        const int e_cur = e_next;
        e_next = next_valid(e_cur + 1);
        if (e_next < ntile) fetch(a.col_idx[beg + e_next]);

        // S^T = K Q^T for the two 32-key halves
        f32x16 acc_s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc_s[kt][v] = 0.f;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&Ks[(32 * kt + l32) * KS + 16 * c + 8 * hh]);
                acc_s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], acc_s[kt], 0, 0, 0);
            }
        }
        // online softmax in the log2 domain; this lane owns query l32
        float mt = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc_s[kt][v] *= a.scale_log2;
                mt = fmaxf(mt, acc_s[kt][v]);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = exp2f(acc_s[kt][v] - m_new);
                acc_s[kt][v] = p;
                ls += p;
            }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc_o[i][v] *= alpha;

        // O^T += V^T P^T over four 16-key chunks
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const f32x16 &s = acc_s[kc >> 1];
            const int b = 8 * (kc & 1);
            u32x4 pw;
            pw[0] = pack_bf16x2(s[b + 0], s[b + 1]);
            pw[1] = pack_bf16x2(s[b + 2], s[b + 3]);
            pw[2] = pack_bf16x2(s[b + 4], s[b + 5]);
            pw[3] = pack_bf16x2(s[b + 6], s[b + 7]);
            const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&Vt[(32 * dt + l32) * VS + 16 * kc + 8 * hh]);
                acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc_o[dt], 0, 0, 0);
            }
        }
    }

    // epilogue: normalise and store; lane owns query l32, d = 32 dt + 8 rr + 4 hh + {0..3}
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t qrow = bh * N + (row % a.nB) * 64 + 32 * wave + l32;
    __bf16 *og = (__bf16 *)a.out + qrow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            uint2 w;
            w.x = pack_bf16x2(acc_o[dt][4 * rr + 0] * inv, acc_o[dt][4 * rr + 1] * inv);
            w.y = pack_bf16x2(acc_o[dt][4 * rr + 2] * inv, acc_o[dt][4 * rr + 3] * inv);
            *reinterpret_cast<uint2 *>(og + 32 * dt + 8 * rr + 4 * hh) = w;
        }
    if (a.lse && hh == 0) a.lse[qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 inputs, fp32 MFMA (v_mfma_f32_32x32x2_f32).  Same structure; with
// k = 2 per instruction the S^T accumulators map one-to-one onto the P^T
// operand, so V stays row-major in LDS.
template <int D>
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

    for (int e = 0; e < ntile; ++e) {
        const int col = a.col_idx[beg + e];
        if ((unsigned)col >= (unsigned)a.nB) continue;
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
        float mt = -INFINITY;
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc_s[kt2][v] *= a.scale_log2;
                mt = fmaxf(mt, acc_s[kt2][v]);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
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
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t qrow = bh * N + (row % a.nB) * 64 + 32 * wave + l32;
    float *og = (float *)a.out + qrow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            f32x4 w;
#pragma unroll
            for (int s = 0; s < 4; ++s) w[s] = acc_o[dt][4 * rr + s] * inv;
            *reinterpret_cast<f32x4 *>(og + 32 * dt + 8 * rr + 4 * hh) = w;
        }
    if (a.lse && hh == 0) a.lse[qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

int launch_attention(const AttnArgs &a, int dtype, int d, hipStream_t s) {
    const dim3 grid((unsigned)a.rows), block(128);
    if (dtype == 1 && d == 128)
        attn_bf16_kernel<128><<<grid, block, 0, s>>>(a);
    else if (dtype == 1 && d == 64)
        attn_bf16_kernel<64><<<grid, block, 0, s>>>(a);
    else if (dtype == 0 && d == 128)
        attn_f32_kernel<128><<<grid, block, 0, s>>>(a);
    else
        attn_f32_kernel<64><<<grid, block, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
