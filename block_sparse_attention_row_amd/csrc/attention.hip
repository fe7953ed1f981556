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
//
// K and V tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (lane p of a wave-wide load lands at M0 + 16 p),
// row-major, the 16-byte slots of row r XOR-swizzled by r mod (slots per row) so
// that operand reads of 16 consecutive rows hit 16 different bank groups.  V is
// read transposed with ds_read_b64_tr_b16: within each 16-lane group, source
// lane 4e + c names 4 consecutive d of key row e, and output lane i receives the
// 4 keys at d = i -- the A-operand layout of O^T = V^T P^T.
//
// The direct loads are issued from inline asm and waited for explicitly, so the
// next K streams in during the softmax and P V of the current tile and the next V
// during the next Q K^T.  Column indices come through the scalar cache.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One wave-wide 16-byte-per-lane load from sbase + voff into LDS at lds_addr + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, const void *sbase) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(4))) int32_t const_i32;

template <int D>
__global__ __launch_bounds__(128, 2) void attn_bf16_kernel(AttnArgs a) {
    constexpr int ROWB = D * 2;                   // bytes per token row
    constexpr int SLOTS = ROWB / 16;              // 16-byte slots per row
    constexpr int RPI = 1024 / ROWB;              // rows written by one wave-wide direct load
    constexpr int IPW = 32 / RPI;                 // direct loads per wave per tile (each wave: 32 rows)
    constexpr int NPAT = SLOTS / RPI;             // distinct per-lane swizzle patterns
    constexpr int NDT = D / 32;                   // 32-wide d tiles of the output
    static_assert(NPAT * RPI * ROWB == ROWB * SLOTS, "pattern period");
    __shared__ __attribute__((aligned(1024))) char Ks[64 * ROWB];
    __shared__ __attribute__((aligned(1024))) char Vs[64 * ROWB];

    const int t = threadIdx.x, lane = t & 63, hh = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t row = xcd_remap(blockIdx.x, a.rows);
    const int64_t bh = row / a.nB;
    const int64_t N = (int64_t)a.nB * 64;
    const __bf16 *qg = (const __bf16 *)a.q + (bh * N + (row % a.nB) * 64) * D;
    const char *kg = (const char *)a.k + bh * N * ROWB + 32 * wave * ROWB;
    const char *vg = (const char *)a.v + bh * N * ROWB + 32 * wave * ROWB;
    const_i32 *rp = (const_i32 *)a.row_ptr;
    const_i32 *cidx = (const_i32 *)a.col_idx;

    int64_t beg = rp[row], end = rp[row + 1];
    end = end < a.col_count ? end : a.col_count;
    beg = beg < 0 ? 0 : beg;
    const int ntile = end > beg ? (int)(end - beg) : 0;

    // Q fragments (B operand of S^T): query 32*wave + l32, d = 16c + 8hh .. +7
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = *reinterpret_cast<const bf16x8 *>(qg + (32 * wave + l32) * D + 16 * c + 8 * hh);
    // settle the Q loads here (vmcnt(0) through the builtin, which the compiler's own
    // wait tracking sees), so that no wait for them lands inside the tile loop, where
    // it would also wait for the in-flight direct loads
    __builtin_amdgcn_s_waitcnt(0x0f70);

    // per-lane source offsets of the direct loads, one per swizzle pattern
    uint32_t voff[NPAT];
#pragma unroll
    for (int j = 0; j < NPAT; ++j) {
        const int r = RPI * j + lane / SLOTS, sl = lane % SLOTS;
        voff[j] = r * ROWB + 16 * (sl ^ (r % SLOTS));
    }
    const uint32_t ks_base = (uint32_t)(uintptr_t)(lds_char *)Ks + 32 * wave * ROWB;
    const uint32_t vs_base = (uint32_t)(uintptr_t)(lds_char *)Vs + 32 * wave * ROWB;
    auto issue = [&](const char *tile, uint32_t lds) {
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            dma16(lds + RPI * i * ROWB, voff[i % NPAT], tile + (i / NPAT) * (NPAT * RPI * ROWB));
    };
    // byte offset of element (r, col) in a swizzled tile (col a multiple of 4)
    auto swz = [](int r, int col) { return r * ROWB + 16 * ((col >> 3) ^ (r % SLOTS)) + 2 * (col & 7); };

    // transposed-read coordinates for the V operand: group g = lane/16, source lane j = 4e + c
    const int tr_e = (lane & 15) >> 2, tr_c = lane & 3, tr_g = lane >> 4;

    f32x16 acc_o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[i][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    auto next_valid = [&](int from) {
        while (from < ntile && (unsigned)cidx[beg + from] >= (unsigned)a.nB) ++from;
        return from;
    };
    int e_cur = next_valid(0);
    if (e_cur < ntile) {
        const int64_t col = cidx[beg + e_cur];
        issue(kg + col * 64 * ROWB, ks_base);
        issue(vg + col * 64 * ROWB, vs_base);
    }

    while (e_cur < ntile) {
        const int e_next = next_valid(e_cur + 1);
        const bool more = e_next < ntile;
        const int64_t col_next = more ? cidx[beg + e_next] : 0;

        wait_vmcnt<IPW>();          // this wave's K loads landed (its V loads may still fly)
        __syncthreads();

        // S^T = K Q^T for the two 32-key halves
        f32x16 acc_s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc_s[kt][v] = 0.f;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + swz(32 * kt + l32, 16 * c + 8 * hh));
                acc_s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], acc_s[kt], 0, 0, 0);
            }
        }
        __syncthreads();            // both waves are done with Ks
        if (more) issue(kg + col_next * 64 * ROWB, ks_base);

        // online softmax; this lane owns query l32.  The running max is kept in raw
        // dot-product units and only moved when a new score exceeds it by more than
        // kLazy (in log2 units): in between, P = 2^(s*c - m*c) stays below 2^kLazy and
        // the output needs no rescaling.  The result is the same softmax.
        float mt = fmaxf(acc_s[0][0], acc_s[0][1]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = (kt == 0 ? 2 : 0); v < 16; v += 2) mt = fmaxf(mt, fmaxf(acc_s[kt][v], acc_s[kt][v + 1]));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const bool grow = (mt - m_run) * a.scale_log2 > kLazy;
        if (__ballot(grow)) {
            const float m_new = grow ? mt : m_run;
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NDT; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc_o[i][v] *= alpha;
        }
        const float mc = m_run * a.scale_log2;
        bf16x8 pf[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            f32x8 pv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[kc >> 1][8 * (kc & 1) + e], a.scale_log2, -mc));
                pv[e] = p;
                l_run += p;
            }
            pf[kc] = __builtin_convertvector(pv, bf16x8);
        }

        if (more) wait_vmcnt<IPW>(); else wait_vmcnt<0>();   // this wave's V loads landed
        __syncthreads();

        // O^T += V^T P^T over four 16-key chunks; slot e of chunk kc is key
        // 16 kc + (e < 4 ? 4 hh + e : 8 + 4 hh + e - 4), matching the accumulators of P
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int col = 32 * dt + 16 * (tr_g & 1) + 4 * tr_c;
                const int r0 = 16 * kc + 4 * (tr_g >> 1) + tr_e;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Vs + swz(r0, col)));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Vs + swz(r0 + 8, col)));
                const bf16x8 vf = __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kc], acc_o[dt], 0, 0, 0);
            }
        }
        __syncthreads();            // both waves are done with Vs
        if (more) issue(vg + col_next * 64 * ROWB, vs_base);
        e_cur = e_next;
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
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = acc_o[dt][4 * rr + e] * inv;
            *reinterpret_cast<bf16x4 *>(og + 32 * dt + 8 * rr + 4 * hh) = __builtin_convertvector(w, bf16x4);
        }
    if (a.lse && hh == 0) a.lse[qrow] = l_tot > 0.f ? (m_run * a.scale_log2 + __log2f(l_tot)) * kLn2 : -INFINITY;
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
