// Token reordering between raster order and tile-major order (gfx950).
//
// The NABLA summary page ("NABLA: Neighborhood Adaptive Block-Level Attention",
// section "Methodologie : NABLA", item "Fractal Flattening") reorders the tokens so
// that those of each spatial patch are contiguous; with 64-token tiles that is one
// level of tiling: block b = (bt, by, bx) holds the tokens of tile b, row-major inside
// the tile.  Pure data movement: one workgroup per tile copies its 64 token rows in
// 16-byte pieces; each wave moves whole tile rows, which are contiguous in both
// orders (a tile row is tile_w consecutive raster tokens).
#include "common.h"
#include "kernels.h"

namespace sattn {

template <int RL>   // log2 of the 16-byte pieces per token row
__global__ __launch_bounds__(256) void reorder_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                      ReorderArgs a) {
    constexpr int PER = 64 << RL, IT = PER / 256;       // pieces per tile, per thread
    const int64_t b = blockIdx.x;                        // tile over B*H*nB
    const int64_t bh = b / a.nB;
    const int blk = (int)(b - bh * a.nB);
    const int bt = blk / (a.nTy * a.nTx), by = (blk / a.nTx) % a.nTy, bx = blk % a.nTx;
    const int64_t N = (int64_t)a.nB * 64;
    const int64_t tile0 = (bh * N + (int64_t)blk * 64) << RL;                  // 16-byte units
    const int tyx = a.th * a.tw;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int c = 256 * i + threadIdx.x;
        const int u = c >> RL, off = c & ((1 << RL) - 1);
        const int ut = u / tyx, uy = (u / a.tw) % a.th, ux = u % a.tw;
        const int t0 = bt * a.tt + ut, y0 = by * a.th + uy, x0 = bx * a.tw + ux;
        const bool in = t0 < a.gt && y0 < a.gh && x0 < a.gw;       // else a partial tile's padding slot
        const int64_t tok = ((int64_t)t0 * a.gh + y0) * a.gw + x0;
        const int64_t r = ((bh * a.nr + tok) << RL) + off;
        const int64_t t = tile0 + c;
        if (a.inverse) {
            if (in) dst[r] = src[t];
        } else {
            dst[t] = in ? src[r] : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Raster -> tile-major copy of K and Q with each tile's mean formed on the way (the
// selection's "Sous-echantillonnage" fused into the reorder): one workgroup per tile,
// the key tiles first, then the query tiles.  Thread t moves the 16-byte pieces t,
// t + 256, .. of the tile, which all hold the same column slice (256 is a multiple of
// the pieces per token row), sums them in fp32, and the sums of the threads that
// share a slice meet in LDS.  The mean goes out as a bf16 pair (hi = bf16(x), lo =
// bf16(x - hi)): for keys in the fragment order of kbar_group, for queries as a
// [hi | lo] row per block.  Side jobs for the selection that follows, as in the
// pooling kernel.
template <typename T, int D>
__global__ __launch_bounds__(256) void reorder_pool_kernel(ReorderPoolArgs p) {
    constexpr int VEC = 16 / (int)sizeof(T), PR = D / VEC;   // elements per piece, pieces per token row
    constexpr int PER = 64 * PR, IT = PER / 256, SHARE = 256 / PR;
    static_assert(PER % 256 == 0 && 256 % PR == 0, "pieces per thread");
    __shared__ double red[SHARE][PR][VEC + 1];
    const int t = threadIdx.x;
    const ReorderArgs &a = p.a;
    const int64_t gt = (int64_t)blockIdx.x * blockDim.x + t;
    if (blockIdx.x == 0 && t < p.side.n_thr) p.side.thr_dst[t] = p.side.thr.v[t];
    for (int64_t i = gt; i < p.side.n_status; i += (int64_t)gridDim.x * blockDim.x) p.side.status[i] = 0;
    if (gt == 0) {
        p.side.ticket[0] = 0u;
        p.side.ticket[1] = 0u;
    }
    const bool keys = (int64_t)blockIdx.x < p.tiles;
    const int64_t b = keys ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - p.tiles;   // tile over B*H*nB
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(keys ? p.k_src : p.q_src);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(keys ? p.k_dst : p.q_dst);
    const int64_t bh = b / a.nB;
    const int blk = (int)(b - bh * a.nB);
    const int bt = blk / (a.nTy * a.nTx), by = (blk / a.nTx) % a.nTy, bx = blk % a.nTx;
    const int64_t N = (int64_t)a.nB * 64;
    const int tyx = a.th * a.tw;
    const int off = t % PR;                                   // the same slice for every piece of this thread
    u32x4 buf[IT];
    int cnt = 0;                                              // grid tokens among this thread's slots
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int u = (256 * i + t) / PR;                     // token inside the tile
        const int ut = u / tyx, uy = (u / a.tw) % a.th, ux = u % a.tw;
        const int t0 = bt * a.tt + ut, y0 = by * a.th + uy, x0 = bx * a.tw + ux;
        const bool in = t0 < a.gt && y0 < a.gh && x0 < a.gw;  // else a partial tile's padding slot
        const int64_t tok = ((int64_t)t0 * a.gh + y0) * a.gw + x0;
        buf[i] = in ? s4[(bh * a.nr + tok) * PR + off] : u32x4{0u, 0u, 0u, 0u};
        cnt += in ? 1 : 0;
    }
    // sums in fp64: exact for 64 bf16 values, so the means are exact
    double acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        d4[(bh * N + (int64_t)blk * 64) * PR + 256 * i + t] = buf[i];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (sizeof(T) == 2) {
                acc[2 * c] += (double)bf16_lo(buf[i][c]);
                acc[2 * c + 1] += (double)bf16_hi(buf[i][c]);
            } else {
                acc[c] += (double)__uint_as_float(buf[i][c]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[t / PR][off][e] = acc[e];
    red[t / PR][off][VEC] = (double)cnt;
    __syncthreads();
    if (t >= PR) return;
    double ntok = 0.0;                                        // tokens of the tile (64 unless partial)
    for (int g = 0; g < SHARE; ++g) ntok += red[g][t][VEC];
    typedef __attribute__((ext_vector_type(VEC))) float fv;
    typedef __attribute__((ext_vector_type(VEC))) __bf16 bv;
    fv xv, rv;
    double x64[VEC];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        double v = 0.0;
        for (int g = 0; g < SHARE; ++g) v += red[g][t][e];
        x64[e] = ntok == 64.0 ? v * (1.0 / 64.0) : v / ntok;
        xv[e] = (float)x64[e];
        ss += xv[e] * xv[e];
    }
    {
        double *m64 = (keys ? p.kbar64 : p.qbar64) + (bh * a.nB + blk) * D + t * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 2) *reinterpret_cast<double2 *>(m64 + e) = double2{x64[e], x64[e + 1]};
    }
    if (keys) {
        // the key mean's norm: the PR threads of the first wave hold its slices
#pragma unroll
        for (int o = 1; o < PR; o <<= 1) ss += __shfl_xor(ss, o, 64);
        if (t == 0) p.knorm[bh * a.nB + blk] = sqrtf(ss);
    }
    const bv hi = __builtin_convertvector(xv, bv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) rv[e] = xv[e] - (float)hi[e];
    const bv lo = __builtin_convertvector(rv, bv);
    const int d0 = t * VEC;                                   // this thread's columns d0 .. d0 + VEC - 1
    if (keys) {
        const int kb = d0 / 32, kq = (d0 % 32) / 8;
        __bf16 *at = p.kbar + kbar_group(bh, p.gph, blk / 16, D) + 512 * kb + 8 * (blk % 16 + 16 * kq) + d0 % 8;
        *reinterpret_cast<bv *>(at) = hi;
        *reinterpret_cast<bv *>(at + 16 * D) = lo;
    } else {
        __bf16 *row = p.qbar + (bh * a.nB + blk) * (2 * D);
        *reinterpret_cast<bv *>(row + d0) = hi;
        *reinterpret_cast<bv *>(row + D + d0) = lo;
    }
}

int launch_reorder_pool(const ReorderPoolArgs &p, int dtype, int d, hipStream_t s) {
    const dim3 g((unsigned)(2 * p.tiles)), blk(256);
    if (dtype == 1 && d == 128)
        reorder_pool_kernel<__bf16, 128><<<g, blk, 0, s>>>(p);
    else if (dtype == 1 && d == 64)
        reorder_pool_kernel<__bf16, 64><<<g, blk, 0, s>>>(p);
    else if (dtype == 0 && d == 128)
        reorder_pool_kernel<float, 128><<<g, blk, 0, s>>>(p);
    else
        reorder_pool_kernel<float, 64><<<g, blk, 0, s>>>(p);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_reorder(const void *src, void *dst, const ReorderArgs &a, int64_t tiles, hipStream_t s) {
    const dim3 g((unsigned)tiles), blk(256);
    if (a.row_log2 == 3)
        reorder_kernel<3><<<g, blk, 0, s>>>((const u32x4 *)src, (u32x4 *)dst, a);
    else if (a.row_log2 == 4)
        reorder_kernel<4><<<g, blk, 0, s>>>((const u32x4 *)src, (u32x4 *)dst, a);
    else
        reorder_kernel<5><<<g, blk, 0, s>>>((const u32x4 *)src, (u32x4 *)dst, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sattn
