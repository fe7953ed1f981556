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
        const int64_t tok = ((int64_t)(bt * a.tt + ut) * a.gh + (by * a.th + uy)) * a.gw + (bx * a.tw + ux);
        const int64_t r = ((bh * N + tok) << RL) + off;
        const int64_t t = tile0 + c;
        if (a.inverse) dst[r] = src[t];
        else dst[t] = src[r];
    }
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
