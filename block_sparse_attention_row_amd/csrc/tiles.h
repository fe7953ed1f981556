// LDS tile machinery shared by the bf16 attention kernels (forward and backward).
#pragma once

#include "common.h"

namespace sattn {

// bf16 inputs, bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// K and V tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (lane p of a wave-wide load lands at M0 + 16 p),
// row-major, the 16-byte slots of row r XOR-swizzled by swz_key(r).  The key is
// chosen for both read patterns: the K operand reads one slot of 16 consecutive
// rows (the keys of rows r mod 16 must all differ), and a transposed V read
// takes 4 consecutive slots of 4 consecutive rows (the keys of those rows must
// move the 4-slot group), so that either fills all 64 banks without conflict.  V is
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

// XOR key of the 16-byte slots of tile row r (see above): a bijection on r mod 16
// for 16-slot rows, and on (r >> 1) mod 8 within each row parity for 8-slot rows
// (128-byte rows: even and odd rows sit on opposite halves of the banks).
template <int SLOTS> __device__ __forceinline__ int swz_key(int r) {
    if constexpr (SLOTS == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Tile geometry of the bf16 kernel.
template <int D> struct TileGeo {
    static constexpr int ROWB = D * 2;            // bytes per token row
    static constexpr int SLOTS = ROWB / 16;       // 16-byte slots per row
    static constexpr int RPI = 1024 / ROWB;       // rows written by one wave-wide direct load
    static constexpr int IPW = 16 / RPI;          // direct loads per wave per tensor (each wave: 16 rows)
    static constexpr int NDT = D / 32;            // 32-wide d tiles of the output
    static constexpr int TILEB = 64 * ROWB;
    // byte offset of element (r, col) in a swizzled tile (col a multiple of 4)
    static __device__ __forceinline__ int swz(int r, int col) {
        return r * ROWB + 16 * ((col >> 3) ^ swz_key<SLOTS>(r)) + 2 * (col & 7);
    }
};


// Per-lane byte offsets of a wave's fragment reads within a tile, formed once.  The
// swizzle key depends on the row mod 16 only, so a read of another 16-row chunk, of
// the other 32-key half or of the other tile buffer is one of these plus a
// compile-time constant, which the LDS read takes as its immediate offset (no
// address arithmetic per read).  The empty asm keeps each offset whole in a VGPR.
template <int D> struct FragOffsets {
    static constexpr int NC = D / 16, NDT = D / 32;
    uint32_t k[NC];                 // K operand of S^T: row l32, d = 16 c + 8 hh
    uint32_t vlo[NDT], vhi[NDT];    // transposed V reads of chunk 0, d tile dt: rows r0 and r0 + 8
    __device__ __forceinline__ void init(int lane) {
        const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            k[c] = (uint32_t)TileGeo<D>::swz(l32, 16 * c + 8 * hh);
            asm volatile("" : "+v"(k[c]));
        }
        const int tr_e = (lane & 15) >> 2, tr_c = lane & 3, tr_g = lane >> 4;
        const int r0 = 4 * (tr_g >> 1) + tr_e;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int cc = 32 * dt + 16 * (tr_g & 1) + 4 * tr_c;
            vlo[dt] = (uint32_t)TileGeo<D>::swz(r0, cc);
            vhi[dt] = (uint32_t)TileGeo<D>::swz(r0 + 8, cc);
            asm volatile("" : "+v"(vlo[dt]), "+v"(vhi[dt]));
        }
    }
    // K fragment of key half kt, d chunk c
    __device__ __forceinline__ bf16x8 kfrag(const char *K, int kt, int c) const {
        return *reinterpret_cast<const bf16x8 *>(K + 32 * kt * TileGeo<D>::ROWB + k[c]);
    }
    // O^T-style operand of a 32x32x16 MFMA read transposed from a tile (rows = the
    // summed index): the A operand of X^T Y with X the tile, for 16-row chunk kc and
    // 32-column d tile dt.  Slot e of the fragment is tile row
    // 16 kc + (e < 4 ? 4 hh + e : 8 + 4 hh + e - 4), the row order of the S^T
    // accumulators the B operand takes from.  Its two halves are the transposed
    // 8-byte reads at rows r0 + 16 kc and r0 + 8 + 16 kc.
    __device__ __forceinline__ bf16x8 vfrag(const char *V, int kc, int dt) const {
        const char *base = V + 16 * kc * TileGeo<D>::ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + vlo[dt]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + vhi[dt]));
        return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
};

// S^T = K Q^T for the two 32-key halves of a tile (K from LDS).
template <int D>
__device__ __forceinline__ void tile_scores(const char *K, const bf16x8 *qf, const FragOffsets<D> &fo, f32x16 *acc_s) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_s[kt][v] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            acc_s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo.kfrag(K, kt, c), qf[c], acc_s[kt], 0, 0, 0);
    }
}

// O^T += V^T P^T over four 16-key chunks; slot e of chunk kc is key
// 16 kc + (e < 4 ? 4 hh + e : 8 + 4 hh + e - 4), matching the accumulators of P.
// The transposed V reads run two MFMAs ahead of their use.

template <int D>
__device__ __forceinline__ void tile_pv(const char *V, const bf16x8 *pf, const FragOffsets<D> &fo, f32x16 *acc_o) {
    constexpr int NDT = TileGeo<D>::NDT, NM = 4 * NDT;
    // four-slot ring: the read for MFMA i+2 lands in the slot MFMA i-2 used, so it
    // can be issued before MFMA i without waiting on MFMA i-1's operand reads
    bf16x8 vf[4];
    vf[0] = fo.vfrag(V, 0, 0);
    vf[1] = fo.vfrag(V, 1 / NDT, 1 % NDT);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        if (i + 2 < NM) vf[(i + 2) % 4] = fo.vfrag(V, (i + 2) / NDT, (i + 2) % NDT);
        acc_o[i % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % 4], pf[i / NDT], acc_o[i % NDT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Scores of a key tile whose block is cut by the grid edge (a partial tile): its
// padding slots get kMaskedScore, so they take no weight.  The value is finite: with
// the running max still at -inf on a row's first tile, -inf - (-inf) would be NaN, and
// the device code is compiled without NaN semantics (the first tile's rescale is
// triggered by an infinite row sum instead).  km: bit u set for the slots that are
// grid tokens; accumulator v of half kt of this lane holds key 32 kt + 8 (v / 4) +
// 4 hh + v % 4 (the 32x32 MFMA output layout, keys along its rows).
constexpr float kMaskedScore = -0x1p100f;
// km is wave-uniform: the lanes that keep element (kt, v) form a scalar lane mask
// (lanes 0-31 hold key b of the element, lanes 32-63 key b + 4), applied by one
// select each, with no per-lane shifts of the 64-bit key mask.
__device__ __forceinline__ void mask_keys(f32x16 *sc, uint64_t km, int hh) {
    (void)hh;
    km = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(km >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)km);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int b = 32 * kt + 8 * (v >> 2) + (v & 3);
            const uint64_t lanes = (((km >> b) & 1ull) ? 0x00000000ffffffffull : 0ull) |
                                   (((km >> (b + 4)) & 1ull) ? 0xffffffff00000000ull : 0ull);
            sc[kt][v] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? sc[kt][v] : kMaskedScore;
        }
}

// The same for a tile gathered from 4-token entries (entry e = keys 4e .. 4e + 3): em,
// wave-uniform, has bit e set for the entries kept.  Accumulator v of half kt holds key
// 32 kt + 8 (v / 4) + 4 hh + v % 4, i.e. entry 2 g + hh with g = 4 kt + v / 4, so the
// four accumulators of one g share one lane mask (entry 2 g in lanes 0-31, entry 2 g + 1
// in lanes 32-63): eight masks for the tile's 32 selects.
__device__ __forceinline__ void mask_entries(f32x16 *sc, uint32_t em) {
    em = (uint32_t)__builtin_amdgcn_readfirstlane((int)em);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const uint64_t lanes = (((em >> (2 * g)) & 1u) ? 0x00000000ffffffffull : 0ull) |
                               (((em >> (2 * g + 1)) & 1u) ? 0xffffffff00000000ull : 0ull);
        const bool keep = __builtin_amdgcn_inverse_ballot_w64(lanes);
#pragma unroll
        for (int v = 4 * (g & 3); v < 4 * (g & 3) + 4; ++v)
            sc[g >> 2][v] = keep ? sc[g >> 2][v] : kMaskedScore;
    }
}

}  // namespace sattn
