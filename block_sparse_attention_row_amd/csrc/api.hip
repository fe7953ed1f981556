// C-ABI entry points of libsparse_attn: argument checks, workspace layout and
// kernel launches on the caller's stream.  Every check runs on the host
// before any HIP call, so a rejected call touches neither the device nor the
// outputs.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/sparse_attn.h"
#include "common.h"
#include "kernels.h"

namespace {

using namespace sattn;

constexpr int64_t kAlign = 256;
constexpr int64_t kFineBlocks = 16;     // 4-token key blocks per 64-token tile

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Dims {
    int64_t B, H, D, N, nB, nBp, nW, rows;
    int64_t Nr;                 // raster tokens per head, grid_t * grid_h * grid_w (<= N)
    int32_t nT, nTy, nTx;
    bool partial;               // the grid ends in partial tiles along some axis
};

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Validates the shape and derives the sizes; returns a status.
int32_t check_shape(const sparse_attn_shape *s, Dims *d) {
    if (!s) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (s->batch < 1 || s->heads < 1 || s->grid_t < 1 || s->grid_h < 1 || s->grid_w < 1 || s->tile_t < 1 ||
        s->tile_h < 1 || s->tile_w < 1)
        return SPARSE_ATTN_INVALID_ARGUMENT;
    if (s->dtype != SPARSE_ATTN_F32 && s->dtype != SPARSE_ATTN_BF16) return SPARSE_ATTN_UNSUPPORTED;
    if (s->head_dim != 64 && s->head_dim != 128) return SPARSE_ATTN_UNSUPPORTED;
    if ((int64_t)s->tile_t * s->tile_h * s->tile_w != 64) return SPARSE_ATTN_UNSUPPORTED;
    if (!isfinite(s->scale) || s->scale < 0.f) return SPARSE_ATTN_INVALID_ARGUMENT;
    d->B = s->batch;
    d->H = s->heads;
    d->D = s->head_dim;
    // ceil(grid / tile) tiles; the last along an axis may be partial
    d->nT = (s->grid_t + s->tile_t - 1) / s->tile_t;
    d->nTy = (s->grid_h + s->tile_h - 1) / s->tile_h;
    d->nTx = (s->grid_w + s->tile_w - 1) / s->tile_w;
    d->partial = (s->grid_t % s->tile_t) || (s->grid_h % s->tile_h) || (s->grid_w % s->tile_w);
    d->Nr = (int64_t)s->grid_t * s->grid_h * s->grid_w;
    d->nB = (int64_t)d->nT * d->nTy * d->nTx;
    d->N = d->nB * 64;
    d->nBp = align_up(d->nB, 64);
    d->nW = d->nBp / 64;
    d->rows = d->B * d->H * d->nB;
    // row_ptr / col_idx are int32: the worst-case nnz must fit.
    if (d->rows > INT32_MAX / d->nB) return SPARSE_ATTN_UNSUPPORTED;
    return SPARSE_ATTN_OK;
}

SlotGeo slot_geo(const sparse_attn_shape *s, const Dims &d) {
    SlotGeo g;
    g.nTy = d.nTy;
    g.nTx = d.nTx;
    g.tt = s->tile_t;
    g.th = s->tile_h;
    g.tw = s->tile_w;
    g.gt = s->grid_t;
    g.gh = s->grid_h;
    g.gw = s->grid_w;
    g.partial = d.partial ? 1 : 0;
    return g;
}

float effective_scale(const sparse_attn_shape *s) {
    return s->scale != 0.f ? s->scale : (float)(1.0 / sqrt((double)s->head_dim));
}

int64_t groups_per_head(const Dims &d) { return (d.nB + kGroupRows - 1) / kGroupRows; }
int64_t n_groups(const Dims &d) { return d.B * d.H * groups_per_head(d); }

int64_t n_pairs(const Dims &d) { return d.B * d.H * ((d.nB + 1) / 2); }
int64_t long_slots(const Dims &d) { return n_pairs(d) * 4 < kLongSlots ? n_pairs(d) * 4 : kLongSlots; }
int64_t max_slots(const Dims &d) {
    return long_slots(d) + (n_pairs(d) >= 2 * kResidentPairs ? (int64_t)kTailPairs * kTailPieces : 0);
}

struct Layout {
    int64_t thr, kbar, qbar, status, ticket;                             // selection
    int64_t kbar64, qbar64, knorm;                                       // selection: exact means
    int64_t bits, counts, groups;                                        // external masks
    int64_t items, plan_counts, pair_flag, merge, part_o, part_lse;      // attention row splitting
    int64_t part_b;                                                      // backward: second partial rows
    int64_t col_ptr, lse2, dn;                                           // backward
    int64_t mix;                                                         // clustering selector rows
    int64_t slot_mask;                                                   // partial tiles: token slots per block
    int64_t total;
};

// The clustering selector keeps one fp32 row per pair of query blocks; heads are
// processed in chunks so that the rows take at most about 64 MiB.
int64_t ibcs_row_floats(const Dims &d) { return ((d.nB + 1) / 2) * d.nBp; }
int64_t ibcs_heads_per_launch(const Dims &d) {
    const int64_t per_head = 4 * ibcs_row_floats(d);
    int64_t h = ((int64_t)64 << 20) / (per_head > 0 ? per_head : 1);
    h = h < 1 ? 1 : h;
    return h < d.B * d.H ? h : d.B * d.H;
}

Layout layout(const Dims &d) {
    Layout l;
    int64_t off = 0;
    l.thr = off;
    off = align_up(off + 4 * d.H, kAlign);
    l.kbar = off;
    off = align_up(off + 4 * d.B * d.H * groups_per_head(d) * kGroupRows * d.D, kAlign);   // key means, 16-key groups
    l.qbar = off;
    off = align_up(off + 4 * d.B * d.H * d.nB * d.D, kAlign);   // query means (raster selection)
    l.status = off;
    off = align_up(off + 8 * n_groups(d), kAlign);
    l.ticket = off;
    off = align_up(off + 16, kAlign);
    l.kbar64 = off;
    off = align_up(off + 8 * d.B * d.H * d.nB * d.D, kAlign);   // exact key means
    l.knorm = off;
    off = align_up(off + 4 * d.B * d.H * d.nB, kAlign);         // their norms
    l.qbar64 = off;
    off = align_up(off + 8 * d.B * d.H * d.nB * d.D, kAlign);   // exact query means (raster selection)
    l.bits = off;
    off = align_up(off + 8 * d.rows * d.nW, kAlign);
    l.counts = off;
    off = align_up(off + 4 * d.rows, kAlign);
    l.groups = off;
    off = align_up(off + 4 * n_groups(d), kAlign);
    const int64_t ms = max_slots(d);
    l.items = off;
    off = align_up(off + (int64_t)sizeof(SplitItem) * ms, kAlign);
    l.plan_counts = off;
    off = align_up(off + 16, kAlign);
    l.pair_flag = off;
    off = align_up(off + 4 * n_pairs(d), kAlign);
    l.merge = off;
    off = align_up(off + 12 * ms, kAlign);
    l.part_o = off;
    off = align_up(off + 4 * ms * 2 * 64 * d.D, kAlign);
    l.part_lse = off;
    off = align_up(off + 4 * ms * 2 * 64, kAlign);
    l.part_b = off;
    off = align_up(off + 4 * ms * 2 * 64 * d.D, kAlign);
    l.col_ptr = off;
    off = align_up(off + 4 * (d.rows + 1), kAlign);
    l.lse2 = off;                                   // lse2 then dn: one direct load reaches both
    off = align_up(off + 4 * d.rows * 64, kAlign);
    l.dn = off;
    off = align_up(off + 4 * d.rows * 64, kAlign);
    l.mix = off;
    off = align_up(off + 4 * ibcs_heads_per_launch(d) * ibcs_row_floats(d), kAlign);
    l.slot_mask = off;
    off = align_up(off + 8 * d.nB, kAlign);
    l.total = off;
    return l;
}

bool bad_thr(float t) { return !(t > 0.f); }   // also rejects NaN

// Polls of the selection's look-back before it gives up: kSpinCap, or the value of
// SPARSE_ATTN_LOOKBACK_SPIN_CAP (a debugging knob; 0 gives up at the first poll).
uint32_t lookback_spin_cap() {
    const char *e = getenv("SPARSE_ATTN_LOOKBACK_SPIN_CAP");
    if (!e || !*e) return kSpinCap;
    char *end = nullptr;
    const unsigned long v = strtoul(e, &end, 10);
    return (end && *end == 0 && v <= kSpinCap) ? (uint32_t)v : kSpinCap;
}

int32_t emit_csr(const Dims &d, uint64_t *bits, int32_t *counts, int32_t *groups, int32_t *row_ptr,
                 int32_t *col_idx, hipStream_t st) {
    if (launch_emit(bits, counts, groups, d.rows, (int32_t)d.nB, (int32_t)d.nW, row_ptr, col_idx, st))
        return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

}  // namespace

extern "C" {

int32_t sparse_attn_version(void) { return SPARSE_ATTN_VERSION; }

const char *sparse_attn_status_string(int32_t status) {
    switch (status) {
    case SPARSE_ATTN_OK: return "ok";
    case SPARSE_ATTN_INVALID_ARGUMENT: return "invalid argument";
    case SPARSE_ATTN_UNSUPPORTED: return "unsupported dtype, head_dim, tile or size";
    case SPARSE_ATTN_CAPACITY: return "col_idx capacity below the worst case B*H*nB*nB";
    case SPARSE_ATTN_WORKSPACE: return "workspace smaller than sparse_attn_workspace_size";
    case SPARSE_ATTN_HIP_ERROR: return "HIP kernel launch failed";
    case SPARSE_ATTN_LOOKBACK_FAULT: return "a selection gave up waiting in its CSR look-back; its block list is invalid";
    case SPARSE_ATTN_SCRATCH: return "the shape needs more than the allocation-free selection's 96 MiB static scratch";
    default: return "unknown status";
    }
}

int64_t sparse_attn_csr_capacity(const sparse_attn_shape *shape) {
    Dims d;
    const int32_t st = check_shape(shape, &d);
    if (st) return st;
    return d.rows * d.nB;
}

int64_t sparse_attn_workspace_size(const sparse_attn_shape *shape) {
    Dims d;
    const int32_t st = check_shape(shape, &d);
    if (st) return st;
    return layout(d).total;
}

int32_t sparse_attn_select_check(const sparse_attn_shape *shape, const void *workspace, int64_t workspace_bytes,
                                 void *stream) {
    Dims d;
    const int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!workspace || !aligned(workspace, 16)) return SPARSE_ATTN_INVALID_ARGUMENT;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint32_t word = 0;
    const uint32_t *fault = (const uint32_t *)((const char *)workspace + L.ticket) + 1;
    if (hipMemcpyAsync(&word, fault, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess) return SPARSE_ATTN_HIP_ERROR;
    if (hipStreamSynchronize(s) != hipSuccess) return SPARSE_ATTN_HIP_ERROR;
    return word ? SPARSE_ATTN_LOOKBACK_FAULT : SPARSE_ATTN_OK;
}

static ReorderArgs reorder_args(const sparse_attn_shape *shape, const Dims &d, int inverse) {
    const int64_t rowb = d.D * (shape->dtype == SPARSE_ATTN_BF16 ? 2 : 4);
    ReorderArgs a;
    a.nB = (int32_t)d.nB;
    a.nTy = d.nTy;
    a.nTx = d.nTx;
    a.tt = shape->tile_t;
    a.th = shape->tile_h;
    a.tw = shape->tile_w;
    a.gt = shape->grid_t;
    a.gh = shape->grid_h;
    a.gw = shape->grid_w;
    a.nr = d.Nr;
    a.row_log2 = 0;
    while ((16LL << a.row_log2) < rowb) ++a.row_log2;
    a.inverse = inverse;
    return a;
}

// Device memory the CDF selection works in: per-head thresholds, the key block means,
// the query block means (raster inputs only), the look-back words and the ticket with
// the fault word after it.
struct SelectScratch {
    float *thr;
    __bf16 *kbar, *qbar;
    double *kbar64, *qbar64;
    float *knorm;
    uint64_t *status;
    uint32_t *ticket;
};

// Argument checks of the CDF selection that do not involve the workspace.
static int32_t select_checks(const sparse_attn_shape *shape, const sparse_attn_select_params *params, const void *q,
                             const void *k, int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity, void *q_tiles,
                             void *k_tiles, Dims &d) {
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!params || !q || !k || !row_ptr || !col_idx) return SPARSE_ATTN_INVALID_ARGUMENT;
    const bool raster = q_tiles != nullptr || k_tiles != nullptr;
    if (raster) {
        if (!q_tiles || !k_tiles || q_tiles == k_tiles || q_tiles == q || q_tiles == k || k_tiles == q ||
            k_tiles == k || !aligned(q_tiles, 16) || !aligned(k_tiles, 16))
            return SPARSE_ATTN_INVALID_ARGUMENT;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(row_ptr, 4) || !aligned(col_idx, 4))
        return SPARSE_ATTN_INVALID_ARGUMENT;
    if (d.nBp > kSelectMaxBlocks) return SPARSE_ATTN_UNSUPPORTED;   // a row is held in registers
    if (bad_thr(params->threshold)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (params->head_thresholds)
        for (int64_t h = 0; h < d.H; ++h)
            if (bad_thr(params->head_thresholds[h])) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (col_capacity < d.rows * d.nB) return SPARSE_ATTN_CAPACITY;
    return SPARSE_ATTN_OK;
}

// The CDF selection's launches, once every argument has been checked.  q_tiles ==
// k_tiles == null: q and k are tile-major and the selection pools them.  Otherwise q
// and k are in raster order: they are copied to q_tiles / k_tiles in tile-major order
// and their block means are formed by that copy.
static int32_t select_launch(const sparse_attn_shape *shape, const sparse_attn_select_params *params, const Dims &d,
                             const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                             const SelectScratch &w, void *stream, void *q_tiles, void *k_tiles) {
    const bool raster = q_tiles != nullptr;
    hipStream_t s = (hipStream_t)stream;
    float *thr = w.thr;

    // thresholds: the first ThrChunk::kMax travel with the pooling kernel, any others
    // through small fill kernels
    PoolSide side;
    side.n_thr = (int32_t)(d.H < ThrChunk::kMax ? d.H : ThrChunk::kMax);
    for (int i = 0; i < side.n_thr; ++i)
        side.thr.v[i] = params->head_thresholds ? params->head_thresholds[i] : params->threshold;
    side.thr_dst = thr;
    side.status = w.status;
    side.n_status = n_groups(d);
    side.ticket = w.ticket;
    for (int64_t h0 = ThrChunk::kMax; h0 < d.H; h0 += ThrChunk::kMax) {
        float tmp[ThrChunk::kMax];
        const int n = (int)((d.H - h0) < ThrChunk::kMax ? (d.H - h0) : ThrChunk::kMax);
        for (int i = 0; i < n; ++i)
            tmp[i] = params->head_thresholds ? params->head_thresholds[h0 + i] : params->threshold;
        if (launch_fill_thresholds(tmp, n, thr + h0, s)) return SPARSE_ATTN_HIP_ERROR;
    }
    if (raster) {
        ReorderPoolArgs rp;
        rp.a = reorder_args(shape, d, 0);
        rp.k_src = k;
        rp.q_src = q;
        rp.k_dst = k_tiles;
        rp.q_dst = q_tiles;
        rp.kbar = w.kbar;
        rp.qbar = w.qbar;
        rp.kbar64 = w.kbar64;
        rp.qbar64 = w.qbar64;
        rp.knorm = w.knorm;
        rp.tiles = d.B * d.H * d.nB;
        rp.gph = (int32_t)groups_per_head(d);
        rp.side = side;
        if (launch_reorder_pool(rp, shape->dtype, (int)d.D, s)) return SPARSE_ATTN_HIP_ERROR;
    } else if (launch_pool_keys(k, w.kbar, w.kbar64, w.knorm, d.B * d.H * d.nB, d.nB, shape->dtype, (int)d.D, side,
                                slot_geo(shape, d), s)) {
        return SPARSE_ATTN_HIP_ERROR;
    }

    SelectArgs a = {};
    a.q = raster ? q_tiles : q;
    a.qbar = raster ? w.qbar : nullptr;
    a.qbar64 = raster ? w.qbar64 : nullptr;
    a.kbar = w.kbar;
    a.kbar64 = w.kbar64;
    a.knorm = w.knorm;
    a.geo = slot_geo(shape, d);
    a.thr = thr;
    a.status = w.status;
    a.ticket = w.ticket;
    a.fault = w.ticket + 1;
    a.spin_cap = lookback_spin_cap();
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.rows = d.rows;
    a.groups_per_head = (int32_t)groups_per_head(d);
    a.n_groups = n_groups(d);
    a.H = (int32_t)d.H;
    a.nB = (int32_t)d.nB;
    a.nBp = (int32_t)d.nBp;
    a.nTy = d.nTy;
    a.nTx = d.nTx;
    a.window = params->win_t >= 0 && params->win_h >= 0 && params->win_w >= 0;
    a.wt = params->win_t;
    a.wh = params->win_h;
    a.ww = params->win_w;
    a.scale_log2 = effective_scale(shape) * kLog2e;
    if (launch_select(a, (int)d.D, shape->dtype, s)) return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

static int32_t select_impl(const sparse_attn_shape *shape, const sparse_attn_select_params *params, const void *q,
                           const void *k, int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                           void *workspace, int64_t workspace_bytes, void *stream, void *q_tiles, void *k_tiles) {
    Dims d;
    int32_t st = select_checks(shape, params, q, k, row_ptr, col_idx, col_capacity, q_tiles, k_tiles, d);
    if (st) return st;
    if (!workspace || !aligned(workspace, 16)) return SPARSE_ATTN_INVALID_ARGUMENT;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;
    char *ws = (char *)workspace;
    SelectScratch w;
    w.thr = (float *)(ws + L.thr);
    w.kbar = (__bf16 *)(ws + L.kbar);
    w.qbar = (__bf16 *)(ws + L.qbar);
    w.kbar64 = (double *)(ws + L.kbar64);
    w.qbar64 = (double *)(ws + L.qbar64);
    w.knorm = (float *)(ws + L.knorm);
    w.status = (uint64_t *)(ws + L.status);
    w.ticket = (uint32_t *)(ws + L.ticket);
    return select_launch(shape, params, d, q, k, row_ptr, col_idx, w, stream, q_tiles, k_tiles);
}

int32_t sparse_attn_select(const sparse_attn_shape *shape, const sparse_attn_select_params *params, const void *q,
                           const void *k, int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                           void *workspace, int64_t workspace_bytes, void *stream) {
    return select_impl(shape, params, q, k, row_ptr, col_idx, col_capacity, workspace, workspace_bytes, stream,
                       nullptr, nullptr);
}

int32_t sparse_attn_select_raster(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                  const void *q, const void *k, void *q_tiles, void *k_tiles, int32_t *row_ptr,
                                  int32_t *col_idx, int64_t col_capacity, void *workspace, int64_t workspace_bytes,
                                  void *stream) {
    if (!q_tiles || !k_tiles) return SPARSE_ATTN_INVALID_ARGUMENT;
    return select_impl(shape, params, q, k, row_ptr, col_idx, col_capacity, workspace, workspace_bytes, stream,
                       q_tiles, k_tiles);
}

}  // extern "C"

namespace {
// kpt: key blocks per 64-key tile named by col_idx (1: tiles; 16: 4-token blocks,
// gathered into tiles by the bf16 kernel).
int32_t forward_impl(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                     const int32_t *row_ptr, const int32_t *col_idx, const float *col_bias, int64_t col_count,
                     void *out, float *lse, void *workspace, int64_t workspace_bytes, void *stream, int32_t kpt = 1) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!q || !k || !v || !row_ptr || !out || !workspace) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (col_count < 0 || (col_count > 0 && !col_idx)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(row_ptr, 4) ||
        !aligned(col_idx, 4) || !aligned(col_bias, 4) || !aligned(lse, 4) || !aligned(workspace, 16))
        return SPARSE_ATTN_INVALID_ARGUMENT;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;

    AttnArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.col_bias = col_bias;
    a.col_count = col_count;
    a.out = out;
    a.lse = lse;
    a.rows = d.rows;
    a.pairs_per_head = (int32_t)((d.nB + 1) / 2);
    a.pair_stride = d.nT >= 2 ? (int32_t)(d.nTy * d.nTx) : 1;   // frame-neighbour pairs
    a.n_pairs = n_pairs(d);
    a.nB = (int32_t)d.nB;
    a.nK = (int32_t)(d.nB * kpt);
    a.kpt = kpt;
    a.scale_log2 = effective_scale(shape) * kLog2e;
    char *ws = (char *)workspace;
    a.plan.items = (SplitItem *)(ws + L.items);
    a.plan.counts = (int32_t *)(ws + L.plan_counts);
    a.plan.pair_flag = (int32_t *)(ws + L.pair_flag);
    a.plan.merge = (int32_t *)(ws + L.merge);
    a.plan.part_o = (float *)(ws + L.part_o);
    a.plan.part_lse = (float *)(ws + L.part_lse);
    a.plan.max_slots = (int32_t)max_slots(d);
    a.plan.long_slots = (int32_t)long_slots(d);
    a.geo = slot_geo(shape, d);
    if (d.partial && shape->dtype == SPARSE_ATTN_BF16) {
        a.slot_mask_w = (uint64_t *)(ws + L.slot_mask);
        a.slot_mask = a.slot_mask_w;
    }
    if (launch_attention(a, shape->dtype, (int)d.D, (hipStream_t)stream)) return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

}  // namespace

extern "C" {

int32_t sparse_attn_forward(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                            const int32_t *row_ptr, const int32_t *col_idx, int64_t col_count, void *out,
                            float *lse, void *workspace, int64_t workspace_bytes, void *stream) {
    return forward_impl(shape, q, k, v, row_ptr, col_idx, nullptr, col_count, out, lse, workspace, workspace_bytes,
                        stream);
}

int32_t sparse_attn_forward_gather(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                                   const int32_t *row_ptr, const int32_t *col_idx, int64_t col_count, void *out,
                                   float *lse, void *workspace, int64_t workspace_bytes, void *stream) {
    Dims d;
    const int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (shape->dtype != SPARSE_ATTN_BF16 || d.partial) return SPARSE_ATTN_UNSUPPORTED;
    if (d.nB * kFineBlocks > INT32_MAX) return SPARSE_ATTN_UNSUPPORTED;
    return forward_impl(shape, q, k, v, row_ptr, col_idx, nullptr, col_count, out, lse, workspace, workspace_bytes,
                        stream, kFineBlocks);
}

int32_t sparse_attn_forward_biased(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                                   const int32_t *row_ptr, const int32_t *col_idx, const float *col_bias,
                                   int64_t col_count, void *out, float *lse, void *workspace,
                                   int64_t workspace_bytes, void *stream) {
    if (col_count > 0 && !col_bias) return SPARSE_ATTN_INVALID_ARGUMENT;
    // an empty list has no offsets to apply: the plain kernel gives the same result
    return forward_impl(shape, q, k, v, row_ptr, col_idx, col_count > 0 ? col_bias : nullptr, col_count, out, lse,
                        workspace, workspace_bytes, stream);
}

int32_t sparse_attn_select_sip(const sparse_attn_shape *shape, const sparse_attn_sip_params *params, const void *q,
                               const void *k, int32_t *row_ptr, int32_t *col_idx, float *col_bias,
                               int64_t col_capacity, void *workspace, int64_t workspace_bytes, void *stream) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!params || !q || !k || !row_ptr || !col_idx || !col_bias || !workspace) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(col_bias, 4) ||
        !aligned(workspace, 16))
        return SPARSE_ATTN_INVALID_ARGUMENT;
    if (d.nBp > kSelectMaxBlocks) return SPARSE_ATTN_UNSUPPORTED;   // a row is held in registers
    if (!(params->budget > 0.f) || !(params->budget < INFINITY)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (col_capacity < d.rows * d.nB) return SPARSE_ATTN_CAPACITY;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    __bf16 *kbar = (__bf16 *)(ws + L.kbar);
    uint64_t *status = (uint64_t *)(ws + L.status);
    uint32_t *ticket = (uint32_t *)(ws + L.ticket);
    PoolSide side;
    side.n_thr = 0;
    side.thr_dst = (float *)(ws + L.thr);
    side.status = status;
    side.n_status = n_groups(d);
    side.ticket = ticket;
    if (launch_pool_keys(k, kbar, (double *)(ws + L.kbar64), (float *)(ws + L.knorm), d.B * d.H * d.nB, d.nB,
                         shape->dtype, (int)d.D, side, slot_geo(shape, d), s))
        return SPARSE_ATTN_HIP_ERROR;

    SelectArgs a = {};
    a.q = q;
    a.kbar = kbar;
    a.thr = (const float *)(ws + L.thr);
    a.status = status;
    a.ticket = ticket;
    a.fault = ticket + 1;
    a.spin_cap = lookback_spin_cap();
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.rows = d.rows;
    a.groups_per_head = (int32_t)groups_per_head(d);
    a.n_groups = n_groups(d);
    a.H = (int32_t)d.H;
    a.nB = (int32_t)d.nB;
    a.nBp = (int32_t)d.nBp;
    a.nTy = d.nTy;
    a.nTx = d.nTx;
    a.window = 0;
    a.geo = slot_geo(shape, d);
    a.scale_log2 = effective_scale(shape) * kLog2e;
    a.budget = params->budget;
    a.seed = params->seed;
    a.col_bias = col_bias;
    if (launch_select_sip(a, (int)d.D, shape->dtype, s)) return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

int32_t sparse_attn_select_ibcs(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                                int64_t col_capacity, void *workspace, int64_t workspace_bytes, void *stream) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (d.partial) return SPARSE_ATTN_UNSUPPORTED;   // the 128-token clusters take whole tiles
    if (!params || !q || !k || !row_ptr || !col_idx || !workspace) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(row_ptr, 4) || !aligned(col_idx, 4) ||
        !aligned(workspace, 16))
        return SPARSE_ATTN_INVALID_ARGUMENT;
    if (d.nBp > kSelectMaxBlocks) return SPARSE_ATTN_UNSUPPORTED;   // a row is held in registers
    if (bad_thr(params->threshold)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (params->head_thresholds)
        for (int64_t h = 0; h < d.H; ++h)
            if (bad_thr(params->head_thresholds[h])) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (col_capacity < d.rows * d.nB) return SPARSE_ATTN_CAPACITY;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    float *thr = (float *)(ws + L.thr);
    __bf16 *kbar = (__bf16 *)(ws + L.kbar);
    uint64_t *status = (uint64_t *)(ws + L.status);
    uint32_t *ticket = (uint32_t *)(ws + L.ticket);
    float *rows = (float *)(ws + L.mix);
    PoolSide side;
    side.n_thr = (int32_t)(d.H < ThrChunk::kMax ? d.H : ThrChunk::kMax);
    for (int i = 0; i < side.n_thr; ++i)
        side.thr.v[i] = params->head_thresholds ? params->head_thresholds[i] : params->threshold;
    side.thr_dst = thr;
    side.status = status;
    side.n_status = n_groups(d);
    side.ticket = ticket;
    for (int64_t h0 = ThrChunk::kMax; h0 < d.H; h0 += ThrChunk::kMax) {
        float tmp[ThrChunk::kMax];
        const int n = (int)((d.H - h0) < ThrChunk::kMax ? (d.H - h0) : ThrChunk::kMax);
        for (int i = 0; i < n; ++i)
            tmp[i] = params->head_thresholds ? params->head_thresholds[h0 + i] : params->threshold;
        if (launch_fill_thresholds(tmp, n, thr + h0, s)) return SPARSE_ATTN_HIP_ERROR;
    }
    if (launch_pool_keys(k, kbar, (double *)(ws + L.kbar64), (float *)(ws + L.knorm), d.B * d.H * d.nB, d.nB,
                         shape->dtype, (int)d.D, side, slot_geo(shape, d), s))
        return SPARSE_ATTN_HIP_ERROR;

    IbcsArgs m;
    m.q = q;
    m.kbar = kbar;
    m.rows = rows;
    m.nB = (int32_t)d.nB;
    m.nBp = (int32_t)d.nBp;
    m.pairs_per_head = (int32_t)((d.nB + 1) / 2);
    m.scale_log2 = effective_scale(shape) * kLog2e;
    SelectArgs a = {};
    a.q = q;
    a.kbar = kbar;
    a.thr = thr;
    a.status = status;
    a.ticket = ticket;
    a.fault = ticket + 1;
    a.spin_cap = lookback_spin_cap();
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.rows = d.rows;
    a.groups_per_head = (int32_t)groups_per_head(d);
    a.n_groups = n_groups(d);
    a.H = (int32_t)d.H;
    a.nB = (int32_t)d.nB;
    a.nBp = (int32_t)d.nBp;
    a.nTy = d.nTy;
    a.nTx = d.nTx;
    a.window = params->win_t >= 0 && params->win_h >= 0 && params->win_w >= 0;
    a.wt = params->win_t;
    a.wh = params->win_h;
    a.ww = params->win_w;
    a.scale_log2 = m.scale_log2;
    a.mix_rows = rows;
    // heads in chunks: the rows of a chunk, then its groups' cut (tickets and
    // look-back words continue across the chunks, so the CSR offsets chain through)
    const int64_t BH = d.B * d.H, hpl = ibcs_heads_per_launch(d);
    for (int64_t h0 = 0; h0 < BH; h0 += hpl) {
        const int64_t nh = BH - h0 < hpl ? BH - h0 : hpl;
        m.head0 = h0;
        a.head0 = h0;
        if (launch_ibcs_mix(m, nh, (int)d.D, shape->dtype, s)) return SPARSE_ATTN_HIP_ERROR;
        if (launch_select_rows(a, nh * groups_per_head(d), s)) return SPARSE_ATTN_HIP_ERROR;
    }
    return SPARSE_ATTN_OK;
}

int32_t sparse_attn_mask_to_csr(const sparse_attn_shape *shape, const uint8_t *block_mask, int32_t *row_ptr,
                                int32_t *col_idx, int64_t col_capacity, void *workspace, int64_t workspace_bytes,
                                void *stream) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!block_mask || !row_ptr || !col_idx || !workspace) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(workspace, 16)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (col_capacity < d.rows * d.nB) return SPARSE_ATTN_CAPACITY;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    uint64_t *bits = (uint64_t *)(ws + L.bits);
    int32_t *counts = (int32_t *)(ws + L.counts);
    int32_t *groups = (int32_t *)(ws + L.groups);
    if (launch_mask_bits(block_mask, d.B * d.H, (int32_t)d.nB, (int32_t)d.nW, bits, counts, groups, s))
        return SPARSE_ATTN_HIP_ERROR;
    return emit_csr(d, bits, counts, groups, row_ptr, col_idx, s);
}

int32_t sparse_attn_radial_csr(const sparse_attn_shape *shape, const sparse_attn_radial_params *params,
                               int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity, void *workspace,
                               int64_t workspace_bytes, void *stream) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!params || !row_ptr || !col_idx || !workspace) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(workspace, 16)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!(params->r0 >= 0.f) || !(params->r0 < INFINITY) || !(params->gamma > 0.f) || !(params->gamma <= 1.f) ||
        params->lambda < 0)
        return SPARSE_ATTN_INVALID_ARGUMENT;
    if (d.nB > kSelectMaxBlocks) return SPARSE_ATTN_UNSUPPORTED;   // the radius table sits in LDS
    if (col_capacity < d.rows * d.nB) return SPARSE_ATTN_CAPACITY;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    uint64_t *bits = (uint64_t *)(ws + L.bits);
    int32_t *counts = (int32_t *)(ws + L.counts);
    int32_t *groups = (int32_t *)(ws + L.groups);
    RadialArgs a;
    a.nT = d.nT;
    a.nTy = d.nTy;
    a.nTx = d.nTx;
    a.r0 = params->r0;
    a.gamma = params->gamma;
    a.lambda = params->lambda;
    if (launch_radial_bits(a, d.B * d.H, (int32_t)d.nB, (int32_t)d.nW, bits, counts, groups, s))
        return SPARSE_ATTN_HIP_ERROR;
    return emit_csr(d, bits, counts, groups, row_ptr, col_idx, s);
}

int32_t sparse_attn_backward(const sparse_attn_shape *shape, const void *q, const void *k, const void *v,
                             const void *out, const float *lse, const void *dout, const int32_t *row_ptr,
                             const int32_t *col_idx, int64_t col_count, void *dq, void *dk, void *dv,
                             int32_t *t_idx, void *workspace, int64_t workspace_bytes, void *stream) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (d.nB > kSelectMaxBlocks) return SPARSE_ATTN_UNSUPPORTED;   // a row's bitmask is held in LDS
    if (!q || !k || !v || !out || !lse || !dout || !row_ptr || !dq || !dk || !dv || !workspace)
        return SPARSE_ATTN_INVALID_ARGUMENT;
    if (col_count < 0 || (col_count > 0 && (!col_idx || !t_idx))) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(row_ptr, 4) ||
        !aligned(col_idx, 4) || !aligned(t_idx, 4) || !aligned(workspace, 16))
        return SPARSE_ATTN_INVALID_ARGUMENT;
    const Layout L = layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;
    char *ws = (char *)workspace;
    BwdLaunch b;
    b.args.q = q;
    b.args.k = k;
    b.args.v = v;
    b.args.dout = dout;
    b.args.lse2 = (float *)(ws + L.lse2);
    b.args.dn = (float *)(ws + L.dn);
    b.args.n_pairs = n_pairs(d);
    b.args.pairs_per_head = (int32_t)((d.nB + 1) / 2);
    b.args.pair_stride = d.nT >= 2 ? (int32_t)(d.nTy * d.nTx) : 1;   // frame-neighbour pairs
    b.args.nB = (int32_t)d.nB;
    b.args.scale = effective_scale(shape);
    b.args.scale_log2 = b.args.scale * kLog2e;
    b.args.plan.items = (SplitItem *)(ws + L.items);
    b.args.plan.counts = (int32_t *)(ws + L.plan_counts);
    b.args.plan.pair_flag = (int32_t *)(ws + L.pair_flag);
    b.args.plan.merge = (int32_t *)(ws + L.merge);
    b.args.plan.part_o = nullptr;
    b.args.plan.part_lse = nullptr;
    b.args.plan.max_slots = (int32_t)max_slots(d);
    b.args.plan.long_slots = (int32_t)long_slots(d);
    b.args.part = (float *)(ws + L.part_o);
    b.args.part2 = (float *)(ws + L.part_b);
    b.geo = slot_geo(shape, d);
    b.args.geo = b.geo;
    b.f32 = shape->dtype == SPARSE_ATTN_F32;
    b.slot_mask_w = (d.partial && !b.f32) ? (uint64_t *)(ws + L.slot_mask) : nullptr;
    b.args.slot_mask = b.slot_mask_w;
    b.out = out;
    b.lse = lse;
    b.lse2 = (float *)(ws + L.lse2);
    b.dn = (float *)(ws + L.dn);
    b.row_ptr = row_ptr;
    b.col_idx = col_idx;
    b.col_count = col_count;
    b.bits = (uint64_t *)(ws + L.bits);
    b.colcount = (int32_t *)(ws + L.counts);
    b.col_ptr = (int32_t *)(ws + L.col_ptr);
    b.t_idx = t_idx;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.rows = d.rows;
    b.BH = d.B * d.H;
    b.nB = (int32_t)d.nB;
    b.nW = (int32_t)d.nW;
    b.d = (int32_t)d.D;
    if (launch_backward(b, (hipStream_t)stream)) return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

int32_t sparse_attn_full_csr(const sparse_attn_shape *shape, int32_t *row_ptr, int32_t *col_idx,
                             int64_t col_capacity, void *stream) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!row_ptr || !col_idx) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(row_ptr, 4) || !aligned(col_idx, 4)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (col_capacity < d.rows * d.nB) return SPARSE_ATTN_CAPACITY;
    if (launch_full_csr(d.rows, (int32_t)d.nB, row_ptr, col_idx, (hipStream_t)stream)) return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

static int32_t reorder(const sparse_attn_shape *shape, const void *src, void *dst, void *stream, int inverse) {
    Dims d;
    int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (!src || !dst || src == dst) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(src, 16) || !aligned(dst, 16)) return SPARSE_ATTN_INVALID_ARGUMENT;
    const ReorderArgs a = reorder_args(shape, d, inverse);
    if (launch_reorder(src, dst, a, d.B * d.H * d.nB, (hipStream_t)stream)) return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

int32_t sparse_attn_to_tiles(const sparse_attn_shape *shape, const void *src, void *dst, void *stream) {
    return reorder(shape, src, dst, stream, 0);
}

int32_t sparse_attn_from_tiles(const sparse_attn_shape *shape, const void *src, void *dst, void *stream) {
    return reorder(shape, src, dst, stream, 1);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Selection of 4-token key blocks (AB-Attention's fine blocks) per 64-token query
// block, with NABLA's CDF cut.  Its workspace: thresholds, the fp32 key-block means
// in planes of 4 columns and their norms, look-back words, ticket and fault word.
namespace {

constexpr int64_t kFineMaxBlocks = 512;   // nB: 8 words of 64 keys a lane per wave

struct FineLayout {
    int64_t thr, kf, knorm, status, ticket, total;
};

int64_t fine_groups(const Dims &d) { return d.B * d.H * ((d.nB + fine_rows(fine_words(d.nB * kFineBlocks)) - 1) /
                                                          fine_rows(fine_words(d.nB * kFineBlocks))); }

FineLayout fine_layout(const Dims &d) {
    const int64_t nK = d.nB * kFineBlocks;
    FineLayout l;
    int64_t off = 0;
    l.thr = off;
    off = align_up(off + 4 * d.H, kAlign);
    l.kf = off;
    off = align_up(off + 4 * d.B * d.H * nK * d.D, kAlign);
    l.knorm = off;
    off = align_up(off + 4 * d.B * d.H * nK, kAlign);
    l.status = off;
    off = align_up(off + 8 * fine_groups(d), kAlign);
    l.ticket = off;
    off = align_up(off + 16, kAlign);
    l.total = off;
    return l;
}

// Shape checks of the fine selection: bf16, whole tiles, nB <= kFineMaxBlocks, and a
// worst case of rows * 16 nB entries that int32 offsets can address.
int32_t fine_shape(const sparse_attn_shape *shape, Dims &d) {
    const int32_t st = check_shape(shape, &d);
    if (st) return st;
    if (shape->dtype != SPARSE_ATTN_BF16 || d.partial || d.nB > kFineMaxBlocks) return SPARSE_ATTN_UNSUPPORTED;
    if (d.rows > INT32_MAX / (d.nB * kFineBlocks)) return SPARSE_ATTN_UNSUPPORTED;
    return SPARSE_ATTN_OK;
}

}  // namespace

extern "C" {

int64_t sparse_attn_fine_csr_capacity(const sparse_attn_shape *shape) {
    Dims d;
    const int32_t st = fine_shape(shape, d);
    return st ? st : d.rows * d.nB * kFineBlocks;
}

int64_t sparse_attn_fine_workspace_size(const sparse_attn_shape *shape) {
    Dims d;
    const int32_t st = fine_shape(shape, d);
    return st ? st : fine_layout(d).total;
}

int32_t sparse_attn_select_fine(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                                int64_t col_capacity, void *workspace, int64_t workspace_bytes, void *stream) {
    Dims d;
    int32_t st = fine_shape(shape, d);
    if (st) return st;
    if (!params || !q || !k || !row_ptr || !col_idx || !workspace) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(workspace, 16))
        return SPARSE_ATTN_INVALID_ARGUMENT;
    if (bad_thr(params->threshold)) return SPARSE_ATTN_INVALID_ARGUMENT;
    if (params->head_thresholds)
        for (int64_t h = 0; h < d.H; ++h)
            if (bad_thr(params->head_thresholds[h])) return SPARSE_ATTN_INVALID_ARGUMENT;
    // the window is a box in 64-token block coordinates: not defined for 4-token blocks
    if (params->win_t >= 0 && params->win_h >= 0 && params->win_w >= 0) return SPARSE_ATTN_UNSUPPORTED;
    const int64_t nK = d.nB * kFineBlocks;
    if (col_capacity < d.rows * nK) return SPARSE_ATTN_CAPACITY;
    const FineLayout L = fine_layout(d);
    if (workspace_bytes < L.total) return SPARSE_ATTN_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    float *thr = (float *)(ws + L.thr);
    PoolSide side;
    side.n_thr = (int32_t)(d.H < ThrChunk::kMax ? d.H : ThrChunk::kMax);
    for (int i = 0; i < side.n_thr; ++i)
        side.thr.v[i] = params->head_thresholds ? params->head_thresholds[i] : params->threshold;
    side.thr_dst = thr;
    side.status = (uint64_t *)(ws + L.status);
    side.n_status = fine_groups(d);
    side.ticket = (uint32_t *)(ws + L.ticket);
    for (int64_t h0 = ThrChunk::kMax; h0 < d.H; h0 += ThrChunk::kMax) {
        float tmp[ThrChunk::kMax];
        const int n = (int)((d.H - h0) < ThrChunk::kMax ? (d.H - h0) : ThrChunk::kMax);
        for (int i = 0; i < n; ++i)
            tmp[i] = params->head_thresholds ? params->head_thresholds[h0 + i] : params->threshold;
        if (launch_fill_thresholds(tmp, n, thr + h0, s)) return SPARSE_ATTN_HIP_ERROR;
    }
    float *kf = (float *)(ws + L.kf);
    float *knorm = (float *)(ws + L.knorm);
    if (launch_fine_pool((const __bf16 *)k, kf, knorm, nK, d.B * d.H * nK, (int)d.D, side, s))
        return SPARSE_ATTN_HIP_ERROR;
    const int W = fine_words(nK), R = fine_rows(W);
    FineArgs a = {};
    a.q = (const __bf16 *)q;
    a.k = (const __bf16 *)k;
    a.kf = kf;
    a.knorm = knorm;
    a.thr = thr;
    a.status = side.status;
    a.ticket = side.ticket;
    a.fault = side.ticket + 1;
    a.spin_cap = lookback_spin_cap();
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.rows = d.rows;
    a.groups_per_head = (int32_t)((d.nB + R - 1) / R);
    a.n_groups = fine_groups(d);
    a.H = (int32_t)d.H;
    a.nB = (int32_t)d.nB;
    a.nK = (int32_t)nK;
    a.S = (int32_t)((nK + kFineWaves - 1) / kFineWaves);
    a.scale_log2 = effective_scale(shape) * kLog2e;
    if (launch_fine_select(a, (int)d.D, s)) return SPARSE_ATTN_HIP_ERROR;
    return SPARSE_ATTN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free selection.  The CDF selection's scratch (thresholds, key block
// means, look-back words, ticket and fault word) lives in a static device array
// instead of a caller's workspace.  Each GPU holds its own copy of the array at its
// own address, which hipGetSymbolAddress returns with that device current; host code
// uses only that address (the array's name on the host is a stand-in, not a device
// address).  Every call on one GPU shares its array; the pooling kernel clears the
// look-back words, the ticket and the fault word at the start of each call.
static __device__ __align__(256) unsigned char scratch[SPARSE_ATTN_SCRATCH_BYTES];

namespace {

constexpr int64_t kScratchBytes = SPARSE_ATTN_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array, looked up once per device.
int32_t device_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SPARSE_ATTN_HIP_ERROR;
    if (dev < 0 || dev >= kMaxDevices) return SPARSE_ATTN_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPARSE_ATTN_HIP_ERROR;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPARSE_ATTN_OK;
}

// The selection's part of the workspace, packed: thresholds, key means, look-back
// words, ticket.
struct ScratchLayout {
    int64_t thr, kbar, kbar64, knorm, status, ticket, total;
};
ScratchLayout scratch_layout(const Dims &d) {
    ScratchLayout l;
    int64_t off = 0;
    l.thr = off;
    off = align_up(off + 4 * d.H, kAlign);
    l.kbar = off;
    off = align_up(off + 4 * d.B * d.H * groups_per_head(d) * kGroupRows * d.D, kAlign);
    l.kbar64 = off;
    off = align_up(off + 8 * d.B * d.H * d.nB * d.D, kAlign);
    l.knorm = off;
    off = align_up(off + 4 * d.B * d.H * d.nB, kAlign);
    l.status = off;
    off = align_up(off + 8 * n_groups(d), kAlign);
    l.ticket = off;
    off = align_up(off + 16, kAlign);
    l.total = off;
    return l;
}

}  // namespace

extern "C" {

int64_t sparse_attn_select_noalloc_bytes(const sparse_attn_shape *shape) {
    Dims d;
    const int32_t st = check_shape(shape, &d);
    if (st) return st;
    return scratch_layout(d).total;
}

int32_t sparse_attn_select_noalloc(const sparse_attn_shape *shape, const sparse_attn_select_params *params,
                                   const void *q, const void *k, int32_t *row_ptr, int32_t *col_idx,
                                   int64_t col_capacity, void *stream) {
    Dims d;
    int32_t st = select_checks(shape, params, q, k, row_ptr, col_idx, col_capacity, nullptr, nullptr, d);
    if (st) return st;
    const ScratchLayout L = scratch_layout(d);
    if (L.total > kScratchBytes) return SPARSE_ATTN_SCRATCH;
    void *base = nullptr;
    st = device_scratch(&base);
    if (st) return st;
    char *ws = (char *)base;
    SelectScratch w;
    w.thr = (float *)(ws + L.thr);
    w.kbar = (__bf16 *)(ws + L.kbar);
    w.qbar = nullptr;
    w.kbar64 = (double *)(ws + L.kbar64);
    w.qbar64 = nullptr;
    w.knorm = (float *)(ws + L.knorm);
    w.status = (uint64_t *)(ws + L.status);
    w.ticket = (uint32_t *)(ws + L.ticket);
    return select_launch(shape, params, d, q, k, row_ptr, col_idx, w, stream, nullptr, nullptr);
}

}  // extern "C"
