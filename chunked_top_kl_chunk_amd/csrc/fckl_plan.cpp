// fckl_plan.cpp -- argument checks, workspace layout and the chunk scheduler.
//
// Host-only code: nothing here calls HIP, so it is usable (and tested) without a GPU.
// The method processes the sequence one chunk of tokens at a time and discards each
// chunk's intermediate results before the next ("Breaking the Bottleneck with Offline
// Caching and Chunked Loss", axbrief.com); the scheduler below decides how many tokens
// a chunk holds so that every intermediate fits a memory budget that does not grow
// with N.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fckl_internal.h"

namespace fckl {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
static int64_t tiles(int64_t n, int64_t t) { return (n + t - 1) / t; }

fckl_status check_desc(const fckl_desc *d)
{
    if (!d)
        return FCKL_ERR_INVALID_ARG;
    if (d->N < 1 || d->N > INT32_MAX || d->H < 8 || d->V < 1 || d->K < 1)
        return FCKL_ERR_INVALID_ARG;
    if (!(d->T > 0.0f) || !std::isfinite(d->T))
        return FCKL_ERR_INVALID_ARG;
    if (d->K > d->V || d->chunk < 0 || d->vocab_slab < 0 || d->vocab_slab % kVocabTile != 0)
        return FCKL_ERR_INVALID_ARG;
    if (d->logit_dtype != FCKL_DTYPE_BF16 && d->logit_dtype != FCKL_DTYPE_F32)
        return FCKL_ERR_INVALID_ARG;
    if (d->flags & ~(uint32_t)(FCKL_FLAG_VALIDATE | FCKL_FLAG_DW_ACCUMULATE | FCKL_FLAG_TOPK_FULL_FIRST_PASS))
        return FCKL_ERR_INVALID_ARG;
    if (d->H % 8 != 0)
        return FCKL_ERR_UNSUPPORTED;
    if (d->K > kMaxK || d->H > 65536 || d->V > kMaxPitch)
        return FCKL_ERR_UNSUPPORTED;
    if (tiles(d->V, kVocabTile) * tiles(d->H, kHiddenTile) > kMaxTiles)
        return FCKL_ERR_UNSUPPORTED;
    return FCKL_OK;
}

// The token dimension of a chunk of Cpad tokens (padded) within the kernels' limits
// (see kMaxPitch and kMaxTiles).
static bool chunk_supported(int64_t Cpad, int32_t H)
{
    return Cpad <= kMaxPitch && tiles(Cpad, kTokenTile) * tiles(H, kHiddenTile) <= kMaxTiles &&
           Cpad * (int64_t)H <= kMaxChunkElems;
}

// Number of vocabulary splits of the dH product (its reduction runs over V).  Each
// split streams a V/S slice of W; enough splits keep that slice inside the 256 MB
// last-level cache, and among the candidates the one whose work-group count
// best fills whole waves of the 256 compute units wins.  At least 4 k-steps of 64 per
// split; at most 32 splits.
static int32_t dh_split_count(int32_t Cpad, int32_t H, int32_t Vpad)
{
    const int64_t tiles = (int64_t)(Cpad / kTokenTile) * ((H + kHiddenTile - 1) / kHiddenTile);
    // bytes of W per split: inside the 256 MB last-level cache; 224 rather than 192 MB lets
    // a 274-tile vocabulary slab at H = 2880 (404 MB) take 2 splits rather than 4 (-0.17 ms
    // per step at 32K tokens, and two fewer partial sums)
    const int64_t slice_cap = (int64_t)224 << 20;
    int64_t smin = ((int64_t)Vpad * H * 2 + slice_cap - 1) / slice_cap;
    int64_t smax = std::min<int64_t>(32, Vpad / 256);
    smin = std::max<int64_t>(1, std::min(smin, smax));
    // the smallest split count from smin that fills 97% of its waves, else the best fill
    int64_t best = smin;
    double best_eff = -1.0;
    for (int64_t s = smin; s <= smax; ++s) {
        const int64_t wgs = tiles * s;
        const int64_t waves = (wgs + 255) / 256;
        const double eff = (double)wgs / (double)(waves * 256);
        if (eff >= 0.97)
            return (int32_t)s;
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = s;
        }
    }
    return (int32_t)best;
}

int32_t slab_split_count(int32_t Cpad, int32_t H, int32_t nvt)
{
    return dh_split_count(Cpad, H, nvt * kVocabTile);
}

void slab_tiles_of(const Layout &L, int32_t s, int32_t *vt0, int32_t *nvt)
{
    *vt0 = s * L.slab_tiles;
    *nvt = s + 1 < L.nslab ? L.slab_tiles : L.nVt - *vt0;
}

void slab_split_rows(const Layout &L, int32_t V, int32_t H, int32_t s, int32_t *ksplit, int32_t *used)
{
    int32_t vt0, nvt;
    slab_tiles_of(L, s, &vt0, &nvt);
    const int32_t splits = slab_split_count(L.Cpad, H, nvt);
    const int32_t rows = nvt * kVocabTile, vrows = std::min(V - vt0 * kVocabTile, rows);
    *ksplit = ((rows + splits - 1) / splits + kDhStep - 1) / kDhStep * kDhStep;
    *used = (vrows + *ksplit - 1) / *ksplit;
}

int32_t dh_partials(const Layout &L, int32_t V, int32_t H, int32_t nslabs)
{
    int32_t total = 0;
    for (int32_t s = 0; s < nslabs; ++s) {
        int32_t ksplit = 0, used = 0;
        slab_split_rows(L, V, H, s, &ksplit, &used);
        total += used;
    }
    return total;
}

// Slabs of the two-pass backward: the descriptor's, else whole multiples of
// kSlabTileStep tiles whose g^T holds at most about kSlabBytes, as many as round
// nVt / slab to the nearest (the last slab takes the remainder).
static void plan_slabs(const fckl_desc *d, Layout &o)
{
    int32_t st = o.nVt;
    if (d->vocab_slab > 0) {
        st = d->vocab_slab / kVocabTile;
    } else {
        const size_t tile_bytes = (size_t)kVocabTile * (size_t)o.Cpad * 2;
        st = std::max<int32_t>(kSlabTileStep, (int32_t)(kSlabBytes / tile_bytes) / kSlabTileStep * kSlabTileStep);
    }
    if (st >= o.nVt) {
        o.nslab = 1;
        o.slab_tiles = o.nVt;
    } else {
        o.nslab = d->vocab_slab > 0 ? o.nVt / st : std::max<int32_t>(1, (o.nVt + st / 2) / st);
        o.slab_tiles = o.nslab > 1 ? st : o.nVt;
    }
    o.gT_tiles = 0;
    o.dh_splits = 0;
    for (int32_t s = 0; s < o.nslab; ++s) {
        int32_t vt0, nvt;
        slab_tiles_of(o, s, &vt0, &nvt);
        o.gT_tiles = std::max(o.gT_tiles, nvt);
        o.dh_splits += slab_split_count(o.Cpad, d->H, nvt);
    }
}

fckl_status make_layout(const fckl_desc *d, int32_t chunk, Layout *L, LayoutKind kind)
{
    fckl_status st = check_desc(d);
    if (st != FCKL_OK)
        return st;
    if (chunk < 1 || !L)
        return FCKL_ERR_INVALID_ARG;
    if (!chunk_supported((int64_t)align_up((size_t)chunk, kTokenTile), d->H))
        return FCKL_ERR_UNSUPPORTED;
    Layout o;
    o.kind = kind;
    const bool keep = kind == LayoutKind::Keep, fwd_only = kind == LayoutKind::ForwardOnly;
    o.C = chunk;
    o.Cpad = (int32_t)align_up((size_t)chunk, kTokenTile);
    o.nVt = (d->V + kVocabTile - 1) / kVocabTile;
    o.Vpad = o.nVt * kVocabTile;
    o.cnt_stride = (int32_t)align_up((size_t)o.nVt + 1, 16);
    o.dh_splits = dh_split_count(o.Cpad, d->H, o.Vpad);
    o.nslab = 1;
    o.slab_tiles = o.gT_tiles = o.nVt;
    if (kind != LayoutKind::ForwardOnly)
        plan_slabs(d, o);
    const size_t Cp = (size_t)o.Cpad, K = (size_t)d->K;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    o.off_idx = take(Cp * K * 4);
    o.off_p = take(Cp * K * 4);
    o.off_zk = take(Cp * K * 4);
    o.off_psum = take(Cp * 4);
    o.off_negent = take(Cp * 4);
    o.off_cnt = take(Cp * (size_t)o.cnt_stride);
    o.off_part = take((size_t)o.nVt * Cp * 8);
    if (fwd_only) {
        o.dh_splits = 0;
        o.off_err = take(16);
        o.total = off;
        *L = o;
        return FCKL_OK;
    }
    o.off_mw = keep ? take((size_t)o.nVt * 2 * Cp * 4) : 0;
    o.off_wsum = take(16);
    o.off_ex = keep ? take(Cp * (size_t)o.Vpad * 2) : 0;
    o.off_gT = take(Cp * (size_t)o.gT_tiles * kVocabTile * 2);
    o.off_hT = take(Cp * (size_t)d->H * 2);
    o.off_WT = take((size_t)o.Vpad * (size_t)d->H * 2);
    o.off_dhp = take((size_t)o.dh_splits * Cp * (size_t)d->H * 4);
    o.off_err = take(16);
    o.total = off;
    *L = o;
    return FCKL_OK;
}

fckl_status make_topk_layout(const fckl_desc *d, int32_t chunk, TopkLayout *L)
{
    fckl_status st = check_desc(d);
    if (st != FCKL_OK)
        return st;
    if (chunk < 0 || !L)
        return FCKL_ERR_INVALID_ARG;
    if (chunk == 0)
        chunk = (int32_t)std::min<int64_t>(align_up((size_t)d->N, kTokenTile), kMaxChunk);
    if (!chunk_supported((int64_t)align_up((size_t)chunk, kTokenTile), d->H))
        return FCKL_ERR_UNSUPPORTED;
    TopkLayout o;
    o.C = chunk;
    o.Cpad = (int32_t)align_up((size_t)chunk, kTokenTile);
    o.nVt = (d->V + kVocabTile - 1) / kVocabTile;
    // maxima per token of a first pass over every tile: one per tile when there are at
    // least K tiles, else one per 32-row slice (8 per tile), else one per 16-row slice (16
    // per tile).  With fewer than K maxima even then (V <= 2048 for K <= 128) every logit
    // is a candidate, at most V <= kTopkCap of them.
    o.nSubFull = o.nVt >= d->K ? o.nVt
                 : o.nVt * (kVocabTile / 32) >= d->K ? o.nVt * (kVocabTile / 32)
                                                     : o.nVt * (kVocabTile / 16);
    if (o.nSubFull > kTopkMaxSub)
        return FCKL_ERR_UNSUPPORTED;
    // a first pass over every kTopkStride-th tile (one maximum per 64-row slice) when it
    // still gives at least 4 K maxima, unless the caller asks for the full first pass
    const int32_t part = (o.nVt + kTopkStride - 1) / kTopkStride * (kVocabTile / 64);
    o.nSubPart = (part >= 4 * d->K && !(d->flags & FCKL_FLAG_TOPK_FULL_FIRST_PASS)) ? part : 0;
    const size_t Cp = (size_t)o.Cpad;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    o.off_tmax = take((size_t)std::max(o.nSubFull, o.nSubPart) * Cp * 4);
    o.off_thr = take(Cp * 4);
    o.off_count = take(Cp * 4);
    o.off_cand = take(Cp * (size_t)kTopkCap * 8);
    o.off_err = take(16);
    o.total = off;
    *L = o;
    return FCKL_OK;
}

fckl_status make_full_layout(const fckl_desc *d, int32_t Ht, int32_t chunk, FullLayout *L)
{
    if (Ht < 8)
        return FCKL_ERR_INVALID_ARG;
    if (Ht % 8 != 0 || Ht > 65536)
        return FCKL_ERR_UNSUPPORTED;
    FullLayout o;
    fckl_status st = make_layout(d, chunk, &o.base, LayoutKind::Keep);
    if (st != FCKL_OK)
        return st;
    o.Ht = Ht;
    const size_t Cp = (size_t)o.base.Cpad;
    size_t off = o.base.total;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    o.off_at = take((size_t)o.base.Vpad * Cp * 4);
    o.off_part_t = take((size_t)o.base.nVt * Cp * 8);
    o.off_px = take((size_t)o.base.nVt * Cp * 4);
    o.off_lt2 = take(Cp * 4);
    o.off_ls2 = take(Cp * 4);
    o.total = off;
    *L = o;
    return FCKL_OK;
}

fckl_status plan_full_chunk(const fckl_desc *d, int32_t Ht, size_t budget, FullLayout *L)
{
    fckl_status st = check_desc(d);
    if (st != FCKL_OK)
        return st;
    if (d->chunk > 0)
        return make_full_layout(d, Ht, d->chunk, L);
    if (budget == 0)
        budget = kDefaultBudget;
    const int32_t npad = (int32_t)std::min<int64_t>(align_up((size_t)d->N, kTokenTile), kMaxChunk);
    int32_t best = 0;
    for (int32_t c = npad; c >= kTokenTile; c -= kTokenTile) {
        FullLayout t;
        if ((st = make_full_layout(d, Ht, c, &t)) != FCKL_OK)
            return st;
        if (t.total <= budget) {
            best = c;
            break;
        }
    }
    if (best == 0)
        return FCKL_ERR_WORKSPACE;
    // the fewest even chunks that fit (the workspace is not monotone in the chunk)
    for (int64_t nchunks = (d->N + best - 1) / best;; ++nchunks) {
        const int32_t c = (int32_t)align_up((size_t)((d->N + nchunks - 1) / nchunks), kTokenTile);
        FullLayout even;
        if (c <= best && make_full_layout(d, Ht, c, &even) == FCKL_OK && even.total <= budget) {
            *L = even;
            return FCKL_OK;
        }
        if (c <= kTokenTile)
            break;
    }
    return make_full_layout(d, Ht, best, L);
}

fckl_status plan_chunk(const fckl_desc *d, size_t budget, Layout *L, LayoutKind kind)
{
    fckl_status st = check_desc(d);
    if (st != FCKL_OK)
        return st;
    if (d->chunk > 0)
        return make_layout(d, d->chunk, L, kind);
    if (budget == 0)
        budget = kDefaultBudget;
    const int32_t npad = (int32_t)std::min<int64_t>(align_up((size_t)d->N, kTokenTile), kMaxChunk);
    // Largest chunk (a multiple of the token tile) whose workspace fits the budget.
    int32_t best = 0;
    for (int32_t c = npad; c >= kTokenTile; c -= kTokenTile) {
        Layout t;
        if (make_layout(d, c, &t, kind) == FCKL_OK && t.total <= budget) {
            best = c;
            break;
        }
    }
    if (best == 0)
        return FCKL_ERR_WORKSPACE;
    // Even the chunks out: the fewest chunks of equal size (up to the token tile) whose
    // layout fits.  (The workspace is not monotone in the chunk: the dH split count
    // depends on it.)
    for (int64_t nchunks = (d->N + best - 1) / best;; ++nchunks) {
        const int32_t c = (int32_t)align_up((size_t)((d->N + nchunks - 1) / nchunks), kTokenTile);
        Layout even;
        if (c <= best && make_layout(d, c, &even, kind) == FCKL_OK && even.total <= budget) {
            *L = even;
            return FCKL_OK;
        }
        if (c <= kTokenTile)
            break;
    }
    return make_layout(d, best, L, kind);
}

}  // namespace fckl
