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

fckl_status check_desc(const fckl_desc *d)
{
    if (!d)
        return FCKL_ERR_INVALID_ARG;
    if (d->N < 1 || d->N > INT32_MAX || d->H < 8 || d->V < 1 || d->K < 1)
        return FCKL_ERR_INVALID_ARG;
    if (!(d->T > 0.0f) || !std::isfinite(d->T))
        return FCKL_ERR_INVALID_ARG;
    if (d->K > d->V || d->chunk < 0)
        return FCKL_ERR_INVALID_ARG;
    if (d->logit_dtype != FCKL_DTYPE_BF16 && d->logit_dtype != FCKL_DTYPE_F32)
        return FCKL_ERR_INVALID_ARG;
    if (d->flags & ~(uint32_t)(FCKL_FLAG_VALIDATE | FCKL_FLAG_DW_ACCUMULATE))
        return FCKL_ERR_INVALID_ARG;
    if (d->H % 8 != 0)
        return FCKL_ERR_UNSUPPORTED;
    if (d->K > kMaxK || d->H > 65536 || d->V > (1 << 30))
        return FCKL_ERR_UNSUPPORTED;
    return FCKL_OK;
}

// Number of vocabulary splits of the dH product: enough work-groups to cover the
// 256 compute units several times over, but at least 4 k-steps of 64 per split.
static int32_t dh_split_count(int32_t Cpad, int32_t H, int32_t bn, int32_t Vpad)
{
    int64_t tiles = (int64_t)(Cpad / kTokenTile) * ((H + bn - 1) / bn);
    int64_t s = (1024 + tiles - 1) / tiles;
    int64_t smax = Vpad / 256;
    if (s > smax)
        s = smax;
    if (s > 64)
        s = 64;
    return (int32_t)(s < 1 ? 1 : s);
}

fckl_status make_layout(const fckl_desc *d, int32_t chunk, Layout *L)
{
    fckl_status st = check_desc(d);
    if (st != FCKL_OK)
        return st;
    if (chunk < 1 || !L)
        return FCKL_ERR_INVALID_ARG;
    Layout o;
    o.C = chunk;
    o.Cpad = (int32_t)align_up((size_t)chunk, kTokenTile);
    o.nVt = (d->V + kVocabTile - 1) / kVocabTile;
    o.Vpad = o.nVt * kVocabTile;
    o.cnt_stride = (int32_t)align_up((size_t)o.nVt + 1, 16);
    o.dh_bn = (d->H % 256 == 0) ? 256 : (d->H % 192 == 0 ? 192 : 256);
    o.dh_splits = dh_split_count(o.Cpad, d->H, o.dh_bn, o.Vpad);
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
    o.off_g = take(Cp * (size_t)o.Vpad * 2);
    o.off_dhp = take((size_t)o.dh_splits * Cp * (size_t)d->H * 4);
    o.off_err = take(16);
    o.total = off;
    *L = o;
    return FCKL_OK;
}

fckl_status plan_chunk(const fckl_desc *d, size_t budget, Layout *L)
{
    fckl_status st = check_desc(d);
    if (st != FCKL_OK)
        return st;
    if (d->chunk > 0)
        return make_layout(d, d->chunk, L);
    if (budget == 0)
        budget = kDefaultBudget;
    const int32_t npad = (int32_t)std::min<int64_t>(align_up((size_t)d->N, kTokenTile), kMaxChunk);
    // Largest chunk (a multiple of the token tile) whose workspace fits the budget.
    int32_t best = 0;
    for (int32_t c = npad; c >= kTokenTile; c -= kTokenTile) {
        Layout t;
        if (make_layout(d, c, &t) == FCKL_OK && t.total <= budget) {
            best = c;
            break;
        }
    }
    if (best == 0)
        return FCKL_ERR_WORKSPACE;
    // Even the chunks out: same number of chunks, as few padded tokens as possible.
    int64_t nchunks = (d->N + best - 1) / best;
    int32_t c = (int32_t)align_up((size_t)((d->N + nchunks - 1) / nchunks), kTokenTile);
    if (c > best)
        c = best;
    return make_layout(d, c, L);
}

}  // namespace fckl
