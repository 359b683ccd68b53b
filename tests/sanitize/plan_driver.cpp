// Sanitizer driver for the host-side planner (fckl_plan.cpp; no HIP): sweeps valid and
// invalid descriptors, chunk sizes and budgets through every layout and scheduler
// function and checks the layout invariants -- regions 256-byte aligned, in order, not
// overlapping, inside the total; a planned workspace within its budget -- so that
// AddressSanitizer and UndefinedBehaviorSanitizer see overflow and out-of-range paths.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "fckl_internal.h"

using namespace fckl;

static int failures = 0;
#define CHECK(cond)                                                                                           \
    do {                                                                                                      \
        if (!(cond)) {                                                                                        \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);                           \
            ++failures;                                                                                       \
        }                                                                                                     \
    } while (0)

static void check_regions(const std::vector<std::pair<size_t, size_t>> &regions, size_t total)
{
    size_t end = 0;
    for (const auto &r : regions) {
        CHECK(r.first % 256 == 0);
        CHECK(r.first >= end);
        end = r.first + r.second;
    }
    CHECK(end <= total);
}

static void check_layout(const fckl_desc &d, const Layout &L)
{
    const size_t Cp = (size_t)L.Cpad, K = (size_t)d.K;
    CHECK(L.Cpad % kTokenTile == 0 && L.Cpad >= L.C && L.Vpad % kVocabTile == 0 && L.Vpad >= d.V);
    CHECK(L.kind == LayoutKind::ForwardOnly ? L.dh_splits == 0 : L.dh_splits >= 1);
    std::vector<std::pair<size_t, size_t>> regions = {
        {L.off_idx, Cp * K * 4}, {L.off_p, Cp * K * 4}, {L.off_zk, Cp * K * 4}, {L.off_psum, Cp * 4},
        {L.off_negent, Cp * 4}, {L.off_cnt, Cp * (size_t)L.cnt_stride}, {L.off_part, (size_t)L.nVt * Cp * 8}};
    // the kept exponentials and their maxima exist only in a keep layout
    if (L.kind == LayoutKind::ForwardOnly) {
        regions.push_back({L.off_err, 16});
        check_regions(regions, L.total);
        return;
    }
    const bool keep = L.kind == LayoutKind::Keep;
    if (keep)
        regions.push_back({L.off_mw, 2 * (size_t)L.nVt * Cp * 4});
    regions.push_back({L.off_wsum, 8});
    if (keep)
        regions.push_back({L.off_ex, Cp * (size_t)L.Vpad * 2});
    // vocabulary slabs: contiguous, covering every tile, g^T sized for the largest, dH
    // partial sums for every split that holds a row (a keep layout has one slab)
    CHECK(L.nslab >= 1 && L.slab_tiles >= 1 && L.gT_tiles >= 1 && L.gT_tiles <= L.nVt);
    int32_t next = 0, biggest = 0;
    for (int32_t s = 0; s < L.nslab; ++s) {
        int32_t vt0 = -1, nvt = -1;
        slab_tiles_of(L, s, &vt0, &nvt);
        CHECK(vt0 == next && nvt >= 1);
        CHECK(s + 1 == L.nslab ? nvt < 2 * L.slab_tiles || L.nslab == 1 : nvt == L.slab_tiles);
        int32_t ksplit = 0, used = 0;
        slab_split_rows(L, d.V, d.H, s, &ksplit, &used);
        CHECK(ksplit % kDhStep == 0 && ksplit >= kDhStep && used >= 1);
        CHECK((int64_t)used * ksplit >= (int64_t)std::min(d.V - vt0 * kVocabTile, nvt * kVocabTile));
        CHECK((int64_t)(used - 1) * ksplit < (int64_t)std::min(d.V - vt0 * kVocabTile, nvt * kVocabTile));
        next = vt0 + nvt;
        biggest = std::max(biggest, nvt);
    }
    CHECK(next == L.nVt && biggest == L.gT_tiles);
    CHECK(dh_partials(L, d.V, d.H, L.nslab) <= L.dh_splits);
    for (const auto &r : std::vector<std::pair<size_t, size_t>>{
             {L.off_gT, (size_t)L.gT_tiles * kVocabTile * Cp * 2}, {L.off_hT, (size_t)d.H * Cp * 2},
             {L.off_WT, (size_t)d.H * (size_t)L.Vpad * 2},
             {L.off_dhp, (size_t)L.dh_splits * Cp * (size_t)d.H * 4}, {L.off_err, 16}})
        regions.push_back(r);
    check_regions(regions, L.total);
}

int main()
{
    const int64_t Ns[] = {1, 255, 256, 257, 32768, 262144, 2147483647LL};
    const int32_t Hs[] = {8, 136, 2880, 3072, 65536};
    const int32_t Vs[] = {1, 100, 257, 4100, 128256, 201088, 1 << 21, 1 << 24, (1 << 24) + 1};
    const int32_t Ks[] = {1, 10, 100, 128};
    const size_t budgets[] = {0, size_t(1) << 20, size_t(3) << 30, size_t(12) << 30, size_t(64) << 30};
    int planned = 0, rejected = 0;
    for (int64_t N : Ns)
        for (int32_t H : Hs)
            for (int32_t V : Vs)
                for (int32_t K : Ks) {
                    fckl_desc d{};
                    d.N = N;
                    d.H = H;
                    d.V = V;
                    d.K = K;
                    d.T = 1.0f;
                    d.logit_dtype = FCKL_DTYPE_BF16;
                    const int64_t vocab_tiles = ((int64_t)V + 255) / 256 * (((int64_t)H + 255) / 256);
                    if (check_desc(&d) != FCKL_OK) {
                        CHECK(K > V || V > kMaxPitch || vocab_tiles > kMaxTiles);
                        ++rejected;
                        continue;
                    }
                    CHECK(V <= kMaxPitch && vocab_tiles <= kMaxTiles);
                    for (size_t budget : budgets) {
                        for (LayoutKind kind : {LayoutKind::TwoPass, LayoutKind::Keep, LayoutKind::ForwardOnly}) {
                            Layout L;
                            if (plan_chunk(&d, budget, &L, kind) == FCKL_OK) {
                                ++planned;
                                CHECK(L.kind == kind);
                                CHECK(L.total <= (budget ? budget : (size_t(12) << 30)));
                                CHECK(L.C >= 1 && L.C <= kMaxChunk);
                                check_layout(d, L);
                            }
                        }
                        FullLayout F;
                        if (plan_full_chunk(&d, H, budget, &F) == FCKL_OK) {
                            CHECK(F.total <= (budget ? budget : (size_t(12) << 30)));
                            CHECK(F.base.kind == LayoutKind::Keep);
                            check_layout(d, F.base);
                            const size_t Cp = (size_t)F.base.Cpad;
                            check_regions({{F.off_at, (size_t)F.base.Vpad * Cp * 4},
                                           {F.off_part_t, (size_t)F.base.nVt * Cp * 8},
                                           {F.off_px, (size_t)F.base.nVt * Cp * 4}, {F.off_lt2, Cp * 4},
                                           {F.off_ls2, Cp * 4}},
                                          F.total);
                            CHECK(F.off_at >= F.base.total);
                        }
                    }
                    for (int32_t slab : {256, 512, 65536, 100, -256}) {
                        fckl_desc ds = d;
                        ds.vocab_slab = slab;
                        if (slab % 256 != 0 || slab < 0) {
                            CHECK(check_desc(&ds) == FCKL_ERR_INVALID_ARG);
                            continue;
                        }
                        for (int32_t chunk : {256, 8192})
                            for (LayoutKind kind : {LayoutKind::TwoPass, LayoutKind::Keep}) {
                                Layout L;
                                if (make_layout(&ds, chunk, &L, kind) == FCKL_OK) {
                                    check_layout(ds, L);
                                    CHECK(L.nslab == std::max<int32_t>(1, L.nVt / (slab / 256)));
                                    CHECK(L.slab_tiles == (L.nslab > 1 ? slab / 256 : L.nVt));
                                }
                            }
                    }
                    for (int32_t chunk : {1, 256, 1000, 8192, 1 << 20, (1 << 24) + 1}) {
                        Layout L;
                        const int64_t Cpad = ((int64_t)chunk + 255) / 256 * 256;
                        const bool fits = Cpad <= kMaxPitch && Cpad / 256 * (((int64_t)H + 255) / 256) <= kMaxTiles &&
                                          Cpad * H <= kMaxChunkElems;
                        for (LayoutKind kind : {LayoutKind::TwoPass, LayoutKind::Keep, LayoutKind::ForwardOnly}) {
                            const fckl_status ls = make_layout(&d, chunk, &L, kind);
                            CHECK(fits ? ls == FCKL_OK : ls == FCKL_ERR_UNSUPPORTED);
                            if (ls == FCKL_OK)
                                check_layout(d, L);
                        }
                        for (uint32_t flags : {0u, (uint32_t)FCKL_FLAG_TOPK_FULL_FIRST_PASS}) {
                            fckl_desc dt = d;
                            dt.flags = flags;
                            TopkLayout T;
                            if (make_topk_layout(&dt, chunk, &T) == FCKL_OK) {
                                const size_t Cp = (size_t)T.Cpad;
                                CHECK(T.nSubFull >= 1 && T.nSubPart >= 0);
                                CHECK(T.nSubPart == 0 || T.nSubPart >= 4 * d.K);
                                CHECK(!flags || T.nSubPart == 0);
                                const size_t nsub = (size_t)(T.nSubFull > T.nSubPart ? T.nSubFull : T.nSubPart);
                                check_regions({{T.off_tmax, nsub * Cp * 4}, {T.off_thr, Cp * 4}, {T.off_count, Cp * 4},
                                               {T.off_cand, Cp * (size_t)kTopkCap * 8}, {T.off_err, 16}},
                                              T.total);
                            }
                        }
                    }
                }
    // invalid descriptors are rejected, never planned
    fckl_desc bad{};
    bad.N = 0;
    bad.H = 64;
    bad.V = 100;
    bad.K = 4;
    bad.T = 1.0f;
    Layout L;
    CHECK(plan_chunk(&bad, 0, &L) != FCKL_OK);
    bad.N = 10;
    bad.T = -1.0f;
    CHECK(check_desc(&bad) != FCKL_OK);
    bad.T = 1.0f;
    bad.H = 12;
    CHECK(check_desc(&bad) == FCKL_ERR_UNSUPPORTED);
    bad.H = 64;
    bad.flags = 64u;
    CHECK(check_desc(&bad) == FCKL_ERR_INVALID_ARG);
    CHECK(check_desc(nullptr) == FCKL_ERR_INVALID_ARG);
    FullLayout F;
    bad.flags = 0;
    CHECK(make_full_layout(&bad, 7, 256, &F) == FCKL_ERR_INVALID_ARG);
    CHECK(make_full_layout(&bad, 12, 256, &F) == FCKL_ERR_UNSUPPORTED);
    CHECK(make_layout(&bad, 0, &L) == FCKL_ERR_INVALID_ARG);
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("plan driver ok: %d plans, %d rejected descriptors\n", planned, rejected);
    return 0;
}
