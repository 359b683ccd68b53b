// A C++ consumer of the C ABI alone (include/fckl.h and the HIP runtime; no Python, no
// torch): plans a workspace, allocates every buffer with hipMalloc, runs the two passes,
// the single call, the weighted passes, fckl_scale, the full-vocabulary teacher and the
// teacher top-K (both calls) on seeded inputs, and checks what holds for any input --
// finite non-negative losses, the mean, the sum rule sum_v dW[v] = 0, the identity
// <dW, W> = <dH, h>, bitwise repeatability, the single call against the two passes,
// unit weights against no weights, zero weights against zero dH rows, a teacher equal to
// the student against zero loss, top-K ordering and values -- plus the argument errors.
// Exit status 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fckl.h"

static int failures = 0;
#define CHECK(cond)                                                                                           \
    do {                                                                                                      \
        if (!(cond)) {                                                                                        \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);                           \
            ++failures;                                                                                       \
        }                                                                                                     \
    } while (0)
#define HIP_OK(call)                                                                                          \
    do {                                                                                                      \
        hipError_t e_ = (call);                                                                               \
        if (e_ != hipSuccess) {                                                                               \
            std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                           \
            return 2;                                                                                         \
        }                                                                                                     \
    } while (0)

static uint64_t rng_state = 0x2545F4914F6CDD1Dull;
static double uniform01()
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}
static double normal01()
{
    const double u = uniform01() + 1e-300, v = uniform01();
    return std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v);
}
// float -> bf16, round to nearest even (finite inputs)
static uint16_t to_bf16(float x)
{
    uint32_t u;
    std::memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

template <class T> static T *dev_alloc(size_t n)
{
    void *p = nullptr;
    if (hipMalloc(&p, n * sizeof(T) + 256) != hipSuccess)
        return nullptr;
    return static_cast<T *>(p);
}

int main()
{
    const int64_t N = 700;
    const int32_t H = 256, V = 4100, K = 10;
    const float T = 1.3f;
    std::vector<uint16_t> h(N * H), W((size_t)V * H), tl(N * K);
    std::vector<int32_t> idx(N * K);
    for (auto &x : h)
        x = to_bf16((float)normal01());
    for (auto &x : W)
        x = to_bf16((float)(0.125 * normal01()));
    for (int64_t i = 0; i < N; ++i) {
        for (int k = 0; k < K; ++k) {
            int32_t v;
            bool again;
            do {   // K distinct indices per token
                v = (int32_t)(uniform01() * V) % V;
                again = false;
                for (int j = 0; j < k; ++j)
                    again |= idx[i * K + j] == v;
            } while (again);
            idx[i * K + k] = v;
            tl[i * K + k] = to_bf16((float)(2.0 * normal01()));
        }
    }

    fckl_desc d;
    std::memset(&d, 0, sizeof(d));
    d.N = N;
    d.H = H;
    d.V = V;
    d.K = K;
    d.T = T;
    d.logit_dtype = FCKL_DTYPE_BF16;
    int32_t chunk = 0, chunk1 = 0;
    size_t ws_bytes = 0, ws1_bytes = 0;
    CHECK(fckl_plan(&d, 0, &chunk, &ws_bytes) == FCKL_OK && chunk > 0 && ws_bytes > 0);
    // the single call keeps the chunk's exponentials as well: a larger workspace
    CHECK(fckl_single_plan(&d, 0, &chunk1, &ws1_bytes) == FCKL_OK && chunk1 == chunk && ws1_bytes > ws_bytes);
    ws_bytes = ws1_bytes;

    uint16_t *dh = dev_alloc<uint16_t>(h.size()), *dW_in = dev_alloc<uint16_t>(W.size());
    uint16_t *dtl = dev_alloc<uint16_t>(tl.size());
    int32_t *didx = dev_alloc<int32_t>(idx.size());
    float *loss = dev_alloc<float>(N), *lse = dev_alloc<float>(N), *mean = dev_alloc<float>(1);
    float *dH = dev_alloc<float>((size_t)N * H), *dW = dev_alloc<float>((size_t)V * H);
    void *ws = dev_alloc<char>(ws_bytes);
    if (!dh || !dW_in || !dtl || !didx || !loss || !lse || !mean || !dH || !dW || !ws)
        return 2;
    HIP_OK(hipMemcpy(dh, h.data(), h.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dW_in, W.data(), W.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dtl, tl.data(), tl.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(didx, idx.data(), idx.size() * 4, hipMemcpyHostToDevice));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    auto run_two_pass = [&]() {
        CHECK(fckl_forward(&d, dh, dW_in, didx, dtl, loss, lse, mean, ws, ws_bytes, s) == FCKL_OK);
        CHECK(fckl_backward(&d, dh, dW_in, didx, dtl, lse, 1.0f, dH, dW, ws, ws_bytes, s) == FCKL_OK);
    };
    auto fetch = [&](std::vector<float> &l, std::vector<float> &m, std::vector<float> &gh, std::vector<float> &gw) {
        l.resize(N);
        m.resize(1);
        gh.resize((size_t)N * H);
        gw.resize((size_t)V * H);
        if (hipStreamSynchronize(s) != hipSuccess || hipMemcpy(l.data(), loss, N * 4, hipMemcpyDeviceToHost) ||
            hipMemcpy(m.data(), mean, 4, hipMemcpyDeviceToHost) ||
            hipMemcpy(gh.data(), dH, gh.size() * 4, hipMemcpyDeviceToHost) ||
            hipMemcpy(gw.data(), dW, gw.size() * 4, hipMemcpyDeviceToHost))
            ++failures;
    };
    std::vector<float> l1, m1, gh1, gw1, l2, m2, gh2, gw2;
    run_two_pass();
    fetch(l1, m1, gh1, gw1);
    run_two_pass();
    fetch(l2, m2, gh2, gw2);
    CHECK(l1 == l2 && m1 == m2 && gh1 == gh2 && gw1 == gw2);   // bitwise repeatable

    // the backward in vocabulary slabs of 512 rows (8 slabs, the last with the 4-row
    // tile): the same loss and dW bit for bit, dH up to the order of its split sum
    {
        fckl_desc ds = d;
        ds.vocab_slab = 512;
        size_t slab_ws = 0;
        CHECK(fckl_workspace_size(&ds, chunk, &slab_ws) == FCKL_OK && slab_ws < ws_bytes);
        ds.chunk = chunk;
        CHECK(fckl_forward(&ds, dh, dW_in, didx, dtl, loss, lse, mean, ws, slab_ws, s) == FCKL_OK);
        CHECK(fckl_backward(&ds, dh, dW_in, didx, dtl, lse, 1.0f, dH, dW, ws, slab_ws, s) == FCKL_OK);
        fetch(l2, m2, gh2, gw2);
        CHECK(l1 == l2 && m1 == m2 && gw1 == gw2);
        double e = 0.0, m = 0.0;
        for (size_t q = 0; q < gh1.size(); ++q) {
            e = std::fmax(e, std::fabs(gh1[q] - gh2[q]));
            m = std::fmax(m, std::fabs(gh1[q]));
        }
        CHECK(e <= 1e-5 * m);
        ds.vocab_slab = 100;     // not a multiple of 256
        CHECK(fckl_backward(&ds, dh, dW_in, didx, dtl, lse, 1.0f, dH, dW, ws, ws_bytes, s) == FCKL_ERR_INVALID_ARG);
    }

    double lmax = 0.0, lsum = 0.0;
    for (float x : l1) {
        CHECK(std::isfinite(x));
        lmax = std::fmax(lmax, std::fabs(x));
        lsum += x;
    }
    for (float x : l1)
        CHECK(x >= -1e-5 * lmax);
    CHECK(std::fabs(m1[0] - lsum / N) <= 1e-5 * std::fabs(m1[0]));
    for (int j = 0; j < H; ++j) {
        double sr = 0.0, ar = 0.0;
        for (int v = 0; v < V; ++v) {
            sr += gw1[(size_t)v * H + j];
            ar += std::fabs(gw1[(size_t)v * H + j]);
        }
        CHECK(std::fabs(sr) <= 1e-3 * ar);
    }
    double ipw = 0.0, iph = 0.0;
    for (size_t q = 0; q < W.size(); ++q)
        ipw += gw1[q] * from_bf16(W[q]);
    for (size_t q = 0; q < h.size(); ++q)
        iph += gh1[q] * from_bf16(h[q]);
    CHECK(std::fabs(ipw - iph) <= 2e-2 * std::fmax(std::fabs(ipw), std::fabs(iph)));

    // the single call: the same loss bit for bit, gradients within g's bf16 rounding
    CHECK(fckl_forward_backward(&d, dh, dW_in, didx, dtl, nullptr, 1.0f, loss, lse, mean, dH, dW, ws, ws_bytes, s) ==
          FCKL_OK);
    fetch(l2, m2, gh2, gw2);
    CHECK(l1 == l2 && m1 == m2);
    double eh = 0.0, mh = 0.0, ew = 0.0, mw = 0.0;
    for (size_t q = 0; q < gh1.size(); ++q) {
        eh = std::fmax(eh, std::fabs(gh1[q] - gh2[q]));
        mh = std::fmax(mh, std::fabs(gh1[q]));
    }
    for (size_t q = 0; q < gw1.size(); ++q) {
        ew = std::fmax(ew, std::fabs(gw1[q] - gw2[q]));
        mw = std::fmax(mw, std::fabs(gw1[q]));
    }
    CHECK(eh <= 2e-2 * mh && ew <= 2e-2 * mw);

    // teacher top-K on the same hidden states and head
    size_t tws_bytes = 0;
    CHECK(fckl_topk_workspace_size(&d, 0, &tws_bytes) == FCKL_OK);
    void *tws = dev_alloc<char>(tws_bytes);
    int32_t *ti = dev_alloc<int32_t>((size_t)N * K);
    uint16_t *tv = dev_alloc<uint16_t>((size_t)N * K);
    if (!tws || !ti || !tv)
        return 2;
    CHECK(fckl_topk(&d, dh, dW_in, ti, tv, tws, tws_bytes, s) == FCKL_OK);
    std::vector<int32_t> hi((size_t)N * K);
    std::vector<uint16_t> hv((size_t)N * K);
    HIP_OK(hipMemcpy(hi.data(), ti, hi.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hv.data(), tv, hv.size() * 2, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < N; i += 7) {
        double prev = INFINITY;
        for (int k = 0; k < K; ++k) {
            const int32_t v = hi[i * K + k];
            CHECK(v >= 0 && v < V);
            double z = 0.0;
            for (int j = 0; j < H; ++j)
                z += from_bf16(h[i * H + j]) * from_bf16(W[(size_t)v * H + j]);
            const double zb = from_bf16(hv[i * K + k]);
            CHECK(std::fabs(zb - z) <= 1e-2 * std::fmax(1.0, std::fabs(z)));   // bf16 output
            CHECK(zb <= prev);
            prev = zb;
        }
    }

    // the weighted passes: weights of 1 give the plain passes' results (up to the order of
    // the fp64 sums); a weight of 0 leaves that token's dH row at exactly 0
    std::vector<float> w1(N, 1.0f), w01(N, 1.0f);
    for (int64_t i = 0; i < N; i += 5)
        w01[i] = 0.0f;
    float *dw1 = dev_alloc<float>(N), *dw01 = dev_alloc<float>(N), *two = dev_alloc<float>(1);
    uint32_t *status = dev_alloc<uint32_t>(1);
    if (!dw1 || !dw01 || !two || !status)
        return 2;
    const float two_h = 2.0f;
    HIP_OK(hipMemcpy(dw1, w1.data(), N * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw01, w01.data(), N * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(two, &two_h, 4, hipMemcpyHostToDevice));
    CHECK(fckl_forward_ex(&d, dh, dW_in, didx, dtl, dw1, loss, lse, mean, ws, ws_bytes, s) == FCKL_OK);
    CHECK(fckl_backward_ex(&d, dh, dW_in, didx, dtl, dw1, lse, 1.0f, nullptr, dH, dW, ws, ws_bytes, s) == FCKL_OK);
    fetch(l2, m2, gh2, gw2);
    CHECK(l1 == l2 && std::fabs(m2[0] - m1[0]) <= 1e-6 * std::fabs(m1[0]));
    double e1 = 0.0;
    for (size_t q = 0; q < gw1.size(); ++q)
        e1 = std::fmax(e1, std::fabs(gw1[q] - gw2[q]));
    CHECK(e1 <= 1e-2 * mw);     // w / sum w against 1 / N can move a bf16 rounding of g
    CHECK(fckl_forward_ex(&d, dh, dW_in, didx, dtl, dw01, loss, lse, mean, ws, ws_bytes, s) == FCKL_OK);
    CHECK(fckl_backward_ex(&d, dh, dW_in, didx, dtl, dw01, lse, 1.0f, nullptr, dH, dW, ws, ws_bytes, s) == FCKL_OK);
    fetch(l2, m2, gh2, gw2);
    double wl = 0.0, ws_ = 0.0;
    for (int64_t i = 0; i < N; ++i) {
        wl += (double)w01[i] * l1[i];
        ws_ += w01[i];
    }
    CHECK(std::fabs(m2[0] - wl / ws_) <= 1e-5 * std::fabs(m2[0]));
    for (int64_t i = 0; i < N; i += 5)
        for (int j = 0; j < H; ++j)
            CHECK(gh2[i * H + j] == 0.0f);

    // fckl_scale: dH of the plain pass doubled in place on the device, exactly
    run_two_pass();
    CHECK(fckl_scale(dH, (int64_t)N * H, two, s) == FCKL_OK);
    fetch(l2, m2, gh2, gw2);
    for (size_t q = 0; q < gh1.size(); ++q)
        CHECK(gh2[q] == 2.0f * gh1[q]);

    // the online teacher over the whole vocabulary: teacher = student gives zero loss;
    // another teacher (a rescaled head) gives finite losses >= 0, the sum rule and the
    // <dW, W> = <dH, h> identity
    {
        std::vector<uint16_t> Wt(W.size());
        for (size_t q = 0; q < W.size(); ++q)
            Wt[q] = to_bf16((float)(1.5 * from_bf16(W[q])));
        uint16_t *dWt = dev_alloc<uint16_t>(Wt.size());
        int32_t fchunk = 0;
        size_t fws_bytes = 0;
        CHECK(fckl_full_plan(&d, H, 0, &fchunk, &fws_bytes) == FCKL_OK && fchunk > 0);
        void *fws = dev_alloc<char>(fws_bytes);
        if (!dWt || !fws)
            return 2;
        HIP_OK(hipMemcpy(dWt, Wt.data(), Wt.size() * 2, hipMemcpyHostToDevice));
        CHECK(fckl_full_forward_backward(&d, H, dh, dW_in, dh, dW_in, nullptr, 1.0f, loss, lse, mean, dH, dW, fws,
                                         fws_bytes, s) == FCKL_OK);
        fetch(l2, m2, gh2, gw2);
        for (float x : l2)
            CHECK(std::fabs(x) <= 1e-4);
        CHECK(fckl_full_forward_backward(&d, H, dh, dW_in, dh, dWt, nullptr, 1.0f, loss, lse, mean, dH, dW, fws,
                                         fws_bytes, s) == FCKL_OK);
        fetch(l2, m2, gh2, gw2);
        double fmax = 0.0;
        for (float x : l2) {
            CHECK(std::isfinite(x));
            fmax = std::fmax(fmax, std::fabs(x));
        }
        CHECK(fmax > 1e-3);
        for (float x : l2)
            CHECK(x >= -1e-5 * fmax);
        for (int j = 0; j < H; ++j) {
            double sr = 0.0, ar = 0.0;
            for (int v = 0; v < V; ++v) {
                sr += gw2[(size_t)v * H + j];
                ar += std::fabs(gw2[(size_t)v * H + j]);
            }
            CHECK(std::fabs(sr) <= 1e-3 * ar);
        }
        double fpw = 0.0, fph = 0.0;
        for (size_t q = 0; q < W.size(); ++q)
            fpw += gw2[q] * from_bf16(W[q]);
        for (size_t q = 0; q < h.size(); ++q)
            fph += gh2[q] * from_bf16(h[q]);
        CHECK(std::fabs(fpw - fph) <= 2e-2 * std::fmax(std::fabs(fpw), std::fabs(fph)));
        HIP_OK(hipFree(dWt));
        HIP_OK(hipFree(fws));
    }

    // fckl_topk_async: the same cache as fckl_topk, bit for bit, and status FCKL_OK on the device
    {
        const uint32_t junk = 0xFFFFFFFFu;
        HIP_OK(hipMemcpy(status, &junk, 4, hipMemcpyHostToDevice));
        int32_t *ti2 = dev_alloc<int32_t>((size_t)N * K);
        uint16_t *tv2 = dev_alloc<uint16_t>((size_t)N * K);
        if (!ti2 || !tv2)
            return 2;
        CHECK(fckl_topk_async(&d, dh, dW_in, ti2, tv2, tws, tws_bytes, status, s) == FCKL_OK);
        HIP_OK(hipStreamSynchronize(s));
        uint32_t st = 0;
        std::vector<int32_t> hi2((size_t)N * K);
        std::vector<uint16_t> hv2((size_t)N * K);
        HIP_OK(hipMemcpy(&st, status, 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(hi2.data(), ti2, hi2.size() * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(hv2.data(), tv2, hv2.size() * 2, hipMemcpyDeviceToHost));
        CHECK(st == (uint32_t)FCKL_OK && hi2 == hi && hv2 == hv);
        HIP_OK(hipFree(ti2));
        HIP_OK(hipFree(tv2));
    }

    // argument errors come back as status codes, before any work
    CHECK(fckl_forward(&d, nullptr, dW_in, didx, dtl, loss, lse, mean, ws, ws_bytes, s) == FCKL_ERR_INVALID_ARG);
    CHECK(fckl_forward(&d, dh, dW_in, didx, dtl, loss, lse, mean, ws, 1024, s) == FCKL_ERR_WORKSPACE);
    fckl_desc bad = d;
    bad.T = -1.0f;
    CHECK(fckl_backward(&bad, dh, dW_in, didx, dtl, lse, 1.0f, dH, dW, ws, ws_bytes, s) == FCKL_ERR_INVALID_ARG);
    CHECK(fckl_status_string(FCKL_ERR_WORKSPACE) != nullptr && fckl_version() >= 100);

    HIP_OK(hipStreamDestroy(s));
    for (void *p : {(void *)dh, (void *)dW_in, (void *)dtl, (void *)didx, (void *)loss, (void *)lse, (void *)mean,
                    (void *)dH, (void *)dW, ws, tws, (void *)ti, (void *)tv, (void *)dw1, (void *)dw01, (void *)two,
                    (void *)status})
        HIP_OK(hipFree(p));
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("c abi driver ok: chunk %d, workspace %zu bytes, mean loss %.6f\n", chunk, ws_bytes, m1[0]);
    return 0;
}
