// fckl_api.cpp -- the C ABI declared in include/fckl.h: argument checks, the chunk
// loop and the launch sequence.  No device memory is allocated here; every buffer,
// including the workspace, belongs to the caller.
#include <algorithm>
#include <hip/hip_runtime.h>

#include "fckl_internal.h"

using namespace fckl;

namespace {

// h, W (and the teacher's h_t, W_t) are read, and dH written, in 16-byte pieces.
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fckl_status common_checks(const fckl_desc *d, const void *h, const void *W, const int32_t *idx, const void *tl,
                          void *ws, size_t ws_bytes, Layout *L, LayoutKind kind = LayoutKind::TwoPass)
{
    fckl_status st = check_desc(d);
    if (st != FCKL_OK)
        return st;
    if (!h || !W || !idx || !tl || !ws)
        return FCKL_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || (reinterpret_cast<uintptr_t>(h) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(W) & 15u) != 0)
        return FCKL_ERR_INVALID_ARG;
    st = plan_chunk(d, ws_bytes, L, kind);
    if (st != FCKL_OK)
        return st;
    if (L->total > ws_bytes)
        return FCKL_ERR_WORKSPACE;
    return FCKL_OK;
}

ChunkArgs chunk_args(const fckl_desc *d, const void *h, const void *W, const int32_t *idx, const void *tl,
                     void *ws, const Layout *L, int64_t c0)
{
    ChunkArgs a;
    const size_t esz = d->logit_dtype == FCKL_DTYPE_F32 ? 4 : 2;
    a.h = reinterpret_cast<const uint16_t *>(h) + (size_t)c0 * d->H;
    a.W = reinterpret_cast<const uint16_t *>(W);
    a.idx = idx ? idx + (size_t)c0 * d->K : nullptr;     // NULL in the full-teacher variant
    a.tl = tl ? reinterpret_cast<const char *>(tl) + (size_t)c0 * d->K * esz : nullptr;
    a.logit_f32 = d->logit_dtype == FCKL_DTYPE_F32;
    a.rows = (int32_t)((d->N - c0) < L->C ? (d->N - c0) : L->C);
    a.H = d->H;
    a.V = d->V;
    a.K = d->K;
    a.T = d->T;
    a.ws = reinterpret_cast<char *>(ws);
    a.L = L;
    a.vt0 = 0;
    a.nvt = L->nVt;
    a.split0 = 0;
    return a;
}

// FCKL_FLAG_VALIDATE: run the teacher preparation of every chunk with the index check
// on, then read the flag back (the only host synchronisation in the library).
fckl_status validate_indices(const fckl_desc *d, const void *h, const void *W, const int32_t *idx,
                             const void *tl, void *ws, const Layout &L, void *stream)
{
    uint32_t *flag = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + L.off_err);
    if (launch_zero_flag(flag, stream))
        return FCKL_ERR_HIP;
    for (int64_t c0 = 0; c0 < d->N; c0 += L.C) {
        ChunkArgs a = chunk_args(d, h, W, idx, tl, ws, &L, c0);
        if (launch_prepare(a, true, stream))
            return FCKL_ERR_HIP;
    }
    uint32_t host = 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess)
        return FCKL_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess)
        return FCKL_ERR_HIP;
    return host ? FCKL_ERR_INDEX : FCKL_OK;
}

// Kernels with a vocabulary dimension: by default a launch covers all V rows of it.
constexpr uint32_t kVocabKernels = (1u << FCKL_KERNEL_FWD_LOGITS) | (1u << FCKL_KERNEL_COMBINE) |
                                   (1u << FCKL_KERNEL_BWD_LOGITS) | (1u << FCKL_KERNEL_DH) | (1u << FCKL_KERNEL_DW) |
                                   (1u << FCKL_KERNEL_SOFTMAX_GRAD) | (1u << FCKL_KERNEL_FULL_TEACHER) |
                                   (1u << FCKL_KERNEL_FULL_STUDENT) | (1u << FCKL_KERNEL_FULL_COMBINE) |
                                   (1u << FCKL_KERNEL_FULL_GRAD);

// Brackets one launch with the caller's events when fckl_desc.profile selects it.
// vrows: the vocabulary rows the launch covers (-1: V for a kernel with a vocabulary
// dimension, else 0).
class Timed {
  public:
    Timed(const fckl_desc *d, int kernel, int work, void *stream, int vrows = -1)
        : p_(d->profile), s_(reinterpret_cast<hipStream_t>(stream))
    {
        if (p_ && p_->events && ((p_->kernel_mask >> kernel) & 1u) && p_->count >= 0 &&
            p_->count < p_->capacity) {
            slot_ = p_->count++;
            if (p_->kernel_ids)
                p_->kernel_ids[slot_] = kernel;
            if (p_->work)
                p_->work[slot_] = work;
            if (p_->vocab_rows)
                p_->vocab_rows[slot_] = vrows >= 0 ? vrows : ((kVocabKernels >> kernel) & 1u) ? d->V : 0;
            (void)hipEventRecord(reinterpret_cast<hipEvent_t>(p_->events[2 * slot_]), s_);
        }
    }
    ~Timed()
    {
        if (slot_ >= 0)
            (void)hipEventRecord(reinterpret_cast<hipEvent_t>(p_->events[2 * slot_ + 1]), s_);
    }

  private:
    fckl_profile *p_;
    hipStream_t s_;
    int slot_ = -1;
};

// Sum of the weights and its inverse, into the workspace (weights != NULL).
fckl_status weight_sum(const fckl_desc *desc, const float *weights, void *ws, const Layout &L, void *stream,
                       float **wsum)
{
    *wsum = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.off_wsum);
    Timed t(desc, FCKL_KERNEL_WEIGHTS, (int)desc->N, stream);
    return launch_weight_sum(weights, desc->N, *wsum, stream) ? FCKL_ERR_HIP : FCKL_OK;
}

// The gradient scale of the chunk starting at token c0 (see GradScale).
GradScale chunk_scale(const fckl_desc *desc, float grad_scale, const float *weights, const float *wsum, int64_t c0)
{
    GradScale gs;
    if (weights) {
        gs.coef = (float)((double)grad_scale * (double)desc->T);
        gs.w = weights + c0;
        gs.inv_wsum = wsum + 1;
    } else {
        // d(grad_scale * mean loss)/dz = grad_scale * (T/N) * ((sum p) q - scatter p)
        gs.coef = (float)((double)grad_scale * (double)desc->T / (double)desc->N);
    }
    return gs;
}

fckl_status mean_of(const fckl_desc *desc, const float *loss_tok, const float *weights, float *loss_mean,
                    void *stream)
{
    Timed t(desc, FCKL_KERNEL_MEAN, (int)desc->N, stream);
    const int rc = weights ? launch_weighted_mean(loss_tok, weights, desc->N, loss_mean, stream)
                           : launch_mean(loss_tok, desc->N, loss_mean, stream);
    return rc ? FCKL_ERR_HIP : FCKL_OK;
}

// The forward chunk loop on a workspace whose layout L has been planned and checked.
fckl_status forward_chunks(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                           const void *topk_logit, const float *weights, float *loss_tok, float *lse,
                           float *loss_mean, void *ws, const Layout &L, void *stream)
{
    fckl_status st;
    if (desc->flags & FCKL_FLAG_VALIDATE) {
        st = validate_indices(desc, h, W, topk_idx, topk_logit, ws, L, stream);
        if (st != FCKL_OK)
            return st;
    }
    for (int64_t c0 = 0; c0 < desc->N; c0 += L.C) {
        ChunkArgs a = chunk_args(desc, h, W, topk_idx, topk_logit, ws, &L, c0);
        {
            Timed t(desc, FCKL_KERNEL_PREPARE, a.rows, stream);
            if (launch_prepare(a, false, stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(desc, FCKL_KERNEL_FWD_LOGITS, a.rows, stream);
            if (launch_forward_logits(a, stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(desc, FCKL_KERNEL_COMBINE, a.rows, stream);
            if (launch_combine(a, loss_tok + c0, lse + c0, stream))
                return FCKL_ERR_HIP;
        }
    }
    return loss_mean ? mean_of(desc, loss_tok, weights, loss_mean, stream) : FCKL_OK;
}

fckl_status forward_impl(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                         const void *topk_logit, const float *weights, float *loss_tok, float *lse,
                         float *loss_mean, void *ws, size_t ws_bytes, void *stream)
{
    Layout L;
    fckl_status st = common_checks(desc, h, W, topk_idx, topk_logit, ws, ws_bytes, &L);
    if (st != FCKL_OK)
        return st;
    if (!loss_tok || !lse)
        return FCKL_ERR_INVALID_ARG;
    return forward_chunks(desc, h, W, topk_idx, topk_logit, weights, loss_tok, lse, loss_mean, ws, L, stream);
}

// dH partial sums and dW rows of the slab of `a`, whose g^T and the chunk's h^T are in
// the workspace.
fckl_status slab_products(const fckl_desc *desc, const ChunkArgs &a, int64_t c0, float *dW, void *stream)
{
    const int vrows = std::min(a.V - a.vt0 * kVocabTile, a.nvt * kVocabTile);
    {
        Timed t(desc, FCKL_KERNEL_DH, a.rows, stream, vrows);
        if (launch_dh(a, stream))
            return FCKL_ERR_HIP;
    }
    {
        Timed t(desc, FCKL_KERNEL_DW, a.rows, stream, vrows);
        const bool accumulate = (desc->flags & FCKL_FLAG_DW_ACCUMULATE) != 0 || c0 > 0;
        if (launch_dw(a, dW, accumulate, stream))
            return FCKL_ERR_HIP;
    }
    return FCKL_OK;
}

fckl_status dh_reduce(const fckl_desc *desc, const ChunkArgs &a, int64_t c0, float *dH, void *stream)
{
    Timed t(desc, FCKL_KERNEL_DH_REDUCE, a.rows, stream);
    return launch_dh_reduce(a, dH + (size_t)c0 * desc->H, stream) ? FCKL_ERR_HIP : FCKL_OK;
}

// The chunk's gradient products, one vocabulary slab at a time: `grad` launches the kernel
// that writes the slab's g^T (`kernel`, for the profile), then come the slab's dH splits
// and dW rows; the dH splits of every slab are summed after the last.  The chunk's h^T is
// in the workspace.
template <class Grad>
fckl_status slabbed_products(const fckl_desc *desc, ChunkArgs a, int64_t c0, float *dH, float *dW, int kernel,
                             void *stream, Grad grad)
{
    const Layout &L = *a.L;
    for (int32_t s = 0; s < L.nslab; ++s) {
        slab_tiles_of(L, s, &a.vt0, &a.nvt);
        a.split0 = dh_partials(L, a.V, a.H, s);
        const int vrows = std::min(a.V - a.vt0 * kVocabTile, a.nvt * kVocabTile);
        {
            Timed t(desc, kernel, a.rows, stream, vrows);
            if (grad(a))
                return FCKL_ERR_HIP;
        }
        const fckl_status st = slab_products(desc, a, c0, dW, stream);
        if (st != FCKL_OK)
            return st;
    }
    return dh_reduce(desc, a, c0, dH, stream);
}

fckl_status backward_impl(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                          const void *topk_logit, const float *weights, const float *lse, float grad_scale,
                          const float *grad_scale_dev, float *dH, float *dW, void *ws, size_t ws_bytes,
                          void *stream)
{
    Layout L;
    fckl_status st = common_checks(desc, h, W, topk_idx, topk_logit, ws, ws_bytes, &L);
    if (st != FCKL_OK)
        return st;
    if (!lse || !dH || !dW || !aligned16(dH))
        return FCKL_ERR_INVALID_ARG;
    if (desc->flags & FCKL_FLAG_VALIDATE) {
        st = validate_indices(desc, h, W, topk_idx, topk_logit, ws, L, stream);
        if (st != FCKL_OK)
            return st;
    }
    float *wsum = nullptr;
    if (weights && (st = weight_sum(desc, weights, ws, L, stream, &wsum)) != FCKL_OK)
        return st;
    {
        // W^T once per call: the dH product reduces over the vocabulary
        ChunkArgs a = chunk_args(desc, h, W, topk_idx, topk_logit, ws, &L, 0);
        Timed t(desc, FCKL_KERNEL_TRANSPOSE, 0, stream);
        if (launch_transpose_head(a, stream))
            return FCKL_ERR_HIP;
    }
    for (int64_t c0 = 0; c0 < desc->N; c0 += L.C) {
        ChunkArgs a = chunk_args(desc, h, W, topk_idx, topk_logit, ws, &L, c0);
        GradScale gs = chunk_scale(desc, grad_scale, weights, wsum, c0);
        gs.mul = grad_scale_dev;
        {
            Timed t(desc, FCKL_KERNEL_PREPARE, a.rows, stream);
            if (launch_prepare(a, false, stream, &gs))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(desc, FCKL_KERNEL_TRANSPOSE, a.rows, stream);
            if (launch_transpose_chunk(a, stream))
                return FCKL_ERR_HIP;
        }
        // one vocabulary slab at a time: its logits recomputed into g^T, its products
        st = slabbed_products(desc, a, c0, dH, dW, FCKL_KERNEL_BWD_LOGITS, stream,
                              [&](const ChunkArgs &sa) { return launch_backward_logits(sa, lse + c0, stream); });
        if (st != FCKL_OK)
            return st;
    }
    return FCKL_OK;
}

}  // namespace

extern "C" {

fckl_status fckl_plan(const fckl_desc *desc, size_t budget_bytes, int32_t *chunk_out, size_t *ws_bytes_out)
{
    Layout L;
    fckl_status st = plan_chunk(desc, budget_bytes, &L);
    if (st != FCKL_OK)
        return st;
    if (chunk_out)
        *chunk_out = L.C;
    if (ws_bytes_out)
        *ws_bytes_out = L.total;
    return FCKL_OK;
}

fckl_status fckl_single_plan(const fckl_desc *desc, size_t budget_bytes, int32_t *chunk_out, size_t *ws_bytes_out)
{
    Layout L;
    fckl_status st = plan_chunk(desc, budget_bytes, &L, LayoutKind::Keep);
    if (st != FCKL_OK)
        return st;
    if (chunk_out)
        *chunk_out = L.C;
    if (ws_bytes_out)
        *ws_bytes_out = L.total;
    return FCKL_OK;
}

fckl_status fckl_workspace_size(const fckl_desc *desc, int32_t chunk, size_t *ws_bytes_out)
{
    Layout L;
    fckl_status st = make_layout(desc, chunk, &L);
    if (st != FCKL_OK)
        return st;
    if (ws_bytes_out)
        *ws_bytes_out = L.total;
    return FCKL_OK;
}

fckl_status fckl_forward(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                         const void *topk_logit, float *loss_tok, float *lse, float *loss_mean, void *ws,
                         size_t ws_bytes, void *stream)
{
    return forward_impl(desc, h, W, topk_idx, topk_logit, nullptr, loss_tok, lse, loss_mean, ws, ws_bytes, stream);
}

fckl_status fckl_forward_ex(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                            const void *topk_logit, const float *weights, float *loss_tok, float *lse,
                            float *loss_mean, void *ws, size_t ws_bytes, void *stream)
{
    return forward_impl(desc, h, W, topk_idx, topk_logit, weights, loss_tok, lse, loss_mean, ws, ws_bytes, stream);
}

fckl_status fckl_forward_noalloc(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                                 const void *topk_logit, const float *weights, float *loss_tok, float *lse,
                                 float *loss_mean, void *stream)
{
    fckl_status st = check_desc(desc);
    if (st != FCKL_OK)
        return st;
    if (!h || !W || !topk_idx || !topk_logit || !loss_tok || !lse || !aligned16(h) || !aligned16(W))
        return FCKL_ERR_INVALID_ARG;
    // the forward buffers of a chunk in the library's device array: the largest chunk
    // that fits (or desc->chunk, refused when it does not fit)
    Layout L;
    st = plan_chunk(desc, kScratchBytes, &L, LayoutKind::ForwardOnly);
    if (st != FCKL_OK)
        return st;
    if (L.total > kScratchBytes)
        return FCKL_ERR_WORKSPACE;
    void *ws = nullptr;
    if (scratch_address(&ws) != 0)
        return FCKL_ERR_HIP;
    return forward_chunks(desc, h, W, topk_idx, topk_logit, weights, loss_tok, lse, loss_mean, ws, L, stream);
}

fckl_status fckl_backward(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                          const void *topk_logit, const float *lse, float grad_scale, float *dH, float *dW,
                          void *ws, size_t ws_bytes, void *stream)
{
    return backward_impl(desc, h, W, topk_idx, topk_logit, nullptr, lse, grad_scale, nullptr, dH, dW, ws, ws_bytes,
                         stream);
}

fckl_status fckl_backward_ex(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                             const void *topk_logit, const float *weights, const float *lse, float grad_scale,
                             const float *grad_scale_dev, float *dH, float *dW, void *ws, size_t ws_bytes,
                             void *stream)
{
    return backward_impl(desc, h, W, topk_idx, topk_logit, weights, lse, grad_scale, grad_scale_dev, dH, dW, ws,
                         ws_bytes, stream);
}

fckl_status fckl_forward_backward(const fckl_desc *desc, const void *h, const void *W, const int32_t *topk_idx,
                                  const void *topk_logit, const float *weights, float grad_scale,
                                  float *loss_tok, float *lse, float *loss_mean, float *dH, float *dW, void *ws,
                                  size_t ws_bytes, void *stream)
{
    Layout L;
    fckl_status st = common_checks(desc, h, W, topk_idx, topk_logit, ws, ws_bytes, &L, LayoutKind::Keep);
    if (st != FCKL_OK)
        return st;
    if (!loss_tok || !lse || !dH || !dW || !aligned16(dH))
        return FCKL_ERR_INVALID_ARG;
    if (desc->flags & FCKL_FLAG_VALIDATE) {
        st = validate_indices(desc, h, W, topk_idx, topk_logit, ws, L, stream);
        if (st != FCKL_OK)
            return st;
    }
    float *wsum = nullptr;
    if (weights && (st = weight_sum(desc, weights, ws, L, stream, &wsum)) != FCKL_OK)
        return st;
    {
        ChunkArgs a = chunk_args(desc, h, W, topk_idx, topk_logit, ws, &L, 0);
        Timed t(desc, FCKL_KERNEL_TRANSPOSE, 0, stream);
        if (launch_transpose_head(a, stream))
            return FCKL_ERR_HIP;
    }
    for (int64_t c0 = 0; c0 < desc->N; c0 += L.C) {
        ChunkArgs a = chunk_args(desc, h, W, topk_idx, topk_logit, ws, &L, c0);
        const GradScale gs = chunk_scale(desc, grad_scale, weights, wsum, c0);
        {
            Timed t(desc, FCKL_KERNEL_PREPARE, a.rows, stream);
            if (launch_prepare(a, false, stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(desc, FCKL_KERNEL_FWD_LOGITS, a.rows, stream);
            if (launch_forward_logits(a, stream, true))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(desc, FCKL_KERNEL_COMBINE, a.rows, stream);
            if (launch_combine(a, loss_tok + c0, lse + c0, stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(desc, FCKL_KERNEL_TRANSPOSE, a.rows, stream);
            if (launch_transpose_chunk(a, stream))
                return FCKL_ERR_HIP;
        }
        // one vocabulary slab at a time: g^T from the kept exponentials, its products
        st = slabbed_products(desc, a, c0, dH, dW, FCKL_KERNEL_SOFTMAX_GRAD, stream,
                              [&](const ChunkArgs &sa) { return launch_softmax_grad(sa, lse + c0, gs, stream); });
        if (st != FCKL_OK)
            return st;
    }
    return loss_mean ? mean_of(desc, loss_tok, weights, loss_mean, stream) : FCKL_OK;
}

namespace {

// The loss descriptor with the fields the full-teacher variant does not read made valid.
fckl_desc full_desc(const fckl_desc *desc)
{
    fckl_desc d = *desc;
    d.K = 1;
    d.logit_dtype = FCKL_DTYPE_BF16;
    d.flags &= ~(uint32_t)FCKL_FLAG_VALIDATE;
    return d;
}

}  // namespace

fckl_status fckl_full_plan(const fckl_desc *desc, int32_t H_teacher, size_t budget_bytes, int32_t *chunk_out,
                           size_t *ws_bytes_out)
{
    if (!desc)
        return FCKL_ERR_INVALID_ARG;
    const fckl_desc d = full_desc(desc);
    FullLayout F;
    fckl_status st = plan_full_chunk(&d, H_teacher, budget_bytes, &F);
    if (st != FCKL_OK)
        return st;
    if (chunk_out)
        *chunk_out = F.base.C;
    if (ws_bytes_out)
        *ws_bytes_out = F.total;
    return FCKL_OK;
}

fckl_status fckl_full_forward_backward(const fckl_desc *desc, int32_t H_teacher, const void *h, const void *W,
                                       const void *h_t, const void *W_t, const float *weights, float grad_scale,
                                       float *loss_tok, float *lse, float *loss_mean, float *dH, float *dW,
                                       void *ws, size_t ws_bytes, void *stream)
{
    if (!desc)
        return FCKL_ERR_INVALID_ARG;
    const fckl_desc d = full_desc(desc);
    fckl_status st = check_desc(&d);
    if (st != FCKL_OK)
        return st;
    if (!h || !W || !h_t || !W_t || !ws || !loss_tok || !lse || !dH || !dW)
        return FCKL_ERR_INVALID_ARG;
    for (const void *ptr : {h, W, h_t, W_t, (const void *)dH})
        if (!aligned16(ptr))
            return FCKL_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return FCKL_ERR_INVALID_ARG;
    FullLayout F;
    if ((st = plan_full_chunk(&d, H_teacher, ws_bytes, &F)) != FCKL_OK)
        return st;
    if (F.total > ws_bytes)
        return FCKL_ERR_WORKSPACE;
    const Layout &L = F.base;
    float *wsum = nullptr;
    if (weights && (st = weight_sum(&d, weights, ws, L, stream, &wsum)) != FCKL_OK)
        return st;
    {
        ChunkArgs a = chunk_args(&d, h, W, nullptr, nullptr, ws, &L, 0);
        Timed t(&d, FCKL_KERNEL_TRANSPOSE, 0, stream);
        if (launch_transpose_head(a, stream))
            return FCKL_ERR_HIP;
    }
    for (int64_t c0 = 0; c0 < d.N; c0 += L.C) {
        ChunkArgs a = chunk_args(&d, h, W, nullptr, nullptr, ws, &L, c0);
        const GradScale gs = chunk_scale(&d, grad_scale, weights, wsum, c0);
        const uint16_t *ht_c = reinterpret_cast<const uint16_t *>(h_t) + (size_t)c0 * H_teacher;
        {
            Timed t(&d, FCKL_KERNEL_FULL_TEACHER, a.rows, stream);
            if (launch_full_teacher(a, F, ht_c, reinterpret_cast<const uint16_t *>(W_t), stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(&d, FCKL_KERNEL_FULL_COMBINE, a.rows, stream);
            if (launch_full_combine_teacher(a, F, stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(&d, FCKL_KERNEL_FULL_STUDENT, a.rows, stream);
            if (launch_full_student(a, F, stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(&d, FCKL_KERNEL_FULL_COMBINE, a.rows, stream);
            if (launch_full_combine_student(a, F, loss_tok + c0, lse + c0, stream))
                return FCKL_ERR_HIP;
        }
        {
            Timed t(&d, FCKL_KERNEL_TRANSPOSE, a.rows, stream);
            if (launch_transpose_chunk(a, stream))
                return FCKL_ERR_HIP;
        }
        // one vocabulary slab at a time: g^T from the kept values and a_t, its products
        st = slabbed_products(&d, a, c0, dH, dW, FCKL_KERNEL_FULL_GRAD, stream,
                              [&](const ChunkArgs &sa) { return launch_full_grad(sa, F, gs, stream); });
        if (st != FCKL_OK)
            return st;
    }
    return loss_mean ? mean_of(&d, loss_tok, weights, loss_mean, stream) : FCKL_OK;
}

fckl_status fckl_topk_workspace_size(const fckl_desc *desc, int32_t chunk, size_t *ws_bytes_out)
{
    TopkLayout T;
    fckl_status st = make_topk_layout(desc, chunk, &T);
    if (st != FCKL_OK)
        return st;
    if (ws_bytes_out)
        *ws_bytes_out = T.total;
    return FCKL_OK;
}

fckl_status fckl_topk_async(const fckl_desc *desc, const void *h, const void *W, int32_t *topk_idx,
                            void *topk_logit, void *ws, size_t ws_bytes, uint32_t *status, void *stream)
{
    TopkLayout T;
    fckl_status st = make_topk_layout(desc, desc ? desc->chunk : 0, &T);
    if (st != FCKL_OK)
        return st;
    if (!h || !W || !topk_idx || !topk_logit || !ws || !status)
        return FCKL_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || (reinterpret_cast<uintptr_t>(h) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(W) & 15u) != 0)
        return FCKL_ERR_INVALID_ARG;
    if (T.total > ws_bytes)
        return FCKL_ERR_WORKSPACE;
    uint32_t *flag = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + T.off_err);
    uint32_t *retry = flag + 1;
    if (launch_zero_flag(flag, stream))
        return FCKL_ERR_HIP;
    const bool f32 = desc->logit_dtype == FCKL_DTYPE_F32;
    const size_t esz = f32 ? 4 : 2;
    for (int64_t c0 = 0; c0 < desc->N; c0 += T.C) {
        ChunkArgs a;
        a.h = reinterpret_cast<const uint16_t *>(h) + (size_t)c0 * desc->H;
        a.W = reinterpret_cast<const uint16_t *>(W);
        a.rows = (int32_t)((desc->N - c0) < T.C ? (desc->N - c0) : T.C);
        a.H = desc->H;
        a.V = desc->V;
        a.K = desc->K;
        a.T = desc->T;
        a.ws = reinterpret_cast<char *>(ws);
        int32_t *idx_c = topk_idx + (size_t)c0 * desc->K;
        void *logit_c = reinterpret_cast<char *>(topk_logit) + (size_t)c0 * desc->K * esz;
        if (T.nSubPart > 0) {
            // first pass over a quarter of the vocabulary; the chunk's retry flag is raised
            // when a token then has more candidates than fit, and the guarded sequence
            // below redoes the chunk with a first pass over every tile
            if (launch_topk_max(a, T, true, nullptr, stream) ||
                launch_topk_threshold(a, T, true, nullptr, retry, stream) || launch_topk_collect(a, T, nullptr, stream) ||
                launch_topk_select(a, T, idx_c, logit_c, f32, nullptr, retry, stream))
                return FCKL_ERR_HIP;
        }
        const uint32_t *guard = T.nSubPart > 0 ? retry : nullptr;
        if (launch_topk_max(a, T, false, guard, stream) ||
            launch_topk_threshold(a, T, false, guard, nullptr, stream) || launch_topk_collect(a, T, guard, stream) ||
            launch_topk_select(a, T, idx_c, logit_c, f32, guard, nullptr, stream))
            return FCKL_ERR_HIP;
    }
    return launch_topk_status(flag, status, (uint32_t)FCKL_ERR_UNSUPPORTED, stream) ? FCKL_ERR_HIP : FCKL_OK;
}

fckl_status fckl_topk(const fckl_desc *desc, const void *h, const void *W, int32_t *topk_idx, void *topk_logit,
                      void *ws, size_t ws_bytes, void *stream)
{
    TopkLayout T;
    fckl_status st = make_topk_layout(desc, desc ? desc->chunk : 0, &T);
    if (st != FCKL_OK)
        return st;
    if (!ws || T.total > ws_bytes)
        return ws ? FCKL_ERR_WORKSPACE : FCKL_ERR_INVALID_ARG;
    // the status word goes to the workspace's error slot (word 2), read back once
    uint32_t *status = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + T.off_err) + 2;
    if ((st = fckl_topk_async(desc, h, W, topk_idx, topk_logit, ws, ws_bytes, status, stream)) != FCKL_OK)
        return st;
    uint32_t host = 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&host, status, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return FCKL_ERR_HIP;
    return (fckl_status)host;
}

fckl_status fckl_scale(float *x, int64_t n, const float *scale, void *stream)
{
    if (!x || !scale || n < 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0)
        return FCKL_ERR_INVALID_ARG;
    if (n == 0)
        return FCKL_OK;
    return launch_scale(x, n, scale, stream) ? FCKL_ERR_HIP : FCKL_OK;
}

const char *fckl_status_string(fckl_status s)
{
    switch (s) {
    case FCKL_OK:
        return "success";
    case FCKL_ERR_INVALID_ARG:
        return "invalid argument";
    case FCKL_ERR_UNSUPPORTED:
        return "unsupported shape or option";
    case FCKL_ERR_WORKSPACE:
        return "workspace too small";
    case FCKL_ERR_INDEX:
        return "cached index out of range or repeated";
    case FCKL_ERR_HIP:
        return "HIP runtime error";
    }
    return "unknown status";
}

int32_t fckl_version(void) { return 400; }

}  // extern "C"
