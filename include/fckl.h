/*
 * fckl.h -- C ABI of the fused chunked top-K KL distillation loss (gfx950 / MI355X).
 *
 * The operation.  A student's final hidden states h[N,H] are projected through its
 * LM head W[V,H] (no bias) and each token's KL divergence is taken against a teacher
 * cache that holds, per token, K logits and their vocabulary indices.  The
 * projection is part of the loss and the tokens are processed one chunk at a time,
 * so the N x V logit grid is never stored, forward or backward.  Sources (the web
 * pages the method is described on):
 *   - "What actually changed?", calcaas.com: the fused chunked loss folds the output
 *     projection into the loss and processes one slice of the sequence at a time, so
 *     the vocabulary-by-sequence grid is never built;
 *   - "Breaking the Bottleneck with Offline Caching and Chunked Loss", axbrief.com:
 *     the teacher's top-100 logits are cached once; the loss takes one chunk,
 *     computes its part and discards it; the backward pass re-projects each chunk;
 *   - "Preparing Offline Top-K Logits", getaibook.com: the cache stores the top-K
 *     logits together with their indices, K configurable (10 and 100 are named);
 *   - "Two Architectural Innovations", keepingupwith.ai: gradients are processed in
 *     small tiles rather than over the full vocabulary x sequence tensor.
 *
 * Definition (IEEE real arithmetic; the GPU computes it with bf16 inputs and fp32
 * accumulation):
 *   p[i,k]  = softmax_k(topk_logit[i,:] / T)           (renormalised over the K entries)
 *   z[i,v]  = sum_j h[i,j] * W[v,j]
 *   lse[i]  = log sum_v exp(z[i,v] / T)
 *   loss[i] = T^2 * sum_k p[i,k] * (log p[i,k] - (z[i, idx[i,k]] / T - lse[i]))
 *   loss_mean = (1/N) * sum_i loss[i]
 *   g[i,v]  = grad_scale * (T/N) * ((sum_k p[i,k]) * exp(z[i,v]/T - lse[i])
 *                                   - sum_k p[i,k] * [idx[i,k] == v])
 *   dH = g W,  dW = g^T h          (the gradients of grad_scale * loss_mean)
 *
 * Conventions for every entry point:
 *   - All tensors are dense and row-major.  Pointers marked "device" are device
 *     memory of the current HIP device; the library reads and writes them only from
 *     kernels launched on `stream`.  The caller owns every buffer, including the
 *     workspace; the library allocates no device memory and keeps no global state.
 *   - fckl_forward_noalloc is the exception: it keeps one device array per device (see
 *     there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls are
 *     asynchronous: outputs are valid once the stream has reached the call.  The only
 *     host synchronisation is the index check requested by FCKL_FLAG_VALIDATE.
 *   - Errors are returned as status codes; nothing throws across the ABI.  Argument
 *     errors are detected before any HIP call and leave every output untouched.
 *   - Limits of this version: 1 <= K <= 128, K <= V, H % 8 == 0, H <= 65536,
 *     V <= 2^24 with ceil(V/256) * ceil(H/256) < 2^23, N <= 2^31 - 1, T finite and
 *     > 0; a chunk of C tokens (C rounded up to a multiple of 256) needs C <= 2^24,
 *     ceil(C/256) * ceil(H/256) < 2^23 and C * H <= 2^33 (the scheduler's chunks, at
 *     most 8192 tokens, always do).  Outside these limits the calls return
 *     FCKL_ERR_UNSUPPORTED.  Cached indices must be distinct
 *     within a token and lie in [0, V); with FCKL_FLAG_VALIDATE the call checks them
 *     and returns FCKL_ERR_INDEX, otherwise results for such inputs are undefined
 *     (no out-of-bounds memory access is made either way).
 */
#ifndef FCKL_H
#define FCKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fckl_status {
    FCKL_OK = 0,
    FCKL_ERR_INVALID_ARG = 1,   /* null or misaligned pointer, bad size, T <= 0 */
    FCKL_ERR_UNSUPPORTED = 2,   /* a valid request outside this version's limits */
    FCKL_ERR_WORKSPACE = 3,     /* workspace too small for the chosen chunk */
    FCKL_ERR_INDEX = 4,         /* FCKL_FLAG_VALIDATE found an index out of range or repeated */
    FCKL_ERR_HIP = 5            /* a HIP runtime call failed (launch, sync, copy) */
} fckl_status;

/* Element type of topk_logit. */
enum { FCKL_DTYPE_BF16 = 0, FCKL_DTYPE_F32 = 1 };

/* Flags (bitwise or). */
enum {
    FCKL_FLAG_VALIDATE = 1u,       /* check indices on the GPU and report FCKL_ERR_INDEX (syncs the stream) */
    FCKL_FLAG_DW_ACCUMULATE = 2u,  /* backward adds into dW instead of overwriting it */
    FCKL_FLAG_TOPK_FULL_FIRST_PASS = 4u /* fckl_topk: first pass over the whole vocabulary (see there) */
};

/* Kernels of the path, for fckl_profile.kernel_mask (bit 1u << id). */
enum {
    FCKL_KERNEL_PREPARE = 0,       /* teacher softmax over the K entries, entries sorted by index */
    FCKL_KERNEL_FWD_LOGITS = 1,    /* forward logit GEMM + online logsumexp / pick epilogue */
    FCKL_KERNEL_COMBINE = 2,       /* per-token logsumexp over tiles and KL */
    FCKL_KERNEL_MEAN = 3,          /* mean of the per-token loss */
    FCKL_KERNEL_BWD_LOGITS = 4,    /* recompute GEMM + gradient epilogue, writes g^T */
    FCKL_KERNEL_DH = 5,            /* dH = g W (vocabulary splits) */
    FCKL_KERNEL_DH_REDUCE = 6,     /* fixed-order sum of the dH splits */
    FCKL_KERNEL_DW = 7,            /* dW += g^T h */
    FCKL_KERNEL_TRANSPOSE = 8,     /* W^T once per backward call, h^T once per chunk */
    FCKL_KERNEL_SOFTMAX_GRAD = 9,  /* fckl_forward_backward: g from the kept exponentials */
    FCKL_KERNEL_WEIGHTS = 10,      /* sum of the per-token weights */
    FCKL_KERNEL_FULL_TEACHER = 11, /* fckl_full_*: teacher logit GEMM, keeps its logits */
    FCKL_KERNEL_FULL_STUDENT = 12, /* fckl_full_*: student logit GEMM + cross-entropy epilogue */
    FCKL_KERNEL_FULL_COMBINE = 13, /* fckl_full_*: per-token logsumexp (teacher, then student + loss) */
    FCKL_KERNEL_FULL_GRAD = 14,    /* fckl_full_*: g = c (q - p) */
    FCKL_KERNEL_COUNT = 15
};

/*
 * Optional per-kernel timing (caller-owned).  When fckl_desc.profile is not NULL, every
 * launch of a kernel selected by kernel_mask is bracketed by two hipEventRecord calls on
 * the call's stream, using events[2*i] and events[2*i+1] for the i-th bracketed launch
 * (i = count, then count is incremented; launches beyond capacity are not timed).  The
 * caller creates the hipEvent_t handles (passed as void*) and reads the elapsed times
 * after synchronising.  kernel_ids[i] receives the FCKL_KERNEL_* id of launch i,
 * work[i] the number of tokens that launch processed and, when vocab_rows is not NULL,
 * vocab_rows[i] the vocabulary rows it covered: V, except for the launches of the
 * two-pass backward, which run one vocabulary slab at a time (fckl_desc.vocab_slab), and
 * 0 for kernels without a vocabulary dimension (transposes, reductions, weights).
 */
typedef struct fckl_profile {
    uint32_t kernel_mask;
    int32_t capacity;
    int32_t count;
    void **events;           /* host array of 2 * capacity hipEvent_t */
    int32_t *kernel_ids;     /* host array of capacity */
    int32_t *work;           /* host array of capacity */
    int32_t *vocab_rows;     /* host array of capacity, or NULL */
} fckl_profile;

/* Problem description shared by every call. */
typedef struct fckl_desc {
    int64_t N;            /* tokens (batch x sequence, flattened) */
    int32_t H;            /* hidden size */
    int32_t V;            /* vocabulary size */
    int32_t K;            /* cached teacher entries per token */
    float T;              /* temperature (student and teacher logits are divided by it) */
    int32_t chunk;        /* tokens per chunk; 0 = let fckl_plan choose */
    int32_t logit_dtype;  /* FCKL_DTYPE_BF16 or FCKL_DTYPE_F32 */
    uint32_t flags;       /* FCKL_FLAG_* */
    fckl_profile *profile;/* optional kernel timing, NULL = none */
    int32_t vocab_slab;   /* vocabulary rows per slab of the two-pass backward: a multiple
                             of 256, or 0 = the library's choice (see fckl_backward) */
} fckl_desc;

/*
 * Chunk scheduler (the method handles one slice of the tokens at a time and drops its
 * intermediates before the next: axbrief.com, "Breaking the Bottleneck with Offline
 * Caching and Chunked Loss"; sized here for the 288 GB of HBM3E of one MI355X).  Pure
 * host function, no HIP call.
 * Chooses the number of tokens per chunk for `desc` so that the workspace fits in
 * `budget_bytes` (0 = the library default, 12 GiB), preferring the largest chunk up to
 * 8192 tokens (beyond that the saving in re-streamed W and in dW's per-chunk fp32
 * additions is small, and the logit products' grids grow past where they gain) and then
 * evening out the chunks.  If desc->chunk > 0 that chunk is kept and only its workspace
 * size is reported.
 *   chunk_out    host, may be NULL: tokens per chunk.
 *   ws_bytes_out host, may be NULL: workspace bytes fckl_forward/fckl_backward need.
 * Returns FCKL_ERR_WORKSPACE when even the smallest chunk does not fit.
 */
fckl_status fckl_plan(const fckl_desc *desc, size_t budget_bytes, int32_t *chunk_out,
                      size_t *ws_bytes_out);

/*
 * Workspace bytes needed for `desc` run with `chunk` tokens per chunk (chunk >= 1).
 * The workspace depends on chunk, H, V, K and desc->vocab_slab only, never on N: peak
 * memory has no N x V term.  Pure host function.
 */
fckl_status fckl_workspace_size(const fckl_desc *desc, int32_t chunk, size_t *ws_bytes_out);

/*
 * Forward pass: per-token loss, saved lse, and the mean loss.
 *   h          device, bf16 [N,H]      student hidden states (16-byte aligned)
 *   W          device, bf16 [V,H]      student LM head (16-byte aligned)
 *   topk_idx   device, int32 [N,K]     teacher's cached vocabulary indices
 *   topk_logit device, bf16 or f32 [N,K] (desc->logit_dtype) teacher's cached logits
 *   loss_tok   device, f32 [N]         out: loss[i]
 *   lse        device, f32 [N]         out: log sum_v exp(z[i,v]/T), kept for fckl_backward
 *   loss_mean  device, f32 [1]         out: mean of loss_tok (may be NULL)
 *   ws         device, ws_bytes bytes, 256-byte aligned; contents on entry are ignored
 * Chunk: desc->chunk, or fckl_plan(desc, ws_bytes) when it is 0.
 * Deterministic: the same inputs give bit-identical outputs.
 */
fckl_status fckl_forward(const fckl_desc *desc, const void *h, const void *W,
                         const int32_t *topk_idx, const void *topk_logit,
                         float *loss_tok, float *lse, float *loss_mean,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * Backward pass: gradients of grad_scale * loss_mean with respect to h and W.  Each
 * chunk's logits are recomputed with the same tiles as the forward pass; the chunk's
 * gradient g (bf16, written once, vocabulary-major, in the workspace) feeds the dH and
 * dW products (the backward pass repeats the projection per chunk: axbrief.com,
 * "Breaking the Bottleneck with Offline Caching and Chunked Loss").  A chunk is worked
 * through in slabs of the vocabulary: the logits, g, the slab's share of dH and its
 * rows of dW of one slab before the next, so the workspace holds g for one slab only.
 * desc->vocab_slab sets the slab (rows, a multiple of 256; the last slab also takes
 * the remainder, up to twice that); 0 lets the planner choose slabs of 64-tile
 * multiples holding at most about 1.25 GB of g each (at 8192 tokens per chunk: 65536
 * rows, so three slabs at V = 201088), and one slab when that is the whole vocabulary.
 * The slabs change the order of the dH sum only; loss, lse and dW do not depend on them.
 *   lse        device, f32 [N]         the lse written by fckl_forward for these inputs
 *   grad_scale                         upstream gradient of loss_mean (1 for a plain loss)
 *   dH         device, f32 [N,H]       out: overwritten (16-byte aligned)
 *   dW         device, f32 [V,H]       out: overwritten, or added to with FCKL_FLAG_DW_ACCUMULATE;
 *                                      accumulated in fp32 across chunks in chunk order
 * Other arguments as in fckl_forward.  Deterministic.
 */
fckl_status fckl_backward(const fckl_desc *desc, const void *h, const void *W,
                          const int32_t *topk_idx, const void *topk_logit, const float *lse,
                          float grad_scale, float *dH, float *dW,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Token masks and per-token weights (padded batches).  The same passes with weights
 * w[N] (device, f32; a masked token has w = 0; NULL = every weight 1, which is
 * fckl_forward / fckl_backward):
 *   loss_mean = sum_i w[i] loss[i] / sum_i w[i]                  (0 when all w are 0)
 *   g[i,v]    = grad_scale * T * w[i] / sum_j w[j] * ((sum_k p[i,k]) exp(z[i,v]/T - lse[i])
 *                                                     - sum_k p[i,k] [idx[i,k] == v])
 * loss_tok and lse stay per token and unweighted.  The pages speak of no masks; this
 * is the reduction that losses with ignored positions use.  Weights must be finite and
 * >= 0 (not checked).  The sums over tokens run in a fixed order in fp64, so results
 * stay deterministic.  grad_scale_dev (device, f32 [1], may be NULL) multiplies
 * grad_scale on the device, for an upstream gradient that is itself on the GPU (an
 * autograd graph) and should not be read back to the host first.
 */
fckl_status fckl_forward_ex(const fckl_desc *desc, const void *h, const void *W,
                            const int32_t *topk_idx, const void *topk_logit, const float *weights,
                            float *loss_tok, float *lse, float *loss_mean,
                            void *ws, size_t ws_bytes, void *stream);
fckl_status fckl_backward_ex(const fckl_desc *desc, const void *h, const void *W,
                             const int32_t *topk_idx, const void *topk_logit, const float *weights,
                             const float *lse, float grad_scale, const float *grad_scale_dev,
                             float *dH, float *dW, void *ws, size_t ws_bytes, void *stream);

/*
 * fckl_forward_ex without a caller workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The chunk's buffers live in a device array of the library instead (64 MiB
 * per device, held from the first call on that device until the process ends; the first
 * call on a device looks up its address once).  The call allocates nothing; the caller
 * still passes the inputs and outputs, as for fckl_forward_ex (weights may be NULL).
 * The chunk is desc->chunk, or, when it is 0, the largest chunk (up to 8192 tokens,
 * evened out over N) whose forward buffers fit the array: about 4 V + 12 K bytes per
 * token of the chunk (7936 tokens at V = 201088, K = 100).
 * Returns FCKL_ERR_WORKSPACE, before any HIP call, when desc->chunk's buffers do not fit
 * the array or even a 256-token chunk does not (V above about 7.3 million).  Every call on
 * a device uses that device's one array, which keeps the last call's contents: calls that
 * overlap on one device (two streams, two host threads) race and must be serialised by
 * the caller.  Results are those of fckl_forward_ex run with the same chunk, bit for bit.
 */
fckl_status fckl_forward_noalloc(const fckl_desc *desc, const void *h, const void *W,
                                 const int32_t *topk_idx, const void *topk_logit, const float *weights,
                                 float *loss_tok, float *lse, float *loss_mean, void *stream);

/*
 * Forward and backward in one call, for a loss that is the last operation of the step,
 * so that its upstream gradient grad_scale is known before the forward pass runs.  The
 * outputs are those of fckl_forward_ex followed by fckl_backward_ex (weights may be NULL).
 * The logits are formed once per chunk instead of twice: the forward epilogue keeps
 * 2^(z/T log2 e - m) in bf16 in the workspace, with m the maximum over each 128-row half
 * of a 256-row vocabulary tile, and once the chunk's lse is known a streaming kernel
 * turns those values into g.  That is 6 N V H flop instead of 8.  g differs from the
 * two-call path by the bf16 rounding of the kept values, which has the same relative size
 * as the rounding of g itself.  g, dH and dW are formed one vocabulary slab at a time, as
 * in fckl_backward (desc->vocab_slab).  Workspace: the kept values take 2 V bytes per
 * token of the chunk more than the two-call path needs; fckl_single_plan gives the size
 * (and, with desc->chunk = 0, the chunk as fckl_plan chooses it for that layout), and the
 * call uses the chunk fckl_single_plan(desc, ws_bytes) reports.
 */
fckl_status fckl_single_plan(const fckl_desc *desc, size_t budget_bytes, int32_t *chunk_out,
                             size_t *ws_bytes_out);
fckl_status fckl_forward_backward(const fckl_desc *desc, const void *h, const void *W,
                                  const int32_t *topk_idx, const void *topk_logit,
                                  const float *weights, float grad_scale,
                                  float *loss_tok, float *lse, float *loss_mean,
                                  float *dH, float *dW, void *ws, size_t ws_bytes, void *stream);

/*
 * Teacher-side top-K extraction: the cache the loss reads.  The teacher's top logits
 * (100, or 10) and their vocabulary indices are extracted once per position and stored
 * ("Preparing Offline Top-K Logits", getaibook.com; "Breaking the Bottleneck with
 * Offline Caching and Chunked Loss", axbrief.com).  For each token i, the K entries of
 * z[i,v] = sum_j h[i,j] W[v,j] with the largest z, in descending order of z; equal
 * values are ordered by the smaller index first.  z is accumulated in fp32 from bf16
 * inputs (the same GEMM tiles as the loss).  Two passes of the product: the maxima of z
 * over K or more disjoint row slices of the vocabulary give a threshold at or below the
 * K-th largest z, and the logits at or above it are sorted.  The first pass covers
 * every 4th 256-row tile (64-row slices) when that gives at least 4 K maxima, so it
 * costs a quarter of the product; a chunk in which some token then has more than 2048
 * candidates is redone on the GPU with a first pass over every tile (no host round
 * trip).  FCKL_FLAG_TOPK_FULL_FIRST_PASS always takes the first pass over every tile.
 * The result does not depend on which first pass ran.
 *   desc       N, H, V, K (K <= 128), chunk (0 = up to 8192 tokens); logit_dtype selects
 *              the type of topk_logit; flags: FCKL_FLAG_TOPK_FULL_FIRST_PASS or 0; T and
 *              profile are not used (T must be valid)
 *   h          device, bf16 [N,H]      the teacher's final hidden states
 *   W          device, bf16 [V,H]      the teacher's LM head
 *   topk_idx   device, int32 [N,K]     out: indices, descending z
 *   topk_logit device, bf16 or f32 [N,K] out: z at those indices (bf16: rounded to nearest even)
 *   ws         device, fckl_topk_workspace_size bytes, 256-byte aligned
 * Returns FCKL_ERR_UNSUPPORTED when V > 2097152, when more than 2048 logits of one
 * token lie at or above its threshold even after a first pass over every tile (massive
 * ties, e.g. a zero head), or when a token has fewer than K comparable logits (a NaN
 * in its hidden row makes them all NaN); the outputs are then undefined.  Checking that
 * needs one host synchronisation at the end of the call.
 */
fckl_status fckl_topk_workspace_size(const fckl_desc *desc, int32_t chunk, size_t *ws_bytes_out);
fckl_status fckl_topk(const fckl_desc *desc, const void *h, const void *W, int32_t *topk_idx,
                      void *topk_logit, void *ws, size_t ws_bytes, void *stream);

/*
 * fckl_topk without the host synchronisation: the status the call would return for the
 * data (FCKL_OK, or FCKL_ERR_UNSUPPORTED for a candidate overflow or NaN logits) is
 * written on the stream to `status` (device, one uint32), which the caller reads when
 * it chooses.  The call records only kernel launches, so it can be captured in a HIP
 * graph.  Argument errors are still returned before any HIP call; `status` must not be
 * NULL.
 */
fckl_status fckl_topk_async(const fckl_desc *desc, const void *h, const void *W, int32_t *topk_idx,
                            void *topk_logit, void *ws, size_t ws_bytes, uint32_t *status,
                            void *stream);

/*
 * Online distillation against the teacher's whole distribution: the setting the cached
 * top-K teacher replaces, where the teacher's full-vocabulary distribution is computed
 * beside the student's ("The Distillation Bottleneck", getaibook.com; the teacher run on
 * the fly, "The 250GB VRAM Wall in Long-Context Distillation", axbrief.com).  The teacher's
 * final hidden states and LM head are inputs; the teacher's logits are formed chunk by
 * chunk like the student's and never exist for all N tokens.  With
 *   p = softmax(h_t W_t^T / T), q = softmax(h W^T / T) over the whole vocabulary,
 *   loss_tok[i] = T^2 sum_v p[i,v] (log p[i,v] - log q[i,v]),
 *   lse[i] = log sum_v exp(z[i,v] / T) of the student,
 *   loss_mean = sum_i w_i loss_tok[i] / sum_i w_i (weights NULL: the plain mean),
 *   dH, dW = the gradients of grad_scale * loss_mean with respect to h and W, through
 *   g[i,v] = grad_scale T w_i / sum_j w_j (q[i,v] - p[i,v]) (weights NULL: w_i / sum = 1/N).
 * The teacher receives no gradient.  Per chunk the teacher product keeps its logits in
 * fp32 (4 V bytes per token of workspace) and the student product keeps 2^(z/T log2 e - m)
 * in bf16, as fckl_forward_backward does, so the logits of each model are formed once:
 * 2 N V Ht + 6 N V H flop.
 *   desc       N, H (the student's), V, T, chunk, flags (FCKL_FLAG_DW_ACCUMULATE), profile,
 *              vocab_slab (g, dH and dW one vocabulary slab at a time, as in fckl_backward);
 *              K and logit_dtype are not read; FCKL_FLAG_VALIDATE has no effect
 *   H_teacher  the teacher's hidden size (a multiple of 8, at most 65536)
 *   h, W       device, bf16 [N,H], [V,H]            the student
 *   h_t, W_t   device, bf16 [N,H_teacher], [V,H_teacher]  the teacher (same vocabulary)
 *              (h, W, h_t, W_t and dH 16-byte aligned)
 *   weights    device, f32 [N] or NULL              per-token weights: finite and >= 0 (not
 *              checked); all 0 gives loss_mean = 0 and zero gradients
 *   loss_tok, lse  device, f32 [N]  out;  loss_mean device, f32 [1] out or NULL
 *   dH         device, f32 [N,H] out;  dW device, f32 [V,H] out (or accumulated)
 *   ws         device, 256-byte aligned; fckl_full_plan gives the size
 * fckl_full_plan chooses the chunk as fckl_plan does, for this workspace (budget 0 = 12 GiB).
 */
fckl_status fckl_full_plan(const fckl_desc *desc, int32_t H_teacher, size_t budget_bytes,
                           int32_t *chunk_out, size_t *ws_bytes_out);
fckl_status fckl_full_forward_backward(const fckl_desc *desc, int32_t H_teacher, const void *h,
                                       const void *W, const void *h_t, const void *W_t,
                                       const float *weights, float grad_scale, float *loss_tok,
                                       float *lse, float *loss_mean, float *dH, float *dW, void *ws,
                                       size_t ws_bytes, void *stream);

/*
 * x[i] *= *scale for i in [0, n): the chain rule for an upstream gradient that arrives
 * after the gradients were formed.  The torch module ("Configuring Fused Chunked KL
 * Loss", getaibook.com: the fused loss replaces the stock loss in the training loop)
 * runs fckl_forward_backward in its forward pass with grad_scale = 1 and, in its
 * backward pass, scales dH and dW by the upstream gradient where it already lives, on
 * the device, without a host read-back.
 *   x      device, f32 [n], in place (16-byte aligned)
 *   n      >= 0
 *   scale  device, f32 [1]
 * Returns FCKL_ERR_INVALID_ARG for NULL pointers, n < 0 or a misaligned x.
 */
fckl_status fckl_scale(float *x, int64_t n, const float *scale, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *fckl_status_string(fckl_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t fckl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FCKL_H */
