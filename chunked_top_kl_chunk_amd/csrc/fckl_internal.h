// fckl_internal.h -- host-side plan, workspace layout and kernel launchers (not part of the ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fckl.h"

namespace fckl {

// Token tile and vocabulary tile of the logit GEMMs (rows of W x tokens of h).
constexpr int kVocabTile = 256;
constexpr int kTokenTile = 256;
// Hidden-dimension tile of the dH and dW products.  A hidden size that is not a
// multiple (2880) leaves the last tile partly masked; measured on the 32K-token,
// 201088-entry vocabulary shape, 256-wide tiles with that waste beat exact 192-wide ones
// for dH (higher operand reuse per loaded byte) and tie for dW.
constexpr int kHiddenTile = 256;
constexpr int kMaxK = 128;
// Teacher top-K extraction: candidates kept per token (the logits at or above the K-th
// largest of the token's 32-row sub-tile maxima), and the most sub-tile maxima per token
// (V <= 2^21; their buffer is 4 bytes per maximum and token of a chunk).
constexpr int kTopkCap = 2048;
constexpr int kTopkStride = 4;      // the partial first pass visits every 4th vocabulary tile
constexpr int kTopkSortSub = 2048;  // slice maxima per token up to which the threshold is found by a sort
constexpr int kTopkMaxSub = 65536;
constexpr int32_t kMaxChunk = 8192;
constexpr size_t kDefaultBudget = size_t(12) << 30;  // 12 GiB of the 288 GB HBM3E
// The two-pass backward works through a chunk's vocabulary in slabs whose g^T holds at
// most about this many bytes, in whole multiples of 64 vocabulary tiles (unless the
// descriptor sets the slab).  64 tiles times a hidden size of 12 or 16 tiles gives dW
// launches of whole rounds of 256 work-groups.
constexpr size_t kSlabBytes = size_t(1250) << 20;
constexpr int32_t kSlabTileStep = 64;

// Kernel limits.  The GEMM operand loaders keep each lane's offset inside a 256-row
// tile in 32 bits (up to 255 rows of the operand's pitch; the transposed g^T operand of
// dH spans 64 rows of a k-step), and the pitch of W^T is Vpad, that of g^T and h^T the
// padded chunk: both at most kMaxPitch elements.  A
// non-persistent GEMM launches one 512-thread work-group per 256 x 256 output tile, and
// HIP counts a grid dimension in 32-bit work-items: at most kMaxTiles tiles.  The dH
// split reduce runs one thread per 4 elements of a chunk's dH: at most kMaxChunkElems
// elements.
constexpr int64_t kMaxPitch = int64_t(1) << 24;
constexpr int64_t kMaxTiles = (int64_t(1) << 23) - 1;
constexpr int64_t kMaxChunkElems = int64_t(1) << 33;

// Which calls a workspace layout serves: the two passes, the single call and the
// full-teacher variant (whose forward product keeps its exponentials: off_mw and off_ex
// added), or the forward pass alone (the buffers of the forward pass only, up to off_part,
// with off_err; the others are left at 0).
enum class LayoutKind { TwoPass, Keep, ForwardOnly };

// Where each per-chunk buffer lives inside the caller's workspace.  Every buffer is
// sized by the chunk, never by N.
struct Layout {
    LayoutKind kind = LayoutKind::TwoPass;
    int32_t C = 0;          // tokens per chunk
    int32_t Cpad = 0;       // C rounded up to kTokenTile
    int32_t nVt = 0;        // vocabulary tiles: ceil(V / kVocabTile)
    int32_t Vpad = 0;       // nVt * kVocabTile (row pitch of g)
    int32_t cnt_stride = 0; // bytes per token of the per-tile entry-count table
    int32_t dh_splits = 0;  // vocabulary splits of the dH product, over all slabs
    int32_t nslab = 1;      // vocabulary slabs of the gradient products (1 in a forward-only layout)
    int32_t slab_tiles = 0; // vocabulary tiles per slab; the last slab takes the remainder
    int32_t gT_tiles = 0;   // vocabulary tiles of the largest slab (rows of g^T / kVocabTile)
    size_t off_idx = 0;     // int32 [Cpad, K]   cached indices, sorted ascending per token
    size_t off_p = 0;       // f32   [Cpad, K]   teacher probabilities in the same order
    size_t off_zk = 0;      // f32   [Cpad, K]   student logit at each sorted index
    size_t off_psum = 0;    // f32   [Cpad]      sum_k p
    size_t off_negent = 0;  // f32   [Cpad]      sum_k p log p
    size_t off_cnt = 0;     // u8    [Cpad, cnt_stride] entries below each vocabulary tile start
    size_t off_part = 0;    // f32x2 [nVt, Cpad] per-tile (max, sum exp) of z/T, base 2
    size_t off_mw = 0;      // f32   [2 nVt, Cpad] max of z/T (base 2) per 128-row half tile,
                            //       kept with the exponentials (keep layouts only)
    size_t off_wsum = 0;    // f32   [2]         sum of the token weights and its inverse
    size_t off_ex = 0;      // bf16  [Cpad, Vpad] kept 2^(z/T log2 e - m) (keep layouts only)
    size_t off_gT = 0;      // bf16  [gT_tiles * 256, Cpad] chunk gradient w.r.t. the logits of
                            //       one slab, vocabulary-major (the operand of both products)
    size_t off_hT = 0;      // bf16  [H, Cpad]    chunk hidden states, transposed (dW operand)
    size_t off_WT = 0;      // bf16  [H, Vpad]    LM head, transposed (dH operand)
    size_t off_dhp = 0;     // f32   [dh_splits, Cpad, H] split partial sums of dH
    size_t off_err = 0;     // u32   [4]         index-check flag
    size_t total = 0;
};

// Workspace of the teacher top-K extraction (its own, much smaller than the loss's).
struct TopkLayout {
    int32_t C = 0, Cpad = 0, nVt = 0;
    int32_t nSubFull = 0;   // maxima per token of a first pass over every tile (per tile, or per 32- or
                            // 16-row slice)
    int32_t nSubPart = 0;   // maxima per token of a first pass over every kTopkStride-th tile (64-row
                            // slices); 0 = that pass is not used
    size_t off_tmax = 0;    // f32   [max(nSubFull, nSubPart), Cpad]  slice maxima
    size_t off_thr = 0;     // f32   [Cpad]        K-th largest of a token's maxima
    size_t off_count = 0;   // u32   [Cpad]        candidates found per token
    size_t off_cand = 0;    // u64   [Cpad, kTopkCap] candidate keys
    size_t off_err = 0;     // u32   [4]           [0] error flag, [1] the chunk's retry flag
    size_t total = 0;
};

// Workspace of the full-teacher variant: the loss layout (for the student) followed by
// the teacher's fp32 logits of the chunk and the per-tile partials of both products.
struct FullLayout {
    Layout base;
    int32_t Ht = 0;
    size_t off_at = 0;      // f32   [Vpad, Cpad]  a_t = z_t log2(e) / T
    size_t off_part_t = 0;  // f32x2 [nVt, Cpad]   teacher (max, sum) per tile
    size_t off_px = 0;      // f32   [nVt, Cpad]   sum over the tile of p (a_t - a_s)
    size_t off_lt2 = 0;     // f32   [Cpad]        teacher base-2 logsumexp
    size_t off_ls2 = 0;     // f32   [Cpad]        student base-2 logsumexp
    size_t total = 0;
};

fckl_status check_desc(const fckl_desc *d);
fckl_status make_topk_layout(const fckl_desc *d, int32_t chunk, TopkLayout *L);
fckl_status make_full_layout(const fckl_desc *d, int32_t Ht, int32_t chunk, FullLayout *L);
fckl_status plan_full_chunk(const fckl_desc *d, int32_t Ht, size_t budget, FullLayout *L);
fckl_status make_layout(const fckl_desc *d, int32_t chunk, Layout *L, LayoutKind kind = LayoutKind::TwoPass);
fckl_status plan_chunk(const fckl_desc *d, size_t budget, Layout *L, LayoutKind kind = LayoutKind::TwoPass);
// Slab s of L (0 <= s < L.nslab): its first vocabulary tile and its tile count.
void slab_tiles_of(const Layout &L, int32_t s, int32_t *vt0, int32_t *nvt);
// dH splits of a slab of nvt vocabulary tiles with Cpad tokens and hidden size H.
int32_t slab_split_count(int32_t Cpad, int32_t H, int32_t nvt);
// The dH product's k-step (vocabulary rows); a split is a whole number of them.
constexpr int32_t kDhStep = 64;
// Slab s's dH splits: vocabulary rows per split and the number of splits holding at
// least one row of the V-row vocabulary (the slab's partial sums are that many).
void slab_split_rows(const Layout &L, int32_t V, int32_t H, int32_t s, int32_t *ksplit, int32_t *used);
// dH partial sums of the first nslabs slabs (all of them: the count the reduce sums).
int32_t dh_partials(const Layout &L, int32_t V, int32_t H, int32_t nslabs);

// The allocation-free forward pass (fckl_forward_noalloc) runs in a device array of the
// library instead of a caller's workspace: its size, and the lookup of its address on the
// current device (once per device; a HIP status).
constexpr size_t kScratchBytes = size_t(64) << 20;
int scratch_address(void **ptr);

// ------------------------------------------------------------------ launchers
// All return hipSuccess (0) or the launch error; they never synchronise.

struct ChunkArgs {
    const uint16_t *h;          // chunk's first row of h [.., H]
    const uint16_t *W;          // [V, H]
    const int32_t *idx;         // chunk's first row of topk_idx [.., K]
    const void *tl;             // chunk's first row of topk_logit
    int logit_f32;
    int32_t rows;               // valid tokens in this chunk (<= C)
    int32_t H, V, K;
    float T;
    char *ws;
    const Layout *L;
    // The vocabulary slab the backward launches cover: its first tile, its tile count and
    // the index of its first dH split (the whole vocabulary and 0 outside the two-pass
    // backward).
    int32_t vt0 = 0, nvt = 0, split0 = 0;
};

// Per-token scale of the gradient with respect to z: coef * w[i] * (*inv_wsum) with
// weights, coef alone without (w == NULL), times *mul when mul is set.  coef = grad_scale * T, divided by N when
// there are no weights.
struct GradScale {
    float coef = 0.0f;
    const float *w = nullptr;         // chunk's first token, or NULL
    const float *inv_wsum = nullptr;  // device scalar, used with w
    const float *mul = nullptr;       // device scalar multiplying coef, or NULL
};

// `gs` != NULL: the teacher probabilities and their sum are stored multiplied by the
// token's gradient scale (the backward pass uses them only in that form).
int launch_prepare(const ChunkArgs &a, bool validate, void *stream, const GradScale *gs = nullptr);
// keep_exp: also write 2^(z/T log2 e - m) in bf16 to the kept-exponential buffer and
// the half-tile maxima m (single-call path; a keep layout).
int launch_forward_logits(const ChunkArgs &a, void *stream, bool keep_exp = false);
int launch_combine(const ChunkArgs &a, float *loss_tok, float *lse, void *stream);
int launch_mean(const float *loss_tok, int64_t N, float *loss_mean, void *stream);
int launch_weighted_mean(const float *loss_tok, const float *w, int64_t N, float *loss_mean, void *stream);
int launch_weight_sum(const float *w, int64_t N, float *out2, void *stream);
int launch_backward_logits(const ChunkArgs &a, const float *lse, void *stream);
// Single-call path: g (both layouts) from the kept exponentials, the chunk's lse and gs.
int launch_softmax_grad(const ChunkArgs &a, const float *lse, const GradScale &gs, void *stream);
int launch_dh(const ChunkArgs &a, void *stream);
int launch_dh_reduce(const ChunkArgs &a, float *dH, void *stream);
int launch_dw(const ChunkArgs &a, float *dW, bool accumulate, void *stream);
int launch_transpose_head(const ChunkArgs &a, void *stream);
int launch_transpose_chunk(const ChunkArgs &a, void *stream);
int launch_zero_flag(uint32_t *flag, void *stream);
int launch_scale(float *x, int64_t n, const float *scale, void *stream);
// *status = *flag ? code : 0 (one thread).
int launch_topk_status(const uint32_t *flag, uint32_t *status, uint32_t code, void *stream);

// Teacher top-K extraction of one chunk (a.L is unused; T is the top-K layout): the
// 32-row sub-tile maxima of z, the per-token threshold, the candidates at or above it,
// and the ordered selection (topk_logit written as f32 or bf16).  Candidate overflow
// sets the error flag.
// Full-teacher variant, per chunk (a.L is the student's loss layout inside F).
int launch_full_teacher(const ChunkArgs &a, const FullLayout &F, const uint16_t *h_t, const uint16_t *W_t,
                        void *stream);
int launch_full_combine_teacher(const ChunkArgs &a, const FullLayout &F, void *stream);
int launch_full_student(const ChunkArgs &a, const FullLayout &F, void *stream);
int launch_full_combine_student(const ChunkArgs &a, const FullLayout &F, float *loss_tok, float *lse, void *stream);
int launch_full_grad(const ChunkArgs &a, const FullLayout &F, const GradScale &gs, void *stream);

// Teacher top-K, per chunk.  `partial`: the first pass over every kTopkStride-th tile;
// `guard` (may be NULL): the kernel returns at once unless *guard != 0.
int launch_topk_max(const ChunkArgs &a, const TopkLayout &T, bool partial, const uint32_t *guard, void *stream);
int launch_topk_threshold(const ChunkArgs &a, const TopkLayout &T, bool partial, const uint32_t *guard,
                          uint32_t *retry_reset, void *stream);
int launch_topk_collect(const ChunkArgs &a, const TopkLayout &T, const uint32_t *guard, void *stream);
int launch_topk_select(const ChunkArgs &a, const TopkLayout &T, int32_t *topk_idx, void *topk_logit, bool logit_f32,
                       const uint32_t *guard, uint32_t *retry, void *stream);

}  // namespace fckl
