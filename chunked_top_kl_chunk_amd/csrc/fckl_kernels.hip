// fckl_kernels.hip -- gfx950 kernels of the fused chunked top-K KL loss.
//
// Per chunk of tokens (one slice of the sequence at a time, "Breaking the Bottleneck
// with Offline Caching and Chunked Loss", axbrief.com; the output projection is folded
// into the loss, "What actually changed?", calcaas.com):
//
//   prepare          teacher softmax over the K cached logits, entries sorted by index,
//                    per-vocabulary-tile entry counts
//   forward_logits   z^T tile = W_tile . h_tile^T on MFMA (bf16 in, fp32 accumulate);
//                    the epilogue keeps z in registers, reduces max / sum exp(z/T) over
//                    the tile's 256 vocabulary rows per token and picks z at the cached
//                    indices owned by the tile.  Only (max, sum) per tile and the K
//                    picked logits per token leave the chip.
//   combine          per token: logsumexp over the tiles, the KL term, the loss
//   backward_logits  the same MFMA tiles recompute z (the extra projection in the
//                    backward pass that the chunked loss pays for, axbrief.com) over one
//                    vocabulary slab of the chunk; the epilogue forms
//                    g = c((sum p) softmax(z/T) - scatter(p, idx)), rounds it to bf16 and
//                    writes the slab's g once, vocabulary-major g^T [slab rows, C], the
//                    operand of both products below
//   dh               the slab's share of dH_chunk^T = W^T . g^T over the vocabulary (g^T
//                    read through transposing LDS reads; split over the slab's rows; one
//                    fixed-order reduce of every slab's splits after the last slab)
//   dw               the slab's rows of dW += g^T . h_chunk (fp32, chunk after chunk: the
//                    first chunk stores, the others add with fp32 atomics at L2, one adder
//                    per element)
//   transpose        W -> W^T once per backward call, h_chunk -> h_chunk^T per chunk
//
// GEMM core: 256 x 256 tiles, 512 threads = 8 wave64s, each wave owns a 128 x 64 block
// of fp32 accumulators in the v_mfma_f32_32x32x16_bf16 output layout.  The logit
// products run 32x32x16 MFMAs; dH and dW run v_mfma_f32_16x16x32_bf16, which holds a
// higher clock under the board's power limit, and move their accumulators into the
// 32x32x16 layout after the k loop, so every epilogue indexes one layout.  Operands are
// read k-major (contiguous along the reduction), which is why the backward products use
// W^T and h_chunk^T; the one exception is g^T in the dH product, whose fragments come
// from gfx950's transposing LDS reads.  Each lane's 16-byte piece goes from global
// memory straight into LDS (global_load_lds_dwordx4, no register staging); two LDS
// stages of 64-deep k-steps, one barrier per step, and an XOR swizzle of the 16-byte
// chunks that keeps the MFMA operand reads free of bank conflicts.
// The two logit kernels are persistent (one work-group per compute unit looping over
// tiles), which removes the per-work-group dispatch gap between tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>

#include <type_traits>

#include "fckl_internal.h"

namespace fckl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------------ small helpers

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values -> packed bf16 pair (lo in bits 0-15), rounded to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Merge two (max, sum) pairs of base-2 exponentials: sum_a 2^(x-ma) + sum_b 2^(x-mb).
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2)
{
    float M = fmaxf(m, m2);
    if (M == kNegInf) {
        // both empty (sums 0), or values that were all NaN (fmaxf skipped them, their
        // sum is NaN): keep the NaN so that it reaches the lse
        s += s2;
        return;
    }
    s = s * fast_exp2(m - M) + s2 * fast_exp2(m2 - M);
    m = M;
}

// Work-group id -> (tile along M, tile along N).  Work-groups are dealt to the eight
// XCDs round-robin; renumber them so that each XCD runs a contiguous range, then walk
// that range in groups of GM tiles along M x all tiles along N, so that the tiles in
// flight on one XCD share operand rows in its L2.
__device__ __forceinline__ void map_tile(int bid, int nM, int nN, int GM, int &tm, int &tn)
{
    const int total = nM * nN;
    const int per = total >> 3;
    int id = bid;
    if (bid < (per << 3))
        id = (bid & 7) * per + (bid >> 3);
    const int group = GM * nN;
    const int g = id / group;
    const int first = g * GM;
    const int gm = min(nM - first, GM);
    const int r = id - g * group;
    tm = first + r % gm;
    tn = r / gm;
}

// ------------------------------------------------------------------ GEMM core, direct-to-LDS

// Lanes whose 16-byte piece of an operand lies outside it (rows past the end, k past
// the reduction length) load these zeros instead, so partial tiles need no branches.
__device__ __attribute__((aligned(16))) const uint32_t kZeroPage[4] = {0u, 0u, 0u, 0u};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// global_load_lds_dwordx4: each lane of the wave copies 16 bytes from `src` to LDS at
// lds_wave_base + 16 * lane (lds_wave_base is the same for the whole wave; M0 holds it).
// ASM: written as inline asm, so that the compiler does not see an LDS write through a
// global instruction.  While it sees one in flight it waits for every LDS read
// (lgkmcnt(0)) wherever a fragment read's result is used, which the 16x16x32 loop, with
// fragment reads a full row group ahead, cannot afford.  The copies' completion is then
// tracked by hand: every LDS read of copied data follows an explicit vmcnt wait and a
// barrier.  No other code here uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool ASM = false>
__device__ __forceinline__ void copy16_to_lds(const void *src, char *lds_wave_base)
{
    if constexpr (ASM) {
        const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m)
                     : "memory", "m0");
    } else {
        __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds_wave_base, 16, 0, 0);
    }
}
#pragma clang diagnostic pop

// global_load_lds_dword: 4 bytes per lane to lds_wave_base + 4 * lane.
__device__ __forceinline__ void copy4_to_lds(const void *src, char *lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds_wave_base, 4, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time unrolled).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their no-wait maxima).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Operand tile whose k dimension is contiguous: ROWS rows x BKK k, one row = BKK/8
// 16-byte chunks.  gfx950's LDS serves 256 bytes (64 banks) per cycle, i.e. 16 lanes
// of a ds_read_b128; the fragment read has those 16 lanes on 16 consecutive rows at
// one chunk, so the chunk index is XOR-swizzled with the row to spread them over all
// 16 bank groups.
template <int ROWS, int BKK, int NT>
struct KTile {
    static constexpr int CPR = BKK / 8;
    static constexpr int CHUNKS = ROWS * CPR;
    static_assert(CHUNKS % NT == 0, "whole wave instructions");
    static constexpr int PER = CHUNKS / NT;
    static constexpr int BYTES = CHUNKS * 16;

    static_assert(CPR == 8 || CPR == 4, "k-step of 64 or 32");
    __device__ __forceinline__ static int sw(int row)
    {
        return CPR == 8 ? ((row & 7) ^ ((row >> 3) & 1)) : ((row >> 2) & 3);
    }

    // Source state.  Piece i of a lane covers tile row r + i * RSTRIDE at 16-byte k-chunk
    // kc, with r and kc the same for every piece: the slot of piece i is
    // (i * NT/64 + wave) * 64 + lane, i.e. row (i * NT/64 + wave) * 64/CPR + lane/CPR and
    // chunk lane % CPR, and the swizzle of a row depends only on row bits that i does not
    // change.  So a lane keeps the element offset of its first piece, its k offset
    // kc * 8 (the k-range check) and the rows left below the operand's end; `base`
    // (uniform) points at row row0, column k0 of the current k-slice.
    static constexpr int RSTRIDE = NT / CPR;
    static_assert((NT / 64) % 2 == 0 || CPR == 4, "swizzle invariant across pieces");
    struct Src {
        const uint16_t *base;
        uint32_t off0;          // element offset of piece 0 from base
        uint32_t step;          // element offset between consecutive pieces (RSTRIDE rows)
        int kc8;                // k offset of the lane's chunk within the slice
        int rlim;               // rows_valid - row0 - (row of piece 0)
    };
    __device__ __forceinline__ static void init(Src &s, const uint16_t *base, int64_t ld, int row0, int rows_valid,
                                                int k_begin)
    {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        s.base = base + (int64_t)row0 * ld + k_begin;
        const int pslot = wave * 64 + lane;
        const int row = pslot / CPR, pc = pslot % CPR;
        s.kc8 = (pc ^ sw(row)) * 8;
        s.off0 = (uint32_t)(row * ld + s.kc8);
        s.step = (uint32_t)(RSTRIDE * ld);
        s.rlim = rows_valid - row0 - row;
    }
    // Piece i of the k-slice [k0, k0 + BKK) into `tile` (a piece past k_valid or past
    // the last row comes from the zero page).
    template <bool ASM = false>
    __device__ __forceinline__ static void issue_one(const Src &s, int i, int k0, int k_valid, char *tile)
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const bool ok = RSTRIDE * i < s.rlim && k0 + s.kc8 < k_valid;
        const void *src = ok ? static_cast<const void *>(s.base + s.off0 + (uint32_t)i * s.step)
                             : static_cast<const void *>(kZeroPage);
        copy16_to_lds<ASM>(src, tile + (i * (NT / 64) + wave) * 1024);
    }
    // Move the source to the next k-slice.
    __device__ __forceinline__ static void advance(Src &s, int64_t) { s.base += BKK; }
    // 8 k-values (chunk kc) of tile row `row`, the MFMA operand of one lane.
    __device__ __forceinline__ static bf16x8 frag(const char *tile, int row, int kc)
    {
        return *reinterpret_cast<const bf16x8 *>(tile + (row * CPR + (kc ^ sw(row))) * 16);
    }
};

// Operand tile whose n dimension is contiguous in memory, B(n, k) = src[k * ld + n]:
// BKK rows of k, each COLS elements of n, copied as they lie (16-byte pieces of n).
// The MFMA wants 8 consecutive k per lane, so the fragment is read with two gfx950
// transposing reads (ds_read_b64_tr_b16): in a group of 16 lanes, lane l addresses
// the 4 elements of row k + l/4 at columns n + 4 (l % 4), and every lane receives the
// 4 rows k .. k+3 of column n + l.  Half a wave (two groups) reads 4 rows x 4
// consecutive 16-byte chunks; the chunk index is XOR-swizzled by 4 (row % 4) so those
// 16 chunks fall on 16 different bank groups.
template <int COLS, int BKK, int NT, bool SW16 = false>
struct KTileT {
    static constexpr int CPR = COLS / 8;         // 16-byte chunks per k-row
    static constexpr int RB = COLS * 2;          // bytes per k-row
    static constexpr int CHUNKS = BKK * CPR;
    static_assert(CHUNKS % NT == 0, "whole wave instructions");
    static_assert(CPR % 16 == 0, "rows of at least 16 chunks");
    static constexpr int PER = CHUNKS / NT;
    static constexpr int BYTES = CHUNKS * 16;
    static constexpr int RSTRIDE = NT / CPR;     // k-rows between a lane's pieces
    static_assert(RSTRIDE % 4 == 0, "swizzle invariant across pieces");
    // SW16 (the 16x16x32 reads, below): bit 4 of the row also flips bit 1 of the chunk,
    // which separates the two 8-row k blocks that one half-wave reads at once.  A
    // lane's pieces lie RSTRIDE = 16 rows apart, so their chunk alternates with i.
    static_assert(!SW16 || RSTRIDE == 16, "pieces alternate bit 4 of the row");
    __device__ __forceinline__ static int sw(int krow)
    {
        return SW16 ? (((krow & 3) << 2) ^ (((krow >> 4) & 1) << 1)) : ((krow & 3) << 2);
    }

    struct Src {
        const uint16_t *base;   // row k of the current slice, column n0
        uint32_t off0;          // element offset of piece 0 from base
        int32_t odd;            // SW16: element offset of odd pieces' chunk from piece 0's
        uint32_t step;          // element offset between pieces (RSTRIDE rows)
        int krow0;              // k-row of piece 0 within the slice
        bool nok, nok_odd;      // the lane's 8 columns start inside the operand
    };
    __device__ __forceinline__ static void init(Src &s, const uint16_t *base, int64_t ld, int n0, int n_valid,
                                                int k_begin)
    {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        s.base = base + (int64_t)k_begin * ld + n0;
        const int slot = wave * 64 + lane;
        s.krow0 = slot / CPR;
        const int gc = (slot % CPR) ^ sw(s.krow0);
        s.off0 = (uint32_t)(s.krow0 * ld + 8 * gc);
        s.step = (uint32_t)(RSTRIDE * ld);
        s.nok = n0 + 8 * gc < n_valid;
        const int gco = SW16 ? gc ^ 2 : gc;
        s.odd = 8 * (gco - gc);
        s.nok_odd = n0 + 8 * gco < n_valid;
    }
    template <bool ASM = false>
    __device__ __forceinline__ static void issue_one(const Src &s, int i, int k0, int k_valid, char *tile)
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const bool odd = SW16 && (i & 1);
        const bool ok = (odd ? s.nok_odd : s.nok) && k0 + s.krow0 + RSTRIDE * i < k_valid;
        const void *src = ok ? static_cast<const void *>(s.base + (s.off0 + (odd ? s.odd : 0)) + (uint32_t)i * s.step)
                             : static_cast<const void *>(kZeroPage);
        copy16_to_lds<ASM>(src, tile + (i * (NT / 64) + wave) * 1024);
    }
    __device__ __forceinline__ static void advance(Src &s, int64_t ld) { s.base += (int64_t)BKK * ld; }
    // The MFMA operand of one lane for the 32 columns starting at nb and the 16 k-rows
    // starting at 16 ks: column nb + lane % 32, rows 16 ks + 8 (lane / 32) + 0..7.
    __device__ __forceinline__ static bf16x8 frag(const char *tile, int nb, int ks, int lane)
    {
        const int gl = lane & 15, grp = lane >> 4;
        const int n = nb + 16 * (grp & 1) + 4 * (gl & 3);
        const int k = ks * 16 + 8 * (grp >> 1) + (gl >> 2);
        const char *a = tile + k * RB + (((n >> 3) ^ sw(k)) << 4) + (n & 7) * 2;
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a + 4 * RB));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
    // The 16x16x32 operand of one lane: column nb + lane % 16, the 8 k-rows of block kb8
    // (rows 8 kb8 .. 8 kb8 + 7).  Each 16-lane row reads its own block; with SW16 the two
    // blocks a half-wave reads (16 rows apart) fall on different bank groups.
    __device__ __forceinline__ static bf16x8 frag16(const char *tile, int nb, int kb8, int lane)
    {
        const int gl = lane & 15;
        const int n = nb + 4 * (gl & 3);
        const int k = 8 * kb8 + (gl >> 2);
        const char *a = tile + k * RB + (((n >> 3) ^ sw(k)) << 4) + (n & 7) * 2;
        const char *b = tile + (k + 4) * RB + (((n >> 3) ^ sw(k + 4)) << 4) + (n & 7) * 2;
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(b));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
};

// C[m, n] = sum_k A(m, k) * B(n, k) for one BM x BN tile, operands streamed
// global -> LDS by the DMA path with S stages in flight (no staging registers).
// Both operands k-major: A(m,k) = A[m*lda + k], B(n,k) = B[n*ldb + k].
struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

// Swaps the odd 16-lane rows of x with the even 16-lane rows of y (gfx950
// v_permlane16_swap_b32): lane l of x with l in [16,32) or [48,64) takes y from lane
// l - 16, and lane l of y with l in [0,16) or [32,48) takes x from lane l + 16.  Written
// as asm: the compiler merges distinct calls of its builtin for this instruction.
__device__ __forceinline__ void permlane16_swap(float &x, float &y)
{
    asm volatile("v_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}

template <int BM_, int BN_, int WM_, int WN_, int BKK, int S, bool SPREAD = false, bool BTR = false, bool MI16 = !BTR>
struct GemmD {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BKK;
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MB = WTM / 32, NB = WTN / 32;
    static_assert(MB * 32 == WTM && NB * 32 == WTN, "wave tile");
    using AT = KTile<BM, BKK, NT>;
    using BT = std::conditional_t<BTR, KTileT<BN, BKK, NT, MI16>, KTile<BN, BKK, NT>>;
    static constexpr int STAGE = AT::BYTES + BT::BYTES;
    static constexpr int LDS_BYTES = S * STAGE;
    static constexpr int L = AT::PER + BT::PER;     // DMA loads per thread per k-step
    static_assert(S >= 2 && (S - 2) * L < 64, "stages");

    __device__ __forceinline__ static int row_of(int wm, int mb, int r, int lane)
    {
        return wm * WTM + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    // SPREAD: the 32-column fragment blocks of the waves interleave (block nb of wave wn
    // is block nb * WN + wn) and wm varies fastest over the waves, whose SIMD is wave % 4.
    // A tile whose last columns are past the operand's end then leaves its live column
    // blocks spread over all four SIMDs, and run<.., true> skips the dead blocks' MFMAs.
    __device__ __forceinline__ static int col_of(int wn, int nb, int lane)
    {
        return SPREAD ? (nb * WN + wn) * 32 + (lane & 31) : wn * WTN + nb * 32 + (lane & 31);
    }
    __device__ __forceinline__ static int wm_of(int wave) { return SPREAD ? wave % WM : wave / WN; }
    __device__ __forceinline__ static int wn_of(int wave) { return SPREAD ? wave / WM : wave % WN; }

    struct Frags {
        bf16x8 a[MB], b[NB];
    };

    // ilive / jlive: bit i (j) set when fragment row block i (column block j) of the wave
    // holds live rows (columns); only looked at when TAIL.
    template <bool TAIL = false>
    __device__ __forceinline__ static void load_frags(const char *stage, int ks, int wm, int wn, int lane, Frags &f,
                                                      uint32_t ilive = ~0u, uint32_t jlive = ~0u)
    {
#pragma unroll
        for (int i = 0; i < MB; ++i)
            if (!TAIL || ((ilive >> i) & 1u))
                f.a[i] = AT::frag(stage, wm * WTM + i * 32 + (lane & 31), ks * 2 + (lane >> 5));
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (!TAIL || ((jlive >> j) & 1u)) {
                if constexpr (BTR)
                    f.b[j] = BT::frag(stage + AT::BYTES, col_of(wn, j, 0), ks, lane);
                else
                    f.b[j] = BT::frag(stage + AT::BYTES, col_of(wn, j, lane), ks * 2 + (lane >> 5));
            }
    }

    template <bool TAIL = false>
    __device__ __forceinline__ static void mma(const Frags &f, f32x16 (&acc)[MB][NB], uint32_t ilive = ~0u,
                                               uint32_t jlive = ~0u)
    {
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (!TAIL || ((jlive >> j) & 1u)) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    if (!TAIL || ((ilive >> i) & 1u))
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
            }
    }

    // DS-read instructions per fragment set (one ds_read_b128 per fragment).
    static constexpr int DS_PER_SUB = MB + NB;
    static constexpr int SUB = BKK / 16;
    // The L loads of one k-step are spread over the first ISSUE_SUBS substeps of the
    // step before, P per substep.
    static constexpr int ISSUE_SUBS = (S == 2 && SUB > 2) ? SUB / 2 : SUB;
    static constexpr int P = (L + ISSUE_SUBS - 1) / ISSUE_SUBS;

    // Scheduling hint for one substep: MFMAs interleaved one-for-one with the LDS reads
    // of the next substep's fragments and with this substep's global->LDS loads.
    template <int NDS, int NVM>
    __device__ __forceinline__ static void interleave()
    {
#pragma unroll
        for (int i = 0; i < MB * NB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
            if (i < NDS)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            if (i < NVM)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read (to LDS)
        }
        if constexpr (NDS > MB * NB)
            __builtin_amdgcn_sched_group_barrier(0x100, NDS - MB * NB, 0);
        if constexpr (NVM > MB * NB)
            __builtin_amdgcn_sched_group_barrier(0x020, NVM - MB * NB, 0);
    }

    // S LDS stages.  While k-step kb is computed, the loads of step kb + S - 1 are issued
    // (a few per substep, interleaved with the MFMAs) into the stage step kb - 1 used.
    // Fragments are read one 16-deep substep ahead of the MFMAs that use them.  Before
    // the last substep's MFMAs the wave waits for step kb + 1 (steps kb+2 .. kb+S-1 may
    // stay in flight) and the barrier retires stage kb (its last fragments are already
    // in registers); those MFMAs then run while the first fragments of step kb + 1 are
    // read, so no wave starts a step waiting on LDS.  Steps past the end load zeros,
    // which keeps the wait counts uniform.  `hook` runs once, right after the first
    // stage has landed: loads it issues are older than every k-step load, so the first
    // step's wait covers them.
    // TAIL: the tile's rows or columns end inside it (m_valid < m0 + BM or n_valid <
    // n0 + BN); fragment blocks wholly past them are neither read nor multiplied (their
    // accumulators stay 0).
    template <class Hook = NoHook, bool TAIL = false>
    __device__ static void run(char *smem, const uint16_t *A, int64_t lda, int m0, int m_valid, int ka_valid,
                               const uint16_t *B, int64_t ldb, int n0, int n_valid, int kb_valid, int k_begin,
                               int k_end, f32x16 (&acc)[MB][NB], const Hook &hook = Hook())
    {
        if constexpr (MI16)
            run16<Hook, TAIL>(smem, A, lda, m0, m_valid, ka_valid, B, ldb, n0, n_valid, kb_valid, k_begin, k_end, acc,
                              hook);
        else
            run32<Hook, TAIL>(smem, A, lda, m0, m_valid, ka_valid, B, ldb, n0, n_valid, kb_valid, k_begin, k_end, acc,
                              hook);
    }

    // ---- 16x16x32 form.  Under the board's power limit gfx950 sustains more bf16 flops
    // with v_mfma_f32_16x16x32_bf16 than with the 32x32x16 form (in register-only loops
    // over every compute unit, about 2.2 against 1.95 PFLOP/s: the clock settles higher).
    // Each 32 x 32 accumulator block is computed as four 16 x 16 blocks (R, C) and, after
    // the k loop, moved into the 32x32x16 output layout, which the epilogues index:
    // lane l, element r holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
    //   A 16x16x32 product leaves lane l with rows 4 (l / 16) + 0..3 of column l % 16.
    //   Block (R, C) takes the block's columns 16 C .. 16 C + 15 and, for its row rho,
    //   block row phi_R(rho) = 16 R + 8 ((rho / 4) % 2) + 4 (rho / 8) + rho % 4.  Lane l
    //   (16-lane row g = l / 16) then holds its own column in block (R, g % 2) and the
    //   column of lane l ^ 16 in block (R, 1 - g % 2); one permlane16 swap per register
    //   pair trades those, after which both registers hold the lane's column, at block
    //   rows 16 R + 4 (g / 2) + r and 16 R + 8 + 4 (g / 2) + r: elements 8 R + r and
    //   8 R + 4 + r of the 32x32x16 layout.
    static_assert(!MI16 || BKK == 64, "64-deep k-steps: two 32-deep substeps");
    // The fragment rows of the first BAR row blocks of a step's last substep run before
    // the step's barrier, the others after it, covering the reads of the next step's
    // first fragments.
    static constexpr int BAR = MB / 2;
    // The copies of step kb + S are issued right after step kb's barrier (the stage they
    // fill was last read before it), spread over the COPY_ROWS fragment rows that follow
    // it, so that they have a whole step to land.
    static constexpr int COPY_ROWS = 2 * (MB - BAR);
    static constexpr int CPRW = (L + COPY_ROWS - 1) / COPY_ROWS;   // copies per such row
    __device__ __forceinline__ static int phi(int R, int rho)
    {
        return 16 * R + 8 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
    }
    // The 16-byte k-chunk (of the step's 8) that 16-lane row g = lane / 16 of a fragment
    // holds in 32-deep substep ks; A and B use the same map, so each MFMA still pairs
    // equal k.  The LDS serves a 16-byte read in passes that take lanes l and l + 32
    // together: substep ks takes chunks ks, ks + 2 (rows 0, 1) and their XOR with 5 (rows
    // 2, 3), which puts the two lanes of a pass in different bank groups both for A's row
    // order phi and for B's consecutive rows under the tile's swizzle.
    __device__ __forceinline__ static int kchunk16(int ks, int lane)
    {
        const int g = lane >> 4;
        return (2 * (g & 1) + ks) ^ (5 * (g >> 1));
    }
    __device__ __forceinline__ static bf16x8 frag_a16(const char *stage, int wm, int i, int R, int ks, int lane)
    {
        return AT::frag(stage, wm * WTM + 32 * i + phi(R, lane & 15), kchunk16(ks, lane));
    }
    __device__ __forceinline__ static bf16x8 frag_b16(const char *stage, int wn, int j, int C, int ks, int lane)
    {
        if constexpr (BTR)
            return BT::frag16(stage + AT::BYTES, col_of(wn, j, 0) + 16 * C, kchunk16(ks, lane), lane);
        else
            return BT::frag(stage + AT::BYTES, col_of(wn, j, 0) + 16 * C + (lane & 15), kchunk16(ks, lane));
    }

    template <class Hook = NoHook, bool TAIL = false>
    __device__ static void run16(char *smem, const uint16_t *A, int64_t lda, int m0, int m_valid, int ka_valid,
                                 const uint16_t *B, int64_t ldb, int n0, int n_valid, int kb_valid, int k_begin,
                                 int k_end, f32x16 (&acc)[MB][NB], const Hook &hook)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wm_of(wave), wn = wn_of(wave);
        uint32_t ilive = ~0u, jlive = ~0u;
        if constexpr (TAIL) {
            const int live_cols = n_valid - n0, live_rows = m_valid - m0;
            ilive = jlive = 0u;
#pragma unroll
            for (int i = 0; i < MB; ++i)
                if (wm * WTM + i * 32 < live_rows)
                    ilive |= 1u << i;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (col_of(wn, j, 0) < live_cols)
                    jlive |= 1u << j;
            ilive = __builtin_amdgcn_readfirstlane(ilive);
            jlive = __builtin_amdgcn_readfirstlane(jlive);
        }
        const auto ion = [&](int i) { return !TAIL || ((ilive >> i) & 1u); };
        const auto jon = [&](int j) { return !TAIL || ((jlive >> j) & 1u); };
        f32x4 q[MB][NB][2][2];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int R = 0; R < 2; ++R)
#pragma unroll
                    for (int C = 0; C < 2; ++C)
                        q[i][j][R][C] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const int nk = (k_end - k_begin + BKK - 1) / BKK;
        if (nk > 0) {
            typename AT::Src sa;
            typename BT::Src sb;
            AT::init(sa, A, lda, m0, m_valid, k_begin);
            BT::init(sb, B, ldb, n0, n_valid, k_begin);
            auto issue = [&](int step) {
                char *st = smem + (step % S) * STAGE;
                const int k0 = k_begin + step * BKK;
#pragma unroll
                for (int x = 0; x < AT::PER; ++x)
                    AT::template issue_one<true>(sa, x, k0, ka_valid, st);
#pragma unroll
                for (int x = 0; x < BT::PER; ++x)
                    BT::template issue_one<true>(sb, x, k0, kb_valid, st + AT::BYTES);
                AT::advance(sa, lda);
                BT::advance(sb, ldb);
            };
#pragma unroll
            for (int st = 0; st + 1 < S; ++st)
                issue(st);
            wait_vmcnt<(S - 2) * L>();
            __builtin_amdgcn_s_barrier();
            hook();
            // stage S - 1 has never been read
            issue(S - 1);
            bf16x8 fa[MB][2], fb[NB][2], fbn[NB][2];
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int R = 0; R < 2; ++R)
                    if (ion(i))
                        fa[i][R] = frag_a16(smem, wm, i, R, 0, lane);
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int C = 0; C < 2; ++C)
                    if (jon(j))
                        fb[j][C] = frag_b16(smem, wn, j, C, 0, lane);
            // The MFMAs of fragment row (i, R): one per column block (j, C).
            auto mma_row = [&](int i, int R) {
                if (ion(i)) {
#pragma unroll
                    for (int j = 0; j < NB; ++j)
#pragma unroll
                        for (int C = 0; C < 2; ++C)
                            if (jon(j))
                                q[i][j][R][C] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i][R], fb[j][C],
                                                                                        q[i][j][R][C], 0, 0, 0);
                }
            };
            auto load_b = [&](const char *stage, int ks) {
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int C = 0; C < 2; ++C)
                        if (jon(j))
                            fbn[j][C] = frag_b16(stage, wn, j, C, ks, lane);
            };
            auto load_a_row = [&](const char *stage, int ks, int i, int R) {
                if (ion(i))
                    fa[i][R] = frag_a16(stage, wm, i, R, ks, lane);
            };
            auto take_b = [&]() {
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int C = 0; C < 2; ++C)
                        fb[j][C] = fbn[j][C];
            };
            constexpr int ROWMMA = NB * 2;     // MFMAs per fragment row
            // One fragment row: its MFMAs, then (optionally) one global->LDS copy and the
            // read that refills the row's A fragment for the next substep.  The fence
            // after it keeps the rows in this order: a refill then has the other 2 MB - 1
            // rows of MFMAs to land before its next use.
            auto row_group = [&](auto has_vm, auto has_ds) {
                if constexpr (!TAIL) {
                    __builtin_amdgcn_sched_group_barrier(0x008, ROWMMA, 0);
                    if constexpr (decltype(has_vm)::value)
                        __builtin_amdgcn_sched_group_barrier(0x020, CPRW, 0);
                    if constexpr (decltype(has_ds)::value)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            // One 64-deep step: substep 0 runs every fragment row and refills its A fragment
            // (and all B fragments) for substep 1 from the same stage; substep 1 runs its
            // first BAR row blocks, crosses the step's barrier, then runs the others while
            // the next step's first fragments are read and the copies of step kb + S go out.
            auto step = [&](int kb, auto last_c) {
                constexpr bool last = decltype(last_c)::value;
                const char *cur = smem + (kb % S) * STAGE;
                char *cdst = smem + ((kb + S) % S) * STAGE;       // the stage step kb + S fills
                const int k0c = k_begin + (kb + S) * BKK;
                // the copies that go with fragment row `row` after the barrier (A pieces
                // first, then B pieces)
                auto copies = [&](auto rowc) {
                    constexpr int row = decltype(rowc)::value;
                    static_for<CPRW>([&](auto cc) {
                        constexpr int x = row * CPRW + decltype(cc)::value;
                        if constexpr (x < L) {
                            if constexpr (x < AT::PER)
                                AT::template issue_one<true>(sa, x, k0c, ka_valid, cdst);
                            else
                                BT::template issue_one<true>(sb, x - AT::PER, k0c, kb_valid, cdst + AT::BYTES);
                        }
                    });
                    if constexpr (row + 1 == COPY_ROWS) {
                        AT::advance(sa, lda);
                        BT::advance(sb, ldb);
                    }
                };
                // substep 0
                load_b(cur, 1);
                __builtin_amdgcn_sched_barrier(0);
                static_for<2 * MB>([&](auto rc) {
                    constexpr int row = decltype(rc)::value;
                    mma_row(row / 2, row % 2);
                    load_a_row(cur, 1, row / 2, row % 2);
                    row_group(std::false_type{}, std::true_type{});
                });
                take_b();
                // substep 1
                if constexpr (!last) {
                    static_for<2 * BAR>([&](auto rc) {
                        constexpr int row = decltype(rc)::value;
                        mma_row(row / 2, row % 2);
                        row_group(std::false_type{}, std::false_type{});
                    });
                    // step kb + 1 has landed for this wave (later steps may stay in
                    // flight), and every read of stage kb is done; after the barrier that
                    // holds for all waves
                    wait_vmcnt<(S - 2) * L>();
                    wait_lgkmcnt0();
                    __builtin_amdgcn_s_barrier();
                    const char *nst = smem + ((kb + 1) % S) * STAGE;
                    load_b(nst, 0);
#pragma unroll
                    for (int i = 0; i < BAR; ++i)
#pragma unroll
                        for (int R = 0; R < 2; ++R)
                            load_a_row(nst, 0, i, R);
                    __builtin_amdgcn_sched_barrier(0);
                    static_for<COPY_ROWS>([&](auto rc) {
                        constexpr int row = 2 * BAR + decltype(rc)::value;
                        mma_row(row / 2, row % 2);
                        copies(rc);
                        load_a_row(nst, 0, row / 2, row % 2);
                        row_group(std::true_type{}, std::true_type{});
                    });
                    take_b();
                } else {
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int R = 0; R < 2; ++R)
                            mma_row(i, R);
                }
            };
            for (int kb = 0; kb + 1 < nk; ++kb)
                step(kb, std::false_type{});
            step(nk - 1, std::true_type{});
        } else {
            hook();
        }
        // every wave is done reading LDS (and no load is in flight) before the caller reuses it
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // Into the 32x32x16 layout.  The fence keeps every MFMA above it, and the waits
        // give the last MFMA results time to land before the swaps read them.
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int R = 0; R < 2; ++R)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = q[i][j][R][0][r], y = q[i][j][R][1][r];
                        permlane16_swap(x, y);
                        acc[i][j][8 * R + r] = x;
                        acc[i][j][8 * R + 4 + r] = y;
                    }
    }

    // ---- 32x32x16 form (the logit products and the transposed-B product)
    // Issue priority falls over a step's substeps (3 in the first, 0 in the last): of the
    // two waves that share a SIMD, the one further behind in the step wins the issue
    // slots, so that both reach the step's barrier about together (-0.5% per step against
    // none; rising or two-level orders were slower).
    template <int SS>
    __device__ __forceinline__ static void wave_priority()
    {
        __builtin_amdgcn_s_setprio(SS < 3 ? 3 - SS : 0);
    }
    template <class Hook = NoHook, bool TAIL = false>
    __device__ static void run32(char *smem, const uint16_t *A, int64_t lda, int m0, int m_valid, int ka_valid,
                                 const uint16_t *B, int64_t ldb, int n0, int n_valid, int kb_valid, int k_begin,
                                 int k_end, f32x16 (&acc)[MB][NB], const Hook &hook)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wm_of(wave), wn = wn_of(wave);
        uint32_t ilive = ~0u, jlive = ~0u;
        if constexpr (TAIL) {
            const int live_cols = n_valid - n0, live_rows = m_valid - m0;
            ilive = jlive = 0u;
#pragma unroll
            for (int i = 0; i < MB; ++i)
                if (wm * WTM + i * 32 < live_rows)
                    ilive |= 1u << i;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (col_of(wn, j, 0) < live_cols)
                    jlive |= 1u << j;
            ilive = __builtin_amdgcn_readfirstlane(ilive);
            jlive = __builtin_amdgcn_readfirstlane(jlive);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;
        const int nk = (k_end - k_begin + BKK - 1) / BKK;
        if (nk <= 0) {
            hook();
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            return;
        }
        typename AT::Src sa;
        typename BT::Src sb;
        AT::init(sa, A, lda, m0, m_valid, k_begin);
        BT::init(sb, B, ldb, n0, n_valid, k_begin);
        // Loads [first, last) of k-step `step` (0..L-1: A pieces, then B pieces).  The
        // k-steps are issued in order; the sources advance after a step's last load.
        auto issue = [&](int step, auto first_c, auto last_c) {
            constexpr int first = decltype(first_c)::value, last = decltype(last_c)::value;
            char *st = smem + (step % S) * STAGE;
            const int k0 = k_begin + step * BKK;
#pragma unroll
            for (int x = first; x < last; ++x) {
                if (x < AT::PER)
                    AT::issue_one(sa, x, k0, ka_valid, st);
                else
                    BT::issue_one(sb, x - AT::PER, k0, kb_valid, st + AT::BYTES);
            }
            if constexpr (last == L) {
                AT::advance(sa, lda);
                BT::advance(sb, ldb);
            }
        };
#pragma unroll
        for (int st = 0; st + 1 < S; ++st)
            issue(st, std::integral_constant<int, 0>{}, std::integral_constant<int, L>{});
        wait_vmcnt<(S - 2) * L>();
        __builtin_amdgcn_s_barrier();
        hook();
        Frags f, fn;
        load_frags<TAIL>(smem, 0, wm, wn, lane, f, ilive, jlive);
        auto step = [&](int kb, auto last_c) {
            constexpr bool last = decltype(last_c)::value;
            const char *cur = smem + (kb % S) * STAGE;
            const int next = kb + S - 1;
            static_for<SUB>([&](auto ssc) {
                constexpr int ss = decltype(ssc)::value;
                wave_priority<ss>();
                constexpr int lo = ss * P < L ? ss * P : L;
                constexpr int hi = (ss + 1) * P < L ? (ss + 1) * P : L;
                if constexpr (lo < hi)
                    issue(next, std::integral_constant<int, lo>{}, std::integral_constant<int, hi>{});
                if constexpr (ss + 1 < SUB) {
                    load_frags<TAIL>(cur, ss + 1, wm, wn, lane, fn, ilive, jlive);
                    mma<TAIL>(f, acc, ilive, jlive);
                    if constexpr (!TAIL)
                        interleave<DS_PER_SUB, hi - lo>();
                    f = fn;
                } else if constexpr (!last) {
                    wait_vmcnt<(S - 2) * L>();
                    wait_lgkmcnt0();
                    __builtin_amdgcn_s_barrier();
                    load_frags<TAIL>(smem + ((kb + 1) % S) * STAGE, 0, wm, wn, lane, fn, ilive, jlive);
                    mma<TAIL>(f, acc, ilive, jlive);
                    if constexpr (!TAIL)
                        interleave<DS_PER_SUB, 0>();
                    f = fn;
                } else {
                    mma<TAIL>(f, acc, ilive, jlive);
                }
            });
        };
        if constexpr (!BTR) {
            for (int kb = 0; kb + 1 < nk; ++kb)
                step(kb, std::false_type{});
            step(nk - 1, std::true_type{});
        } else {
            // Transposing reads of B.  They may not overlap a global -> LDS copy in flight
            // (the compiler waits for every copy before such a read), so all B fragments
            // of a k-step are read right after its barrier, when no copy is in flight, and
            // the next step's copies are issued after them.
            bf16x8 bq[SUB][NB];
            auto load_b = [&](const char *stage) {
                static_for<SUB>([&](auto kc) {
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        if (!TAIL || ((jlive >> j) & 1u))
                            bq[decltype(kc)::value][j] = BT::frag(stage + AT::BYTES, col_of(wn, j, 0), decltype(kc)::value, lane);
                });
            };
            auto load_a = [&](const char *stage, int ks, Frags &g) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    if (!TAIL || ((ilive >> i) & 1u))
                        g.a[i] = AT::frag(stage, wm * WTM + i * 32 + (lane & 31), ks * 2 + (lane >> 5));
            };
            load_b(smem);
            auto stepT = [&](int kb, auto last_c) {
                constexpr bool last = decltype(last_c)::value;
                const char *cur = smem + (kb % S) * STAGE;
                const int next = kb + S - 1;
                static_for<SUB>([&](auto ssc) {
                    constexpr int ss = decltype(ssc)::value;
                    wave_priority<ss>();
                    constexpr int lo = ss * P < L ? ss * P : L;
                    constexpr int hi = (ss + 1) * P < L ? (ss + 1) * P : L;
                    if constexpr (lo < hi)
                        issue(next, std::integral_constant<int, lo>{}, std::integral_constant<int, hi>{});
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        f.b[j] = bq[ss][j];
                    if constexpr (ss + 1 < SUB) {
                        load_a(cur, ss + 1, fn);
                        mma<TAIL>(f, acc, ilive, jlive);
                        if constexpr (!TAIL)
                            interleave<MB, hi - lo>();
#pragma unroll
                        for (int i = 0; i < MB; ++i)
                            f.a[i] = fn.a[i];
                    } else if constexpr (!last) {
                        wait_vmcnt<(S - 2) * L>();
                        wait_lgkmcnt0();
                        __builtin_amdgcn_s_barrier();
                        const char *nst = smem + ((kb + 1) % S) * STAGE;
                        load_b(nst);
                        load_a(nst, 0, fn);
                        mma<TAIL>(f, acc, ilive, jlive);
#pragma unroll
                        for (int i = 0; i < MB; ++i)
                            f.a[i] = fn.a[i];
                    } else {
                        mma<TAIL>(f, acc, ilive, jlive);
                    }
                });
            };
            for (int kb = 0; kb + 1 < nk; ++kb)
                stepT(kb, std::false_type{});
            stepT(nk - 1, std::true_type{});
        }
        __builtin_amdgcn_s_setprio(0);
        // every wave is done reading LDS (and no load is in flight) before the caller reuses it
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
};

// The logit GEMM: rows = vocabulary (W), columns = tokens (h), k = hidden.
using LogitGemm = GemmD<256, 256, 2, 4, 64, 2, false, false, false>;
static_assert(LogitGemm::BM == kVocabTile, "entry counts are kept per 256-row vocabulary tile");
static_assert(kTokenTile % LogitGemm::BN == 0, "chunk padding covers whole token tiles");
constexpr int kGStagePitch = 256 * 2 + 16;   // bytes per token row of the staged bf16 g tile
static_assert(LogitGemm::BM <= 256 && LogitGemm::BN <= 256, "staging tile");
constexpr int kLogitLds = (LogitGemm::LDS_BYTES > 256 * kGStagePitch) ? LogitGemm::LDS_BYTES : 256 * kGStagePitch;

// The first kPre cached entries of every token of a logit tile that fall into the tile's
// vocabulary rows (index and, for the backward, teacher probability) are copied into
// LDS, behind the GEMM operands, while the main loop runs.  The epilogues then find
// them without a global load that has to wait for the entry count first; a token with
// more entries in one tile (rare) reads the rest from global memory.
constexpr int kPre = LogitGemm::NT / LogitGemm::BN;
constexpr int kPreLds = 2 * LogitGemm::NT * 4;
static_assert(kPre * LogitGemm::BN == LogitGemm::NT, "one prefetched entry per thread");
static_assert(kLogitLds + kPreLds <= 160 * 1024, "LDS");

struct EntryPrefetch {
    const void *src_idx = nullptr, *src_p = nullptr;

    // Thread t takes entry (start + t / BN) of token n0 + t % BN.
    __device__ __forceinline__ void init(const uint8_t *cnt, int cnt_stride, int tm, int n0, int rows, int K,
                                         const int32_t *idx_s, const float *p_s)
    {
        const int nl = threadIdx.x % LogitGemm::BN, slot = threadIdx.x / LogitGemm::BN;
        const int tok = n0 + nl;
        if (tok < rows) {
            const uint8_t *c = cnt + (size_t)tok * cnt_stride + tm;
            const int e = c[0] + slot;
            if (e < c[1]) {
                src_idx = idx_s + (size_t)tok * K + e;
                if (p_s)
                    src_p = p_s + (size_t)tok * K + e;
            }
        }
    }
    // Copies into pre[0 .. NT) (indices) and pre[NT .. 2 NT) (probabilities).
    __device__ __forceinline__ void issue(char *pre) const
    {
        char *base = pre + (threadIdx.x & ~63) * 4;
        if (src_idx)
            copy4_to_lds(src_idx, base);
        if (src_p)
            copy4_to_lds(src_p, base + LogitGemm::NT * 4);
    }
};

// Select acc[mb][nb][r] for a run-time (mb*16 + r) without indexing registers.
template <int MB, int NB>
__device__ __forceinline__ float pick(const f32x16 (&acc)[MB][NB], int nb, int sel)
{
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (j == nb) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    v = (i * 16 + r == sel) ? acc[i][j][r] : v;
        }
    return v;
}

template <int MB, int NB>
__device__ __forceinline__ void sub_at(f32x16 (&acc)[MB][NB], int nb, int sel, float d)
{
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (j == nb) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = (i * 16 + r == sel) ? acc[i][j][r] - d : acc[i][j][r];
        }
}

// ------------------------------------------------------------------ prepare

struct PrepParams {
    const int32_t *idx;     // [rows, K] chunk's cached indices
    const void *tl;         // [rows, K] chunk's cached logits
    int logit_f32;
    int rows, K, V, nVt, cnt_stride;
    float scale2;           // log2(e) / T
    int32_t *idx_s;         // [Cpad, K] out
    float *p_s;             // [Cpad, K] out
    float *zk;              // [Cpad, K] out: NaN until the forward epilogue fills it
    float *psum;            // [Cpad] out
    float *negent;          // [Cpad] out: sum_k p log p (natural log)
    uint8_t *cnt;           // [Cpad, cnt_stride] out
    uint32_t *err;          // index-check flag (validate only)
    int validate;
    // scaled != 0: p_s and psum are stored times the token's gradient scale
    // gcoef * (gw ? gw[t] * *ginv : 1) * (gmul ? *gmul : 1)
    int scaled;
    float gcoef;
    const float *gw;        // chunk's first token, or NULL
    const float *ginv;      // 1 / sum of all weights (device scalar)
    const float *gmul;      // device scalar multiplying gcoef, or NULL
};

// One wave per token.  Teacher distribution p = softmax(tl/T) over the K entries
// ("Preparing Offline Top-K Logits", getaibook.com: the cache holds the top-K logits
// and their indices); entries are sorted by vocabulary index (rank = number of entries
// with a smaller index, ties by position) so that each vocabulary tile owns one
// contiguous range of them, whose bounds cnt[] records.
__global__ __launch_bounds__(256) void prepare_kernel(PrepParams p)
{
    __shared__ int s_idx[4][kMaxK];
    __shared__ int s_sorted[4][kMaxK];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + w;
    const bool live = t < p.rows;
    const int K = p.K;
    float a[2], pr[2];
    int ix[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = lane + 64 * h;
        a[h] = kNegInf;
        ix[h] = 0x7fffffff;
        if (live && e < K) {
            const size_t o = (size_t)t * K + e;
            const float x = p.logit_f32 ? reinterpret_cast<const float *>(p.tl)[o]
                                        : bf16_to_f32(reinterpret_cast<const uint16_t *>(p.tl)[o]);
            a[h] = x * p.scale2;
            ix[h] = p.idx[o];
        }
        if (e < kMaxK)
            s_idx[w][e] = ix[h];
    }
    const float m = wave_max(fmaxf(a[0], a[1]));
    const float ms = (m == kNegInf) ? 0.0f : m;
    const float s = wave_sum(fast_exp2(a[0] - ms) + fast_exp2(a[1] - ms));
    const float lse2 = ms + log2f(s);
    float ps = 0.0f, ne = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bool in = lane + 64 * h < K;
        pr[h] = in ? fast_exp2(a[h] - lse2) : 0.0f;
        ps += pr[h];
        ne += in ? pr[h] * (a[h] - lse2) * kLn2 : 0.0f;
    }
    ps = wave_sum(ps);
    ne = wave_sum(ne);
    if (p.scaled && live) {
        const float gsc = (p.gw ? p.gcoef * p.gw[t] * *p.ginv : p.gcoef) * (p.gmul ? *p.gmul : 1.0f);
        // A token whose scale is 0 (a masked token) contributes nothing to the gradient,
        // whatever its cached logits hold: padding rows often carry -inf or NaN there,
        // and 0 times the NaN they give would reach every row of dW.
        pr[0] = gsc != 0.0f ? pr[0] * gsc : 0.0f;
        pr[1] = gsc != 0.0f ? pr[1] * gsc : 0.0f;
        ps = gsc != 0.0f ? ps * gsc : 0.0f;
    }
    __syncthreads();
    bool bad = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = lane + 64 * h;
        if (live && e < K) {
            const int v = ix[h];
            int rank = 0;
            for (int j = 0; j < K; ++j) {
                const int u = s_idx[w][j];
                rank += (u < v || (u == v && j < e)) ? 1 : 0;
                bad |= (u == v && j != e);
            }
            bad |= (v < 0 || v >= p.V);
            const size_t o = (size_t)t * K + rank;
            p.idx_s[o] = v;
            p.p_s[o] = pr[h];
            p.zk[o] = __builtin_nanf("");
            s_sorted[w][rank] = v;
        }
    }
    if (live && lane == 0) {
        p.psum[t] = ps;
        p.negent[t] = ne;
    }
    if (p.validate && bad)
        *p.err = 1u;
    __syncthreads();
    if (!live)
        return;
    // cnt[vt] = number of sorted entries below vt * 256 (lower bound in s_sorted).
    uint8_t *crow = p.cnt + (size_t)t * p.cnt_stride;
    for (int vt = lane; vt <= p.nVt; vt += 64) {
        const int key = vt * kVocabTile;
        int lo = 0, hi = K;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_sorted[w][mid] < key)
                lo = mid + 1;
            else
                hi = mid;
        }
        crow[vt] = (uint8_t)lo;
    }
}

// ------------------------------------------------------------------ forward logits

// From a bf16 tile staged in LDS as [token][vocab] (TOK token rows of 256 vocabulary
// columns, row pitch kGStagePitch bytes), writes the transposed tile to
// dst[(m0 + vocab) * pitch + n0 + token] with 16-byte stores, reading it back with
// transposing LDS reads: in a 16-lane group, lane l addresses the 8-byte piece of token
// row t + l/4 at vocabulary columns v + 4(l%4), and every lane receives 4 consecutive
// tokens of vocabulary column v + l.  Two such reads give a lane 8 tokens = one 16-byte
// piece of a transposed row.  A wave covers 16 vocabulary rows x 32 tokens per step
// (its 4 groups take 8 tokens each).
template <int TOK, int NWAVES>
__device__ __forceinline__ void store_vocab_major(const char *smem, uint16_t *dst, size_t pitch, int m0, int n0)
{
    static_assert(TOK % 32 == 0, "whole 32-token blocks");
    constexpr int kTokBlocks = TOK / 32;
    constexpr int kBlocks = (256 / 16) * kTokBlocks;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 4, gl = lane & 15;
    for (int b = wave; b < kBlocks; b += NWAVES) {
        const int vb = (b / kTokBlocks) * 16, tb = (b % kTokBlocks) * 32 + grp * 8;
        const char *src = smem + (tb + (gl >> 2)) * kGStagePitch + (vb + 4 * (gl & 3)) * 2;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(src));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(src + 4 * kGStagePitch));
        u32x4 v;
        v[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
        v[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
        v[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
        v[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
        *reinterpret_cast<u32x4 *>(dst + (size_t)(m0 + vb + gl) * pitch + n0 + tb) = v;
    }
}

// Rounds the tile held in `acc` to bf16, stages it in LDS as [token][vocab] (row pitch
// kGStagePitch) and writes its rows to dst[(n0 + token) * pitch + m0 + vocab] with
// 16-byte stores.  The staged tile stays in LDS for the caller; LDS must be free on
// entry (every wave past its last read of the previous contents).
template <class G>
__device__ __forceinline__ void stage_token_major(const f32x16 (&acc)[G::MB][G::NB], char *smem)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int nl = G::col_of(wn, j, lane);
#pragma unroll
        for (int i = 0; i < G::MB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ml = G::row_of(wm, i, 4 * q, lane);
                u32x2 pk;
                pk[0] = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
                pk[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                *reinterpret_cast<u32x2 *>(smem + nl * kGStagePitch + ml * 2) = pk;
            }
    }
    __syncthreads();
}

template <class G>
__device__ __forceinline__ void store_token_major(const f32x16 (&acc)[G::MB][G::NB], char *smem, uint16_t *dst,
                                                  size_t pitch, int m0, int n0)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int nl = G::col_of(wn, j, lane);
#pragma unroll
        for (int i = 0; i < G::MB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ml = G::row_of(wm, i, 4 * q, lane);
                u32x2 pk;
                pk[0] = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
                pk[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                *reinterpret_cast<u32x2 *>(smem + nl * kGStagePitch + ml * 2) = pk;
            }
    }
    __syncthreads();
    constexpr int kChunks = G::BN * (G::BM * 2 / 16);
    constexpr int kRowChunks = G::BM / 8;       // 16-byte pieces per token row of the tile
    // Non-temporal stores: every compute unit reaches this point at about the same time,
    // and the next tile's first load wait also waits for these stores (vmcnt counts
    // both).  Streaming them past the cache shortens that wait: -0.2 ms per backward
    // launch (8.44-8.48 against 8.64-8.72 ms at 8192 tokens, alternating runs on one
    // device); the same for the g^T stores was slower.
#pragma unroll 4
    for (int c = threadIdx.x; c < kChunks; c += G::NT) {
        const int nl = c / kRowChunks, col = (c % kRowChunks) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + nl * kGStagePitch + col * 2);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + (size_t)(n0 + nl) * pitch + m0 + col));
    }
}

struct FwdParams {
    const uint16_t *W;      // [V, H]
    const uint16_t *h;      // [rows, H] chunk
    int H, V, rows, Cpad, K, nVt, nNt, cnt_stride;
    float scale2;           // log2(e) / T
    const int32_t *idx_s;
    const uint8_t *cnt;
    float *zk;
    float2 *part;           // [nVt, Cpad]
    // single-call path only: kept exponentials and their half-tile maxima
    uint16_t *ex;           // [Cpad, Vpad] bf16
    float *mw;              // [2 nVt, Cpad]
    int Vpad;
};

// KEEP (single-call path): besides the forward outputs, the tile's 2^(z/T log2 e - m)
// are written in bf16 to p.ex, m being the maximum over the wave's 128 vocabulary rows
// (stored in p.mw), so that the backward needs no second product.
template <bool KEEP>
__device__ __forceinline__ void forward_tile(const FwdParams &p, char *smem, int t)
{
    using G = LogitGemm;
    int tm, tn;
    map_tile(t, p.nVt, p.nNt, 4, tm, tn);
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
    char *pre = smem + kLogitLds;
    EntryPrefetch pf;
    pf.init(p.cnt, p.cnt_stride, tm, n0, p.rows, p.K, p.idx_s, nullptr);

    // Entry range of this vocabulary tile for each of the lane's tokens.
    int cs[G::NB], ce[G::NB];
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int tok = n0 + G::col_of(wn, j, lane);
        cs[j] = ce[j] = 0;
        if (tok < p.rows) {
            const uint8_t *c = p.cnt + (size_t)tok * p.cnt_stride + tm;
            cs[j] = c[0];
            ce[j] = c[1];
        }
    }

    f32x16 acc[G::MB][G::NB];
    G::run(smem, p.W, p.H, m0, p.V, p.H, p.h, p.H, n0, p.rows, p.H, 0, p.H, acc, [&] { pf.issue(pre); });

    // Pick z at the cached indices this tile owns: the lane holding that row writes it.
    const int wrow0 = m0 + wm * G::WTM;
    const int32_t *pre_idx = reinterpret_cast<const int32_t *>(pre);
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int nl = G::col_of(wn, j, lane), tok = n0 + nl;
        for (int e = cs[j]; e < ce[j]; ++e) {
            const int v = (e - cs[j] < kPre) ? pre_idx[(e - cs[j]) * G::BN + nl] : p.idx_s[(size_t)tok * p.K + e];
            const int row = v - wrow0;
            if (row >= 0 && row < G::WTM && v < p.V) {
                const int r32 = row & 31;
                if (((r32 >> 2) & 1) == (lane >> 5)) {
                    const int sel = (row >> 5) * 16 + ((r32 >> 3) << 2) + (r32 & 3);
                    p.zk[(size_t)tok * p.K + e] = pick(acc, j, sel);
                }
            }
        }
    }

    // Per token, over the wave's 128 vocabulary rows: max and sum of 2^(z*log2e/T - max).
    // Without KEEP every tile but the last vocabulary tile skips the row check.  With
    // KEEP the accumulators are rewritten, and one code path with a per-lane row limit
    // (as in the backward epilogue) avoids holding two versions of them.
    float *red = reinterpret_cast<float *>(smem);   // [WM][BN][2]
    const int lim = p.V - m0 - G::row_of(wm, 0, 0, lane);
    auto reduce = [&](auto interior_c) {
        constexpr bool interior = decltype(interior_c)::value;
#pragma unroll
        for (int j = 0; j < G::NB; ++j) {
            // the scale log2(e)/T is positive, so scaling the largest value gives the
            // largest scaled value, bit for bit
            float mx = kNegInf;
#pragma unroll
            for (int i = 0; i < G::MB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool in = interior || 32 * i + 8 * (r >> 2) + (r & 3) < lim;
                    mx = fmaxf(mx, in ? acc[i][j][r] : kNegInf);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * p.scale2;
            const float ms = (mx == kNegInf) ? 0.0f : mx;
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < G::MB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool in = interior || 32 * i + 8 * (r >> 2) + (r & 3) < lim;
                    const float e = in ? fast_exp2(acc[i][j][r] * p.scale2 - ms) : 0.0f;
                    sum += e;
                    if constexpr (KEEP)
                        acc[i][j][r] = e;
                }
            sum += __shfl_xor(sum, 32);
            if (lane < 32) {
                const int nl = G::col_of(wn, j, lane);
                red[(wm * G::BN + nl) * 2 + 0] = mx;
                red[(wm * G::BN + nl) * 2 + 1] = sum;
                if constexpr (KEEP)
                    p.mw[(size_t)(2 * tm + wm) * p.Cpad + n0 + nl] = ms;
            }
        }
    };
    if (!KEEP && m0 + G::BM <= p.V)
        reduce(std::true_type{});
    else
        reduce(std::false_type{});
    __syncthreads();
    for (int nl = threadIdx.x; nl < G::BN; nl += G::NT) {
        if (n0 + nl < p.rows) {
            float m = red[nl * 2 + 0], s = red[nl * 2 + 1];
#pragma unroll
            for (int w2 = 1; w2 < G::WM; ++w2)
                lse_merge(m, s, red[(w2 * G::BN + nl) * 2 + 0], red[(w2 * G::BN + nl) * 2 + 1]);
            p.part[(size_t)tm * p.Cpad + n0 + nl] = make_float2(m, s);
        }
    }
    if constexpr (KEEP) {
        __syncthreads();    // the merge above has read `red` before the staging overwrites it
        store_token_major<G>(acc, smem, p.ex, (size_t)p.Vpad, m0, n0);
    }
}

// Persistent: one work-group per compute unit walks the tiles b, b + grid, ...  The
// grid is a multiple of 8, so all tiles of a work-group map to its own XCD, and the
// XCD's work-groups move through its tile range together, as one wave of
// non-persistent work-groups would.
template <bool KEEP>
__global__ __launch_bounds__(LogitGemm::NT) void forward_logits_kernel(FwdParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[kLogitLds + kPreLds];
    for (int t = blockIdx.x; t < p.nVt * p.nNt; t += gridDim.x) {
        forward_tile<KEEP>(p, smem, t);
        __syncthreads();    // every wave is done with LDS before the next tile's loads land
    }
}

// ------------------------------------------------------------------ combine

struct CombineParams {
    const float2 *part;
    const float *zk, *p_s, *psum, *negent;
    int rows, Cpad, nVt, K;
    float T;
    float *loss_tok;        // chunk's first token
    float *lse;             // chunk's first token
};

// 32 tokens x 8 slices of the vocabulary tiles per block.
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p)
{
    __shared__ float s_m[8][32], s_s[8][32], s_d[8][32];
    const int tl = threadIdx.x & 31, sp = threadIdx.x >> 5;
    const int t = blockIdx.x * 32 + tl;
    float m = kNegInf, s = 0.0f, d = 0.0f;
    if (t < p.rows) {
        for (int vt = sp; vt < p.nVt; vt += 8) {
            const float2 q = p.part[(size_t)vt * p.Cpad + t];
            lse_merge(m, s, q.x, q.y);
        }
        for (int e = sp; e < p.K; e += 8)
            d += p.p_s[(size_t)t * p.K + e] * p.zk[(size_t)t * p.K + e];
    }
    s_m[sp][tl] = m;
    s_s[sp][tl] = s;
    s_d[sp][tl] = d;
    __syncthreads();
    if (sp == 0 && t < p.rows) {
#pragma unroll
        for (int k = 1; k < 8; ++k) {
            lse_merge(m, s, s_m[k][tl], s_s[k][tl]);
            d += s_d[k][tl];
        }
        const float lse = (m + log2f(s)) * kLn2;    // log sum_v exp(z_v / T)
        // T^2 * sum_k p (log p - z_k/T + lse)
        const float loss = p.T * p.T * (p.negent[t] - d / p.T + p.psum[t] * lse);
        p.loss_tok[t] = loss;
        p.lse[t] = lse;
    }
}

// ------------------------------------------------------------------ mean

__global__ __launch_bounds__(1024) void mean_kernel(const float *x, int64_t n, float *out)
{
    __shared__ double s[1024];
    double a = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 1024)
        a += (double)x[i];
    s[threadIdx.x] = a;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o)
            s[threadIdx.x] += s[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        *out = (float)(s[0] / (double)n);
}

// Weighted mean sum_i w_i x_i / sum_i w_i (0 when the weights sum to 0), fixed order, fp64.
// Tokens of weight 0 are left out of the numerator, so a masked token whose loss is not
// finite (cached logits of -inf or NaN) does not reach the mean.
__global__ __launch_bounds__(1024) void weighted_mean_kernel(const float *x, const float *w, int64_t n, float *out)
{
    __shared__ double s[1024], sw[1024];
    double a = 0.0, b = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) {
        if (w[i] != 0.0f)
            a += (double)w[i] * (double)x[i];
        b += (double)w[i];
    }
    s[threadIdx.x] = a;
    sw[threadIdx.x] = b;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o) {
            s[threadIdx.x] += s[threadIdx.x + o];
            sw[threadIdx.x] += sw[threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0)
        *out = sw[0] > 0.0 ? (float)(s[0] / sw[0]) : 0.0f;
}

// out2[0] = sum of the weights, out2[1] = its inverse (0 when the sum is 0); fixed order, fp64.
__global__ __launch_bounds__(1024) void weight_sum_kernel(const float *w, int64_t n, float *out2)
{
    __shared__ double s[1024];
    double a = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 1024)
        a += (double)w[i];
    s[threadIdx.x] = a;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o)
            s[threadIdx.x] += s[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out2[0] = (float)s[0];
        out2[1] = s[0] > 0.0 ? (float)(1.0 / s[0]) : 0.0f;
    }
}

// ------------------------------------------------------------------ backward logits

struct BwdParams {
    const uint16_t *W, *h;
    int H, V, rows, Cpad, Vpad, K, nVt, nNt, cnt_stride;
    int vt0;                // first vocabulary tile of the slab; nVt tiles from there
    float scale2;           // log2(e) / T
    const float *lse;       // chunk's first token (natural log, z/T units)
    const int32_t *idx_s;
    const float *p_s, *psum;    // stored times each token's gradient scale
    const uint8_t *cnt;
    uint16_t *gT;           // [nVt * 256, Cpad] bf16: the slab's rows
};

__device__ __forceinline__ void backward_tile(const BwdParams &p, char *smem, int t)
{
    using G = LogitGemm;
    int tm, tn;
    map_tile(t, p.nVt, p.nNt, 4, tm, tn);
    tm += p.vt0;
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
    char *pre = smem + kLogitLds;
    EntryPrefetch pf;
    pf.init(p.cnt, p.cnt_stride, tm, n0, p.rows, p.K, p.idx_s, p.p_s);

    int cs[G::NB], ce[G::NB];
    float l2[G::NB], amp[G::NB];
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int tok = n0 + G::col_of(wn, j, lane);
        cs[j] = ce[j] = 0;
        l2[j] = 0.0f;
        amp[j] = 0.0f;
        if (tok < p.rows) {
            const uint8_t *c = p.cnt + (size_t)tok * p.cnt_stride + tm;
            cs[j] = c[0];
            ce[j] = c[1];
            l2[j] = p.lse[tok] * kLog2e;
            amp[j] = p.psum[tok];
        }
    }

    f32x16 acc[G::MB][G::NB];
    G::run(smem, p.W, p.H, m0, p.V, p.H, p.h, p.H, n0, p.rows, p.H, 0, p.H, acc, [&] { pf.issue(pre); });

    // g = c ((sum p) exp(z/T - lse) - scatter(p, idx)), with the token's gradient scale c
    // already folded into p and sum p; zero outside [0,V) x [0,rows).
    // The row test is against a per-lane limit: element (i, r) sits row_of(wm, i, r, lane)
    // = row_of(wm, 0, 0, lane) + 32 i + 8 (r / 4) + r % 4, so it is inside when that
    // constant offset is below V - m0 - row_of(wm, 0, 0, lane) (and -1 for a padded token).
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const bool tok_in = n0 + G::col_of(wn, j, lane) < p.rows;
        const int lim = tok_in ? p.V - m0 - G::row_of(wm, 0, 0, lane) : -1;
#pragma unroll
        for (int i = 0; i < G::MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool in = 32 * i + 8 * (r >> 2) + (r & 3) < lim;
                acc[i][j][r] = in ? amp[j] * fast_exp2(acc[i][j][r] * p.scale2 - l2[j]) : 0.0f;
            }
    }
    const int wrow0 = m0 + wm * G::WTM;
    const int32_t *pre_idx = reinterpret_cast<const int32_t *>(pre);
    const float *pre_p = reinterpret_cast<const float *>(pre + G::NT * 4);
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int nl = G::col_of(wn, j, lane), tok = n0 + nl;
        for (int e = cs[j]; e < ce[j]; ++e) {
            const bool in_lds = e - cs[j] < kPre;
            const int v = in_lds ? pre_idx[(e - cs[j]) * G::BN + nl] : p.idx_s[(size_t)tok * p.K + e];
            const int row = v - wrow0;
            if (row >= 0 && row < G::WTM && v < p.V) {
                const int r32 = row & 31;
                if (((r32 >> 2) & 1) == (lane >> 5)) {
                    const int sel = (row >> 5) * 16 + ((r32 >> 3) << 2) + (r32 & 3);
                    const float pe = in_lds ? pre_p[(e - cs[j]) * G::BN + nl] : p.p_s[(size_t)tok * p.K + e];
                    sub_at(acc, j, sel, pe);
                }
            }
        }
    }
    // The bf16 tile, [vocab][token], the operand of both the dH and the dW product.  (The
    // main loop ended with a barrier, so the operand buffers are free.)
    stage_token_major<G>(acc, smem);
    store_vocab_major<G::BN, G::NT / 64>(smem, p.gT, (size_t)p.Cpad, m0 - p.vt0 * G::BM, n0);
}

__global__ __launch_bounds__(LogitGemm::NT) void backward_logits_kernel(BwdParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[kLogitLds + kPreLds];
    for (int t = blockIdx.x; t < p.nVt * p.nNt; t += gridDim.x) {
        backward_tile(p, smem, t);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ single-call gradient

struct SoftGradParams {
    const uint16_t *ex;     // [Cpad, Vpad] bf16: the kept 2^(z/T log2 e - m)
    uint16_t *gT;           // [slab rows, Cpad] bf16 out
    int vt0;                // first vocabulary tile of the slab
    const float *mw;        // [2 nVt, Cpad] the half-tile maxima m (base 2)
    const float *lse;       // chunk's first token (natural log, z/T units)
    const float *psum;      // [Cpad] sum_k p
    const int32_t *idx_s;   // [Cpad, K] sorted cached indices
    const float *p_s;       // [Cpad, K] p in the same order
    const uint8_t *cnt;     // [Cpad, cnt_stride]
    int rows, Cpad, Vpad, K, cnt_stride;
    float coef;             // grad_scale * T (/ N without weights)
    const float *w;         // chunk's first token, or NULL
    const float *inv_wsum;  // device scalar, used with w
    const float *mul;       // device scalar multiplying coef, or NULL
};

constexpr int kSgTok = 128;       // tokens per block of the gradient kernel
constexpr int kSgThreads = 512;   // its threads: 32 per token row, kSgThreads / 32 rows at a time

// One block per (256-row vocabulary tile, kSgTok tokens).  With c the token's gradient scale:
//   g = c ((sum p) 2^(z/T log2 e - lse log2 e) - scatter(p, idx))
//     = c ((sum p) E 2^(m - lse log2 e) - scatter(p, idx)),   E the kept value,
// rounded to bf16, staged [token][vocab] in LDS and written as g^T.
__global__ __launch_bounds__(kSgThreads) void softmax_grad_kernel(SoftGradParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[kSgTok * kGStagePitch];
    constexpr int kStride = kSgThreads / 32;
    constexpr int kRows = kSgTok / kStride;     // token rows per thread
    const int tm = p.vt0 + blockIdx.x, n0 = blockIdx.y * kSgTok, m0 = tm * 256;
    const int c = threadIdx.x & 31;     // 16-byte piece of the tile row
    const int half = c >> 4;            // its 128-row half of the vocabulary tile
    const int r0 = threadIdx.x >> 5;
    // Every load first, so that they are in flight together.  Rows past the chunk read row 0.
    u32x4 e[kRows];
    float f[kRows], gsc[kRows];
    int ks[kRows], ke[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int tok = n0 + r0 + kStride * i;
        const int t = tok < p.rows ? tok : 0;
        e[i] = *reinterpret_cast<const u32x4 *>(p.ex + (size_t)t * p.Vpad + m0 + 8 * c);
        gsc[i] = (p.w ? p.coef * p.w[t] * *p.inv_wsum : p.coef) * (p.mul ? *p.mul : 1.0f);
        f[i] = p.psum[t] * fast_exp2(p.mw[(size_t)(2 * tm + half) * p.Cpad + t] - p.lse[t] * kLog2e);
        const uint8_t *cr = p.cnt + (size_t)t * p.cnt_stride + tm;
        ks[i] = cr[0];
        ke[i] = tok < p.rows ? cr[1] : cr[0];
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int rl = r0 + kStride * i, tok = n0 + rl;
        u32x4 out = {0u, 0u, 0u, 0u};
        if (tok < p.rows && gsc[i] != 0.0f) {    // a masked token (scale 0) gets g = 0
            const float fs = gsc[i] * f[i];
            float v[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[2 * q] = fs * __uint_as_float(e[i][q] << 16);
                v[2 * q + 1] = fs * __uint_as_float(e[i][q] & 0xffff0000u);
            }
            // the token's cached entries in this vocabulary tile that fall in this piece
            for (int k = ks[i]; k < ke[i]; ++k) {
                const int col = p.idx_s[(size_t)tok * p.K + k] - m0 - 8 * c;
                if (col >= 0 && col < 8) {
                    const float d = gsc[i] * p.p_s[(size_t)tok * p.K + k];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        v[q] -= (q == col) ? d : 0.0f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                out[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
        }
        *reinterpret_cast<u32x4 *>(smem + rl * kGStagePitch + 16 * c) = out;
    }
    __syncthreads();
    store_vocab_major<kSgTok, kSgThreads / 64>(smem, p.gT, (size_t)p.Cpad, m0 - p.vt0 * 256, n0);
}

// ------------------------------------------------------------------ full teacher distribution

// Online distillation against the teacher's whole distribution ("The Distillation
// Bottleneck", getaibook.com, the full-vocabulary teacher the cache replaces): with
// a = z log2(e) / T, p = 2^(a_t - L_t), q = 2^(a_s - L_s) (L the base-2 logsumexp),
//   loss = T^2 ln2 (sum_v p (a_t - a_s) - L_t + L_s),   g = c (q - p).
// Per chunk: the teacher product keeps a_t in fp32 and its partials, the student product
// forms sum p (a_t - a_s) per tile from those fp32 values while it keeps its own
// exponentials (bf16) as the single-call path does, and a streaming kernel forms g.
//
// a_t is kept in the product's register order, not as a matrix: for logit tile (tm, tn),
// wave, 32-column block j and lane, 16 float4 pieces, piece q holding rows
// row_of(wm, q / 4, 4 (q % 4) + 0..3, lane) of column col_of(wn, j, lane).  Each piece is
// one 1 KB access of the whole wave at an immediate offset from one base address, for
// the teacher's store and for both readers.
__device__ __forceinline__ size_t at_frag(int tm, int tn, int nNt, int wave, int j, int lane)
{
    return ((((size_t)tm * nNt + tn) * (LogitGemm::NT / 64) + wave) * LogitGemm::NB + j) * 4096 + 4 * lane;
}

struct FullTeacherParams {
    const uint16_t *W, *h;  // the teacher's head [V, Ht] and chunk of hidden states
    int H, V, rows, Cpad, nVt, nNt;
    float scale2;           // log2(e) / T
    float2 *part;           // [nVt, Cpad] (max, sum 2^(a - max)) of a_t per tile
    float *at;              // Vpad * Cpad floats, a_t in fragment order (at_frag)
};

__device__ __forceinline__ void full_teacher_tile(const FullTeacherParams &p, char *smem, int t)
{
    using G = LogitGemm;
    int tm, tn;
    map_tile(t, p.nVt, p.nNt, 4, tm, tn);
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
    f32x16 acc[G::MB][G::NB];
    G::run(smem, p.W, p.H, m0, p.V, p.H, p.h, p.H, n0, p.rows, p.H, 0, p.H, acc);
    const int lim = p.V - m0 - G::row_of(wm, 0, 0, lane);
    float *red = reinterpret_cast<float *>(smem);   // [WM][BN][2]
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int nl = G::col_of(wn, j, lane);
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < G::MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool in = 32 * i + 8 * (r >> 2) + (r & 3) < lim;
                mx = fmaxf(mx, in ? acc[i][j][r] * p.scale2 : -__builtin_inff());
            }
        // padded rows and columns hold a = 0 (the product zero-fills them); readers mask them
        float4 *dst = reinterpret_cast<float4 *>(p.at + at_frag(tm, tn, p.Cpad / G::BN, wave, j, lane));
#pragma unroll
        for (int q = 0; q < 16; ++q)
            dst[64 * q] = make_float4(acc[q >> 2][j][4 * (q & 3) + 0] * p.scale2, acc[q >> 2][j][4 * (q & 3) + 1] * p.scale2,
                                      acc[q >> 2][j][4 * (q & 3) + 2] * p.scale2, acc[q >> 2][j][4 * (q & 3) + 3] * p.scale2);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = (mx == -__builtin_inff()) ? 0.0f : mx;
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < G::MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sum += (32 * i + 8 * (r >> 2) + (r & 3) < lim) ? fast_exp2(acc[i][j][r] * p.scale2 - ms) : 0.0f;
        sum += __shfl_xor(sum, 32);
        if (lane < 32) {
            red[(wm * G::BN + nl) * 2 + 0] = mx;
            red[(wm * G::BN + nl) * 2 + 1] = sum;
        }
    }
    __syncthreads();
    for (int nl = threadIdx.x; nl < G::BN; nl += G::NT)
        if (n0 + nl < p.rows) {
            float m = red[nl * 2 + 0], s = red[nl * 2 + 1];
#pragma unroll
            for (int w2 = 1; w2 < G::WM; ++w2)
                lse_merge(m, s, red[(w2 * G::BN + nl) * 2 + 0], red[(w2 * G::BN + nl) * 2 + 1]);
            p.part[(size_t)tm * p.Cpad + n0 + nl] = make_float2(m, s);
        }
}

__global__ __launch_bounds__(LogitGemm::NT) void full_teacher_kernel(FullTeacherParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[LogitGemm::LDS_BYTES];
    for (int t = blockIdx.x; t < p.nVt * p.nNt; t += gridDim.x) {
        full_teacher_tile(p, smem, t);
        __syncthreads();
    }
}

struct FullStudentParams {
    const uint16_t *W, *h;  // the student's head [V, Hs] and chunk of hidden states
    int H, V, rows, Cpad, Vpad, nVt, nNt;
    float scale2;           // log2(e) / T
    const float *at;        // a_t in fragment order (at_frag)
    const float *lt2;       // [Cpad] L_t
    float2 *part;           // [nVt, Cpad] (max, sum 2^(a - max)) of a_s per tile
    float *px;              // [nVt, Cpad] sum over the tile of p (a_t - a_s)
    uint16_t *ex;           // [Cpad, Vpad] bf16 2^(a_s - m), m the wave's 128-row maximum
    float *mw;              // [2 nVt, Cpad] those maxima
};

__device__ __forceinline__ void full_student_tile(const FullStudentParams &p, char *smem, int t)
{
    using G = LogitGemm;
    int tm, tn;
    map_tile(t, p.nVt, p.nNt, 4, tm, tn);
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
    float lt[G::NB];
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int tok = n0 + G::col_of(wn, j, lane);
        lt[j] = tok < p.rows ? p.lt2[tok] : 0.0f;
    }
    f32x16 acc[G::MB][G::NB];
    G::run(smem, p.W, p.H, m0, p.V, p.H, p.h, p.H, n0, p.rows, p.H, 0, p.H, acc);
    const int lim = p.V - m0 - G::row_of(wm, 0, 0, lane);
    float *red = reinterpret_cast<float *>(smem);               // [WM][BN][2]
    float *redx = red + 2 * G::WM * G::BN;                       // [WM][BN]
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int nl = G::col_of(wn, j, lane), tok = n0 + nl;
        const bool tok_in = tok < p.rows;
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < G::MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, (32 * i + 8 * (r >> 2) + (r & 3) < lim) ? acc[i][j][r] * p.scale2 : -__builtin_inff());
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = (mx == -__builtin_inff()) ? 0.0f : mx;
        float sum = 0.0f, x = 0.0f;
        const float4 *src = reinterpret_cast<const float4 *>(p.at + at_frag(tm, tn, p.Cpad / G::BN, wave, j, lane));
#pragma unroll
        for (int i = 0; i < G::MB; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 t4 = src[64 * (4 * i + q)];
                const float at[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * q + c;
                    const bool in = 32 * i + 8 * q + c < lim;
                    const float as = acc[i][j][r] * p.scale2;
                    const float e = in ? fast_exp2(as - ms) : 0.0f;
                    sum += e;
                    if (in && tok_in)
                        x += fast_exp2(at[c] - lt[j]) * (at[c] - as);
                    acc[i][j][r] = e;
                }
            }
        }
        sum += __shfl_xor(sum, 32);
        x += __shfl_xor(x, 32);
        if (lane < 32) {
            red[(wm * G::BN + nl) * 2 + 0] = mx;
            red[(wm * G::BN + nl) * 2 + 1] = sum;
            redx[wm * G::BN + nl] = x;
            p.mw[(size_t)(2 * tm + wm) * p.Cpad + tok] = ms;
        }
    }
    __syncthreads();
    for (int nl = threadIdx.x; nl < G::BN; nl += G::NT)
        if (n0 + nl < p.rows) {
            float m = red[nl * 2 + 0], s = red[nl * 2 + 1], x = redx[nl];
#pragma unroll
            for (int w2 = 1; w2 < G::WM; ++w2) {
                lse_merge(m, s, red[(w2 * G::BN + nl) * 2 + 0], red[(w2 * G::BN + nl) * 2 + 1]);
                x += redx[w2 * G::BN + nl];
            }
            p.part[(size_t)tm * p.Cpad + n0 + nl] = make_float2(m, s);
            p.px[(size_t)tm * p.Cpad + n0 + nl] = x;
        }
    __syncthreads();    // the merge has read `red` before the staging overwrites it
    store_token_major<G>(acc, smem, p.ex, (size_t)p.Vpad, m0, n0);
}

__global__ __launch_bounds__(LogitGemm::NT) void full_student_kernel(FullStudentParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[kLogitLds];
    for (int t = blockIdx.x; t < p.nVt * p.nNt; t += gridDim.x) {
        full_student_tile(p, smem, t);
        __syncthreads();
    }
}

// 32 tokens x 8 slices of the vocabulary tiles per block: L = the base-2 logsumexp over
// the tiles.  With px (student pass) also the loss T^2 ln2 (sum px - L_t + L_s), the sum
// and the difference taken in fp64, and lse = L_s ln2.
__global__ __launch_bounds__(256) void full_combine_kernel(const float2 *part, const float *px, int nVt, int Cpad,
                                                           int rows, float T, const float *lt2, float *l2_out,
                                                           float *loss_tok, float *lse)
{
    __shared__ float s_m[8][32], s_s[8][32];
    __shared__ double s_x[8][32];
    const int tl = threadIdx.x & 31, sp = threadIdx.x >> 5;
    const int tok = blockIdx.x * 32 + tl;
    float m = kNegInf, s = 0.0f;
    double x = 0.0;
    if (tok < rows)
        for (int vt = sp; vt < nVt; vt += 8) {
            const float2 q = part[(size_t)vt * Cpad + tok];
            lse_merge(m, s, q.x, q.y);
            if (px)
                x += (double)px[(size_t)vt * Cpad + tok];
        }
    s_m[sp][tl] = m;
    s_s[sp][tl] = s;
    s_x[sp][tl] = x;
    __syncthreads();
    if (sp != 0 || tok >= rows)
        return;
#pragma unroll
    for (int k = 1; k < 8; ++k) {
        lse_merge(m, s, s_m[k][tl], s_s[k][tl]);
        x += s_x[k][tl];
    }
    const float L = m + log2f(s);
    if (l2_out)
        l2_out[tok] = L;
    if (px) {
        loss_tok[tok] = (float)((double)T * T * (double)kLn2 * (x - (double)lt2[tok] + (double)L));
        lse[tok] = L * kLn2;
    }
}

struct FullGradParams {
    const uint16_t *ex;     // [Cpad, Vpad] the student's kept exponentials
    uint16_t *gT;           // [slab rows, Cpad] out
    int vt0;                // first vocabulary tile of the slab
    const float *at;        // a_t in fragment order (at_frag)
    const float *mw;        // [2 nVt, Cpad]
    const float *ls2, *lt2; // [Cpad] L_s, L_t
    int rows, Cpad, Vpad, V;
    float coef;             // grad_scale * T (/ N without weights)
    const float *w;         // chunk's first token, or NULL
    const float *inv_wsum;
};

// One block per (256-row vocabulary tile, 64 tokens), four waves, each taking the
// fragments of one (128-row half, 32-token block) of a_t exactly as the logit product's
// wave held them, so that each lane has one token.  The student's kept values are staged
// [token][vocab] in LDS; each lane forms, for its 64 values,
//   g = c (E 2^(m - L_s) - 2^(a_t - L_t)),
// writes them back into the staged tile, whose columns are then written as g^T.
__global__ __launch_bounds__(256) void full_grad_kernel(FullGradParams p)
{
    using G = LogitGemm;
    constexpr int kTok = 64;
    __shared__ __attribute__((aligned(16))) char smem[kTok * kGStagePitch];
    const int tm = p.vt0 + blockIdx.x, n0 = blockIdx.y * kTok, m0 = tm * 256;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv >> 1, j = wv & 1;
    const int tn = n0 / G::BN, wn = (n0 % G::BN) / G::WTN;
    const int nl = 32 * j + (lane & 31), tok = n0 + nl;
    const bool tok_in = tok < p.rows;
    const float4 *src = reinterpret_cast<const float4 *>(p.at + at_frag(tm, tn, p.Cpad / G::BN, wm * G::WN + wn, j, lane));
    float4 a4[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        a4[q] = src[64 * q];
    const int ts = tok_in ? tok : 0;
    const float cc = tok_in ? (p.w ? p.coef * p.w[ts] * *p.inv_wsum : p.coef) : 0.0f;
    const float lt = p.lt2[ts];
    const float sq = p.mw[(size_t)(2 * tm + wm) * p.Cpad + ts] - p.ls2[ts];
    for (int c = threadIdx.x; c < kTok * 32; c += 256) {
        const int rl = c >> 5, pc = c & 31, t = n0 + rl;
        u32x4 e = {0u, 0u, 0u, 0u};
        if (t < p.rows)
            e = *reinterpret_cast<const u32x4 *>(p.ex + (size_t)t * p.Vpad + m0 + 8 * pc);
        *reinterpret_cast<u32x4 *>(smem + rl * kGStagePitch + 16 * pc) = e;
    }
    __syncthreads();
    const float fq = fast_exp2(sq);
    const int vlim = p.V - m0 - G::row_of(wm, 0, 0, lane);    // rows at or past it are padding
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int rb = 32 * (q >> 2) + 8 * (q & 3);          // row of the piece's first value - row_of(wm, 0, 0, lane)
        uint32_t *cell = reinterpret_cast<uint32_t *>(smem + nl * kGStagePitch + 2 * (G::row_of(wm, 0, 0, lane) + rb));
        const uint32_t e01 = cell[0], e23 = cell[1];
        const float e[4] = {__uint_as_float(e01 << 16), __uint_as_float(e01 & 0xffff0000u),
                            __uint_as_float(e23 << 16), __uint_as_float(e23 & 0xffff0000u)};
        const float a[4] = {a4[q].x, a4[q].y, a4[q].z, a4[q].w};
        float g[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            g[c] = (rb + c < vlim && cc != 0.0f) ? cc * (e[c] * fq - fast_exp2(a[c] - lt)) : 0.0f;
        cell[0] = pack_bf16x2(g[0], g[1]);
        cell[1] = pack_bf16x2(g[2], g[3]);
    }
    __syncthreads();
    store_vocab_major<kTok, 4>(smem, p.gT, (size_t)p.Cpad, m0 - p.vt0 * 256, n0);
}

// ------------------------------------------------------------------ teacher top-K

// The teacher's cache holds, per position, its top logits and their indices, extracted
// once ("Preparing Offline Top-K Logits", getaibook.com).  Exact top-K of z = h W^T per
// token in two passes of the logit GEMM:
//   1. maxima of z per token over disjoint row slices of the vocabulary;
//   2. tau = the K-th largest of those maxima is at most the K-th largest logit (the
//      maxima are K actual logits of distinct rows), so every logit >= tau is collected
//      as a candidate (tau comes from a per-token min-heap of K entries);
//   3. the candidates are sorted by (z descending, index ascending) and the first K kept.
// Any set of at least K disjoint slices gives a valid tau, so the first pass only needs
// part of the vocabulary: every 4th 256-row tile, with one maximum per 64-row slice,
// costs a quarter of the product and leaves a few times K candidates.  When a token of
// the chunk then has more than kTopkCap candidates (its large logits all outside that
// quarter), the chunk is redone with a first pass over every tile (one maximum per
// tile, or per 32-row slice when there are fewer tiles than K); the redo kernels are
// launched regardless and return at once unless the chunk's retry flag is set, so no
// host synchronisation is needed.  z is bitwise the same in every pass (same tiles,
// same accumulation order), so the logit that attains a maximum passes its own threshold.

struct TopkParams {
    const uint16_t *W;      // [V, H]
    const uint16_t *h;      // [rows, H] chunk
    int H, V, rows, Cpad, nVt, nNt;
    int stride;             // pass 1 visits vocabulary tiles 0, stride, 2 stride, ... (pass 2: 1)
    int nTm;                // vocabulary tiles visited: ceil(nVt / stride)
    int slices;             // maxima per visited tile: 1, 4 (64-row slices), 8 (32-row slices) or 16
                            // (16-row slices: the rows one lane holds of a 32-row block)
    const uint32_t *guard;  // NULL, or run only when *guard != 0
    float *tmax;            // [slices nTm, Cpad] maxima (pass 1)
    const float *thr;       // [Cpad] thresholds (pass 2)
    uint32_t *count;        // [Cpad] candidates per token (pass 2)
    uint64_t *cand;         // [Cpad, kTopkCap] candidate keys (pass 2)
};

// Unsigned key whose ascending order is z descending, then index ascending: the high
// word is the complement of an order-preserving image of z (-0 taken as +0), the low
// word the index.
__device__ __forceinline__ uint32_t topk_zkey(float z)
{
    uint32_t u = __float_as_uint(z + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~u;
}
__device__ __forceinline__ float topk_zkey_value(uint32_t key)
{
    uint32_t u = ~key;
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(u);
}

template <bool COLLECT>
__device__ __forceinline__ void topk_tile(const TopkParams &p, char *smem, int t)
{
    using G = LogitGemm;
    int ts, tn;
    map_tile(t, p.nTm, p.nNt, 4, ts, tn);
    const int tm = ts * p.stride;
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
    float thr[G::NB];
    if constexpr (COLLECT) {
#pragma unroll
        for (int j = 0; j < G::NB; ++j) {
            const int tok = n0 + G::col_of(wn, j, lane);
            thr[j] = tok < p.rows ? p.thr[tok] : __builtin_inff();
        }
    }
    f32x16 acc[G::MB][G::NB];
    G::run(smem, p.W, p.H, m0, p.V, p.H, p.h, p.H, n0, p.rows, p.H, 0, p.H, acc);
    // element (i, r) of the lane sits at row row_of(wm, 0, 0, lane) + 32 i + 8 (r/4) + r%4
    const int lim = p.V - m0 - G::row_of(wm, 0, 0, lane);
    float tile_mx[G::NB];
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int tok = n0 + G::col_of(wn, j, lane);
        tile_mx[j] = -__builtin_inff();
        float pair_mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < G::MB; ++i) {
            if constexpr (!COLLECT) {
                // 32-row block i of the wave: 16 rows in this lane, 16 in lane ^ 32
                float mx = -__builtin_inff();
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, (32 * i + 8 * (r >> 2) + (r & 3) < lim) ? acc[i][j][r] : -__builtin_inff());
                if (p.slices == 16 && tok < p.rows)
                    p.tmax[(size_t)(16 * ts + 2 * (G::WTM / 32) * wm + 2 * i + (lane >> 5)) * p.Cpad + tok] = mx;
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                tile_mx[j] = fmaxf(tile_mx[j], mx);
                pair_mx = fmaxf(pair_mx, mx);
                if (p.slices == 8 && lane < 32 && tok < p.rows)
                    p.tmax[(size_t)(8 * ts + (G::WTM / 32) * wm + i) * p.Cpad + tok] = mx;
                if (p.slices == 4 && (i & 1) && lane < 32 && tok < p.rows)
                    p.tmax[(size_t)(4 * ts + (G::WTM / 64) * wm + (i >> 1)) * p.Cpad + tok] = pair_mx;
                if (i & 1)
                    pair_mx = -__builtin_inff();
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float z = acc[i][j][r];
                    if (32 * i + 8 * (r >> 2) + (r & 3) < lim && z >= thr[j]) {
                        const uint32_t slot = atomicAdd(p.count + tok, 1u);
                        if (slot < (uint32_t)kTopkCap)
                            p.cand[(size_t)tok * kTopkCap + slot] =
                                ((uint64_t)topk_zkey(z) << 32) | (uint32_t)(m0 + G::row_of(wm, i, r, lane));
                    }
                }
            }
        }
    }
    if constexpr (!COLLECT) {
        if (p.slices == 1) {
            // the two waves holding a token's 256 rows merge their maxima through LDS
            float *red = reinterpret_cast<float *>(smem);   // [WM][BN]
#pragma unroll
            for (int j = 0; j < G::NB; ++j)
                if (lane < 32)
                    red[wm * G::BN + G::col_of(wn, j, lane)] = tile_mx[j];
            __syncthreads();
            for (int nl = threadIdx.x; nl < G::BN; nl += G::NT)
                if (n0 + nl < p.rows) {
                    float m = red[nl];
#pragma unroll
                    for (int w2 = 1; w2 < G::WM; ++w2)
                        m = fmaxf(m, red[w2 * G::BN + nl]);
                    p.tmax[(size_t)ts * p.Cpad + n0 + nl] = m;
                }
        }
    }
}

template <bool COLLECT>
__global__ __launch_bounds__(LogitGemm::NT) void topk_logits_kernel(TopkParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[LogitGemm::LDS_BYTES];
    if (p.guard && *p.guard == 0u)
        return;
    for (int t = blockIdx.x; t < p.nTm * p.nNt; t += gridDim.x) {
        topk_tile<COLLECT>(p, smem, t);
        __syncthreads();
    }
}

// Ascending bitonic sort of s[0, P) (P a power of two) by one wave.
template <class T>
__device__ void wave_bitonic_sort(T *s, int P)
{
    const int lane = threadIdx.x & 63;
    for (int k = 2; k <= P; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int q = lane; q < P / 2; q += 64) {
                const int i = 2 * q - (q & (j - 1));    // the pair (i, i + j), bit j of i clear
                const T a = s[i], b = s[i + j];
                if ((a > b) == ((i & k) == 0)) {
                    s[i] = b;
                    s[i + j] = a;
                }
            }
            __syncthreads();
        }
}

// Restores the min-heap order below entry j of a heap of n floats whose entry e sits at
// hp[e * 64] (one heap per lane, interleaved so that the lanes' accesses do not collide).
__device__ __forceinline__ void heap_sift_down(float *hp, int j, int n)
{
    const float v = hp[j * 64];
    for (;;) {
        const int l = 2 * j + 1;
        if (l >= n)
            break;
        const int m = (l + 1 < n && hp[(l + 1) * 64] < hp[l * 64]) ? l + 1 : l;
        if (!(hp[m * 64] < v))
            break;
        hp[j * 64] = hp[m * 64];
        j = m;
    }
    hp[j * 64] = v;
}

// One lane per token: tau = the K-th largest of the token's nSub slice maxima (-inf
// when there are fewer than K) as the root of a K-entry min-heap, and the token's
// candidate count reset.  Consecutive lanes read consecutive tokens of each maxima row.
// With `guard`, runs only when *guard != 0; `retry_reset` (may be NULL) is cleared.
__global__ __launch_bounds__(64) void topk_threshold_kernel(const float *tmax, int nSub, int Cpad, int rows, int K,
                                                          float *thr, uint32_t *count, const uint32_t *guard,
                                                          uint32_t *retry_reset)
{
    __shared__ float heap[kMaxK * 64];
    if (guard && *guard == 0u)
        return;
    const int lane = threadIdx.x, tok = blockIdx.x * 64 + lane;
    if (retry_reset && tok == 0)
        *retry_reset = 0u;
    if (tok >= rows)
        return;
    count[tok] = 0u;
    if (K > nSub) {
        thr[tok] = -__builtin_inff();
        return;
    }
    float *hp = heap + lane;
    for (int j = 0; j < K; ++j)
        hp[j * 64] = tmax[(size_t)j * Cpad + tok];
    for (int j = K / 2 - 1; j >= 0; --j)
        heap_sift_down(hp, j, K);
    constexpr int kBatch = 8;
    int i = K;
    for (; i + kBatch <= nSub; i += kBatch) {
        float v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            v[q] = tmax[(size_t)(i + q) * Cpad + tok];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (v[q] > hp[0]) {
                hp[0] = v[q];
                heap_sift_down(hp, 0, K);
            }
    }
    for (; i < nSub; ++i) {
        const float v = tmax[(size_t)i * Cpad + tok];
        if (v > hp[0]) {
            hp[0] = v;
            heap_sift_down(hp, 0, K);
        }
    }
    thr[tok] = hp[0];
}

// One wave per token: tau = the K-th largest of the token's nSub slice maxima by an
// ascending bitonic sort of them in LDS (nSub <= kTopkSortSub), and the token's
// candidate count reset; with many tokens this keeps every compute unit busy where the
// heap kernel above has one lane per token.  `guard` and `retry_reset` as there.
__global__ __launch_bounds__(64) void topk_threshold_sort_kernel(const float *tmax, int nSub, int Cpad, int K,
                                                               float *thr, uint32_t *count, const uint32_t *guard,
                                                               uint32_t *retry_reset)
{
    __shared__ float s[kTopkSortSub];
    if (guard && *guard == 0u)
        return;
    const int tok = blockIdx.x, lane = threadIdx.x;
    if (lane == 0) {
        count[tok] = 0u;
        if (retry_reset && tok == 0)
            *retry_reset = 0u;
    }
    if (K > nSub) {
        if (lane == 0)
            thr[tok] = -__builtin_inff();
        return;
    }
    int P = 64;
    while (P < nSub)
        P <<= 1;
    for (int i = lane; i < P; i += 64)
        s[i] = i < nSub ? tmax[(size_t)i * Cpad + tok] : -__builtin_inff();
    __syncthreads();
    wave_bitonic_sort(s, P);
    if (lane == 0)
        thr[tok] = s[P - K];
}

// One wave per token: sort the candidates and write the first K (index, z).  Fewer
// candidates than K raise the error flag; more than kTopkCap raise `retry` when it is
// given (a first pass over part of the vocabulary: the chunk is redone), else the error
// flag (many logits tied at the threshold).  With `guard`, runs only when *guard != 0.
__global__ __launch_bounds__(64) void topk_select_kernel(const uint64_t *cand, const uint32_t *count, int K,
                                                         int32_t *idx_out, void *logit_out, int logit_f32,
                                                         uint32_t *err, const uint32_t *guard, uint32_t *retry)
{
    __shared__ uint64_t s[kTopkCap];
    if (guard && *guard == 0u)
        return;
    const int tok = blockIdx.x, lane = threadIdx.x;
    const uint32_t n = count[tok];
    if (n > (uint32_t)kTopkCap || n < (uint32_t)K) {
        if (lane == 0)
            *((retry && n >= (uint32_t)K) ? retry : err) = 1u;
        return;
    }
    int P = 1;
    while (P < (int)n)
        P <<= 1;
    for (int i = lane; i < P; i += 64)
        s[i] = i < (int)n ? cand[(size_t)tok * kTopkCap + i] : ~0ull;
    __syncthreads();
    wave_bitonic_sort(s, P);
    for (int k = lane; k < K; k += 64) {
        const uint64_t key = s[k];
        const float z = topk_zkey_value((uint32_t)(key >> 32));
        idx_out[(size_t)tok * K + k] = (int32_t)(uint32_t)key;
        if (logit_f32)
            reinterpret_cast<float *>(logit_out)[(size_t)tok * K + k] = z;
        else
            reinterpret_cast<uint16_t *>(logit_out)[(size_t)tok * K + k] = (uint16_t)pack_bf16x2(z, 0.0f);
    }
}

// ------------------------------------------------------------------ dH = g . W

struct DhParams {
    const uint16_t *gT;     // [V rows of the slab, Cpad]
    const uint16_t *WT;     // the slab's first column of W^T [H, row pitch Vpad]
    int H, V, Vpad, rows, Cpad, nMt, nNt, ksplit;   // V: the slab's vocabulary rows
    int GM;                 // hidden tiles per group of the fallback tile order
    int split0;             // index of the slab's first split among all partial sums
    int xblk;               // 1: XCD blocks of 4 hidden x 8 token tiles (see dh_kernel)
    float *part;            // [splits, Cpad, H]
};

template <class G>
__global__ __launch_bounds__(G::NT) void dh_kernel(DhParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
    int tm, tn, split;
    if (p.xblk) {
        // Work-group L of the launch runs on XCD L % 8.  The launch is cut into blocks of
        // 4 hidden x 8 token tiles of one split (splits outermost, then token groups, then
        // hidden groups), and the w-th work-group of an XCD takes tile w % 32 (hidden
        // fastest) of block (w / 32) * 8 + L % 8.  The 32 work-groups an XCD runs at a
        // time then read 4 row blocks of W^T and 8 column blocks of g^T per k-step, and
        // the eight XCDs of a round read the same split.
        const int L = blockIdx.y * gridDim.x + blockIdx.x;
        const int w = L >> 3, q = w & 31;
        const int beta = (w >> 5) * 8 + (L & 7);
        const int hgs = p.nMt >> 2, bps = hgs * (p.nNt >> 3);
        split = beta / bps;
        const int b = beta - split * bps;
        tm = (b % hgs) * 4 + (q & 3);
        tn = (b / hgs) * 8 + (q >> 2);
    } else {
        // groups of GM hidden tiles with all token tiles, hidden tile fastest
        map_tile(blockIdx.x, p.nMt, p.nNt, p.GM, tm, tn);
        split = blockIdx.y;
    }
    const int m0 = tm * G::BM, n0 = tn * G::BN;     // m: hidden, n: tokens
    const int k_begin = split * p.ksplit;
    const int k_end = min(p.V, k_begin + p.ksplit);
    f32x16 acc[G::MB][G::NB];
    // dH^T tile: A(m = hidden, k = vocab) = WT[m][k]; B(n = token, k = vocab) = gT[k][n].
    if (m0 + G::BM <= p.H)
        G::run(smem, p.WT, p.Vpad, m0, p.H, k_end, p.gT, p.Cpad, n0, p.rows, k_end, k_begin, k_end, acc);
    else
        G::template run<NoHook, true>(smem, p.WT, p.Vpad, m0, p.H, k_end, p.gT, p.Cpad, n0, p.rows, k_end, k_begin,
                                      k_end, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
    float *out = p.part + (size_t)(p.split0 + split) * p.Cpad * p.H;
    // each lane holds 4 consecutive hidden entries of one token per (i, j, q)
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int t = n0 + G::col_of(wn, j, lane);
        if (t < p.rows) {
#pragma unroll
            for (int i = 0; i < G::MB; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int hh = m0 + G::row_of(wm, i, 4 * q, lane);
                    if (hh < p.H)
                        *reinterpret_cast<float4 *>(out + (size_t)t * p.H + hh) =
                            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                        acc[i][j][4 * q + 3]);
                }
        }
    }
}

// dH[row] = sum over splits, in split order.
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float *part, int splits, size_t split_stride,
                                                         size_t n4, float *dH)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4)
        return;
    float4 a = reinterpret_cast<const float4 *>(part)[i];
    for (int s = 1; s < splits; ++s) {
        const float4 b = reinterpret_cast<const float4 *>(part + s * split_stride)[i];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    reinterpret_cast<float4 *>(dH)[i] = a;
}

// ------------------------------------------------------------------ dW += g^T . h

struct DwParams {
    const uint16_t *gT;     // [Vpad, Cpad]: the slab's rows, Vpad = its tiles * 256
    const uint16_t *hT;     // [H, Cpad]
    int H, V, Vpad, Cpad, rows, nMt, nNt, accumulate;   // V: the slab's vocabulary rows
    float *dW;              // the slab's first row of dW [V, H]
};

template <class G>
__global__ __launch_bounds__(G::NT) void dw_kernel(DwParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
    int tm, tn;
    // pairs of vocabulary row-blocks, all hidden tiles of a pair before the next pair:
    // -2% against one row-block at a time (four or more are slower)
    map_tile(blockIdx.x, p.nMt, p.nNt, 2, tm, tn);
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    f32x16 acc[G::MB][G::NB];
    // A(m = vocab, k = token) = gT[m][k]; B(n = hidden, k = token) = hT[n][k].
    if (n0 + G::BN <= p.H)
        G::run(smem, p.gT, p.Cpad, m0, p.Vpad, p.rows, p.hT, p.Cpad, n0, p.H, p.rows, 0, p.rows, acc);
    else
        G::template run<NoHook, true>(smem, p.gT, p.Cpad, m0, p.Vpad, p.rows, p.hT, p.Cpad, n0, p.H, p.rows, 0,
                                      p.rows, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = G::wm_of(wave), wn = G::wn_of(wave);
    // Each lane owns one hidden column of 16 * MB rows per fragment column.  Every dW
    // element is written by one work-group per launch, and the launches run chunk after
    // chunk, so adding with a hardware fp32 atomic (no return value) gives the same sum
    // as a read-modify-write without waiting for the old value.
#pragma unroll
    for (int j = 0; j < G::NB; ++j) {
        const int col = n0 + G::col_of(wn, j, lane);
        if (col < p.H) {
#pragma unroll
            for (int i = 0; i < G::MB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + G::row_of(wm, i, r, lane);
                    if (row < p.V) {
                        float *dst = p.dW + (size_t)row * p.H + col;
                        if (p.accumulate)
                            unsafeAtomicAdd(dst, acc[i][j][r]);
                        else
                            *dst = acc[i][j][r];
                    }
                }
        }
    }
}

using DGemm = GemmD<kHiddenTile, 256, 2, 4, 64, 2, false, true, true>;   // dH^T: hidden x tokens, k = vocabulary
using WGemm = GemmD<256, kHiddenTile, 2, 4, 64, 2, true>;   // dW: vocabulary x hidden, k = tokens

// dst[c][r] = src[r][c] for r < rows, c < cols; dst[c][r] = 0 for rows <= r < rpad.
// 64 x 64 tiles through LDS, 16-byte pieces on both sides: each thread loads two
// 8-element row pieces and stores two 8-element column pieces.  cols is a multiple of
// 8 (H), rpad a multiple of 64, both leading dimensions multiples of 8.
// LDS: 128-byte rows, with the 16-byte chunk of element (r, c) XORed with (r / 8) % 8.
// A wave's element reads take one column c per group of 8 lanes at rows r8 + j with
// r8 = 0, 8, .., 56: in one row the 8 rows would share their bank offsets (a 128-byte
// pitch puts every other row at the same bank; padding cannot help while rows stay
// 16-byte aligned), and the swizzle moves them to 8 distinct chunks instead, so the
// wave's 64 reads hit 32 distinct dwords in 32 distinct banks.
__device__ __forceinline__ int transpose_lds_index(int r, int c)
{
    return r * 64 + ((((c >> 3) ^ (r >> 3)) & 7) << 3) + (c & 7);
}

__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *src, int64_t ld_src, int rows, int cols,
                                                        uint16_t *dst, int64_t ld_dst, int rpad)
{
    __shared__ __attribute__((aligned(16))) uint16_t t[64 * 64];
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = threadIdx.x + 256 * q;
        const int r = e >> 3, c8 = (e & 7) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r0 + r < rows && c0 + c8 < cols)
            v = *reinterpret_cast<const u32x4 *>(src + (int64_t)(r0 + r) * ld_src + c0 + c8);
        *reinterpret_cast<u32x4 *>(t + transpose_lds_index(r, c8)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = threadIdx.x + 256 * q;
        const int c = e >> 3, r8 = (e & 7) * 8;
        if (c0 + c < cols && r0 + r8 < rpad) {
            u32x4 v;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                v[w] = (uint32_t)t[transpose_lds_index(r8 + 2 * w, c)] |
                       ((uint32_t)t[transpose_lds_index(r8 + 2 * w + 1, c)] << 16);
            *reinterpret_cast<u32x4 *>(dst + (int64_t)(c0 + c) * ld_dst + r0 + r8) = v;
        }
    }
}

// x[i] *= *scale, four floats per thread (x 16-byte aligned), a grid-stride loop.
__global__ __launch_bounds__(256) void scale_kernel(float *x, int64_t n, const float *scale)
{
    const float c = *scale;
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        float4 v = reinterpret_cast<float4 *>(x)[i];
        v.x *= c;
        v.y *= c;
        v.z *= c;
        v.w *= c;
        reinterpret_cast<float4 *>(x)[i] = v;
    }
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)(n - 4 * n4))
        x[4 * n4 + threadIdx.x] *= c;
}

__global__ void topk_status_kernel(const uint32_t *flag, uint32_t *status, uint32_t code)
{
    if (threadIdx.x == 0)
        *status = *flag ? code : 0u;
}

__global__ void zero_u32_kernel(uint32_t *p, int n)
{
    if ((int)threadIdx.x < n)
        p[threadIdx.x] = 0u;
}

}  // namespace

// ------------------------------------------------------------------ allocation-free workspace

// The workspace of fckl_forward_noalloc: a device array of the library, so that the call
// needs no memory from its caller (each device the library runs on holds it until the
// process ends).  In host code `scratch` is only a stand-in for the symbol; its device
// address on the current device comes from hipGetSymbolAddress, looked up once per
// device and kept below.  Calls that overlap on one device share the array and race.
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::once_flag g_scratch_once[kMaxDevices];
static void *g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];

int scratch_address(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev < 0 || dev >= kMaxDevices)
        return (int)hipErrorInvalidDevice;
    // with `dev` current (this thread's device), once per device
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess)
        return (int)g_scratch_err[dev];
    *ptr = g_scratch_ptr[dev];
    return 0;
}

// ------------------------------------------------------------------ launchers

static inline hipStream_t S(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Work-groups of a persistent logit kernel: one per compute unit of the current device
// (rounded up to a multiple of the 8 XCDs), never more than there are tiles.  The count
// is asked of the runtime on every launch (it answers from the device properties it
// holds), so the library keeps no state of its own.
static int persistent_grid(int tiles)
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    n = (n + 7) / 8 * 8;
    return tiles < n ? tiles : n;
}

int launch_prepare(const ChunkArgs &a, bool validate, void *stream, const GradScale *gs)
{
    const Layout &L = *a.L;
    PrepParams p;
    p.idx = a.idx;
    p.tl = a.tl;
    p.logit_f32 = a.logit_f32;
    p.rows = a.rows;
    p.K = a.K;
    p.V = a.V;
    p.nVt = L.nVt;
    p.cnt_stride = L.cnt_stride;
    p.scale2 = kLog2e / a.T;
    p.idx_s = reinterpret_cast<int32_t *>(a.ws + L.off_idx);
    p.p_s = reinterpret_cast<float *>(a.ws + L.off_p);
    p.zk = reinterpret_cast<float *>(a.ws + L.off_zk);
    p.psum = reinterpret_cast<float *>(a.ws + L.off_psum);
    p.negent = reinterpret_cast<float *>(a.ws + L.off_negent);
    p.cnt = reinterpret_cast<uint8_t *>(a.ws + L.off_cnt);
    p.err = reinterpret_cast<uint32_t *>(a.ws + L.off_err);
    p.validate = validate ? 1 : 0;
    p.scaled = gs ? 1 : 0;
    p.gcoef = gs ? gs->coef : 1.0f;
    p.gw = gs ? gs->w : nullptr;
    p.ginv = gs ? gs->inv_wsum : nullptr;
    p.gmul = gs ? gs->mul : nullptr;
    hipLaunchKernelGGL(prepare_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, S(stream), p);
    return (int)hipGetLastError();
}

int launch_forward_logits(const ChunkArgs &a, void *stream, bool keep_exp)
{
    const Layout &L = *a.L;
    FwdParams p;
    p.W = a.W;
    p.h = a.h;
    p.H = a.H;
    p.V = a.V;
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.K = a.K;
    p.nVt = L.nVt;
    p.nNt = (a.rows + LogitGemm::BN - 1) / LogitGemm::BN;
    p.cnt_stride = L.cnt_stride;
    p.scale2 = kLog2e / a.T;
    p.idx_s = reinterpret_cast<const int32_t *>(a.ws + L.off_idx);
    p.cnt = reinterpret_cast<const uint8_t *>(a.ws + L.off_cnt);
    p.zk = reinterpret_cast<float *>(a.ws + L.off_zk);
    p.part = reinterpret_cast<float2 *>(a.ws + L.off_part);
    p.ex = reinterpret_cast<uint16_t *>(a.ws + L.off_ex);
    p.mw = reinterpret_cast<float *>(a.ws + L.off_mw);
    p.Vpad = L.Vpad;
    const dim3 grid(persistent_grid(p.nVt * p.nNt));
    if (keep_exp)
        hipLaunchKernelGGL(forward_logits_kernel<true>, grid, dim3(LogitGemm::NT), 0, S(stream), p);
    else
        hipLaunchKernelGGL(forward_logits_kernel<false>, grid, dim3(LogitGemm::NT), 0, S(stream), p);
    return (int)hipGetLastError();
}

int launch_combine(const ChunkArgs &a, float *loss_tok, float *lse, void *stream)
{
    const Layout &L = *a.L;
    CombineParams p;
    p.part = reinterpret_cast<const float2 *>(a.ws + L.off_part);
    p.zk = reinterpret_cast<const float *>(a.ws + L.off_zk);
    p.p_s = reinterpret_cast<const float *>(a.ws + L.off_p);
    p.psum = reinterpret_cast<const float *>(a.ws + L.off_psum);
    p.negent = reinterpret_cast<const float *>(a.ws + L.off_negent);
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.nVt = L.nVt;
    p.K = a.K;
    p.T = a.T;
    p.loss_tok = loss_tok;
    p.lse = lse;
    hipLaunchKernelGGL(combine_kernel, dim3((a.rows + 31) / 32), dim3(256), 0, S(stream), p);
    return (int)hipGetLastError();
}

int launch_mean(const float *loss_tok, int64_t N, float *loss_mean, void *stream)
{
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, S(stream), loss_tok, N, loss_mean);
    return (int)hipGetLastError();
}

int launch_weighted_mean(const float *loss_tok, const float *w, int64_t N, float *loss_mean, void *stream)
{
    hipLaunchKernelGGL(weighted_mean_kernel, dim3(1), dim3(1024), 0, S(stream), loss_tok, w, N, loss_mean);
    return (int)hipGetLastError();
}

int launch_weight_sum(const float *w, int64_t N, float *out2, void *stream)
{
    hipLaunchKernelGGL(weight_sum_kernel, dim3(1), dim3(1024), 0, S(stream), w, N, out2);
    return (int)hipGetLastError();
}

int launch_softmax_grad(const ChunkArgs &a, const float *lse, const GradScale &gs, void *stream)
{
    const Layout &L = *a.L;
    SoftGradParams p;
    p.ex = reinterpret_cast<const uint16_t *>(a.ws + L.off_ex);
    p.gT = reinterpret_cast<uint16_t *>(a.ws + L.off_gT);
    p.mw = reinterpret_cast<const float *>(a.ws + L.off_mw);
    p.lse = lse;
    p.psum = reinterpret_cast<const float *>(a.ws + L.off_psum);
    p.idx_s = reinterpret_cast<const int32_t *>(a.ws + L.off_idx);
    p.p_s = reinterpret_cast<const float *>(a.ws + L.off_p);
    p.cnt = reinterpret_cast<const uint8_t *>(a.ws + L.off_cnt);
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.Vpad = L.Vpad;
    p.K = a.K;
    p.cnt_stride = L.cnt_stride;
    p.coef = gs.coef;
    p.w = gs.w;
    p.inv_wsum = gs.inv_wsum;
    p.mul = gs.mul;
    p.vt0 = a.vt0;
    hipLaunchKernelGGL(softmax_grad_kernel, dim3(a.nvt, (a.rows + kSgTok - 1) / kSgTok), dim3(kSgThreads), 0,
                       S(stream), p);
    return (int)hipGetLastError();
}

int launch_backward_logits(const ChunkArgs &a, const float *lse, void *stream)
{
    const Layout &L = *a.L;
    BwdParams p;
    p.W = a.W;
    p.h = a.h;
    p.H = a.H;
    p.V = a.V;
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.Vpad = L.Vpad;
    p.K = a.K;
    p.nVt = a.nvt;
    p.vt0 = a.vt0;
    p.nNt = (a.rows + LogitGemm::BN - 1) / LogitGemm::BN;
    p.cnt_stride = L.cnt_stride;
    p.scale2 = kLog2e / a.T;
    p.lse = lse;
    p.idx_s = reinterpret_cast<const int32_t *>(a.ws + L.off_idx);
    p.p_s = reinterpret_cast<const float *>(a.ws + L.off_p);
    p.psum = reinterpret_cast<const float *>(a.ws + L.off_psum);
    p.cnt = reinterpret_cast<const uint8_t *>(a.ws + L.off_cnt);
    p.gT = reinterpret_cast<uint16_t *>(a.ws + L.off_gT);
    hipLaunchKernelGGL(backward_logits_kernel, dim3(persistent_grid(p.nVt * p.nNt)), dim3(LogitGemm::NT), 0, S(stream), p);
    return (int)hipGetLastError();
}

// The slab a covers: its index among the layout's slabs.
static int32_t slab_index(const ChunkArgs &a)
{
    return a.L->slab_tiles > 0 ? a.vt0 / a.L->slab_tiles : 0;
}

int launch_dh(const ChunkArgs &a, void *stream)
{
    static_assert(DGemm::BK == kDhStep, "dH splits are whole k-steps");
    const Layout &L = *a.L;
    const int v0 = a.vt0 * kVocabTile;
    DhParams p;
    p.gT = reinterpret_cast<const uint16_t *>(a.ws + L.off_gT);
    p.WT = reinterpret_cast<const uint16_t *>(a.ws + L.off_WT) + v0;
    p.H = a.H;
    p.V = std::min(a.V - v0, a.nvt * kVocabTile);
    p.Vpad = L.Vpad;
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.nMt = (a.H + kHiddenTile - 1) / kHiddenTile;
    p.nNt = (a.rows + 255) / 256;
    int32_t ksplit = 0, used = 0;
    slab_split_rows(L, a.V, a.H, slab_index(a), &ksplit, &used);
    p.ksplit = ksplit;
    p.split0 = a.split0;
    // Tile order.  A dH work-group waits on its global -> LDS loads (a part-filled hidden
    // tile takes as long as a full one), so the order is chosen for L2 hits.  When the
    // launch divides into whole rounds of 4 x 8-tile blocks, one per XCD (H = 2880 and
    // 4096 at a chunk of 8192 do), each XCD works on such blocks: 22% fewer L2-miss bytes
    // than the order below, and no slower.  Otherwise each XCD
    // takes one eighth of a split's tiles; with groups of GM hidden tiles, GM the smallest
    // whole multiple of nMt / gcd(nMt, 8) (so that no XCD's share straddles two groups)
    // that is at least nMt / 4, an XCD pair covers a quarter of the hidden tiles and half
    // of the token tiles.  At H = 2880 (12 tiles) and 4096 (16) that is 3 and 4 tiles,
    // 2-4% faster than all hidden tiles of a token tile at a time; groups of 1, 2, 4
    // and 6 (of 12 tiles) or 2 (of 16) are slower than 3 and 4.
    {
        int g = 8, m = p.nMt;
        while (m) {
            const int t = g % m;
            g = m;
            m = t;
        }
        const int base = p.nMt / g;
        p.GM = base * std::max(1, (p.nMt / 4 + base - 1) / base);
        p.GM = std::min(p.GM, p.nMt);
    }
    p.xblk = (p.nMt % 4 == 0 && p.nNt % 8 == 0 && ((p.nMt / 4) * (p.nNt / 8) * used) % 8 == 0) ? 1 : 0;
    p.part = reinterpret_cast<float *>(a.ws + L.off_dhp);
    dim3 grid(p.nMt * p.nNt, used);
    hipLaunchKernelGGL(dh_kernel<DGemm>, grid, dim3(DGemm::NT), 0, S(stream), p);
    return (int)hipGetLastError();
}

int launch_dh_reduce(const ChunkArgs &a, float *dH, void *stream)
{
    const Layout &L = *a.L;
    const int32_t used = dh_partials(L, a.V, a.H, L.nslab);
    const float *part = reinterpret_cast<const float *>(a.ws + L.off_dhp);
    const size_t n4 = (size_t)a.rows * a.H / 4;
    hipLaunchKernelGGL(dh_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, S(stream), part, used,
                       (size_t)L.Cpad * a.H, n4, dH);
    return (int)hipGetLastError();
}

int launch_dw(const ChunkArgs &a, float *dW, bool accumulate, void *stream)
{
    const Layout &L = *a.L;
    const int v0 = a.vt0 * kVocabTile;
    DwParams p;
    p.gT = reinterpret_cast<const uint16_t *>(a.ws + L.off_gT);
    p.hT = reinterpret_cast<const uint16_t *>(a.ws + L.off_hT);
    p.H = a.H;
    p.V = std::min(a.V - v0, a.nvt * kVocabTile);
    p.Vpad = a.nvt * kVocabTile;
    p.Cpad = L.Cpad;
    p.rows = a.rows;
    p.nMt = a.nvt;
    p.nNt = (a.H + kHiddenTile - 1) / kHiddenTile;
    p.accumulate = accumulate ? 1 : 0;
    p.dW = dW + (size_t)v0 * a.H;
    dim3 grid(p.nMt * p.nNt);
    hipLaunchKernelGGL(dw_kernel<WGemm>, grid, dim3(WGemm::NT), 0, S(stream), p);
    return (int)hipGetLastError();
}

// W [V, H] -> WT [H, Vpad] (columns V..Vpad-1 zero).
int launch_transpose_head(const ChunkArgs &a, void *stream)
{
    const Layout &L = *a.L;
    uint16_t *WT = reinterpret_cast<uint16_t *>(a.ws + L.off_WT);
    dim3 grid((L.Vpad + 63) / 64, (a.H + 63) / 64);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, S(stream), a.W, (int64_t)a.H, a.V, a.H, WT,
                       (int64_t)L.Vpad, L.Vpad);
    return (int)hipGetLastError();
}

// chunk's h [rows, H] -> hT [H, Cpad] (columns rows..Cpad-1 zero).
int launch_transpose_chunk(const ChunkArgs &a, void *stream)
{
    const Layout &L = *a.L;
    uint16_t *hT = reinterpret_cast<uint16_t *>(a.ws + L.off_hT);
    dim3 grid((L.Cpad + 63) / 64, (a.H + 63) / 64);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, S(stream), a.h, (int64_t)a.H, a.rows, a.H, hT,
                       (int64_t)L.Cpad, L.Cpad);
    return (int)hipGetLastError();
}

int launch_scale(float *x, int64_t n, const float *scale, void *stream)
{
    const int64_t n4 = n / 4;
    const int64_t blocks = std::min<int64_t>(std::max<int64_t>((n4 + 255) / 256, 1), 8192);
    hipLaunchKernelGGL(scale_kernel, dim3((unsigned)blocks), dim3(256), 0, S(stream), x, n, scale);
    return (int)hipGetLastError();
}

int launch_topk_status(const uint32_t *flag, uint32_t *status, uint32_t code, void *stream)
{
    hipLaunchKernelGGL(topk_status_kernel, dim3(1), dim3(64), 0, S(stream), flag, status, code);
    return (int)hipGetLastError();
}

int launch_zero_flag(uint32_t *flag, void *stream)
{
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, S(stream), flag, 4);
    return (int)hipGetLastError();
}

int launch_full_teacher(const ChunkArgs &a, const FullLayout &F, const uint16_t *h_t, const uint16_t *W_t,
                        void *stream)
{
    const Layout &L = F.base;
    FullTeacherParams p;
    p.W = W_t;
    p.h = h_t;
    p.H = F.Ht;
    p.V = a.V;
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.nVt = L.nVt;
    p.nNt = (a.rows + LogitGemm::BN - 1) / LogitGemm::BN;
    p.scale2 = kLog2e / a.T;
    p.part = reinterpret_cast<float2 *>(a.ws + F.off_part_t);
    p.at = reinterpret_cast<float *>(a.ws + F.off_at);
    hipLaunchKernelGGL(full_teacher_kernel, dim3(persistent_grid(p.nVt * p.nNt)), dim3(LogitGemm::NT), 0,
                       S(stream), p);
    return (int)hipGetLastError();
}

int launch_full_combine_teacher(const ChunkArgs &a, const FullLayout &F, void *stream)
{
    hipLaunchKernelGGL(full_combine_kernel, dim3((a.rows + 31) / 32), dim3(256), 0, S(stream),
                       reinterpret_cast<const float2 *>(a.ws + F.off_part_t), (const float *)nullptr, F.base.nVt,
                       F.base.Cpad, a.rows, a.T, (const float *)nullptr, reinterpret_cast<float *>(a.ws + F.off_lt2),
                       (float *)nullptr, (float *)nullptr);
    return (int)hipGetLastError();
}

int launch_full_student(const ChunkArgs &a, const FullLayout &F, void *stream)
{
    const Layout &L = F.base;
    FullStudentParams p;
    p.W = a.W;
    p.h = a.h;
    p.H = a.H;
    p.V = a.V;
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.Vpad = L.Vpad;
    p.nVt = L.nVt;
    p.nNt = (a.rows + LogitGemm::BN - 1) / LogitGemm::BN;
    p.scale2 = kLog2e / a.T;
    p.at = reinterpret_cast<const float *>(a.ws + F.off_at);
    p.lt2 = reinterpret_cast<const float *>(a.ws + F.off_lt2);
    p.part = reinterpret_cast<float2 *>(a.ws + L.off_part);
    p.px = reinterpret_cast<float *>(a.ws + F.off_px);
    p.ex = reinterpret_cast<uint16_t *>(a.ws + L.off_ex);
    p.mw = reinterpret_cast<float *>(a.ws + L.off_mw);
    hipLaunchKernelGGL(full_student_kernel, dim3(persistent_grid(p.nVt * p.nNt)), dim3(LogitGemm::NT), 0,
                       S(stream), p);
    return (int)hipGetLastError();
}

int launch_full_combine_student(const ChunkArgs &a, const FullLayout &F, float *loss_tok, float *lse, void *stream)
{
    hipLaunchKernelGGL(full_combine_kernel, dim3((a.rows + 31) / 32), dim3(256), 0, S(stream),
                       reinterpret_cast<const float2 *>(a.ws + F.base.off_part),
                       reinterpret_cast<const float *>(a.ws + F.off_px), F.base.nVt, F.base.Cpad, a.rows, a.T,
                       reinterpret_cast<const float *>(a.ws + F.off_lt2), reinterpret_cast<float *>(a.ws + F.off_ls2),
                       loss_tok, lse);
    return (int)hipGetLastError();
}

int launch_full_grad(const ChunkArgs &a, const FullLayout &F, const GradScale &gs, void *stream)
{
    const Layout &L = F.base;
    FullGradParams p;
    p.ex = reinterpret_cast<const uint16_t *>(a.ws + L.off_ex);
    p.gT = reinterpret_cast<uint16_t *>(a.ws + L.off_gT);
    p.at = reinterpret_cast<const float *>(a.ws + F.off_at);
    p.mw = reinterpret_cast<const float *>(a.ws + L.off_mw);
    p.ls2 = reinterpret_cast<const float *>(a.ws + F.off_ls2);
    p.lt2 = reinterpret_cast<const float *>(a.ws + F.off_lt2);
    p.rows = a.rows;
    p.Cpad = L.Cpad;
    p.Vpad = L.Vpad;
    p.V = a.V;
    p.coef = gs.coef;
    p.w = gs.w;
    p.inv_wsum = gs.inv_wsum;
    p.vt0 = a.vt0;
    hipLaunchKernelGGL(full_grad_kernel, dim3(a.nvt, (a.rows + 63) / 64), dim3(256), 0, S(stream), p);
    return (int)hipGetLastError();
}

static TopkParams topk_params(const ChunkArgs &a, const TopkLayout &T, const uint32_t *guard)
{
    TopkParams p;
    p.W = a.W;
    p.h = a.h;
    p.H = a.H;
    p.V = a.V;
    p.rows = a.rows;
    p.Cpad = T.Cpad;
    p.nVt = T.nVt;
    p.nNt = (a.rows + LogitGemm::BN - 1) / LogitGemm::BN;
    p.stride = 1;
    p.nTm = T.nVt;
    p.slices = 1;
    p.guard = guard;
    p.tmax = reinterpret_cast<float *>(a.ws + T.off_tmax);
    p.thr = reinterpret_cast<const float *>(a.ws + T.off_thr);
    p.count = reinterpret_cast<uint32_t *>(a.ws + T.off_count);
    p.cand = reinterpret_cast<uint64_t *>(a.ws + T.off_cand);
    return p;
}

int launch_topk_max(const ChunkArgs &a, const TopkLayout &T, bool partial, const uint32_t *guard, void *stream)
{
    TopkParams p = topk_params(a, T, guard);
    if (partial) {
        p.stride = kTopkStride;
        p.nTm = (T.nVt + kTopkStride - 1) / kTopkStride;
        p.slices = kVocabTile / 64;
    } else {
        p.slices = T.nSubFull / T.nVt;
    }
    hipLaunchKernelGGL(topk_logits_kernel<false>, dim3(persistent_grid(p.nTm * p.nNt)), dim3(LogitGemm::NT), 0,
                       S(stream), p);
    return (int)hipGetLastError();
}

int launch_topk_threshold(const ChunkArgs &a, const TopkLayout &T, bool partial, const uint32_t *guard,
                          uint32_t *retry_reset, void *stream)
{
    const int nSub = partial ? T.nSubPart : T.nSubFull;
    const float *tmax = reinterpret_cast<const float *>(a.ws + T.off_tmax);
    float *thr = reinterpret_cast<float *>(a.ws + T.off_thr);
    uint32_t *count = reinterpret_cast<uint32_t *>(a.ws + T.off_count);
    if (nSub <= kTopkSortSub)
        hipLaunchKernelGGL(topk_threshold_sort_kernel, dim3(a.rows), dim3(64), 0, S(stream), tmax, nSub, T.Cpad, a.K,
                           thr, count, guard, retry_reset);
    else
        hipLaunchKernelGGL(topk_threshold_kernel, dim3((a.rows + 63) / 64), dim3(64), 0, S(stream), tmax, nSub,
                           T.Cpad, a.rows, a.K, thr, count, guard, retry_reset);
    return (int)hipGetLastError();
}

int launch_topk_collect(const ChunkArgs &a, const TopkLayout &T, const uint32_t *guard, void *stream)
{
    const TopkParams p = topk_params(a, T, guard);
    hipLaunchKernelGGL(topk_logits_kernel<true>, dim3(persistent_grid(p.nTm * p.nNt)), dim3(LogitGemm::NT), 0,
                       S(stream), p);
    return (int)hipGetLastError();
}

int launch_topk_select(const ChunkArgs &a, const TopkLayout &T, int32_t *topk_idx, void *topk_logit, bool logit_f32,
                       const uint32_t *guard, uint32_t *retry, void *stream)
{
    hipLaunchKernelGGL(topk_select_kernel, dim3(a.rows), dim3(64), 0, S(stream),
                       reinterpret_cast<const uint64_t *>(a.ws + T.off_cand),
                       reinterpret_cast<const uint32_t *>(a.ws + T.off_count), a.K, topk_idx, topk_logit,
                       logit_f32 ? 1 : 0, reinterpret_cast<uint32_t *>(a.ws + T.off_err), guard, retry);
    return (int)hipGetLastError();
}

}  // namespace fckl
