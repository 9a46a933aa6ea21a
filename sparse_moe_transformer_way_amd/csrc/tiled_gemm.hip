// LDS-tiled MFMA grouped GEMM for many rows per expert (bf16, row tile 256).
//
// The two expert projections of the SwiGLU experts (Mixtral of Experts,
// paper-graph-ui page, section 3.4, "Expert Network Structure (SwiGLU)"):
//   gate/up : h[p, f]  = SiLU(sum_k x[tok(p), k] w1[e, f, k]) * (sum_k x[tok(p), k] w3[e, f, k])
//   down    : y[p, j]  = sum_k h[p, k] w2[e, j, k]
// over the expert-grouped rows p of expert e's segment.  Both are dense
// contractions with k contiguous in both operands.
//
// Tiling (gfx950: 256 CUs, 4 SIMDs each, 160 KB LDS per CU):
//   * one workgroup = 4 waves = one 256 (weight rows) x 256 (token rows) tile;
//     gate/up tiles hold 128 rows of w1 and the same 128 rows of w3 so that the
//     SiLU gate is formed in registers.  Each wave owns 128 x 128 outputs as
//     4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane,
//     kept in AGPRs; one wave per SIMD).
//   * K advances 64 per LDS buffer ("block").  A block is 256 weight rows +
//     256 token rows of 128 bytes = 64 KB, copied HBM/L2 -> LDS by buffer loads
//     with the LDS destination bit (no register staging), 8 rows x 128 bytes
//     per wave instruction, so every request covers a whole 128-byte line
//     (measured on MI355X: half-line copies of 32-k stages issued twice the L2
//     requests and ran the kernels 8-11% slower).  Gate/up: two buffers, block
//     kb+2 is copied while block kb+1 lands and block kb is consumed.  Down:
//     two weight and three token buffers of 32 KB (all of the LDS), so the
//     token rows of block kb+3 are copied while block kb is consumed.
//   * A block is consumed as two 32-k stages of 32 MFMAs; each stage's 16
//     fragments are read into a second register set under the previous
//     stage's MFMAs, one read per two MFMAs; the copies of a block go out
//     during its second stage (spread over it for gate/up, over its first half
//     for the down projection).  One barrier per block, before
//     its second stage: it waits for block kb+1's copies and for every wave's
//     reads of block kb, so block kb+2 may then be copied over it.  (Measured:
//     bursts of fragment reads just ahead of their MFMAs left the matrix cores
//     a third idle; this spacing keeps them busy.)
//   * Copies address a wave-uniform buffer resource plus a 32-bit per-lane
//     offset, with the k of the block (and the row group) as the scalar offset.
//   * LDS rows are 8 chunks of 16 bytes; chunk c of row r sits at c ^ g(r) with
//     g(r) = r1 | r2 << 1 | r4 << 2 (bits of r).  gfx950's LDS has 64 banks; a
//     32-row fragment read (ds_read_b128) is served in 16-lane phases (lanes
//     0-7 with 16-23, 8-15 with 24-31, measured with SQ_LDS_BANK_CONFLICT);
//     in each phase the 8 even rows and the 8 odd rows get 8 distinct chunks,
//     so the phase covers all 64 banks.  The copies write whole 1 KB runs.
//   * Tile order (tile_contiguous, tile_by_column): workgroup b runs on XCD
//     b % 8; the tiles the segments actually hold are enumerated on the device
//     from the segment offsets (the grid is sized for the worst case and the
//     spare workgroups exit), in groups of a few weight tiles x all of an
//     expert's token tiles, so the tiles an XCD runs at once share their data
//     in its L2.
//   * An expert's last token tile with at most 128 real rows runs as a narrow
//     tile (narrow_tile): 64 or 128 token rows, the weight rows split over the
//     four waves.  A 64-row narrow tile moves 128 k per buffer (two 64-k
//     blocks of 40 KB), so its two buffers take 80 KB each.
//   * Padding rows of a token tile copy a real row (gate/up) or the padded rows
//     of h (down).  Gate/up writes zeros for them into h; down writes whatever
//     they sum to (y_perm rows past an expert's count are unspecified).
//   * Epilogue stores: gate/up pairs lanes l and l + 32 with a permlane32 swap
//     so that each lane stores 16 bytes of h; down stages its fp32 rows through
//     LDS (store_rows_staged) into row-contiguous runs.
//   * K may be cut into two parts (down projection with few tiles, as the
//     plan of down_plan decides on the device): part s covers k in
//     [s*K/2, (s+1)*K/2) and writes its own fp32 output buffer.
#include "moe_common.h"

#include <utility>

namespace moe {

namespace {

constexpr int kTW = 256;                     // weight rows per tile
constexpr int kTT = kTiledRows;              // token rows per tile
constexpr int kBK = 64;                      // k per LDS buffer (one "block")
constexpr int kChunks = kBK / 8;             // 16-byte chunks per LDS row (128-byte rows)
constexpr int kBufVec = (kTW + kTT) * kChunks;  // uint4 per buffer (64 KB)
constexpr int kCopies = 16;                  // copies per lane per block
constexpr int kGroupVec = 8 * kChunks;       // uint4 of one 8-row copy group (1 KB)
constexpr int kXcdTiles = 32;                // tiles an XCD runs at once (its CUs)
// Each of the two LDS buffers: a full tile's block, or two 64-k blocks of a
// 64-row narrow tile (2 x 40 KB), so the kernel takes all 160 KB of LDS.
constexpr int kLdsVec = kBufVec > 2 * (kTW + 64) * kChunks ? kBufVec : 2 * (kTW + 64) * kChunks;

typedef void __attribute__((address_space(3)))* lptr_t;

// g(r) = r1 | r2 << 1 | r4 << 2
__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) | (((row >> 4) & 1) << 2); }

// Token tiles of an expert's segment (length len, padded to kTT, count rows).
// With tail_rows > 0 a last tile holding at most tail_rows real rows is left
// to the weight-streaming kernels (it would cost a whole tile here); the
// kernel only does so when that saves a round of tiles (down_plan).
__device__ __forceinline__ int token_tiles(int len, int count, int tail_rows) {
    const int r = count % kTT;
    return (r > 0 && r <= tail_rows) ? count / kTT : len / kTT;
}

// Buffer resource over [base, base + 4 GiB); every offset the kernel adds is
// in range by construction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    // dword 3 = 0x00020000: 32-bit data format, the raw-buffer setting of gfx9
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}

// Workgroup barrier: waits until at most N of this wave's vector-memory
// operations are outstanding and all its LDS reads are done.  The empty asm
// statements only stop the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef u32x4_t Frag16[16];  // one 32-k stage's fragments: [k16 half][4 weight blocks, 4 token blocks]

struct TileCtx {
    __amdgpu_buffer_rsrc_t wres;  // this wave's 64 weight rows (k origin at the part's start)
    __amdgpu_buffer_rsrc_t tres;  // gate/up: x; down: this wave's 64 rows of h
    uint32_t wo[2];               // lane byte offsets into the weight rows, groups j with bit 1 clear / set
    uint32_t to[8];               // gate/up: lane byte offsets of its 8 token rows; down: to[0..1] like wo
    int wstride;                  // bytes between 8-row weight groups
    int tstride;                  // down: bytes between 8-row token groups; 0 for gate/up
    int dma;                      // uint4 offset of this wave's first copy group in a buffer
    int rd[4];                    // per (half of the block, k16 half): fragment index in weight block 0
    int rdt;                      // uint4 distance from weight block 0 to token block 0
    uint32_t pfo;                 // lane byte offset of its prefetch, weight row `lane`
};

// Weight block j of this wave (uint4 offset from block 0).  Gate/up: blocks 0,
// 1 are w1 rows, 2, 3 the same rows of w3 (LDS rows 128 on).
template <bool DUAL>
__device__ __forceinline__ constexpr int wblk(int j) {
    return (DUAL ? ((j < 2 ? 0 : kTW / 2) + (j & 1) * 32) : j * 32) * kChunks;
}

// Copy j (0-7 weights, 8-15 tokens) of a block: one wave instruction fills
// one 8-row group (1 KB) of LDS, lane l at byte 16*l of it (row l/8).
template <bool DUAL>
__device__ __forceinline__ void copy_one(const TileCtx& c, uint4* __restrict__ buf, int k0, int j) {
    // address-space conversion needs a C-style cast
    if (j < 8) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.wres, (lptr_t)(buf + c.dma + j * kGroupVec), 16,
                                                 c.wo[(j >> 1) & 1], j * c.wstride + 2 * k0, 0, 0);
    } else {
        const int jj = j - 8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.tres, (lptr_t)(buf + kTW * kChunks + c.dma + jj * kGroupVec),
                                                 16, DUAL ? c.to[jj] : c.to[(jj >> 1) & 1],
                                                 DUAL ? 2 * k0 : jj * c.tstride + 2 * k0, 0, 0);
    }
}

// Fragments of half s (k 32s .. 32s+31) of the block in `buf`.
template <bool DUAL>
__device__ __forceinline__ void read_half(const TileCtx& c, const uint4* __restrict__ buf, int s, Frag16& f) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4* p = buf + c.rd[2 * s + h];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[8 * h + j] = __builtin_bit_cast(u32x4_t, p[wblk<DUAL>(j)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[8 * h + 4 + i] = __builtin_bit_cast(u32x4_t, p[c.rdt + i * 32 * kChunks]);
    }
}

__device__ __forceinline__ void mfma_half(const Frag16& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(f[8 * h + j]),
                                                                    as_bf16x8(f[8 * h + 4 + i]), acc[j][i], 0, 0, 0);
}

constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;

// 32 MFMAs with, after every second one, a fragment read (READ), and the
// block's 16 copies (COPY): one per two MFMAs over the stage (SPREAD, gate/up)
// or one after each of the first 16 MFMAs (down).  Every copy must land by
// the next block's barrier, so a copy issued late in the stage has less of a
// block to land in.  Measured on MI355X: the down projection, whose copies come
// from HBM, runs 3-4% faster front-loaded; gate/up runs 6% slower (its issue
// stalls on the vector-memory queue when the copies bunch up).
template <bool READ, bool COPY, bool SPREAD = true>
__device__ __forceinline__ void sched_half() {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (COPY && !SPREAD && u < 8) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
        if (READ) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (COPY && SPREAD) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
        if (COPY && !SPREAD && u < 8) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Weight-line prefetch: at the end of block kb each wave also loads one dword
// from each of its 64 weight rows in block kb + 3 (a 128-byte line per row),
// which brings that block's weight lines into L2 a block before they are
// copied.  w2 and h do not fit the MALL together, so every down tile waits on
// HBM for its copies and prefetches.  In gate/up (its gathered x fits the
// MALL) only the first token tile of each weight column prefetches: it is the
// one that reads the column's weights from HBM, the later tiles of the column
// find them in L2, and a prefetch there is only one more load in flight.
constexpr int kPrefetchAhead = 3;
template <bool DUAL>
constexpr bool kPrefetch = !DUAL;

// Block kb (in `cur`) as two 32-k stages.  On entry its first half's fragments
// are in f0 and, for every wave, the block is complete in `cur`.
//   first half : read the second half's fragments into f1; MFMAs on f0.
//   second half: (NEXT) barrier - block kb+1 (copied one block ago) has landed
//                and every wave has read all of `cur` - then (COPY) copy block
//                kb+2 into `cur` and read block kb+1's first half into f0 from
//                `nxt`; MFMAs on f1.
//   then       : (PF, prefetching tiles) the prefetch of block kb + 3 into pf, after a
//                scheduling fence, so it is the wave's last memory operation.
// The barrier waits for block kb+1's copies, issued a block earlier: for every
// outstanding vector-memory operation (vmcnt 0), or (PFWAIT) for all but the
// last one, the prefetch issued after those copies.  A prefetch's register is
// written two blocks after its load (the load of block kb - 2 has completed by
// block kb's barrier); CONSUME marks it as read there, so the compiler keeps
// the load and never has to wait for it.
template <bool DUAL, bool ACTIVE, bool COPY, bool NEXT, bool PFWAIT = false, bool CONSUME = false, bool PF = false,
          bool PFON = kPrefetch<DUAL>>
__device__ __forceinline__ void block_step(const TileCtx& c, uint4* __restrict__ cur, const uint4* __restrict__ nxt,
                                           int kb, int nb, Frag16& f0, Frag16& f1, f32x16_t (&acc)[4][4],
                                           uint32_t& pf) {
    constexpr bool kPf = PFON;
    if (ACTIVE) {
        read_half<DUAL>(c, cur, 1, f1);
        mfma_half(f0, acc);
        sched_half<true, false>();
    }
    if (NEXT) block_barrier<(kPf && PFWAIT) ? 1 : 0>();
    if (kPf && CONSUME) asm volatile("" ::"v"(pf));
    if (COPY) {
#pragma unroll
        for (int j = 0; j < kCopies; ++j) copy_one<DUAL>(c, cur, (kb + 2) * kBK, j);
    }
    if (ACTIVE) {
        if (NEXT) read_half<DUAL>(c, nxt, 0, f0);
        mfma_half(f1, acc);
        sched_half<NEXT, COPY, DUAL>();
    }
    if (kPf && PF) {
        __builtin_amdgcn_sched_barrier(0);
        pf = __builtin_amdgcn_raw_buffer_load_b32(c.wres, c.pfo, 2 * min(kb + kPrefetchAhead, nb - 1) * kBK, 0);
    }
}

// The K loop over nb blocks (nb a multiple of 4, >= 4).  Before it: blocks 0
// and 1 are being copied into b0 and b1, the weights of both first, then the
// tokens of block 0, then those of block 1.  Blocks 0 and 1 are peeled: no
// prefetch is outstanding at block 0's barrier, and none is consumed before
// block 2.  PFON: this tile prefetches its weight lines.
template <bool DUAL, bool ACTIVE, bool PFON = kPrefetch<DUAL>>
__device__ __forceinline__ void main_loop(const TileCtx& c, uint4* b0, uint4* b1, int nb, f32x16_t (&acc)[4][4]) {
    block_barrier<kCopies / 2>();  // block 0 has landed (block 1's token copies may not have)
    Frag16 f0, f1;
    uint32_t pf0 = 0, pf1 = 0;  // prefetch registers of the even and the odd blocks
    if (ACTIVE) read_half<DUAL>(c, b0, 0, f0);
    block_step<DUAL, ACTIVE, true, true, false, false, true, PFON>(c, b0, b1, 0, nb, f0, f1, acc, pf0);
    block_step<DUAL, ACTIVE, true, true, true, false, true, PFON>(c, b1, b0, 1, nb, f0, f1, acc, pf1);
    int kb = 2;
    while (kb < nb - 2) {
        block_step<DUAL, ACTIVE, true, true, true, true, true, PFON>(c, b0, b1, kb, nb, f0, f1, acc, pf0);
        block_step<DUAL, ACTIVE, true, true, true, true, true, PFON>(c, b1, b0, kb + 1, nb, f0, f1, acc, pf1);
        kb += 2;
    }
    // the barrier of block nb - 2 waits for everything: the last prefetch is
    // consumed only after the loop, so the compiler may sink it past that
    // barrier (the weights are restrict-qualified)
    block_step<DUAL, ACTIVE, false, true, false, true, false, PFON>(c, b0, b1, kb, nb, f0, f1, acc, pf0);
    block_step<DUAL, ACTIVE, false, false, false, false, false, PFON>(c, b1, b0, kb + 1, nb, f0, f1, acc, pf1);
    if (PFON) asm volatile("" ::"v"(pf1));
}

// ---- Down projection with three token buffers.  LDS (160 KB) holds two
// weight buffers W0, W1 and three token buffers T0-T2 of 32 KB each; block kb
// takes W[kb % 2] and T[kb % 3].  At block kb's barrier both of its buffers
// are free: the weights of block kb + 2 and the tokens of block kb + 3 are
// copied into them, so the token rows (h, from HBM) have two blocks to land
// and the weight rows one (their lines were brought into L2 by the prefetch).
constexpr int kHalfVec = kTW * kChunks;  // uint4 of one 32 KB buffer (256 rows of one operand)
static_assert(5 * kHalfVec <= 2 * kLdsVec, "two weight and three token buffers fit the LDS");

__device__ __forceinline__ void read_half_t3(const TileCtx& c, const uint4* __restrict__ wbuf,
                                             const uint4* __restrict__ tbuf, int s, Frag16& f) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4* pw = wbuf + c.rd[2 * s + h];
        const uint4* pt = tbuf + (c.rdt - kHalfVec) + c.rd[2 * s + h];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[8 * h + j] = __builtin_bit_cast(u32x4_t, pw[wblk<false>(j)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[8 * h + 4 + i] = __builtin_bit_cast(u32x4_t, pt[i * 32 * kChunks]);
    }
}

// token copy jj (8-row group) of the block at k0 into the token buffer tbuf
__device__ __forceinline__ void copy_t_t3(const TileCtx& c, uint4* __restrict__ tbuf, int k0, int jj) {
    // address-space conversion needs a C-style cast
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.tres, (lptr_t)(tbuf + c.dma + jj * kGroupVec), 16,
                                             c.to[(jj >> 1) & 1], jj * c.tstride + 2 * k0, 0, 0);
}

// Block kb: as block_step, with the barrier leaving the N youngest vector-
// memory operations in flight, then (WCOPY) the weight copies of block kb + 2
// into wcur and (TCOPY) the token copies of block kb + 3 into tcur.
template <bool ACTIVE, bool WCOPY, bool TCOPY, bool NEXT, int N, bool CONSUME, bool PF>
__device__ __forceinline__ void block_step_t3(const TileCtx& c, uint4* __restrict__ wcur,
                                              const uint4* __restrict__ wnxt, uint4* __restrict__ tcur,
                                              const uint4* __restrict__ tnxt, int kb, int nb, Frag16& f0,
                                              Frag16& f1, f32x16_t (&acc)[4][4], uint32_t& pf) {
    if (ACTIVE) {
        read_half_t3(c, wcur, tcur, 1, f1);
        mfma_half(f0, acc);
        sched_half<true, false>();
    }
    if (NEXT) block_barrier<N>();
    if (CONSUME) asm volatile("" ::"v"(pf));
    if (WCOPY) {
#pragma unroll
        for (int j = 0; j < 8; ++j) copy_one<false>(c, wcur, (kb + 2) * kBK, j);
    }
    if (TCOPY) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) copy_t_t3(c, tcur, (kb + 3) * kBK, jj);
    }
    if (ACTIVE) {
        if (NEXT) read_half_t3(c, wnxt, tnxt, 0, f0);
        mfma_half(f1, acc);
        sched_half<NEXT, WCOPY, false>();
    }
    if (PF) {
        __builtin_amdgcn_sched_barrier(0);
        pf = __builtin_amdgcn_raw_buffer_load_b32(c.wres, c.pfo, 2 * min(kb + kPrefetchAhead, nb - 1) * kBK, 0);
    }
}

// The K loop of a full down tile (nb a multiple of 4, >= 4).  Before it: the
// weight copies of blocks 0 and 1 into W0 and W1.  After the token copies of
// blocks 0-2 a prefetch (of block 2's weight lines) goes out too, so that at
// every barrier of the loop the youngest 9 operations (8 token copies and a
// prefetch) are the ones that may stay in flight.
template <bool ACTIVE>
__device__ __forceinline__ void main_loop_t3(const TileCtx& c, uint4* lds, int nb, f32x16_t (&acc)[4][4]) {
    uint4* const W0 = lds;
    uint4* const W1 = lds + kHalfVec;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) copy_t_t3(c, lds + 2 * kHalfVec, 0, jj);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) copy_t_t3(c, lds + 3 * kHalfVec, kBK, jj);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) copy_t_t3(c, lds + 4 * kHalfVec, 2 * kBK, jj);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pf0 = 0;  // prefetch registers of the even and the odd blocks
    uint32_t pf1 = __builtin_amdgcn_raw_buffer_load_b32(c.wres, c.pfo, 2 * min(2, nb - 1) * kBK, 0);
    block_barrier<17>();  // block 0 (and the weights of block 1) have landed
    Frag16 f0, f1;
    uint4* ta = lds + 2 * kHalfVec;  // T[kb % 3]
    uint4* tb = lds + 3 * kHalfVec;  // T[(kb + 1) % 3]
    uint4* tc = lds + 4 * kHalfVec;  // T[(kb + 2) % 3]
    if (ACTIVE) read_half_t3(c, W0, ta, 0, f0);
    int kb = 0;
    while (kb <= nb - 5) {
        block_step_t3<ACTIVE, true, true, true, 9, true, true>(c, W0, W1, ta, tb, kb, nb, f0, f1, acc, pf0);
        block_step_t3<ACTIVE, true, true, true, 9, true, true>(c, W1, W0, tb, tc, kb + 1, nb, f0, f1, acc, pf1);
        uint4* const t = ta;
        ta = tc;
        tc = tb;
        tb = t;
        kb += 2;
    }
    // kb = nb - 4: the last token copies (block nb - 1), then the last weight
    // copies (with no prefetch: its block is being copied), then the barrier
    // of block nb - 2 waits for everything.  A prefetch consumed only after
    // the loop could be sunk past that barrier by the compiler (the weights
    // are restrict-qualified), so none is left in flight there.
    block_step_t3<ACTIVE, true, true, true, 9, true, true>(c, W0, W1, ta, tb, kb, nb, f0, f1, acc, pf0);
    block_step_t3<ACTIVE, true, false, true, 9, true, false>(c, W1, W0, tb, tc, kb + 1, nb, f0, f1, acc, pf1);
    block_step_t3<ACTIVE, false, false, true, 0, true, false>(c, W0, W1, tc, ta, kb + 2, nb, f0, f1, acc, pf0);
    block_step_t3<ACTIVE, false, false, false, 0, false, false>(c, W1, W0, ta, tb, kb + 3, nb, f0, f1, acc, pf1);
}

// ---- Narrow tiles.  An expert's last token tile often holds few real rows
// (its count just past a multiple of 256).  In the layout above the waves
// with any real row still run their whole 128 x 128 block of MFMAs, so such a
// tile costs about as much as a full one.  A narrow tile keeps the 256 weight
// rows but takes TN = 32 * TB token rows (TB = 2 or 4), and the four waves
// split the weight rows instead: wave w owns LDS weight rows 32w.. and
// 128 + 32w.. (gate/up: the same 32 rows f of w1 and of w3) or 64w .. 64w + 63
// (down), against all TN token rows: 2 x TB blocks of 32 x 32, a quarter or
// half of a full tile's MFMAs.  The weight copies are the full tile's; each
// wave copies TN / 4 token rows.
// (A plain struct: the host pass of hipcc rejects a class template holding a
// buffer resource when it is passed on to a templated device function.)
struct NarrowCtx {
    __amdgpu_buffer_rsrc_t tres;
    uint32_t to[4];   // lane byte offsets of token copy group jj (TB of them)
    int tstride;      // down: bytes between 8-row token groups; 0 for gate/up
    int dmat;         // uint4 offset of this wave's first token copy group (token half)
    int rd[4];        // per (half of the block, k16 half): fragment index of the lane's row in a block
    int wb[2];        // uint4 offset of this wave's two weight blocks
};

template <bool DUAL, int TB>
__device__ __forceinline__ void copy_narrow(const TileCtx& c, const NarrowCtx& n, uint4* __restrict__ buf,
                                            int k0, int j) {
    if (j < 8) {
        copy_one<DUAL>(c, buf, k0, j);
    } else {
        const int jj = j - 8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(n.tres, (lptr_t)(buf + kTW * kChunks + n.dmat + jj * kGroupVec),
                                                 16, n.to[jj], DUAL ? 2 * k0 : jj * n.tstride + 2 * k0, 0, 0);
    }
}

// Fragments of half s of the block: [k16 half h][2 weight blocks, TB token blocks]
template <int TB>
__device__ __forceinline__ void read_narrow(const NarrowCtx& n, const uint4* __restrict__ buf, int s,
                                            u32x4_t (&f)[2 * (2 + TB)]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4* p = buf + n.rd[2 * s + h];
#pragma unroll
        for (int b = 0; b < 2; ++b) f[h * (2 + TB) + b] = __builtin_bit_cast(u32x4_t, p[n.wb[b]]);
#pragma unroll
        for (int i = 0; i < TB; ++i)
            f[h * (2 + TB) + 2 + i] = __builtin_bit_cast(u32x4_t, p[(kTW + 32 * i) * kChunks]);
    }
}

template <int TB>
__device__ __forceinline__ void mfma_narrow(const u32x4_t (&f)[2 * (2 + TB)], f32x16_t (&acc)[2][TB]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < TB; ++i)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[b][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(f[h * (2 + TB) + b]), as_bf16x8(f[h * (2 + TB) + 2 + i]), acc[b][i], 0, 0, 0);
}

// 4 * TB MFMAs, each followed by its share of the stage's fragment reads
// (READ) and of NC copies (FRONT: the copies over the first half of the
// MFMAs, as the full tiles of the down projection do).
template <int TB, bool READ, int NC, int U, bool FRONT = false>
__device__ __forceinline__ void sched_narrow_unit() {
    constexpr int kM = 4 * TB;
    constexpr int kR = (U + 1) * 2 * (2 + TB) / kM - U * 2 * (2 + TB) / kM;
    constexpr int kMc = FRONT ? kM / 2 : kM;
    constexpr int kC = U < kMc ? (U + 1) * NC / kMc - U * NC / kMc : 0;
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (READ && kR > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kR, 0);
    if constexpr (kC > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmem, kC, 0);
}

template <int TB, bool READ, int NC, bool FRONT, int... U>
__device__ __forceinline__ void sched_narrow_seq(std::integer_sequence<int, U...>) {
    (sched_narrow_unit<TB, READ, NC, U, FRONT>(), ...);
    __builtin_amdgcn_sched_barrier(0);
}

template <int TB, bool READ, int NC, bool FRONT = false>
__device__ __forceinline__ void sched_narrow() {
    sched_narrow_seq<TB, READ, NC, FRONT>(std::make_integer_sequence<int, 4 * TB>{});
}

// uint4 of one 64-k block of a narrow tile (weight rows, then its token rows)
template <int TB>
constexpr int kNarrowVec = (kTW + 32 * TB) * kChunks;

// block_step for a narrow tile (every wave is active).  A narrow block is SUB
// consecutive 64-k blocks (SUB = 1 or 2), stored one after the other in the
// buffer, consumed as 2 * SUB stages of 32 k; the barrier and the next
// block's copies come before the last stage.  Narrow tiles do a quarter or
// half of a full tile's MFMAs per block, so with one 64-k block in flight they
// wait on the copies' latency; SUB = 2 keeps twice the bytes in flight.
template <bool DUAL, int TB, int SUB, bool COPY, bool NEXT>
__device__ __forceinline__ void narrow_step(const TileCtx& c, const NarrowCtx& n, uint4* __restrict__ cur,
                                            const uint4* __restrict__ nxt, int kb, u32x4_t (&f0)[2 * (2 + TB)],
                                            u32x4_t (&f1)[2 * (2 + TB)], f32x16_t (&acc)[2][TB]) {
    read_narrow<TB>(n, cur, 1, f1);
    mfma_narrow<TB>(f0, acc);
    sched_narrow<TB, true, 0>();
    if constexpr (SUB == 2) {
        read_narrow<TB>(n, cur + kNarrowVec<TB>, 0, f0);
        mfma_narrow<TB>(f1, acc);
        sched_narrow<TB, true, 0>();
        read_narrow<TB>(n, cur + kNarrowVec<TB>, 1, f1);
        mfma_narrow<TB>(f0, acc);
        sched_narrow<TB, true, 0>();
    }
    if (NEXT) block_barrier<0>();
    if (COPY) {
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
            for (int j = 0; j < 8 + TB; ++j)
                copy_narrow<DUAL, TB>(c, n, cur + sb * kNarrowVec<TB>, ((kb + 2) * SUB + sb) * kBK, j);
    }
    if (NEXT) read_narrow<TB>(n, nxt, 0, f0);
    mfma_narrow<TB>(f1, acc);
    sched_narrow<TB, NEXT, COPY ? SUB * (8 + TB) : 0, !DUAL>();  // the down projection front-loads its copies
}

// The whole narrow tile: copies, K loop, epilogue.  Gate/up also writes zeros
// to the segment's rows past the TN token rows (its padding rows), in the
// tile's 128 columns of h.
template <bool DUAL, int TB, int SUB>
__device__ __forceinline__ void narrow_tile(const TileCtx& c, const bf16_t* __restrict__ act,
                                            const int32_t* __restrict__ row_src, void* __restrict__ out,
                                            uint4* b0, uint4* b1, int kpart, int kbase, int ld_act, int ld_out,
                                            int n_src, int topk, int wt, int p0, int valid, int row_end) {
    constexpr int TN = 32 * TB;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = lane & 31;
    const int fk = lane >> 5;
    const int rl = lane >> 3;

    // token copy group jj of wave w fills token rows r = w * TN/4 + 8 jj + l/8.
    // As in the full tile: the row loads, then the weight copies of blocks 0
    // and 1, which do not wait for them.
    const int r0 = wave * (TN / 4);
    int srcs[TB];
    if (DUAL) {
#pragma unroll
        for (int jj = 0; jj < TB; ++jj) srcs[jj] = row_src[p0 + min(r0 + 8 * jj + rl, valid - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int j = 0; j < 8; ++j) copy_one<DUAL>(c, b0 + sb * kNarrowVec<TB>, sb * kBK, j);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int j = 0; j < 8; ++j) copy_one<DUAL>(c, b1 + sb * kNarrowVec<TB>, (SUB + sb) * kBK, j);

    NarrowCtx n;
    {
        // bit 4 of r (the only bit of g(r) above the row-in-group bits) is fixed per group
        const int ch0 = (lane & 7) ^ swz(rl);
        const int ch1 = (lane & 7) ^ swz(16 + rl);
        if (DUAL) {
            n.tres = make_rsrc(act + kbase);
#pragma unroll
            for (int jj = 0; jj < TB; ++jj) {
                int src = srcs[jj];
                if (src < 0 || src >= n_src) src = 0;
                const int ch = (((r0 + 8 * jj) >> 4) & 1) ? ch1 : ch0;
                n.to[jj] = static_cast<uint32_t>(
                    (static_cast<size_t>(div_topk(static_cast<uint32_t>(src), topk)) * ld_act + 8 * ch) * 2);
            }
            n.tstride = 0;
        } else {
            // rows p0 + r0 .. + TN/4 of h, inside the expert's padded segment
            n.tres = make_rsrc(act + static_cast<size_t>(p0 + r0) * ld_act + kbase);
#pragma unroll
            for (int jj = 0; jj < TB; ++jj) {
                const int ch = (((r0 + 8 * jj) >> 4) & 1) ? ch1 : ch0;
                n.to[jj] = (static_cast<uint32_t>(rl) * ld_act + 8u * ch) * 2u;
            }
            n.tstride = 8 * ld_act * 2;
        }
        n.dmat = r0 * kChunks;
#pragma unroll
        for (int q = 0; q < 4; ++q) n.rd[q] = fr * kChunks + ((2 * q + fk) ^ swz(fr));
        n.wb[0] = (DUAL ? 32 * wave : 64 * wave) * kChunks;
        n.wb[1] = (DUAL ? kTW / 2 + 32 * wave : 64 * wave + 32) * kChunks;
    }

    f32x16_t acc[2][TB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < TB; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[b][i][q] = 0.0f;

    const int nb = kpart / (SUB * kBK);  // even and >= 4 (the caller picks SUB so)
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int j = 8; j < 8 + TB; ++j) copy_narrow<DUAL, TB>(c, n, b0 + sb * kNarrowVec<TB>, sb * kBK, j);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int j = 8; j < 8 + TB; ++j) copy_narrow<DUAL, TB>(c, n, b1 + sb * kNarrowVec<TB>, (SUB + sb) * kBK, j);
    block_barrier<SUB * TB>();  // block 0 has landed (block 1's token copies may not have)
    u32x4_t f0[2 * (2 + TB)], f1[2 * (2 + TB)];
    read_narrow<TB>(n, b0, 0, f0);
    int kb = 0;
    do {
        narrow_step<DUAL, TB, SUB, true, true>(c, n, b0, b1, kb, f0, f1, acc);
        narrow_step<DUAL, TB, SUB, true, true>(c, n, b1, b0, kb + 1, f0, f1, acc);
        kb += 2;
    } while (kb < nb - 2);
    narrow_step<DUAL, TB, SUB, false, true>(c, n, b0, b1, kb, f0, f1, acc);
    narrow_step<DUAL, TB, SUB, false, false>(c, n, b1, b0, kb + 1, f0, f1, acc);

    // epilogue (32x32 C layout as in the full tile)
#pragma unroll
    for (int i = 0; i < TB; ++i) {
        const int rt = 32 * i + fr;
        const int p = p0 + rt;
        if (p >= row_end) continue;
        const bool real = rt < valid;
        if (DUAL) {
            bf16_t* hrow = static_cast<bf16_t*>(out) + static_cast<size_t>(p) * ld_out;
            const int fb = wt * (kTW / 2) + 32 * wave;
            const uint32_t keep = real ? 0xffffffffu : 0u;
            uint2 o[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float hv = silu_f32(acc[0][i][4 * q4 + u]) * acc[1][i][4 * q4 + u];
                    v[u] = __uint_as_float(__float_as_uint(hv) & keep);
                }
                o[q4].x = pack_bf16x2(v[0], v[1]);
                o[q4].y = pack_bf16x2(v[2], v[3]);
            }
            // 16-byte stores after a permlane32 swap, as in the full tile
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const auto sx = __builtin_amdgcn_permlane32_swap(o[2 * pr].x, o[2 * pr + 1].x, false, false);
                const auto sy = __builtin_amdgcn_permlane32_swap(o[2 * pr].y, o[2 * pr + 1].y, false, false);
                *reinterpret_cast<uint4*>(hrow + fb + 8 * (2 * pr + fk)) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
            }
        } else {
            if (!real) continue;
            float* yrow = static_cast<float*>(out) + static_cast<size_t>(p) * ld_out;
            const int jb = wt * kTW + 64 * wave;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    f32x4_t v = {acc[b][i][4 * q4], acc[b][i][4 * q4 + 1], acc[b][i][4 * q4 + 2],
                                 acc[b][i][4 * q4 + 3]};
                    *reinterpret_cast<f32x4_t*>(yrow + jb + 32 * b + 8 * q4 + 4 * fk) = v;
                }
        }
    }
    if (DUAL) {
        // padding rows p0 + TN .. of the segment: 128 columns of zeros (16 x 16 bytes) each
        const int z0 = p0 + TN;
        const int z1 = min(p0 + kTT, row_end);
        for (int q = tid; q < (z1 - z0) * 16; q += 256) {
            bf16_t* hrow = static_cast<bf16_t*>(out) + static_cast<size_t>(z0 + (q >> 4)) * ld_out;
            *reinterpret_cast<uint4*>(hrow + wt * (kTW / 2) + 8 * (q & 15)) = make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

// ---- Which tile a workgroup computes.  Workgroup b runs on XCD b % 8 and is
// that XCD's (b / 8)-th; an XCD's workgroups are dispatched in that order to
// its 32 CUs.  Both schemes below enumerate only the tiles the segments hold.
// Within one expert the tiles of a set of weight tiles are taken in groups of
// gn weight tiles x all of the expert's ntt token tiles, token-major, with
// gn ~ 32 / ntt: the ~32 tiles an XCD runs at once then read the same few
// weight and token tiles, so each k-slice comes from HBM once and from the
// XCD's L2 after that (measured on MI355X: with every tile's data L2-resident
// the kernels ran 16% (gate/up) and 35% (down) faster than with an order that
// let a round straddle two experts).
struct TileId {
    int split, e, ttl, wt;
    int seg, seg_end, cnt;  // the expert's segment: offsets[e], offsets[e + 1], counts[e]
};

// Down projection: XCD x takes the x-th of 8 equal contiguous runs of the
// expert-major enumeration (K part, expert, group).  The token side (h rows,
// 28 KB each) is then read by one or two XCDs only.  The expert is found
// across the expert lanes (prefix sum and ballot).
__device__ __forceinline__ bool tile_contiguous(const LaneSeg& s, int n_wt, int ksplit, int tail_rows, TileId& t) {
    const int ntt = token_tiles(s.end - s.off, s.cnt, tail_rows);  // 0 for an empty segment
    const int w = ntt * n_wt;
    const int ps = expert_prefix(w);
    const int per_split = __builtin_amdgcn_readlane(ps, 15);
    const int total = per_split * ksplit;
    const int run = (total + 7) >> 3;
    if (static_cast<int>(blockIdx.x >> 3) >= run) return false;
    const int L_all = (blockIdx.x & 7) * run + (blockIdx.x >> 3);
    if (L_all >= total) return false;
    t.split = L_all / per_split;
    int L = L_all - t.split * per_split;
    const int h = expert_holding(ps, L);
    if (h < 0) return false;
    L -= __builtin_amdgcn_readlane(ps - w, h);
    t.e = h;
    t.seg = __builtin_amdgcn_readlane(s.off, h);
    t.seg_end = __builtin_amdgcn_readlane(s.end, h);
    t.cnt = __builtin_amdgcn_readlane(s.cnt, h);
    const int nt = __builtin_amdgcn_readlane(ntt, h);
    const int gn = max(1, min(n_wt, kXcdTiles / nt));
    const int g = L / (gn * nt);
    const int rem = L - g * gn * nt;
    const int gw = min(gn, n_wt - g * gn);  // the last group may be narrower
    t.ttl = rem / gw;
    t.wt = g * gn + (rem - t.ttl * gw);
    return true;
}

// Gate/up: the weight tiles ("columns", numbered c = (K part * n_exp + e) *
// n_wt + wt) are dealt to the XCDs, column c to XCD c % 8, each with all of
// its expert's token tiles.  Every XCD then gets the same mix of every
// expert's tiles, so the narrow tiles of the experts with short tails (cheaper
// than full ones) are spread evenly: with contiguous runs, half of the XCDs
// got none of them and ran 15% more full tiles than the others.  A column's
// tiles stay on one XCD, so the weights keep their L2 reuse; the gathered
// token rows (x is 32 MB) are read by every XCD.  An XCD holds at most
// ceil(n_wt / 8) columns of an expert: its count exceeds total / 8 by at most
// the number of token tiles, which the grid allows for.  ksplit <= 2.  Lane
// j < 32 stands for (K part j / 16, expert j % 16) and holds that pair's tile
// count on this XCD; a prefix sum over those lanes and a ballot find the pair
// that holds the workgroup's tile.  Gate/up keeps every token tile (its short
// tails run as narrow tiles).
__device__ __forceinline__ bool tile_by_column(const LaneSeg& s, int n_exp, int n_wt, int ksplit, TileId& t) {
    const int lane = threadIdx.x & 63;
    const int x = blockIdx.x & 7;
    const int i = blockIdx.x >> 3;
    const int sp = lane >> 4;
    const int e = lane & 15;
    int ntt = 0, f = 0, kk = 0;
    if (sp < ksplit && e < n_exp) {
        ntt = (s.end - s.off) / kTT;
        f = (x - (((sp * n_exp + e) * n_wt) & 7) + 8) & 7;  // this XCD's first weight tile
        kk = f < n_wt ? ((n_wt - 1 - f) >> 3) + 1 : 0;     // its weight tiles of expert e
    }
    const int w = kk * ntt;
    int ps = w;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        const int u = __shfl_up(ps, o, 64);
        if (lane >= o) ps += u;
    }
    const uint64_t hit = __ballot(lane < 32 && ps > i);
    if (hit == 0) return false;
    const int h = static_cast<int>(__builtin_ctzll(hit));
    const int li = i - __builtin_amdgcn_readlane(ps - w, h);
    t.split = h >> 4;
    t.e = h & 15;
    t.seg = __builtin_amdgcn_readlane(s.off, h);
    t.seg_end = __builtin_amdgcn_readlane(s.end, h);
    t.cnt = __builtin_amdgcn_readlane(s.cnt, h);
    const int nt = __builtin_amdgcn_readlane(ntt, h);
    const int first = __builtin_amdgcn_readlane(f, h);
    const int k = __builtin_amdgcn_readlane(kk, h);
    const int gn = max(1, min(k, kXcdTiles / nt));
    const int g = li / (gn * nt);
    const int rem = li - g * gn * nt;
    const int gw = min(gn, k - g * gn);
    t.ttl = rem / gw;
    t.wt = first + 8 * (g * gn + (rem - t.ttl * gw));
    return true;
}

// PREACT (with DUAL): store the pre-activations a1 = w1 . x and a3 = w3 . x
// in fp32 (out [P, 2 Nw]: a1 in columns 0..Nw-1, a3 after, in the 32 x 32
// blocks of preact_block) instead of h, for the backward pass.
template <bool DUAL, bool PREACT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void tiled_kernel(
    const bf16_t* __restrict__ act, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const bf16_t* __restrict__ wa, const bf16_t* __restrict__ wb, void* __restrict__ out,
    int Kdim, int Nw /* weight rows per expert (F or d) */, int ld_act, int n_wt,
    int ld_out, int n_src, int P, int ksplit, size_t split_stride, int n_exp, int topk, int tail_rows) {
    __shared__ uint4 lds[2 * kLdsVec];
    uint4* const b0 = lds;
    uint4* const b1 = lds + kLdsVec;

    // ---- tile of this workgroup (the grid covers the worst case; spare
    // workgroups exit here)
    TileId t;
    {
        const LaneSeg ls = lane_segment(offsets, counts, n_exp);
        if constexpr (DUAL) {
            // gate/up launches pass no tail_rows
            if (!tile_by_column(ls, n_exp, n_wt, ksplit, t)) return;
        } else {
            // down projection: ksplit is the largest K split allowed, the plan
            // picks the split and whether the short tails go to the streaming pass
            const DownPlan plan = down_plan(ls, n_wt, ksplit);
            ksplit = plan.ks;
            tail_rows = min(tail_rows, plan.tail_rows);
            if (!tile_contiguous(ls, n_wt, ksplit, tail_rows, t)) return;
        }
    }
    const int split = t.split, e = t.e, ttl = t.ttl, wt = t.wt;
    const int kpart = Kdim / ksplit;
    const int kbase = split * kpart;
    out = static_cast<char*>(out) + split * split_stride * (DUAL && !PREACT ? sizeof(bf16_t) : sizeof(float));

    const int p0 = t.seg + ttl * kTT;
    const int row_end = min(t.seg_end, P);
    const int valid = min(min(kTT, t.seg + t.cnt - p0), row_end - p0);
    if (valid <= 0) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_w = wave & 1;
    const int wave_t = wave >> 1;
    const int fr = lane & 31;  // fragment row / token column of this lane
    const int fk = lane >> 5;  // k-group of this lane within a k16 half

    // Copies: wave w fills LDS rows w*64 .. +64 of the weight half and of the
    // token half as 8 groups of 8 rows; lane l of group j writes row
    // w*64 + 8j + l/8, physical chunk l%8, so it reads logical chunk
    // (l%8) ^ g(row).  g() of that row depends on l and on j's bit 1 only.
    const int rl = lane >> 3;
    const int ch0 = (lane & 7) ^ swz(rl);
    const int ch1 = (lane & 7) ^ swz(16 + rl);
    TileCtx c;
    {
        // Gate/up: LDS weight rows 0-127 (waves 0, 1) are w1 rows, 128-255
        // (waves 2, 3) the same rows of w3.
        const bf16_t* wm = (DUAL && wave >= 2) ? wb : wa;
        const int wrow = DUAL ? wt * (kTW / 2) + (wave & 1) * 64 : wt * kTW + wave * 64;
        c.wres = make_rsrc(wm + (static_cast<size_t>(e) * Nw + wrow) * Kdim + kbase);
        c.wo[0] = (static_cast<uint32_t>(rl) * Kdim + 8u * ch0) * 2u;
        c.wo[1] = (static_cast<uint32_t>(rl) * Kdim + 8u * ch1) * 2u;
        c.wstride = 8 * Kdim * 2;
        c.dma = wave * 64 * kChunks;
        c.pfo = static_cast<uint32_t>(lane) * Kdim * 2u;
    }

    if (!PREACT && valid <= 128) {
        // K parts are multiples of 256: kpart / 128 is even, and at least 4 from 512 on
        if (valid <= 64 && kpart >= 512)
            narrow_tile<DUAL, 2, 2>(c, act, row_src, out, b0, b1, kpart, kbase, ld_act, ld_out, n_src, topk, wt,
                                    p0, valid, row_end);
        else if (valid <= 64)
            narrow_tile<DUAL, 2, 1>(c, act, row_src, out, b0, b1, kpart, kbase, ld_act, ld_out, n_src, topk, wt,
                                    p0, valid, row_end);
        else
            narrow_tile<DUAL, 4, 1>(c, act, row_src, out, b0, b1, kpart, kbase, ld_act, ld_out, n_src, topk, wt,
                                    p0, valid, row_end);
        return;
    }

    // Gate/up: the rows of x this lane copies (padding rows copy the tile's
    // last real row).  The loads are unconditional, so all eight are in flight
    // at once, and they go out ahead of the weight copies of blocks 0 and 1,
    // which do not depend on them: waiting for these loads leaves the copies
    // in flight.
    int srcs[8];
    if (DUAL) {
#pragma unroll
        for (int j = 0; j < 8; ++j) srcs[j] = row_src[p0 + min(wave * 64 + 8 * j + rl, valid - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) copy_one<DUAL>(c, b0, 0, j);
#pragma unroll
    for (int j = 0; j < 8; ++j) copy_one<DUAL>(c, DUAL ? b1 : lds + kHalfVec, kBK, j);
    {
        if (DUAL) {
            c.tres = make_rsrc(act + kbase);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int src = srcs[j];
                if (src < 0 || src >= n_src) src = 0;
                c.to[j] = static_cast<uint32_t>(
                    (static_cast<size_t>(div_topk(static_cast<uint32_t>(src), topk)) * ld_act + 8 * (((j >> 1) & 1) ? ch1 : ch0)) * 2);
            }
            c.tstride = 0;
        } else {
            // the tile's 256 rows of h, padding rows included (all inside the
            // expert's padded segment, hence inside h)
            c.tres = make_rsrc(act + static_cast<size_t>(p0 + wave * 64) * ld_act + kbase);
            c.to[0] = (static_cast<uint32_t>(rl) * ld_act + 8u * ch0) * 2u;
            c.to[1] = (static_cast<uint32_t>(rl) * ld_act + 8u * ch1) * 2u;
#pragma unroll
            for (int j = 2; j < 8; ++j) c.to[j] = 0;
            c.tstride = 8 * ld_act * 2;
        }
        // Fragment reads: blocks start at multiples of 32 rows, so g() of a
        // block row is g(fr).  Logical chunk of half s, k16 half h: 4s + 2h + fk.
        const int row0 = wave_w * (DUAL ? 64 : 128) + fr;
#pragma unroll
        for (int q = 0; q < 4; ++q) c.rd[q] = row0 * kChunks + ((2 * q + fk) ^ swz(fr));
        c.rdt = (kTW + wave_t * 128 - wave_w * (DUAL ? 64 : 128)) * kChunks;
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.0f;

    const int nb = kpart / kBK;  // a multiple of 4, >= 4 (K parts are multiples of 256)
    if constexpr (DUAL) {
#pragma unroll
        for (int j = 8; j < kCopies; ++j) copy_one<DUAL>(c, b0, 0, j);
#pragma unroll
        for (int j = 8; j < kCopies; ++j) copy_one<DUAL>(c, b1, kBK, j);
    }
    // A wave whose 128 token rows are all padding skips its reads and MFMAs.
    // In gate/up the first token tile of a weight column prefetches its lines.
    const bool leader = DUAL && ttl == 0;
    if constexpr (!DUAL) {
        if (__builtin_amdgcn_readfirstlane(valid > wave_t * 128 ? 1 : 0) != 0)
            main_loop_t3<true>(c, lds, nb, acc);
        else
            main_loop_t3<false>(c, lds, nb, acc);
    } else {
        if (__builtin_amdgcn_readfirstlane(valid > wave_t * 128 ? 1 : 0) != 0) {
            if (leader) main_loop<DUAL, true, true>(c, b0, b1, nb, acc);
            else main_loop<DUAL, true>(c, b0, b1, nb, acc);
        } else {
            if (leader) main_loop<DUAL, false, true>(c, b0, b1, nb, acc);
            else main_loop<DUAL, false>(c, b0, b1, nb, acc);
        }
    }

    // ---- epilogue.  32x32 C layout: lane l holds token column l%32 and weight
    // rows 8*(q/4) + 4*(l/32) + q%4 of each block, q = 0..15.
    if (!DUAL) {
        // y_perm rows (tokens) of this wave, staged through LDS into row-
        // contiguous stores once every wave is done with the last block.  Its
        // padding rows get the (zero or padding-row) sums too: rows of a
        // segment past the expert's count are unspecified in y_perm.
        block_barrier<0>();
        store_rows_staged(acc, reinterpret_cast<f32x4_t*>((wave < 2 ? b0 : b1) + (wave & 1) * (kBufVec / 2)),
                          static_cast<float*>(out), ld_out, p0 + wave_t * 128, wt * kTW + wave_w * 128,
                          row_end - (p0 + wave_t * 128), lane);
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rt = wave_t * 128 + i * 32 + fr;  // token row within the tile
        const int p = p0 + rt;
        if (p >= row_end) continue;
        const bool real = rt < valid;
        if (DUAL && PREACT) {
            // a in 32 x 32 blocks (preact_block): this block's 16 values of
            // the lane are contiguous
            const int pb = (p0 + wave_t * 128 + i * 32) / 32;
            const int fbk = (wt * (kTW / 2) + wave_w * 64) / 32;
            const uint32_t keep = real ? 0xffffffffu : 0u;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float* a1b = static_cast<float*>(out) + preact_block(pb, fbk + jj, Nw) + lane * 16;
                float* a3b = static_cast<float*>(out) + preact_block(pb, fbk + jj + Nw / 32, Nw) + lane * 16;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    f32x4_t a1, a3;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        a1[u] = __uint_as_float(__float_as_uint(acc[jj][i][4 * q4 + u]) & keep);
                        a3[u] = __uint_as_float(__float_as_uint(acc[jj + 2][i][4 * q4 + u]) & keep);
                    }
                    *reinterpret_cast<f32x4_t*>(a1b + 4 * q4) = a1;
                    *reinterpret_cast<f32x4_t*>(a3b + 4 * q4) = a3;
                }
            }
        } else if (DUAL) {
            bf16_t* hrow = static_cast<bf16_t*>(out) + static_cast<size_t>(p) * ld_out;
            const int fb = wt * (kTW / 2) + wave_w * 64;
            // padding rows are written as zeros; a bit mask (not a branch or
            // a multiply) clears them, whatever their accumulators hold
            const uint32_t keep = real ? 0xffffffffu : 0u;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                uint2 o[4];  // the lane's 4 h values of each q4 (f = 8 q4 + 4 fk + u), bf16
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float hv = silu_f32(acc[jj][i][4 * q4 + u]) * acc[jj + 2][i][4 * q4 + u];
                        v[u] = __uint_as_float(__float_as_uint(hv) & keep);
                    }
                    o[q4].x = pack_bf16x2(v[0], v[1]);
                    o[q4].y = pack_bf16x2(v[2], v[3]);
                }
                // Lanes l and l + 32 hold the two halves of each 8-wide run of f
                // of the same row.  v_permlane32_swap hands lane l its partner's
                // half of the even runs and lane l + 32 lane l's half of the odd
                // ones (measured on gfx950), so each lane stores 16 bytes: run
                // 2 pr + fk, half the store instructions of 8-byte stores.
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const auto sx = __builtin_amdgcn_permlane32_swap(o[2 * pr].x, o[2 * pr + 1].x, false, false);
                    const auto sy = __builtin_amdgcn_permlane32_swap(o[2 * pr].y, o[2 * pr + 1].y, false, false);
                    *reinterpret_cast<uint4*>(hrow + fb + jj * 32 + 8 * (2 * pr + fk)) =
                        make_uint4(sx[0], sy[0], sx[1], sy[1]);
                }
            }
        } else {
            if (!real) continue;
            float* yrow = static_cast<float*>(out) + static_cast<size_t>(p) * ld_out;
            const int jb = wt * kTW + wave_w * 128;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    f32x4_t v = {acc[j][i][4 * q4], acc[j][i][4 * q4 + 1], acc[j][i][4 * q4 + 2],
                                 acc[j][i][4 * q4 + 3]};
                    *reinterpret_cast<f32x4_t*>(yrow + jb + j * 32 + 8 * q4 + 4 * fk) = v;
                }
        }
    }
}

}  // namespace

bool tiled_fits(const Shape& s) {
    return static_cast<unsigned long long>(s.T) * s.d * 2 + 2ull * s.d < (1ull << 32);
}

int tiled_down_ksplit(const Shape& s) {
    // Allow the down projection's K to be cut in two when the worst-case tiles
    // would not fill four rounds of the 256 CUs; down_plan takes the split on
    // the device only where it shortens the last round.
    const int P = s.T * s.K + s.n * (kTT - 1);
    const int n_tt = (P + kTT - 1) / kTT;
    const int n_wt = s.d / kTW;
    return (n_tt * n_wt < 4 * 256 && (s.F / 2) % (4 * kBK) == 0) ? 2 : 1;
}

hipError_t launch_tiled(const Shape& s, bool gate_up, const void* act, const int32_t* row_src,
                        const int32_t* counts, const int32_t* offsets, const void* wa, const void* wb,
                        void* out, hipStream_t st, int ksplit, int tail_rows) {
    if (!tiled_fits(s) || ksplit < 1 || ksplit > 2) return hipErrorInvalidValue;
    const int P = s.T * s.K + s.n * (kTT - 1);
    const int n_tt = (P + kTT - 1) / kTT;
    const int n_wt = gate_up ? s.F / (kTW / 2) : s.d / kTW;
    // gate/up: an XCD may hold up to n_tt * ksplit tiles more than an eighth
    const int G = ((n_tt * n_wt * ksplit + 7) / 8 + (gate_up ? n_tt * ksplit : 0)) * 8;
    const size_t split_stride = static_cast<size_t>(P) * (gate_up ? s.F : s.d);
    if (gate_up)
        tiled_kernel<true><<<G, 256, 0, st>>>(static_cast<const bf16_t*>(act), row_src, counts, offsets,
                                              static_cast<const bf16_t*>(wa), static_cast<const bf16_t*>(wb),
                                              out, s.d, s.F, s.d, n_wt, s.F, s.T * s.K, P,
                                              ksplit, split_stride, s.n, s.K, tail_rows);
    else
        tiled_kernel<false><<<G, 256, 0, st>>>(static_cast<const bf16_t*>(act), nullptr, counts, offsets,
                                               static_cast<const bf16_t*>(wa), nullptr, out, s.F, s.d, s.F,
                                               n_wt, s.d, s.T * s.K, P, ksplit, split_stride, s.n, s.K, tail_rows);
    return hipGetLastError();
}

hipError_t launch_tiled_preact(const Shape& s, const void* x, const int32_t* row_src, const int32_t* counts,
                               const int32_t* offsets, const void* w1, const void* w3, float* a, hipStream_t st) {
    if (!tiled_fits(s)) return hipErrorInvalidValue;
    const int P = s.T * s.K + s.n * (kTT - 1);
    const int n_tt = (P + kTT - 1) / kTT;
    const int n_wt = s.F / (kTW / 2);
    const int G = ((n_tt * n_wt + 7) / 8 + n_tt) * 8;
    tiled_kernel<true, true><<<G, 256, 0, st>>>(static_cast<const bf16_t*>(x), row_src, counts, offsets,
                                                static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w3), a,
                                                s.d, s.F, s.d, n_wt, 2 * s.F, s.T * s.K, P, 1, 0, s.n, s.K, 0);
    return hipGetLastError();
}

}  // namespace moe
