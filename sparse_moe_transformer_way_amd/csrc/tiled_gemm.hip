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
//   * K advances 32 per stage.  A stage is 256 weight rows + 256 token rows of
//     64 bytes = 32 KB, copied HBM/L2 -> LDS by global_load_lds_dwordx4 (no
//     register staging).  Four stage buffers form a ring with three stages in
//     flight; the loop is unrolled by four so that every copy and every LDS
//     read names one fixed buffer.  One barrier per stage.
//   * MFMA fragments are double-buffered in registers: the second k16 half of
//     a stage and the first half of the next stage are read while the MFMAs of
//     the previous half run.
//   * LDS rows are 4 chunks of 16 bytes; chunk c of row r sits at c ^ g(r) with
//     g(r) = (r2 ^ r3) | (r3 ^ r4) << 1 (bits of r).  gfx950's LDS has 64
//     banks; a 32-row fragment read (ds_read_b128) is served in 16-lane phases
//     (lanes 0-7 with 16-23, 8-15 with 24-31, measured with
//     SQ_LDS_BANK_CONFLICT), and this g gives each phase all 64 banks, as it
//     also does for 16 consecutive lanes.
//   * Tile order: workgroup b runs on XCD b % 8; each XCD gets a contiguous run
//     of tiles, enumerated as groups of GN weight tiles x all token tiles (token
//     tiles of one expert are adjacent), so the ~32 tiles an XCD runs at once
//     share a few weight tiles and a few token tiles in its L2.
//   * Padding rows of a token tile copy a real row (the copy cannot write
//     zeros); their outputs are masked in the epilogue.  A wave whose 128 token
//     rows are all padding skips its MFMAs.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kExperts = 8;
constexpr int kTW = 256;                     // weight rows per tile
constexpr int kTT = 256;                     // token rows per tile
constexpr int kBK = 32;                      // k per stage
constexpr int kChunks = kBK / 8;             // 16-byte chunks per LDS row
constexpr int kStageVec = (kTW + kTT) * kChunks;  // uint4 per stage (32 KB)
constexpr int kDmaPerStage = 8;              // global_load_lds per lane per stage

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

__device__ __forceinline__ int swz(int row) {
    return (((row >> 2) ^ (row >> 3)) & 1) | ((((row >> 3) ^ (row >> 4)) & 1) << 1);
}

__device__ __forceinline__ void dma16(const bf16_t* src, uint4* lds_wave_base) {
    // address-space conversions need C-style casts
    __builtin_amdgcn_global_load_lds((gptr_t)(src), (lptr_t)(lds_wave_base), 16, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding): at most N vector-memory operations of
// this wave outstanding and none of its LDS reads (lgkmcnt 0); export count not
// waited on.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier for the stage ring.  __syncthreads() carries a release
// fence that waits for every outstanding copy into LDS (vmcnt 0), which would
// drain the ring; here the caller waits for exactly the stage it needs, and the
// empty asm statements only stop the compiler from moving memory accesses
// across the barrier.
template <int N>
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(N));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int p) {
    int e = 0;
#pragma unroll
    for (int j = 1; j < kExperts; ++j) e = (p >= offsets[j]) ? j : e;
    return e;
}

struct Frags {
    uint4 a[4];  // weight blocks
    uint4 b[4];  // token blocks
};

template <bool DUAL>
struct TileCtx {
    const bf16_t* gw[4];  // this lane's 4 weight source rows (+ chunk offset)
    const bf16_t* gt[4];  // this lane's 4 token source rows (+ chunk offset)
    int dma_w;            // uint4 offset of this wave's first weight DMA block in a stage
    int dma_t;            // uint4 offset of this wave's first token DMA block in a stage
    int rd[2];            // per-lane uint4 offset of its fragment row/chunk, k16 half 0 / 1
    int wblk[4];          // weight block base rows (uint4 units, = row * kChunks)
    int tblk0;            // token block base (uint4 units)
};

template <bool DUAL>
__device__ __forceinline__ void issue_stage(const TileCtx<DUAL>& c, uint4* __restrict__ buf, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(c.gw[j] + k0, buf + c.dma_w + j * 16 * kChunks);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(c.gt[j] + k0, buf + c.dma_t + j * 16 * kChunks);
}

template <bool DUAL>
__device__ __forceinline__ void read_frags(const TileCtx<DUAL>& c, const uint4* __restrict__ buf, int half,
                                           Frags& f) {
    const uint4* p = buf + c.rd[half];
#pragma unroll
    for (int j = 0; j < 4; ++j) f.a[j] = p[c.wblk[j]];
#pragma unroll
    for (int i = 0; i < 4; ++i) f.b[i] = p[c.tblk0 + i * 32 * kChunks];
}

// MFMAs number q = LO .. HI-1 of the 16 of a k16 half (token block q/4, weight block q%4).
template <int LO, int HI>
__device__ __forceinline__ void mfma_range(const Frags& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
    for (int q = LO; q < HI; ++q) {
        const int i = q / 4, j = q % 4;
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(f.a[j]), as_bf16x8(f.b[i]),
                                                            acc[j][i], 0, 0, 0);
    }
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;

// One stage of the main loop: stage kt lives in `cur`, `nxt` holds stage kt+1
// and `dma` receives stage kt+3.  LATER = stages issued after kt+1 that may
// still be in flight (2 in steady state, 1 and 0 at the tail); DMA = whether
// stage kt+3 exists; NEXT = whether stage kt+1 exists.
template <bool DUAL, bool ACTIVE, bool DMA, int LATER, bool NEXT>
__device__ __forceinline__ void stage_step(const TileCtx<DUAL>& c, const uint4* __restrict__ cur,
                                           const uint4* __restrict__ nxt, uint4* __restrict__ dma,
                                           int kt, Frags& f0, Frags& f1, f32x16_t (&acc)[4][4]) {
    if (!ACTIVE) {
        if (DMA) issue_stage(c, dma, (kt + 3) * kBK);
        if (NEXT) ring_barrier<LATER * kDmaPerStage>();
        return;
    }
    // First k16 half: its 16 MFMAs carry the reads of the second half's
    // fragments and the copies of stage kt+3, one between each pair of MFMAs.
    if (DMA) issue_stage(c, dma, (kt + 3) * kBK);
    read_frags(c, cur, 1, f1);
    mfma_range<0, 16>(f0, acc);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (DMA) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // A few MFMAs of the second half stay in the pipe across the barrier.
    mfma_range<0, 4>(f1, acc);
    __builtin_amdgcn_sched_barrier(0);
    if (NEXT) {
        ring_barrier<LATER * kDmaPerStage>();
        read_frags(c, nxt, 0, f0);
    }
    mfma_range<4, 16>(f1, acc);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (NEXT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// The K loop over nk stages (nk a multiple of 4, >= 4); stages 0..2 are
// already being copied into st0..st2.
template <bool DUAL, bool ACTIVE>
__device__ __forceinline__ void main_loop(const TileCtx<DUAL>& c, uint4* st0, uint4* st1, uint4* st2,
                                          uint4* st3, int nk, f32x16_t (&acc)[4][4]) {
    ring_barrier<2 * kDmaPerStage>();
    Frags f0, f1;
    read_frags(c, st0, 0, f0);
    int kt = 0;
    for (; kt + 4 < nk; kt += 4) {
        stage_step<DUAL, ACTIVE, true, 2, true>(c, st0, st1, st3, kt + 0, f0, f1, acc);
        stage_step<DUAL, ACTIVE, true, 2, true>(c, st1, st2, st0, kt + 1, f0, f1, acc);
        stage_step<DUAL, ACTIVE, true, 2, true>(c, st2, st3, st1, kt + 2, f0, f1, acc);
        stage_step<DUAL, ACTIVE, true, 2, true>(c, st3, st0, st2, kt + 3, f0, f1, acc);
    }
    // last four stages: kt = nk-4 .. nk-1
    stage_step<DUAL, ACTIVE, true, 2, true>(c, st0, st1, st3, kt + 0, f0, f1, acc);
    stage_step<DUAL, ACTIVE, false, 1, true>(c, st1, st2, st0, kt + 1, f0, f1, acc);
    stage_step<DUAL, ACTIVE, false, 0, true>(c, st2, st3, st1, kt + 2, f0, f1, acc);
    stage_step<DUAL, ACTIVE, false, 0, false>(c, st3, st0, st2, kt + 3, f0, f1, acc);
}

template <bool DUAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void tiled_kernel(
    const bf16_t* __restrict__ act, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const bf16_t* __restrict__ wa, const bf16_t* __restrict__ wb, void* __restrict__ out,
    int Kdim, int Nw /* weight rows per expert (F or d) */, int ld_act, int n_tt, int n_wt, int GN,
    int ld_out, int n_src, int P, int ksplit, size_t split_stride) {
    __shared__ uint4 st0[kStageVec];
    __shared__ uint4 st1[kStageVec];
    __shared__ uint4 st2[kStageVec];
    __shared__ uint4 st3[kStageVec];

    // ---- tile of this workgroup
    const int nblk = gridDim.x;  // a multiple of 8
    const int L_all = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    // K may be cut into `ksplit` parts; part s adds over k in [s*K/ksplit,
    // (s+1)*K/ksplit) and writes its own output buffer (out + s*split_stride).
    const int split = L_all / (n_tt * n_wt);
    const int L = L_all - split * (n_tt * n_wt);
    if (split >= ksplit) return;
    const int kpart = Kdim / ksplit;
    const int kbase = split * kpart;
    out = static_cast<char*>(out) + split * split_stride * (DUAL ? sizeof(bf16_t) : sizeof(float));
    const int per_group = n_tt * GN;
    const int grp = L / per_group;
    const int rem = L - grp * per_group;
    const int tt = rem / GN;
    const int wt = grp * GN + (rem - (rem / GN) * GN);

    const int p0 = tt * kTT;
    if (p0 >= offsets[kExperts]) return;
    const int e = expert_of_row(offsets, p0);
    const int row_end = min(offsets[e + 1], P);
    const int valid = min(min(kTT, offsets[e] + counts[e] - p0), row_end - p0);
    if (valid <= 0) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_w = wave & 1;
    const int wave_t = wave >> 1;

    // ---- copy assignment: wave w copies weight rows and token rows
    // [w*64, w*64+64) in 4 blocks of 16 rows; lane l of a block writes LDS row
    // (block row + l/4), physical chunk l%4, so it reads logical chunk
    // (l%4) ^ g(row).
    TileCtx<DUAL> c;
    {
        const int first_src = DUAL ? row_src[p0] : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wave * 64 + j * 16 + (lane >> 2);
            const int chunk = (lane & 3) ^ swz(r);
            if (DUAL) {
                const int f0 = wt * (kTW / 2);
                const bf16_t* base = (r < kTW / 2) ? wa : wb;
                c.gw[j] = base + (static_cast<size_t>(e) * Nw + f0 + (r & (kTW / 2 - 1))) * Kdim + kbase + 8 * chunk;
                int src = (r < valid) ? row_src[p0 + r] : first_src;
                if (src < 0 || src >= n_src) src = first_src;
                if (src < 0 || src >= n_src) src = 0;
                c.gt[j] = act + static_cast<size_t>(src >> 1) * ld_act + kbase + 8 * chunk;
            } else {
                c.gw[j] = wa + (static_cast<size_t>(e) * Nw + wt * kTW + r) * Kdim + kbase + 8 * chunk;
                const int pr = (r < valid) ? p0 + r : p0;
                c.gt[j] = act + static_cast<size_t>(pr) * ld_act + kbase + 8 * chunk;
            }
        }
        c.dma_w = (wave * 64) * kChunks;
        c.dma_t = (kTW + wave * 64) * kChunks;
        const int fr = lane & 31;
        const int fk = lane >> 5;
        c.rd[0] = fr * kChunks + ((0 + fk) ^ swz(fr));
        c.rd[1] = fr * kChunks + ((2 + fk) ^ swz(fr));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rowb = DUAL ? ((j < 2 ? 0 : kTW / 2) + wave_w * 64 + (j & 1) * 32) : (wave_w * 128 + j * 32);
            c.wblk[j] = rowb * kChunks;
        }
        c.tblk0 = (kTW + wave_t * 128) * kChunks;
    }
    const bool active = __builtin_amdgcn_readfirstlane(valid > wave_t * 128 ? 1 : 0) != 0;

    f32x16_t acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.0f;

    const int nk = kpart / kBK;  // a multiple of 4
    issue_stage(c, st0, 0);
    issue_stage(c, st1, kBK);
    issue_stage(c, st2, 2 * kBK);
    if (active)
        main_loop<DUAL, true>(c, st0, st1, st2, st3, nk, acc);
    else
        main_loop<DUAL, false>(c, st0, st1, st2, st3, nk, acc);

    // ---- epilogue.  32x32 C layout: lane l holds token column l%32 and weight
    // rows 8*(q/4) + 4*(l/32) + q%4 of each block, q = 0..15.
    const int fr = lane & 31;
    const int fk = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave_t * 128 + i * 32 + fr;  // token row within the tile
        const int p = p0 + r;
        if (p >= row_end) continue;
        const bool real = r < valid;
        if (DUAL) {
            bf16_t* hrow = static_cast<bf16_t*>(out) + static_cast<size_t>(p) * ld_out;
            const int fb = wt * (kTW / 2) + wave_w * 64;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        v[u] = real ? silu_f32(acc[jj][i][4 * q4 + u]) * acc[jj + 2][i][4 * q4 + u] : 0.0f;
                    uint2 o;
                    o.x = pack_bf16x2(v[0], v[1]);
                    o.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2*>(hrow + fb + jj * 32 + 8 * q4 + 4 * fk) = o;
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

int group_size(int n_wt) {
    for (int g = 8; g > 1; g >>= 1)
        if (n_wt % g == 0) return g;
    return 1;
}

}  // namespace

int tiled_down_ksplit(const Shape& s) {
    // Cut the down projection's K in two when its tiles would not fill four
    // rounds of the 256 CUs (the last, partly empty round then costs less).
    const int P = s.T * s.K + s.n * (kTT - 1);
    const int n_tt = (P + kTT - 1) / kTT;
    const int n_wt = s.d / kTW;
    return (n_tt * n_wt < 4 * 256 && (s.F / 2) % (4 * kBK) == 0) ? 2 : 1;
}

hipError_t launch_tiled(const Shape& s, bool gate_up, const void* act, const int32_t* row_src,
                        const int32_t* counts, const int32_t* offsets, const void* wa, const void* wb,
                        void* out, hipStream_t st, int ksplit) {
    const int P = s.T * s.K + s.n * (kTT - 1);
    const int n_tt = (P + kTT - 1) / kTT;
    const int n_wt = gate_up ? s.F / (kTW / 2) : s.d / kTW;
    const int GN = group_size(n_wt);
    const int G = (n_tt * n_wt * ksplit + 7) / 8 * 8;
    const size_t split_stride = static_cast<size_t>(P) * (gate_up ? s.F : s.d);
    if (gate_up)
        tiled_kernel<true><<<G, 256, 0, st>>>(static_cast<const bf16_t*>(act), row_src, counts, offsets,
                                              static_cast<const bf16_t*>(wa), static_cast<const bf16_t*>(wb),
                                              out, s.d, s.F, s.d, n_tt, n_wt, GN, s.F, s.T * s.K, P,
                                              ksplit, split_stride);
    else
        tiled_kernel<false><<<G, 256, 0, st>>>(static_cast<const bf16_t*>(act), nullptr, counts, offsets,
                                               static_cast<const bf16_t*>(wa), nullptr, out, s.F, s.d, s.F,
                                               n_tt, n_wt, GN, s.d, s.T * s.K, P, ksplit, split_stride);
    return hipGetLastError();
}

}  // namespace moe
