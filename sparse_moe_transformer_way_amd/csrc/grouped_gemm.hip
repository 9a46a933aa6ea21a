// Grouped expert GEMMs of the SwiGLU experts, over the expert-grouped row layout.
//
// Expert i computes E_i(x) = w2_i . (SiLU(w1_i . x) * (w3_i . x)) (Mixtral of
// Experts, paper-graph-ui page, section 3.4, "Expert Network Structure
// (SwiGLU)", with w1 = gate, w3 = up, w2 = down).  Each expert sees only the
// rows routed to it (dropless top-K routing, K = 2 in Mixtral; same section,
// routing paragraphs), packed contiguously per expert and padded to the row
// tile.
//
// Both projections are "NT" contractions: out[row][j] = sum_k act[row][k] *
// W[j][k] with k contiguous in both operands (W is [out_features, in_features]
// row-major).  The MFMA "A" operand is the weight tile and the "B" operand is
// the activation tile, so one lane's accumulators hold 4 consecutive output
// features of one row and the epilogue writes 8-byte (bf16) / 16-byte (fp32)
// runs.
//
// Three kernel families:
//   * stream (tile_m 16, bf16 or FP8 weights): few rows per expert, the layer
//     is bound by reading the expert weights once from HBM.  A block owns a
//     slab of weight rows of one expert; its 4 waves split K, stream their
//     weights through per-wave LDS slices into MFMA registers and reduce
//     through LDS.  Experts with no rows are skipped.
//   * tiled (tile_m 256, bf16): many rows per expert, MFMA-bound; in
//     tiled_gemm.hip.
//   * fp32 (tile_m 16): plain LDS-tiled FMA kernel for fp32 layers.
#include "moe_common.h"

namespace moe {

namespace {

// ---------------------------------------------------------------------------
// Helpers
// ---------------------------------------------------------------------------

// Expert owning permuted row p (segments are laid out in expert order).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int n_exp, int p) {
    int e = 0;
    for (int j = 1; j < n_exp; ++j) e = (p >= offsets[j]) ? j : e;
    return e;
}

// ===========================================================================
// Weight-streaming kernel (bf16, tile_m = 16)
// ===========================================================================
//
// Block = 4 waves, one expert (blockIdx.y), one slab of 64 weight rows
// (blockIdx.x).  Wave w covers the K range [w*K/4, (w+1)*K/4) in stages of 64.
// A stage of the wave's 64 rows (8 KB) is copied into the wave's own slice of
// LDS by buffer loads with the LDS destination bit, 8 rows x 128 bytes per
// instruction, so each request is a whole 128-byte line (streams at ~6.8 TB/s
// on MI355X, against ~5.9 TB/s for the 16 rows x 64 bytes that loading
// straight into MFMA operand registers allows).  Two stage buffers per wave:
// stage s+1 is copied while stage s is read and multiplied.  No wave reads
// another wave's slice, so there are no barriers in the K loop: the
// compiler's wait for the copy into the buffer a read names is the only
// synchronisation, and each stage's copy is issued after that stage's reads
// so the wait never covers the next copy.
//
// Fragments: MFMA 16x16x32, weights as the A operand.  In 32-k step t of a
// stage, lane (r = l%16, g = l/16) takes row r of a 16-row block at logical
// chunk 4t + g (k = 32t + 8g .. +8); the activation rows are read straight
// from global memory (they are few and L2-resident) at the same k.  Chunk c
// of LDS row r sits at c ^ f(r), f(r) = 2 * ((r >> 1) & 3): in each 16-lane
// phase of a fragment read (lanes 0-7 with 16-23) the even rows and the odd
// rows each get 8 distinct chunks, so the phase covers all 64 banks.
//
// DUAL (gate/up): rows 0-31 of the slab are w1 rows f0..f0+31, rows 32-63 the
// same rows of w3; the epilogue forms SiLU(a1) * a3.  Otherwise (down): w2 rows
// j0..j0+63, fp32 output.

constexpr int kStreamRB = 4;       // 16-row weight blocks per wave
constexpr int kStreamMaxTB = 4;    // 16-row token blocks per pass
constexpr int kStreamWaveVec = 512;  // uint4 of one wave's stage slice (64 rows x 128 B)

typedef void __attribute__((address_space(3)))* lds_ptr_t;

__device__ __forceinline__ int stream_swz(int row) { return ((row >> 1) & 3) << 1; }

// Buffer resource over [base, base + 4 GiB) for a wave-uniform base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base) {
    // dword 3 = 0x00020000: 32-bit data format, the raw-buffer setting of gfx9
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}

struct StreamCtx {
    __amdgpu_buffer_rsrc_t wres[2];  // weight rows 0-31 and 32-63 of the slab (k origin: the wave's range)
    uint32_t wo;                     // lane byte offset of its copy source within an 8-row group
    int wgrp;                        // bytes between 8-row groups
    int slice;                       // uint4 offset of this wave's stage slice
    int rd[2];                       // per 32-k step: uint4 index of this lane's fragment in block 0
};

// Copy stage s (k = 64s .. 64s+63 of the wave's range) into `buf`.  The
// weights are read once per layer, so the copies carry the streaming (slc)
// cache hint: measured on MI355X, 5.9 -> 6.6 TB/s for both projections.
constexpr int kStreamingLoad = 2;  // aux bit 1: slc

__device__ __forceinline__ void stream_copy(const StreamCtx& c, uint4* __restrict__ buf, int s) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        // address-space conversion needs a C-style cast
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.wres[j >> 2], (lds_ptr_t)(buf + c.slice + j * 64), 16, c.wo,
                                                 (j & 3) * c.wgrp + 128 * s, 0, kStreamingLoad);
}

typedef const __attribute__((address_space(1))) u32x4_t* gvec_t;

// 16 E4M3 weights (k = 0..15 of a chunk, byte i = k i) to two bf16x8 MFMA
// operands, k 0-7 and k 8-15.  E4M3 values are exact in bf16; the conversion
// scale is 1.
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4_t& q, bf16x8_t& lo, bf16x8_t& hi) {
    u32x4_t a, b;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        a[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[w], 1.0f, false));
        a[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[w], 1.0f, true));
        b[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[w + 2], 1.0f, false));
        b[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[w + 2], 1.0f, true));
    }
    lo = as_bf16x8(a);
    hi = as_bf16x8(b);
}

// One stage: token fragments from global memory, weight fragments from `cur`,
// then (COPY) the next stage's copy into `nxt`, then the MFMAs.  Every lane
// loads a real row (arow) and masks it (amask: all ones, or zero for a row
// past the segment), so the loads stay plain global loads without branches.
//
// bf16 weights: a stage is 64 k; step t (32 k) reads chunk 4t + g of the row
// (k = 32t + 8g .. +8) and the token row at the same k.
// FP8 weights: a stage is 128 k (still 128 bytes per row); step u (64 k)
// reads chunk 4u + g, i.e. 16 weights k = 64u + 16g .. +16, which feed two
// MFMAs (k 0-7 and 8-15 of the chunk); the token row is read at the same k.
template <int NTP, bool COPY, bool FP8, int MT>
__device__ __forceinline__ void stream_stage(const StreamCtx& c, const uint4* __restrict__ cur,
                                             uint4* __restrict__ nxt, int s,
                                             const bf16_t* const (&arow)[MT],
                                             const uint32_t (&amask)[MT],
                                             f32x4_t (&acc)[MT][kStreamRB]) {
    constexpr int kTV = FP8 ? 4 : 2;  // 8-element token fragments per stage
    u32x4_t tv[NTP][kTV];
#pragma unroll
    for (int tb = 0; tb < NTP; ++tb)
#pragma unroll
        for (int t = 0; t < kTV; ++t)
            tv[tb][t] = FP8 ? *(gvec_t)(arow[tb] + 128 * s + 64 * (t >> 1) + 8 * (t & 1))
                            : *(gvec_t)(arow[tb] + 64 * s + 32 * t);
#pragma unroll
    for (int tb = 0; tb < NTP; ++tb)
#pragma unroll
        for (int t = 0; t < kTV; ++t) tv[tb][t] &= amask[tb];
    u32x4_t wv[2][kStreamRB];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < kStreamRB; ++b) wv[t][b] = __builtin_bit_cast(u32x4_t, cur[c.rd[t] + b * 128]);
    if (COPY) stream_copy(c, nxt, s + 1);
    if constexpr (FP8) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int b = 0; b < kStreamRB; ++b) {
                bf16x8_t lo, hi;
                fp8x16_to_bf16(wv[u][b], lo, hi);
#pragma unroll
                for (int tb = 0; tb < NTP; ++tb) {
                    acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, as_bf16x8(tv[tb][2 * u]), acc[tb][b], 0, 0, 0);
                    acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, as_bf16x8(tv[tb][2 * u + 1]), acc[tb][b], 0, 0, 0);
                }
            }
    } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int tb = 0; tb < NTP; ++tb)
#pragma unroll
                for (int b = 0; b < kStreamRB; ++b)
                    acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[t][b]), as_bf16x8(tv[tb][t]),
                                                                         acc[tb][b], 0, 0, 0);
    }
    // keep the next stage's reads (which wait for its copy) after these MFMAs
    __builtin_amdgcn_sched_barrier(0);
}

// The K loop of one pass over NTP token blocks: ns stages (ns even, >= 2).
template <int NTP, bool FP8, int MT>
__device__ __forceinline__ void stream_k_loop(const StreamCtx& c, uint4* sb0, uint4* sb1, int ns,
                                              const bf16_t* const (&arow)[MT],
                                              const uint32_t (&amask)[MT],
                                              f32x4_t (&acc)[MT][kStreamRB]) {
    stream_copy(c, sb0, 0);
    int s = 0;
    for (; s + 2 < ns; s += 2) {
        stream_stage<NTP, true, FP8, MT>(c, sb0, sb1, s, arow, amask, acc);
        stream_stage<NTP, true, FP8, MT>(c, sb1, sb0, s + 1, arow, amask, acc);
    }
    stream_stage<NTP, true, FP8, MT>(c, sb0, sb1, s, arow, amask, acc);
    stream_stage<NTP, false, FP8, MT>(c, sb1, sb0, s + 1, arow, amask, acc);
}

// FP8: wa/wb hold E4M3 codes and sa/sb one fp32 scale per weight row, applied
// to the K sums before the epilogue; otherwise bf16 weights and no scales.
template <bool DUAL, bool FP8, int MT = kStreamMaxTB>
__global__ __launch_bounds__(256) void stream_kernel(
    const bf16_t* __restrict__ act, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const void* __restrict__ wa, const void* __restrict__ wb, const float* __restrict__ sa,
    const float* __restrict__ sb, void* __restrict__ out,
    int Kdim, int Nw /* weight rows per expert */, int ld_act, int n_src, int P, int topk, int tail_rows,
    float* __restrict__ out_hi, int plan_ks_max) {
    // Two stage buffers (each 4 wave slices of 8 KB); after the K loop they
    // hold the cross-wave reduction [wave][token block][weight block][lane].
    __shared__ uint4 sb0[4 * kStreamWaveVec];
    __shared__ uint4 sb1[4 * kStreamWaveVec];

    const int e = blockIdx.y;
    // K parts (gridDim.z): the down tails may be cut in two, part 1 writing the
    // second K-partial of tail row i of expert e to row e * kTailRows + i of
    // out_hi, which the combine adds
    const int parts = gridDim.z;
    const int part = blockIdx.z;
    int seg = offsets[e];
    // rows [seg, seg_end) may be read and written: the segment, clamped to the buffers
    const int seg_end = min(offsets[e + 1], P);
    int cnt = min(counts[e], seg_end - seg);
    int tail0 = 0;  // first permuted row of the tail (tail pass only)
    if (!DUAL && tail_rows > 0) {
        // Tile-256 layout, down projection: only an expert's short tail past
        // its full tiles (the tiled kernel skips those tiles), when the plan
        // that the tiled kernel and the combine also take says so (gridDim.x is
        // Nw / 64 here; the tiled kernel's weight tiles are Nw / 256).
        const int r = cnt % kTiledRows;
        if (r == 0 || r > tail_rows) return;
        const LaneSeg ls = lane_segment(offsets, counts, gridDim.y);
        if (r > down_plan(ls, Nw / kTiledRows, plan_ks_max).tail_rows) return;
        seg += cnt - r;
        cnt = r;
        tail0 = seg;
    }
    if (cnt <= 0) return;
    const int ntb = (cnt + 15) >> 4;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int r = lane & 15;
    const int g = lane >> 4;
    const int kq = Kdim / (4 * parts);
    const int kbeg = part * (Kdim / parts) + wave * kq;
    constexpr int kEsz = FP8 ? 1 : 2;  // bytes per weight
    // stages of 128 bytes per row: even (K / parts is a multiple of 512, of 1024 for FP8)
    const int ns = kq * kEsz / 128;

    StreamCtx c;
    {
        // copy lane l: row l/8 of an 8-row group, physical chunk l%8, so it
        // reads logical chunk (l%8) ^ f(row) (f depends on the row's low bits only)
        const int rl = lane >> 3;
        const int lch = (lane & 7) ^ stream_swz(rl);
        c.wo = static_cast<uint32_t>(rl) * Kdim * kEsz + 16u * lch;
        c.wgrp = 8 * Kdim * kEsz;
        const char* wab = static_cast<const char*>(wa);
        if (DUAL) {
            const size_t f0 = static_cast<size_t>(e) * Nw + blockIdx.x * 32;
            c.wres[0] = stream_rsrc(wab + (f0 * Kdim + kbeg) * kEsz);
            c.wres[1] = stream_rsrc(static_cast<const char*>(wb) + (f0 * Kdim + kbeg) * kEsz);
        } else {
            const size_t j0 = static_cast<size_t>(e) * Nw + blockIdx.x * 64;
            c.wres[0] = stream_rsrc(wab + (j0 * Kdim + kbeg) * kEsz);
            c.wres[1] = stream_rsrc(wab + ((j0 + 32) * Kdim + kbeg) * kEsz);
        }
        c.slice = wave * kStreamWaveVec;
#pragma unroll
        for (int t = 0; t < 2; ++t) c.rd[t] = c.slice + r * 8 + ((4 * t + g) ^ stream_swz(r));
    }

    for (int tb0 = 0; tb0 < ntb; tb0 += MT) {
        const int ntp = min(MT, ntb - tb0);
        // Activation row of this lane in each token block, at the wave's k
        // origin and this lane's k-group; rows past the segment read the
        // segment's first row and are masked to zero.
        const bf16_t* arow[MT];
        uint32_t amask[MT];
        const int src0 = DUAL ? row_src[seg] : 0;
        const int row0 = DUAL ? ((src0 >= 0 && src0 < n_src) ? static_cast<int>(div_topk(static_cast<uint32_t>(src0), topk)) : 0) : seg;
#pragma unroll
        for (int tb = 0; tb < MT; ++tb) {
            const int p = seg + (tb0 + tb) * 16 + r;
            int row = row0;
            bool real = false;
            if (tb < ntp && p < seg + cnt) {
                if (DUAL) {
                    const int src = row_src[p];
                    real = src >= 0 && src < n_src;
                    if (real) row = static_cast<int>(div_topk(static_cast<uint32_t>(src), topk));
                } else {
                    real = true;
                    row = p;
                }
            }
            arow[tb] = act + static_cast<size_t>(row) * ld_act + kbeg + (FP8 ? 16 : 8) * g;
            amask[tb] = real ? 0xffffffffu : 0u;
        }

        f32x4_t acc[MT][kStreamRB];
#pragma unroll
        for (int tb = 0; tb < MT; ++tb)
#pragma unroll
            for (int b = 0; b < kStreamRB; ++b) acc[tb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        switch (ntp) {
            case 1: stream_k_loop<1, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
            case 2: stream_k_loop<2, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
            case 3: stream_k_loop<3, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
            case 4: stream_k_loop<4, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
            default:
                if constexpr (MT == 8) {
                    switch (ntp) {
                        case 5: stream_k_loop<5, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
                        case 6: stream_k_loop<6, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
                        case 7: stream_k_loop<7, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
                        default: stream_k_loop<8, FP8, MT>(c, sb0, sb1, ns, arow, amask, acc); break;
                    }
                }
                break;
        }

        // Cross-wave K reduction in a fixed order through the stage buffers,
        // four token blocks at a time (wave w finishes token block q + w).
        f32x4_t* red0 = reinterpret_cast<f32x4_t*>(sb0);  // waves 0, 1
        f32x4_t* red1 = reinterpret_cast<f32x4_t*>(sb1);  // waves 2, 3
        auto red = [&](int w, int tb, int b) -> f32x4_t& {
            const int i = (((w & 1) * kStreamMaxTB + tb) * kStreamRB + b) * 64 + lane;
            return (w < 2 ? red0 : red1)[i];
        };
#pragma unroll
        for (int q = 0; q < MT; q += kStreamMaxTB) {
            if (q >= ntp) continue;  // uniform: ntp is the same for the whole block
            __syncthreads();
#pragma unroll
            for (int tb = 0; tb < kStreamMaxTB; ++tb)
                if (q + tb < ntp)
#pragma unroll
                    for (int b = 0; b < kStreamRB; ++b) red(wave, tb, b) = acc[q + tb][b];
            __syncthreads();
            if (q + wave < ntp && seg + (tb0 + q + wave) * 16 + r < seg_end) {
                const int tb = wave;
                f32x4_t sum[kStreamRB];
#pragma unroll
                for (int b = 0; b < kStreamRB; ++b) {
                    sum[b] = red(0, tb, b);
#pragma unroll
                    for (int w = 1; w < 4; ++w) sum[b] += red(w, tb, b);
                }
                // C layout of 16x16 MFMA: lane l holds column (token) l%16 and rows
                // (weight rows) 4*(l/16) + i, i = 0..3.
                const int p = seg + (tb0 + q + tb) * 16 + r;
                if (DUAL) {
                    const int f0 = blockIdx.x * 32;
                    bf16_t* hrow = static_cast<bf16_t*>(out) + static_cast<size_t>(p) * Nw;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        f32x4_t a1 = sum[half], a3 = sum[half + 2];
                        if constexpr (FP8) {
                            const size_t f = static_cast<size_t>(e) * Nw + f0 + half * 16 + 4 * g;
                            a1 *= *reinterpret_cast<const f32x4_t*>(sa + f);
                            a3 *= *reinterpret_cast<const f32x4_t*>(sb + f);
                        }
                        uint2 o;
                        o.x = pack_bf16x2(silu_f32(a1[0]) * a3[0], silu_f32(a1[1]) * a3[1]);
                        o.y = pack_bf16x2(silu_f32(a1[2]) * a3[2], silu_f32(a1[3]) * a3[3]);
                        *reinterpret_cast<uint2*>(hrow + f0 + half * 16 + 4 * g) = o;
                    }
                } else {
                    const int j0 = blockIdx.x * 64;
                    float* yrow = part ? out_hi + static_cast<size_t>(e * kTailRows + (p - tail0)) * Nw
                                       : static_cast<float*>(out) + static_cast<size_t>(p) * Nw;
#pragma unroll
                    for (int b = 0; b < kStreamRB; ++b) {
                        if constexpr (FP8)
                            sum[b] *= *reinterpret_cast<const f32x4_t*>(sa + static_cast<size_t>(e) * Nw + j0 + b * 16 + 4 * g);
                        *reinterpret_cast<f32x4_t*>(yrow + j0 + b * 16 + 4 * g) = sum[b];
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ===========================================================================
// fp32 kernel (tile_m = 16)
// ===========================================================================
//
// Block = 16 permuted rows x 64 output features, BK = 32, plain fp32 FMA.
// Thread (ty, tx) owns row ty and features tx + 16u, u = 0..3.

template <bool DUAL>
__global__ __launch_bounds__(256) void f32_kernel(
    const float* __restrict__ act, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const float* __restrict__ wa, const float* __restrict__ wb, float* __restrict__ out,
    int Kdim, int Nw, int ld_act, int n_src, int P, int n_exp, int topk) {
    __shared__ float sa[16][33];
    __shared__ float s1[64][33];
    __shared__ float s3[DUAL ? 64 : 1][33];

    const int p0 = blockIdx.x * 16;
    if (p0 >= offsets[n_exp]) return;
    const int e = expert_of_row(offsets, n_exp, p0);
    const int row_end = min(offsets[e + 1], P);
    const int valid = min(min(16, offsets[e] + counts[e] - p0), row_end - p0);
    if (valid <= 0) return;
    const int n0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;

    // activation row of each of the 16 tile rows (nullptr = zero)
    const float* arow = nullptr;
    {
        const int rr = tid >> 4;  // row loaded by this thread (2 elements per k-tile)
        if (rr < valid) {
            if (DUAL) {
                const int src = row_src[p0 + rr];
                if (src >= 0 && src < n_src) arow = act + static_cast<size_t>(div_topk(static_cast<uint32_t>(src), topk)) * ld_act;
            } else {
                arow = act + static_cast<size_t>(p0 + rr) * ld_act;
            }
        }
    }

    float acc1[4] = {0.f, 0.f, 0.f, 0.f}, acc3[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < Kdim; k0 += 32) {
        {
            const int rr = tid >> 4, kk = (tid & 15) * 2;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int k = k0 + kk + u;
                sa[rr][kk + u] = (arow != nullptr && k < Kdim) ? arow[k] : 0.0f;
            }
        }
        for (int q = tid; q < 64 * 32; q += 256) {
            const int rr = q >> 5, kk = q & 31;
            const int k = k0 + kk;
            const int n = n0 + rr;
            const bool ok = (k < Kdim) && (n < Nw);
            const size_t wi = (static_cast<size_t>(e) * Nw + n) * Kdim + k;
            s1[rr][kk] = ok ? wa[wi] : 0.0f;
            if (DUAL) s3[rr][kk] = ok ? wb[wi] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < 32; ++kk) {
            const float a = sa[ty][kk];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc1[u] = fmaf(a, s1[tx + 16 * u][kk], acc1[u]);
                if (DUAL) acc3[u] = fmaf(a, s3[tx + 16 * u][kk], acc3[u]);
            }
        }
        __syncthreads();
    }
    const int p = p0 + ty;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int n = n0 + tx + 16 * u;
        if (n < Nw && p < row_end) {
            const float v = DUAL ? silu_f32(acc1[u]) * acc3[u] : acc1[u];
            out[static_cast<size_t>(p) * Nw + n] = v;
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static int pmax_rows(const Shape& s, int tile_m) {
    return s.T * s.K + s.n * (tile_m - 1);
}

static int max_tiles(const Shape& s, int tile_m) {
    return (pmax_rows(s, tile_m) + tile_m - 1) / tile_m;
}

hipError_t launch_gate_up(const Shape& s, int tile_m, const void* x, const int32_t* row_src,
                          const int32_t* counts, const int32_t* offsets, const void* w1,
                          const void* w3, void* h, hipStream_t st) {
    if (!s.bf16) {
        dim3 grid(max_tiles(s, 16), (s.F + 63) / 64);
        f32_kernel<true><<<grid, 256, 0, st>>>(static_cast<const float*>(x), row_src, counts,
                                               offsets, static_cast<const float*>(w1),
                                               static_cast<const float*>(w3),
                                               static_cast<float*>(h), s.d, s.F, s.d, s.T * s.K,
                                               pmax_rows(s, 16), s.n, s.K);
    } else if (tile_m == 16) {
        dim3 grid(s.F / 32, s.n);
        stream_kernel<true, false><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), row_src, counts,
                                                         offsets, w1, w3, nullptr, nullptr, h, s.d, s.F, s.d,
                                                         s.T * s.K, pmax_rows(s, 16), s.K, 0, nullptr, 1);
    } else {
        // (a short tail costs gate/up less than a full tile: its idle waves skip
        // their reads and MFMAs, so streaming the tail does not pay here)
        return launch_tiled(s, true, x, row_src, counts, offsets, w1, w3, h, st);
    }
    return hipGetLastError();
}

hipError_t launch_down(const Shape& s, int tile_m, const void* h, const int32_t* counts,
                       const int32_t* offsets, const void* w2, float* y_perm, hipStream_t st,
                       float* y_perm_hi, float* y_tail_hi, int* ks_max) {
    if (ks_max != nullptr) *ks_max = 1;
    if (!s.bf16) {
        dim3 grid(max_tiles(s, 16), (s.d + 63) / 64);
        f32_kernel<false><<<grid, 256, 0, st>>>(static_cast<const float*>(h), nullptr, counts,
                                                offsets, static_cast<const float*>(w2), nullptr,
                                                y_perm, s.F, s.d, s.F, s.T * s.K,
                                                pmax_rows(s, 16), s.n, s.K);
    } else if (tile_m == 16) {
        dim3 grid(s.d / 64, s.n);
        stream_kernel<false, false><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(h), nullptr, counts,
                                                          offsets, w2, nullptr, nullptr, nullptr,
                                                          y_perm, s.F, s.d, s.F, s.T * s.K,
                                                          pmax_rows(s, 16), s.K, 0, nullptr, 1);
    } else {
        int ks = 1;
        if (y_perm_hi != nullptr) {
            ks = tiled_down_ksplit(s);
            // the second part lands one P x d block after y_perm
            const size_t P = static_cast<size_t>(pmax_rows(s, 256));
            if (ks == 2 && y_perm_hi != y_perm + P * s.d) ks = 1;
        }
        if (ks_max != nullptr) *ks_max = ks;
        hipError_t err = launch_tiled(s, false, h, nullptr, counts, offsets, w2, nullptr, y_perm, st, ks, kTailRows);
        if (err != hipSuccess) return err;
        // The tails (a few experts' w2, streamed with at most kTailRows rows
        // each, all of them in one pass over the weights) run one block per
        // 64 rows of w2 per expert; with a tail buffer they also
        // cut K in two, which doubles the blocks of this latency-bound pass
        // (measured at prefill: 140 -> 90-98 us).
        const int parts = (y_tail_hi != nullptr && s.F % 1024 == 0) ? 2 : 1;
        dim3 grid(s.d / 64, s.n, parts);
        stream_kernel<false, false, kTailRows / 16><<<grid, 256, 0, st>>>(
            static_cast<const bf16_t*>(h), nullptr, counts, offsets, w2, nullptr, nullptr, nullptr, y_perm, s.F, s.d,
            s.F, s.T * s.K, pmax_rows(s, 256), s.K, kTailRows, parts == 2 ? y_tail_hi : nullptr, ks);
    }
    return hipGetLastError();
}

hipError_t launch_gate_up_fp8(const Shape& s, const void* x, const int32_t* row_src, const int32_t* counts,
                              const int32_t* offsets, const uint8_t* w1, const float* s1, const uint8_t* w3,
                              const float* s3, void* h, hipStream_t st) {
    dim3 grid(s.F / 32, s.n);
    stream_kernel<true, true><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), row_src, counts, offsets, w1,
                                                    w3, s1, s3, h, s.d, s.F, s.d, s.T * s.K, pmax_rows(s, 16),
                                                    s.K, 0, nullptr, 1);
    return hipGetLastError();
}

hipError_t launch_down_fp8(const Shape& s, const void* h, const int32_t* counts, const int32_t* offsets,
                           const uint8_t* w2, const float* s2, float* y_perm, hipStream_t st) {
    dim3 grid(s.d / 64, s.n);
    stream_kernel<false, true><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(h), nullptr, counts, offsets, w2,
                                                     nullptr, s2, nullptr, y_perm, s.F, s.d, s.F, s.T * s.K,
                                                     pmax_rows(s, 16), s.K, 0, nullptr, 1);
    return hipGetLastError();
}

}  // namespace moe
