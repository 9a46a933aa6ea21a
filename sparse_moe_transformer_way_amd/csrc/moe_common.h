// Shared device helpers and the internal launcher interface of the gfx950 MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an IEEE fp32)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN): gfx950 converts in
// hardware (v_cvt_pk_bf16_f32, two values per instruction).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Widen the 8 bf16 values held in a 16-byte word.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// SiLU(z) = z / (1 + e^-z) in fp32 from the hardware base-2 exponential
// (v_exp_f32) and reciprocal (v_rcp_f32), each within about one ulp, instead
// of the library expf and a true division: four VALU operations instead of
// about twenty, which matters in the gate/up epilogue (128 SiLUs per lane).
// e^-z overflowing to +inf gives z * 0 = -0, the limit for z -> -inf.
__device__ __forceinline__ float silu_f32(float z) {
    constexpr float kLog2e = 1.4426950408889634f;
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * z));
}

// sigma(z) = 1 / (1 + exp(-z)), with the same hardware exp2 and reciprocal.
__device__ __forceinline__ float sigmoid_f32(float z) {
    constexpr float kLog2e = 1.4426950408889634f;
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * z));
}

// ---------------------------------------------------------------------------
// Internal launchers (host side).  Each enqueues on `stream` and returns the
// hipGetLastError() status of its launches.  Shapes are validated by the ABI.
// ---------------------------------------------------------------------------
// Token rows of a tile of the LDS-tiled MFMA kernels, and the largest
// remainder of an expert's rows (past its full tiles) that the weight-streaming
// kernels take over from them in the tile-256 layout: such a tail would cost a
// whole tile there, while streaming reads the expert's weights once.
constexpr int kTiledRows = 256;
constexpr int kTailRows = 128;
constexpr int kComputeUnits = 256;  // MI355X: a round of tiled-kernel tiles

// Layout of the backward pass's fp32 pre-activations a = [a1 | a3], logically
// [P, 2F]: 32 x 32 blocks in the C layout of a 32x32 MFMA whose columns are the
// rows p and whose rows are the features f.  Block (p / 32, f / 32) starts at
// float (p / 32 * (2F / 32) + f / 32) * 1024; in it, lane l holds row p % 32 =
// l % 32 and features 8 (q / 4) + 4 (l / 32) + q % 4, q = 0..15, as 16
// contiguous floats from l * 16.  The kernel that writes a block and the one
// that reads it move 64 contiguous bytes per lane (4 KB per wave), where rows of
// [P, 2F] would take 32 rows x 32 bytes per instruction.
__device__ __forceinline__ size_t preact_block(int pb, int fb, int F) {
    return (static_cast<size_t>(pb) * (2 * F / 32) + fb) * 1024;
}

// Store a wave's 128 x 128 fp32 results acc[bu][bv] (32x32 MFMA C layout:
// rows v = 32 bv + lane % 32, columns u = 32 bu + 8 (q / 4) + 4 (lane / 32) +
// q % 4) to dst[v_base + v][u_base + u], for v < rows only, through a 32 KB
// LDS region stg that no other wave uses.  In the C layout a store instruction would write 32 rows x 32
// bytes; staged, 64 rows at a time, each store writes 2 rows x 512 contiguous
// bytes (measured: the scattered stores made the weight-gradient products
// about a fifth slower).  LDS row r holds 128 floats as 32 chunks of 16 bytes,
// chunk c at c ^ (r % 32): the 32 rows of a write instruction and the 32
// chunks of a read hit distinct chunk slots.  LDS runs one wave's
// instructions in order, so no barrier is needed between the writes and the
// reads, nor between the two halves.
__device__ __forceinline__ void store_rows_staged(const f32x16_t (&acc)[4][4], f32x4_t* stg, float* dst,
                                                  int64_t ldc, int v_base, int u_base, int rows, int lane) {
    const int fk = lane >> 5;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            const int r = b2 * 32 + (lane & 31);  // row within the half
#pragma unroll
            for (int bu = 0; bu < 4; ++bu)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x16_t& c = acc[bu][2 * half + b2];
                    const int chunk = bu * 8 + 2 * q4 + fk;
                    stg[r * 32 + (chunk ^ (r & 31))] = f32x4_t{c[4 * q4], c[4 * q4 + 1], c[4 * q4 + 2], c[4 * q4 + 3]};
                }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int r = 2 * i + (lane >> 5);
            const int chunk = lane & 31;
            const f32x4_t o = stg[r * 32 + (chunk ^ (r & 31))];
            if (half * 64 + r < rows)
                *reinterpret_cast<f32x4_t*>(dst + static_cast<int64_t>(v_base + half * 64 + r) * ldc + u_base +
                                            4 * chunk) = o;
        }
    }
}

// a / topk for topk in 1..4 (uniform), the token of an assignment index:
// shifts, and for 3 a multiply-high by ceil(2^33 / 3), exact for every 32-bit
// a (a run-time integer division is a few dozen instructions per lane)
__device__ __forceinline__ uint32_t div_topk(uint32_t a, int topk) {
    return topk == 2 ? a >> 1 : topk == 4 ? a >> 2 : topk == 3 ? __umulhi(a, 0xAAAAAAABu) >> 1 : a;
}

// Largest expert count and top-k the kernels are built for (Mixtral: 8, 2).
constexpr int kMaxExperts = 16;
constexpr int kMaxTopK = 4;

// Every expert's segment, one expert per lane: in each group of 16 lanes,
// lane e < n_exp holds expert e's offset, end and count, the other lanes an
// empty segment.  Kernels that need a sum or a search over the experts do it
// across the lanes (a few shuffles and a ballot) rather than as a loop over 16
// expert slots in scalar registers: such a loop is a chain of several hundred
// dependent scalar instructions, which a wave issues one per 4 cycles (~1-2 us
// at the clock the chip holds under load, paid by every workgroup).  Every
// lane of the wave must be active where these are called.
struct LaneSeg {
    int off, end, cnt;
};

__device__ __forceinline__ LaneSeg lane_segment(const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ counts, int n_exp) {
    const int e = threadIdx.x & 15;
    LaneSeg s{0, 0, 0};
    if (e < n_exp) {
        s.off = offsets[e];
        s.end = offsets[e + 1];
        s.cnt = counts[e];
    }
    return s;
}

// Sum of v over lanes 0-15 (the expert lanes), the same in every lane.
__device__ __forceinline__ int expert_sum(int v) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return __builtin_amdgcn_readfirstlane(v);
}

// Inclusive prefix sum of v over lanes 0-15 (lanes past 15 keep their sums
// of their own group of 16, which no caller reads).
__device__ __forceinline__ int expert_prefix(int v) {
    const int lane = threadIdx.x & 15;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const int u = __shfl_up(v, o, 16);
        if (lane >= o) v += u;
    }
    return v;
}

// The lane of the first expert whose inclusive prefix ps exceeds i (uniform
// i, 0 <= i < the total), or -1.
__device__ __forceinline__ int expert_holding(int ps, int i) {
    const uint64_t hit = __ballot((threadIdx.x & 63) < 16 && ps > i);
    return hit == 0 ? -1 : static_cast<int>(__builtin_ctzll(hit));
}

// The down projection's plan for one call, taken on the device from the real
// counts by every kernel that needs it (the tiled kernel, the tail pass and the
// combine), so that they agree without a host round trip:
//   ks   K parts of the tiled kernel: 2 only when ks_max allows it and it
//        lowers the K-weighted round count, ceil(2 t / CUs) / 2 < ceil(t / CUs)
//        for t tiles (a last round of few tiles is then half as long); each
//        part writes its own fp32 partial sum, which the combine adds.
//   tail_rows  the experts' short tails (at most tail_rows rows past their
//        full tiles) go to the streaming pass, when that lowers the round
//        count: tails up to kTailRows rows while at most five 4096-wide
//        experts' worth of tails go there (at most 640 streaming blocks, K cut
//        in two), else tails up to kTailRows / 2 rows.  Measured: with 128-row
//        tails the 32-block stack ran 3.5% faster; with six streamed tails
//        (skewed routing) the longer pass cost more than the narrow tiles it
//        replaced, which is what the cap keeps out.
struct DownPlan {
    int ks;
    int tail_rows;  // tails of at most this many rows go to the streaming pass (0: none)
};

__device__ __forceinline__ DownPlan down_plan(const LaneSeg& s, int n_wt, int ks_max) {
    // per expert (lane), then summed over the experts
    const int len = s.end - s.off;
    const int c = s.cnt;
    const int r = c % kTiledRows;
    const int without = expert_sum(len / kTiledRows);
    const int with_short = expert_sum((r > 0 && r <= kTailRows / 2) ? c / kTiledRows : len / kTiledRows);
    const int with_long = expert_sum((r > 0 && r <= kTailRows) ? c / kTiledRows : len / kTiledRows);
    const int n_long = expert_sum((r > 0 && r <= kTailRows) ? 1 : 0);
    // (lanes past the experts hold empty segments, which add nothing)
    // the tail pass runs 8 blocks per tail expert per 256 weight rows (64 rows
    // each, K in two parts): at most 640 of them
    const bool long_ok = 4 * (n_long * n_wt * 8) <= 5 * (2 * kComputeUnits);
    const int with_tail = long_ok ? with_long : with_short;
    const int tail_max = long_ok ? kTailRows : kTailRows / 2;
    DownPlan best{1, 0};
    int best_r = 0;
    for (int ks = 1; ks <= ks_max; ++ks) {
        const int per = n_wt * ks;
        const int r_with = (with_tail * per + kComputeUnits - 1) / kComputeUnits;
        const int r_without = (without * per + kComputeUnits - 1) / kComputeUnits;
        const bool tail = r_with < r_without;
        const int rr = tail ? r_with : r_without;
        // rr rounds of K / ks each: compare rr / ks across ks (the smaller ks on a tie)
        if (ks == 1 || rr * best.ks < best_r * ks) {
            best = DownPlan{ks, tail ? tail_max : 0};
            best_r = rr;
        }
    }
    return best;
}

struct Shape {
    int T, d, F, n, K;  // n <= kMaxExperts, K <= min(n, kMaxTopK)
    bool bf16;
};

hipError_t launch_router_topk(const Shape& s, const void* x, const float* wg, int32_t* idx,
                              float* gate, float* logits, hipStream_t st);

hipError_t launch_permute(const Shape& s, int tile_m, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* row_src, int32_t* row_of, hipStream_t st);

// Grouped SwiGLU projections.  tile_m selects the kernel family.
hipError_t launch_gate_up(const Shape& s, int tile_m, const void* x, const int32_t* row_src,
                          const int32_t* counts, const int32_t* offsets, const void* w1,
                          const void* w3, void* h, hipStream_t st);
// tile_m 256 only, both optional:
//   y_perm_hi [P, d]: lets the tiled kernel cut K in two (the plan's ks); part 1
//     writes it for the rows of the tiles it computes.
//   y_tail_hi [n * kTailRows, d]: lets the tail pass cut K in two; part 1 writes
//     tail row i of expert e to row e * kTailRows + i.
// *ks_max receives the largest K split the plan could take (1 or 2), which the
// combine needs to take the same plan.
hipError_t launch_down(const Shape& s, int tile_m, const void* h, const int32_t* counts,
                       const int32_t* offsets, const void* w2, float* y_perm, hipStream_t st,
                       float* y_perm_hi = nullptr, float* y_tail_hi = nullptr, int* ks_max = nullptr);

// FP8 (E4M3) expert weights, weight-streaming kernels (tile_m 16, bf16
// activations): w1/w3 [n, F, d] and w2 [n, d, F] codes with one fp32 scale per
// row (s1, s3 [n, F], s2 [n, d]).  d and F must be multiples of 1024.
hipError_t launch_gate_up_fp8(const Shape& s, const void* x, const int32_t* row_src, const int32_t* counts,
                              const int32_t* offsets, const uint8_t* w1, const float* s1, const uint8_t* w3,
                              const float* s3, void* h, hipStream_t st);
hipError_t launch_down_fp8(const Shape& s, const void* h, const int32_t* counts, const int32_t* offsets,
                           const uint8_t* w2, const float* s2, float* y_perm, hipStream_t st);
// Per-row E4M3 quantization of a bf16 [rows, cols] matrix (cols % 8 == 0).
hipError_t launch_quantize_fp8(int64_t rows, int cols, const void* w, uint8_t* q, float* scale, hipStream_t st);

// Backward pass (bf16).  Workspace pieces, carved by backward_workspace_bytes
// (base == nullptr only sizes it).  Rows are padded to 256 per expert.
struct BackwardWs {
    int32_t* idx;
    float* gate;
    int32_t* counts;
    int32_t* offsets;
    int32_t* row_src;
    int32_t* row_of;
    bf16_t* xp;       // [P, d] gathered x
    bf16_t* dyp;      // [P, d] gathered dy
    float* gp;        // [P] gate of each row
    float* a;         // [P, 2F] pre-activations a1 | a3, in 32 x 32 blocks (preact_block)
    bf16_t* da;       // [P, 2F] their gradients
    bf16_t* hg;       // [P, F] gate * h
    float* dgp;       // [F / 256, P] partial gate gradients
    float* dxp;       // [P, d] per-row input gradients
    float* dl;        // [T, n] router logit gradients
    float* dwg_part;  // [ceil(T / 64), d, n]
    int P;
};
size_t backward_workspace_bytes(const Shape& s, BackwardWs* w, char* base);
bool backward_fits(const Shape& s);
hipError_t launch_zero_grads(const Shape& s, float* dwg, float* dw1, float* dw3, float* dw2, hipStream_t st);
hipError_t launch_layer_backward(const Shape& s, const void* x, const float* wg, const void* w1, const void* w3,
                                 const void* w2, const void* dy, void* dx, float* dwg, float* dw1, float* dw3,
                                 float* dw2, const BackwardWs& w, hipStream_t st);

// Whether the tiled kernels can address this shape's token rows (gate/up
// reaches the rows of x through 32-bit byte offsets: T * d_model * 2 bytes
// must stay below 4 GiB).
bool tiled_fits(const Shape& s);
// Number of K parts the tiled down projection uses when allowed to split.
int tiled_down_ksplit(const Shape& s);

// LDS-tiled MFMA kernels (bf16, tile_m 256): gate_up selects SiLU(act.wa) * (act.wb)
// into bf16 `out`, otherwise act.wa into fp32 `out`.
// tail_rows > 0: an expert's last tile holding at most tail_rows real rows is
// skipped (left to the weight-streaming kernels).
hipError_t launch_tiled(const Shape& s, bool gate_up, const void* act, const int32_t* row_src,
                        const int32_t* counts, const int32_t* offsets, const void* wa, const void* wb,
                        void* out, hipStream_t st, int ksplit = 1, int tail_rows = 0);

// The gate/up tiled kernel storing the pre-activations a1 = w1 . x, a3 = w3 . x
// in fp32 (a [P, 2F], padding rows zero) for the backward pass.
hipError_t launch_tiled_preact(const Shape& s, const void* x, const int32_t* row_src, const int32_t* counts,
                               const int32_t* offsets, const void* w1, const void* w3, float* a, hipStream_t st);

// y_perm_hi / y_tail_hi (optional, with the counts, offsets and ks_max given to
// launch_down): the second K-partials of the down projection, added to y_perm
// row by row as the down plan wrote them.
hipError_t launch_combine(const Shape& s, const float* y_perm, const int32_t* row_of,
                          const float* gate, const void* residual, void* y, hipStream_t st,
                          const float* y_perm_hi = nullptr, const float* y_tail_hi = nullptr,
                          const int32_t* counts = nullptr, const int32_t* offsets = nullptr, int ks_max = 1);

hipError_t launch_rmsnorm(int T, int d, bool bf16, const void* h, float eps, void* x_out,
                          hipStream_t st);

}  // namespace moe
