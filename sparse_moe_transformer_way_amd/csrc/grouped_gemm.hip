// Grouped expert GEMMs of the SwiGLU experts, over the expert-grouped row layout.
//
// Expert i computes E_i(x) = w2_i . (SiLU(w1_i . x) * (w3_i . x)) (Mixtral of
// Experts, paper-graph-ui page, section 3.4, "Expert Network Structure
// (SwiGLU)", with w1 = gate, w3 = up, w2 = down).  Each expert sees only the
// rows routed to it (dropless top-2, same section, routing paragraphs), packed
// contiguously per expert and padded to the row tile.
//
// Both projections are "NT" contractions: out[row][j] = sum_k act[row][k] *
// W[j][k] with k contiguous in both operands (W is [out_features, in_features]
// row-major).  The MFMA "A" operand is the weight tile and the "B" operand is
// the activation tile, so one lane's accumulators hold 4 consecutive output
// features of one row and the epilogue writes 8-byte (bf16) / 16-byte (fp32)
// runs.
//
// Three kernel families:
//   * stream (tile_m 16, bf16): few rows per expert, the layer is bound by
//     reading the expert weights once from HBM.  A block owns a slab of weight
//     rows of one expert; its 4 waves split K, stream their weights straight
//     into MFMA registers (no LDS staging: each weight is used by at most a few
//     row blocks) and reduce through LDS.  Experts with no rows are skipped.
//   * tiled (tile_m 256, bf16): many rows per expert, MFMA-bound; in
//     tiled_gemm.hip.
//   * fp32 (tile_m 16): plain LDS-tiled FMA kernel for fp32 layers.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kExperts = 8;

// ---------------------------------------------------------------------------
// Helpers
// ---------------------------------------------------------------------------

// Expert owning permuted row p (segments are laid out in expert order).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int p) {
    int e = 0;
#pragma unroll
    for (int j = 1; j < kExperts; ++j) e = (p >= offsets[j]) ? j : e;
    return e;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// ===========================================================================
// Weight-streaming kernel (bf16, tile_m = 16)
// ===========================================================================
//
// Block = 4 waves, one expert (blockIdx.y), one slab of kRB*16 weight rows
// (blockIdx.x).  Wave w covers K range [w*K/4, (w+1)*K/4) in super-steps of 128.
// Load j (0..3) of a super-step gives lane (r = l%16, g = l/16) the 8 elements
// k = base + 32j + 8g .. +8 of weight row r of a 16-row block, so one load
// instruction reads 64 contiguous bytes of each of 16 rows (this streams at
// ~5.9 TB/s on MI355X, against ~3.6 TB/s when each lane instead reads 64
// contiguous bytes by itself).  The activation rows are loaded the same way and
// MFMA j pairs load j of both operands: the contraction pairs equal k on both
// sides, so this permutation of k is exact.
//
// DUAL (gate/up): row blocks 0,1 are w1 rows f0..f0+31, blocks 2,3 are w3 rows
// f0..f0+31; the epilogue forms SiLU(a1) * a3.  Otherwise (down): 4 blocks of
// w2 rows j0..j0+63, fp32 output.

constexpr int kStreamRB = 4;     // 16-row weight blocks per wave
constexpr int kStreamMaxTB = 4;  // 16-row token blocks per pass

template <bool DUAL>
__global__ __launch_bounds__(256) void stream_kernel(
    const bf16_t* __restrict__ act, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const bf16_t* __restrict__ wa, const bf16_t* __restrict__ wb, void* __restrict__ out,
    int Kdim, int Nw /* weight rows per expert */, int ld_act, int n_src, int P) {
    __shared__ f32x4_t red[4][kStreamMaxTB][kStreamRB][64];  // 64 KB

    const int e = blockIdx.y;
    const int seg = offsets[e];
    // rows [seg, seg_end) may be read and written: the segment, clamped to the buffers
    const int seg_end = min(offsets[e + 1], P);
    const int cnt = min(counts[e], seg_end - seg);
    if (cnt <= 0) return;
    const int ntb = (cnt + 15) >> 4;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int kq = Kdim >> 2;
    const int kbeg = wave * kq;

    // Weight row pointers of this lane's 4 row blocks.
    const bf16_t* wrow[kStreamRB];
    if (DUAL) {
        const int f0 = blockIdx.x * 32;
#pragma unroll
        for (int b = 0; b < kStreamRB; ++b) {
            const bf16_t* base = (b < 2) ? wa : wb;
            wrow[b] = base + (static_cast<size_t>(e) * Nw + f0 + (b & 1) * 16 + r) * Kdim + 8 * g;
        }
    } else {
        const int j0 = blockIdx.x * 64;
#pragma unroll
        for (int b = 0; b < kStreamRB; ++b)
            wrow[b] = wa + (static_cast<size_t>(e) * Nw + j0 + b * 16 + r) * Kdim + 8 * g;
    }

    for (int tb0 = 0; tb0 < ntb; tb0 += kStreamMaxTB) {
        const int ntp = min(kStreamMaxTB, ntb - tb0);
        // Activation row of this lane in each token block (nullptr = zero row).
        const bf16_t* arow[kStreamMaxTB];
#pragma unroll
        for (int tb = 0; tb < kStreamMaxTB; ++tb) {
            arow[tb] = nullptr;
            const int p = seg + (tb0 + tb) * 16 + r;
            if (tb < ntp) {
                if (DUAL) {
                    const int src = (p < seg + cnt) ? row_src[p] : -1;
                    if (src >= 0 && src < n_src) arow[tb] = act + static_cast<size_t>(src >> 1) * ld_act + 8 * g;
                } else if (p < seg + cnt) {
                    arow[tb] = act + static_cast<size_t>(p) * ld_act + 8 * g;
                }
            }
        }

        f32x4_t acc[kStreamMaxTB][kStreamRB];
#pragma unroll
        for (int tb = 0; tb < kStreamMaxTB; ++tb)
#pragma unroll
            for (int b = 0; b < kStreamRB; ++b) acc[tb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int k = kbeg; k < kbeg + kq; k += 128) {
            u32x4_t wv[kStreamRB][4];
#pragma unroll
            for (int b = 0; b < kStreamRB; ++b) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    wv[b][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wrow[b] + k + 32 * j));
            }
#pragma unroll
            for (int tb = 0; tb < kStreamMaxTB; ++tb) {
                if (tb < ntp) {
                    uint4 av[4];
                    if (arow[tb] != nullptr) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const uint4*>(arow[tb] + k + 32 * j);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) av[j] = zero4();
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int b = 0; b < kStreamRB; ++b)
                            acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(wv[b][j]), as_bf16x8(av[j]), acc[tb][b], 0, 0, 0);
                }
            }
        }

        // Cross-wave K reduction in a fixed order, then wave w finishes token block w.
#pragma unroll
        for (int tb = 0; tb < kStreamMaxTB; ++tb)
            if (tb < ntp)
#pragma unroll
                for (int b = 0; b < kStreamRB; ++b) red[wave][tb][b][lane] = acc[tb][b];
        __syncthreads();
        if (wave < ntp && seg + (tb0 + wave) * 16 + r < seg_end) {
            const int tb = wave;
            f32x4_t s[kStreamRB];
#pragma unroll
            for (int b = 0; b < kStreamRB; ++b) {
                s[b] = red[0][tb][b][lane];
#pragma unroll
                for (int w = 1; w < 4; ++w) s[b] += red[w][tb][b][lane];
            }
            // C layout of 16x16 MFMA: lane l holds column (token) l%16 and rows
            // (weight rows) 4*(l/16) + i, i = 0..3.
            const int p = seg + (tb0 + tb) * 16 + r;
            if (DUAL) {
                const int f0 = blockIdx.x * 32;
                bf16_t* hrow = static_cast<bf16_t*>(out) + static_cast<size_t>(p) * Nw;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const f32x4_t a1 = s[half], a3 = s[half + 2];
                    uint2 o;
                    o.x = pack_bf16x2(silu_f32(a1[0]) * a3[0], silu_f32(a1[1]) * a3[1]);
                    o.y = pack_bf16x2(silu_f32(a1[2]) * a3[2], silu_f32(a1[3]) * a3[3]);
                    *reinterpret_cast<uint2*>(hrow + f0 + half * 16 + 4 * g) = o;
                }
            } else {
                const int j0 = blockIdx.x * 64;
                float* yrow = static_cast<float*>(out) + static_cast<size_t>(p) * Nw;
#pragma unroll
                for (int b = 0; b < kStreamRB; ++b)
                    *reinterpret_cast<f32x4_t*>(yrow + j0 + b * 16 + 4 * g) = s[b];
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
    int Kdim, int Nw, int ld_act, int n_src, int P) {
    __shared__ float sa[16][33];
    __shared__ float s1[64][33];
    __shared__ float s3[DUAL ? 64 : 1][33];

    const int p0 = blockIdx.x * 16;
    if (p0 >= offsets[kExperts]) return;
    const int e = expert_of_row(offsets, p0);
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
                if (src >= 0 && src < n_src) arow = act + static_cast<size_t>(src >> 1) * ld_act;
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
                                               pmax_rows(s, 16));
    } else if (tile_m == 16) {
        dim3 grid(s.F / 32, s.n);
        stream_kernel<true><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), row_src, counts,
                                                  offsets, static_cast<const bf16_t*>(w1),
                                                  static_cast<const bf16_t*>(w3), h, s.d, s.F, s.d,
                                                  s.T * s.K, pmax_rows(s, 16));
    } else {
        return launch_tiled(s, true, x, row_src, counts, offsets, w1, w3, h, st);
    }
    return hipGetLastError();
}

hipError_t launch_down(const Shape& s, int tile_m, const void* h, const int32_t* counts,
                       const int32_t* offsets, const void* w2, float* y_perm, hipStream_t st,
                       float* y_perm_hi, int* n_parts) {
    if (n_parts != nullptr) *n_parts = 1;
    if (!s.bf16) {
        dim3 grid(max_tiles(s, 16), (s.d + 63) / 64);
        f32_kernel<false><<<grid, 256, 0, st>>>(static_cast<const float*>(h), nullptr, counts,
                                                offsets, static_cast<const float*>(w2), nullptr,
                                                y_perm, s.F, s.d, s.F, s.T * s.K,
                                                pmax_rows(s, 16));
    } else if (tile_m == 16) {
        dim3 grid(s.d / 64, s.n);
        stream_kernel<false><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(h), nullptr, counts,
                                                   offsets, static_cast<const bf16_t*>(w2), nullptr,
                                                   y_perm, s.F, s.d, s.F, s.T * s.K,
                                                pmax_rows(s, 16));
    } else {
        int ks = 1;
        if (y_perm_hi != nullptr) {
            ks = tiled_down_ksplit(s);
            // the second part lands one P x d block after y_perm
            const size_t P = static_cast<size_t>(pmax_rows(s, 256));
            if (ks == 2 && y_perm_hi != y_perm + P * s.d) ks = 1;
        }
        if (n_parts != nullptr) *n_parts = ks;
        return launch_tiled(s, false, h, nullptr, counts, offsets, w2, nullptr, y_perm, st, ks);
    }
    return hipGetLastError();
}

}  // namespace moe
