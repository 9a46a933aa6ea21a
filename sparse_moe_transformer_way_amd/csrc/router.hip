// Router: logits l = x . W_g (fp32), Top-2 with ties to the lower expert index,
// and the softmax over the two survivors.
//
// Mixtral of Experts, paper-graph-ui page, section 3.4 "MoE Layer Formulation"
// (G(x) = Softmax(TopK(x . W_g)), TopK sets the non-selected logits to -inf) and
// "Top-K Gating Mechanism and Routing" (no bias; pick the two largest, mask,
// softmax).  Softmax of a vector whose other entries are -inf reduces to the
// two-term form g0 = 1/(1+e), g1 = e/(1+e), e = exp(l_second - l_first).
//
// Layout: a block of 4 waves handles TOK tokens (8, or 1 for small batches so
// that a decode step still spreads over T blocks); the d channels are cut into
// 8-channel chunks and wave w takes the w-th quarter of the chunks, so a token's
// dot products are spread over 256 lanes (few sequential steps even at decode
// batch sizes).  Lane j of a wave covers chunks j, j+64, ... of its quarter:
// x loads are 16-byte (bf16) or 32-byte (fp32) per lane and contiguous across
// the wave, and the matching 8 rows of W_g (8 x 8 fp32 = 256 B) are contiguous
// per lane.  Per-lane partial sums go through an xor butterfly inside the wave,
// then the 4 wave sums are added in wave order through LDS (a fixed order, so
// the logits are deterministic), and lane t of wave 0 finishes token t.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kExperts = 8;
constexpr int kWaves = 4;         // waves per block, splitting d
constexpr int kSmallT = 256;      // up to this many tokens: one token per block

template <bool BF16, int kTok>
__global__ __launch_bounds__(256) void router_topk_kernel(const void* __restrict__ xv,
                                                          const float* __restrict__ wg, int T,
                                                          int d, int32_t* __restrict__ idx,
                                                          float* __restrict__ gate,
                                                          float* __restrict__ logits) {
    __shared__ float part[kWaves][kTok][kExperts];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kTok;
    const int nch = d >> 3;
    const int cbeg = wave * nch / kWaves;
    const int cend = (wave + 1) * nch / kWaves;

    float acc[kTok][kExperts];
#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
        for (int e = 0; e < kExperts; ++e) acc[t][e] = 0.0f;

    for (int ch = cbeg + lane; ch < cend; ch += 64) {
        const int k0 = ch * 8;
        float w[8][kExperts];
        const float4* wp = reinterpret_cast<const float4*>(wg + static_cast<size_t>(k0) * kExperts);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float4 a = wp[2 * j], b = wp[2 * j + 1];
            w[j][0] = a.x; w[j][1] = a.y; w[j][2] = a.z; w[j][3] = a.w;
            w[j][4] = b.x; w[j][5] = b.y; w[j][6] = b.z; w[j][7] = b.w;
        }
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
            if (t0 + t < T) {
                float xf[8];
                if (BF16) {
                    const bf16_t* xr = static_cast<const bf16_t*>(xv) + static_cast<size_t>(t0 + t) * d + k0;
                    unpack_bf16x8(*reinterpret_cast<const uint4*>(xr), xf);
                } else {
                    const float* xr = static_cast<const float*>(xv) + static_cast<size_t>(t0 + t) * d + k0;
                    const float4 a = reinterpret_cast<const float4*>(xr)[0];
                    const float4 b = reinterpret_cast<const float4*>(xr)[1];
                    xf[0] = a.x; xf[1] = a.y; xf[2] = a.z; xf[3] = a.w;
                    xf[4] = b.x; xf[5] = b.y; xf[6] = b.z; xf[7] = b.w;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int e = 0; e < kExperts; ++e) acc[t][e] = fmaf(xf[j], w[j][e], acc[t][e]);
            }
        }
    }

#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
        for (int e = 0; e < kExperts; ++e) {
            float v = acc[t][e];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[t][e] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < kTok; ++t)
#pragma unroll
            for (int e = 0; e < kExperts; ++e) part[wave][t][e] = acc[t][e];
    }
    __syncthreads();
    if (wave != 0 || lane >= kTok) return;
    const int t = lane;
    const int tok = t0 + t;
    if (tok >= T) return;
    float l[kExperts];
#pragma unroll
    for (int e = 0; e < kExperts; ++e)
        l[e] = ((part[0][t][e] + part[1][t][e]) + part[2][t][e]) + part[3][t][e];
    // Order key (logit descending, index ascending): strict '>' keeps the
    // earlier (lower) index on equality.
    int i0 = 0, i1 = -1;
    float v0 = l[0], v1 = -INFINITY;
#pragma unroll
    for (int e = 1; e < kExperts; ++e) {
        const float v = l[e];
        if (v > v0) {
            i1 = i0; v1 = v0; i0 = e; v0 = v;
        } else if (v > v1 || i1 < 0) {
            i1 = e; v1 = v;
        }
    }
    const float ex = expf(v1 - v0);
    const float sum = 1.0f + ex;
    idx[2 * tok] = i0;
    idx[2 * tok + 1] = i1;
    gate[2 * tok] = 1.0f / sum;
    gate[2 * tok + 1] = ex / sum;
    if (logits != nullptr) {
        float4* lp = reinterpret_cast<float4*>(logits + static_cast<size_t>(tok) * kExperts);
        lp[0] = make_float4(l[0], l[1], l[2], l[3]);
        lp[1] = make_float4(l[4], l[5], l[6], l[7]);
    }
}

}  // namespace

hipError_t launch_router_topk(const Shape& s, const void* x, const float* wg, int32_t* idx,
                              float* gate, float* logits, hipStream_t st) {
    // Each block reads all of W_g (d x 8 fp32, from L2): one token per block
    // for small batches, eight when W_g reuse matters more than parallelism.
    if (s.T <= kSmallT) {
        if (s.bf16)
            router_topk_kernel<true, 1><<<s.T, 256, 0, st>>>(x, wg, s.T, s.d, idx, gate, logits);
        else
            router_topk_kernel<false, 1><<<s.T, 256, 0, st>>>(x, wg, s.T, s.d, idx, gate, logits);
    } else {
        const int blocks = (s.T + 7) / 8;
        if (s.bf16)
            router_topk_kernel<true, 8><<<blocks, 256, 0, st>>>(x, wg, s.T, s.d, idx, gate, logits);
        else
            router_topk_kernel<false, 8><<<blocks, 256, 0, st>>>(x, wg, s.T, s.d, idx, gate, logits);
    }
    return hipGetLastError();
}

}  // namespace moe
