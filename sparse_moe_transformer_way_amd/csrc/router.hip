// Router: logits l = x . W_g (fp32), Top-K with ties to the lower expert index,
// and the softmax over the K survivors.
//
// Mixtral of Experts, paper-graph-ui page, section 3.4 "MoE Layer Formulation"
// (G(x) = Softmax(TopK(x . W_g)), TopK sets the non-selected logits to -inf) and
// "Top-K Gating Mechanism and Routing" (no bias; pick the largest, mask,
// softmax; Mixtral takes K = 2 of n = 8).  Softmax of a vector whose other
// entries are -inf reduces to the K-term form over the survivors only.
//
// Layout: a block of 4 waves handles TOK tokens (8, 4 with 16 expert slots, or 1 for small batches so
// that a decode step still spreads over T blocks); the d channels are cut into
// 8-channel chunks and wave w takes the w-th quarter of the chunks, so a token's
// dot products are spread over 256 lanes (few sequential steps even at decode
// batch sizes).  Lane j of a wave covers chunks j, j+64, ... of its quarter:
// x loads are 16-byte (bf16) or 32-byte (fp32) per lane and contiguous across
// the wave, and the matching 8 rows of W_g (8 x 8 fp32 = 256 B) are contiguous
// per lane.  Per-lane partial sums go through an xor butterfly inside the wave,
// then the 4 wave sums are added in wave order through LDS (a fixed order, so
// the logits are deterministic), and lane t of wave 0 finishes token t.
// NE is the compile-time expert slot count (8 or 16); W_g takes the vector
// path when n == NE and a scalar one otherwise.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kWaves = 4;         // waves per block, splitting d
constexpr int kSmallT = 256;      // up to this many tokens: one token per block

// Whether (v, i) comes before (w, j) in the order key (logit descending, then
// expert index ascending); j < 0 marks an empty slot.
__device__ __forceinline__ bool before(float v, int i, float w, int j) {
    return j < 0 || v > w || (v == w && i < j);
}

// The lane's dot products over chunks cb, cb + 64, ... of [cbeg, cend) for
// TOK tokens (rows past T read row T - 1; their sums are never used).  U
// chunks per pass, all of their loads issued before any multiply-add: at
// d = 4096 a decode block's lanes cover two chunks each, and one pass then
// costs one memory round trip instead of two.  FULL: W_g rows are NE floats
// (vector loads); otherwise n floats, padded with zeros.
template <bool BF16, int TOK, int NE, bool FULL>
__device__ __forceinline__ void chunk_dots(const void* __restrict__ xv, const float* __restrict__ wg, int T, int d,
                                           int n, int t0, int cbeg, int cend, int lane, float (&acc)[TOK][NE]) {
    constexpr int U = (TOK == 1 && NE == 8) ? 2 : 1;
    for (int cb = cbeg + lane; cb < cend; cb += 64 * U) {
        float w[U][8][NE];
        float xf[U][TOK][8];
        bool in[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ch = cb + 64 * u;
            in[u] = ch < cend;  // a chunk past the wave's range is loaded in range, then zeroed
            const int k0 = (in[u] ? ch : cbeg) * 8;
            if (FULL) {
                const float4* wp = reinterpret_cast<const float4*>(wg + static_cast<size_t>(k0) * NE);
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int q = 0; q < NE / 4; ++q) {
                        const float4 a = wp[j * (NE / 4) + q];
                        w[u][j][4 * q] = a.x; w[u][j][4 * q + 1] = a.y; w[u][j][4 * q + 2] = a.z; w[u][j][4 * q + 3] = a.w;
                    }
            } else {
                const float* wr = wg + static_cast<size_t>(k0) * n;
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int e = 0; e < NE; ++e) w[u][j][e] = e < n ? wr[j * n + e] : 0.0f;
            }
#pragma unroll
            for (int t = 0; t < TOK; ++t) {
                const int tok = min(t0 + t, T - 1);
                if (BF16) {
                    const bf16_t* xr = static_cast<const bf16_t*>(xv) + static_cast<size_t>(tok) * d + k0;
                    unpack_bf16x8(*reinterpret_cast<const uint4*>(xr), xf[u][t]);
                } else {
                    const float* xr = static_cast<const float*>(xv) + static_cast<size_t>(tok) * d + k0;
                    const float4 a = reinterpret_cast<const float4*>(xr)[0];
                    const float4 b = reinterpret_cast<const float4*>(xr)[1];
                    xf[u][t][0] = a.x; xf[u][t][1] = a.y; xf[u][t][2] = a.z; xf[u][t][3] = a.w;
                    xf[u][t][4] = b.x; xf[u][t][5] = b.y; xf[u][t][6] = b.z; xf[u][t][7] = b.w;
                }
            }
        }
        // An unused chunk adds 0 * 0 (selected, not branched around: a branch
        // lets the compiler sink that chunk's loads behind the first one's
        // multiply-adds, a second round trip).
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < TOK; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int e = 0; e < NE; ++e)
                        acc[t][e] = fmaf(in[u] ? xf[u][t][j] : 0.0f, in[u] ? w[u][j][e] : 0.0f, acc[t][e]);
    }
}

// TOK tokens per block, NE = expert slots (n <= NE experts are real).
template <bool BF16, int TOK, int NE>
__global__ __launch_bounds__(256) void router_topk_kernel(const void* __restrict__ xv,
                                                          const float* __restrict__ wg, int T, int d, int n,
                                                          int K, int32_t* __restrict__ idx,
                                                          float* __restrict__ gate,
                                                          float* __restrict__ logits) {
    __shared__ float part[kWaves][TOK][NE];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * TOK;
    const int nch = d >> 3;
    const int cbeg = wave * nch / kWaves;
    const int cend = (wave + 1) * nch / kWaves;

    float acc[TOK][NE];
#pragma unroll
    for (int t = 0; t < TOK; ++t)
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[t][e] = 0.0f;
    if (n == NE)
        chunk_dots<BF16, TOK, NE, true>(xv, wg, T, d, n, t0, cbeg, cend, lane, acc);
    else
        chunk_dots<BF16, TOK, NE, false>(xv, wg, T, d, n, t0, cbeg, cend, lane, acc);

    // Wave sums of the V = TOK * NE partial sums by recursive halving: at the
    // step with lane offset o, a lane keeps half of its remaining values (the
    // upper half if its lane bit o is set), sends the other half to lane ^ o
    // and adds what it receives.  After log2 V steps lane L holds value
    // L >> (6 - log2 V) summed over the V lanes that share its low bits; a
    // butterfly over those bits completes the sum.  63 exchanges for 64
    // values, against 384 for a butterfly per value.
    constexpr int V = TOK * NE;
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "a power of two up to 64 values");
    float vals[V];
#pragma unroll
    for (int t = 0; t < TOK; ++t)
#pragma unroll
        for (int e = 0; e < NE; ++e) vals[t * NE + e] = acc[t][e];
#pragma unroll
    for (int half = V / 2, off = 32; half >= 1; half >>= 1, off >>= 1) {
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = upper ? vals[i] : vals[i + half];
            const float keep = upper ? vals[i + half] : vals[i];
            vals[i] = keep + __shfl_xor(send, off, 64);
        }
    }
    constexpr int kLow = 64 / V;  // lanes that hold parts of the same value
#pragma unroll
    for (int off = kLow / 2; off >= 1; off >>= 1) vals[0] += __shfl_xor(vals[0], off, 64);
    if ((lane & (kLow - 1)) == 0) (&part[wave][0][0])[lane / kLow] = vals[0];
    __syncthreads();
    if (wave != 0 || lane >= TOK) return;
    const int t = lane;
    const int tok = t0 + t;
    if (tok >= T) return;
    float l[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e)
        l[e] = ((part[0][t][e] + part[1][t][e]) + part[2][t][e]) + part[3][t][e];
    // Top-K by the order key: each expert, in index order, is bubbled into the
    // sorted slots; a displaced entry moves down with a full key comparison.
    int ix[kMaxTopK];
    float vx[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        ix[s] = -1;
        vx[s] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        float v = l[e];
        int i = e;
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s) {
            if (e < n && s < K && before(v, i, vx[s], ix[s])) {
                const float tv = vx[s];
                const int ti = ix[s];
                vx[s] = v;
                ix[s] = i;
                v = tv;
                i = ti;
            }
        }
    }
    // Softmax over the K survivors (the others are -inf): e_s = exp(l_s - l_0),
    // g_s = e_s / sum_j e_j, summed in slot order.  For K = 2 this is
    // g0 = 1 / (1 + e), g1 = e / (1 + e) with e = exp(l_1 - l_0).
    float ex[kMaxTopK];
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        ex[s] = s == 0 ? 1.0f : (s < K ? expf(vx[s] - vx[0]) : 0.0f);
        if (s < K) sum += ex[s];
    }
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s < K) {
            idx[static_cast<size_t>(tok) * K + s] = ix[s];
            gate[static_cast<size_t>(tok) * K + s] = ex[s] / sum;
        }
    }
    if (logits != nullptr) {
        float* lp = logits + static_cast<size_t>(tok) * n;
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (e < n) lp[e] = l[e];
    }
}

template <int TOK, int NE>
void launch_router(const Shape& s, const void* x, const float* wg, int32_t* idx, float* gate, float* logits,
                   hipStream_t st) {
    const int blocks = (s.T + TOK - 1) / TOK;
    if (s.bf16)
        router_topk_kernel<true, TOK, NE><<<blocks, 256, 0, st>>>(x, wg, s.T, s.d, s.n, s.K, idx, gate, logits);
    else
        router_topk_kernel<false, TOK, NE><<<blocks, 256, 0, st>>>(x, wg, s.T, s.d, s.n, s.K, idx, gate, logits);
}

}  // namespace

hipError_t launch_router_topk(const Shape& s, const void* x, const float* wg, int32_t* idx,
                              float* gate, float* logits, hipStream_t st) {
    // Each block reads all of W_g (d x n fp32, from L2): one token per block
    // for small batches, several when W_g reuse matters more than parallelism.
    const bool small = s.T <= kSmallT;
    if (s.n <= 8) {
        if (small)
            launch_router<1, 8>(s, x, wg, idx, gate, logits, st);
        else
            launch_router<8, 8>(s, x, wg, idx, gate, logits, st);
    } else {
        if (small)
            launch_router<1, 16>(s, x, wg, idx, gate, logits, st);
        else
            launch_router<4, 16>(s, x, wg, idx, gate, logits, st);
    }
    return hipGetLastError();
}

}  // namespace moe
