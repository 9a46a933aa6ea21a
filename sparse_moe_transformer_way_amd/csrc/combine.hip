// Gate-weighted combine of the K selected expert outputs (+ optional residual)
// and the unit-gain RMSNorm of the decoder block.
//
// Combine: y = sum_s w_s E_{i_s}(x) (Mixtral of Experts, paper-graph-ui page,
// section 3.4, output equation; two terms in Mixtral), summed in fp32 in slot order; the
// residual-stream add (section 3.2) comes after, then one rounding.
// RMSNorm: x = h / sqrt(mean(h^2) + eps) (section 3.4, "Architectural
// Inheritance from Mistral 7B", layer normalization; unit gain).
//
// Both are HBM-bound streaming kernels: one block per token row, 16-byte
// vector loads of fp32 y_perm rows, 8-byte (bf16) or 16-byte (fp32) stores.
#include "moe_common.h"

namespace moe {

namespace {

// One 4-column group c of token t's output from its loaded slot values a[s]
// (the two K-parts already added; dropped slots are zero) and the residual.
template <bool BF16, int K, bool RES>
__device__ __forceinline__ void combine_store(const float4 (&a)[K], const float (&g)[K], const void* residual,
                                              void* y, size_t o) {
    float v[4] = {g[0] * a[0].x, g[0] * a[0].y, g[0] * a[0].z, g[0] * a[0].w};
#pragma unroll
    for (int s = 1; s < K; ++s) {
        v[0] += g[s] * a[s].x; v[1] += g[s] * a[s].y; v[2] += g[s] * a[s].z; v[3] += g[s] * a[s].w;
    }
    if (BF16) {
        if constexpr (RES) {
            const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(residual) + o);
            v[0] += __uint_as_float(r.x << 16); v[1] += __uint_as_float(r.x & 0xffff0000u);
            v[2] += __uint_as_float(r.y << 16); v[3] += __uint_as_float(r.y & 0xffff0000u);
        }
        uint2 out;
        out.x = pack_bf16x2(v[0], v[1]);
        out.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(y) + o) = out;
    } else {
        if constexpr (RES) {
            const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(residual) + o);
            v[0] += r.x; v[1] += r.y; v[2] += r.z; v[3] += r.w;
        }
        *reinterpret_cast<float4*>(static_cast<float*>(y) + o) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// Slot s of group c: y_perm row r[s] (+ its second K-part where the down
// projection wrote one: hkeep[s] all ones), zero for a dropped slot (r < 0
// reads row 0 and discards it).
__device__ __forceinline__ float masked(float v, uint32_t m) { return __uint_as_float(__float_as_uint(v) & m); }

template <int K, bool HI>
__device__ __forceinline__ void combine_load(const float4* const (&p)[K], const float4* const (&q)[K],
                                             const uint32_t (&keep)[K], const uint32_t (&hkeep)[K], int c,
                                             float4 (&a)[K]) {
#pragma unroll
    for (int s = 0; s < K; ++s) {
        float4 v = p[s][c];
        if constexpr (HI) {
            const float4 v2 = q[s][c];
            v.x += masked(v2.x, hkeep[s]); v.y += masked(v2.y, hkeep[s]);
            v.z += masked(v2.z, hkeep[s]); v.w += masked(v2.w, hkeep[s]);
        }
        // a bit mask, not a select: the compiler turns a select on a uniform
        // flag into a branch and sinks the loads into it
        a[s] = make_float4(__uint_as_float(__float_as_uint(v.x) & keep[s]), __uint_as_float(__float_as_uint(v.y) & keep[s]),
                           __uint_as_float(__float_as_uint(v.z) & keep[s]), __uint_as_float(__float_as_uint(v.w) & keep[s]));
    }
}

// Token t's d outputs: full passes of U groups per thread with every load
// issued before the first store (a decode row, d = 4096, is one pass), then a
// plain loop for what is left.
template <bool BF16, int K, bool HI, bool RES, int U>
__device__ __forceinline__ void combine_rows(const float4* const (&p)[K], const float4* const (&q)[K],
                                             const uint32_t (&keep)[K], const uint32_t (&hkeep)[K],
                                             const float (&g)[K], const void* residual, void* y, int t, int d) {
    const int n4 = d / 4;
    int c = threadIdx.x;
    for (; c + (U - 1) * 256 < n4; c += U * 256) {
        float4 a[U][K];
#pragma unroll
        for (int u = 0; u < U; ++u) combine_load<K, HI>(p, q, keep, hkeep, c + 256 * u, a[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            combine_store<BF16, K, RES>(a[u], g, residual, y, static_cast<size_t>(t) * d + 4 * (c + 256 * u));
    }
    for (; c < n4; c += 256) {
        float4 a[K];
        combine_load<K, HI>(p, q, keep, hkeep, c, a);
        combine_store<BF16, K, RES>(a, g, residual, y, static_cast<size_t>(t) * d + 4 * c);
    }
}

// The down projection's second K-partials (HI): the tiled kernel's part 1 in
// y_perm_hi (rows of the tiles it computed, when the plan cut K in two) and the
// tail pass's part 1 in y_tail_hi (tail row i of expert e at row
// e * kTailRows + i).  The combine takes the same plan from the same counts.
struct HiParts {
    const float* y_perm_hi;
    const float* y_tail_hi;
    const int32_t* counts;
    const int32_t* offsets;
    int n_exp;
    int ks_max;
};

// One block of 256 threads per token.  HI: the layer's down projection may
// have written second K-partials; RES: a residual is added.  residual may be
// y itself (the in-place update of a residual stream): neither is marked
// __restrict__, and each element of the residual is read by the thread that
// writes it, before that write.
template <bool BF16, int K, bool HI, bool RES>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gate,
                                                      const void* residual, void* y,
                                                      int d, HiParts hp) {
    constexpr int U = 4;
    const int t = blockIdx.x;
    float g[K];
    uint32_t keep[K];   // all ones for a kept slot, zero for a dropped one
    uint32_t hkeep[K];  // all ones where the slot's row has a second K-partial
    const float4* p[K];
    const float4* q[K];
    LaneSeg ls{0, 0, 0};
    DownPlan plan{1, 0};
    if (HI) {
        ls = lane_segment(hp.offsets, hp.counts, hp.n_exp);
        plan = down_plan(ls, d / kTiledRows, hp.ks_max);
    }
#pragma unroll
    for (int s = 0; s < K; ++s) {
        const int r = row_of[K * t + s];
        g[s] = gate[K * t + s];
        keep[s] = r >= 0 ? 0xffffffffu : 0u;
        const int rr = r < 0 ? 0 : r;
        const size_t row = static_cast<size_t>(rr) * d;
        p[s] = reinterpret_cast<const float4*>(y_perm + row);
        q[s] = p[s];
        hkeep[s] = 0u;
        if (HI && (plan.tail_rows > 0 || plan.ks == 2)) {
            // the expert of row rr (the same in every lane: one token per
            // block): the last expert whose segment starts at or before it
            const int ru = __builtin_amdgcn_readfirstlane(rr);
            const uint64_t at = __ballot(static_cast<int>(threadIdx.x & 63) < hp.n_exp && ls.off <= ru);
            const int e = at == 0 ? 0 : 63 - static_cast<int>(__builtin_clzll(at));
            const int off = __builtin_amdgcn_readlane(ls.off, e);
            const int c = __builtin_amdgcn_readlane(ls.cnt, e);
            const int rem = c % kTiledRows;
            const int tail0 = off + c - rem;
            if (rem > 0 && rem <= plan.tail_rows && rr >= tail0) {
                if (hp.y_tail_hi != nullptr) {
                    q[s] = reinterpret_cast<const float4*>(hp.y_tail_hi +
                                                           static_cast<size_t>(e * kTailRows + rr - tail0) * d);
                    hkeep[s] = 0xffffffffu;
                }
            } else if (plan.ks == 2) {
                q[s] = reinterpret_cast<const float4*>(hp.y_perm_hi + row);
                hkeep[s] = 0xffffffffu;
            }
        }
    }
    // Most tokens have no second partial in any slot (at prefill only the few
    // tail rows do): those take the plain loop, without the extra loads.
    uint32_t any = 0;
#pragma unroll
    for (int s = 0; s < K; ++s) any |= hkeep[s];
    if (HI && __builtin_amdgcn_readfirstlane(any) != 0)
        combine_rows<BF16, K, HI, RES, U>(p, q, keep, hkeep, g, residual, y, t, d);
    else
        combine_rows<BF16, K, false, RES, U>(p, q, keep, hkeep, g, residual, y, t, d);
}

template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ h, float eps,
                                                      void* __restrict__ x, int d) {
    __shared__ float s_part[4];
    const int t = blockIdx.x;
    const size_t base = static_cast<size_t>(t) * d;
    float ss = 0.0f;
    for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
        float f[8];
        if (BF16) {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(h) + base + 8 * c), f);
        } else {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(h) + base + 8 * c);
            const float4 a = p[0], b = p[1];
            f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(f[j], f[j], ss);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float total = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
    const float denom = sqrtf(total / static_cast<float>(d) + eps);
    for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
        float f[8];
        if (BF16) {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(h) + base + 8 * c), f);
            uint4 o;
            o.x = pack_bf16x2(f[0] / denom, f[1] / denom);
            o.y = pack_bf16x2(f[2] / denom, f[3] / denom);
            o.z = pack_bf16x2(f[4] / denom, f[5] / denom);
            o.w = pack_bf16x2(f[6] / denom, f[7] / denom);
            *reinterpret_cast<uint4*>(static_cast<bf16_t*>(x) + base + 8 * c) = o;
        } else {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(h) + base + 8 * c);
            const float4 a = p[0], b = p[1];
            float4* q = reinterpret_cast<float4*>(static_cast<float*>(x) + base + 8 * c);
            q[0] = make_float4(a.x / denom, a.y / denom, a.z / denom, a.w / denom);
            q[1] = make_float4(b.x / denom, b.y / denom, b.z / denom, b.w / denom);
        }
    }
}

}  // namespace

template <bool BF16, bool HI, bool RES>
static void combine_k(const Shape& s, const float* y_perm, const int32_t* row_of, const float* gate,
                      const void* residual, void* y, hipStream_t st, const HiParts& hp) {
    switch (s.K) {
        case 1: combine_kernel<BF16, 1, HI, RES><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, hp); break;
        case 2: combine_kernel<BF16, 2, HI, RES><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, hp); break;
        case 3: combine_kernel<BF16, 3, HI, RES><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, hp); break;
        default: combine_kernel<BF16, 4, HI, RES><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, hp); break;
    }
}

template <bool BF16>
static void combine_dispatch(const Shape& s, const float* y_perm, const int32_t* row_of, const float* gate,
                             const void* residual, void* y, hipStream_t st, const HiParts& hp) {
    const bool hi = hp.y_perm_hi != nullptr || hp.y_tail_hi != nullptr, res = residual != nullptr;
    if (hi && res) combine_k<BF16, true, true>(s, y_perm, row_of, gate, residual, y, st, hp);
    else if (hi) combine_k<BF16, true, false>(s, y_perm, row_of, gate, residual, y, st, hp);
    else if (res) combine_k<BF16, false, true>(s, y_perm, row_of, gate, residual, y, st, hp);
    else combine_k<BF16, false, false>(s, y_perm, row_of, gate, residual, y, st, hp);
}

hipError_t launch_combine(const Shape& s, const float* y_perm, const int32_t* row_of,
                          const float* gate, const void* residual, void* y, hipStream_t st,
                          const float* y_perm_hi, const float* y_tail_hi, const int32_t* counts,
                          const int32_t* offsets, int ks_max) {
    static_assert(kMaxTopK == 4, "one combine instance per K");
    if (s.K < 1 || s.K > kMaxTopK) return hipErrorInvalidValue;
    if ((y_perm_hi != nullptr || y_tail_hi != nullptr) && (counts == nullptr || offsets == nullptr))
        return hipErrorInvalidValue;
    const HiParts hp{y_perm_hi, y_tail_hi, counts, offsets, s.n, ks_max};
    if (s.bf16)
        combine_dispatch<true>(s, y_perm, row_of, gate, residual, y, st, hp);
    else
        combine_dispatch<false>(s, y_perm, row_of, gate, residual, y, st, hp);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int T, int d, bool bf16, const void* h, float eps, void* x_out,
                          hipStream_t st) {
    if (bf16)
        rmsnorm_kernel<true><<<T, 256, 0, st>>>(h, eps, x_out, d);
    else
        rmsnorm_kernel<false><<<T, 256, 0, st>>>(h, eps, x_out, d);
    return hipGetLastError();
}

}  // namespace moe
