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

template <bool BF16, int K>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gate,
                                                      const void* __restrict__ residual, void* y,
                                                      int d, const float* __restrict__ y_perm_hi) {
    const int t = blockIdx.x;
    int r[K];
    float g[K];
    const float4* p[K];
#pragma unroll
    for (int s = 0; s < K; ++s) {
        r[s] = row_of[K * t + s];
        g[s] = gate[K * t + s];
        p[s] = reinterpret_cast<const float4*>(y_perm + static_cast<size_t>(r[s] < 0 ? 0 : r[s]) * d);
    }
    for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < K; ++s) {
            if (r[s] < 0) continue;
            float4 a = p[s][c];
            if (y_perm_hi != nullptr) {
                const float4 a2 = reinterpret_cast<const float4*>(y_perm_hi + static_cast<size_t>(r[s]) * d)[c];
                a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
            }
            if (s == 0) {
                v[0] = g[s] * a.x; v[1] = g[s] * a.y; v[2] = g[s] * a.z; v[3] = g[s] * a.w;
            } else {
                v[0] += g[s] * a.x; v[1] += g[s] * a.y; v[2] += g[s] * a.z; v[3] += g[s] * a.w;
            }
        }
        const size_t o = static_cast<size_t>(t) * d + 4 * c;
        if (BF16) {
            if (residual != nullptr) {
                const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(residual) + o);
                v[0] += __uint_as_float(r.x << 16); v[1] += __uint_as_float(r.x & 0xffff0000u);
                v[2] += __uint_as_float(r.y << 16); v[3] += __uint_as_float(r.y & 0xffff0000u);
            }
            uint2 out;
            out.x = pack_bf16x2(v[0], v[1]);
            out.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(y) + o) = out;
        } else {
            if (residual != nullptr) {
                const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(residual) + o);
                v[0] += r.x; v[1] += r.y; v[2] += r.z; v[3] += r.w;
            }
            *reinterpret_cast<float4*>(static_cast<float*>(y) + o) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
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

template <bool BF16>
static void combine_k(const Shape& s, const float* y_perm, const int32_t* row_of, const float* gate,
                      const void* residual, void* y, hipStream_t st, const float* y_perm_hi) {
    switch (s.K) {
        case 1: combine_kernel<BF16, 1><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, y_perm_hi); break;
        case 2: combine_kernel<BF16, 2><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, y_perm_hi); break;
        case 3: combine_kernel<BF16, 3><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, y_perm_hi); break;
        default: combine_kernel<BF16, 4><<<s.T, 256, 0, st>>>(y_perm, row_of, gate, residual, y, s.d, y_perm_hi); break;
    }
}

hipError_t launch_combine(const Shape& s, const float* y_perm, const int32_t* row_of,
                          const float* gate, const void* residual, void* y, hipStream_t st,
                          const float* y_perm_hi) {
    static_assert(kMaxTopK == 4, "one combine instance per K");
    if (s.K < 1 || s.K > kMaxTopK) return hipErrorInvalidValue;
    if (s.bf16)
        combine_k<true>(s, y_perm, row_of, gate, residual, y, st, y_perm_hi);
    else
        combine_k<false>(s, y_perm, row_of, gate, residual, y, st, y_perm_hi);
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
