// Per-row FP8 (OCP E4M3) quantization of bf16 expert weights.
//
// The pages name FP8 weights as the next step for serving Mixtral but fix no
// format (paper-graph-ui page, section 3.4, "TensorRT-LLM integration"
// paragraph; section 6.1, "Mitigation status").  The format here is OCP E4M3
// (bias 7, subnormals, no infinities, largest finite 448) with one fp32 scale
// per weight row: scale = max|row| / 448 (1 for an all-zero row) and
// code = RNE(w / scale), the division in fp32, saturating at 448.  Scaling by
// rows (output features) lets the GEMMs run on the exact E4M3 values and apply
// the scale once to each output's sum.
//
// One block of 256 threads per row: a max-reduction over the row, then one
// pass that writes 8 codes (8 bytes) per thread step.  HBM-bound; it runs once
// per set of weights, outside the layer.
#include "moe_common.h"

namespace moe {

namespace {

constexpr float kE4M3Max = 448.0f;

// E4M3 code of v, rounded to nearest (ties to an even mantissa), |v| >= 448
// saturated to 448.  The rounding is done on the fp32 bit pattern: in the
// normal range the exponent and top 3 mantissa bits are kept and the 20 bits
// below decide the rounding (a carry moves to the next exponent by itself);
// below 2^-6 the quantum is the subnormal step 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7fffffffu;
    uint32_t code;
    if (a >= 0x43e00000u) {          // |v| >= 448
        code = 0x7eu;
    } else if (a >= 0x3c800000u) {   // |v| >= 2^-6: normal
        const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // fp32 exponent << 3 | 3 mantissa bits
        code = min(r - (120u << 3), 0x7eu);                         // rebias 127 -> 7
    } else {                          // subnormal steps of 2^-9 (8 steps reach 2^-6, code 0x08)
        code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
    }
    return code | sign;
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(const bf16_t* __restrict__ w, int cols,
                                                            uint8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float s_max[4];
    const size_t row = blockIdx.x;
    const uint4* wr = reinterpret_cast<const uint4*>(w + row * cols);
    const int nvec = cols / 8;
    float m = 0.0f;
    for (int c = threadIdx.x; c < nvec; c += 256) {
        float f[8];
        unpack_bf16x8(wr[c], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float s = amax > 0.0f ? amax / kE4M3Max : 1.0f;  // IEEE division
    if (threadIdx.x == 0) scale[row] = s;
    uint2* qr = reinterpret_cast<uint2*>(q + row * cols);
    for (int c = threadIdx.x; c < nvec; c += 256) {
        float f[8];
        unpack_bf16x8(wr[c], f);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo |= e4m3_rne(f[j] / s) << (8 * j);
            hi |= e4m3_rne(f[j + 4] / s) << (8 * j);
        }
        qr[c] = make_uint2(lo, hi);
    }
}

}  // namespace

hipError_t launch_quantize_fp8(int64_t rows, int cols, const void* w, uint8_t* q, float* scale, hipStream_t st) {
    quantize_rows_kernel<<<static_cast<unsigned>(rows), 256, 0, st>>>(static_cast<const bf16_t*>(w), cols, q,
                                                                       scale);
    return hipGetLastError();
}

}  // namespace moe
