// C ABI of the MoE layer library: argument validation, workspace carving and
// launch sequencing.  Every entry point validates synchronously, enqueues its
// kernels on the caller's stream and returns without synchronising.
#include <atomic>
#include <mutex>
#include <new>

#include "../../include/moe.h"
#include "moe_common.h"

namespace {

constexpr int32_t kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int dtype_size(int32_t dt) { return dt == MOE_BF16 ? 2 : 4; }

// Shape checks shared by every call.
moe_status_t check_desc(const moe_layer_desc_t* d) {
    if (d == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (d->d_model <= 0 || d->d_ffn <= 0 || d->n_experts <= 0 || d->top_k <= 0)
        return MOE_ERR_INVALID_ARGUMENT;
    if (d->top_k > d->n_experts) return MOE_ERR_INVALID_ARGUMENT;
    if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (d->weight_dtype != MOE_F32 && d->weight_dtype != MOE_BF16 && d->weight_dtype != MOE_FP8_E4M3)
        return MOE_ERR_INVALID_ARGUMENT;
    if (d->d_model % 8 != 0 || d->d_ffn % 8 != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (d->weight_dtype == MOE_FP8_E4M3) {
        // FP8 weights: bf16 activations, weight-streaming kernels (128-k stages per wave)
        if (d->act_dtype != MOE_BF16 || d->d_model % 1024 != 0 || d->d_ffn % 1024 != 0)
            return MOE_ERR_UNSUPPORTED;
    } else if (d->act_dtype != d->weight_dtype) {
        return MOE_ERR_UNSUPPORTED;
    }
    if (d->n_experts > moe::kMaxExperts || d->top_k > moe::kMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (d->act_dtype == MOE_BF16 && (d->d_model % 512 != 0 || d->d_ffn % 512 != 0))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t check_T(int32_t T, const moe_layer_desc_t* d) {
    if (T < 0) return MOE_ERR_INVALID_ARGUMENT;
    // Permuted row indices and T*K assignment ids are int32.
    const long long P = static_cast<long long>(T) * d->top_k + static_cast<long long>(d->n_experts) * 255;
    if (P > 0x7fffffffLL) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

moe::Shape shape_of(const moe_layer_desc_t* d, int32_t T) {
    return moe::Shape{T, d->d_model, d->d_ffn, d->n_experts, d->top_k, d->act_dtype == MOE_BF16};
}

bool is_fp8(const moe_layer_desc_t* d) { return d->weight_dtype == MOE_FP8_E4M3; }

int default_tile(const moe_layer_desc_t* d, int32_t T) {
    if (d->act_dtype != MOE_BF16 || is_fp8(d)) return 16;
    return (T <= 64 || !moe::tiled_fits(shape_of(d, T))) ? 16 : 256;
}

moe_status_t check_tile(const moe_layer_desc_t* d, int32_t T, int32_t tile_m) {
    if (tile_m == 16) return MOE_OK;
    if (tile_m == 256)
        return (d->act_dtype == MOE_BF16 && !is_fp8(d) && moe::tiled_fits(shape_of(d, T))) ? MOE_OK
                                                                                           : MOE_ERR_UNSUPPORTED;
    return MOE_ERR_INVALID_ARGUMENT;
}

long long pmax(const moe_layer_desc_t* d, int32_t T, int32_t tile_m) {
    return static_cast<long long>(T) * d->top_k + static_cast<long long>(d->n_experts) * (tile_m - 1);
}


moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }


// Workspace carving of moe_layer_forward.
struct LayerWs {
    int32_t* idx;
    float* gate;
    int32_t* counts;
    int32_t* offsets;
    int32_t* row_src;
    int32_t* row_of;
    void* h;
    float* y_perm;
    float* y_perm_hi;  // second K-partial of the tiled down projection, or nullptr
    float* y_tail_hi;  // second K-partial of the down tail pass [n * kTailRows, d], or nullptr
    size_t bytes;
};

LayerWs carve_layer(const moe_layer_desc_t* d, int32_t T, int32_t tile_m, char* base) {
    LayerWs w{};
    const size_t TK = static_cast<size_t>(T) * d->top_k;
    const size_t P = static_cast<size_t>(pmax(d, T, tile_m));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base == nullptr ? nullptr : base + off;
        off += align_up(bytes);
        return p;
    };
    w.idx = reinterpret_cast<int32_t*>(take(TK * 4));
    w.gate = reinterpret_cast<float*>(take(TK * 4));
    w.counts = reinterpret_cast<int32_t*>(take(static_cast<size_t>(d->n_experts) * 4));
    w.offsets = reinterpret_cast<int32_t*>(take(static_cast<size_t>(d->n_experts + 1) * 4));
    w.row_src = reinterpret_cast<int32_t*>(take(P * 4));
    w.row_of = reinterpret_cast<int32_t*>(take(TK * 4));
    w.h = take(P * static_cast<size_t>(d->d_ffn) * dtype_size(d->act_dtype));
    // the tiled down projection may write two K-partial sums back to back
    const int parts = (tile_m == 256) ? moe::tiled_down_ksplit(shape_of(d, T)) : 1;
    w.y_perm = reinterpret_cast<float*>(take(parts * P * static_cast<size_t>(d->d_model) * 4));
    w.y_perm_hi = parts == 2 && base != nullptr ? w.y_perm + P * static_cast<size_t>(d->d_model) : nullptr;
    // and the tail pass cuts K in two with its second partial in a small buffer
    const bool tail_hi = tile_m == 256 && d->d_ffn % 1024 == 0;
    w.y_tail_hi = reinterpret_cast<float*>(
        take(tail_hi ? static_cast<size_t>(d->n_experts) * moe::kTailRows * d->d_model * 4 : 0));
    if (!tail_hi) w.y_tail_hi = nullptr;
    w.bytes = off;
    return w;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The layer for either weight format (scales non-null = FP8).
struct ExpertWeights {
    const void* w1;
    const void* w3;
    const void* w2;
    const float* s1;
    const float* s3;
    const float* s2;
};

// Argument checks of the layer (everything but the workspace), before any launch.
moe_status_t check_layer_args(const moe_layer_desc_t* desc, int32_t T, const void* x, const float* w_gate,
                              const ExpertWeights& ew, const void* residual, const void* y) {
    const bool fp8 = is_fp8(desc);
    if (x == nullptr || w_gate == nullptr || ew.w1 == nullptr || ew.w3 == nullptr || ew.w2 == nullptr ||
        y == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (fp8 && (ew.s1 == nullptr || ew.s3 == nullptr || ew.s2 == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    if (x == y) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(ew.w1) || !aligned16(ew.w3) || !aligned16(ew.w2) ||
        !aligned16(y) || (residual != nullptr && !aligned16(residual)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (fp8 && (!aligned16(ew.s1) || !aligned16(ew.s3) || !aligned16(ew.s2))) return MOE_ERR_INVALID_ARGUMENT;
    (void)T;
    return MOE_OK;
}

// The layer's launches on a checked workspace of w.bytes bytes.
// With `marks` (kLayerMarks events, or nullptr) an event is recorded on the
// stream before the router and after each stage.
constexpr int kLayerMarks = 6;

moe_status_t run_layer(const moe_layer_desc_t* desc, int32_t T, int tile_m, const LayerWs& w, const void* x,
                       const float* w_gate, const ExpertWeights& ew, const void* residual, void* y,
                       int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out, void* stream,
                       void* const* marks = nullptr) {
    const bool fp8 = is_fp8(desc);
    const moe::Shape sh = shape_of(desc, T);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int mark = 0;
    auto record = [&]() {
        return marks == nullptr || hipEventRecord(static_cast<hipEvent_t>(marks[mark++]), st) == hipSuccess;
    };
    int32_t* idx = topk_idx_out != nullptr ? topk_idx_out : w.idx;
    float* gate = topk_gate_out != nullptr ? topk_gate_out : w.gate;
    int32_t* counts = counts_out != nullptr ? counts_out : w.counts;
    if (!record()) return MOE_ERR_HIP;
    if (moe::launch_router_topk(sh, x, w_gate, idx, gate, nullptr, st) != hipSuccess || !record())
        return MOE_ERR_HIP;
    if (moe::launch_permute(sh, tile_m, idx, counts, w.offsets, w.row_src, w.row_of, st) != hipSuccess ||
        !record())
        return MOE_ERR_HIP;
    int ks_max = 1;
    if (fp8) {
        const auto* q1 = static_cast<const uint8_t*>(ew.w1);
        const auto* q3 = static_cast<const uint8_t*>(ew.w3);
        const auto* q2 = static_cast<const uint8_t*>(ew.w2);
        if (moe::launch_gate_up_fp8(sh, x, w.row_src, counts, w.offsets, q1, ew.s1, q3, ew.s3, w.h, st) !=
                hipSuccess ||
            !record())
            return MOE_ERR_HIP;
        if (moe::launch_down_fp8(sh, w.h, counts, w.offsets, q2, ew.s2, w.y_perm, st) != hipSuccess || !record())
            return MOE_ERR_HIP;
    } else {
        if (moe::launch_gate_up(sh, tile_m, x, w.row_src, counts, w.offsets, ew.w1, ew.w3, w.h, st) != hipSuccess ||
            !record())
            return MOE_ERR_HIP;
        if (moe::launch_down(sh, tile_m, w.h, counts, w.offsets, ew.w2, w.y_perm, st, w.y_perm_hi, w.y_tail_hi,
                             &ks_max) != hipSuccess ||
            !record())
            return MOE_ERR_HIP;
    }
    if (moe::launch_combine(sh, w.y_perm, w.row_of, gate, residual, y, st, ks_max == 2 ? w.y_perm_hi : nullptr,
                            w.y_tail_hi, counts, w.offsets, ks_max) != hipSuccess ||
        !record())
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status_t layer_forward(const moe_layer_desc_t* desc, int32_t T, const void* x, const float* w_gate,
                           const ExpertWeights& ew, const void* residual, void* y, int32_t* topk_idx_out,
                           float* topk_gate_out, int32_t* counts_out, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* marks = nullptr) {
    moe_status_t s;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if ((s = check_layer_args(desc, T, x, w_gate, ew, residual, y)) != MOE_OK) return s;
    if (workspace == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_ERR_INVALID_ARGUMENT;
    const int tile_m = default_tile(desc, T);
    const LayerWs w = carve_layer(desc, T, tile_m, static_cast<char*>(workspace));
    if (workspace_bytes < w.bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return run_layer(desc, T, tile_m, w, x, w_gate, ew, residual, y, topk_idx_out, topk_gate_out, counts_out,
                     stream, marks);
}

// ---- Scratch of moe_layer_forward_noalloc: one array per GPU in the code
// object's device memory, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it names a stand-in, not
// device memory): each device's address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is used.
constexpr size_t kNoAllocBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

moe_status_t device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

int32_t moe_version(void) { return kVersion; }

int32_t moe_default_tile_m(const moe_layer_desc_t* desc, int32_t T) {
    if (check_desc(desc) != MOE_OK || T < 0) return 0;
    return default_tile(desc, T);
}

int64_t moe_max_permuted_rows(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m) {
    if (check_desc(desc) != MOE_OK || check_T(T, desc) != MOE_OK) return -1;
    if (tile_m == 0) tile_m = default_tile(desc, T);
    if (check_tile(desc, T, tile_m) != MOE_OK) return -1;
    return pmax(desc, T, tile_m);
}

size_t moe_workspace_size(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m) {
    if (check_desc(desc) != MOE_OK || check_T(T, desc) != MOE_OK) return 0;
    if (tile_m == 0) tile_m = default_tile(desc, T);
    if (check_tile(desc, T, tile_m) != MOE_OK) return 0;
    return carve_layer(desc, T, tile_m, nullptr).bytes;
}

moe_status_t moe_router_topk(const moe_layer_desc_t* desc, int32_t T, const void* x,
                             const float* w_gate, int32_t* topk_idx, float* topk_gate,
                             float* logits_out, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (x == nullptr || w_gate == nullptr || topk_idx == nullptr || topk_gate == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w_gate) || (logits_out != nullptr && !aligned16(logits_out)))
        return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_router_topk(shape_of(desc, T), x, w_gate, topk_idx, topk_gate,
                                              logits_out, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                         const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                         int32_t* row_src, int32_t* row_of, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if ((s = check_tile(desc, T, tile_m)) != MOE_OK) return s;
    if (counts == nullptr || offsets == nullptr || row_src == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (T > 0 && (topk_idx == nullptr || row_of == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    // T == 0 still writes counts = 0, offsets = 0 and the all-padding row_src.
    return hip_status(moe::launch_permute(shape_of(desc, T), tile_m, topk_idx, counts, offsets,
                                          row_src, row_of, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_gate_up(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                                const void* x, const int32_t* row_src, const int32_t* counts,
                                const int32_t* offsets, const void* w1, const void* w3, void* h,
                                void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;  // FP8 weights take the _fp8 entry points
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if ((s = check_tile(desc, T, tile_m)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (x == nullptr || row_src == nullptr || counts == nullptr || offsets == nullptr ||
        w1 == nullptr || w3 == nullptr || h == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w1) || !aligned16(w3) || !aligned16(h))
        return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_gate_up(shape_of(desc, T), tile_m, x, row_src, counts, offsets,
                                          w1, w3, h, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_down(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                             const void* h, const int32_t* counts, const int32_t* offsets,
                             const void* w2, float* y_perm, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;  // FP8 weights take the _fp8 entry points
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if ((s = check_tile(desc, T, tile_m)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (h == nullptr || counts == nullptr || offsets == nullptr || w2 == nullptr || y_perm == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(h) || !aligned16(w2) || !aligned16(y_perm)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_down(shape_of(desc, T), tile_m, h, counts, offsets, w2, y_perm,
                                       static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_swiglu(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                                const void* x, const int32_t* row_src, const int32_t* counts,
                                const int32_t* offsets, const void* w1, const void* w3,
                                const void* w2, void* h, float* y_perm, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;  // FP8 weights take the _fp8 entry points
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if ((s = check_tile(desc, T, tile_m)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (w2 == nullptr || y_perm == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    s = moe_expert_gate_up(desc, T, tile_m, x, row_src, counts, offsets, w1, w3, h, stream);
    if (s != MOE_OK) return s;
    return moe_expert_down(desc, T, tile_m, h, counts, offsets, w2, y_perm, stream);
}

moe_status_t moe_combine(const moe_layer_desc_t* desc, int32_t T, const float* y_perm,
                         const int32_t* row_of, const float* topk_gate, const void* residual,
                         void* y, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (y_perm == nullptr || row_of == nullptr || topk_gate == nullptr || y == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(y_perm) || !aligned16(y) || (residual != nullptr && !aligned16(residual)))
        return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_combine(shape_of(desc, T), y_perm, row_of, topk_gate, residual, y,
                                          static_cast<hipStream_t>(stream)));
}

moe_status_t moe_rmsnorm(int32_t T, int32_t d, int32_t dtype, const void* h, float eps,
                         void* x_out, void* stream) {
    if (T < 0 || d <= 0 || d % 8 != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (!(eps >= 0.0f)) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (h == nullptr || x_out == nullptr || h == x_out) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(h) || !aligned16(x_out)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_rmsnorm(T, d, dtype == MOE_BF16, h, eps, x_out,
                                          static_cast<hipStream_t>(stream)));
}

moe_status_t moe_layer_forward(const moe_layer_desc_t* desc, int32_t T, const void* x,
                               const float* w_gate, const void* w1, const void* w3,
                               const void* w2, const void* residual, void* y,
                               int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;  // FP8 weights take the _fp8 entry points
    return layer_forward(desc, T, x, w_gate, ExpertWeights{w1, w3, w2, nullptr, nullptr, nullptr}, residual, y,
                         topk_idx_out, topk_gate_out, counts_out, workspace, workspace_bytes, stream);
}

moe_status_t moe_layer_forward_timed(const moe_layer_desc_t* desc, int32_t T, const void* x,
                                     const float* w_gate, const void* w1, const void* w3, const void* w2,
                                     const void* residual, void* y, int32_t* topk_idx_out, float* topk_gate_out,
                                     int32_t* counts_out, void* workspace, size_t workspace_bytes,
                                     void* const* events, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;
    if (events == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < kLayerMarks; ++i)
        if (events[i] == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    return layer_forward(desc, T, x, w_gate, ExpertWeights{w1, w3, w2, nullptr, nullptr, nullptr}, residual, y,
                         topk_idx_out, topk_gate_out, counts_out, workspace, workspace_bytes, stream, events);
}

moe_status_t moe_layer_forward_noalloc(const moe_layer_desc_t* desc, int32_t T, const void* x,
                                       const float* w_gate, const void* w1, const void* w3, const void* w2,
                                       const void* residual, void* y, int32_t* topk_idx_out,
                                       float* topk_gate_out, int32_t* counts_out, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    const ExpertWeights ew{w1, w3, w2, nullptr, nullptr, nullptr};
    if ((s = check_layer_args(desc, T, x, w_gate, ew, residual, y)) != MOE_OK) return s;
    const int tile_m = default_tile(desc, T);
    if (carve_layer(desc, T, tile_m, nullptr).bytes > kNoAllocBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if ((s = device_scratch(&ws)) != MOE_OK) return s;
    const LayerWs w = carve_layer(desc, T, tile_m, static_cast<char*>(ws));
    return run_layer(desc, T, tile_m, w, x, w_gate, ew, residual, y, topk_idx_out, topk_gate_out, counts_out,
                     stream);
}

size_t moe_block_workspace_size(const moe_layer_desc_t* desc, int32_t T) {
    if (check_desc(desc) != MOE_OK || check_T(T, desc) != MOE_OK) return 0;
    const size_t xn = align_up(static_cast<size_t>(T) * desc->d_model * dtype_size(desc->act_dtype));
    return xn + carve_layer(desc, T, default_tile(desc, T), nullptr).bytes;
}

moe_status_t moe_block_forward(const moe_layer_desc_t* desc, int32_t T, const void* h,
                               float eps, const float* w_gate, const void* w1, const void* w3,
                               const void* w2, void* h_out, int32_t* topk_idx_out,
                               int32_t* counts_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if (!(eps >= 0.0f)) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (h == nullptr || h_out == nullptr || workspace == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_ERR_INVALID_ARGUMENT;
    const size_t need = moe_block_workspace_size(desc, T);
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    const size_t xn = align_up(static_cast<size_t>(T) * desc->d_model * dtype_size(desc->act_dtype));
    char* ws = static_cast<char*>(workspace);
    s = moe_rmsnorm(T, desc->d_model, desc->act_dtype, h, eps, ws, stream);
    if (s != MOE_OK) return s;
    return moe_layer_forward(desc, T, ws, w_gate, w1, w3, w2, h, h_out, topk_idx_out, nullptr,
                             counts_out, ws + xn, workspace_bytes - xn, stream);
}

moe_status_t moe_quantize_fp8(int64_t rows, int32_t cols, const void* w, uint8_t* q, float* scale,
                              void* stream) {
    if (rows < 0 || rows > 0x7fffffffLL || cols <= 0 || cols % 8 != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (rows == 0) return MOE_OK;
    if (w == nullptr || q == nullptr || scale == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(w) || (reinterpret_cast<uintptr_t>(q) & 7u) != 0) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_quantize_fp8(rows, cols, w, q, scale, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_gate_up_fp8(const moe_layer_desc_t* desc, int32_t T, const void* x,
                                    const int32_t* row_src, const int32_t* counts, const int32_t* offsets,
                                    const uint8_t* w1, const float* s1, const uint8_t* w3, const float* s3,
                                    void* h, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (!is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (x == nullptr || row_src == nullptr || counts == nullptr || offsets == nullptr || w1 == nullptr ||
        s1 == nullptr || w3 == nullptr || s3 == nullptr || h == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w1) || !aligned16(w3) || !aligned16(s1) || !aligned16(s3) || !aligned16(h))
        return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_gate_up_fp8(shape_of(desc, T), x, row_src, counts, offsets, w1, s1, w3, s3, h,
                                              static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_down_fp8(const moe_layer_desc_t* desc, int32_t T, const void* h, const int32_t* counts,
                                 const int32_t* offsets, const uint8_t* w2, const float* s2, float* y_perm,
                                 void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (!is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (h == nullptr || counts == nullptr || offsets == nullptr || w2 == nullptr || s2 == nullptr ||
        y_perm == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(h) || !aligned16(w2) || !aligned16(s2) || !aligned16(y_perm)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_down_fp8(shape_of(desc, T), h, counts, offsets, w2, s2, y_perm,
                                           static_cast<hipStream_t>(stream)));
}

moe_status_t moe_layer_forward_fp8(const moe_layer_desc_t* desc, int32_t T, const void* x, const float* w_gate,
                                   const uint8_t* w1, const float* s1, const uint8_t* w3, const float* s3,
                                   const uint8_t* w2, const float* s2, const void* residual, void* y,
                                   int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (!is_fp8(desc)) return MOE_ERR_INVALID_ARGUMENT;
    return layer_forward(desc, T, x, w_gate, ExpertWeights{w1, w3, w2, s1, s3, s2}, residual, y, topk_idx_out,
                         topk_gate_out, counts_out, workspace, workspace_bytes, stream);
}

size_t moe_backward_workspace_size(const moe_layer_desc_t* desc, int32_t T) {
    if (check_desc(desc) != MOE_OK || check_T(T, desc) != MOE_OK) return 0;
    if (desc->act_dtype != MOE_BF16 || is_fp8(desc)) return 0;
    const moe::Shape sh = shape_of(desc, T);
    if (!moe::backward_fits(sh)) return 0;
    return moe::backward_workspace_bytes(sh, nullptr, nullptr);
}

moe_status_t moe_layer_backward(const moe_layer_desc_t* desc, int32_t T, const void* x, const float* w_gate,
                                const void* w1, const void* w3, const void* w2, const void* dy, void* dx,
                                float* dw_gate, float* dw1, float* dw3, float* dw2, void* workspace,
                                size_t workspace_bytes, void* stream) {
    moe_status_t s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (desc->act_dtype != MOE_BF16 || is_fp8(desc)) return MOE_ERR_UNSUPPORTED;
    if ((s = check_T(T, desc)) != MOE_OK) return s;
    const moe::Shape sh = shape_of(desc, T);
    if (!moe::backward_fits(sh)) return MOE_ERR_UNSUPPORTED;
    if (dw_gate == nullptr || dw1 == nullptr || dw3 == nullptr || dw2 == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(dw_gate) || !aligned16(dw1) || !aligned16(dw3) || !aligned16(dw2))
        return MOE_ERR_INVALID_ARGUMENT;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) return hip_status(moe::launch_zero_grads(sh, dw_gate, dw1, dw3, dw2, st));
    if (x == nullptr || w_gate == nullptr || w1 == nullptr || w3 == nullptr || w2 == nullptr || dy == nullptr ||
        dx == nullptr || workspace == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (dx == x || dx == dy) return MOE_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w1) || !aligned16(w3) || !aligned16(w2) ||
        !aligned16(dy) || !aligned16(dx))
        return MOE_ERR_INVALID_ARGUMENT;
    moe::BackwardWs w;
    if (workspace_bytes < moe::backward_workspace_bytes(sh, &w, static_cast<char*>(workspace)))
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(moe::launch_layer_backward(sh, x, w_gate, w1, w3, w2, dy, dx, dw_gate, dw1, dw3, dw2, w, st));
}

}  // extern "C"
