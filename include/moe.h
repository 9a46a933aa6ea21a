/*
 * moe.h - C ABI of the MI355X (gfx950) sparse mixture-of-experts feed-forward layer.
 *
 * The layer (Mixtral of Experts; paper-graph-ui page, section 3.4 "MoE Layer
 * Formulation" and "Expert Network Structure (SwiGLU)"; xyznot.com reading
 * guide, "Method (with the key equations)"):
 *
 *     l    = x . W_g                          router logits, W_g in R^{d x n}, no bias
 *     G(x) = Softmax(TopK(l))                 TopK keeps the K largest logits, -inf elsewhere
 *     E_i  = w2_i . (SiLU(w1_i . x) * (w3_i . x))   SwiGLU expert, SiLU(z) = z sigmoid(z)
 *     y    = sum_i G(x)_i E_i(x)              only the K selected experts contribute
 *
 * Weight names: w1 = gate projection (the one that gets SiLU), w3 = up
 * projection (linear), w2 = down projection.  The paper-graph-ui page labels the
 * same three matrices W_{1,i}, W_{2,i}, W_{3,i}; only the labels differ.
 *
 * Conventions for every call:
 *   - Every pointer is a DEVICE pointer (hipMalloc'd or equivalent), row-major,
 *     contiguous, 16-byte aligned.  The caller owns all memory; the library
 *     allocates nothing, keeps no state, retains no pointer and never
 *     synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream) and buffers must stay alive until the stream has passed it.
 *   - Arguments are validated synchronously before anything is enqueued; a
 *     failed validation enqueues nothing and returns the status.  A launch
 *     failure reported by the HIP runtime returns MOE_ERR_HIP.  No C++
 *     exception crosses this interface.
 *   - T == 0 is a valid no-op returning MOE_OK.
 *   - Non-finite inputs give unspecified (but memory-safe) results.
 *   - Tensor shapes: x [T, d]; W_g [d, n] fp32; w1, w3 [n, F, d]; w2 [n, d, F];
 *     y [T, d].  Activations and expert weights share one dtype (fp32 or bf16);
 *     W_g is always fp32.  Accumulation is fp32 throughout.
 *   - Supported: 1 <= top_k <= n_experts, n_experts <= 16, top_k <= 4 (Mixtral
 *     itself is n_experts = 8, top_k = 2; larger values return MOE_ERR_UNSUPPORTED).
 *       fp32: d % 8 == 0, F % 8 == 0.
 *       bf16: d % 512 == 0, F % 512 == 0 (the Mixtral shape d=4096, F=14336 qualifies).
 *     Other shapes return MOE_ERR_UNSUPPORTED.
 *   - Calls on different streams may run concurrently; the library is
 *     stateless and thread-safe.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,   /* null required pointer, negative size, bad tile_m ... */
    MOE_ERR_UNSUPPORTED = 2,        /* valid but not implemented (n > 16, K > 4, shape) */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4                 /* the HIP runtime reported an error at launch */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype_t;

/* Layer shape.  d_model = d, d_ffn = F, n_experts = n, top_k = K. */
typedef struct {
    int32_t d_model;
    int32_t d_ffn;
    int32_t n_experts;
    int32_t top_k;
    int32_t act_dtype;     /* moe_dtype_t of x, y and h: MOE_F32 or MOE_BF16 */
    int32_t weight_dtype;  /* act_dtype, or MOE_FP8_E4M3 with bf16 activations (the _fp8 calls) */
} moe_layer_desc_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char* moe_status_string(moe_status_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t moe_version(void);

/* Padding granularity of the permuted layout that moe_layer_forward uses for T
 * tokens: 16 for fp32 and for bf16 with T <= 64 (weight-streaming kernels),
 * 256 for larger bf16 batches (LDS-tiled MFMA kernels) while tile_m 256 is
 * supported for T (see moe_expert_gate_up), else 16.  Returns 0 if the
 * descriptor is invalid or unsupported. */
int32_t moe_default_tile_m(const moe_layer_desc_t* desc, int32_t T);

/* Worst-case row count P_max of the permuted layout: T*K + n*(tile_m - 1)
 * (every expert segment rounded up to a multiple of tile_m).  Returns -1 on an
 * invalid argument.  tile_m == 0 selects moe_default_tile_m. */
int64_t moe_max_permuted_rows(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m);

/* Bytes of workspace moe_layer_forward needs for T tokens (tile_m == 0 selects
 * the default).  Returns 0 on an invalid argument. */
size_t moe_workspace_size(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m);

/*
 * Router: logits, Top-K and the softmax over the K survivors.
 * (paper-graph-ui page 3.4: gating equation, TopK equation, and the three
 * mechanical steps under "Top-K Gating Mechanism and Routing".)
 *
 *   x          [T, d]  act dtype
 *   w_gate     [d, n]  fp32
 *   topk_idx   [T, K]  int32 out: selected experts, slot 0 = larger logit.
 *                      Ties go to the lower expert index.
 *   topk_gate  [T, K]  fp32 out: softmax weights of the selected experts
 *                      (g0 = 1/(1+exp(l1-l0)), g1 = exp(l1-l0)/(1+exp(l1-l0))).
 *   logits_out [T, n]  fp32 out, optional (NULL skips it).
 * Logits are fp32 sums of fp32 products (bf16 x is widened exactly).
 */
moe_status_t moe_router_topk(const moe_layer_desc_t* desc, int32_t T, const void* x,
                             const float* w_gate, int32_t* topk_idx, float* topk_gate,
                             float* logits_out, void* stream);

/*
 * Dropless grouping of the T*K assignments by expert (the "pack all experts'
 * tokens into one matrix" step that the paper-graph-ui page's "Megablocks
 * kernels" paragraph describes; no capacity limit, no dropping).
 *
 *   topk_idx  [T, K]    int32 in; entries outside [0, n) are ignored (row_of = -1).
 *   counts    [n]       int32 out: assignments per expert.
 *   offsets   [n + 1]   int32 out: segment starts; each segment is padded to a
 *                       multiple of tile_m; offsets[n] = total padded rows.
 *   row_src   [P_max]   int32 out: assignment t*K+s of each permuted row, -1 for
 *                       padding (all P_max entries are written).
 *   row_of    [T, K]    int32 out: permuted row of each assignment.
 * Inside a segment assignments keep ascending t*K+s order (deterministic).
 * tile_m must be 16 or 256 (256 only for bf16 with T > 64 use; see below).
 */
moe_status_t moe_permute(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                         const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                         int32_t* row_src, int32_t* row_of, void* stream);

/*
 * Grouped expert up/gate projection with the SwiGLU gate fused in:
 * for each permuted row p of expert e's segment holding assignment a,
 *     h[p, :] = SiLU(w1[e] . x[a / K]) * (w3[e] . x[a / K])
 * (paper-graph-ui page 3.4, SwiGLU equation).  Padding rows of h are written
 * as zeros.  h [P_max, F] act dtype (bf16 h is rounded once from fp32).
 * counts/offsets/row_src are moe_permute's outputs for the same tile_m.
 * tile_m == 16 selects weight-streaming kernels (suited to few rows per
 * expert; correct for any count), tile_m == 256 selects the LDS-tiled MFMA
 * kernels (bf16 only, and only while T * d_model * 2 bytes stay below 4 GiB;
 * beyond that every call taking tile_m 256 returns MOE_ERR_UNSUPPORTED).
 */
moe_status_t moe_expert_gate_up(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                                const void* x, const int32_t* row_src, const int32_t* counts,
                                const int32_t* offsets, const void* w1, const void* w3,
                                void* h, void* stream);

/*
 * Grouped expert down projection: y_perm[p, :] = w2[e] . h[p, :] for every
 * row of expert e's segment (SwiGLU equation, outer product with w2).
 * y_perm [P_max, d] fp32.  Rows of a segment past counts[e] are unspecified.
 */
moe_status_t moe_expert_down(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                             const void* h, const int32_t* counts, const int32_t* offsets,
                             const void* w2, float* y_perm, void* stream);

/* moe_expert_gate_up followed by moe_expert_down on the same stream. */
moe_status_t moe_grouped_swiglu(const moe_layer_desc_t* desc, int32_t T, int32_t tile_m,
                                const void* x, const int32_t* row_src, const int32_t* counts,
                                const int32_t* offsets, const void* w1, const void* w3,
                                const void* w2, void* h, float* y_perm, void* stream);

/*
 * Gate-weighted combine (paper-graph-ui page 3.4, output equation
 * y = w_1 E_{i1}(x) + w_2 E_{i2}(x)):
 *     y[t, :] = sum_s topk_gate[t, s] * y_perm[row_of[t, s], :]  (+ residual[t, :])
 * summed in fp32 in slot order, then rounded once to the act dtype.
 *   residual [T, d] act dtype or NULL (the residual-stream add of a decoder block).
 *   y        [T, d] act dtype out (may alias residual).
 * row_of entries < 0 contribute nothing.
 */
moe_status_t moe_combine(const moe_layer_desc_t* desc, int32_t T, const float* y_perm,
                         const int32_t* row_of, const float* topk_gate, const void* residual,
                         void* y, void* stream);

/*
 * RMSNorm with unit gain: x_out[t, :] = h[t, :] / sqrt(mean(h[t, :]^2) + eps)
 * (pre-norm before the MoE block; paper-graph-ui page 3.4, "Architectural
 * Inheritance from Mistral 7B", layer normalization).  fp32 arithmetic, one
 * rounding to `dtype`.  d % 8 == 0.  x_out must not alias h.
 */
moe_status_t moe_rmsnorm(int32_t T, int32_t d, int32_t dtype, const void* h, float eps,
                         void* x_out, void* stream);

/*
 * The whole layer, y = sum_i G(x)_i E_i(x) with G(x) = Softmax(TopK(x . W_g))
 * and SwiGLU experts E_i (paper-graph-ui page, section 3.4 "MoE Layer
 * Formulation": gating, TopK and output equations, and "Expert Network
 * Structure (SwiGLU)"; xyznot.com reading guide, "Method (with the key
 * equations)"), computed sparsely: router -> permute -> gate/up + SwiGLU ->
 * down -> combine, so only the K selected experts run on each token.
 *   x, w_gate, w1, w3, w2   as above
 *   residual                [T, d] or NULL; added to y when present
 *   y                       [T, d] out (may alias residual, must not alias x)
 *   topk_idx_out [T,K], topk_gate_out [T,K], counts_out [n]: optional copies of
 *                           the routing (NULL skips each)
 *   workspace               device buffer of at least moe_workspace_size(desc, T, 0)
 *                           bytes, 256-byte aligned; its contents are scratch.
 */
moe_status_t moe_layer_forward(const moe_layer_desc_t* desc, int32_t T, const void* x,
                               const float* w_gate, const void* w1, const void* w3,
                               const void* w2, const void* residual, void* y,
                               int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_layer_forward with a HIP event recorded on `stream` before the router and
 * after each of the layer's five stages, so that each stage's duration inside
 * the layer's own launch sequence can be measured (events[i+1] - events[i]:
 * router + top-k, grouping, gate/up + SwiGLU, down projection with its K split
 * and tail pass when the layer takes them, combine).
 *   events  6 hipEvent_t handles, created by the caller (timing enabled);
 *           none may be NULL.  Everything else is as for moe_layer_forward
 *           (bf16 and fp32 descriptors; FP8 returns MOE_ERR_INVALID_ARGUMENT).
 * T == 0 records nothing.
 */
moe_status_t moe_layer_forward_timed(const moe_layer_desc_t* desc, int32_t T, const void* x,
                                     const float* w_gate, const void* w1, const void* w3,
                                     const void* w2, const void* residual, void* y,
                                     int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                                     void* workspace, size_t workspace_bytes, void* const* events,
                                     void* stream);

/*
 * moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call itself allocates nothing: its
 * intermediates live in a scratch array of MOE_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds in each GPU's memory until the process ends (one
 * copy per device, taken on the device current at the call, which must be
 * the device of the buffers and the stream).  The caller still passes inputs
 * and outputs, exactly as for moe_layer_forward.
 *   - T with moe_workspace_size(desc, T, 0) > MOE_NOALLOC_SCRATCH_BYTES returns
 *     MOE_ERR_WORKSPACE_TOO_SMALL (at d = 4096, F = 14336, n = 8, K = 2 that
 *     is every T above 64; decode batches up to 64 tokens fit).
 *   - Every call on a GPU shares that GPU's scratch: calls that overlap on one
 *     GPU (other streams, other host threads) race and must be serialised by
 *     the caller.  Nothing needs clearing between calls: every scratch byte a
 *     call reads is written earlier in the same call.
 *   - FP8 descriptors return MOE_ERR_INVALID_ARGUMENT.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status_t moe_layer_forward_noalloc(const moe_layer_desc_t* desc, int32_t T, const void* x,
                                       const float* w_gate, const void* w1, const void* w3,
                                       const void* w2, const void* residual, void* y,
                                       int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                                       void* stream);

/*
 * One decoder MoE block with attention omitted:
 *     h_out = h + moe_layer(RMSNorm(h))
 * (paper-graph-ui page, section 3.2: the MoE output is added to the residual
 * stream; pre-norm RMSNorm as for moe_rmsnorm).  h_out may alias h.
 * workspace: at least moe_block_workspace_size(desc, T) bytes.
 */
size_t moe_block_workspace_size(const moe_layer_desc_t* desc, int32_t T);
moe_status_t moe_block_forward(const moe_layer_desc_t* desc, int32_t T, const void* h,
                               float eps, const float* w_gate, const void* w1, const void* w3,
                               const void* w2, void* h_out, int32_t* topk_idx_out,
                               int32_t* counts_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * FP8 expert weights.  The pages name FP8 weights as the next serving step
 * (paper-graph-ui page, section 3.4, "TensorRT-LLM integration" paragraph;
 * section 6.1, "Mitigation status") but fix no format.  Here: OCP E4M3 codes
 * (1 byte: sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals; no
 * infinities; largest finite 448) and one fp32 scale per weight row, so that
 * weight[r, c] = decode(code[r, c]) * scale[r].
 *
 * moe_quantize_fp8: per-row quantization of a bf16 matrix w [rows, cols]
 * (cols % 8 == 0; w 16-byte and q 8-byte aligned):
 *     scale[r]  = max_c |w[r, c]| / 448 in fp32 (1 for an all-zero row)
 *     q[r, c]   = E4M3 code of the fp32 quotient w[r, c] / scale[r], rounded
 *                 to nearest with ties to an even mantissa, saturating at 448.
 * Expert weights quantize as rows = n*F (w1, w3) or n*d (w2), cols = d or F.
 */
moe_status_t moe_quantize_fp8(int64_t rows, int32_t cols, const void* w, uint8_t* q, float* scale,
                              void* stream);

/*
 * FP8 variants of the expert projections and of the layer: desc->weight_dtype
 * must be MOE_FP8_E4M3 (bf16 activations; d_model and d_ffn multiples of
 * 1024), and the other expert entry points reject such a descriptor with
 * MOE_ERR_INVALID_ARGUMENT.  Weights: w1, w3 [n, F, d] and w2 [n, d, F] codes;
 * s1, s3 [n, F] and s2 [n, d] fp32 scales (16-byte aligned).  The products
 * run on the exact E4M3 values in bf16 MFMAs with fp32 accumulation; each
 * output's sum is multiplied by its row's scale before the SiLU gate (gate/up)
 * or the store (down).  Always the weight-streaming kernels (tile_m 16):
 * moe_permute's layout must be built with tile_m 16, and moe_workspace_size
 * with tile_m 0 gives the layer's workspace.  Everything else is as for the
 * bf16 calls of the same name.
 */
moe_status_t moe_expert_gate_up_fp8(const moe_layer_desc_t* desc, int32_t T, const void* x,
                                    const int32_t* row_src, const int32_t* counts, const int32_t* offsets,
                                    const uint8_t* w1, const float* s1, const uint8_t* w3, const float* s3,
                                    void* h, void* stream);
moe_status_t moe_expert_down_fp8(const moe_layer_desc_t* desc, int32_t T, const void* h, const int32_t* counts,
                                 const int32_t* offsets, const uint8_t* w2, const float* s2, float* y_perm,
                                 void* stream);
moe_status_t moe_layer_forward_fp8(const moe_layer_desc_t* desc, int32_t T, const void* x, const float* w_gate,
                                   const uint8_t* w1, const float* s1, const uint8_t* w3, const float* s3,
                                   const uint8_t* w2, const float* s2, const void* residual, void* y,
                                   int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of the layer (bf16 activations and weights).  For the upstream
 * gradient dy of y = sum_i G(x)_i E_i(x) it writes the gradients of
 * sum(dy * y) with respect to every input, by the chain rule through the
 * gating equation, the TopK selection (held fixed: masked logits get no
 * gradient), the softmax over the K survivors and the SwiGLU experts
 * (paper-graph-ui page, section 3.4: gating, TopK, output and SwiGLU
 * equations):
 *   dx      [T, d]     bf16 out (must not alias x or dy)
 *   dw_gate [d, n]     fp32 out
 *   dw1, dw3 [n, F, d], dw2 [n, d, F]   fp32 out (overwritten, not accumulated)
 * Nothing of the forward pass is needed: the routing and the gate/up
 * pre-activations are recomputed from x.  Arithmetic: bf16 MFMA products with
 * fp32 accumulation; the pre-activations stay fp32, their gradients and g*h
 * are rounded once to bf16 (the operands of the next products); every
 * reduction over tokens runs in fp32 in a fixed order (deterministic).
 * T == 0 writes zero weight gradients.  Supported: bf16 layers with
 * (T * K + 255) * 2F * 2 bytes below 4 GiB (the longest 32-bit addressed span:
 * one expert's rows of the pre-activation gradients); else MOE_ERR_UNSUPPORTED.
 * workspace: at least moe_backward_workspace_size(desc, T) bytes, 256-byte
 * aligned (0 = unsupported descriptor).
 */
size_t moe_backward_workspace_size(const moe_layer_desc_t* desc, int32_t T);
moe_status_t moe_layer_backward(const moe_layer_desc_t* desc, int32_t T, const void* x, const float* w_gate,
                                const void* w1, const void* w3, const void* w2, const void* dy, void* dx,
                                float* dw_gate, float* dw1, float* dw3, float* dw2, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
