// Backward pass of the Mixtral sparse-MoE layer (bf16 activations and weights,
// fp32 gradients of the weights).
//
// The layer is y = sum_i G(x)_i E_i(x), G(x) = Softmax(TopK(x . W_g)),
// E_i(x) = w2_i . (SiLU(w1_i . x) * (w3_i . x)) (Mixtral of Experts,
// paper-graph-ui page, section 3.4: gating, output and SwiGLU equations).  By
// the chain rule, for a routed assignment (token t, slot s, expert e, gate g)
// at permuted row p:
//   G_p   = w2_e^T dy_t                  [F]   (unscaled down-projection gradient)
//   dg_s  = G_p . h_p                          (= dy_t . E_e(x_t))
//   dh_p  = g G_p,  da3 = dh SiLU(a1),  da1 = dh a3 SiLU'(a1)
//   dx_t += w1_e^T da1 + w3_e^T da3
//   dw2_e += g dy_t (x) h_p,  dw1_e += da1 (x) x_t,  dw3_e += da3 (x) x_t
// and the router gradient is the softmax Jacobian on the K selected logits:
//   dl_s = g_s (dg_s - sum_j g_j dg_j),  dW_g += x_t (x) dl,  dx_t += W_g dl.
//
// The pass recomputes the routing and the gate/up pre-activations a1, a3
// (nothing of the forward pass is kept), then runs five grouped GEMMs through
// MFMA kernels, over the expert-grouped rows padded to 256 (the first product
// reuses the forward pass's tiled gate/up kernel, the others share one kernel):
//   1. a = [a1 | a3] = xp . [w1; w3]^T       K = d, fp32 in 32 x 32 blocks (preact_block;
//                                             the forward gate/up tiled kernel)
//   2. G = dyp . w2                           u = F, v = rows, K = d; epilogue
//      forms h, dg partial sums, da = [da1 | da3] and hg = g h
//   3. dxp = da . [w1; w3]                    u = d, v = rows, K = 2F
//   4. dw2_e = hg^T dyp                       u = F, v = d, K = the expert's rows
//   5. [dw1; dw3]_e = xp^T da                 u = d, v = 2F, K = the expert's rows
// where xp, dyp are x and dy gathered into permuted rows (zero for padding).
// Products 3-5 store their fp32 rows through LDS (store_rows_staged); product
// 2 stores its bf16 outputs 16 bytes per lane after a permlane32 swap.
//
// The GEMM computes C[u][v] = sum_k X[u][k] Y[v][k].  Each operand is stored
// either k-contiguous ([rows][k]) or row-contiguous ([k][rows]); both are
// copied into LDS unchanged by buffer loads with the LDS bit.  Row-contiguous
// tiles feed the MFMAs through the transposing LDS read of gfx950
// (ds_read_b64_tr_b16): in a 16-lane group, lane i addresses row k0 + i/4,
// columns c0 + 4(i%4) .. +3 of a [k][c] tile, and lane j = 4a + b receives
// element b of lanes a, a+4, a+8, a+12, i.e. column c0 + j at k0 .. k0+3 (the
// lane layout was measured on MI355X).
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kTU = 256;  // block tile along u (MFMA rows)
constexpr int kTV = 256;  // block tile along v (MFMA columns); row padding of the layout
constexpr int kBK = 32;   // k per stage
constexpr int kXVec = kTU * kBK * 2 / 16;  // uint4 of an X stage (16 KB)
constexpr int kYVec = kTV * kBK * 2 / 16;  // uint4 of a Y stage (16 KB)
constexpr int kStageVec = kXVec + kYVec;
constexpr int kStages = 4;                 // LDS ring: copies run kStages - 1 stages ahead
constexpr int kCopiesPerStage = (kTU + kTV) / 64;  // buffer loads per thread per stage

// Wait until at most N of this wave's buffer loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // vmcnt bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) left at their maximum
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

typedef void __attribute__((address_space(3)))* lds_ptr_t;
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_t;
typedef __attribute__((address_space(3))) char* lds_char_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bwd_rsrc(const void* base) {
    // dword 3 = 0x00020000: 32-bit data format, the raw-buffer setting of gfx9
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}

// ---------------------------------------------------------------------------
// Operand copies and fragment reads
// ---------------------------------------------------------------------------
//
// k-contiguous tile, ROWS x 32 k, 64 bytes per row: 16-byte granule g of row r
// sits at g ^ f(r), f(r) = ((r >> 2) ^ (r >> 3)) & 3, so the 16 rows of a
// fragment-read phase hit 16 distinct 4-bank groups.  One copy instruction
// fills 16 rows (lane l: row l/4, physical granule l%4).
// Row-contiguous tile, 32 k x ROWS, 2*ROWS bytes per k-row: granule g of k-row
// k sits at g ^ 4(k & 3), so the 4 k-rows of a transposing read land in 4
// different bank groups.  One copy instruction fills 512/ROWS k-rows.

__device__ __forceinline__ int kc_swz(int r) { return ((r >> 2) ^ (r >> 3)) & 3; }

// (a plain struct: the host pass of hipcc rejects a class template holding a
// buffer resource once two kernels share a helper that passes it to a builtin)
struct Operand {
    __amdgpu_buffer_rsrc_t res[2];  // source halves (the second from stage `split` on)
    uint32_t vo[2];                 // lane byte offset, by copy-instruction parity
    uint32_t wfirst;                // bytes from the tile origin to this wave's first copy
    uint32_t jstep;                 // bytes between this wave's copy instructions
    uint32_t kstep;                 // bytes per stage
    int split;                      // first stage read from res[1]
    int rd[4];                      // lane byte offsets of the fragment reads (per 32-row block class)
};

// Copy set-up for an operand whose memory rows have `ld` elements.  The tile's
// origin (row 0 / k 0) is the resource base.
template <bool RC, int ROWS>
__device__ __forceinline__ void operand_setup(Operand& o, int ld, int wave, int lane) {
    constexpr int kInstr = ROWS / 64;  // copy instructions per thread per stage
    if (!RC) {
        // instruction j of wave w: rows w*ROWS/4 + 16j .. +15
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int row = wave * (ROWS / 4) + 16 * par + (lane >> 2);
            const int glog = (lane & 3) ^ kc_swz(row);
            o.vo[par] = static_cast<uint32_t>((lane >> 2) * ld + 8 * glog) * 2u;
        }
        o.wfirst = static_cast<uint32_t>(wave * (ROWS / 4)) * ld * 2u;
        o.jstep = 16u * ld * 2u;
        o.kstep = kBK * 2;
    } else {
        constexpr int kKR = 512 / ROWS;        // k-rows per copy instruction
        constexpr int kGr = ROWS / 8;          // granules per k-row
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int k = (wave * kInstr + par) * kKR + lane / kGr;
            const int glog = (lane % kGr) ^ (4 * (k & 3));
            o.vo[par] = static_cast<uint32_t>((lane / kGr) * ld + 8 * glog) * 2u;
        }
        o.wfirst = static_cast<uint32_t>(wave * kInstr * kKR) * ld * 2u;
        o.jstep = static_cast<uint32_t>(kKR) * ld * 2u;
        o.kstep = static_cast<uint32_t>(kBK) * ld * 2u;
    }
}

// Fragment-read offsets: `rb` = first row of the wave's part of the tile
// (a multiple of 32); block b adds 32 rows.
template <bool RC, int ROWS>
__device__ __forceinline__ void operand_reads(Operand& o, int rb, int lane) {
    const int fk = lane >> 5;
    if (!RC) {
        // 32x32x16 operand: lane (r = l%32, fk) takes k 8fk..8fk+7 of row r;
        // class t = k16 step (0, 1) of the stage; blocks add 32 rows (f unchanged)
        const int row = rb + (lane & 31);
#pragma unroll
        for (int t = 0; t < 2; ++t) o.rd[t] = row * 64 + (((2 * t + fk) ^ kc_swz(row)) << 4);
    } else {
        // transposing reads: lane i of a 16-lane group addresses k-row
        // k0 + i/4 (k0 = 16t + 8fk + 4r), columns c0 + 4(i%4), c0 = row block + 16((l/16)&1)
        const int q = (lane & 15) >> 2;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = rb + 32 * b + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            o.rd[b] = (8 * fk + q) * ROWS * 2 + (((col >> 3) ^ (4 * q)) << 4) + (col & 7) * 2;
        }
    }
}

template <bool RC, int ROWS>
__device__ __forceinline__ void operand_copy(const Operand& o, uint4* dst, int stage, int wave) {
    constexpr int kInstr = ROWS / 64;
    const int half = stage >= o.split ? 1 : 0;
    const uint32_t soff0 = o.wfirst + static_cast<uint32_t>(stage - half * o.split) * o.kstep;
#pragma unroll
    for (int j = 0; j < kInstr; ++j) {
        // LDS destination: this wave's j-th kilobyte of the tile
        __builtin_amdgcn_raw_ptr_buffer_load_lds(half ? o.res[1] : o.res[0], (lds_ptr_t)(dst + (wave * kInstr + j) * 64), 16,
                                                 o.vo[j & 1], soff0 + j * o.jstep, 0, 0);
    }
}

// The 8 k-consecutive bf16 of block b at k16 step t.
template <bool RC, int ROWS>
__device__ __forceinline__ bf16x8_t operand_frag(const Operand& o, const uint4* tile, int b, int t) {
    if (!RC) {
        const int off = o.rd[t] + b * 32 * 64;
        return as_bf16x8(*reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + off));
    } else {
        lds_char_t base = (lds_char_t)(tile);
        const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t)(base + o.rd[b] + (16 * t) * ROWS * 2));
        const v4s_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t)(base + o.rd[b] + (16 * t + 4) * ROWS * 2));
        u32x4_t v;
        v[0] = static_cast<uint16_t>(lo[0]) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[1])) << 16);
        v[1] = static_cast<uint16_t>(lo[2]) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[3])) << 16);
        v[2] = static_cast<uint16_t>(hi[0]) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[1])) << 16);
        v[3] = static_cast<uint16_t>(hi[2]) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[3])) << 16);
        return as_bf16x8(v);
    }
}

// ---------------------------------------------------------------------------
// The grouped GEMM
// ---------------------------------------------------------------------------

typedef bf16x8_t StageFrags[2][4];  // [k16 step][32-row block]

template <bool XRC, bool YRC>
__device__ __forceinline__ void read_stage(const Operand& ox, const Operand& oy, const uint4* cur, StageFrags& xf,
                                           StageFrags& yf) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int b = 0; b < 4; ++b) xf[t][b] = operand_frag<XRC, kTU>(ox, cur, b, t);
#pragma unroll
        for (int b = 0; b < 4; ++b) yf[t][b] = operand_frag<YRC, kTV>(oy, cur + kXVec, b, t);
    }
}

__device__ __forceinline__ void mfma_stage(const StageFrags& xf, const StageFrags& yf, f32x16_t (&acc)[4][4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int bu = 0; bu < 4; ++bu)
#pragma unroll
            for (int bv = 0; bv < 4; ++bv)
                acc[bu][bv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[t][bu], yf[t][bv], acc[bu][bv], 0, 0, 0);
}

constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;

// Issue order of one stage: an MFMA then a fragment read of the next stage,
// NREAD times, with the next copies after the first of them; the remaining MFMAs.
template <int NREAD>
__device__ __forceinline__ void sched_stage() {
#pragma unroll
    for (int u = 0; u < NREAD; ++u) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        // the copies early in the stage, one after each of the first MFMAs: a
        // copy has until the barrier three stages on to land (measured: 3%
        // faster backward than with the copies after the reads)
        if (u < kCopiesPerStage) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 32 - NREAD, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Stage s of the K loop.  The ring's four stage buffers are distinct LDS
// arrays, so the compiler's own wait before an LDS read covers only the copies
// into the buffer it reads.  On entry `cx`, `cy` hold stage s's fragments
// (reads in flight at most).  NEXT: wait until stage s+1 has landed for every
// wave (the copies of stage s+2 stay in flight), read it from `rd` into `nx`,
// `ny`, copy stage min(s+3, ns-1) into `cp` (the buffer of stage s-1, which
// every wave finished with before this barrier; a repeated last stage only
// refills a free buffer and keeps the count of copies in flight uniform),
// then the MFMAs of stage s, interleaved with those reads.
template <bool XRC, bool YRC, bool NEXT>
__device__ __forceinline__ void k_stage(const Operand& ox, const Operand& oy, const uint4* rd, uint4* cp, int s,
                                        int ns, int wave, const StageFrags& cx, const StageFrags& cy, StageFrags& nx,
                                        StageFrags& ny, f32x16_t (&acc)[4][4]) {
    constexpr int kRead = (XRC ? 16 : 8) + (YRC ? 16 : 8);  // LDS read instructions per stage
    if (NEXT) {
        wait_vm<kCopiesPerStage>();
        // a bare barrier: __syncthreads() would also wait for the copies in flight
        __builtin_amdgcn_s_barrier();
        read_stage<XRC, YRC>(ox, oy, rd, nx, ny);
        const int sn = min(s + kStages - 1, ns - 1);
        operand_copy<XRC, kTU>(ox, cp, sn, wave);
        operand_copy<YRC, kTV>(oy, cp + kXVec, sn, wave);
    }
    mfma_stage(cx, cy, acc);
    if (NEXT) sched_stage<kRead>();
}

enum Epi { kEpiGrad = 1, kEpiDx = 2, kEpiDw = 3 };

struct GemmArgs {
    // X (u operand): tile origin = x0 + (u0 or k0 rows) ...; see the tile set-up
    const bf16_t* xa;       // first half
    const bf16_t* xb;       // second half (split along u for k-contiguous X, along k for row-contiguous X)
    int64_t x_estride;      // elements between experts (weights) or 0 (per-row data)
    int ldx;
    int xsplit;             // u (k-contiguous) or k (row-contiguous) where xb takes over; 0 = none
    // Y (v operand)
    const bf16_t* y;
    int ldy;
    // shape
    int U, V, K;            // V or K = 0: taken from the expert segments
    const int32_t* offsets; // [n + 1] expert segments of the permuted rows
    int n_exp;
    // outputs
    void* c0;
    void* c1;
    int64_t c_estride;
    int ldc;
    int csplit;             // v where c1 takes over (kEpiDw), else 0
    // kEpiGrad
    const float* a;         // [P, 2F] pre-activations (fp32, 32 x 32 blocks: preact_block)
    const float* gp;        // [P] gate of each row (0 for padding)
    bf16_t* hg;             // [P, F]
    float* dgp;             // [U / kTU, P] partial dg sums
    int P;
    // TOKEN_V with row-contiguous X: ksplit 2 cuts K at xsplit (X = xa for the
    // first part, xb for the second) and writes the second part's sums
    // c_split_stride elements after c0
    int ksplit;
    int64_t c_split_stride;
};

template <bool XRC, bool YRC, int EPI, bool TOKEN_V>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_gemm_kernel(GemmArgs g) {
    static_assert(kStages == 4, "the K loop is unrolled over a ring of four buffers");
    __shared__ uint4 sb0[kStageVec];
    __shared__ uint4 sb1[kStageVec];
    __shared__ uint4 sb2[kStageVec];
    __shared__ uint4 sb3[kStageVec];
    uint4* const smem = sb0;  // the epilogue's reduction space

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int wu = wave & 1, wv = wave >> 1;
    const int nut = g.U / kTU;

    // ---- tile of this block: (expert e, u tile ut, v tile vt), XCD-aware.
    // The search over the experts runs across lanes: lane e (of each 16) holds
    // expert e's segment, and a prefix sum over those lanes and a ballot find
    // the expert (a loop over the experts waited one memory latency per expert).
    const int lane16 = threadIdx.x & 15;
    const int s0 = lane16 < g.n_exp ? g.offsets[lane16] : 0;
    const int s1 = lane16 < g.n_exp ? g.offsets[lane16 + 1] : 0;
    int e = 0, ut = 0, vt = 0, kbeg = 0, klen = g.K, ksp = 0;
    if (TOKEN_V) {
        // v runs over the expert's rows: expert e owns nut * (len_e / kTV) tiles
        const int nv = (s1 - s0) / kTV;
        const int w = nv * nut;
        const int ps = expert_prefix(w);
        const int total = __builtin_amdgcn_readlane(ps, 15);
        const int tiles = total * g.ksplit;
        const int run = (tiles + 7) >> 3;
        if (static_cast<int>(blockIdx.x >> 3) >= run) return;
        int L = (blockIdx.x & 7) * run + (blockIdx.x >> 3);
        if (L >= tiles) return;
        ksp = L / total;
        L -= ksp * total;
        e = expert_holding(ps, L);
        if (e < 0) return;
        L -= __builtin_amdgcn_readlane(ps - w, e);
        const int nve = __builtin_amdgcn_readlane(nv, e);
        ut = L / nve;
        vt = L - ut * nve;
        vt = __builtin_amdgcn_readlane(s0, e) / kTV + vt;  // global v tile (row block of the permuted layout)
    } else {
        // fixed U x V per expert, K = the expert's rows, which differ between
        // experts (rows padded to 256): the v columns of every expert are dealt
        // over the XCDs, column (e, vt) to XCD (e * nvt + vt) % 8, each with its
        // nut tiles (which share the column's Y slice) back to back, so every
        // XCD gets the same mix of experts.  (Contiguous runs gave each XCD one
        // expert: at prefill four XCDs ran K = 1280 while four ran 1024.)
        const int nvt = g.V / kTV;
        const int x = blockIdx.x & 7;
        const int i = blockIdx.x >> 3;
        int f = 0, kk = 0;
        if (lane16 < g.n_exp) {
            f = (x - (lane16 * nvt) % 8 + 8) % 8;       // this XCD's first column of expert lane16
            kk = f < nvt ? (nvt - 1 - f) / 8 + 1 : 0;  // its columns of that expert
        }
        const int w = kk * nut;
        const int ps = expert_prefix(w);
        e = expert_holding(ps, i);
        if (e < 0) return;
        const int li = i - __builtin_amdgcn_readlane(ps - w, e);
        const int col = li / nut;
        ut = li - col * nut;
        vt = __builtin_amdgcn_readlane(f, e) + 8 * col;
        kbeg = __builtin_amdgcn_readlane(s0, e);
        klen = __builtin_amdgcn_readlane(s1, e) - kbeg;
    }
    const int u0 = ut * kTU, v0 = vt * kTV;
    if (TOKEN_V && g.ksplit > 1) klen = g.K / g.ksplit;
    const int ns = klen / kBK;

    // ---- operands
    Operand ox;
    Operand oy;
    operand_setup<XRC, kTU>(ox, g.ldx, wave, lane);
    operand_setup<YRC, kTV>(oy, g.ldy, wave, lane);
    if (!XRC) {
        // X rows u (weights [e][u][k]): the second half holds u >= xsplit
        const bool second = g.xsplit > 0 && u0 >= g.xsplit;
        const bf16_t* base = (second ? g.xb : g.xa) + e * g.x_estride +
                             static_cast<int64_t>(u0 - (second ? g.xsplit : 0)) * g.ldx;
        ox.res[0] = ox.res[1] = bwd_rsrc(base);
        ox.split = 1 << 30;
    } else if (TOKEN_V) {
        // X = weights [e][k][u] (k = d or F rows), second half for k >= xsplit;
        // with the K split each part reads one half
        if (g.ksplit > 1) {
            ox.res[0] = ox.res[1] = bwd_rsrc((ksp ? g.xb : g.xa) + e * g.x_estride + u0);
            ox.split = 1 << 30;
        } else {
            ox.res[0] = bwd_rsrc(g.xa + e * g.x_estride + u0);
            ox.res[1] = bwd_rsrc((g.xsplit > 0 ? g.xb : g.xa) + e * g.x_estride + u0);
            ox.split = g.xsplit > 0 ? g.xsplit / kBK : (1 << 30);
        }
    } else {
        // X = per-row data [p][u], k = the expert's rows
        ox.res[0] = ox.res[1] = bwd_rsrc(g.xa + static_cast<int64_t>(kbeg) * g.ldx + u0);
        ox.split = 1 << 30;
    }
    if (!YRC) {
        // Y rows v = permuted rows [p][k], from this part's first k
        oy.res[0] = oy.res[1] = bwd_rsrc(g.y + static_cast<int64_t>(v0) * g.ldy + ksp * klen);
    } else {
        // Y = per-row data [p][v], k = the expert's rows
        oy.res[0] = oy.res[1] = bwd_rsrc(g.y + static_cast<int64_t>(kbeg) * g.ldy + v0);
    }
    oy.split = 1 << 30;
    operand_reads<XRC, kTU>(ox, wu * 128, lane);
    operand_reads<YRC, kTV>(oy, wv * 128, lane);

    f32x16_t acc[4][4];
#pragma unroll
    for (int bu = 0; bu < 4; ++bu)
#pragma unroll
        for (int bv = 0; bv < 4; ++bv)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[bu][bv][q] = 0.0f;

    // ---- K loop over a ring of four LDS buffers, copies three stages ahead;
    // each stage's MFMAs overlap the next stage's fragment reads.  ns is a
    // multiple of 8 (K is d, 2F or a segment length: multiples of 256), so the
    // loop runs in groups of four stages and the last group is peeled: no
    // branch carries the accumulators.
    if (ns > 0) {
        operand_copy<XRC, kTU>(ox, sb0, 0, wave);
        operand_copy<YRC, kTV>(oy, sb0 + kXVec, 0, wave);
        operand_copy<XRC, kTU>(ox, sb1, 1, wave);
        operand_copy<YRC, kTV>(oy, sb1 + kXVec, 1, wave);
        operand_copy<XRC, kTU>(ox, sb2, 2, wave);
        operand_copy<YRC, kTV>(oy, sb2 + kXVec, 2, wave);
        StageFrags xa, ya, xb, yb;
        wait_vm<2 * kCopiesPerStage>();
        __builtin_amdgcn_s_barrier();
        read_stage<XRC, YRC>(ox, oy, sb0, xa, ya);
        int s = 0;
        for (; s + 4 < ns; s += 4) {
            k_stage<XRC, YRC, true>(ox, oy, sb1, sb3, s, ns, wave, xa, ya, xb, yb, acc);
            k_stage<XRC, YRC, true>(ox, oy, sb2, sb0, s + 1, ns, wave, xb, yb, xa, ya, acc);
            k_stage<XRC, YRC, true>(ox, oy, sb3, sb1, s + 2, ns, wave, xa, ya, xb, yb, acc);
            k_stage<XRC, YRC, true>(ox, oy, sb0, sb2, s + 3, ns, wave, xb, yb, xa, ya, acc);
        }
        k_stage<XRC, YRC, true>(ox, oy, sb1, sb3, s, ns, wave, xa, ya, xb, yb, acc);
        k_stage<XRC, YRC, true>(ox, oy, sb2, sb0, s + 1, ns, wave, xb, yb, xa, ya, acc);
        k_stage<XRC, YRC, true>(ox, oy, sb3, sb1, s + 2, ns, wave, xa, ya, xb, yb, acc);
        k_stage<XRC, YRC, false>(ox, oy, sb0, sb2, s + 3, ns, wave, xb, yb, xa, ya, acc);
        wait_vm<0>();  // the repeated tail copies, before the LDS is reused
        __builtin_amdgcn_s_barrier();
    }

    // ---- epilogue.  32x32 C layout: lane l holds column v = l%32 of each
    // block and rows u = 8*(q/4) + 4*(l/32) + q%4, q = 0..15.
    const int fk = lane >> 5;
    if (EPI == kEpiDx || EPI == kEpiDw) {
        // fp32 results, row v and column u of the destination.  Weight
        // gradients: dw1 / dw3 (split at csplit) or dw2 of expert e; dx
        // partials: part ksp of dxp.
        float* dst;
        int vb = v0;
        if (EPI == kEpiDw) {
            const bool second = g.csplit > 0 && v0 >= g.csplit;
            dst = static_cast<float*>(second ? g.c1 : g.c0) + e * g.c_estride;
            vb = v0 - (second ? g.csplit : 0);
        } else {
            dst = static_cast<float*>(g.c0) + ksp * g.c_split_stride;
        }
        store_rows_staged(acc, reinterpret_cast<f32x4_t*>(wave == 0 ? sb0 : wave == 1 ? sb1 : wave == 2 ? sb2 : sb3),
                          dst, g.ldc, vb + wv * 128, u0 + wu * 128, 128, lane);
    } else {
        // kEpiGrad: u = feature f of F, v = permuted row p.  With a1 = a[p][f],
        // a3 = a[p][F + f], gate gv:  h = SiLU(a1) a3, dg += G h,
        // da3 = gv G SiLU(a1), da1 = gv G a3 SiLU'(a1), hg = gv h.
        // a is read in its 32 x 32 blocks (preact_block), which follow this C
        // layout: the lane's 16 values of a block are contiguous.
        const int F = g.U;
        float dg[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int bv = 0; bv < 4; ++bv) {
            const int p = v0 + wv * 128 + bv * 32 + (lane & 31);
            const int pb = (v0 + wv * 128 + bv * 32) / 32;
            const float gv = g.gp[p];
            bf16_t* darow = static_cast<bf16_t*>(g.c0) + static_cast<int64_t>(p) * 2 * F;
            bf16_t* hrow = g.hg + static_cast<int64_t>(p) * F;
#pragma unroll
            for (int bu = 0; bu < 4; ++bu) {
                const int fbk = (u0 + wu * 128 + bu * 32) / 32;
                const float* a1b = g.a + preact_block(pb, fbk, F) + lane * 16;
                const float* a3b = g.a + preact_block(pb, fbk + F / 32, F) + lane * 16;
                uint2 o1[4], o3[4], oh[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(a1b + 4 * q4);
                    const f32x4_t a3 = *reinterpret_cast<const f32x4_t*>(a3b + 4 * q4);
                    float d1[4], d3[4], hv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float G = acc[bu][bv][4 * q4 + i];
                        const float sg = sigmoid_f32(a1[i]);
                        const float si = a1[i] * sg;
                        const float h = si * a3[i];
                        dg[bv] = fmaf(G, h, dg[bv]);
                        const float dh = gv * G;
                        d3[i] = dh * si;
                        d1[i] = dh * a3[i] * (sg * (1.0f + a1[i] * (1.0f - sg)));
                        hv[i] = gv * h;
                    }
                    o1[q4].x = pack_bf16x2(d1[0], d1[1]);
                    o1[q4].y = pack_bf16x2(d1[2], d1[3]);
                    o3[q4].x = pack_bf16x2(d3[0], d3[1]);
                    o3[q4].y = pack_bf16x2(d3[2], d3[3]);
                    oh[q4].x = pack_bf16x2(hv[0], hv[1]);
                    oh[q4].y = pack_bf16x2(hv[2], hv[3]);
                }
                // Lanes l and l + 32 hold the two halves of each 8-wide run of f
                // of row p; after a v_permlane32_swap each lane stores a whole
                // run (run 2 pr + fk) in 16 bytes.
                const int fr0 = u0 + wu * 128 + bu * 32;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int f8 = fr0 + 8 * (2 * pr + fk);
                    auto sx = __builtin_amdgcn_permlane32_swap(o1[2 * pr].x, o1[2 * pr + 1].x, false, false);
                    auto sy = __builtin_amdgcn_permlane32_swap(o1[2 * pr].y, o1[2 * pr + 1].y, false, false);
                    *reinterpret_cast<uint4*>(darow + f8) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
                    sx = __builtin_amdgcn_permlane32_swap(o3[2 * pr].x, o3[2 * pr + 1].x, false, false);
                    sy = __builtin_amdgcn_permlane32_swap(o3[2 * pr].y, o3[2 * pr + 1].y, false, false);
                    *reinterpret_cast<uint4*>(darow + F + f8) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
                    sx = __builtin_amdgcn_permlane32_swap(oh[2 * pr].x, oh[2 * pr + 1].x, false, false);
                    sy = __builtin_amdgcn_permlane32_swap(oh[2 * pr].y, oh[2 * pr + 1].y, false, false);
                    *reinterpret_cast<uint4*>(hrow + f8) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
                }
            }
        }
        // dg partial over the block's 256 features, in a fixed order: the two
        // k-group lanes of a column, then the two u halves of the block
#pragma unroll
        for (int bv = 0; bv < 4; ++bv) dg[bv] += __shfl_xor(dg[bv], 32, 64);
        __syncthreads();  // the stage buffers are free
        float* red = reinterpret_cast<float*>(smem);
        if (fk == 0) {
#pragma unroll
            for (int bv = 0; bv < 4; ++bv) red[(wu * 2 + wv) * 128 + bv * 32 + lane] = dg[bv];
        }
        __syncthreads();
        if (wu == 0 && fk == 0) {
#pragma unroll
            for (int bv = 0; bv < 4; ++bv) {
                const int p = v0 + wv * 128 + bv * 32 + lane;
                g.dgp[static_cast<int64_t>(ut) * g.P + p] =
                    red[(0 * 2 + wv) * 128 + bv * 32 + lane] + red[(1 * 2 + wv) * 128 + bv * 32 + lane];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row gathers, router gradient, dx and dW_g
// ---------------------------------------------------------------------------

// xp[p] = x[t], dyp[p] = dy[t], gp[p] = gate of assignment a = row_src[p]
// (t = a / K); zeros for padding rows.
__global__ __launch_bounds__(256) void bwd_gather_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy,
                                                         const float* __restrict__ gate,
                                                         const int32_t* __restrict__ row_src, int d, int K,
                                                         int n_src, bf16_t* __restrict__ xp, bf16_t* __restrict__ dyp,
                                                         float* __restrict__ gp) {
    const int p = blockIdx.x;
    const int a = row_src[p];
    const bool real = a >= 0 && a < n_src;
    const int t = real ? a / K : 0;
    const uint4* xs = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * d);
    const uint4* ds = reinterpret_cast<const uint4*>(dy + static_cast<int64_t>(t) * d);
    uint4* xo = reinterpret_cast<uint4*>(xp + static_cast<int64_t>(p) * d);
    uint4* dout = reinterpret_cast<uint4*>(dyp + static_cast<int64_t>(p) * d);
    for (int c = threadIdx.x; c < d / 8; c += 256) {
        uint4 xv = make_uint4(0, 0, 0, 0), dv = make_uint4(0, 0, 0, 0);
        if (real) {
            xv = xs[c];
            dv = ds[c];
        }
        xo[c] = xv;
        dout[c] = dv;
    }
    if (threadIdx.x == 0) gp[p] = real ? gate[a] : 0.0f;
}

// dl[t, :]: zero except the K selected experts, dl_s = g_s (dg_s - sum_j g_j dg_j),
// dg_s = the sum of the row's partials over the nut feature tiles (lane-strided
// sums, then a butterfly: a fixed order).
__global__ __launch_bounds__(256) void bwd_router_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ gate,
                                                         const int32_t* __restrict__ row_of,
                                                         const float* __restrict__ dgp, int nut, int P, int T,
                                                         int n, int K, float* __restrict__ dl) {
    // one wave per token: lane u adds the partial sums u, u + 64, ... of each
    // slot's row, then a butterfly (a fixed order) completes them
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float dg[kMaxTopK], gs[kMaxTopK];
    float S = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        dg[s] = 0.0f;
        gs[s] = 0.0f;
        if (s < K) {
            const int p = row_of[t * K + s];
            float v = 0.0f;
            if (p >= 0)
                for (int u = lane; u < nut; u += 64) v += dgp[static_cast<int64_t>(u) * P + p];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            dg[s] = v;
            gs[s] = gate[t * K + s];
            S = fmaf(gs[s], dg[s], S);
        }
    }
    float* row = dl + static_cast<int64_t>(t) * n;
    if (lane < n) {
        float v = 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s)
            if (s < K && idx[t * K + s] == lane) v = gs[s] * (dg[s] - S);
        row[lane] = v;
    }
}

// dx[t] = sum_s (dxp + dxp_hi)[row_of[t, s]] (slot order) + sum_s dl[t, e_s] W_g[:, e_s], one
// rounding to bf16; dxp and dxp_hi are the w1 and w3 parts of the per-row input gradients.
template <int K>
__device__ __forceinline__ void bwd_dx_group(const float4* const (&pa)[K], const float4* const (&pb)[K],
                                             const int (&es)[K], const float* __restrict__ wg, int n, int c,
                                             float4 (&x)[K], float4 (&y)[K], float (&w)[K][4]) {
#pragma unroll
    for (int s = 0; s < K; ++s) {
        x[s] = pa[s][c];
        y[s] = pb[s][c];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[s][i] = wg[static_cast<int64_t>(4 * c + i) * n + es[s]];
    }
}

// The w1 and w3 parts of each slot, in slot order; a slot with no row is
// cleared by a bit mask (a select on the uniform flag becomes a branch that the
// loads sink into).  Then the router term and one rounding.
template <int K>
__device__ __forceinline__ void bwd_dx_store(const float4 (&x)[K], const float4 (&y)[K], const float (&w)[K][4],
                                             const uint32_t (&keep)[K], const float (&ls)[K],
                                             bf16_t* __restrict__ out) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K; ++s) {
        v[0] += __uint_as_float(__float_as_uint(x[s].x + y[s].x) & keep[s]);
        v[1] += __uint_as_float(__float_as_uint(x[s].y + y[s].y) & keep[s]);
        v[2] += __uint_as_float(__float_as_uint(x[s].z + y[s].z) & keep[s]);
        v[3] += __uint_as_float(__float_as_uint(x[s].w + y[s].w) & keep[s]);
    }
#pragma unroll
    for (int s = 0; s < K; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fmaf(ls[s], w[s][i], v[i]);
    uint2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(out) = o;
}

// One block of 256 threads per token; full passes take U column groups per
// thread with every load issued before the first store, then a plain loop.
template <int K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void bwd_dx_kernel(const float* __restrict__ dxp, const float* __restrict__ dxp_hi,
                                                     const int32_t* __restrict__ row_of,
                                                     const int32_t* __restrict__ idx, const float* __restrict__ dl,
                                                     const float* __restrict__ wg, int d, int n,
                                                     bf16_t* __restrict__ dx) {
    constexpr int U = 4;
    const int t = blockIdx.x;
    int es[K];
    float ls[K];
    uint32_t keep[K];
    const float4* pa[K];
    const float4* pb[K];
#pragma unroll
    for (int s = 0; s < K; ++s) {
        const int p = row_of[t * K + s];
        es[s] = idx[t * K + s];
        ls[s] = dl[static_cast<int64_t>(t) * n + es[s]];
        keep[s] = p >= 0 ? 0xffffffffu : 0u;
        const int64_t row = static_cast<int64_t>(p < 0 ? 0 : p) * d;
        pa[s] = reinterpret_cast<const float4*>(dxp + row);
        pb[s] = reinterpret_cast<const float4*>(dxp_hi + row);
    }
    bf16_t* out = dx + static_cast<int64_t>(t) * d;
    const int n4 = d / 4;
    int c = threadIdx.x;
    for (; c + (U - 1) * 256 < n4; c += U * 256) {
        float4 x[U][K], y[U][K];
        float w[U][K][4];
#pragma unroll
        for (int u = 0; u < U; ++u) bwd_dx_group<K>(pa, pb, es, wg, n, c + 256 * u, x[u], y[u], w[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) bwd_dx_store<K>(x[u], y[u], w[u], keep, ls, out + 4 * (c + 256 * u));
    }
    for (; c < n4; c += 256) {
        float4 x[K], y[K];
        float w[K][4];
        bwd_dx_group<K>(pa, pb, es, wg, n, c, x, y, w);
        bwd_dx_store<K>(x, y, w, keep, ls, out + 4 * c);
    }
}

constexpr int kDwgTokens = 64;  // tokens per partial sum of dW_g

// part[chunk][k][e] = sum over the chunk's tokens of x[t][k] dl[t][e]
// One wave per (512 columns of x, kDwgTokens tokens): lane l sums columns
// 8l .. 8l + 7 of its block (one 16-byte load of x per token) against the
// chunk's dl rows, in token order.
__global__ __launch_bounds__(64) void bwd_dwg_partial_kernel(const bf16_t* __restrict__ x,
                                                             const float* __restrict__ dl, int T, int d, int n,
                                                             float* __restrict__ part) {
    __shared__ float s_dl[kDwgTokens * kMaxExperts];
    const int lane = threadIdx.x;
    const int k0 = blockIdx.x * 512 + 8 * lane;
    const int t0 = blockIdx.y * kDwgTokens;
    const int nt = min(kDwgTokens, T - t0);
    for (int i = lane; i < nt * n; i += 64) s_dl[i] = dl[static_cast<int64_t>(t0) * n + i];
    __syncthreads();
    float acc[8][kMaxExperts];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < kMaxExperts; ++e) acc[j][e] = 0.0f;
    for (int i = 0; i < nt; ++i) {
        float xv[8];
        unpack_bf16x8(*reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t0 + i) * d + k0), xv);
#pragma unroll
        for (int e = 0; e < kMaxExperts; ++e) {
            if (e < n) {
                const float w = s_dl[i * n + e];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j][e] = fmaf(xv[j], w, acc[j][e]);
            }
        }
    }
    float* out = part + (static_cast<int64_t>(blockIdx.y) * d + k0) * n;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < kMaxExperts; ++e)
            if (e < n) out[j * n + e] = acc[j][e];
}

// dW_g = the chunk partials summed in chunk order; four outputs per thread.
__global__ __launch_bounds__(256) void bwd_dwg_reduce_kernel(const float* __restrict__ part, int chunks, int dn,
                                                             float* __restrict__ dwg) {
    const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
    if (i >= dn) return;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int c = 0; c < chunks; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(part + static_cast<int64_t>(c) * dn + i);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    *reinterpret_cast<float4*>(dwg + i) = s;
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) p[i] = 0.0f;
}

template <bool XRC, bool YRC, int EPI, bool TOKEN_V>
hipError_t launch_gemm(const GemmArgs& g, int grid, hipStream_t st) {
    if (grid <= 0) return hipSuccess;
    bwd_gemm_kernel<XRC, YRC, EPI, TOKEN_V><<<grid, 256, 0, st>>>(g);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(const Shape& s, BackwardWs* w, char* base) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base == nullptr ? nullptr : base + off;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    const size_t TK = static_cast<size_t>(s.T) * s.K;
    const size_t P = TK + static_cast<size_t>(s.n) * (kTV - 1);
    const size_t nut = static_cast<size_t>(s.F) / kTU;
    const size_t chunks = (static_cast<size_t>(s.T) + kDwgTokens - 1) / kDwgTokens;
    BackwardWs v{};
    v.idx = reinterpret_cast<int32_t*>(take(TK * 4));
    v.gate = reinterpret_cast<float*>(take(TK * 4));
    v.counts = reinterpret_cast<int32_t*>(take(static_cast<size_t>(s.n) * 4));
    v.offsets = reinterpret_cast<int32_t*>(take(static_cast<size_t>(s.n + 1) * 4));
    v.row_src = reinterpret_cast<int32_t*>(take(P * 4));
    v.row_of = reinterpret_cast<int32_t*>(take(TK * 4));
    v.xp = reinterpret_cast<bf16_t*>(take(P * s.d * 2));
    v.dyp = reinterpret_cast<bf16_t*>(take(P * s.d * 2));
    v.gp = reinterpret_cast<float*>(take(P * 4));
    v.a = reinterpret_cast<float*>(take(P * 2 * s.F * 4));
    v.da = reinterpret_cast<bf16_t*>(take(P * 2 * s.F * 2));
    v.hg = reinterpret_cast<bf16_t*>(take(P * s.F * 2));
    v.dgp = reinterpret_cast<float*>(take(nut * P * 4));
    v.dxp = reinterpret_cast<float*>(take(2 * P * s.d * 4));  // the w1 part, then the w3 part
    v.dl = reinterpret_cast<float*>(take(static_cast<size_t>(s.T) * s.n * 4));
    v.dwg_part = reinterpret_cast<float*>(take(chunks * s.d * s.n * 4));
    v.P = static_cast<int>(P);
    if (w != nullptr) *w = v;
    return off;
}

bool backward_fits(const Shape& s) {
    // Buffer resources are based at each tile's (or expert's) origin and
    // offset in 32 bits: the longest such span is one expert's rows of da
    // (at most T*K + 255 rows of 2F bf16), or one expert's weights.  The fp32
    // pre-activations and every other per-row buffer are addressed through
    // 64-bit pointers.
    const long long rows = static_cast<long long>(s.T) * s.K + (kTV - 1);
    return tiled_fits(s) && rows * 2LL * s.F * 2 < (1LL << 32) && 2LL * s.F * s.d * 2 < (1LL << 32) &&
           s.F % kTU == 0 && s.d % kTU == 0;
}

hipError_t launch_zero_grads(const Shape& s, float* dwg, float* dw1, float* dw3, float* dw2, hipStream_t st) {
    const int64_t nw = static_cast<int64_t>(s.n) * s.F * s.d;
    bwd_zero_kernel<<<1024, 256, 0, st>>>(dw1, nw);
    bwd_zero_kernel<<<1024, 256, 0, st>>>(dw3, nw);
    bwd_zero_kernel<<<1024, 256, 0, st>>>(dw2, nw);
    bwd_zero_kernel<<<16, 256, 0, st>>>(dwg, static_cast<int64_t>(s.d) * s.n);
    return hipGetLastError();
}

hipError_t launch_layer_backward(const Shape& s, const void* x, const float* wg, const void* w1, const void* w3,
                                 const void* w2, const void* dy, void* dx, float* dwg, float* dw1, float* dw3,
                                 float* dw2, const BackwardWs& w, hipStream_t st) {
    hipError_t err;
    const int d = s.d, F = s.F, n = s.n, K = s.K, T = s.T;
    const int P = w.P;
    const int TK = T * K;
    const auto* xb = static_cast<const bf16_t*>(x);
    const auto* w1b = static_cast<const bf16_t*>(w1);
    const auto* w3b = static_cast<const bf16_t*>(w3);
    const auto* w2b = static_cast<const bf16_t*>(w2);
    if ((err = launch_router_topk(s, x, wg, w.idx, w.gate, nullptr, st)) != hipSuccess) return err;
    if ((err = launch_permute(s, kTV, w.idx, w.counts, w.offsets, w.row_src, w.row_of, st)) != hipSuccess) return err;
    bwd_gather_kernel<<<P, 256, 0, st>>>(xb, static_cast<const bf16_t*>(dy), w.gate, w.row_src, d, K, TK, w.xp, w.dyp,
                                          w.gp);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    const int vmax = (P + kTV - 1) / kTV;  // worst-case row tiles
    auto grid8 = [](long long tiles) { return static_cast<int>((tiles + 7) / 8 * 8); };
    // weight-gradient products: an XCD takes ceil(nvt / 8) columns of nut tiles of each expert
    auto dw_grid = [&](int nut, int nvt) { return static_cast<int>(8LL * n * ((nvt + 7) / 8) * nut); };

    // 1. a = [a1 | a3] in fp32: the forward pass's tiled gate/up kernel with a
    //    pre-activation epilogue (same rows, same tile order)
    if ((err = launch_tiled_preact(s, x, w.row_src, w.counts, w.offsets, w1, w3, w.a, st)) != hipSuccess) return err;

    GemmArgs g{};
    // 2. G = dyp . w2 with the gradient epilogue: X = w2[e] as [k = d][u = F]
    g.xa = w2b; g.xb = w2b; g.x_estride = static_cast<int64_t>(d) * F; g.ldx = F; g.xsplit = 0;
    g.y = w.dyp; g.ldy = d;
    g.U = F; g.V = 0; g.K = d; g.offsets = w.offsets; g.n_exp = n;
    g.c0 = w.da; g.ldc = 2 * F;
    g.a = w.a; g.gp = w.gp; g.hg = w.hg; g.dgp = w.dgp; g.P = P; g.ksplit = 1;
    if ((err = launch_gemm<true, false, kEpiGrad, true>(g, grid8(static_cast<long long>(F / kTU) * vmax), st)) !=
        hipSuccess)
        return err;

    // 3. dxp = da . [w1; w3]: X = w1[e] (k < F) then w3[e], as [k][u = d]
    g = GemmArgs{};
    g.xa = w1b; g.xb = w3b; g.x_estride = static_cast<int64_t>(F) * d; g.ldx = d; g.xsplit = F;
    g.y = w.da; g.ldy = 2 * F;
    g.U = d; g.V = 0; g.K = 2 * F; g.offsets = w.offsets; g.n_exp = n;
    g.c0 = w.dxp; g.ldc = d; g.P = P;
    g.ksplit = 2;  // K = 2F cut at F: the w1 part and the w3 part, two partial buffers
    g.c_split_stride = static_cast<int64_t>(P) * d;
    if ((err = launch_gemm<true, false, kEpiDx, true>(g, grid8(2LL * (d / kTU) * vmax), st)) != hipSuccess)
        return err;

    // 4. dw2[e][j][f] = sum_p hg[p][f] dyp[p][j]: u = f, v = j
    g = GemmArgs{};
    g.xa = w.hg; g.xb = w.hg; g.ldx = F;
    g.y = w.dyp; g.ldy = d;
    g.U = F; g.V = d; g.K = 0; g.offsets = w.offsets; g.n_exp = n;
    g.c0 = dw2; g.c1 = dw2; g.c_estride = static_cast<int64_t>(d) * F; g.ldc = F; g.csplit = 0; g.P = P;
    g.ksplit = 1;
    if ((err = launch_gemm<true, true, kEpiDw, false>(g, dw_grid(F / kTU, d / kTV), st)) != hipSuccess) return err;

    // 5. dw1/dw3[e][f][j] = sum_p da[p][f'] xp[p][j]: u = j, v = f' (f' >= F: dw3)
    g = GemmArgs{};
    g.xa = w.xp; g.xb = w.xp; g.ldx = d;
    g.y = w.da; g.ldy = 2 * F;
    g.U = d; g.V = 2 * F; g.K = 0; g.offsets = w.offsets; g.n_exp = n;
    g.c0 = dw1; g.c1 = dw3; g.c_estride = static_cast<int64_t>(F) * d; g.ldc = d; g.csplit = F; g.P = P;
    g.ksplit = 1;
    if ((err = launch_gemm<true, true, kEpiDw, false>(g, dw_grid(d / kTU, 2 * F / kTV), st)) != hipSuccess)
        return err;

    // router gradient, dx, dW_g
    bwd_router_kernel<<<(T + 3) / 4, 256, 0, st>>>(w.idx, w.gate, w.row_of, w.dgp, F / kTU, P, T, n, K, w.dl);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    {
        const float* hi = w.dxp + static_cast<int64_t>(P) * d;
        bf16_t* dxo = static_cast<bf16_t*>(dx);
        switch (K) {
            case 1: bwd_dx_kernel<1><<<T, 256, 0, st>>>(w.dxp, hi, w.row_of, w.idx, w.dl, wg, d, n, dxo); break;
            case 2: bwd_dx_kernel<2><<<T, 256, 0, st>>>(w.dxp, hi, w.row_of, w.idx, w.dl, wg, d, n, dxo); break;
            case 3: bwd_dx_kernel<3><<<T, 256, 0, st>>>(w.dxp, hi, w.row_of, w.idx, w.dl, wg, d, n, dxo); break;
            default: bwd_dx_kernel<4><<<T, 256, 0, st>>>(w.dxp, hi, w.row_of, w.idx, w.dl, wg, d, n, dxo); break;
        }
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int chunks = (T + kDwgTokens - 1) / kDwgTokens;
    bwd_dwg_partial_kernel<<<dim3(d / 512, chunks), 64, 0, st>>>(xb, w.dl, T, d, n, w.dwg_part);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    bwd_dwg_reduce_kernel<<<(d * n / 4 + 255) / 256, 256, 0, st>>>(w.dwg_part, chunks, d * n, dwg);
    return hipGetLastError();
}

}  // namespace moe
