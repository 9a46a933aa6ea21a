// Dropless grouping of the T*K routing assignments by expert: histogram,
// exclusive scan into tile-padded segment offsets, stable scatter.
//
// Mixtral routes every token to its two experts with no capacity limit and no
// dropping (paper-graph-ui page, section 3.4 "Top-K Gating Mechanism and
// Routing", load-balancing paragraph) and runs all experts' tokens as one packed
// matrix (same section, "Megablocks kernels" paragraph).  The grouped GEMMs need
// each expert's rows contiguous and padded to their row-tile size.
//
// One block of 1024 threads.  Thread i owns the contiguous assignment range
// [i*per, (i+1)*per), so scattering each thread's assignments in order at its
// exclusive prefix keeps ascending assignment order inside a segment: the
// result is deterministic and matches a stable sort by expert.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// NE expert slots; experts 0..n-1 are real, any other index is ignored.
// A thread's assignments (at most HELD = 8, or at most 32 with HELD = 0) are
// loaded once, all at the same time, and kept in registers for the scatter;
// with HELD = 0 and more than 32 per thread they are read as they are counted
// and read again for the scatter.  (A compile-time 16 or 32 held ran out of
// the 128 registers a 1024-thread block allows and spilled.)
template <int NE, int HELD>
__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ idx, int TK, int n,
                                                           int tile_m, int P_max,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_src,
                                                           int32_t* __restrict__ row_of) {
    __shared__ int s_wave[kWaves][NE];
    __shared__ int s_total[NE];
    __shared__ int s_off[NE + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int per = (TK + kThreads - 1) / kThreads;
    const int a0 = min(TK, tid * per);
    const int a1 = min(TK, a0 + per);

    constexpr int kHeld = HELD > 0 ? HELD : 32;
    const bool held = HELD > 0 || per <= kHeld;
    int ev[kHeld];
    if (held) {
#pragma unroll
        for (int i = 0; i < kHeld; ++i) ev[i] = a0 + i < a1 ? idx[a0 + i] : -1;
    }
    int c[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) c[e] = 0;
    if (held) {
#pragma unroll
        for (int i = 0; i < kHeld; ++i)
#pragma unroll
            for (int j = 0; j < NE; ++j) c[j] += (ev[i] == j && j < n) ? 1 : 0;
    } else {
        for (int a = a0; a < a1; ++a) {
            const int e = idx[a];
#pragma unroll
            for (int j = 0; j < NE; ++j) c[j] += (e == j && j < n) ? 1 : 0;
        }
    }

    // Inclusive scan of each expert's count across the wave.
    int incl[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        int v = c[e];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(v, off, 64);
            if (lane >= off) v += u;
        }
        incl[e] = v;
    }
    if (lane == 63) {
#pragma unroll
        for (int e = 0; e < NE; ++e) s_wave[wave][e] = incl[e];
    }
    __syncthreads();
    if (tid < NE) {
        int run = 0;
        for (int w = 0; w < kWaves; ++w) {
            const int v = s_wave[w][tid];
            s_wave[w][tid] = run;
            run += v;
        }
        s_total[tid] = run;
    }
    __syncthreads();
    if (tid == 0) {
        int off = 0;
        for (int e = 0; e < NE; ++e) {
            s_off[e] = off;
            if (e < n) {
                counts[e] = s_total[e];
                offsets[e] = off;
            }
            off += (s_total[e] + tile_m - 1) / tile_m * tile_m;  // zero past n
        }
        s_off[NE] = off;
        offsets[n] = off;
    }
    __syncthreads();

    int pos[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) pos[e] = s_off[e] + s_wave[wave][e] + incl[e] - c[e];
    auto place = [&](int a, int e) {
        int p = -1;
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            if (e == j && j < n) {
                p = pos[j];
                pos[j] = p + 1;
            }
        }
        if (p >= 0) row_src[p] = a;
        row_of[a] = p;
    };
    if (held) {
#pragma unroll
        for (int i = 0; i < kHeld; ++i)
            if (a0 + i < a1) place(a0 + i, ev[i]);
    } else {
        for (int a = a0; a < a1; ++a) place(a, idx[a]);
    }

    // Padding rows of every segment, then everything past the last segment.
    for (int e = 0; e < n; ++e) {
        const int lo = s_off[e] + s_total[e];
        const int hi = s_off[e + 1];
        for (int p = lo + tid; p < hi; p += kThreads) row_src[p] = -1;
    }
    for (int p = s_off[NE] + tid; p < P_max; p += kThreads) row_src[p] = -1;
}

// Up to 64 assignments (a decode step): one wave, lane a holds assignment a.
// Expert e's members are the lanes of ballot(idx == e); a member's rank among
// them (the popcount of the lower lanes) is its place in the segment, so the
// order is the same ascending-assignment order as above, without a barrier.
__global__ __launch_bounds__(64) void permute_wave_kernel(const int32_t* __restrict__ idx, int TK, int n,
                                                          int tile_m, int P_max, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_src,
                                                          int32_t* __restrict__ row_of) {
    const int lane = threadIdx.x;
    const int mine = lane < TK ? idx[lane] : -1;
    const bool real = mine >= 0 && mine < n;
    int seg_off[kMaxExperts + 1], seg_cnt[kMaxExperts];
    int off = 0, pos = -1;
#pragma unroll
    for (int e = 0; e < kMaxExperts; ++e) {
        seg_off[e] = off;
        seg_cnt[e] = 0;
        if (e < n) {
            const unsigned long long m = __ballot(real && mine == e);
            const int c = __popcll(m);
            seg_cnt[e] = c;
            if (lane == 0) {
                counts[e] = c;
                offsets[e] = off;
            }
            if (real && mine == e) pos = off + __popcll(m & ((1ull << lane) - 1ull));
            off += (c + tile_m - 1) / tile_m * tile_m;
        }
    }
    seg_off[kMaxExperts] = off;
    if (lane == 0) offsets[n] = off;
    if (lane < TK) row_of[lane] = pos;
    if (pos >= 0) row_src[pos] = lane;
    // every other row is padding: inside a segment past its count, or past the last segment
    for (int p = lane; p < P_max; p += 64) {
        bool pad = p >= off;
#pragma unroll
        for (int e = 0; e < kMaxExperts; ++e)
            if (e < n && p >= seg_off[e] + seg_cnt[e] && p < seg_off[e + 1]) pad = true;
        if (pad) row_src[p] = -1;
    }
}

}  // namespace

hipError_t launch_permute(const Shape& s, int tile_m, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* row_src, int32_t* row_of, hipStream_t st) {
    const int TK = s.T * s.K;
    const int P_max = TK + s.n * (tile_m - 1);
    if (TK <= 64) {
        permute_wave_kernel<<<1, 64, 0, st>>>(idx, TK, s.n, tile_m, P_max, counts, offsets, row_src, row_of);
        return hipGetLastError();
    }
    // assignments per thread: up to 8 take the kernel that holds exactly 8
    const int per = (TK + kThreads - 1) / kThreads;
    const int held = per <= 8 ? 8 : 0;
#define MOE_PERMUTE(NE, H) \
    permute_kernel<NE, H><<<1, kThreads, 0, st>>>(idx, TK, s.n, tile_m, P_max, counts, offsets, row_src, row_of)
    if (s.n <= 8) {
        if (held == 8) MOE_PERMUTE(8, 8);
        else MOE_PERMUTE(8, 0);
    } else {
        MOE_PERMUTE(16, 0);  // held 8 with 16 expert slots spills
    }
#undef MOE_PERMUTE
    return hipGetLastError();
}

}  // namespace moe
