// Tree preprocessing inside one workgroup: validation, inclusive ancestor bitmask, depth and
// the log cumulative decay l_i = log alpha_i + l_parent(i) ("The tree closed form" on the
// canopy project page).
#pragma once
#include "canopy_device.hpp"
#include <limits.h>

namespace canopy {

template <int MAXT>
struct PrepSmem {
    static constexpr int MW = MAXT / 32;
    int32_t jump[MAXT];
    uint32_t mask[MAXT][MW];
    alignas(16) double ell[MAXT];  // path sums of log2 alpha: l = ell ln 2, P = 2^ell
    int bad;
};

// Per-thread inputs of the preprocessing: the parent and alpha of nodes tid, tid + NT, ...
// Loading them first (before any bulk loads) keeps their latency off the critical path.
template <int MAXT, int NT>
struct PrepIn {
    static constexpr int NPT = (MAXT + NT - 1) / NT;
    int p[NPT];
    float al[NPT];
    __device__ __forceinline__ void load(const int32_t *parent_b, const float *alpha_h, int astride,
                                         int T) {
#pragma unroll
        for (int t = 0; t < NPT; ++t) {
            const int i = threadIdx.x + t * NT;
            const int ic = min(i, T - 1);
            p[t] = parent_b[ic];
            al[t] = alpha_h[static_cast<size_t>(ic) * astride];
        }
    }
};

// All NT threads of the block call this, T being the tree's node count (nodes at or past T are
// not part of it, whatever the inputs hold there). Returns 0 for a valid tree, else 1 + the
// first node whose parent lies outside -1..i-1 (the block's result is then undefined apart
// from that).
//
// The nodes are cut into 64-node chunks, one wave (one lane per node) per chunk at a time.
// Inside a chunk, pointer jumping over lane shuffles gathers, for every node, the mask bits,
// the log-decay sum and the exit (the first ancestor outside the chunk, -1 for none) of its
// in-chunk root path; after round r a jump pointer is 2^(r+1) levels up, so ceil(log2(d+1))
// rounds cover an in-chunk depth d. Parents precede children, so every exit lies in an earlier
// chunk: the chunks are then completed in order, each node taking its exit's full mask words
// and log-decay sum.
template <int MAXT, int NT>
__device__ int tree_prep_compute(PrepSmem<MAXT> &s, const PrepIn<MAXT, NT> &in, int T) {
    constexpr int MW = MAXT / 32;
    constexpr int NPT = PrepIn<MAXT, NT>::NPT;
    constexpr int NW = NT / 64;
    constexpr int NCH = MAXT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s.bad = INT_MAX;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NPT; ++t) {
        const int c = wave + t * NW;  // the chunk of node tid + t * NT
        if (c >= NCH) continue;
        const int i = 64 * c + lane;
        const bool real = i < T;
        int p = real ? in.p[t] : -1;
        if (real && (p < -1 || p >= i)) {
            atomicMin(&s.bad, i + 1);
            p = -1;
        }
        unsigned long long m = real ? (1ull << lane) : 0ull;
        // log2 alpha by the hardware logarithm (about 1 ulp, relative to each term); the path
        // sums in fp64
        double l = real ? static_cast<double>(__builtin_amdgcn_logf(in.al[t])) : 0.0;
        const bool inside = p >= 64 * c;
        int jmp = inside ? p - 64 * c : -1;
        int ex = inside ? -1 : p;  // set again from the in-chunk root when the jumps reach it
        for (int round = 0; round < 6 && __any(jmp >= 0); ++round) {
            const int src = jmp >= 0 ? jmp : lane;
            const unsigned long long pm = __shfl(m, src, 64);
            const double pl = __shfl(l, src, 64);
            const int pj = __shfl(jmp, src, 64);
            const int pe = __shfl(ex, src, 64);
            const bool up = jmp >= 0;
            m = up ? (m | pm) : m;
            l = up ? l + pl : l;
            ex = up ? pe : ex;
            jmp = up ? pj : jmp;
        }
        s.jump[i] = ex;
        s.ell[i] = l;
#pragma unroll
        for (int w = 0; w < MW; ++w)
            s.mask[i][w] = w == 2 * c ? static_cast<uint32_t>(m)
                                      : (w == 2 * c + 1 ? static_cast<uint32_t>(m >> 32) : 0u);
    }
    __syncthreads();
    if (s.bad != INT_MAX) return s.bad;
#pragma unroll
    for (int c = 1; c < NCH; ++c) {
        if (64 * c >= T) break;
        if (wave == c % NW) {
            const int i = 64 * c + lane;
            const int e = s.jump[i];
            if (e >= 0) {
#pragma unroll
                for (int w = 0; w < 2 * c; ++w) s.mask[i][w] = s.mask[e][w];
                s.ell[i] += s.ell[e];
            }
        }
        __syncthreads();
    }
    return 0;
}

// T: the arrays' node extent (loads stay below it); n: the tree's node count (n <= T).
template <int MAXT, int NT>
__device__ int tree_prep_block(PrepSmem<MAXT> &s, const int32_t *parent_b, const float *alpha_h,
                               int astride, int T, int n) {
    PrepIn<MAXT, NT> in;
    in.load(parent_b, alpha_h, astride, T);
    return tree_prep_compute<MAXT, NT>(s, in, n);
}

// Popcount of a node's mask row, minus one: |A(i)|.
template <int MAXT>
__device__ __forceinline__ int node_depth(const PrepSmem<MAXT> &s, int i) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < MAXT / 32; ++w) c += __popc(s.mask[i][w]);
    return c - 1;
}

}  // namespace canopy
