// Tree preprocessing inside one workgroup: validation, inclusive ancestor bitmask, depth and
// the log cumulative decay l_i = log alpha_i + l_parent(i) ("The tree closed form" on the
// canopy project page). Pointer jumping: after round r every node knows the union of the
// masks and the sum of log alpha over the next 2^r nodes of its root path, so ceil(log2(d+1))
// rounds cover a tree of depth d.
#pragma once
#include "canopy_device.hpp"
#include <limits.h>

namespace canopy {

template <int MAXT>
struct PrepSmem {
    static constexpr int MW = MAXT / 32;
    int32_t jump[MAXT];
    uint32_t mask[MAXT][MW];
    double ell[MAXT];
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

// All NT threads of the block call this. Returns 0 for a valid tree, else 1 + the first node
// whose parent lies outside -1..i-1 (the block's result is then undefined apart from that).
template <int MAXT, int NT>
__device__ int tree_prep_compute(PrepSmem<MAXT> &s, const PrepIn<MAXT, NT> &in, int T) {
    constexpr int MW = MAXT / 32;
    constexpr int NPT = PrepIn<MAXT, NT>::NPT;
    const int tid = threadIdx.x;
    if (tid == 0) s.bad = INT_MAX;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NPT; ++t) {
        const int i = tid + t * NT;
        if (i < MAXT) {
            int p = -1;
            double l = 0.0;
            if (i < T) {
                p = in.p[t];
                if (p < -1 || p >= i) {
                    atomicMin(&s.bad, i + 1);
                    p = -1;
                }
                l = log(static_cast<double>(in.al[t]));
            }
            s.jump[i] = p;
            s.ell[i] = l;
#pragma unroll
            for (int w = 0; w < MW; ++w)
                s.mask[i][w] = (i < T && w == (i >> 5)) ? (1u << (i & 31)) : 0u;
        }
    }
    __syncthreads();
    if (s.bad != INT_MAX) return s.bad;

    for (int round = 0; round < 10; ++round) {
        uint32_t nm[NPT][MW];
        double nl[NPT];
        int nj[NPT];
        int more = 0;
#pragma unroll
        for (int t = 0; t < NPT; ++t) {
            const int i = tid + t * NT;
            if (i < MAXT) {
                const int j = s.jump[i];
                nl[t] = s.ell[i];
                nj[t] = j;
#pragma unroll
                for (int w = 0; w < MW; ++w) nm[t][w] = s.mask[i][w];
                if (j >= 0) {
                    nl[t] += s.ell[j];
                    nj[t] = s.jump[j];
#pragma unroll
                    for (int w = 0; w < MW; ++w) nm[t][w] |= s.mask[j][w];
                }
                more |= (nj[t] >= 0);
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NPT; ++t) {
            const int i = tid + t * NT;
            if (i < MAXT) {
                s.jump[i] = nj[t];
                s.ell[i] = nl[t];
#pragma unroll
                for (int w = 0; w < MW; ++w) s.mask[i][w] = nm[t][w];
            }
        }
        if (!__syncthreads_or(more)) break;
    }
    return 0;
}

template <int MAXT, int NT>
__device__ int tree_prep_block(PrepSmem<MAXT> &s, const int32_t *parent_b, const float *alpha_h,
                               int astride, int T) {
    PrepIn<MAXT, NT> in;
    in.load(parent_b, alpha_h, astride, T);
    return tree_prep_compute<MAXT, NT>(s, in, T);
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
