// Commit of the accepted path ("Design decisions / What the commit kernel stores" on the canopy
// project page):
//   S_new = P_a S0 + sum_{t < m} w_t k_{path[t]} u_{path[t]}^T,
//   w_t = exp(sum_{s > t} log alpha_{path[s]}) = Gamma_{a, path[t]},  P_a = exp(sum_s log alpha).
// One wave per (sequence, head, 8 state rows): lane (h, c) owns rows 4h .. 4h+3 of the 8 at
// float4 column c, so S loads and stores are whole 512-byte rows and a position's key values
// for a lane are one 8-byte (bf16) or 16-byte (fp32) word. No LDS and no barrier: every wave
// walks the path itself, one path position per lane, 64 positions at a time:
//   round 1  the path length and the first 64 path entries (requested together: entries past
//            the path are read but never used)
//   round 2  their parents and alphas, the U rows and key words of the first CGRP positions,
//            addressed by broadcasting each position's node id, and this wave's rows of S0
//   then     the path check (each node a child of the one before), suffix sums of log2 alpha
//            in fp64 over lane shuffles, w = 2^(suffix), and the rank-m update.
// Longer paths go chunk by chunk in path order; before a chunk adds its terms the sum so far is
// scaled by that chunk's total decay, so each weight is a product of short suffix decays, never
// a difference of long cumulative sums.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

constexpr int CROWS = 8;  // state rows per wave
// Path positions whose U rows and keys are requested together. Accepted paths are short (a few
// nodes), and a slot past the path still costs a load, so small groups beat fewer round trips.
constexpr int CGRP = 4;

// Where a node's rows start: U (value head, node stride rs) and k (its q/k head, stride krs).
struct Rows {
    size_t base, rs, kbase, krs;
};

// U rows (float4 column c4) and key words (4 state rows from krow) of NG path positions
// first .. first+NG-1, the positions' node ids broadcast from the lanes that hold them. Slots
// past the chunk's last position repeat its node and get weight 0.
template <bool BF, int NG>
struct NodeGroup {
    float4 u[NG];
    uint32_t k[NG][BF ? 2 : 4];
    __device__ __forceinline__ void load(const CommitArgs &a, const Rows &rw, int krow, int c4, int ndc,
                                         int first, int lastpos) {
#pragma unroll
        for (int tt = 0; tt < NG; ++tt) {
            const int n = __builtin_amdgcn_readlane(ndc, min(first + tt, lastpos));
            const size_t ro = rw.base + static_cast<size_t>(n) * rw.rs;
            const size_t ko = rw.kbase + static_cast<size_t>(n) * rw.krs + krow;
            u[tt] = reinterpret_cast<const float4 *>(a.U + ro)[c4];
            if constexpr (BF) {
                const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.k) + ko);
                k[tt][0] = w.x;
                k[tt][1] = w.y;
            } else {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(static_cast<const float *>(a.k) + ko);
#pragma unroll
                for (int e = 0; e < 4; ++e) k[tt][e] = w[e];
            }
        }
    }
    // acc[q] += sum over the group's positions of w_t k_t[krow + q] u_t
    __device__ __forceinline__ void apply(float4 (&acc)[4], float w, int first, int cnt) const {
#pragma unroll
        for (int tt = 0; tt < NG; ++tt) {
            const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(first + tt, 63)));
            const float wt = first + tt < cnt ? wr : 0.f;
            const float4 uu = u[tt];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float kq;
                if constexpr (BF)
                    kq = bf16_to_f32(static_cast<uint16_t>((q & 1) ? (k[tt][q >> 1] >> 16) : (k[tt][q >> 1] & 0xFFFFu)));
                else
                    kq = __uint_as_float(k[tt][q]);
                const float kw = wt * kq;
                acc[q].x += kw * uu.x;
                acc[q].y += kw * uu.y;
                acc[q].z += kw * uu.z;
                acc[q].w += kw * uu.w;
            }
        }
    }
};

// One 64-position chunk c of the path (lane = position 64c + lane). issue() requests the parents,
// the alphas and the first group's U rows and keys; finish() checks the path, forms the weights
// and folds the chunk into the running sum.
template <bool BF, int NG>
struct Chunk {
    int c, cnt, nd, ndc, par_nd;
    float al;
    NodeGroup<BF, NG> grp;
    __device__ __forceinline__ void issue(const CommitArgs &a, const int32_t *par, int c_, int mv, int nd_,
                                          const Rows &rw, size_t abase, int krow, int c4) {
        c = c_;
        nd = nd_;
        ndc = min(max(nd, 0), a.T - 1);
        cnt = min(64, mv - 64 * c);  // positions in this chunk (at least 1)
        par_nd = par[ndc];
        al = a.alpha[abase + static_cast<size_t>(ndc) * a.H];
        grp.load(a, rw, krow, c4, ndc, 0, cnt - 1);
    }
    // prev_last: the node at position 64c - 1 (unused for c = 0); on return, the node at 64c + 63.
    __device__ __forceinline__ void finish(const CommitArgs &a, int mv, int Tb, const Rows &rw, int krow,
                                           int c4, float4 (&acc)[4], double &tot, int &prev_last,
                                           int &bad) const {
        const int lane = threadIdx.x;
        const int t = 64 * c + lane;
        const bool inp = t < mv;
        // path check: position t holds a node in range whose parent is position t-1's node
        const int up = __shfl_up(nd, 1, 64);
        const int prev = t == 0 ? -1 : (lane == 0 ? prev_last : up);
        const bool ok = (!inp) | ((nd >= 0) & (nd < Tb) & (par_nd == prev));
        const unsigned long long badm = __ballot(!ok);
        if (badm) bad = min(bad, 64 * c + __ffsll(static_cast<unsigned long long>(badm)));
        prev_last = __builtin_amdgcn_readlane(nd, 63);
        // suffix sums of log2 alpha inside the chunk (fp64). Lanes past the chunk's cnt
        // positions hold 0, so shuffle steps 1 and 2 cover every sum of a chunk of at most 4
        // positions (accepted paths are short); longer chunks take all six.
        const double la = inp ? static_cast<double>(__builtin_amdgcn_logf(al)) : 0.0;
        double v = la;
        if (cnt <= 4) {
#pragma unroll
            for (int off = 1; off < 4; off <<= 1) {
                const double tv = __shfl_down(v, off, 64);
                v = lane + off < 64 ? v + tv : v;
            }
        } else {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const double tv = __shfl_down(v, off, 64);
                v = lane + off < 64 ? v + tv : v;
            }
        }
        const double ctot = __shfl(v, 0, 64);  // log2 of the chunk's total decay
        tot += ctot;
        if (c > 0) {  // the terms of earlier positions decay through the whole chunk
            const float sc = __builtin_amdgcn_exp2f(static_cast<float>(ctot));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[q].x *= sc;
                acc[q].y *= sc;
                acc[q].z *= sc;
                acc[q].w *= sc;
            }
        }
        const float w = __builtin_amdgcn_exp2f(static_cast<float>(v - la));  // decay after position t
        grp.apply(acc, w, 0, cnt);
        for (int g0 = NG; g0 < cnt; g0 += NG) {  // more than NG positions in this chunk
            NodeGroup<BF, NG> more;
            more.load(a, rw, krow, c4, ndc, g0, cnt - 1);
            more.apply(acc, w, g0, cnt);
        }
    }
};

// The commit of workgroup g's (sequence, head, 8 state rows).
template <bool BF, int NG>
__device__ __forceinline__ void commit_body(const CommitArgs &a, int g) {
    const int chunk = g % (D / CROWS);
    const int bh = g / (D / CROWS);
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x;
    const int c4 = lane & 31;                            // float4 column
    const int krow = chunk * CROWS + 4 * (lane >> 5);    // first of this lane's 4 rows
    const int32_t *pb = a.path + static_cast<size_t>(b) * T;
    const int32_t *par = a.parent + static_cast<size_t>(b) * T;
    const Rows rw{(static_cast<size_t>(b) * T * H + h) * D, static_cast<size_t>(H) * D,
                  qk_base(b, h, H, a.HK, T), static_cast<size_t>(a.HK) * D};
    const size_t abase = static_cast<size_t>(b) * T * H + h;

    // ---- round 1
    const int m = a.path_len[b];
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int nd0 = pb[min(lane, T - 1)];
    const bool lenok = !sl.bad && m >= 0 && m <= sl.n;
    const int mv = lenok ? m : 0;
    const int nch = (mv + 63) / 64;
    // ---- round 2: the first chunk's parents, alphas, U rows and keys, then this wave's rows of
    // S0, which are needed last (requests return in order)
    Chunk<BF, NG> first;
    first.issue(a, par, 0, max(mv, 1), nd0, rw, abase, krow, c4);
    __builtin_amdgcn_sched_barrier(0);
    const float *S0 = a.S0 + static_cast<size_t>(bh) * D * D;
    float4 s0[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) s0[q] = reinterpret_cast<const float4 *>(S0 + (krow + q) * D)[c4];
    __builtin_amdgcn_sched_barrier(0);

    float4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    double tot = 0.0;  // log2 of the decay over the chunks folded in so far
    int prev_last = -1, bad = INT_MAX;
    if (nch > 0) first.finish(a, mv, sl.n, rw, krow, c4, acc, tot, prev_last, bad);
    for (int c = 1; c < nch; ++c) {  // paths longer than 64 nodes
        Chunk<BF, NG> ch;
        ch.issue(a, par, c, mv, pb[min(64 * c + lane, T - 1)], rw, abase, krow, c4);
        ch.finish(a, mv, sl.n, rw, krow, c4, acc, tot, prev_last, bad);
    }
    const int st = !lenok ? -1 : (bad == INT_MAX ? 0 : bad);
    if (a.path_status && h == 0 && chunk == 0 && lane == 0) a.path_status[b] = st;
    const float Pa = __builtin_amdgcn_exp2f(static_cast<float>(tot));
    float *Sn = a.S_new + static_cast<size_t>(bh) * D * D;
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 o = st != 0 ? make_float4(qnan, qnan, qnan, qnan)
                                 : make_float4(Pa * s0[q].x + acc[q].x, Pa * s0[q].y + acc[q].y,
                                               Pa * s0[q].z + acc[q].z, Pa * s0[q].w + acc[q].w);
        __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w}, reinterpret_cast<f32x4 *>(Sn + (krow + q) * D) + c4);
    }
}

template <bool BF, int NG>
__global__ __launch_bounds__(64) void commit_kernel(CommitArgs a) {
    commit_body<BF, NG>(a, xcd_remap(blockIdx.x, gridDim.x));
}

// Every layer's commit in one launch: the layers share the tree and the accepted path, each has
// its own state, keys, pseudo-values and gates. Layer 0 writes the path status.
template <bool BF, int NG>
__global__ __launch_bounds__(64) void commit_layers_kernel(CommitLayersArgs la) {
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int per_layer = la.base.B * la.base.H * (D / CROWS);
    const int l = g / per_layer;
    CommitArgs a = la.base;
    a.S0 = la.S0[l];
    a.k = la.k[l];
    a.U = la.U[l];
    a.alpha = la.alpha[l];
    a.S_new = la.S_new[l];
    if (l != 0) a.path_status = nullptr;
    commit_body<BF, NG>(a, g - l * per_layer);
}

hipError_t launch_commit_layers(const CommitLayersArgs &la, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(la.L * la.base.B * la.base.H * (D / CROWS))), block(64);
    if (la.base.bf16)
        hipLaunchKernelGGL((commit_layers_kernel<true, CGRP>), grid, block, 0, stream, la);
    else
        hipLaunchKernelGGL((commit_layers_kernel<false, CGRP>), grid, block, 0, stream, la);
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * (D / CROWS))), block(64);
    if (a.bf16)
        hipLaunchKernelGGL((commit_kernel<true, CGRP>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((commit_kernel<false, CGRP>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace canopy
