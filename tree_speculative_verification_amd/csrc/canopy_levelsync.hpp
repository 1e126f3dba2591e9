// Level-synchronous solve over a whole tree by ancestor gathers, for bf16 inputs ("The tree
// closed form" on the canopy project page: any topological order works, level order leaves no
// coupling between nodes of one depth, and the level-synchronous solve takes the levels in
// order, U_L = R_L - G_{L,:} U).
//
// Row i of G and of C is non-zero only at the ancestors of i (and C also at i), so a node's
// equation involves its depth d_i ancestors and nothing else:
//   u_i = r_i - sum_{j in A(i)} G_ij u_j,   o_i = P_i q_i^T S0 + C_ii u_i + sum_{j in A(i)} C_ij u_j.
// One workgroup (8 waves, 16 value columns each) holds, in LDS, a table with one entry per
// (node, ancestor) pair (-G_ij, C_ij and where u_j is kept) and a table of the u rows of every
// node that has a child. Phases:
//   build  per-node depth, child flag and level rank; prefix sums give each node's first pair,
//          its U-table row and its place in the level order; the pairs come from the ancestor
//          bitmask (ancestors in index order are the root path in depth order). k of every node
//          is copied into LDS meanwhile.
//   gram   the dot products k_i.k_j and q_i.k_j of every pair (and q_i.k_i) on the matrix cores:
//          16 pairs per 16 x 16 x 128 product (row m of A is k_i of pair m, column m of B is k_j
//          of pair m), whose diagonal holds the 16 dot products; G and C as fp32 entries
//   project  K S0 and Q S0 on the matrix cores, 16 nodes at a time in index order (each wave
//          its 16 value columns): r_i = beta_i (v_i - P_i S0^T k_i) and P_i S0^T q_i, parked in
//          the U and O outputs
//   levels the levels in order (a barrier after each), the nodes of a level spread over the
//          waves, one node per wave at a time: u_i and o_i completed from the parked values by
//          the gathers over the ancestor entries, in fp32.
// The tables bound the trees this path takes (pairs and nodes with a child); a tree beyond them
// takes the blocked solve. Measured on MI355X (T = 256 random recursive trees) the path runs at
// about the blocked solve's time per (sequence, head), every phase bound by latency with the
// one workgroup per CU that its 141 KiB of tables allow, so it is taken on request only.
#pragma once
#include "canopy_prep.hpp"

namespace canopy {

// One (node i, ancestor j) pair.
struct LsPair {
    float g;      // -G_ij = -beta_i Gamma_ij k_i.k_j
    float c;      // C_ij = Gamma_ij q_i.k_j
    int uoff;     // offset (floats) of u_j's row in the U table
    uint32_t ij;  // i | j << 16
};

// One node, at its place in the level order.
struct LsNode {
    float P;      // P_i = exp(l_i)
    float beta;   // beta_i
    int off;      // first pair of node i
    int uoff;     // offset (floats) of u_i's row in the U table (the spare row for a leaf)
    float cdiag;  // C_ii = q_i.k_i
    int node;     // i
    int step;     // 1; 0 in the entry for a missing row, which reads the zero pair throughout
    int pad;
};

template <int MAXT>
struct LsSmem {
    static constexpr int NI = 160;   // nodes with a child whose u rows the table holds
    static constexpr int NP = 2560;  // (node, ancestor) pairs
    static constexpr int UST = 132;  // U-table row stride (floats): rows 4 banks apart
    static constexpr int NWS = MAXT / 64;
    union {
        alignas(16) float utab[(NI + 1) * UST];           // row NI: written by leaves, never read
        alignas(16) uint8_t kst[MAXT * Ops<true>::ROWB];  // k of every node (Gram phase)
    };
    alignas(16) LsPair pairs[NP + 1];  // entry NP: zero
    alignas(16) LsNode rec[MAXT + 1];  // by level-order position; entry MAXT: a missing row
    int off[MAXT];         // first pair of node i
    int uoff[MAXT];        // U-table offset of node i
    int cnt[MAXT];         // nodes per level
    int isint[MAXT];       // node i has a child
    int lstart[MAXT];      // first position of level L in the level order
    int bstart[MAXT];      // first batch of level L
    uint32_t batch[MAXT];  // position | count << 9 | level << 14
    int wsum[NWS][4];
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_sum(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Builds the level order, the batches and the pair list of the tree (n nodes, preprocessed into
// ps; s_beta and s_P hold beta_i and P_i), and copies k of every node into LDS. `par` is the
// parent of node threadIdx.x. Called by every thread of the workgroup; returns the number of
// batches, or 0 when the tree exceeds the tables (the memory may then be reused).
template <int MAXT, int NT>
__device__ int ls_build(LsSmem<MAXT> &s, const PrepSmem<MAXT> &ps, const float *s_beta, const float *s_P,
                        int par, int n, const void *kin, size_t qkbase, size_t qkrs) {
    static_assert(MAXT <= NT && MAXT % 64 == 0, "one thread per node");
    using S = LsSmem<MAXT>;
    constexpr int BLK = 64 * Ops<true>::ROWB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // k of every node into LDS for the Gram phase (rows past n repeat row n - 1), in flight
    // while the tables are built
    for (int blk = 0; 64 * blk < n; ++blk) dma_block<true, NT>(s.kst + blk * BLK, kin, qkbase, qkrs, 64 * blk, n);
    const bool own = tid < MAXT;
    const int i = tid;
    const bool real = own && i < n;
    const int d = real ? node_depth<MAXT>(ps, i) : 0;
    if (own) {
        s.isint[i] = 0;
        s.cnt[i] = 0;
    }
    __syncthreads();
    int rank = 0;
    if (real) {
        if (par >= 0) s.isint[par] = 1;
        rank = atomicAdd(&s.cnt[d], 1);
    }
    __syncthreads();
    // Exclusive prefix sums over nodes (depth -> first pair, child flag -> U-table row) and over
    // levels (count -> first position, batches of 16 -> first batch).
    const int x0 = d, x1 = real ? s.isint[i] : 0;
    const int c = own ? s.cnt[i] : 0;
    const int x2 = c, x3 = (c + 15) >> 4;
    const int y0 = wave_incl_sum(x0, lane), y1 = wave_incl_sum(x1, lane);
    const int y2 = wave_incl_sum(x2, lane), y3 = wave_incl_sum(x3, lane);
    if (own && lane == 63) {
        s.wsum[wave][0] = y0;
        s.wsum[wave][1] = y1;
        s.wsum[wave][2] = y2;
        s.wsum[wave][3] = y3;
    }
    __syncthreads();
    int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < S::NWS; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            tot[q] += s.wsum[w][q];
            if (w < wave) pre[q] += s.wsum[w][q];
        }
    if (tot[0] > S::NP || tot[1] > S::NI) {
        wait_vmem();      // the staged k has landed, and
        __syncthreads();  // every thread has read the sums, before the memory is reused
        return 0;
    }
    const int myoff = pre[0] + y0 - x0;
    const int myuoff = x1 ? (pre[1] + y1 - x1) * S::UST : S::NI * S::UST;
    if (own) {
        s.off[i] = myoff;
        s.uoff[i] = myuoff;
        s.lstart[i] = pre[2] + y2 - x2;
        s.bstart[i] = pre[3] + y3 - x3;
    }
    __syncthreads();
    if (real) {
        s.rec[s.lstart[d] + rank] = LsNode{s_P[i], s_beta[i], myoff, myuoff, 0.f, i, 1, 0};
        int p = myoff;
#pragma unroll
        for (int w = 0; w < MAXT / 32; ++w) {
            uint32_t m = ps.mask[i][w];
            if (w == (i >> 5)) m &= ~(1u << (i & 31));
            while (m) {
                const int j = 32 * w + __builtin_ctz(m);
                m &= m - 1u;
                s.pairs[p].uoff = s.uoff[j];
                s.pairs[p].ij = static_cast<uint32_t>(i) | (static_cast<uint32_t>(j) << 16);
                ++p;
            }
        }
    }
    if (tid == 0) {
        s.pairs[S::NP] = LsPair{0.f, 0.f, 0, 0u};
        s.rec[MAXT] = LsNode{0.f, 0.f, S::NP, S::NI * S::UST, 0.f, 0, 0, 0};
    }
    if (own && c > 0) {
        const int b0 = s.bstart[i], p0 = s.lstart[i];
        for (int q = 0; 16 * q < c; ++q)
            s.batch[b0 + q] = static_cast<uint32_t>(p0 + 16 * q) |
                              (static_cast<uint32_t>(min(16, c - 16 * q)) << 9) |
                              (static_cast<uint32_t>(i) << 14);
    }
    wait_vmem();
    __syncthreads();
    return tot[3];
}

// The Gram entries of every pair, and C_ii, spread over the workgroup's NW waves: one tile of
// 16 pairs (or, past the pairs, the nodes at 16 level-order positions, with j = i) per step,
// k_i and k_j from the staged k, q_i from global memory requested three steps ahead into a
// fixed ring of registers (loads are issued on every path, node 0 standing in for a missing
// row, so that the waits for them stay exact).
template <int MAXT, int NW>
__device__ void ls_gram(LsSmem<MAXT> &s, const PrepSmem<MAXT> &ps, const float *s_beta, const uint16_t *qp,
                        size_t qkbase, size_t qkrs, int n) {
    constexpr int BLK = 64 * Ops<true>::ROWB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int npairs = s.off[n - 1] + node_depth<MAXT>(ps, n - 1);
    const int npt = (npairs + 15) >> 4;
    const int nt = npt + ((n + 15) >> 4);
    const bool diag = (lr >> 2) == lg;  // this lane holds output (lr, lr)
    const BufRsrc rq = buf_rsrc(qp + qkbase);
    const uint32_t rsb = static_cast<uint32_t>(qkrs) * 2;  // node stride (bytes)
    struct Slot {
        int i, j, p;  // rows of this lane (-1: none); pair index, or -1 - position
        bf16x8 q[4];
    };
    auto fill = [&](int t, Slot &x) {
        x.i = x.j = -1;
        x.p = 0;
        if (t < npt) {
            const int p = 16 * t + lr;
            if (p < npairs) {
                const uint32_t ij = s.pairs[p].ij;
                x.i = static_cast<int>(ij & 0xFFFFu);
                x.j = static_cast<int>(ij >> 16);
                x.p = p;
            }
        } else if (t < nt) {
            const int pos = 16 * (t - npt) + lr;
            if (pos < n) {
                x.i = x.j = s.rec[pos].node;
                x.p = -1 - pos;
            }
        }
        const uint32_t vo = static_cast<uint32_t>(x.i >= 0 ? x.i : 0) * rsb + 16u * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            x.q[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, vo, 64 * ks, 0));
    };
    auto work = [&](const Slot &x) {
        const int ri = x.i >= 0 ? x.i : 0, rj = x.j >= 0 ? x.j : 0;
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 ka = Ops<true>::lds_frag(s.kst + (ri >> 6) * BLK, ri & 63, 4 * ks + lg).x;
            const bf16x8 kb = Ops<true>::lds_frag(s.kst + (rj >> 6) * BLK, rj & 63, 4 * ks + lg).x;
            kk = mfma_bf16(ka, kb, kk);
            qk = mfma_bf16(x.q[ks], kb, qk);
        }
        if (diag && x.i >= 0) {
            const int e = lr & 3;
            const float vkk = e == 0 ? kk[0] : e == 1 ? kk[1] : e == 2 ? kk[2] : kk[3];
            const float vqk = e == 0 ? qk[0] : e == 1 ? qk[1] : e == 2 ? qk[2] : qk[3];
            if (x.p >= 0) {
                // Gamma_ij = 2^(ell_i - ell_j), the log2 path sums differenced in fp64
                const float gam = __builtin_amdgcn_exp2f(static_cast<float>(ps.ell[x.i] - ps.ell[x.j]));
                s.pairs[x.p].g = -s_beta[x.i] * gam * vkk;
                s.pairs[x.p].c = gam * vqk;
            } else {
                s.rec[-1 - x.p].cdiag = vqk;
            }
        }
    };
    Slot a, b, c;
    fill(wave, a);
    fill(wave + NW, b);
    fill(wave + 2 * NW, c);
    for (int t = wave; t < nt; t += 3 * NW) {
        work(a);
        fill(t + 3 * NW, a);
        if (t + NW >= nt) break;
        work(b);
        fill(t + 4 * NW, b);
        if (t + 2 * NW >= nt) break;
        work(c);
        fill(t + 5 * NW, c);
    }
}

// The projections of every node, in index order, for this wave's 16 value columns col0 ..
// col0+15: r_i = beta_i (v_i - P_i S0^T k_i) into U and P_i S0^T q_i into O, the two values the
// level loop then completes. k_i from the staged k; q_i through a two-slot ring in LDS that
// waves 0-3 fill one 16-node tile at a time (each 1 KB of it, requested four tiles ahead into
// registers), so that every q row is fetched once per workgroup rather than once per wave; v_i
// from global memory four tiles ahead. The tile loop has a fixed trip count (MAXT / 16), fully
// unrolled so that the waits for the loads in flight are exact, with a workgroup barrier per
// tile; rows past the tree repeat node n - 1, whose values they then store again unchanged.
// s0f: the wave's S0 columns as split B operands. All threads of the workgroup call it. The
// caller waits for the stores before the level loop reads them back.
template <int MAXT, int NT>
__device__ void ls_project(LsSmem<MAXT> &s, const float *s_beta, const float *s_P, const uint16_t *qp,
                           const uint16_t *vp, size_t qkbase, size_t qkrs, size_t base, size_t rs, int col0,
                           const Ops<true>::Sp (&s0f)[4], int n, float *Uo, float *Oo) {
    constexpr int BLK = 64 * Ops<true>::ROWB;
    constexpr int TILEB = 16 * Ops<true>::ROWB;  // one 16-row tile of q in LDS (4 KB)
    constexpr int NTILE = MAXT / 16;
    constexpr int DIST = 4;
    static_assert(static_cast<int>(sizeof(s.utab)) - MAXT * Ops<true>::ROWB >= 2 * TILEB, "room for the q ring");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int col = col0 + lr;
    uint8_t *ring = s.kst + MAXT * Ops<true>::ROWB;  // two q tiles, in the U table's spare memory
    const BufRsrc rq = buf_rsrc(qp + qkbase), rv = buf_rsrc(vp + base);
    const BufRsrc ru = buf_rsrc(Uo + base), ro = buf_rsrc(Oo + base);
    const uint32_t qkb = static_cast<uint32_t>(qkrs) * 2;
    const uint32_t vrs = static_cast<uint32_t>(rs);
    const bool filler = wave < 4;  // waves 0-3 carry the q tiles, 1 KB each
    // the LDS offset this lane fills within a tile, and the swizzled global chunk that goes there
    const int fo = 1024 * (wave & 3) + 16 * lane;
    const int frow = fo / Ops<true>::ROWB, fch = ((fo % Ops<true>::ROWB) >> 4) ^ (frow & 15);
    auto qload = [&](int t) {
        const int row = min(16 * t + frow, n - 1);
        return __builtin_amdgcn_raw_buffer_load_b128(rq, static_cast<uint32_t>(row) * qkb + 16u * fch, 0, 0);
    };
    auto qstore = [&](int t, u32x4 x) { *reinterpret_cast<u32x4 *>(ring + (t & 1) * TILEB + fo) = x; };
    auto vload = [&](int t, uint16_t (&v)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = min(16 * t + 4 * lg + e, n - 1);
            v[e] = __builtin_amdgcn_raw_buffer_load_b16(rv, (static_cast<uint32_t>(i) * vrs + col) * 2, 0, 0);
        }
    };
    auto work = [&](int t, const uint16_t (&v)[4]) {
        const int ra = min(16 * t + lr, n - 1);
        f32x4 ksum = {0.f, 0.f, 0.f, 0.f}, qsum = {0.f, 0.f, 0.f, 0.f};
        f32x4 klo = {0.f, 0.f, 0.f, 0.f}, qlo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 ka = Ops<true>::lds_frag(s.kst + (ra >> 6) * BLK, ra & 63, 4 * ks + lg).x;
            const bf16x8 qa = Ops<true>::lds_frag(ring + (t & 1) * TILEB, lr, 4 * ks + lg).x;
            ksum = mfma_bf16(ka, s0f[ks].hi, ksum);
            klo = mfma_bf16(ka, s0f[ks].lo, klo);
            qsum = mfma_bf16(qa, s0f[ks].hi, qsum);
            qlo = mfma_bf16(qa, s0f[ks].lo, qlo);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = min(16 * t + 4 * lg + e, n - 1);
            const float P = s_P[i];
            const float r = s_beta[i] * (bf16_to_f32(v[e]) - P * (ksum[e] + klo[e]));
            const float o = P * (qsum[e] + qlo[e]);
            const uint32_t go = (static_cast<uint32_t>(i) * vrs + col) * 4;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(r), ru, go, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ro, go, 0, 0);
        }
    };
    u32x4 qr[DIST];
    uint16_t vr[DIST][4];
#pragma unroll
    for (int t = 0; t < DIST && t < NTILE; ++t) {
        if (filler) qr[t] = qload(t);
        vload(t, vr[t]);
    }
    if (filler) qstore(0, qr[0]);
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
        // tile t is in its slot, and every wave is done with tile t - 1, whose slot takes t + 1
        lds_barrier();
        if (filler) {
            if (t + 1 < NTILE) qstore(t + 1, qr[(t + 1) % DIST]);
            if (t + 1 + DIST - 1 < NTILE) qr[(t + DIST) % DIST] = qload(t + DIST);
        }
        work(t, vr[t % DIST]);
        if (t + DIST < NTILE) vload(t + DIST, vr[t % DIST]);
    }
}

// The level loop. The levels are taken in order, a workgroup barrier after each (a level reads
// the u rows of the levels before it); inside a level the waves take its nodes round-robin by
// level-order position, two nodes per wave at a time (both of depth L, so their gather loops
// run in step and their LDS round trips overlap), two value columns per lane. A node's u_i and
// o_i are completed from the projections (read back from U and O) by the gathers over its
// ancestor entries in fp32: the entries are read once (one lane each) and handed to the whole
// wave by readlane, so that the LDS traffic is the u rows alone. A missing second node reads
// the entry for a missing row (zero pairs, the spare U-table row) and stores nothing. Global
// accesses go through buffer resources with 32-bit offsets (the caller checks that one
// sequence's rows span less than 2^31 bytes).
template <int MAXT, int NW>
__device__ void ls_levels(LsSmem<MAXT> &s, size_t base, size_t rs, int n, int nbatch, float *Uo, float *Oo) {
    using S = LsSmem<MAXT>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const BufRsrc ru = buf_rsrc(Uo + base), ro = buf_rsrc(Oo + base);
    const uint32_t vrs = static_cast<uint32_t>(rs);
    const int nlev = static_cast<int>(s.batch[nbatch - 1] >> 14) + 1;
    struct Nd {
        LsNode rd;
        float r0, r1, o0, o1;
        LsPair pe;
    };
    auto open = [&](int p, bool ok, int L, Nd &x) {
        x.rd = s.rec[ok ? p : MAXT];
        const uint32_t go = (static_cast<uint32_t>(x.rd.node) * vrs + 2 * lane) * 4;
        x.r0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ru, go, 0, 0));
        x.r1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ru, go, 4, 0));
        x.o0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, go, 0, 0));
        x.o1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, go, 4, 0));
        x.pe = LsPair{0.f, 0.f, S::NI * S::UST, 0u};
        if (ok && lane < L) x.pe = s.pairs[x.rd.off + lane];
    };
    auto step = [&](Nd &x, int a) {
        const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x.pe.g), a));
        const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x.pe.c), a));
        const int uo = __builtin_amdgcn_readlane(x.pe.uoff, a);
        const float2 ua = *reinterpret_cast<const float2 *>(&s.utab[uo + 2 * lane]);
        x.r0 = fmaf(g, ua.x, x.r0);
        x.r1 = fmaf(g, ua.y, x.r1);
        x.o0 = fmaf(c, ua.x, x.o0);
        x.o1 = fmaf(c, ua.y, x.o1);
    };
    auto close = [&](Nd &x, bool ok) {
        x.o0 = fmaf(x.rd.cdiag, x.r0, x.o0);
        x.o1 = fmaf(x.rd.cdiag, x.r1, x.o1);
        *reinterpret_cast<float2 *>(&s.utab[x.rd.uoff + 2 * lane]) = make_float2(x.r0, x.r1);
        if (ok) {
            const uint32_t go = (static_cast<uint32_t>(x.rd.node) * vrs + 2 * lane) * 4;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x.r0), ru, go, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x.r1), ru, go, 4, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x.o0), ro, go, 0, 2);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x.o1), ro, go, 4, 2);
        }
    };
    for (int L = 0; L < nlev; ++L) {
        const int end = L + 1 < nlev ? s.lstart[L + 1] : n;
        for (int p = s.lstart[L] + wave; p < end; p += 2 * NW) {
            const bool ok2 = p + NW < end;
            Nd x, y;
            open(p, true, L, x);
            open(p + NW, ok2, L, y);
            for (int a0 = 0; a0 < L; a0 += 64) {
                if (a0 > 0) {
                    x.pe = LsPair{0.f, 0.f, S::NI * S::UST, 0u};
                    y.pe = x.pe;
                    if (a0 + lane < L) {
                        x.pe = s.pairs[x.rd.off + a0 + lane];
                        if (ok2) y.pe = s.pairs[y.rd.off + a0 + lane];
                    }
                }
                const int na = min(64, L - a0);
                for (int a = 0; a < na; ++a) {
                    step(x, a);
                    step(y, a);
                }
            }
            close(x, true);
            close(y, ok2);
        }
        lds_barrier();
    }
}

}  // namespace canopy
