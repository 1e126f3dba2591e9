// Tree verification for trees of 65 to 256 nodes with bf16 inputs ("The tree closed form" on
// the canopy project page), for batches small enough that one workgroup per (sequence, head,
// 16 value columns) does not oversubscribe the GPU. One wave per 16-node sub-block (up to 16
// waves): wave p owns nodes 16p .. 16p+15.
//   prep   64-node chunks, one wave per chunk: pointer jumping over lane shuffles inside the
//          chunk, then the chunks completed in order through their exits (each node's first
//          ancestor outside its chunk), into a shared LDS table of 256-bit ancestor masks,
//          fp64 path sums of log2 alpha, beta and P
//   stage  keys (each wave its own 16 rows) and the workgroup's S0 columns, transposed and
//          split into bf16 hi + lo, in LDS once per workgroup
//   a2     K_p S0 and Q_p S0 for the wave's rows (MFMA); R_p and diag(P) Q_p S0
//   a3/a4  forward substitution over the sub-blocks ("Design decisions / Two solve
//          strategies", blocked by 16 nodes): U_p = (I + G_pp)^-1 (R_p - sum_{c<p} G_pc U_c).
//          The diagonal inverse is the squaring product (I + N)(I + N^2)(I + N^4)(I + N^8),
//          N = -G_pp, truncated at the sub-block's depth and multiplied out before it is
//          needed. The Gram tiles G_pc, C_pc are formed one at a time as U_c arrives (K_c as
//          the A operand, so each tile lands in the A placement of a 16-long reduction); the
//          tile needed last, (p, p-1), is formed first so that the sequential part is two
//          products per sub-block. Solved tiles pass between waves through LDS flags, as bf16
//          hi + lo parts; every 16-long product of the chain takes three bf16 matrix-core passes
//          (hi hi + hi lo + lo hi, relative error about 2^-16).
//   a5     O_p = diag(P) Q_p S0 + sum_{c<=p} C_pc U_c, accumulated as the U_c arrive
// Node-by-column tiles (R, U) sit with rows 4g..4g+3 of column r in lane (g, r), the result
// placement of an MFMA and the B placement of the 16-long reduction.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

constexpr int WMAXT = 256;
constexpr int WMW = WMAXT / 32;  // mask words per node

template <int NCT>
struct WideSmem {
    uint8_t k[WMAXT * Ops<true>::ROWB];
    union {
        uint8_t s0[16 * NCT * 512];  // S0 columns as bf16 hi rows, then lo rows
        float4 x[WMAXT / 16][NCT][64];  // solved U tiles as bf16 hi (8 bytes) + lo (8 bytes)
    } u;
    double lam[WMAXT];
    uint32_t mask[WMAXT][WMW];
    float beta[WMAXT];
    float P[WMAXT];
    int exitn[WMAXT];
    int ready[WMAXT / 16];
    int bad;
};

// One Gram tile (p, c): lane (lg, lr) gets row i = 16p + lr and columns j = 16c + 4lg + e of
// -G (strict ancestors) and C (path), from K_c (A operand, LDS) and the wave's K_p, Q_p.
template <int NCT>
__device__ __forceinline__ void wide_tile(const WideSmem<NCT> &sm, const Ops<true>::In (&kp)[4],
                                          const Ops<true>::In (&qp)[4], int p, int c, int lr, int lg,
                                          float (&g)[4], float (&cm)[4], f32x4 &kk_out) {
    using Op = Ops<true>;
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const Op::In kc = Op::lds_frag(sm.k, 16 * c + lr, 4 * ks + lg);
        kk = Op::mma(kc, kp[ks], kk);
        qk = Op::mma(kc, qp[ks], qk);
    }
    const int i = 16 * p + lr;
    const int j0 = 16 * c + 4 * lg;
    const double li = sm.lam[i];
    const float bi = sm.beta[i];
    const uint32_t mbits = sm.mask[i][c >> 1] >> (16 * (c & 1) + 4 * lg);  // bit e: j0 + e on path(i)
    const double2 l01 = *reinterpret_cast<const double2 *>(&sm.lam[j0]);
    const double2 l23 = *reinterpret_cast<const double2 *>(&sm.lam[j0 + 2]);
    const double lj[4] = {l01.x, l01.y, l23.x, l23.y};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // Off the path the exponent may overflow; the selects drop those entries.
        const float gam = __builtin_amdgcn_exp2f(static_cast<float>(li - lj[e]));
        const bool onpath = (mbits >> e) & 1u;
        cm[e] = onpath ? gam * qk[e] : 0.f;
        g[e] = (onpath && i != j0 + e) ? -bi * gam * kk[e] : 0.f;
    }
    kk_out = kk;
}

// A solved U tile (rows 4 lg .. 4 lg + 3 of column lr in lane (lg, lr)) as bf16 hi and lo parts,
// 16 bytes per lane in the tile's LDS slot.
template <int NCT>
__device__ __forceinline__ void wide_put_tile(WideSmem<NCT> &sm, int s, int ct, int lane, Ops<true>::Sp4 t) {
    const uint2 h = __builtin_bit_cast(uint2, t.hi), l = __builtin_bit_cast(uint2, t.lo);
    sm.u.x[s][ct][lane] = make_float4(__uint_as_float(h.x), __uint_as_float(h.y), __uint_as_float(l.x),
                                      __uint_as_float(l.y));
}
template <int NCT>
__device__ __forceinline__ Ops<true>::Sp4 wide_get_tile(const WideSmem<NCT> &sm, int s, int ct, int lane) {
    const float4 x = sm.u.x[s][ct][lane];
    Ops<true>::Sp4 t;
    t.hi = __builtin_bit_cast(i16x4, make_uint2(__float_as_uint(x.x), __float_as_uint(x.y)));
    t.lo = __builtin_bit_cast(i16x4, make_uint2(__float_as_uint(x.z), __float_as_uint(x.w)));
    return t;
}

template <int NCT>
__global__ __launch_bounds__(1024) void verify_wide_kernel(VerifyArgs a) {
    using Op = Ops<true>;
    using In = Op::In;
    using Sp = Op::Sp;
    using Smem = WideSmem<NCT>;
    constexpr int GROUPS = D / (16 * NCT);  // workgroups per head
    __shared__ __align__(16) Smem sm;

    const int gid = xcd_remap(blockIdx.x, gridDim.x);
    const int grp = gid % GROUPS;
    const int bh = gid / GROUPS;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int NT = blockDim.x;
    const int tid = threadIdx.x;
    const int nsb = NT >> 6;
    // This wave's sub-block. Waves w, w+4, w+8, w+12 share a SIMD and sub-block p carries work
    // proportional to p, so each full group of four waves takes its sub-blocks in alternating
    // order: the SIMDs then get equal shares.
    const int p = [&] {
        const int w = tid >> 6, grpw = w >> 2, j = w & 3;
        if (4 * grpw + 4 > nsb) return w;
        return (grpw & 1) ? 4 * grpw + 3 - j : w;
    }();
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int nch = (T + 63) >> 6;  // 64-node chunks of the prep
    const int colw = grp * 16 * NCT;
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;
    const size_t qkrs = static_cast<size_t>(a.HK) * D;
    const size_t qkbase = qk_base(b, h, H, a.HK, T);
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;  // this sequence's node count
    const bool writer = grp == 0;  // this head's workgroup for the per-node outputs
    const int32_t *par = a.parent + static_cast<size_t>(b) * T;

    // ---- every load up front, unconditional (rows and nodes past T read row or node T-1; rows
    // and nodes past Tb are padding, dropped by selects later):
    // the prep chunk of a wave p < nch (lane = node 64p + lane), the wave's K and Q rows, the
    // thread's share of the S0 columns and the wave's V rows.
    // Only the prep waves (one per 64-node chunk) load the tree and gates, and only the first
    // NPAIR threads load S0: at the start of the kernel every wave's requests queue behind each
    // other, so requests nothing reads cost time.
    const bool chunkw = p < nch;
    const int cnode = 64 * p + lane;
    const int cnodec = min(cnode, T - 1);
    int par_in = -1;
    float alpha_in = 1.f, beta_in = 0.f;
    if (chunkw) {
        par_in = par[cnodec];
        alpha_in = a.alpha[sbase + static_cast<size_t>(cnodec) * H];
        beta_in = a.beta[sbase + static_cast<size_t>(cnodec) * H];
    }
    In kp[4], qp[4];
    {
        const size_t er = qkbase + static_cast<size_t>(min(16 * p + lr, T - 1)) * qkrs + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kp[ks] = Op::template load_frag<In>(a.k, er + 32 * ks, true);
            qp[ks] = Op::template load_frag<In>(a.q, er + 32 * ks, true);
        }
    }
    constexpr int NPAIR = 16 * NCT * 16;  // (column, 8-index chunk) pairs; 320+ threads
    constexpr int PPT = (NPAIR + 319) / 320;
    float s0v[PPT][8];
    {
        const float *S0p = a.S0 + static_cast<size_t>(bh) * D * D + colw;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            const int x = tid + m * NT;
            if (x < NPAIR) {
                const int c = x % (16 * NCT), kc = x / (16 * NCT);
#pragma unroll
                for (int e = 0; e < 8; ++e) s0v[m][e] = S0p[(8 * kc + e) * D + c];
            }
        }
    }
    uint16_t vraw[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vraw[ct][e] = static_cast<const uint16_t *>(a.v)[base + static_cast<size_t>(min(16 * p + 4 * lg + e, T - 1)) * rs +
                                                           colw + 16 * ct + lr];

    // ---- prep, phase 1: each chunk's in-chunk paths (malformed parents read as -1)
    if (tid == 0) sm.bad = INT_MAX;
    if (tid < WMAXT / 16) sm.ready[tid] = 0;
    __syncthreads();
    if (chunkw) {
        const bool real = cnode < Tb;
        int pp = real ? par_in : -1;
        if (real && (pp < -1 || pp >= cnode)) {
            atomicMin(&sm.bad, cnode + 1);
            pp = -1;
        }
        unsigned long long m = real ? (1ull << lane) : 0ull;
        double l = real ? static_cast<double>(__builtin_amdgcn_logf(alpha_in)) : 0.0;
        const bool inside = pp >= 64 * p;
        int jmp = inside ? pp - 64 * p : -1;
        int ex = inside ? -1 : pp;  // set again from the in-chunk root when the jumps reach it
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
        sm.exitn[cnode] = ex;
        sm.lam[cnode] = l;
        sm.beta[cnode] = real ? beta_in : 0.f;
#pragma unroll
        for (int w = 0; w < WMW; ++w)
            sm.mask[cnode][w] = w == 2 * p ? static_cast<uint32_t>(m)
                                           : (w == 2 * p + 1 ? static_cast<uint32_t>(m >> 32) : 0u);
    }
    // ---- stage: keys and S0 columns (bf16 hi rows, then lo rows)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Op::lds_put(sm.k, 16 * p + lr, 4 * ks + lg, kp[ks]);
#pragma unroll
    for (int m = 0; m < PPT; ++m) {
        const int x = tid + m * NT;
        if (x < NPAIR) {
            const int c = x % (16 * NCT), kc = x / (16 * NCT);
            const Sp sp = Op::split(s0v[m]);
            In hi, lo;
            hi.x = sp.hi;
            lo.x = sp.lo;
            Op::lds_put(sm.u.s0, c, kc, hi);
            Op::lds_put(sm.u.s0 + 16 * NCT * 256, c, kc, lo);
        }
    }
    __syncthreads();
    const int bad = sl.bad ? -1 : (sm.bad == INT_MAX ? 0 : sm.bad);
    // ---- prep, phase 2: chunks completed in order (every exit lies in an earlier chunk)
    for (int c = 1; c < nch; ++c) {
        if (p == c) {
            const int e = sm.exitn[cnode];
            if (e >= 0) {
#pragma unroll
                for (int w = 0; w < WMW; ++w)
                    if (w < 2 * c) sm.mask[cnode][w] = sm.mask[e][w];
                sm.lam[cnode] += sm.lam[e];
            }
        }
        __syncthreads();
    }
    if (chunkw) {
        const bool real = cnode < Tb;
        const double lam = sm.lam[cnode];
        sm.P[cnode] = real ? __builtin_amdgcn_exp2f(static_cast<float>(lam)) : 0.f;
        if (writer && real) {
            const float ellf = static_cast<float>(lam * 0.69314718055994530942);  // l = ln P
            a.ell[sbase + static_cast<size_t>(cnode) * H] = bad ? __builtin_nanf("") : ellf;
        }
        if (writer && h == 0 && real) {
            const int W = (T + 31) >> 5;
            int dep = -1;
#pragma unroll
            for (int w = 0; w < WMW; ++w) dep += __popc(sm.mask[cnode][w]);
            if (a.depth) a.depth[static_cast<size_t>(b) * T + cnode] = bad ? 0 : dep;
            if (a.anc_mask)
                for (int w = 0; w < W; ++w)
                    a.anc_mask[(static_cast<size_t>(b) * T + cnode) * W + w] = bad ? 0u : sm.mask[cnode][w];
        }
        if (writer && h == 0 && tid == 0 && a.tree_status) a.tree_status[b] = bad;
    }
    __syncthreads();

    // ---- a2: projections of the wave's rows; result order (rows 16p + 4lg + e, column lr)
    float rhs[NCT][4];
    f32x4 oacc[NCT];
    {
        const float4 b4 = *reinterpret_cast<const float4 *>(&sm.beta[16 * p + 4 * lg]);
        const float4 p4 = *reinterpret_cast<const float4 *>(&sm.P[16 * p + 4 * lg]);
        const float bi[4] = {b4.x, b4.y, b4.z, b4.w}, Pi[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Sp sf;
                sf.hi = Op::lds_frag(sm.u.s0, 16 * ct + lr, 4 * ks + lg).x;
                sf.lo = Op::lds_frag(sm.u.s0 + 16 * NCT * 256, 16 * ct + lr, 4 * ks + lg).x;
                ak = Op::mma(kp[ks], sf, ak);
                aq = Op::mma(qp[ks], sf, aq);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * p + 4 * lg + e;  // beta and P are 0 past Tb
                const float r = bi[e] * (bf16_to_f32(vraw[ct][e]) - Pi[e] * ak[e]), o = Pi[e] * aq[e];
                rhs[ct][e] = i < Tb ? r : 0.f;
                oacc[ct][e] = i < Tb ? o : 0.f;
            }
        }
    }
    __syncthreads();  // every wave is done with the S0 staging, which the solve overwrites

    // ---- a3/a4: the diagonal tile and its inverse (in the A placement), built as the
    // truncated product of the factors (I + N^(2^s)); with Z = X Y, Z in the A placement is
    // the product of Y's B placement and X's A placement.
    float cdiag[4], minv[4];
    {
        float nA[4], nB[4];
        f32x4 kk;
        wide_tile<NCT>(sm, kp, qp, p, p, lr, lg, nA, cdiag, kk);
        // transposed placement: row i2 = 16p + 4lg + e, column j2 = 16p + lr
        const int i = 16 * p + lr, j0 = 16 * p + 4 * lg;
        const double li = sm.lam[i];
        const float4 bj4 = *reinterpret_cast<const float4 *>(&sm.beta[j0]);
        const float bj[4] = {bj4.x, bj4.y, bj4.z, bj4.w};
        int dl = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + e;
            const bool on2 = (sm.mask[j][i >> 5] >> (i & 31)) & 1u;
            const float gam2 = __builtin_amdgcn_exp2f(static_cast<float>(sm.lam[j] - li));
            nB[e] = (on2 && i != j) ? -bj[e] * gam2 * kk[e] : 0.f;
        }
        if (i < Tb) dl = __popc((sm.mask[i][p >> 1] >> (16 * (p & 1))) & 0xFFFFu) - 1;
        const int dp = wave_max(dl);
        int nf = 0;
        while ((1 << nf) <= dp) ++nf;
        float xa[4], xb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xa[e] = nA[e];
            xb[e] = nB[e];
            minv[e] = (lr == 4 * lg + e ? 1.f : 0.f) + nA[e];  // I + N
        }
        for (int s = 1; s < nf; ++s) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 ya = mma16f(xb, xa, z);
            const f32x4 yb = mma16f(xa, xb, z);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xa[e] = ya[e];
                xb[e] = yb[e];
            }
            const f32x4 mi = mma16f(xb, minv, f32x4{minv[0], minv[1], minv[2], minv[3]});
#pragma unroll
            for (int e = 0; e < 4; ++e) minv[e] = mi[e];
        }
    }
    bool lost = false;  // a result this wave waited for never came (or came from a lost wait)
    // The tile needed last, (p, p-1), first; then the others in the order the U_s arrive.
    float glast[4] = {0.f, 0.f, 0.f, 0.f}, clast[4] = {0.f, 0.f, 0.f, 0.f};
    if (p >= 1) {
        f32x4 kk;
        wide_tile<NCT>(sm, kp, qp, p, p - 1, lr, lg, glast, clast, kk);
    }
    for (int s = 0; s < p; ++s) {
        float g[4], cm[4];
        if (s + 1 < p) {
            f32x4 kk;
            wide_tile<NCT>(sm, kp, qp, p, s, lr, lg, g, cm, kk);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                g[e] = glast[e];
                cm[e] = clast[e];
            }
        }
        const Op::Sp4 gs = Op::split4(g), cs = Op::split4(cm);
        lost |= wait_flag(&sm.ready[s], a.wait_bound) != 1;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const Op::Sp4 tv = wide_get_tile(sm, s, ct, lane);
            const f32x4 r = Op::mma16(gs, tv, f32x4{rhs[ct][0], rhs[ct][1], rhs[ct][2], rhs[ct][3]});
#pragma unroll
            for (int e = 0; e < 4; ++e) rhs[ct][e] = r[e];
            if (s + 1 < p) oacc[ct] = Op::mma16(cs, tv, oacc[ct]);
        }
    }
    float u[NCT][4];
    Op::Sp4 us[NCT];
    {
        const Op::Sp4 ms = Op::split4(minv);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 y = Op::mma16(ms, Op::split4(rhs[ct]), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) u[ct][e] = y[e];
            us[ct] = Op::split4(u[ct]);
            wide_put_tile(sm, p, ct, lane, us[ct]);
        }
    }
    __hip_atomic_store(&sm.ready[p], lost ? 2 : 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    // ---- a5: the read-out terms left: the last incoming tile and the wave's own
    {
        const Op::Sp4 cl = Op::split4(clast), cd = Op::split4(cdiag);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (p >= 1) oacc[ct] = Op::mma16(cl, wide_get_tile(sm, p - 1, ct, lane), oacc[ct]);
            oacc[ct] = Op::mma16(cd, us[ct], oacc[ct]);
        }
    }

    // ---- a6: outputs (NaN for a malformed tree and for rows computed from a lost hand-off)
    const float qnan = __builtin_nanf("");
    if (lost && lane == 0) report_lost(a.tree_status, b);
    const bool nanout = bad || lost;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * p + 4 * lg + e;
            if (i < Tb) {
                const size_t o = base + static_cast<size_t>(i) * rs + colw + 16 * ct + lr;
                a.U[o] = nanout ? qnan : u[ct][e];
                store_nt(a.O + o, nanout ? qnan : oacc[ct][e]);
            }
        }
    (void)nsb;
}

// col_tiles: 16-column tiles per workgroup (1 or 2).
hipError_t launch_verify_wide(const VerifyArgs &a, int col_tiles, hipStream_t stream) {
    const unsigned heads = static_cast<unsigned>(a.B * a.H);
    const dim3 block(64 * ((a.T + 15) / 16));
    if (col_tiles == 4)
        hipLaunchKernelGGL((verify_wide_kernel<4>), dim3(heads * 2), block, 0, stream, a);
    else if (col_tiles == 2)
        hipLaunchKernelGGL((verify_wide_kernel<2>), dim3(heads * 4), block, 0, stream, a);
    else
        hipLaunchKernelGGL((verify_wide_kernel<1>), dim3(heads * 8), block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace canopy
