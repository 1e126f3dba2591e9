// Tree verification for trees of at most 16 nodes: one wave per (sequence, head, 16 value
// columns), everything in registers, no LDS and no barrier. The same closed form as the
// general kernel (the canopy project page, "The tree closed form"), specialised to a single
// 16-node tile:
//   prep   pointer jumping over lanes (lane i = node i) with shuffles: ancestor mask, depth,
//          path sums of log2 alpha (fp64), l_i = ln 2 times the sum
//   a2     KS = K S0, QS = Q S0 (MFMA, K and Q fragments loaded straight from global memory)
//   a3     K K^T and K Q^T (MFMA with K as the A operand, so lane (g, r) holds row r, columns
//          4g..4g+3), masked and decay-weighted into -G (strict ancestors) and C (path)
//   a4     U = sum_{m=0..d} (-G)^m R, the finite Neumann series with one term per tree level
//          (d = the tree's depth < 16), one 16-long MFMA product per term
//   a5     O = diag(P) QS + C U (MFMA)
// The Gram tiles come out with row r, columns 4g..4g+3 in lane (g, r), and the node-by-column
// tiles (R, the series terms, U) with rows 4g..4g+3 of column r in lane (g, r): exactly the A
// and B placements of a 16-long MFMA reduction, so the series and the read-out move no data
// between lanes. A workgroup holds NWV waves, each on its own 16 value columns of one head.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

template <bool BF, int NWV>
__global__ __launch_bounds__(64 * NWV) void verify_small_kernel(VerifyArgs a) {
    using Op = Ops<BF>;
    using In = typename Op::In;
    using Sp = typename Op::Sp;
    constexpr int TILES = D / 16;
    constexpr int GROUPS = TILES / NWV;  // workgroups per head
    const int gid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (gid % GROUPS) * NWV + static_cast<int>(threadIdx.x >> 6);
    const int bh = gid / GROUPS;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const int col0 = tile * 16;
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;
    const size_t qkrs = static_cast<size_t>(a.HK) * D;
    const size_t qkbase = qk_base(b, h, H, a.HK, T);
    const bool writer = tile == 0;  // this head's wave for the per-node outputs
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;  // this sequence's node count

    // ---- every load up front, unconditional (rows and nodes past T read row or node T-1;
    // rows and nodes past Tb are padding, dropped by selects later), so that they all issue
    // before the first one is waited for: the tree and gates (lane = node), K and Q fragments
    // (row lr), S0 fragments (column col0 + lr), V (result order)
    const int node = lane;
    const bool real = node < Tb;
    const int nodec = min(node, T - 1);
    const int par_in = a.parent[static_cast<size_t>(b) * T + nodec];
    const float alpha_in = a.alpha[sbase + static_cast<size_t>(nodec) * H];
    const float beta_in = a.beta[sbase + static_cast<size_t>(nodec) * H];
    const size_t erow = qkbase + static_cast<size_t>(min(lr, T - 1)) * qkrs + 8 * lg;
    In kf[4], qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = Op::template load_frag<In>(a.k, erow + 32 * ks, true);
        qf[ks] = Op::template load_frag<In>(a.q, erow + 32 * ks, true);
    }
    float s0v[4][8];
    {
        const float *S0p = a.S0 + static_cast<size_t>(bh) * D * D + col0 + lr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) s0v[ks][e] = S0p[(32 * ks + 8 * lg + e) * D];
    }
    typename Op::Raw vraw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        vraw[e] = Op::load_raw(a.v, base + static_cast<size_t>(min(4 * lg + e, T - 1)) * rs + col0 + lr);

    // ---- prep: validation, then pointer jumping across lanes. A malformed tree is computed
    // through like a forest (bad parents read as -1) and replaced by NaN at the stores, so that
    // no branch separates the loads from their uses.
    const bool badn = real && (par_in < -1 || par_in >= node);
    const unsigned long long badm = __ballot(badn);
    // -1 for a length out of range, else 1 + the first bad node
    const int bad = sl.bad ? -1 : (badm ? (__ffsll(static_cast<unsigned long long>(badm))) : 0);
    const float beta = real ? beta_in : 0.f;
    // log2 alpha by the hardware logarithm (about 1 ulp, an error relative to each term, so it
    // stays relative to any difference of path sums); the sums themselves in fp64. ell holds
    // path sums of log2 alpha: l = ell ln 2, P = 2^ell, decay ratios 2^(ell_i - ell_j).
    uint32_t mask = real ? (1u << node) : 0u;
    double ell = real ? static_cast<double>(__builtin_amdgcn_logf(alpha_in)) : 0.0;
    int jmp = (real && !badn) ? par_in : -1;
    // After round r every node's jump pointer is 2^(r+1) levels up; depth < 16 ends it in 4.
    for (int round = 0; round < 4 && __any(jmp >= 0); ++round) {
        const int src = jmp >= 0 ? jmp : lane;
        const uint32_t pm = __shfl(mask, src, 64);
        const double pl = __shfl(ell, src, 64);
        const int pj = __shfl(jmp, src, 64);
        const bool up = jmp >= 0;
        mask = up ? (mask | pm) : mask;
        ell = up ? ell + pl : ell;
        jmp = up ? pj : jmp;
    }
    const float ellf = static_cast<float>(ell * 0.69314718055994530942);  // l = ln P
    const float P = real ? __builtin_amdgcn_exp2f(static_cast<float>(ell)) : 0.f;
    const int depth = real ? __popc(mask) - 1 : -1;
    // Tree depth by ballots on its 4 bits (depth < 16).
    int dmax = 0;
#pragma unroll
    for (int bit = 3; bit >= 0; --bit)
        if (__any(depth >= (dmax | (1 << bit)))) dmax |= 1 << bit;
    if (writer && real) a.ell[sbase + static_cast<size_t>(node) * H] = bad ? __builtin_nanf("") : ellf;
    if (writer && h == 0) {
        if (a.tree_status && lane == 0) a.tree_status[b] = bad;
        if (real && a.depth) a.depth[static_cast<size_t>(b) * T + node] = bad ? 0 : depth;
        if (real && a.anc_mask) a.anc_mask[static_cast<size_t>(b) * T + node] = bad ? 0u : mask;
    }

    // ---- a2: projections; result order: lane (lg, lr) holds rows 4lg+e of column lr
    Sp s0f[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s0f[ks] = Op::split(s0v[ks]);
    f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        ak = Op::mma(kf[ks], s0f[ks], ak);
        aq = Op::mma(qf[ks], s0f[ks], aq);
    }
    float rhs[4];
    f32x4 o0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * lg + e;
        const float bi = __shfl(beta, i, 64), Pi = __shfl(P, i, 64);
        const float r = bi * (Op::raw_f32(vraw[e]) - Pi * ak[e]), o = Pi * aq[e];
        rhs[e] = i < Tb ? r : 0.f;
        o0[e] = i < Tb ? o : 0.f;
    }

    // ---- a3: Gram tile with K as the A operand: lane (lg, lr) holds row i = lr, columns
    // j = 4lg .. 4lg+3 of K K^T and of Q K^T
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kk = Op::mma(kf[ks], kf[ks], kk);
        qk = Op::mma(kf[ks], qf[ks], qk);
    }
    // kk[e] = k_{4lg+e} . k_lr and qk[e] = k_{4lg+e} . q_lr, i.e. row i = lr, column j = 4lg+e
    float gneg[4], cm[4];
    {
        const int i = lr;
        const uint32_t mi = __shfl(mask, i, 64);
        const double li = __shfl(ell, i, 64);
        const float bi = __shfl(beta, i, 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * lg + e;
            const double lj = __shfl(ell, j, 64);
            // Off the path the exponent may overflow; the selects drop those entries.
            const float gam = __builtin_amdgcn_exp2f(static_cast<float>(li - lj));
            const bool onpath = (mi >> j) & 1u;
            cm[e] = onpath ? gam * qk[e] : 0.f;
            gneg[e] = (onpath && i != j) ? -bi * gam * kk[e] : 0.f;
        }
    }
    const typename Op::Sp4 gf = Op::split4(gneg);
    const typename Op::Sp4 cf = Op::split4(cm);

    // ---- a4: U = sum_{m=0..dmax} (-G)^m R; each term in result order is the next B operand
    float u[4], z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = z[e] = rhs[e];
    for (int m = 1; m <= dmax; ++m) {
        f32x4 nz = {0.f, 0.f, 0.f, 0.f};
        nz = Op::mma16(gf, Op::split4(z), nz);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = nz[e];
            u[e] += nz[e];
        }
    }
    // ---- a5: O = diag(P) QS + C U
    const f32x4 oc = Op::mma16(cf, Op::split4(u), o0);

    // ---- a6: outputs (NaN for a malformed tree)
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * lg + e;
        if (i < Tb) {
            a.U[base + static_cast<size_t>(i) * rs + col0 + lr] = bad ? qnan : u[e];
            store_nt(a.O + base + static_cast<size_t>(i) * rs + col0 + lr, bad ? qnan : oc[e]);
        }
    }
}

template <bool BF>
static void launch_small_nwv(const VerifyArgs &a, int nwv, hipStream_t stream) {
    const unsigned heads = static_cast<unsigned>(a.B * a.H);
    switch (nwv) {
        case 1:
            hipLaunchKernelGGL((verify_small_kernel<BF, 1>), dim3(heads * 8), dim3(64), 0, stream, a);
            break;
        case 2:
            hipLaunchKernelGGL((verify_small_kernel<BF, 2>), dim3(heads * 4), dim3(128), 0, stream, a);
            break;
        case 4:
            hipLaunchKernelGGL((verify_small_kernel<BF, 4>), dim3(heads * 2), dim3(256), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((verify_small_kernel<BF, 8>), dim3(heads), dim3(512), 0, stream, a);
            break;
    }
}

// waves: waves per workgroup (1, 2, 4 or 8; 0 picks the default).
hipError_t launch_verify_small(const VerifyArgs &a, int waves, hipStream_t stream) {
    const int nwv = waves == 0 ? 1 : waves;
    if (a.bf16)
        launch_small_nwv<true>(a, nwv, stream);
    else
        launch_small_nwv<false>(a, nwv, stream);
    return hipGetLastError();
}

}  // namespace canopy
