// Tree verification for trees of at most 16 nodes: one wave per (sequence, head, 16 value
// columns), everything in registers, no LDS and no barrier. The same closed form as the
// general kernel (the canopy project page, "The tree closed form"), specialised to a single
// 16-node tile:
//   prep   pointer jumping over lanes (lane i = node i) with shuffles: ancestor mask, depth,
//          l_i = sum of log alpha over path(i) (fp64)
//   a2     KS = K S0, QS = Q S0 (MFMA, K and Q fragments loaded straight from global memory)
//   a3     K K^T and K Q^T (MFMA with K as the A operand, so lane (g, r) holds row r, columns
//          4g..4g+3), masked and decay-weighted into -G (strict ancestors) and C (path)
//   a4     U = sum_{m=0..d} (-G)^m R, the finite Neumann series with one term per tree level
//          (d = the tree's depth < 16), one MFMA product per term
//   a5     O = diag(P) QS + C U (MFMA)
// Operand layout changes between the MFMA result order (lane (g, r): rows 4g..4g+3 of column
// r) and the operand order (lane (g, r): row or column r at reduction indices 8g..8g+7, g < 2)
// use lane shuffles.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

// Values of 4 consecutive rows (result order) or 4 consecutive columns (row order) per lane,
// regrouped into 8 consecutive reduction indices for lanes g = 0, 1 (zero for g = 2, 3):
// lane (g, r) gathers from lanes (2g, r) and (2g + 1, r).
__device__ __forceinline__ void regroup8(const float (&x)[4], int lane, float (&v)[8]) {
    const int r = lane & 15, g = lane >> 4;
    const int src0 = ((2 * g) & 3) * 16 + r, src1 = ((2 * g + 1) & 3) * 16 + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a = __shfl(x[e], src0, 64);
        const float b = __shfl(x[e], src1, 64);
        v[e] = g < 2 ? a : 0.f;
        v[4 + e] = g < 2 ? b : 0.f;
    }
}

template <bool BF>
__global__ __launch_bounds__(64) void verify_small_kernel(VerifyArgs a) {
    using Op = Ops<BF>;
    using In = typename Op::In;
    using Sp = typename Op::Sp;
    constexpr int TILES = D / 16;
    const int gid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = gid % TILES;
    const int bh = gid / TILES;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
    const int col0 = tile * 16;
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;

    // ---- every load up front: the tree and gates (lane = node), K and Q fragments
    // (row lr), S0 fragments (column col0 + lr), V (result order)
    const int node = lane;
    const bool real = node < T;
    int par = real ? a.parent[static_cast<size_t>(b) * T + node] : -1;
    const float alpha = real ? a.alpha[sbase + static_cast<size_t>(node) * H] : 1.f;
    const float beta = real ? a.beta[sbase + static_cast<size_t>(node) * H] : 0.f;
    const bool rowok = lr < T;
    const size_t erow = base + static_cast<size_t>(rowok ? lr : 0) * rs + 8 * lg;
    In kf[4], qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = Op::template load_frag<In>(a.k, erow + 32 * ks, rowok);
        qf[ks] = Op::template load_frag<In>(a.q, erow + 32 * ks, rowok);
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

    // ---- prep: validation, then pointer jumping across lanes
    const bool badn = real && (par < -1 || par >= node);
    const unsigned long long badm = __ballot(badn);
    const int bad = badm ? (__ffsll(static_cast<unsigned long long>(badm))) : 0;  // 1 + first bad node
    if (bad) {
        const float qnan = __builtin_nanf("");
        for (int i = lg; i < T; i += 4) {
            a.O[base + static_cast<size_t>(i) * rs + col0 + lr] = qnan;
            a.U[base + static_cast<size_t>(i) * rs + col0 + lr] = qnan;
        }
        if (tile == 0 && real) a.ell[sbase + static_cast<size_t>(node) * H] = qnan;
        if (tile == 0 && h == 0) {
            if (a.tree_status && lane == 0) a.tree_status[b] = bad;
            if (real && a.depth) a.depth[static_cast<size_t>(b) * T + node] = 0;
            if (real && a.anc_mask) a.anc_mask[static_cast<size_t>(b) * T + node] = 0u;
        }
        return;
    }
    uint32_t mask = real ? (1u << node) : 0u;
    double ell = real ? log(static_cast<double>(alpha)) : 0.0;
    int jmp = real ? par : -1;
#pragma unroll
    for (int round = 0; round < 4; ++round) {  // 2^4 = 16 > any depth here
        const int src = jmp >= 0 ? jmp : lane;
        const uint32_t pm = __shfl(mask, src, 64);
        const double pl = __shfl(ell, src, 64);
        const int pj = __shfl(jmp, src, 64);
        if (jmp >= 0) {
            mask |= pm;
            ell += pl;
            jmp = pj;
        }
    }
    const float P = real ? static_cast<float>(exp(ell)) : 0.f;
    const int depth = real ? __popc(mask) - 1 : -1;
    const int dmax = wave_max(depth);
    if (tile == 0 && real) a.ell[sbase + static_cast<size_t>(node) * H] = static_cast<float>(ell);
    if (tile == 0 && h == 0) {
        if (a.tree_status && lane == 0) a.tree_status[b] = 0;
        if (real && a.depth) a.depth[static_cast<size_t>(b) * T + node] = depth;
        if (real && a.anc_mask) a.anc_mask[static_cast<size_t>(b) * T + node] = mask;
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
    float rhs[4], o0[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * lg + e;
        const float bi = __shfl(beta, i, 64), Pi = __shfl(P, i, 64);
        rhs[e] = i < T ? bi * (Op::raw_f32(vraw[e]) - Pi * ak[e]) : 0.f;
        o0[e] = i < T ? Pi * aq[e] : 0.f;
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
            float gv = 0.f, cv = 0.f;
            if ((mi >> j) & 1u) {
                const float gam = expf(static_cast<float>(li - lj));
                cv = gam * qk[e];
                if (i != j) gv = -bi * gam * kk[e];
            }
            gneg[e] = gv;
            cm[e] = cv;
        }
    }
    float gv8[8], cv8[8];
    regroup8(gneg, lane, gv8);  // A operand: row lr, reduction index = column j
    regroup8(cm, lane, cv8);
    const Sp gf = Op::split(gv8);
    const Sp cf = Op::split(cv8);

    // ---- a4: U = sum_{m=0..dmax} (-G)^m R; Z in result order, regrouped as a B operand
    float u[4], z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = z[e] = rhs[e];
    for (int m = 1; m <= dmax; ++m) {
        float zv[8];
        regroup8(z, lane, zv);
        f32x4 nz = {0.f, 0.f, 0.f, 0.f};
        nz = Op::mma(gf, Op::split(zv), nz);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = nz[e];
            u[e] += nz[e];
        }
    }
    // ---- a5: O = diag(P) QS + C U
    float uv[8];
    regroup8(u, lane, uv);
    f32x4 oc = {o0[0], o0[1], o0[2], o0[3]};
    oc = Op::mma(cf, Op::split(uv), oc);

    // ---- a6: outputs
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * lg + e;
        if (i < T) {
            a.U[base + static_cast<size_t>(i) * rs + col0 + lr] = u[e];
            a.O[base + static_cast<size_t>(i) * rs + col0 + lr] = oc[e];
        }
    }
}

hipError_t launch_verify_small(const VerifyArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * (D / 16))), block(64);
    if (a.bf16)
        hipLaunchKernelGGL(verify_small_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(verify_small_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace canopy
