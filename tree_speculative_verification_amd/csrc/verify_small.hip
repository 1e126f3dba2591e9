// Tree verification for trees of at most 16 nodes: one wave per (sequence, head, NCT 16-column
// tiles of the value columns), everything in registers, no LDS and no barrier. The same closed form as the
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
// between lanes. A workgroup holds NWV waves, each on its own NCT tiles of one head; with two
// tiles a wave computes the tree prep, the key and query fragments, the Gram tile and the path
// operands once for both, and the tiles' series chains interleave.
//
// The fused variant first commits the previous tree's accepted path into the wave's 128 x 16 NCT
// slice of the state ("Design decisions / What the commit kernel stores"): S = P_a S0 +
// sum_t w_t k_t u_t^T as fp32 MFMA products, four path positions per instruction, the key
// rows permuted so that the result lands in the B-operand placement of S0 that the
// projections read. The path is requested first, then its nodes' operands; the slice is
// written out as the new state and the verify runs from it without another pass over memory.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

// SIMDs of the GPU (256 CUs of 4), for the single-pass test of the launch width.
constexpr int kSmallSimds = 1024;

// Fused commit: one node's operands for the rank-update product. Lane (g, r) holds the node of
// its reduction index g and loads the key values at the rows R(t, r) = 32 (r % 4) + 8 (r / 4) + t
// of the 8 output tiles t (8 adjacent rows: one 16-byte load for bf16), and U at columns
// col0 + 16 ct + r of the wave's NCT column tiles. With A[r][g] = k[R(t, r)], the product's lane
// (g, r) receives rows R(t, 4g + e) = 32 e + 8 g + t: value t of the S0 fragment's slice ks = e.
template <bool BF, int NCT>
__device__ __forceinline__ void prev_operands(const PrevCommitArgs &c, size_t kbase, size_t krs,
                                              size_t ubase, size_t urs, int node, int lr,
                                              float (&ka)[8], float (&u)[NCT]) {
    const size_t ko = kbase + static_cast<size_t>(node) * krs + 32 * (lr & 3) + 8 * (lr >> 2);
    if constexpr (BF) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(c.k) + ko);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ka[2 * q] = __uint_as_float(ww[q] << 16);
            ka[2 * q + 1] = __uint_as_float(ww[q] & 0xFFFF0000u);
        }
    } else {
        const float4 f0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(c.k) + ko);
        const float4 f1 = *reinterpret_cast<const float4 *>(static_cast<const float *>(c.k) + ko + 4);
        ka[0] = f0.x; ka[1] = f0.y; ka[2] = f0.z; ka[3] = f0.w;
        ka[4] = f1.x; ka[5] = f1.y; ka[6] = f1.z; ka[7] = f1.w;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) u[ct] = c.U[ubase + static_cast<size_t>(node) * urs + 16 * ct];
}

template <bool BF, int NWV, bool FUSE, int NCT>
__global__ __launch_bounds__(64 * NWV) void verify_small_kernel(VerifyArgs a, PrevCommitArgs c) {
    using Op = Ops<BF>;
    using In = typename Op::In;
    using Sp = typename Op::Sp;
    constexpr int TILES = D / 16;
    constexpr int GROUPS = TILES / (NWV * NCT);  // workgroups per head
    const int gid = xcd_remap(blockIdx.x, gridDim.x);
    // The wave's NCT adjacent 16-column tiles start at `tile`.
    const int tile = ((gid % GROUPS) * NWV + static_cast<int>(threadIdx.x >> 6)) * NCT;
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

    // ---- fused commit, first request: the accepted path (lane = path position)
    int pm = 0, pnd = -1;
    if constexpr (FUSE) {
        pm = c.path_len[b];
        pnd = c.path[static_cast<size_t>(b) * c.T + min(lane, c.T - 1)];
    }

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
    // s0t[ct][t][ks] = S0[32ks + 8lg + t][col0 + 16ct + lr]: row t of the B fragment of reduction
    // slice ks for column tile ct, grouped by t so that each f32x4 is also the accumulator of the
    // fused commit's rank update for its 16 x 16 tile t (the key rows of that update are permuted
    // to land there)
    f32x4 s0t[NCT][8];  // per column tile ct: columns col0 + 16 ct + lr
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const float *S0p = a.S0 + static_cast<size_t>(bh) * D * D + col0 + 16 * ct + lr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) s0t[ct][e][ks] = S0p[(32 * ks + 8 * lg + e) * D];
    }
    typename Op::Raw vraw[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vraw[ct][e] = Op::load_raw(a.v, base + static_cast<size_t>(min(4 * lg + e, T - 1)) * rs + col0 + 16 * ct + lr);

    // ---- fused commit, second request: the path nodes' parents and gates (lane = position)
    // and the operands of positions 0..3 (all that a short accepted path has). Positions past
    // the path take node 0 (a real node of any previous tree), whose finite values meet a zero
    // weight.
    int ppar = -1, pmv = 0;
    SeqLen psl{1, false};
    float pal = 1.f, ka[8], ub[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) ub[ct] = 0.f;
    const size_t pkbase = FUSE ? qk_base(b, h, H, a.HK, c.T) : 0;
    const size_t pubase = (static_cast<size_t>(b) * (FUSE ? c.T : 0) * H + h) * D + col0 + lr;
    if constexpr (FUSE) {
        psl = seq_len(c.tree_len, b, c.T);
        const bool plenok = !psl.bad && pm >= 0 && pm <= psl.n;
        pmv = plenok ? pm : 0;
        const int nsel = min(max(pnd, 0), c.T - 1);
        ppar = c.parent[static_cast<size_t>(b) * c.T + nsel];
        pal = c.alpha[(static_cast<size_t>(b) * c.T + nsel) * H + h];
        const int sn = __shfl(nsel, lg, 64);
        prev_operands<BF, NCT>(c, pkbase, qkrs, pubase, rs, lg < pmv ? sn : 0, lr, ka, ub);
    }

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

    // ---- fused commit: path check (each node a child of the one before, inside the previous
    // tree), suffix sums of log2 alpha in fp64, w_t = 2^(suffix after t), P_a = 2^(total), the
    // rank update on MFMA, then the new state in place of the S0 fragment
    if constexpr (FUSE) {
        const bool inp = lane < pmv;
        const int ndc = min(max(pnd, 0), c.T - 1);
        const int up = __shfl_up(pnd, 1, 64);
        const int prevn = lane == 0 ? -1 : up;
        const bool ok = !inp || (pnd >= 0 && pnd < psl.n && ppar == prevn);
        const unsigned long long pbad = __ballot(!ok);
        const bool plenok = !psl.bad && pm >= 0 && pm <= psl.n;
        // -1 for a length out of range, else 1 + the first bad position
        const int pst = !plenok ? -1 : (pbad ? __ffsll(static_cast<unsigned long long>(pbad)) : 0);
        const double la = inp ? static_cast<double>(__builtin_amdgcn_logf(pal)) : 0.0;
        double sv = la;  // lanes at or past the path hold 0
        if (pmv <= 4) {
#pragma unroll
            for (int off = 1; off < 4; off <<= 1) {
                const double tv = __shfl_down(sv, off, 64);
                sv = lane + off < 64 ? sv + tv : sv;
            }
        } else {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const double tv = __shfl_down(sv, off, 64);
                sv = lane + off < 64 ? sv + tv : sv;
            }
        }
        const float Pa = __builtin_amdgcn_exp2f(static_cast<float>(__shfl(sv, 0, 64)));
        const float w = __builtin_amdgcn_exp2f(static_cast<float>(sv - la));  // decay after t
        // S_new = P_a S0 + sum_t w_t k_t u_t^T, accumulated in place of the S0 fragment
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int t = 0; t < 8; ++t) s0t[ct][t] = Pa * s0t[ct][t];
        {
            const float wv = __shfl(w, lg, 64);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float bu = lg < pmv ? wv * ub[ct] : 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) s0t[ct][t] = mfma_f32(ka[t], bu, s0t[ct][t]);
            }
        }
        for (int p0 = 4; p0 < pmv; p0 += 4) {  // paths longer than 4 nodes
            const int pos = min(p0 + lg, 63);
            const int sn = __shfl(ndc, pos, 64);
            float kx[8], ux[NCT];
            prev_operands<BF, NCT>(c, pkbase, qkrs, pubase, rs, p0 + lg < pmv ? sn : 0, lr, kx, ux);
            const float wv = __shfl(w, pos, 64);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float bu = p0 + lg < pmv ? wv * ux[ct] : 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) s0t[ct][t] = mfma_f32(kx[t], bu, s0t[ct][t]);
            }
        }
        const float qnan = __builtin_nanf("");
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) s0t[ct][t][ks] = pst != 0 ? qnan : s0t[ct][t][ks];
        // The new state as ordinary stores: each lane group writes 64-byte segments of state
        // rows, which streaming stores made slower (B = 16, H = 32, T = 16: 16.9 -> 16.3 us per
        // step with one layer, 27.7 -> 26.3 us per layer with 16 layers run in turn, so that each
        // layer's state has left the caches before its next step).
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float *Sn = c.S_new + static_cast<size_t>(bh) * D * D + col0 + 16 * ct + lr;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) Sn[static_cast<size_t>(32 * ks + 8 * lg + e) * D] = s0t[ct][e][ks];
        }
        if (c.path_status && tile == 0 && h == 0 && lane == 0) c.path_status[b] = pst;
    }

    // ---- a2: projections; result order: lane (lg, lr) holds rows 4lg+e of column lr
    float rhs[NCT][4];
    f32x4 o0[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        Sp s0f[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const float v[8] = {s0t[ct][0][ks], s0t[ct][1][ks], s0t[ct][2][ks], s0t[ct][3][ks],
                                s0t[ct][4][ks], s0t[ct][5][ks], s0t[ct][6][ks], s0t[ct][7][ks]};
            s0f[ks] = Op::split(v);
        }
        f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            ak = Op::mma(kf[ks], s0f[ks], ak);
            aq = Op::mma(qf[ks], s0f[ks], aq);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * lg + e;
            const float bi = __shfl(beta, i, 64), Pi = __shfl(P, i, 64);
            const float r = bi * (Op::raw_f32(vraw[ct][e]) - Pi * ak[e]), o = Pi * aq[e];
            rhs[ct][e] = i < Tb ? r : 0.f;
            o0[ct][e] = i < Tb ? o : 0.f;
        }
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
    // (the column tiles' chains are independent and interleave)
    float u[NCT][4], z[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) u[ct][e] = z[ct][e] = rhs[ct][e];
    for (int m = 1; m <= dmax; ++m) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 nz = {0.f, 0.f, 0.f, 0.f};
            nz = Op::mma16(gf, Op::split4(z[ct]), nz);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[ct][e] = nz[e];
                u[ct][e] += nz[e];
            }
        }
    }
    // ---- a5: O = diag(P) QS + C U, then a6: outputs (NaN for a malformed tree)
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const f32x4 oc = Op::mma16(cf, Op::split4(u[ct]), o0[ct]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * lg + e;
            if (i < Tb) {
                const size_t o = base + static_cast<size_t>(i) * rs + col0 + 16 * ct + lr;
                a.U[o] = bad ? qnan : u[ct][e];
                // O streams past the caches for the verify alone (4% faster at B = 16); the
                // one-launch step stores it like the state (equal with one layer, 1.3% faster
                // with 16 layers run in turn)
                if constexpr (FUSE)
                    a.O[o] = bad ? qnan : oc[e];
                else
                    store_nt(a.O + o, bad ? qnan : oc[e]);
            }
        }
    }
}

template <bool BF, bool FUSE>
static void launch_small_nwv(const VerifyArgs &a, const PrevCommitArgs &c, int nwv, hipStream_t stream) {
    const unsigned heads = static_cast<unsigned>(a.B * a.H);
    switch (nwv) {
        case 1:
            hipLaunchKernelGGL((verify_small_kernel<BF, 1, FUSE, 1>), dim3(heads * 8), dim3(64), 0, stream, a, c);
            break;
        case 2:
            hipLaunchKernelGGL((verify_small_kernel<BF, 2, FUSE, 1>), dim3(heads * 4), dim3(128), 0, stream, a, c);
            break;
        case 4:
            hipLaunchKernelGGL((verify_small_kernel<BF, 4, FUSE, 1>), dim3(heads * 2), dim3(256), 0, stream, a, c);
            break;
        case 8:
            hipLaunchKernelGGL((verify_small_kernel<BF, 8, FUSE, 1>), dim3(heads), dim3(512), 0, stream, a, c);
            break;
        default:  // 16: one wave per workgroup, two column tiles (32 value columns) per wave
            hipLaunchKernelGGL((verify_small_kernel<BF, 1, FUSE, 2>), dim3(heads * 4), dim3(64), 0, stream, a, c);
            break;
    }
}

// Width for waves = 0. Once single-tile waves fill a whole pass of the GPU or more (3 waves per
// SIMD for the one-launch step, whose registers allow no more; 4 for the verify alone), two
// column tiles per wave keep every wave in one pass, give each two independent chains and load
// each head's keys, queries and tree half as often (B = 16, H = 32, T = 16: verify 11.5 ->
// 10.6 us, the one-launch step 18.3 -> 18.0 us).
static int small_auto_width(const VerifyArgs &a, bool fuse) {
    if (!a.bf16) return 1;  // fp32 inputs: two tiles leave one wave per SIMD in the one-launch step
    const long long waves1 = static_cast<long long>(a.B) * a.H * (D / 16);
    const long long slots = static_cast<long long>(kSmallSimds) * (fuse ? 3 : 4);
    return waves1 >= slots ? 16 : 1;
}

// waves: waves per workgroup (1, 2, 4 or 8) each on 16 value columns, 16 for single-wave
// workgroups on 32 columns, 0 to choose.
hipError_t launch_verify_small(const VerifyArgs &a, int waves, hipStream_t stream) {
    const int nwv = waves == 0 ? small_auto_width(a, false) : waves;
    const PrevCommitArgs none{};
    if (a.bf16)
        launch_small_nwv<true, false>(a, none, nwv, stream);
    else
        launch_small_nwv<false, false>(a, none, nwv, stream);
    return hipGetLastError();
}

// The commit of the previous tree's path (c.T <= 64: one path position per lane) fused in front
// of the verify of a tree of at most 16 nodes; a.S0 is the state before the commit.
hipError_t launch_commit_verify_small(const VerifyArgs &a, const PrevCommitArgs &c, int waves,
                                      hipStream_t stream) {
    const int nwv = waves == 0 ? small_auto_width(a, true) : waves;
    if (a.bf16)
        launch_small_nwv<true, true>(a, c, nwv, stream);
    else
        launch_small_nwv<false, true>(a, c, nwv, stream);
    return hipGetLastError();
}

}  // namespace canopy
