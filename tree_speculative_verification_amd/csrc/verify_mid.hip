// Tree verification for trees of 17 to 64 nodes ("The tree closed form" on the canopy project
// page). One workgroup per (sequence, head, NCT x 16 value columns) with one wave per 16-node
// sub-block: wave p owns nodes 16p .. 16p+15.
//   prep   every wave runs the whole tree's pointer jumping over its 64 lanes (lane = node,
//          64-bit ancestor masks, fp64 path sums of log2 alpha) and keeps the per-node results
//          in a private LDS table, read back as vectors wherever a tile needs them
//   stage  the keys (each wave its own 16 rows) and the workgroup's S0 columns, transposed so
//          that each column's 128 values are one row and split into bf16 hi + lo, go to LDS
//          once per workgroup
//   a2     K_p S0 and Q_p S0 for the wave's rows (MFMA); R_p and diag(P) Q_p S0
//   a3     the wave's row of Gram tiles, G_pc and C_pc for c <= p, with K_c as the A operand
//          so that each tile lands in the A placement of a 16-long MFMA reduction
//   a4     forward substitution over the sub-blocks (the blocked form of "Design decisions /
//          Two solve strategies"): U_p = (I + G_pp)^-1 (R_p - sum_{c<p} G_pc U_c). The
//          diagonal inverse is the finite Neumann series of N = -G_pp, taken as the product
//          (I + N)(I + N^2)(I + N^4)(I + N^8) truncated at the sub-block's own depth (the
//          squaring form of "The tree closed form") and multiplied out into one matrix before
//          the right-hand side is known, so the sequential part is one product per tile.
//          With the Neumann solver the whole system instead runs the series
//          U = sum_{m<=d} (-G)^m R, one exchange of the 16 x 16 terms per tree level.
//   a5     O_p = diag(P) Q_p S0 + sum_{c<=p} C_pc U_c, accumulated as the U_c arrive
// Node-by-column tiles (R, U, the series terms) sit with rows 4g..4g+3 of column r in lane
// (g, r), which is both the result placement of an MFMA and the B placement of the 16-long
// reduction, so no product needs lane shuffles. Those 16-long products take fp32 operands
// straight from the VALU on fp32 MFMA (exact products, no bf16 splitting). The NCT column
// tiles of a workgroup share the Gram tiles and the inverse powers and run their solves as
// independent MFMA chains. Decay ratios are powers of two of fp64 differences of log2 sums
// (v_exp_f32), so no cancellation of long path sums enters them.
//
// The fused variant (FUSE) first commits the previous tree's accepted path into the S0 values
// each thread holds ("Design decisions / What the commit kernel stores"): S = P_a S0 +
// sum_t w_t k_t u_t^T on the VALU, four path positions per round of requests (each position's
// 8 key values of the thread's row chunk and the U entry of its column), then writes the new
// state and stages it for the verify in place of S0. Only for shapes whose threads hold at
// most 2 (column, row chunk) pairs, so that a round's operands fit in registers.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

template <bool BF, int NSB, int NCT>
struct MidSmem {
    static constexpr int ROWB = Ops<BF>::ROWB;
    static constexpr int S0B = 16 * NCT * 512;  // S0 columns: fp32 rows, or bf16 hi + lo rows
    static constexpr int XB = 2 * NSB * NCT * 64 * 16;
    uint8_t k[NSB * 16 * ROWB];
    union {
        uint8_t s0[S0B];
        float4 x[2][NSB][NCT][64];
    } u;
    double lam[NSB][64];  // log2 of the cumulative decay P
    unsigned long long mask[NSB][64];
    float beta[NSB][64];
    float P[NSB][64];
    int ready[NSB];  // forward substitution: U_s is in x[0][s]
};

// Fused commit: for path positions first .. first+CG-1 (node 0 past the path, whose finite
// values meet a zero weight), the key values at rows 8kc .. 8kc+7 and the U entry at column cc
// of each (column, row chunk) pair m of this thread.
template <bool BF, int PPT, int CG>
__device__ __forceinline__ void mid_prev_group(const PrevCommitArgs &c, size_t kbase, size_t krs,
                                               size_t ubase, size_t urs, int nsel, int first, int pmv,
                                               const int (&kc)[PPT], const int (&cc)[PPT],
                                               float (&ck)[CG][PPT][8], float (&cu)[CG][PPT]) {
#pragma unroll
    for (int tt = 0; tt < CG; ++tt) {
        const int t = first + tt;
        const int nr = __builtin_amdgcn_readlane(nsel, min(t, 63));
        const int node = t < pmv ? nr : 0;
        const size_t ko = kbase + static_cast<size_t>(node) * krs;
        const size_t uo = ubase + static_cast<size_t>(node) * urs;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            if constexpr (BF) {
                const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(c.k) + ko + 8 * kc[m]);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    ck[tt][m][2 * q] = __uint_as_float(ww[q] << 16);
                    ck[tt][m][2 * q + 1] = __uint_as_float(ww[q] & 0xFFFF0000u);
                }
            } else {
                const float4 f0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(c.k) + ko + 8 * kc[m]);
                const float4 f1 = *reinterpret_cast<const float4 *>(static_cast<const float *>(c.k) + ko + 8 * kc[m] + 4);
                ck[tt][m][0] = f0.x; ck[tt][m][1] = f0.y; ck[tt][m][2] = f0.z; ck[tt][m][3] = f0.w;
                ck[tt][m][4] = f1.x; ck[tt][m][5] = f1.y; ck[tt][m][6] = f1.z; ck[tt][m][7] = f1.w;
            }
            cu[tt][m] = c.U[uo + cc[m]];
        }
    }
}

template <bool BF, int NSB, int NCT, bool FUSE>
__global__ __launch_bounds__(64 * NSB) void verify_mid_kernel(VerifyArgs a, PrevCommitArgs c) {
    using Op = Ops<BF>;
    using In = typename Op::In;
    using Sp = typename Op::Sp;
    using Smem = MidSmem<BF, NSB, NCT>;
    constexpr int NT = 64 * NSB;
    constexpr int GROUPS = D / (16 * NCT);  // workgroups per head
    __shared__ __align__(16) Smem sm;

    const int gid = xcd_remap(blockIdx.x, gridDim.x);
    const int grp = gid % GROUPS;
    const int bh = gid / GROUPS;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int p = tid >> 6;  // this wave's sub-block
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int colw = grp * 16 * NCT;  // the workgroup's first value column
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;
    const size_t qkrs = static_cast<size_t>(a.HK) * D;
    const size_t qkbase = qk_base(b, h, H, a.HK, T);
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;  // this sequence's node count
    const bool writer = grp == 0 && p == 0;  // this head's wave for the per-node outputs

    // ---- fused commit, first request: the accepted path (lane = path position)
    int pm = 0, pnd = -1;
    if constexpr (FUSE) {
        pm = c.path_len[b];
        pnd = c.path[static_cast<size_t>(b) * c.T + min(lane, c.T - 1)];
    }

    // ---- every load up front, unconditional (rows and nodes past T read row or node T-1;
    // rows and nodes past Tb are padding, dropped by selects later): tree and gates (lane = node), the wave's own K and Q rows, the
    // thread's share of the S0 columns (column c, reduction indices 8kc .. 8kc+7) and the
    // wave's V rows.
    const int node = lane;
    const bool real = node < Tb;
    const int nodec = min(node, T - 1);
    const int par_in = a.parent[static_cast<size_t>(b) * T + nodec];
    const float alpha_in = a.alpha[sbase + static_cast<size_t>(nodec) * H];
    const float beta_in = a.beta[sbase + static_cast<size_t>(nodec) * H];
    In kp[4], qp[4];
    {
        const size_t er = qkbase + static_cast<size_t>(min(16 * p + lr, T - 1)) * qkrs + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kp[ks] = Op::template load_frag<In>(a.k, er + 32 * ks, true);
            qp[ks] = Op::template load_frag<In>(a.q, er + 32 * ks, true);
        }
    }
    constexpr int NPAIR = 16 * NCT * 16;                  // (column, 8-index chunk) pairs
    constexpr int PPT = (NPAIR + NT - 1) / NT;
    float s0v[PPT][8];
    {
        const float *S0p = a.S0 + static_cast<size_t>(bh) * D * D + colw;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            const int x = min(tid + m * NT, NPAIR - 1);
            const int c = x % (16 * NCT), kc = x / (16 * NCT);
#pragma unroll
            for (int e = 0; e < 8; ++e) s0v[m][e] = S0p[(8 * kc + e) * D + c];
        }
    }
    typename Op::Raw vraw[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vraw[ct][e] = Op::load_raw(a.v, base + static_cast<size_t>(min(16 * p + 4 * lg + e, T - 1)) * rs +
                                                colw + 16 * ct + lr);

    // ---- fused commit, second request: the path nodes' parents and gates (lane = position) and
    // the operands of path positions 0..3 for this thread's (column, row chunk) pairs
    constexpr int CG = 4;
    constexpr int CGF = FUSE ? CG : 1;
    int pmv = 0, nsel = 0, ppar = -1;
    SeqLen psl{1, false};
    float pal = 1.f, ck[CGF][PPT][8], cu[CGF][PPT];
    int pkc[PPT], pcc[PPT];
#pragma unroll
    for (int m = 0; m < PPT; ++m) {
        const int x = min(tid + m * NT, NPAIR - 1);
        pcc[m] = x % (16 * NCT);
        pkc[m] = x / (16 * NCT);
    }
    const size_t pkbase = FUSE ? qk_base(b, h, H, a.HK, c.T) : 0;
    const size_t pubase = (static_cast<size_t>(b) * (FUSE ? c.T : 0) * H + h) * D + colw;
    if constexpr (FUSE) {
        psl = seq_len(c.tree_len, b, c.T);
        const bool plenok = !psl.bad && pm >= 0 && pm <= psl.n;
        pmv = plenok ? pm : 0;
        nsel = min(max(pnd, 0), c.T - 1);
        ppar = c.parent[static_cast<size_t>(b) * c.T + nsel];
        pal = c.alpha[(static_cast<size_t>(b) * c.T + nsel) * H + h];
        mid_prev_group<BF, PPT, CGF>(c, pkbase, qkrs, pubase, rs, nsel, 0, pmv, pkc, pcc, ck, cu);
    }

    // ---- prep over the wave's lanes. A malformed tree is computed through like a forest (bad
    // parents read as -1) and replaced by NaN at the stores.
    const bool badn = real && (par_in < -1 || par_in >= node);
    const unsigned long long badm = __ballot(badn);
    // -1 for a length out of range, else 1 + the first bad node
    const int bad = sl.bad ? -1 : (badm ? __ffsll(static_cast<unsigned long long>(badm)) : 0);
    const float beta = real ? beta_in : 0.f;
    // log2 alpha in fp32 (its error is relative to each term); the path sums in fp64
    unsigned long long mask = real ? (1ull << node) : 0ull;
    double lam = real ? static_cast<double>(__builtin_amdgcn_logf(alpha_in)) : 0.0;
    int jmp = (real && !badn) ? par_in : -1;
    // After round r every jump pointer is 2^(r+1) levels up; depth < 64 ends it in 6.
    for (int round = 0; round < 6 && __any(jmp >= 0); ++round) {
        const int src = jmp >= 0 ? jmp : lane;
        const unsigned long long pm = __shfl(mask, src, 64);
        const double pl = __shfl(lam, src, 64);
        const int pj = __shfl(jmp, src, 64);
        const bool up = jmp >= 0;
        mask = up ? (mask | pm) : mask;
        lam = up ? lam + pl : lam;
        jmp = up ? pj : jmp;
    }
    const float ellf = static_cast<float>(lam * 0.69314718055994530942);  // l = ln P
    const float P = real ? __builtin_amdgcn_exp2f(static_cast<float>(lam)) : 0.f;
    const int depth = real ? __popcll(mask) - 1 : -1;
    if (writer && real) a.ell[sbase + static_cast<size_t>(node) * H] = bad ? __builtin_nanf("") : ellf;
    if (writer && h == 0) {
        const int W = (T + 31) >> 5;
        if (a.tree_status && lane == 0) a.tree_status[b] = bad;
        if (real && a.depth) a.depth[static_cast<size_t>(b) * T + node] = bad ? 0 : depth;
        if (real && a.anc_mask) {
            uint32_t *mrow = a.anc_mask + (static_cast<size_t>(b) * T + node) * W;
            mrow[0] = bad ? 0u : static_cast<uint32_t>(mask);
            if (W > 1) mrow[1] = bad ? 0u : static_cast<uint32_t>(mask >> 32);
        }
    }
    // Depth inside this wave's sub-block (ancestors within it), which bounds the nilpotency
    // of its diagonal block, and the tree's depth; both by ballots on their bits.
    const int sub = lane >> 4;
    const int dloc = real ? __popcll(mask & (0xFFFFull << (16 * sub))) - 1 : -1;
    int dp = 0;
#pragma unroll
    for (int bit = 3; bit >= 0; --bit)
        if (__any(sub == p && dloc >= (dp | (1 << bit)))) dp |= 1 << bit;
    int dtree = 0;
#pragma unroll
    for (int bit = 5; bit >= 0; --bit)
        if (__any(depth >= (dtree | (1 << bit)))) dtree |= 1 << bit;

    // ---- fused commit: path check (each node a child of the one before, inside the previous
    // tree), suffix sums of log2 alpha in fp64, w_t = 2^(suffix after t), P_a = 2^(total); the
    // rank update of this thread's S0 values, written out as the new state
    if constexpr (FUSE) {
        const bool inp = lane < pmv;
        const int up = __shfl_up(pnd, 1, 64);
        const int prevn = lane == 0 ? -1 : up;
        const bool ok = !inp || (pnd >= 0 && pnd < psl.n && ppar == prevn);
        const unsigned long long pbad = __ballot(!ok);
        const bool plenok = !psl.bad && pm >= 0 && pm <= psl.n;
        // -1 for a length out of range, else 1 + the first bad position
        const int pst = !plenok ? -1 : (pbad ? __ffsll(static_cast<unsigned long long>(pbad)) : 0);
        const double la = inp ? static_cast<double>(__builtin_amdgcn_logf(pal)) : 0.0;
        double sv = la;  // lanes at or past the path hold 0
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double tv = __shfl_down(sv, off, 64);
            sv = lane + off < 64 ? sv + tv : sv;
        }
        const float Pa = __builtin_amdgcn_exp2f(static_cast<float>(__shfl(sv, 0, 64)));
        const float w = __builtin_amdgcn_exp2f(static_cast<float>(sv - la));  // decay after t
        float acc[PPT][8];
#pragma unroll
        for (int m = 0; m < PPT; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
        for (int g0 = 0; g0 < max(pmv, 1); g0 += CG) {
            if (g0 > 0) mid_prev_group<BF, PPT, CGF>(c, pkbase, qkrs, pubase, rs, nsel, g0, pmv, pkc, pcc, ck, cu);
#pragma unroll
            for (int tt = 0; tt < CG; ++tt) {
                const int t = g0 + tt;
                const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(t, 63)));
                const float wt = t < pmv ? wr : 0.f;
#pragma unroll
                for (int m = 0; m < PPT; ++m) {
                    const float wu = wt * cu[tt][m];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[m][e] += wu * ck[tt][m][e];
                }
            }
        }
        const float qnan = __builtin_nanf("");
        float *Sn = c.S_new + static_cast<size_t>(bh) * D * D + colw;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s0v[m][e] = pst != 0 ? qnan : Pa * s0v[m][e] + acc[m][e];
            if (tid + m * NT < NPAIR) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    store_nt(Sn + static_cast<size_t>(8 * pkc[m] + e) * D + pcc[m], s0v[m][e]);
            }
        }
        if (c.path_status && grp == 0 && h == 0 && tid == 0) c.path_status[b] = pst;
    }

    // ---- stage: the per-node table (private to the wave), this wave's keys, the S0 columns
    sm.lam[p][lane] = lam;
    sm.mask[p][lane] = mask;
    sm.beta[p][lane] = beta;
    sm.P[p][lane] = P;
    if (tid < NSB) sm.ready[tid] = 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Op::lds_put(sm.k, 16 * p + lr, 4 * ks + lg, kp[ks]);
#pragma unroll
    for (int m = 0; m < PPT; ++m) {
        const int x = tid + m * NT;
        if (x < NPAIR) {
            const int c = x % (16 * NCT), kc = x / (16 * NCT);
            if constexpr (BF) {
                const Sp sp = Op::split(s0v[m]);
                In hi, lo;
                hi.x = sp.hi;
                lo.x = sp.lo;
                Op::lds_put(sm.u.s0, c, kc, hi);
                Op::lds_put(sm.u.s0 + 16 * NCT * 256, c, kc, lo);
            } else {
                In f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f.x[e] = s0v[m][e];
                Op::lds_put(sm.u.s0, c, kc, f);
            }
        }
    }
    __syncthreads();

    // ---- a2: projections of the wave's rows; result order (rows 16p + 4lg + e, column lr)
    float rhs[NCT][4];
    f32x4 oacc[NCT];
    {
        const float4 b4 = *reinterpret_cast<const float4 *>(&sm.beta[p][16 * p + 4 * lg]);
        const float4 p4 = *reinterpret_cast<const float4 *>(&sm.P[p][16 * p + 4 * lg]);
        const float bi[4] = {b4.x, b4.y, b4.z, b4.w}, Pi[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Sp sf;
                if constexpr (BF) {
                    sf.hi = Op::lds_frag(sm.u.s0, 16 * ct + lr, 4 * ks + lg).x;
                    sf.lo = Op::lds_frag(sm.u.s0 + 16 * NCT * 256, 16 * ct + lr, 4 * ks + lg).x;
                } else {
                    sf = Op::lds_frag(sm.u.s0, 16 * ct + lr, 4 * ks + lg);
                }
                ak = Op::mma(kp[ks], sf, ak);
                aq = Op::mma(qp[ks], sf, aq);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * p + 4 * lg + e;  // beta and P are 0 past Tb
                const float r = bi[e] * (Op::raw_f32(vraw[ct][e]) - Pi[e] * ak[e]), o = Pi[e] * aq[e];
                rhs[ct][e] = i < Tb ? r : 0.f;
                oacc[ct][e] = i < Tb ? o : 0.f;
            }
        }
    }
    __syncthreads();  // every wave is done with the S0 staging, which the solve overwrites

    // ---- a3: the wave's Gram row. Tile (p, c): lane (lg, lr) holds row i = 16p + lr and
    // columns j = 16c + 4lg + e of K K^T and of Q K^T; masked and weighted into -G (strict
    // ancestors) and C (path). The diagonal tile also in the transposed placement (row
    // 16p + 4lg + e, column 16p + lr), which the squaring products need.
    float gn[NSB][4], cn[NSB][4];
    float nA[4], nB[4], cdiag[4];
    {
        const int i = 16 * p + lr;
        const unsigned long long mi = sm.mask[p][i];
        const double li = sm.lam[p][i];
        const float bi = sm.beta[p][i];
#pragma unroll
        for (int c = 0; c < NSB; ++c) {
            if (c > p) continue;
            f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const In kc = Op::lds_frag(sm.k, 16 * c + lr, 4 * ks + lg);
                kk = Op::mma(kc, kp[ks], kk);
                qk = Op::mma(kc, qp[ks], qk);
            }
            const int j0 = 16 * c + 4 * lg;
            const double2 l01 = *reinterpret_cast<const double2 *>(&sm.lam[p][j0]);
            const double2 l23 = *reinterpret_cast<const double2 *>(&sm.lam[p][j0 + 2]);
            const double lj[4] = {l01.x, l01.y, l23.x, l23.y};
            const uint32_t mbits = static_cast<uint32_t>(mi >> j0);  // bit e: j0 + e on path(i)
            float g[4], cm[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // Off the path the exponent may overflow; the selects drop those entries.
                const float gam = __builtin_amdgcn_exp2f(static_cast<float>(li - lj[e]));
                const bool onpath = (mbits >> e) & 1u;
                cm[e] = onpath ? gam * qk[e] : 0.f;
                g[e] = (onpath && i != j0 + e) ? -bi * gam * kk[e] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gn[c][e] = g[e];
                cn[c][e] = cm[e];
            }
            if (c == p) {
                // transposed placement: row i2 = j, column j2 = i
                const ulonglong2 m01 = *reinterpret_cast<const ulonglong2 *>(&sm.mask[p][j0]);
                const ulonglong2 m23 = *reinterpret_cast<const ulonglong2 *>(&sm.mask[p][j0 + 2]);
                const unsigned long long mj[4] = {m01.x, m01.y, m23.x, m23.y};
                const float4 bj4 = *reinterpret_cast<const float4 *>(&sm.beta[p][j0]);
                const float bj[4] = {bj4.x, bj4.y, bj4.z, bj4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = j0 + e;
                    const bool on2 = (mj[e] >> i) & 1ull;
                    const float gam2 = __builtin_amdgcn_exp2f(static_cast<float>(lj[e] - li));
                    nB[e] = (on2 && i != j) ? -bj[e] * gam2 * kk[e] : 0.f;
                    nA[e] = g[e];
                    cdiag[e] = cm[e];
                }
            }
        }
    }

    const float qnan = __builtin_nanf("");
    float u[NCT][4];
    bool lost = false;  // a result this wave waited for never came (or came from a lost wait)
    if (a.solver != CANOPY_SOLVE_NEUMANN) {
        // ---- a4, forward substitution. The diagonal inverse (I + G_pp)^-1 in the A placement,
        // as the product of the ceil(log2(dp + 1)) factors (I + N^(2^s)), N = -G_pp: each power
        // is squared in both placements ((X^2)^T = X^T X^T lands in the A placement), and with
        // Z = X Y, Z in the A placement is the product of Y's B placement and X's A placement.
        // This runs before the right-hand side is final, so the sequential part of the solve
        // is one product per incoming tile and one for the inverse.
        int nf = 0;
        while ((1 << nf) <= dp) ++nf;
        float minv[4];
        {
            float xa[4], xb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xa[e] = nA[e];
                xb[e] = nB[e];
                minv[e] = (lr == 4 * lg + e ? 1.f : 0.f) + nA[e];  // I + N
            }
#pragma unroll
            for (int s = 1; s < 4; ++s) {
                if (s >= nf) break;
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
        // Wave p takes U_s (s < p) as soon as wave s publishes it and folds it into its
        // right-hand side; then it solves and publishes its own tile, and only then forms its
        // read-out. Point-to-point waits: a wave still forming Gram tiles holds up only the
        // waves that need its result.
#pragma unroll
        for (int s = 0; s < NSB; ++s) {
            if (s >= p) break;
            lost |= wait_flag(&sm.ready[s], a.wait_bound) != 1;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float4 t = sm.u.x[0][s][ct][lane];
                const float tv[4] = {t.x, t.y, t.z, t.w};
                const f32x4 r = mma16f(gn[s], tv, f32x4{rhs[ct][0], rhs[ct][1], rhs[ct][2], rhs[ct][3]});
#pragma unroll
                for (int e = 0; e < 4; ++e) rhs[ct][e] = r[e];
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 y = mma16f(minv, rhs[ct], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) u[ct][e] = y[e];
            sm.u.x[0][p][ct][lane] = make_float4(u[ct][0], u[ct][1], u[ct][2], u[ct][3]);
        }
        __hip_atomic_store(&sm.ready[p], lost ? 2 : 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            oacc[ct] = mma16f(cdiag, u[ct], oacc[ct]);
#pragma unroll
            for (int s = 0; s < NSB; ++s) {
                if (s >= p) break;
                const float4 t = sm.u.x[0][s][ct][lane];
                const float tv[4] = {t.x, t.y, t.z, t.w};
                oacc[ct] = mma16f(cn[s], tv, oacc[ct]);
            }
        }
    } else {
        // ---- a4, Neumann series over the whole system: Z <- -G Z, U <- U + Z for each tree
        // level; the new term of sub-block p is sum_{c<=p} (-G_pc) Z_c.
        float z[NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) u[ct][e] = z[ct][e] = rhs[ct][e];
        for (int m = 1; m <= dtree; ++m) {
            const int buf = m & 1;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                sm.u.x[buf][p][ct][lane] = make_float4(z[ct][0], z[ct][1], z[ct][2], z[ct][3]);
            __syncthreads();
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 nz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NSB; ++c) {
                    if (c > p) continue;
                    const float4 t = sm.u.x[buf][c][ct][lane];
                    const float tv[4] = {t.x, t.y, t.z, t.w};
                    nz = mma16f(gn[c], tv, nz);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[ct][e] = nz[e];
                    u[ct][e] += nz[e];
                }
            }
        }
        // ---- a5 for the Neumann form: every U_c, then C U for the wave's rows
        __syncthreads();  // the last round's reads of the term buffers are done
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            sm.u.x[0][p][ct][lane] = make_float4(u[ct][0], u[ct][1], u[ct][2], u[ct][3]);
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int c = 0; c < NSB; ++c) {
                if (c > p) continue;
                const float4 t = sm.u.x[0][c][ct][lane];
                const float tv[4] = {t.x, t.y, t.z, t.w};
                oacc[ct] = mma16f(cn[c], tv, oacc[ct]);
            }
        }
    }

    // ---- a6: outputs (NaN for a malformed tree and for rows computed from a lost hand-off)
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
}

// The fused variant exists only where each thread holds at most 2 (column, row chunk) pairs.
template <bool BF, int NSB, int NCT, bool FUSE>
static void launch_mid_one(const VerifyArgs &a, const PrevCommitArgs &c, hipStream_t stream) {
    if constexpr (!FUSE || 4 * NCT <= 2 * NSB) {
        const unsigned heads = static_cast<unsigned>(a.B * a.H);
        hipLaunchKernelGGL((verify_mid_kernel<BF, NSB, NCT, FUSE>), dim3(heads * (8 / NCT)), dim3(64 * NSB), 0,
                           stream, a, c);
    }
}

template <bool BF, int NSB, bool FUSE>
static void launch_mid_nct(const VerifyArgs &a, const PrevCommitArgs &c, int nct, hipStream_t stream) {
    switch (nct) {
        case 1: launch_mid_one<BF, NSB, 1, FUSE>(a, c, stream); break;
        case 2: launch_mid_one<BF, NSB, 2, FUSE>(a, c, stream); break;
        default: launch_mid_one<BF, NSB, 4, FUSE>(a, c, stream); break;
    }
}

template <bool BF, bool FUSE>
static void launch_mid_dtype(const VerifyArgs &a, const PrevCommitArgs &c, int nct, hipStream_t stream) {
    switch ((a.T + 15) / 16) {
        case 2: launch_mid_nct<BF, 2, FUSE>(a, c, nct, stream); break;
        case 3: launch_mid_nct<BF, 3, FUSE>(a, c, nct, stream); break;
        default: launch_mid_nct<BF, 4, FUSE>(a, c, nct, stream); break;
    }
}

static int mid_col_tiles(const VerifyArgs &a, int col_tiles) {
    if (col_tiles != 0) return col_tiles;
    const long long heads = static_cast<long long>(a.B) * a.H;
    return heads <= 32 ? 1 : (heads <= 64 ? 2 : 4);
}

// col_tiles: 16-column tiles per workgroup (1, 2 or 4); 0 picks by the number of heads.
hipError_t launch_verify_mid(const VerifyArgs &a, int col_tiles, hipStream_t stream) {
    const int nct = mid_col_tiles(a, col_tiles);
    const PrevCommitArgs none{};
    if (a.bf16)
        launch_mid_dtype<true, false>(a, none, nct, stream);
    else
        launch_mid_dtype<false, false>(a, none, nct, stream);
    return hipGetLastError();
}

// Whether the fused commit fits this shape: each thread holds at most 2 (column, row chunk)
// pairs of S0, i.e. 4 * tiles <= 2 * sub-blocks.
bool commit_verify_mid_fits(const VerifyArgs &a, int col_tiles) {
    const int nsb = (a.T + 15) / 16, nct = mid_col_tiles(a, col_tiles);
    return a.T > 16 && a.T <= 64 && 4 * nct <= 2 * nsb;
}

// The commit of the previous tree's path (c.T <= 64: one path position per lane) fused in front
// of the verify of a tree of 17 to 64 nodes; a.S0 is the state before the commit.
hipError_t launch_commit_verify_mid(const VerifyArgs &a, const PrevCommitArgs &c, int col_tiles,
                                    hipStream_t stream) {
    const int nct = mid_col_tiles(a, col_tiles);
    if (a.bf16)
        launch_mid_dtype<true, true>(a, c, nct, stream);
    else
        launch_mid_dtype<false, true>(a, c, nct, stream);
    return hipGetLastError();
}

}  // namespace canopy
