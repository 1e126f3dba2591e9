// Fused tree verification of one Gated DeltaNet layer (gfx950).
//
// One workgroup owns one (sequence b, head h, value tile); each of its NW waves owns 16 value
// columns of that tile. Per the tree closed form on the canopy project page ("The tree closed
// form"; "Design decisions / Two solve strategies", "Batch and heads to CTAs"):
//   prep     l, ancestor bitmask, depth, validation (pointer jumping, in LDS)
//   a2       KS = K S0, QS = Q S0 on MFMA: R_i = beta_i (v_i - P_i KS_i), O_i = P_i QS_i
//   a3       G_rc = -beta_i Gamma_ij k_i.k_j (strict ancestors), C_rc = Gamma_ij q_i.k_j
//            (path) for 64 x 64 node blocks r >= c, MFMA K K^T and Q K^T, staged in LDS
//   a4       blocked solve: RHS_r = R_r - sum_{c<r} G_rc U_c (MFMA), then the diagonal block:
//            FWDSUB  forward substitution over four 16-node sub-blocks, each 16 x 16 diagonal
//                    sub-block inverted by substitution and applied on MFMA (depth-independent)
//            LEVEL   row substitution, rows of equal in-block depth together (cheap when shallow)
//            NEUMANN the finite Neumann series, one MFMA product per in-block level
//            AUTO    NEUMANN for blocks of in-block depth <= 2, else FWDSUB
//   a5       O_r += sum_{c<=r} C_rc U_c (MFMA); O and U stored as fp32.
// G is staged negated so that every coupling term accumulates with a plain MFMA.
//
// Data movement: each 64-node block of K and Q is copied once per workgroup from HBM into a
// swizzled LDS layout, and every wave reads its MFMA operands from there. The tree (parent,
// alpha, beta) is requested first, then block 0 of K and Q (through registers), the wave's S0
// columns and value rows, all before the tree preprocessing runs. The next block's K, Q
// (and K_0) are requested with LDS-bound loads before the current diagonal block is solved,
// and K_{c+1} before the couplings to K_c; each wave waits for its own requests before the
// barrier that ends the pair.
#include <type_traits>

#include "canopy_kernels.hpp"
#include "canopy_levelsync.hpp"
#include "canopy_prep.hpp"
#include "canopy_stage.hpp"

namespace canopy {

constexpr int XS = 68;  // column stride (floats) of the per-wave 64-row x 16-column solve buffer (column-major)
// AUTO sums the finite Neumann series of a diagonal block whose in-block depth is at most this
// (one MFMA product per level, no inverses to build) and substitutes over the 16-node sub-blocks
// in deeper blocks. Measured on level trees (T = 128 and 256, B = 4 and 16): the series is
// 7-15% faster at in-block depth 0-2, forward substitution from depth 3 up, and the level solve
// is never the fastest.
constexpr int kNeumannMaxDepth = 2;

// LS: the instantiation that LEVELSYNC launches, with the gather solve; the others hold the
// blocked solve alone (so that its code and registers are not shaped by the gather path).
template <int NW, bool BF, int NB, bool LS>
__global__ __launch_bounds__(NW * 64) void verify_kernel(VerifyArgs a) {
    using Op = Ops<BF>;
    using In = typename Op::In;
    using Sp = typename Op::Sp;
    using Raw = typename Op::Raw;
    constexpr int MAXT = 64 * NB;
    constexpr int NT = NW * 64;
    constexpr int TILES = D / (16 * NW);
    constexpr int BLK = 64 * Op::ROWB;  // bytes of one staged 64-row block of K or Q
    using BC = BlockCopy<BF, NT>;
    constexpr bool kPF = BC::PER <= 4;  // prefetch blocks through registers (wide workgroups)

    // The level-synchronous gather solve (bf16, all 128 columns in one workgroup, on request)
    // shares its tables' memory with the blocked solve's staging: a workgroup takes one of the two.
    constexpr bool kLS = LS && BF && NW == 8;

    struct Blocked {
        Stage<BF> st;
        alignas(16) float x[NW][16][XS];
        int list[NW][64];
        alignas(16) uint8_t v[NW][64 * 16 * Op::ES];  // V rows x 16 columns
        alignas(16) uint8_t ka[BLK];
        alignas(16) uint8_t qa[BLK];
        alignas(16) uint8_t kb[NB > 1 ? BLK : 16];
    };
    union Work {
        Blocked bl;
        std::conditional_t<kLS, LsSmem<MAXT>, char> ls;
    };
    __shared__ PrepSmem<MAXT> ps;
    __shared__ float s_beta[MAXT], s_P[MAXT];
    __shared__ Work wk;
    Stage<BF> &st = wk.bl.st;
    float(*s_x)[16][XS] = wk.bl.x;
    int(*s_list)[64] = wk.bl.list;
    uint8_t(*s_v)[64 * 16 * Op::ES] = wk.bl.v;
    uint8_t *s_ka = wk.bl.ka;
    uint8_t *s_qa = wk.bl.qa;
    uint8_t *s_kb = wk.bl.kb;

    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = g % TILES;
    const int bh = g / TILES;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int col0 = (tile * NW + wave) * 16;
    const size_t rs = static_cast<size_t>(H) * D;                  // node stride (elements)
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;  // (b, node 0, h, col 0)
    const size_t sbase = (static_cast<size_t>(b) * T * H + h);     // (b, node 0, h) scalars
    const size_t qkrs = static_cast<size_t>(a.HK) * D;              // q/k node stride
    const size_t qkbase = qk_base(b, h, H, a.HK, T);                // (b, node 0, q/k head, col 0)
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;  // this sequence's node count: rows past it are padding
    float(*Xc)[XS] = s_x[wave];  // Xc[column][row]

    // ---- loads, latency-critical first: the tree, then block 0 of K and Q, S0, V
    PrepIn<MAXT, NT> pin;
    pin.load(a.parent + static_cast<size_t>(b) * T, a.alpha + sbase, H, T);
    float bet[PrepIn<MAXT, NT>::NPT];
#pragma unroll
    for (int t = 0; t < PrepIn<MAXT, NT>::NPT; ++t)
        bet[t] = a.beta[sbase + static_cast<size_t>(min(tid + t * NT, T - 1)) * H];
    BC pk, pq;
    if constexpr (kPF) {
        pk.issue(a.k, qkbase, qkrs, 0, T);
        pq.issue(a.q, qkbase, qkrs, 0, T);
    }
    float s0v[4][8];
    {
        const float *S0p = a.S0 + static_cast<size_t>(bh) * D * D + col0 + lr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) s0v[ks][e] = S0p[(32 * ks + 8 * lg + e) * D];
    }
    VCopy<BF> pv;  // this wave's 16 value columns of a 64-row block
    pv.issue(a.v, base, rs, col0, 0, T, lane);

    const int pbad = tree_prep_compute<MAXT, NT>(ps, pin, Tb);
    const int bad = sl.bad ? -1 : pbad;
    if (bad) {
        const float qnan = __builtin_nanf("");
        for (int i = lg; i < Tb; i += 4) {
            a.O[base + i * rs + col0 + lr] = qnan;
            a.U[base + i * rs + col0 + lr] = qnan;
        }
        if (tile == 0)
            for (int i = tid; i < Tb; i += NT) a.ell[sbase + static_cast<size_t>(i) * H] = qnan;
        if (tile == 0 && h == 0) {
            const int W = (T + 31) >> 5;
            if (a.tree_status && tid == 0) a.tree_status[b] = bad;
            if (a.depth)
                for (int i = tid; i < Tb; i += NT) a.depth[static_cast<size_t>(b) * T + i] = 0;
            if (a.anc_mask)
                for (int x = tid; x < Tb * W; x += NT) a.anc_mask[static_cast<size_t>(b) * T * W + x] = 0u;
        }
        return;
    }

#pragma unroll
    for (int t = 0; t < PrepIn<MAXT, NT>::NPT; ++t) {
        const int i = tid + t * NT;
        if (i < MAXT) {
            float P = 0.f;
            if (i < Tb) {
                P = __builtin_amdgcn_exp2f(static_cast<float>(ps.ell[i]));
                if (tile == 0)
                    a.ell[sbase + static_cast<size_t>(i) * H] = static_cast<float>(ps.ell[i] * 0.69314718055994530942);
            }
            s_beta[i] = (i < Tb) ? bet[t] : 0.f;
            s_P[i] = P;
        }
    }
    if (tile == 0 && h == 0) {
        const int W = (T + 31) >> 5;
        if (a.tree_status && tid == 0) a.tree_status[b] = 0;
        for (int i = tid; i < Tb; i += NT) {
            if (a.depth) a.depth[static_cast<size_t>(b) * T + i] = node_depth<MAXT>(ps, i);
            if (a.anc_mask)
                for (int w = 0; w < W; ++w)
                    a.anc_mask[(static_cast<size_t>(b) * T + i) * W + w] = ps.mask[i][w];
        }
    }
    if constexpr (kLS) {
        // LEVELSYNC takes the gather solve whenever the tree fits its tables (and a sequence's
        // rows span less than 2^31 bytes, for its 32-bit offsets).
        const bool fits32 = static_cast<size_t>(T) * rs * 4 < (size_t{1} << 31) &&
                            static_cast<size_t>(T) * qkrs * 2 < (size_t{1} << 31);
        if (a.solver == CANOPY_SOLVE_LEVELSYNC && fits32) {
            const int nbatch = ls_build<MAXT, NT>(wk.ls, ps, s_beta, s_P, pin.p[0], Tb, a.k, qkbase, qkrs);
            if (nbatch > 0) {
                const uint16_t *qp = static_cast<const uint16_t *>(a.q);
                const uint16_t *vp = static_cast<const uint16_t *>(a.v);
                Sp s0f[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) s0f[ks] = Op::split(s0v[ks]);
                ls_project<MAXT, NT>(wk.ls, s_beta, s_P, qp, vp, qkbase, qkrs, base, rs, col0, s0f, Tb, a.U, a.O);
                ls_gram<MAXT, NW>(wk.ls, ps, s_beta, qp, qkbase, qkrs, Tb);
                wait_vmem();      // the parked projections are written, and
                __syncthreads();  // the pair entries are complete and the staged k is no longer read
                ls_levels<MAXT, NW>(wk.ls, base, rs, Tb, nbatch, a.U, a.O);
                return;
            }
        }
    }
    if constexpr (kPF) {
        pk.commit(s_ka);
        pq.commit(s_qa);
    } else {
        copy_block<BF, NT>(s_ka, a.k, qkbase, qkrs, 0, T);
        copy_block<BF, NT>(s_qa, a.q, qkbase, qkrs, 0, T);
    }
    pv.commit(s_v[wave], lane);
    // S0 columns of this wave as B operands of K S0 and Q S0 (reduction index = key row).
    Sp s0f[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s0f[ks] = Op::split(s0v[ks]);
    __syncthreads();

    Sp uf[NB][2];  // U of every solved block, as B operands (reduction index = node)
    const int nb = (Tb + 63) >> 6;

#pragma unroll
    for (int r = 0; r < NB; ++r) {
        if (r >= nb) break;
        f32x4 rhs[4], oacc[4];
        // ---- a2: projections of block r through S0
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int i0 = 64 * r + 16 * ti;
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
            if (i0 < Tb) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const In kf = Op::lds_frag(s_ka, 16 * ti + lr, 4 * ks + lg);
                    const In qf = Op::lds_frag(s_qa, 16 * ti + lr, 4 * ks + lg);
                    ak = Op::mma(kf, s0f[ks], ak);
                    aq = Op::mma(qf, s0f[ks], aq);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + 4 * lg + e;
                float rv = 0.f, ov = 0.f;
                if (i < Tb) {
                    rv = s_beta[i] * (VCopy<BF>::get(s_v[wave], 16 * ti + 4 * lg + e, lr) - s_P[i] * ak[e]);
                    ov = s_P[i] * aq[e];
                }
                rhs[ti][e] = rv;
                oacc[ti][e] = ov;
            }
        }

#pragma unroll
        for (int c = 0; c <= r; ++c) {
            // ---- a3: masked, decay-weighted Gram block pair (r, c), shared by all waves. The
            // MFMA takes K_c as A and K_r / Q_r as B, so each lane ends with 4 consecutive
            // columns j of one row i: one mask word, one row's scalars, 8-byte stores.
            const uint8_t *kc = (c < r) ? s_kb : s_ka;
#pragma unroll 1
            for (int p = wave; p < 16; p += NW) {
                const int ti = p >> 2, tj = p & 3;
                const int i0 = 64 * r + 16 * ti, j0 = 64 * c + 16 * tj;
                const bool need = (i0 < Tb) && (j0 < Tb) && (c < r || tj <= ti);
                if (!need) {
                    st.zero_tile(16 * ti, 16 * tj, lane);
                    continue;
                }
                f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const In kb = Op::lds_frag(kc, 16 * tj + lr, 4 * ks + lg);
                    const In ka = Op::lds_frag(s_ka, 16 * ti + lr, 4 * ks + lg);
                    const In qa = Op::lds_frag(s_qa, 16 * ti + lr, 4 * ks + lg);
                    kk = Op::mma(kb, ka, kk);
                    qk = Op::mma(kb, qa, qk);
                }
                const int i = i0 + lr;
                const int jb = j0 + 4 * lg;  // first of this lane's 4 columns
                const uint32_t bits = (ps.mask[i][jb >> 5] >> (jb & 31)) & 0xFu;
                const double li = ps.ell[i];
                const float bi = s_beta[i];
                const double2 l01 = *reinterpret_cast<const double2 *>(&ps.ell[jb]);
                const double2 l23 = *reinterpret_cast<const double2 *>(&ps.ell[jb + 2]);
                const double lj[4] = {l01.x, l01.y, l23.x, l23.y};
                float gv[4], cv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // exp(l_i - l_j) as 2 to the difference of the log2 path sums. Off the path
                    // the exponent may overflow (or read a node past T); the selects drop those
                    // entries.
                    const float gam = __builtin_amdgcn_exp2f(static_cast<float>(li - lj[e]));
                    const bool on = (bits >> e) & 1u;
                    cv[e] = on ? gam * qk[e] : 0.f;
                    gv[e] = (on && i != jb + e) ? -bi * gam * kk[e] : 0.f;
                }
                st.store4(16 * ti + lr, 16 * tj + 4 * lg, gv, cv);
            }
            lds_barrier();

            if (c < r) {
                // K_c is no longer needed: request K_{c+1} for the next pair of this block.
                const bool more = c + 1 < r;
                if (more) dma_block<BF, NT>(s_kb, a.k, qkbase, qkrs, 64 * (c + 1), T);
                // ---- a4/a5: couplings to the solved block c
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const Sp gf = st.fragG(16 * ti + lr, 32 * ks + 8 * lg);
                        const Sp cf = st.fragC(16 * ti + lr, 32 * ks + 8 * lg);
                        rhs[ti] = Op::mma(gf, uf[c][ks], rhs[ti]);
                        oacc[ti] = Op::mma(cf, uf[c][ks], oacc[ti]);
                    }
                }
                if (more) wait_vmem();
            } else {
                const bool next = r + 1 < nb;
                // Past the staging barrier of the diagonal pair nothing reads block r's K, Q
                // and V or K_c any more (the solve and the read-out use the stage): request
                // the next block's K, Q, V and K_0 now, to land during the solve.
                if (next) {
                    dma_block<BF, NT>(s_ka, a.k, qkbase, qkrs, 64 * (r + 1), T);
                    dma_block<BF, NT>(s_qa, a.q, qkbase, qkrs, 64 * (r + 1), T);
                    if (NB > 1) dma_block<BF, NT>(s_kb, a.k, qkbase, qkrs, 0, T);
                    dma_v<BF>(s_v[wave], a.v, base, rs, col0, 64 * (r + 1), T, lane);
                }
                // ---- a4: the diagonal block, per wave on its 16 columns
                const int ib = 64 * r + lane;
                uint64_t bm = 0;
                if (ib < Tb)
                    bm = (static_cast<uint64_t>(ps.mask[ib][2 * r + 1]) << 32) | ps.mask[ib][2 * r];
                const int ld = (ib < Tb) ? __popcll(bm) - 1 : -1;
                const int maxld = wave_max(ld);
                const bool use_neumann = a.solver == CANOPY_SOLVE_NEUMANN ||
                                         (a.solver == CANOPY_SOLVE_AUTO && maxld <= kNeumannMaxDepth);
                const bool use_level = a.solver == CANOPY_SOLVE_LEVEL;
                const bool use_fwd = !use_neumann && !use_level;
                if (use_fwd) {
                    // Each 16 x 16 unit lower-triangular diagonal sub-block I - N (the stage
                    // holds N = -G_pp) is inverted by one wave as the product of the factors
                    // (I + N^(2^s)) of its finite Neumann series ("The tree closed form", the
                    // squaring form), truncated at the sub-block's own depth, on fp32 MFMA.
                    // The inverse replaces N in the stage, which the substitution below no
                    // longer needs. With Z = X Y, Z in the A placement (row r, columns
                    // 4g..4g+3 in lane (g, r)) is the product of Y's B placement and X's A
                    // placement.
                    constexpr int NINV = NW < 4 ? NW : 4;
                    for (int p = wave; p < 4; p += NINV) {
                        if (64 * r + 16 * p >= Tb) break;
                        const int ip = 64 * r + 16 * p + lr;  // this lane's row in the sub-block
                        const uint32_t wbits = (ip < Tb) ? ps.mask[ip][(2 * r) + (p >> 1)] : 0u;
                        const int dl = (ip < Tb) ? __popc((wbits >> (16 * (p & 1))) & 0xFFFFu) - 1 : -1;
                        const int dp = wave_max(dl);
                        int nf = 0;
                        while ((1 << nf) <= dp) ++nf;
                        float xa[4], xb[4], minv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            xa[e] = st.getG(16 * p + lr, 16 * p + 4 * lg + e);
                            xb[e] = st.getG(16 * p + 4 * lg + e, 16 * p + lr);
                            minv[e] = (lr == 4 * lg + e ? 1.f : 0.f) + xa[e];
                        }
                        for (int s2 = 1; s2 < nf; ++s2) {
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
                        wave_lds_sync();  // every lane has read its operands from the stage
                        st.store4G(16 * p + lr, 16 * p + 4 * lg, minv);
                    }
                    lds_barrier();
                }
                if (use_neumann) {
                    f32x4 z[4];
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) z[ti] = rhs[ti];
                    for (int m = 1; m <= maxld; ++m) {
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                            for (int e = 0; e < 4; ++e) Xc[lr][16 * ti + 4 * lg + e] = z[ti][e];
                        wave_lds_sync();
                        Sp zf[2];
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            float v[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] = Xc[lr][32 * ks + 8 * lg + e];
                            zf[ks] = Op::split(v);
                        }
                        wave_lds_sync();
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti) {
                            f32x4 nz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int ks = 0; ks < 2; ++ks)
                                nz = Op::mma(st.fragG(16 * ti + lr, 32 * ks + 8 * lg), zf[ks], nz);
                            z[ti] = nz;
                            rhs[ti] += nz;
                        }
                    }
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                        for (int e = 0; e < 4; ++e) Xc[lr][16 * ti + 4 * lg + e] = rhs[ti][e];
                    wave_lds_sync();
                } else if (use_level) {
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                        for (int e = 0; e < 4; ++e) Xc[lr][16 * ti + 4 * lg + e] = rhs[ti][e];
                    wave_lds_sync();
                    for (int L = 1; L <= maxld; ++L) {
                        const uint64_t nodes = __ballot(ld == L);
                        if (ld == L) s_list[wave][__popcll(nodes & ((1ull << lane) - 1ull))] = lane;
                        wave_lds_sync();
                        const int cnt = __popcll(nodes);
                        for (int m0 = 0; m0 < cnt; m0 += 4) {
                            const int slot = m0 + lg;
                            if (slot < cnt) {
                                const int n = s_list[wave][slot];
                                const int ni = 64 * r + n;
                                uint64_t am = ((static_cast<uint64_t>(ps.mask[ni][2 * r + 1]) << 32) |
                                               ps.mask[ni][2 * r]) & ~(1ull << n);
                                float acc = Xc[lr][n];
                                while (am) {
                                    const int j = __ffsll(static_cast<unsigned long long>(am)) - 1;
                                    am &= am - 1ull;
                                    acc += st.getG(n, j) * Xc[lr][j];
                                }
                                Xc[lr][n] = acc;
                            }
                        }
                        wave_lds_sync();
                    }
                } else {
                    // Blocked forward substitution inside the block over its four 16-node
                    // sub-blocks, with the inverses of the diagonal sub-blocks in the stage:
                    //   U_p = (I - N_pp)^-1 (RHS_p + sum_{q<p} N_pq U_q),  N = -G.
                    // RHS_p and U_q sit in the result placement (rows 4lg..4lg+3 of column
                    // lr), which is the B placement of a 16-long fp32 MFMA reduction, and the
                    // stage gives N_pq row lr, columns 4lg..4lg+3 (the A placement), so the
                    // whole chain stays in registers. Sub-blocks past T have zero RHS and a
                    // zero stage, so they come out zero.
                    f32x4 u[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        f32x4 acc = rhs[p];
#pragma unroll
                        for (int q = 0; q < p; ++q) {
                            float ga[4];
                            st.getG4(16 * p + lr, 16 * q + 4 * lg, ga);
                            acc = mma16f(ga, u[q], acc);
                        }
                        float mi[4];
                        st.getG4(16 * p + lr, 16 * p + 4 * lg, mi);
                        u[p] = mma16f(mi, acc, f32x4{0.f, 0.f, 0.f, 0.f});
                    }
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        *reinterpret_cast<float4 *>(&Xc[lr][16 * p + 4 * lg]) = make_float4(u[p][0], u[p][1], u[p][2], u[p][3]);
                    wave_lds_sync();
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = Xc[lr][32 * ks + 8 * lg + e];
                    uf[r][ks] = Op::split(v);
                }
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        oacc[ti] = Op::mma(st.fragC(16 * ti + lr, 32 * ks + 8 * lg), uf[r][ks], oacc[ti]);
                // The next block's operands must be in LDS before the barrier. The counter that
                // tracks them also tracks stores, so wait before the stores are issued: nothing
                // needs them complete.
                if (next) wait_vmem();

                // ---- a6: outputs of block r
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int rl = lg + 4 * m;
                    const int i = 64 * r + rl;
                    if (i < Tb) a.U[base + static_cast<size_t>(i) * rs + col0 + lr] = Xc[lr][rl];
                }
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 64 * r + 16 * ti + 4 * lg + e;
                        if (i < Tb) store_nt(a.O + base + static_cast<size_t>(i) * rs + col0 + lr, oacc[ti][e]);
                    }
            }
            // The stage is free and the next operands are in LDS for every wave.
            lds_barrier();
        }
    }
}

template <int NW, bool BF, int NB>
static hipError_t launch_nb(const VerifyArgs &a, hipStream_t stream) {
    const int tiles = D / (16 * NW);
    const dim3 grid(static_cast<unsigned>(a.B * a.H * tiles));
    if constexpr (BF && NW == 8) {
        if (a.solver == CANOPY_SOLVE_LEVELSYNC) {
            hipLaunchKernelGGL((verify_kernel<NW, BF, NB, true>), grid, dim3(NW * 64), 0, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((verify_kernel<NW, BF, NB, false>), grid, dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int NW, bool BF>
static hipError_t launch_nw(const VerifyArgs &a, hipStream_t stream) {
    const int nb = (a.T + 63) / 64;
    switch (nb) {
        case 1: return launch_nb<NW, BF, 1>(a, stream);
        case 2: return launch_nb<NW, BF, 2>(a, stream);
        case 3: return launch_nb<NW, BF, 3>(a, stream);
        default: return launch_nb<NW, BF, 4>(a, stream);
    }
}

hipError_t launch_verify(const VerifyArgs &a, int waves, hipStream_t stream) {
    if (a.bf16) {
        switch (waves) {
            case 1: return launch_nw<1, true>(a, stream);
            case 2: return launch_nw<2, true>(a, stream);
            case 4: return launch_nw<4, true>(a, stream);
            default: return launch_nw<8, true>(a, stream);
        }
    }
    // fp32 inputs stage twice the bytes per block: at most 2 waves fit the LDS budget.
    if (waves == 1) return launch_nw<1, false>(a, stream);
    return launch_nw<2, false>(a, stream);
}

}  // namespace canopy
