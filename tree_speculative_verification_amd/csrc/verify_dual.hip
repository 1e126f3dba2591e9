// Blocked tree verification sized for two workgroups per compute unit (gfx950, bf16 inputs,
// trees of 65 to 256 nodes). It solves the same system as the blocked kernel, in the same
// 64-node blocks, by forward substitution over 16-node sub-blocks ("The tree closed form" on
// the canopy project page; "Design decisions / Two solve strategies", "Batch and heads to
// CTAs"), but holds at most 80 KiB of LDS and 128 VGPRs per lane: at B = 16, H = 32 the 512
// (sequence, head) workgroups then run in one pass, two per CU, and each hides the other's
// dependent latency instead of waiting for a second pass.
//
// One workgroup per (sequence b, head h), eight waves, each owning 16 value columns.
//   LDS       tree prep tables, beta and P, the Gram stage of one block pair (-G and C as bf16
//             hi + lo), the current block's K_r and Q_r
//   registers RHS_r and the read-out O_r of the current block (the wave's columns)
//   re-read   the wave's S0 columns once per block, K_c rows of the wave's Gram tiles for an
//             earlier block c, and the solved U_c of its columns (its own stores, for the
//             couplings): 576 KiB per (sequence, head) at T = 256, which miss the L2 and about
//             double the bytes the kernel moves; it still runs faster than the one-workgroup-
//             per-CU kernel that holds them
// Per block r: a2 projections R_r = beta (V_r - P K_r S0), O_r = P Q_r S0; for each c < r the
// Gram pair (r, c) staged, then RHS_r -= G_rc U_c and O_r += C_rc U_c; the diagonal pair (r, r)
// staged, its 16 x 16 diagonal sub-blocks inverted (squaring form), forward substitution over
// the four sub-blocks, O_r += C_rr U_r; U_r and O_r stored.
#include "canopy_kernels.hpp"
#include "canopy_prep.hpp"
#include "canopy_stage.hpp"

namespace canopy {

namespace {

constexpr int kDualNT = 512;

// Loads and stores address one (sequence, head) through buffer resources with 32-bit byte
// offsets: a per-lane part in one VGPR and a wave-uniform part in an SGPR (the host runs this
// kernel only when a head's rows span less than 2^31 bytes).

// The wave's 16 S0 columns (col0 + lr) at key rows 32 ks + 8 lg + e: the B operands of K S0.
__device__ __forceinline__ void dual_load_s0(float (&s0v)[4][8], BufRsrc rs0, uint32_t vo) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s0v[ks][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs0, vo, (32 * ks + e) * D * 4, 0));
}

// V at node rows row0 + 16 ti + 4 lg + e (rows at or past T read row T - 1; nothing uses
// them) of the lane's column, in the result placement of the projections; colb = the column's
// byte offset in a row.
__device__ __forceinline__ void dual_load_v(uint16_t (&vr)[4][4], BufRsrc rv, uint32_t colb, uint32_t rowb,
                                            int row0, int T, int lg) {
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t row = static_cast<uint32_t>(min(row0 + 16 * ti + 4 * lg + e, T - 1));
            vr[ti][e] = __builtin_amdgcn_raw_buffer_load_b16(rv, row * rowb + colb, 0, 0);
        }
}

// K row row0 + lr (all 128 keys) as A operands (reduction slices ks, lane group lg);
// vo = (lr rows + 8 lg keys) bytes.
__device__ __forceinline__ void dual_load_krow(Ops<true>::In (&kf)[4], BufRsrc rk, uint32_t vo, uint32_t rowb,
                                               int row0) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        kf[ks].x = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, vo, row0 * rowb + 64 * ks, 0));
}

// The lane's row and lane group, re-derived where the loops use them: an empty asm that the
// compiler must assume changes them keeps it from computing every LDS and stage address of
// every loop iteration once up front and holding them all in registers.
__device__ __forceinline__ void dual_lane(int lr0, int lg0, int &lr, int &lg) {
    lr = lr0;
    lg = lg0;
    asm volatile("" : "+v"(lr), "+v"(lg));
}

// The staged -G (or its diagonal inverses) at row r, columns c0 .. c0 + 3 as the hi and lo bf16
// parts of a 16-long reduction's A operand.
__device__ __forceinline__ Ops<true>::Sp4 dual_stage4(const Stage<true> &st, int r, int c0) {
    const int o = Stage<true>::off(r, c0);
    Ops<true>::Sp4 s;
    s.hi = __builtin_bit_cast(i16x4, *reinterpret_cast<const uint2 *>(st.gh + o));
    s.lo = __builtin_bit_cast(i16x4, *reinterpret_cast<const uint2 *>(st.gl + o));
    return s;
}

}  // namespace

template <int NB>
__global__ __launch_bounds__(kDualNT) __attribute__((amdgpu_waves_per_eu(4)))
void verify_dual_kernel(VerifyArgs a) {
    using Op = Ops<true>;
    using In = Op::In;
    using Sp = Op::Sp;
    constexpr int MAXT = 64 * NB;
    constexpr int NT = kDualNT;
    constexpr int BLK = 64 * Op::ROWB;
    __shared__ PrepSmem<MAXT> ps;
    __shared__ float s_beta[MAXT], s_P[MAXT];
    __shared__ Stage<true> st;
    __shared__ __align__(16) uint8_t s_ka[BLK];
    __shared__ __align__(16) uint8_t s_qa[BLK];

    const int bh = xcd_remap(blockIdx.x, gridDim.x);
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
    const int lr0 = lane & 15, lg0 = lane >> 4;
    const int lr = lr0, lg = lg0;
    const int col0 = wave * 16;
    const size_t rs = static_cast<size_t>(H) * D;                  // node stride (elements)
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;  // (b, node 0, h, col 0)
    const size_t sbase = static_cast<size_t>(b) * T * H + h;       // (b, node 0, h) scalars
    const size_t qkrs = static_cast<size_t>(a.HK) * D;
    const size_t qkbase = qk_base(b, h, H, a.HK, T);
    const float *S0h = a.S0 + static_cast<size_t>(bh) * D * D;
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;
    // The wave's Gram tiles of a block pair: rows 16 ti (ti = tiA, tiA + 2) of block r against
    // columns 16 tj of block c; both share the A operand, K_c rows 16 tj + lr.
    const int tj = wave & 3, tiA = wave >> 2;
    const BufRsrc rs0 = buf_rsrc(S0h), rv = buf_rsrc(static_cast<const uint16_t *>(a.v) + base);
    const BufRsrc rk = buf_rsrc(static_cast<const uint16_t *>(a.k) + qkbase);
    const BufRsrc ru = buf_rsrc(a.U + base), ro = buf_rsrc(a.O + base);
    const uint32_t vrow = static_cast<uint32_t>(rs) * 4;     // bytes per node row of U, O
    const uint32_t vrow2 = static_cast<uint32_t>(rs) * 2;    // of V
    const uint32_t krow = static_cast<uint32_t>(qkrs) * 2;   // of K
    const uint32_t vo_s0 = static_cast<uint32_t>((8 * lg0) * D + col0 + lr0) * 4;
    const uint32_t vo_v = (col0 + lr0) * 2;
    const uint32_t vo_k = lr0 * krow + 16 * lg0;
    const uint32_t vo_uc = (8 * lg0) * vrow + (col0 + lr0) * 4;  // U rows 8 lg + e of a 32-row slice
    const uint32_t vo_out = (4 * lg0) * vrow + (col0 + lr0) * 4;  // rows 4 lg + e of a 16-row tile

    // ---- loads: the tree first, then block 0 of K and Q into LDS, S0 and V of block 0
    PrepIn<MAXT, NT> pin;
    pin.load(a.parent + static_cast<size_t>(b) * T, a.alpha + sbase, H, T);
    float bet[PrepIn<MAXT, NT>::NPT];
#pragma unroll
    for (int t = 0; t < PrepIn<MAXT, NT>::NPT; ++t)
        bet[t] = a.beta[sbase + static_cast<size_t>(min(tid + t * NT, T - 1)) * H];
    dma_block<true, NT>(s_ka, a.k, qkbase, qkrs, 0, T);
    dma_block<true, NT>(s_qa, a.q, qkbase, qkrs, 0, T);

    const int pbad = tree_prep_compute<MAXT, NT>(ps, pin, Tb);
    const int bad = sl.bad ? -1 : pbad;
    if (bad) {
        const float qnan = __builtin_nanf("");
        for (int i = lg; i < Tb; i += 4) {
            a.O[base + i * rs + col0 + lr] = qnan;
            a.U[base + i * rs + col0 + lr] = qnan;
        }
        for (int i = tid; i < Tb; i += NT) a.ell[sbase + static_cast<size_t>(i) * H] = qnan;
        if (h == 0) {
            const int W = (T + 31) >> 5;
            if (a.tree_status && tid == 0) a.tree_status[b] = bad;
            if (a.depth)
                for (int i = tid; i < Tb; i += NT) a.depth[static_cast<size_t>(b) * T + i] = 0;
            if (a.anc_mask)
                for (int x = tid; x < Tb * W; x += NT) a.anc_mask[static_cast<size_t>(b) * T * W + x] = 0u;
        }
        wait_vmem();  // block 0's loads into LDS land before the workgroup's LDS is released
        return;
    }
#pragma unroll
    for (int t = 0; t < PrepIn<MAXT, NT>::NPT; ++t) {
        const int i = tid + t * NT;
        if (i < MAXT) {
            float P = 0.f;
            if (i < Tb) {
                P = __builtin_amdgcn_exp2f(static_cast<float>(ps.ell[i]));
                a.ell[sbase + static_cast<size_t>(i) * H] = static_cast<float>(ps.ell[i] * 0.69314718055994530942);
            }
            s_beta[i] = (i < Tb) ? bet[t] : 0.f;
            s_P[i] = P;
        }
    }
    if (h == 0) {
        const int W = (T + 31) >> 5;
        if (a.tree_status && tid == 0) a.tree_status[b] = 0;
        for (int i = tid; i < Tb; i += NT) {
            if (a.depth) a.depth[static_cast<size_t>(b) * T + i] = node_depth<MAXT>(ps, i);
            if (a.anc_mask)
                for (int w = 0; w < W; ++w)
                    a.anc_mask[(static_cast<size_t>(b) * T + i) * W + w] = ps.mask[i][w];
        }
    }

    const int nb = (Tb + 63) >> 6;
#pragma unroll 1
    for (int r = 0; r < nb; ++r) {
        // This wave's share of K_r and Q_r, its S0 and V of block r and its stores of block
        // r - 1 (whose U the couplings read back) are complete; after the barrier every share
        // is in LDS and the stage is free.
        wait_vmem();
        __syncthreads();

        // ---- a2: projections of block r through S0
        f32x4 rhs[4], oacc[4];
        {
            int lr, lg;
            dual_lane(lr0, lg0, lr, lg);
            float s0v[4][8];
            dual_load_s0(s0v, rs0, vo_s0);
            uint16_t vr[4][4];
            dual_load_v(vr, rv, vo_v, vrow2, 64 * r, T, lg);
            f32x4 ak[4], aq[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) ak[ti] = aq[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const Sp sf = Op::split(s0v[ks]);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {  // rows past Tb: staged copies of row T - 1, dropped below
                    const In kf = Op::lds_frag(s_ka, 16 * ti + lr, 4 * ks + lg);
                    const In qf = Op::lds_frag(s_qa, 16 * ti + lr, 4 * ks + lg);
                    ak[ti] = Op::mma(kf, sf, ak[ti]);
                    aq[ti] = Op::mma(qf, sf, aq[ti]);
                }
            }
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 64 * r + 16 * ti + 4 * lg + e;  // < MAXT
                    const float bt = s_beta[i], pp = s_P[i];
                    const float rv = bt * (bf16_to_f32(vr[ti][e]) - pp * ak[ti][e]);
                    rhs[ti][e] = i < Tb ? rv : 0.f;
                    oacc[ti][e] = i < Tb ? pp * aq[ti][e] : 0.f;
                }
        }

#pragma unroll 1
        for (int c = 0; c <= r; ++c) {
            const bool diag = c == r;
            int lr, lg;
            dual_lane(lr0, lg0, lr, lg);
            float ucr[2][8];  // U_c for the couplings, requested once the Gram products are issued
            In kf[4];
            if (diag) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kf[ks] = Op::lds_frag(s_ka, 16 * tj + lr, 4 * ks + lg);
            } else {
                dual_load_krow(kf, rk, vo_k, krow, 64 * c + 16 * tj);
            }

            // ---- a3: the wave's two tiles of the masked, decay-weighted Gram pair (r, c). The
            // MFMA takes K_c as A and K_r / Q_r as B, so each lane ends with 4 consecutive
            // columns j of one row i.
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int ti = tiA + 2 * q;
                const int i0 = 64 * r + 16 * ti, j0 = 64 * c + 16 * tj;
                const bool need = (i0 < Tb) && (j0 < Tb) && (!diag || tj <= ti);
                if (!need) {
                    st.zero_tile(16 * ti, 16 * tj, lane);
                    continue;
                }
                f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const In ka = Op::lds_frag(s_ka, 16 * ti + lr, 4 * ks + lg);
                    const In qa = Op::lds_frag(s_qa, 16 * ti + lr, 4 * ks + lg);
                    kk = Op::mma(kf[ks], ka, kk);
                    qk = Op::mma(kf[ks], qa, qk);
                }
                const int i = i0 + lr;
                const int jb = j0 + 4 * lg;
                const uint32_t bits = (ps.mask[i][jb >> 5] >> (jb & 31)) & 0xFu;
                const double li = ps.ell[i];
                const float bi = s_beta[i];
                const double2 l01 = *reinterpret_cast<const double2 *>(&ps.ell[jb]);
                const double2 l23 = *reinterpret_cast<const double2 *>(&ps.ell[jb + 2]);
                const double lj[4] = {l01.x, l01.y, l23.x, l23.y};
                float gv[4], cv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // exp(l_i - l_j) as 2 to the difference of the log2 path sums; off the path
                    // the exponent may overflow (or read a node past T), the selects drop it
                    const float gam = __builtin_amdgcn_exp2f(static_cast<float>(li - lj[e]));
                    const bool on = (bits >> e) & 1u;
                    cv[e] = on ? gam * qk[e] : 0.f;
                    gv[e] = (on && i != jb + e) ? -bi * gam * kk[e] : 0.f;
                }
                st.store4(16 * ti + lr, 16 * tj + 4 * lg, gv, cv);
            }
            // U_c of the wave's columns as the couplings' B operands (node rows 32 ks + 8 lg + e;
            // every row of an earlier block lies below Tb). Requested here rather than with the
            // key rows, they do not hold 16 registers through the Gram products (2% faster at
            // B = 16, T = 256).
            if (!diag) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ucr[ks][e] = __uint_as_float(
                            __builtin_amdgcn_raw_buffer_load_b32(ru, vo_uc, (64 * c + 32 * ks + e) * vrow, 0));
            }
            lds_barrier();

            if (!diag) {
                // ---- a4/a5: couplings to the solved block c
                Sp uf[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) uf[ks] = Op::split(ucr[ks]);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        rhs[ti] = Op::mma(st.fragG(16 * ti + lr, 32 * ks + 8 * lg), uf[ks], rhs[ti]);
                        oacc[ti] = Op::mma(st.fragC(16 * ti + lr, 32 * ks + 8 * lg), uf[ks], oacc[ti]);
                    }
                lds_barrier();  // the stage is free for the next pair
                continue;
            }

            const bool next = r + 1 < nb;
            // Past the staging barrier nothing reads K_r and Q_r: request block r + 1's.
            if (next) {
                dma_block<true, NT>(s_ka, a.k, qkbase, qkrs, 64 * (r + 1), T);
                dma_block<true, NT>(s_qa, a.q, qkbase, qkrs, 64 * (r + 1), T);
            }
            // ---- a4: the 16 x 16 unit lower-triangular diagonal sub-blocks I - N (the stage
            // holds N = -G_pp), one per wave for waves 0-3, inverted as the product of the
            // factors (I + N^(2^s)) of the finite Neumann series, truncated at the sub-block's
            // depth (the squaring form), on fp32 MFMA; the inverse replaces N in the stage.
            // With Z = X Y, Z in the A placement is the product of Y's B placement and X's A
            // placement.
            if (wave < 4 && 64 * r + 16 * wave < Tb) {
                const int p = wave;
                const int ip = 64 * r + 16 * p + lr;
                const uint32_t wbits = (ip < Tb) ? ps.mask[ip][2 * r + (p >> 1)] : 0u;
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
            // ---- a4: forward substitution over the four sub-blocks of the wave's columns,
            //   U_p = (I - N_pp)^-1 (RHS_p + sum_{q<p} N_pq U_q),
            // RHS_p and U_q in the result placement (rows 4 lg .. 4 lg + 3 of column lr), the B
            // placement of a 16-long reduction; the stage gives N_pq row lr, columns 4 lg ..
            // 4 lg + 3 as its bf16 hi and lo parts. Each product takes three bf16 matrix-core
            // passes (hi hi + hi lo + lo hi, U split likewise; relative error about 2^-16).
            // Sub-blocks past T have zero RHS and a zero stage: U is zero there.
            f32x4 u[4];
            Op::Sp4 us[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                f32x4 acc = rhs[p];
#pragma unroll
                for (int q = 0; q < p; ++q) acc = Op::mma16(dual_stage4(st, 16 * p + lr, 16 * q + 4 * lg), us[q], acc);
                float av[4] = {acc[0], acc[1], acc[2], acc[3]};
                u[p] = Op::mma16(dual_stage4(st, 16 * p + lr, 16 * p + 4 * lg), Op::split4(av),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
                float uv[4] = {u[p][0], u[p][1], u[p][2], u[p][3]};
                us[p] = Op::split4(uv);
            }
            // ---- a5: O_r += C_rr U_r. U_r as B operands of 32-long slices: lane (lg, lr) takes
            // node rows 32 ks + 8 lg + e, i.e. sub-block 2 ks + lg / 2, local row 8 (lg % 2) + e,
            // held by lane group 2 (lg % 2) + e / 4 as its element e % 4.
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float v8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int src = ((2 * (lg & 1) + (e >> 2)) << 4) | lr;
                    const float a0 = __shfl(u[2 * ks][e & 3], src, 64);
                    const float a1 = __shfl(u[2 * ks + 1][e & 3], src, 64);
                    v8[e] = (lg >> 1) ? a1 : a0;
                }
                const Sp ub = Op::split(v8);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
                    oacc[ti] = Op::mma(st.fragC(16 * ti + lr, 32 * ks + 8 * lg), ub, oacc[ti]);
            }
            // ---- a6: outputs of block r, U and O both as ordinary stores (streaming O stores were
            // no faster with one layer and 2.5% slower with four layers run in turn)
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 64 * r + 16 * p + 4 * lg + e;
                    if (i < Tb) {
                        const uint32_t so = (64 * r + 16 * p + e) * vrow;
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(u[p][e]), ru, vo_out, so, 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(oacc[p][e]), ro, vo_out, so, 0);
                    }
                }
        }
    }
}

template <int NB>
static hipError_t launch_dual_nb(const VerifyArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H));
    hipLaunchKernelGGL((verify_dual_kernel<NB>), grid, dim3(kDualNT), 0, stream, a);
    return hipGetLastError();
}

bool dual_fits(int HK, int HV, int T) {
    return static_cast<long long>(T) * HV * D * 4 < (1LL << 31) && static_cast<long long>(T) * HK * D * 2 < (1LL << 31);
}

// bf16 inputs, 65 <= T <= 256; FWDSUB on every diagonal block.
hipError_t launch_verify_dual(const VerifyArgs &a, hipStream_t stream) {
    switch ((a.T + 63) / 64) {
        case 2: return launch_dual_nb<2>(a, stream);
        case 3: return launch_dual_nb<3>(a, stream);
        default: return launch_dual_nb<4>(a, stream);
    }
}

}  // namespace canopy
