// Fused tree verification of one Gated DeltaNet layer (gfx950).
//
// One workgroup owns one (sequence b, head h, value tile); each of its NW waves owns 16 value
// columns of that tile. Per the tree closed form on the canopy project page ("The tree closed
// form"; "Design decisions / Two solve strategies", "Batch and heads to CTAs"):
//   prep     l, ancestor bitmask, depth, validation (pointer jumping, in LDS)
//   a2       KS = K S0, QS = Q S0 on MFMA: R_i = beta_i (v_i - P_i KS_i), O_i = P_i QS_i
//   a3       G_rc = -beta_i Gamma_ij k_i.k_j (strict ancestors), C_rc = Gamma_ij q_i.k_j
//            (path) for 64 x 64 node blocks r >= c, MFMA K K^T and Q K^T, staged in LDS
//   a4       blocked solve: RHS_r = R_r - sum_{c<r} G_rc U_c (MFMA), then the diagonal block
//            by forward substitution (rows of equal in-block depth together) or by the finite
//            Neumann series (one MFMA product per in-block level)
//   a5       O_r += sum_{c<=r} C_rc U_c (MFMA); O and U stored as fp32.
// G is staged negated so that every coupling term accumulates with a plain MFMA.
#include "canopy_prep.hpp"
#include "canopy_kernels.hpp"

namespace canopy {

// Staging of one 64 x 64 block pair of -G and C, in the A-operand order of the MFMA.
template <bool BF>
struct Stage;

template <>
struct Stage<true> {
    static constexpr int LD = 72;  // bf16 elements per row (16 B aligned rows)
    alignas(16) uint16_t gh[64][LD];
    alignas(16) uint16_t gl[64][LD];
    alignas(16) uint16_t ch[64][LD];
    alignas(16) uint16_t cl[64][LD];
    __device__ __forceinline__ void store(int r, int c, float g, float cv) {
        const __bf16 g1 = static_cast<__bf16>(g), c1 = static_cast<__bf16>(cv);
        const __bf16 g2 = static_cast<__bf16>(g - static_cast<float>(g1));
        const __bf16 c2 = static_cast<__bf16>(cv - static_cast<float>(c1));
        gh[r][c] = __builtin_bit_cast(uint16_t, g1);
        gl[r][c] = __builtin_bit_cast(uint16_t, g2);
        ch[r][c] = __builtin_bit_cast(uint16_t, c1);
        cl[r][c] = __builtin_bit_cast(uint16_t, c2);
    }
    __device__ __forceinline__ Ops<true>::Sp frag(const uint16_t (*h)[LD], const uint16_t (*l)[LD],
                                                 int r, int k0) const {
        Ops<true>::Sp s;
        s.hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&h[r][k0]));
        s.lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&l[r][k0]));
        return s;
    }
    __device__ __forceinline__ Ops<true>::Sp fragG(int r, int k0) const { return frag(gh, gl, r, k0); }
    __device__ __forceinline__ Ops<true>::Sp fragC(int r, int k0) const { return frag(ch, cl, r, k0); }
    __device__ __forceinline__ float getG(int r, int c) const {
        return bf16_to_f32(gh[r][c]) + bf16_to_f32(gl[r][c]);
    }
};

template <>
struct Stage<false> {
    static constexpr int LD = 68;
    alignas(16) float g[64][LD];
    alignas(16) float c[64][LD];
    __device__ __forceinline__ void store(int r, int cc, float gv, float cv) {
        g[r][cc] = gv;
        c[r][cc] = cv;
    }
    __device__ __forceinline__ Ops<false>::Sp frag(const float (*m)[LD], int r, int k0) const {
        Ops<false>::Sp s;
        const float4 a = *reinterpret_cast<const float4 *>(&m[r][k0]);
        const float4 b = *reinterpret_cast<const float4 *>(&m[r][k0 + 4]);
        s.x[0] = a.x; s.x[1] = a.y; s.x[2] = a.z; s.x[3] = a.w;
        s.x[4] = b.x; s.x[5] = b.y; s.x[6] = b.z; s.x[7] = b.w;
        return s;
    }
    __device__ __forceinline__ Ops<false>::Sp fragG(int r, int k0) const { return frag(g, r, k0); }
    __device__ __forceinline__ Ops<false>::Sp fragC(int r, int k0) const { return frag(c, r, k0); }
    __device__ __forceinline__ float getG(int r, int cc) const { return g[r][cc]; }
};

constexpr int XS = 17;  // row stride (floats) of the per-wave 64 x 16 solve buffer

template <int NW, bool BF, int NB>
__global__ __launch_bounds__(NW * 64) void verify_kernel(VerifyArgs a) {
    using Op = Ops<BF>;
    using In = typename Op::In;
    using Sp = typename Op::Sp;
    constexpr int MAXT = 64 * NB;
    constexpr int NT = NW * 64;
    constexpr int TILES = D / (16 * NW);

    __shared__ PrepSmem<MAXT> ps;
    __shared__ float s_beta[MAXT], s_P[MAXT];
    __shared__ Stage<BF> st;
    __shared__ float s_x[NW][64][XS];
    __shared__ int s_list[NW][64];

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
    float(*X)[XS] = s_x[wave];

    const int bad = tree_prep_block<MAXT, NT>(ps, a.parent + static_cast<size_t>(b) * T,
                                              a.alpha + sbase, H, T);
    if (bad) {
        const float qnan = __builtin_nanf("");
        for (int i = lg; i < T; i += 4) {
            a.O[base + i * rs + col0 + lr] = qnan;
            a.U[base + i * rs + col0 + lr] = qnan;
        }
        if (tile == 0)
            for (int i = tid; i < T; i += NT) a.ell[sbase + static_cast<size_t>(i) * H] = qnan;
        if (tile == 0 && h == 0) {
            const int W = (T + 31) >> 5;
            if (a.tree_status && tid == 0) a.tree_status[b] = bad;
            if (a.depth)
                for (int i = tid; i < T; i += NT) a.depth[static_cast<size_t>(b) * T + i] = 0;
            if (a.anc_mask)
                for (int x = tid; x < T * W; x += NT) a.anc_mask[static_cast<size_t>(b) * T * W + x] = 0u;
        }
        return;
    }

    for (int i = tid; i < MAXT; i += NT) {
        float be = 0.f, P = 0.f;
        if (i < T) {
            be = a.beta[sbase + static_cast<size_t>(i) * H];
            P = static_cast<float>(exp(ps.ell[i]));
            if (tile == 0) a.ell[sbase + static_cast<size_t>(i) * H] = static_cast<float>(ps.ell[i]);
        }
        s_beta[i] = be;
        s_P[i] = P;
    }
    if (tile == 0 && h == 0) {
        const int W = (T + 31) >> 5;
        if (a.tree_status && tid == 0) a.tree_status[b] = 0;
        for (int i = tid; i < T; i += NT) {
            if (a.depth) a.depth[static_cast<size_t>(b) * T + i] = node_depth<MAXT>(ps, i);
            if (a.anc_mask)
                for (int w = 0; w < W; ++w)
                    a.anc_mask[(static_cast<size_t>(b) * T + i) * W + w] = ps.mask[i][w];
        }
    }

    // S0 columns of this wave as B operands of K S0 and Q S0 (reduction index = key row).
    Sp s0f[4];
    {
        const float *S0p = a.S0 + static_cast<size_t>(bh) * D * D + col0 + lr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = S0p[(32 * ks + 8 * lg + e) * D];
            s0f[ks] = Op::split(v);
        }
    }
    __syncthreads();

    Sp uf[NB][2];  // U of every solved block, as B operands (reduction index = node)
    const int nb = (T + 63) >> 6;

#pragma unroll
    for (int r = 0; r < NB; ++r) {
        if (r >= nb) break;
        f32x4 rhs[4], oacc[4];
        // ---- a2: projections of block r through S0
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int i0 = 64 * r + 16 * ti;
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
            if (i0 < T) {
                const int row = i0 + lr;
                const bool ok = row < T;
                const size_t el = base + static_cast<size_t>(ok ? row : 0) * rs + 8 * lg;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const In kf = Op::load_in(a.k, el + 32 * ks, ok);
                    const In qf = Op::load_in(a.q, el + 32 * ks, ok);
                    ak = Op::mma(kf, s0f[ks], ak);
                    aq = Op::mma(qf, s0f[ks], aq);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + 4 * lg + e;
                float rv = 0.f, ov = 0.f;
                if (i < T) {
                    const float vv = Op::in_scalar(a.v, base + static_cast<size_t>(i) * rs + col0 + lr);
                    rv = s_beta[i] * (vv - s_P[i] * ak[e]);
                    ov = s_P[i] * aq[e];
                }
                rhs[ti][e] = rv;
                oacc[ti][e] = ov;
            }
        }

#pragma unroll
        for (int c = 0; c <= r; ++c) {
            // ---- a3: masked, decay-weighted Gram block pair (r, c), shared by all waves
            __syncthreads();
            for (int p = wave; p < 16; p += NW) {
                const int ti = p >> 2, tj = p & 3;
                const int i0 = 64 * r + 16 * ti, j0 = 64 * c + 16 * tj;
                const bool need = (i0 < T) && (j0 < T) && (c < r || tj <= ti);
                f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
                if (need) {
                    const int ra = i0 + lr, rb = j0 + lr;
                    const bool oka = ra < T, okb = rb < T;
                    const size_t ea = base + static_cast<size_t>(oka ? ra : 0) * rs + 8 * lg;
                    const size_t eb = base + static_cast<size_t>(okb ? rb : 0) * rs + 8 * lg;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const In ka = Op::load_in(a.k, ea + 32 * ks, oka);
                        const In qa = Op::load_in(a.q, ea + 32 * ks, oka);
                        const In kb = Op::load_in(a.k, eb + 32 * ks, okb);
                        kk = Op::mma(ka, kb, kk);
                        qk = Op::mma(qa, kb, qk);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int il = 16 * ti + 4 * lg + e, jl = 16 * tj + lr;
                    const int i = 64 * r + il, j = 64 * c + jl;
                    float gv = 0.f, cv = 0.f;
                    if (need && i < T && j < T && ((ps.mask[i][j >> 5] >> (j & 31)) & 1u)) {
                        const float gam = expf(static_cast<float>(ps.ell[i] - ps.ell[j]));
                        cv = gam * qk[e];
                        if (i != j) gv = -s_beta[i] * gam * kk[e];
                    }
                    st.store(il, jl, gv, cv);
                }
            }
            __syncthreads();

            if (c < r) {
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
            } else {
                // ---- a4: the diagonal block, per wave on its 16 columns
                const int ib = 64 * r + lane;
                uint64_t bm = 0;
                if (ib < T)
                    bm = (static_cast<uint64_t>(ps.mask[ib][2 * r + 1]) << 32) | ps.mask[ib][2 * r];
                const int ld = (ib < T) ? __popcll(bm) - 1 : -1;
                const int maxld = wave_max(ld);
                if (a.solver == CANOPY_SOLVE_NEUMANN) {
                    f32x4 z[4];
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) z[ti] = rhs[ti];
                    for (int m = 1; m <= maxld; ++m) {
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                            for (int e = 0; e < 4; ++e) X[16 * ti + 4 * lg + e][lr] = z[ti][e];
                        wave_lds_sync();
                        Sp zf[2];
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            float v[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] = X[32 * ks + 8 * lg + e][lr];
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
                        for (int e = 0; e < 4; ++e) X[16 * ti + 4 * lg + e][lr] = rhs[ti][e];
                    wave_lds_sync();
                } else {
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                        for (int e = 0; e < 4; ++e) X[16 * ti + 4 * lg + e][lr] = rhs[ti][e];
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
                                float acc = X[n][lr];
                                while (am) {
                                    const int j = __ffsll(static_cast<unsigned long long>(am)) - 1;
                                    am &= am - 1ull;
                                    acc += st.getG(n, j) * X[j][lr];
                                }
                                X[n][lr] = acc;
                            }
                        }
                        wave_lds_sync();
                    }
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = X[32 * ks + 8 * lg + e][lr];
                    uf[r][ks] = Op::split(v);
                }
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        oacc[ti] = Op::mma(st.fragC(16 * ti + lr, 32 * ks + 8 * lg), uf[r][ks], oacc[ti]);
            }
        }

        // ---- a6: outputs of block r
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int rl = lg + 4 * m;
            const int i = 64 * r + rl;
            if (i < T) a.U[base + static_cast<size_t>(i) * rs + col0 + lr] = X[rl][lr];
        }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 64 * r + 16 * ti + 4 * lg + e;
                if (i < T) a.O[base + static_cast<size_t>(i) * rs + col0 + lr] = oacc[ti][e];
            }
    }
}

template <int NW, bool BF, int NB>
static hipError_t launch_nb(const VerifyArgs &a, hipStream_t stream) {
    const int tiles = D / (16 * NW);
    const dim3 grid(static_cast<unsigned>(a.B * a.H * tiles));
    hipLaunchKernelGGL((verify_kernel<NW, BF, NB>), grid, dim3(NW * 64), 0, stream, a);
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

template <bool BF>
static hipError_t launch_bf(const VerifyArgs &a, int waves, hipStream_t stream) {
    switch (waves) {
        case 1: return launch_nw<1, BF>(a, stream);
        case 2: return launch_nw<2, BF>(a, stream);
        case 4: return launch_nw<4, BF>(a, stream);
        default: return launch_nw<8, BF>(a, stream);
    }
}

hipError_t launch_verify(const VerifyArgs &a, int waves, hipStream_t stream) {
    return a.bf16 ? launch_bf<true>(a, waves, stream) : launch_bf<false>(a, waves, stream);
}

}  // namespace canopy
