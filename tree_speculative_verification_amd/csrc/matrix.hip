// Matrix-form solves of the tree system, with the operators of each (sequence, head) built once
// in a caller-supplied workspace ("Design decisions / Two solve strategies" and "Batch and heads
// to CTAs" on the canopy project page; "The tree closed form" for the series and its squaring
// form). Three solvers share the launches:
//   mat_prep_kernel   per (sequence, head): tree prep, N = -G and C (T x T, fp32, row-major
//                     and, for N, column-major too) into the workspace, R into U and
//                     diag(P) Q S0 into O (both overwritten later), the tree depth d
//   mat_square_kernel per (sequence, head), SQUARING and SPLIT only: the powers
//                     P_k = N^(2^k), k < K = ceil(log2(d + 1)); SPLIT also multiplies out
//                     M = (I + N)(I + N^2) ... (I + N^(2^(K-1))) = (I + G)^-1
//   mat_apply_kernel  per (sequence, head, 16 value columns):
//                     SERIES    Z <- N Z, U <- U + Z for d rounds (Bole's finite series)
//                     SQUARING  Z <- Z + P_k Z for k < K (the squaring form)
//                     SPLIT     U = M R (the split design: inverse built once, applied per
//                               value tile)
//                     then O = diag(P) Q S0 + C U.
// With bf16 inputs the products run on v_mfma_f32_16x16x32_bf16, fp32 operands split into bf16
// hi + lo parts (three passes); with fp32 inputs every product runs on fp32 MFMA (exact
// products), as the other fp32 paths do. Accumulation is fp32.
#include <mutex>

#include "canopy_kernels.hpp"
#include "canopy_prep.hpp"

namespace canopy {

namespace {

constexpr int MNT = 512;  // threads of the per-head kernels (8 waves)
constexpr int ANT = 256;  // threads of the apply kernel (4 waves)
constexpr int HDR = 64;   // header bytes per (sequence, head): bad, d, K, tiles

// Matrices of one (sequence, head) in its workspace slot, each Tp x Tp fp32 (Tp: T rounded up
// to 16). Slot layout: header | N | N^T | C | solver part.
struct MatSlot {
    int *hdr;
    float *N, *Nt, *C, *ext;
};
__host__ __device__ inline size_t mat_tp(int T) { return static_cast<size_t>((T + 15) / 16 * 16); }
__host__ __device__ inline int mat_kmax(int T) {
    int k = 0;
    while ((1 << k) < T) ++k;  // K = ceil(log2(d + 1)) <= ceil(log2(T)) as d <= T - 1
    return k;
}
// Matrices past the first three: SQUARING keeps P_1 .. P_{K-1} (row-major) and two column-major
// buffers for the squarings; SPLIT keeps two P, two P^T, two M and two M^T buffers.
__host__ __device__ inline int mat_extra(int solver, int T) {
    if (solver == CANOPY_SOLVE_SQUARING) return (mat_kmax(T) > 1 ? mat_kmax(T) - 1 : 0) + 2;
    if (solver == CANOPY_SOLVE_SPLIT) return 8;
    return 0;
}
__host__ __device__ inline size_t mat_slot_bytes(int solver, int T) {
    const size_t tp = mat_tp(T);
    return HDR + (3 + mat_extra(solver, T)) * tp * tp * 4;
}
__device__ inline MatSlot mat_slot(void *ws, int solver, int T, int bh) {
    const size_t tp = mat_tp(T);
    uint8_t *p = static_cast<uint8_t *>(ws) + static_cast<size_t>(bh) * mat_slot_bytes(solver, T);
    MatSlot s;
    s.hdr = reinterpret_cast<int *>(p);
    float *m = reinterpret_cast<float *>(p + HDR);
    s.N = m;
    s.Nt = m + tp * tp;
    s.C = m + 2 * tp * tp;
    s.ext = m + 3 * tp * tp;
    return s;
}

// 8 consecutive fp32 values at p (32-byte aligned), or zeros.
__device__ __forceinline__ void ld8(const float *p, bool ok, float (&v)[8]) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (ok) {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Tile (it, jt) of X Y accumulated over the 16-wide reduction tiles s0 .. s1, X row-major and Y
// given column-major (rows of Y^T), both Tp x Tp. A 32-long MFMA slice takes reduction tiles
// s and s + 1; lane (lg, lr) supplies row 16it + lr of X and column 16jt + lr of Y at indices
// 16s + 8lg .. +7. The result holds Z[16it + 4lg + e][16jt + lr] in lane (lg, lr).
template <bool BF>
__device__ __forceinline__ f32x4 tile_mm(const float *X, const float *Yt, size_t tp, int it, int jt,
                                         int s0, int s1, int lr, int lg, f32x4 acc) {
    using Op = Ops<BF>;
    const float *xr = X + (16 * it + lr) * tp;
    const float *yr = Yt + (16 * jt + lr) * tp;
    for (int s = s0; s <= s1; s += 2) {
        const int k = 16 * s + 8 * lg;
        const bool ok = k < 16 * (s1 + 1);
        float a[8], b[8];
        ld8(xr + k, ok, a);
        ld8(yr + k, ok, b);
        acc = Op::mma(Op::split(a), Op::split(b), acc);
    }
    return acc;
}

// Store a result tile held as Z[16it + 4lg + e][16jt + lr] into a row-major matrix (if Z is
// given) and a column-major one (if Zt is given).
__device__ __forceinline__ void tile_store(float *Z, float *Zt, size_t tp, int it, int jt, int lr, int lg,
                                           f32x4 v) {
    if (Zt)
        *reinterpret_cast<float4 *>(Zt + (16 * jt + lr) * tp + 16 * it + 4 * lg) = make_float4(v[0], v[1], v[2], v[3]);
    if (Z)
#pragma unroll
        for (int e = 0; e < 4; ++e) Z[(16 * it + 4 * lg + e) * tp + 16 * jt + lr] = v[e];
}

}  // namespace

size_t mat_workspace_bytes(int B, int H, int T, int solver) {
    if (solver != CANOPY_SOLVE_SERIES && solver != CANOPY_SOLVE_SQUARING && solver != CANOPY_SOLVE_SPLIT)
        return 0;
    return static_cast<size_t>(B) * H * mat_slot_bytes(solver, T);
}

// ---------------------------------------------------------------------------------------------
// Per (sequence, head): prep, the operators N = -G and C, R (into U) and diag(P) Q S0 (into O).
template <bool BF>
__global__ __launch_bounds__(MNT) void mat_prep_kernel(VerifyArgs a, void *ws) {
    using Op = Ops<BF>;
    using In = typename Op::In;
    using Sp = typename Op::Sp;
    constexpr int MAXT = 256;
    __shared__ PrepSmem<MAXT> ps;
    __shared__ float s_beta[MAXT], s_P[MAXT];
    __shared__ int s_depth;

    const int bh = xcd_remap(blockIdx.x, gridDim.x);
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;
    const size_t qkrs = static_cast<size_t>(a.HK) * D;
    const size_t qkbase = qk_base(b, h, H, a.HK, T);
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;
    const size_t tp = mat_tp(T);
    const MatSlot slot = mat_slot(ws, a.solver, T, bh);

    const int pbad = tree_prep_block<MAXT, MNT>(ps, a.parent + static_cast<size_t>(b) * T, a.alpha + sbase, H, T, Tb);
    const int bad = sl.bad ? -1 : pbad;
    if (tid == 0) {
        slot.hdr[0] = bad;
        s_depth = 0;
    }
    if (bad) {
        const float qnan = __builtin_nanf("");
        for (int x = tid; x < Tb * D; x += MNT) {
            const size_t o = base + static_cast<size_t>(x / D) * rs + x % D;
            a.O[o] = qnan;
            a.U[o] = qnan;
        }
        for (int i = tid; i < Tb; i += MNT) a.ell[sbase + static_cast<size_t>(i) * H] = qnan;
        if (h == 0) {
            const int W = (T + 31) >> 5;
            if (a.tree_status && tid == 0) a.tree_status[b] = bad;
            if (a.depth)
                for (int i = tid; i < Tb; i += MNT) a.depth[static_cast<size_t>(b) * T + i] = 0;
            if (a.anc_mask)
                for (int x = tid; x < Tb * W; x += MNT) a.anc_mask[static_cast<size_t>(b) * T * W + x] = 0u;
        }
        return;
    }
    __syncthreads();
    for (int i = tid; i < MAXT; i += MNT) {
        float P = 0.f, bt = 0.f;
        if (i < Tb) {
            P = __builtin_amdgcn_exp2f(static_cast<float>(ps.ell[i]));
            bt = a.beta[sbase + static_cast<size_t>(i) * H];
            a.ell[sbase + static_cast<size_t>(i) * H] = static_cast<float>(ps.ell[i] * 0.69314718055994530942);
            atomicMax(&s_depth, node_depth<MAXT>(ps, i));
        }
        s_beta[i] = bt;
        s_P[i] = P;
    }
    if (h == 0) {
        const int W = (T + 31) >> 5;
        if (a.tree_status && tid == 0) a.tree_status[b] = 0;
        for (int i = tid; i < Tb; i += MNT) {
            if (a.depth) a.depth[static_cast<size_t>(b) * T + i] = node_depth<MAXT>(ps, i);
            if (a.anc_mask)
                for (int w = 0; w < W; ++w) a.anc_mask[(static_cast<size_t>(b) * T + i) * W + w] = ps.mask[i][w];
        }
    }
    __syncthreads();
    const int nt = (Tb + 15) / 16;  // 16-node tiles of the sequence: the operators' extent
    if (tid == 0) {
        slot.hdr[1] = s_depth;
        slot.hdr[3] = nt;
    }

    // ---- N = -G and C, tile (it, jt), jt <= it: K_j as the A operand and K_i / Q_i as B, so
    // that lane (lg, lr) ends with row i = 16it + lr, columns j = 16jt + 4lg + e.
    const int ntiles = nt * (nt + 1) / 2;
    for (int t = wave; t < ntiles; t += MNT / 64) {
        int it = 0;
        while ((it + 1) * (it + 2) / 2 <= t) ++it;
        const int jt = t - it * (it + 1) / 2;
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
        const size_t rj = qkbase + static_cast<size_t>(min(16 * jt + lr, T - 1)) * qkrs + 8 * lg;
        const size_t ri = qkbase + static_cast<size_t>(min(16 * it + lr, T - 1)) * qkrs + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const In kj = Op::template load_frag<In>(a.k, rj + 32 * ks, true);
            const In ki = Op::template load_frag<In>(a.k, ri + 32 * ks, true);
            const In qi = Op::template load_frag<In>(a.q, ri + 32 * ks, true);
            kk = Op::mma(kj, ki, kk);
            qk = Op::mma(kj, qi, qk);
        }
        const int i = 16 * it + lr, j0 = 16 * jt + 4 * lg;
        const uint32_t bits = (ps.mask[i][j0 >> 5] >> (j0 & 31)) & 0xFu;
        const double li = ps.ell[i];
        const float bi = s_beta[i];
        float nv[4], cv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // exp(l_i - l_j) from the fp64 log2 path sums; off the path the selects drop it
            const float gam = __builtin_amdgcn_exp2f(static_cast<float>(li - ps.ell[j0 + e]));
            const bool on = (bits >> e) & 1u;
            cv[e] = on ? gam * qk[e] : 0.f;
            nv[e] = (on && i != j0 + e) ? -bi * gam * kk[e] : 0.f;
        }
        *reinterpret_cast<float4 *>(slot.N + i * tp + j0) = make_float4(nv[0], nv[1], nv[2], nv[3]);
        *reinterpret_cast<float4 *>(slot.C + i * tp + j0) = make_float4(cv[0], cv[1], cv[2], cv[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) slot.Nt[(j0 + e) * tp + i] = nv[e];
    }

    // ---- R = beta (V - P K S0) into U and diag(P) Q S0 into O; wave w owns columns 16w ..
    const int col0 = 16 * wave;
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
    for (int it = 0; it < nt; ++it) {
        f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
        const size_t ri = qkbase + static_cast<size_t>(min(16 * it + lr, T - 1)) * qkrs + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const In kf = Op::template load_frag<In>(a.k, ri + 32 * ks, true);
            const In qf = Op::template load_frag<In>(a.q, ri + 32 * ks, true);
            ak = Op::mma(kf, s0f[ks], ak);
            aq = Op::mma(qf, s0f[ks], aq);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * lg + e;
            if (i < Tb) {
                const size_t o = base + static_cast<size_t>(i) * rs + col0 + lr;
                const float v = Op::in_scalar(a.v, o);
                a.U[o] = s_beta[i] * (v - s_P[i] * ak[e]);
                a.O[o] = s_P[i] * aq[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Per (sequence, head), SQUARING and SPLIT: the powers P_k = N^(2^k), and for SPLIT the product
// M = (I + P_0)(I + P_1) ... (I + P_{K-1}). Lower tiles only (every factor is lower triangular);
// the squarings and the product steps alternate with workgroup barriers, since every tile of a
// step reads tiles of the step before.
template <bool BF>
__global__ __launch_bounds__(MNT) void mat_square_kernel(int solver, int B, int H, int T, void *ws) {
    const int bh = xcd_remap(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const size_t tp = mat_tp(T);
    const size_t mm = tp * tp;
    const MatSlot slot = mat_slot(ws, solver, T, bh);
    if (slot.hdr[0] != 0) return;  // malformed tree: outputs are already NaN
    const int d = slot.hdr[1];
    int K = 0;
    while ((1 << K) <= d) ++K;  // ceil(log2(d + 1)) factors
    const int nt = slot.hdr[3];  // only the sequence's tiles were written
    const int ntiles = nt * (nt + 1) / 2;
    auto tile_of = [&](int t, int &it, int &jt) __attribute__((always_inline)) {
        it = 0;
        while ((it + 1) * (it + 2) / 2 <= t) ++it;
        jt = t - it * (it + 1) / 2;
    };
    const bool split = solver == CANOPY_SOLVE_SPLIT;
    // P_k row-major and column-major; SQUARING keeps every P_k row-major for the apply
    // (P_0 = N), SPLIT keeps only the latest power and the latest M.
    float *Pr[2], *Pc[2], *Mr[2], *Mc[2];
    if (split) {
        for (int x = 0; x < 2; ++x) {
            Pr[x] = slot.ext + (2 * x) * mm;
            Pc[x] = slot.ext + (2 * x + 1) * mm;
            Mr[x] = slot.ext + (4 + 2 * x) * mm;
            Mc[x] = slot.ext + (5 + 2 * x) * mm;
        }
        // M_0 = I + N in both layouts (lower tiles)
        for (int t = wave; t < ntiles; t += MNT / 64) {
            int it, jt;
            tile_of(t, it, jt);
            const int i = 16 * it + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * jt + 4 * lg + e;
                const float v = slot.N[i * tp + j] + (i == j ? 1.f : 0.f);
                Mr[0][i * tp + j] = v;
                Mc[0][j * tp + i] = v;
            }
        }
    }
    const float *prev_r = slot.N, *prev_c = slot.Nt;
    for (int k = 1; k < K; ++k) {
        __syncthreads();
        // P_k = P_{k-1} P_{k-1}
        float *out_r = split ? Pr[k & 1] : slot.ext + 2 * mm + static_cast<size_t>(k - 1) * mm;
        float *out_c = split ? Pc[k & 1] : slot.ext + static_cast<size_t>(k & 1) * mm;
        for (int t = wave; t < ntiles; t += MNT / 64) {
            int it, jt;
            tile_of(t, it, jt);
            f32x4 acc = tile_mm<BF>(prev_r, prev_c, tp, it, jt, jt, it, lr, lg, f32x4{0.f, 0.f, 0.f, 0.f});
            tile_store(out_r, out_c, tp, it, jt, lr, lg, acc);
        }
        prev_r = out_r;
        prev_c = out_c;
        if (split) {
            __syncthreads();
            // M <- M + P_k M, both layouts
            const float *mr = Mr[(k - 1) & 1], *mc = Mc[(k - 1) & 1];
            for (int t = wave; t < ntiles; t += MNT / 64) {
                int it, jt;
                tile_of(t, it, jt);
                f32x4 acc = tile_mm<BF>(prev_r, mc, tp, it, jt, jt, it, lr, lg, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += mr[(16 * it + 4 * lg + e) * tp + 16 * jt + lr];
                tile_store(Mr[k & 1], Mc[k & 1], tp, it, jt, lr, lg, acc);
            }
        }
    }
    if (split && tid == 0) slot.hdr[2] = K;
}

// ---------------------------------------------------------------------------------------------
// Per (sequence, head, 16 value columns): the solve on the workgroup's R columns (read from U)
// and the read-out O = diag(P) Q S0 (read from O) + C U. Node-by-column blocks Z sit in LDS
// column-major (zs[column][row]), as the B operand of 32-long reductions.
template <bool BF>
__global__ __launch_bounds__(ANT) void mat_apply_kernel(int solver, int B, int H, int T, const int32_t *tree_len,
                                                          float *U, float *O, void *ws) {
    using Op = Ops<BF>;
    constexpr int ZS = 256 + 8;  // column stride of the LDS blocks (floats)
    __shared__ __attribute__((aligned(16))) float zs[2][16][ZS];
    __shared__ __attribute__((aligned(16))) float us[16][ZS];
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = g % 8, bh = g / 8;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const size_t tp = mat_tp(T);
    const size_t mm = tp * tp;
    const MatSlot slot = mat_slot(ws, solver, T, bh);
    if (slot.hdr[0] != 0) return;
    const int d = slot.hdr[1];
    const SeqLen sl = seq_len(tree_len, b, T);
    const int Tb = sl.n;
    const int nt = (Tb + 15) / 16;
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D + 16 * tile;
    constexpr int NWV = ANT / 64;

    // R (and the starting Z) into LDS: rows past the sequence are zero
    for (int x = tid; x < 16 * static_cast<int>(tp); x += ANT) {
        const int row = x / 16, c = x % 16;
        const float v = row < Tb ? U[base + static_cast<size_t>(row) * rs + c] : 0.f;
        zs[0][c][row] = v;
        us[c][row] = v;
    }
    __syncthreads();

    // One product round: Zout = A Zin (+ Zin when add), for the row tiles of this wave; with
    // acc_u the result is also added to U. A is row-major, lower triangular by tiles.
    auto round = [&](const float *A, int src, int dst, bool add, bool acc_u) __attribute__((always_inline)) {
        for (int it = wave; it < nt; it += NWV) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const float *ar = A + (16 * it + lr) * tp;
            for (int s = 0; s <= it; s += 2) {
                const int k = 16 * s + 8 * lg;
                const bool ok = k < 16 * (it + 1);
                float av[8], zv[8];
                ld8(ar + k, ok, av);
                const float4 z0 = ok ? *reinterpret_cast<const float4 *>(&zs[src][lr][k]) : make_float4(0.f, 0.f, 0.f, 0.f);
                const float4 z1 = ok ? *reinterpret_cast<const float4 *>(&zs[src][lr][k + 4]) : make_float4(0.f, 0.f, 0.f, 0.f);
                zv[0] = z0.x; zv[1] = z0.y; zv[2] = z0.z; zv[3] = z0.w;
                zv[4] = z1.x; zv[5] = z1.y; zv[6] = z1.z; zv[7] = z1.w;
                acc = Op::mma(Op::split(av), Op::split(zv), acc);
            }
            const int r0 = 16 * it + 4 * lg;
            float4 o = make_float4(acc[0], acc[1], acc[2], acc[3]);
            if (add) {
                const float4 zin = *reinterpret_cast<const float4 *>(&zs[src][lr][r0]);
                o.x += zin.x; o.y += zin.y; o.z += zin.z; o.w += zin.w;
            }
            *reinterpret_cast<float4 *>(&zs[dst][lr][r0]) = o;
            if (acc_u) {
                float4 u = *reinterpret_cast<const float4 *>(&us[lr][r0]);
                u.x += o.x; u.y += o.y; u.z += o.z; u.w += o.w;
                *reinterpret_cast<float4 *>(&us[lr][r0]) = u;
            }
        }
    };

    int cur = 0;
    if (solver == CANOPY_SOLVE_SERIES) {
        // Bole's finite series: U = sum_{m=0..d} N^m R, one product per tree level
        for (int m = 1; m <= d; ++m) {
            round(slot.N, cur, cur ^ 1, false, true);
            cur ^= 1;
            __syncthreads();
        }
    } else if (solver == CANOPY_SOLVE_SQUARING) {
        // Z <- (I + P_k) Z for k < K: the first 2^K >= d + 1 terms of the series
        int K = 0;
        while ((1 << K) <= d) ++K;
        for (int k = 0; k < K; ++k) {
            const float *Pk = k == 0 ? slot.N : slot.ext + 2 * mm + static_cast<size_t>(k - 1) * mm;
            round(Pk, cur, cur ^ 1, true, false);
            cur ^= 1;
            __syncthreads();
        }
        for (int x = tid; x < 16 * static_cast<int>(tp); x += ANT) us[x / static_cast<int>(tp)][x % tp] = zs[cur][x / tp][x % tp];
        __syncthreads();
    } else {
        // the split design: U = M R with M = (I + G)^-1 built once per (sequence, head)
        const int K = slot.hdr[2];
        const float *M = slot.ext + (4 + 2 * ((K - 1) & 1)) * mm;
        if (K > 0) {
            round(M, cur, cur ^ 1, false, false);
            cur ^= 1;
            __syncthreads();
            for (int x = tid; x < 16 * static_cast<int>(tp); x += ANT) us[x / static_cast<int>(tp)][x % tp] = zs[cur][x / tp][x % tp];
            __syncthreads();
        }
    }

    // ---- outputs: U, and O = diag(P) Q S0 + C U
    for (int it = wave; it < nt; it += NWV) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const float *cr = slot.C + (16 * it + lr) * tp;
        for (int s = 0; s <= it; s += 2) {
            const int k = 16 * s + 8 * lg;
            const bool ok = k < 16 * (it + 1);
            float cv[8], uv[8];
            ld8(cr + k, ok, cv);
            const float4 u0 = ok ? *reinterpret_cast<const float4 *>(&us[lr][k]) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 u1 = ok ? *reinterpret_cast<const float4 *>(&us[lr][k + 4]) : make_float4(0.f, 0.f, 0.f, 0.f);
            uv[0] = u0.x; uv[1] = u0.y; uv[2] = u0.z; uv[3] = u0.w;
            uv[4] = u1.x; uv[5] = u1.y; uv[6] = u1.z; uv[7] = u1.w;
            acc = Op::mma(Op::split(cv), Op::split(uv), acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * lg + e;
            if (i < Tb) {
                const size_t o = base + static_cast<size_t>(i) * rs + lr;
                U[o] = us[lr][i];
                store_nt(O + o, O[o] + acc[e]);
            }
        }
    }
}

// The workspace of canopy_tree_verify_static, for callers that cannot allocate: one array per
// device, held until the process ends and shared by every call on that device (so calls that
// overlap on one device race). The matrix-form kernels write every workspace word they read
// before reading it, so its contents from an earlier call never matter.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// The device address of this device's scratch array, looked up once per device with that
// device current (host code must not use the symbol itself as an address).
hipError_t mat_static_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *dev_ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    return hipSuccess;
}

hipError_t launch_verify_matrix(const VerifyArgs &a, void *ws, hipStream_t stream) {
    const unsigned heads = static_cast<unsigned>(a.B * a.H);
    const bool sq = a.solver == CANOPY_SOLVE_SQUARING || a.solver == CANOPY_SOLVE_SPLIT;
    if (a.bf16) {
        hipLaunchKernelGGL((mat_prep_kernel<true>), dim3(heads), dim3(MNT), 0, stream, a, ws);
        if (sq) hipLaunchKernelGGL((mat_square_kernel<true>), dim3(heads), dim3(MNT), 0, stream, a.solver, a.B, a.H, a.T, ws);
        hipLaunchKernelGGL((mat_apply_kernel<true>), dim3(heads * 8), dim3(ANT), 0, stream, a.solver, a.B, a.H,
                           a.T, a.tree_len, a.U, a.O, ws);
    } else {
        hipLaunchKernelGGL((mat_prep_kernel<false>), dim3(heads), dim3(MNT), 0, stream, a, ws);
        if (sq) hipLaunchKernelGGL((mat_square_kernel<false>), dim3(heads), dim3(MNT), 0, stream, a.solver, a.B, a.H, a.T, ws);
        hipLaunchKernelGGL((mat_apply_kernel<false>), dim3(heads * 8), dim3(ANT), 0, stream, a.solver, a.B, a.H,
                           a.T, a.tree_len, a.U, a.O, ws);
    }
    return hipGetLastError();
}

}  // namespace canopy
