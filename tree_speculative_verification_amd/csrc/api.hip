// The C ABI of libcanopy (declared in include/canopy.h): host-side argument checks, the launch
// configuration, and nothing else. Every call only enqueues kernels on the caller's stream.
#include <atomic>

#include "canopy_device.hpp"
#include "canopy_kernels.hpp"

using namespace canopy;

namespace {

// Grids have up to B*H*8 workgroups and index arithmetic on (b, h) pairs is 32-bit: keep
// B*H*256 within int range.
bool sizes_ok(int B, int H, int T) {
    return B >= 1 && H >= 1 && T >= 1 && T <= 256 &&
           static_cast<long long>(B) * H * 256 <= 2147483647LL;
}

// q/k heads H and value heads HV: each q/k head serves HV / H value heads.
bool heads_ok(int H, int HV) { return H >= 1 && HV >= H && HV % H == 0; }

// Bound of the waits of one wave for another wave's result (see canopy_set_wait_bound).
std::atomic<int> g_wait_bound{kWaitBound};

canopy_status from_hip(hipError_t e) { return e == hipSuccess ? CANOPY_OK : CANOPY_ERR_HIP; }

// Kernels move 16-byte vectors of these arrays; a misaligned view is rejected on the host.
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Waves per workgroup (16 value columns each) for the verify kernel. One workgroup per
// (sequence, head) with all 128 columns (8 waves) measured fastest on MI355X at every size of
// the benchmark (B = 1..16, T = 16..256): the per-workgroup chain of dependent phases sets the
// time, and narrower tiles repeat the shared Gram work without shortening that chain.
// fp32 inputs stage twice the bytes per block and use 2 waves.
int pick_waves(canopy_dtype dt) { return dt == CANOPY_BF16 ? 8 : 2; }

// Up to this many (sequence, head) pairs the wave-per-sub-block kernel runs trees of 65 to 256
// nodes (1, 2 or 4 column tiles per workgroup at up to 32, 64 and 128 pairs); beyond, the
// blocked kernel's single Gram pass per head wins. Measured on MI355X at B = 4, H = 32: T = 256
// 45.1 us with 4 column tiles against 55.6 us blocked, T = 128 23.8 against 26.9 us.
constexpr long long kWideMaxHeads = 128;

// Beyond this many (sequence, head) pairs (more workgroups than CUs, so the one-per-CU blocked
// kernel would run a second pass) trees of 65 to 256 nodes run the blocked solve sized for two
// workgroups per CU. Measured on MI355X at H = 32, T = 256: B = 16 103-108 us against 115 us
// for the blocked kernel; at B = 8 (256 pairs) the blocked kernel's single pass wins, 60 us
// against 73 us.
constexpr long long kDualMinHeads = 257;

}  // namespace

extern "C" {

int canopy_version(void) { return 200; }

int canopy_set_wait_bound(int sleeps) {
    return g_wait_bound.exchange(sleeps < 0 ? kWaitBound : sleeps, std::memory_order_relaxed);
}

const char *canopy_status_string(canopy_status s) {
    switch (s) {
        case CANOPY_OK: return "ok";
        case CANOPY_ERR_ARG: return "invalid argument (null pointer or size out of range)";
        case CANOPY_ERR_UNSUPPORTED: return "unsupported dtype, solver or waves value";
        case CANOPY_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case CANOPY_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

canopy_status canopy_tree_prep(const int32_t *parent, const int32_t *tree_len, const float *alpha,
                               int B, int HV, int T, uint32_t *anc_mask, int32_t *depth, float *ell,
                               int32_t *tree_status, hipStream_t stream) {
    if (!parent || !alpha || !sizes_ok(B, HV, T)) return CANOPY_ERR_ARG;
    PrepArgs a{parent, tree_len, alpha, B, HV, T, anc_mask, depth, ell, tree_status};
    return from_hip(launch_prep(a, stream));
}

canopy_status canopy_tree_verify(const void *q, const void *k, const void *v,
                                 const float *alpha, const float *beta, const float *S0,
                                 const int32_t *parent, const int32_t *tree_len, int B, int H,
                                 int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                 float *ell, uint32_t *anc_mask, int32_t *depth,
                                 int32_t *tree_status, canopy_solver solver, int waves,
                                 hipStream_t stream) {
    if (!q || !k || !v || !alpha || !beta || !S0 || !parent || !O || !U || !ell)
        return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T) || !heads_ok(H, HV)) return CANOPY_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S0)) return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    if (solver != CANOPY_SOLVE_AUTO && solver != CANOPY_SOLVE_FWDSUB &&
        solver != CANOPY_SOLVE_NEUMANN && solver != CANOPY_SOLVE_LEVEL && solver != CANOPY_SOLVE_LEVELSYNC)
        return CANOPY_ERR_UNSUPPORTED;
    if (waves != 0 && waves != 1 && waves != 2 && waves != 4 && waves != 8 && waves != 16)
        return CANOPY_ERR_UNSUPPORTED;
    if (solver == CANOPY_SOLVE_LEVELSYNC && (in_dtype != CANOPY_BF16 || (waves != 0 && waves != 8)))
        return CANOPY_ERR_UNSUPPORTED;
    // 16: two column tiles per wave for trees of at most 16 nodes (AUTO, NEUMANN); the
    // two-per-CU blocked kernel for bf16 trees of 65 to 256 nodes (AUTO, FWDSUB).
    if (waves == 16 && !(T <= 16 && (solver == CANOPY_SOLVE_AUTO || solver == CANOPY_SOLVE_NEUMANN)) &&
        (in_dtype != CANOPY_BF16 || T <= 64 || !dual_fits(H, HV, T) ||
         (solver != CANOPY_SOLVE_AUTO && solver != CANOPY_SOLVE_FWDSUB)))
        return CANOPY_ERR_UNSUPPORTED;
    VerifyArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta; a.S0 = S0; a.parent = parent; a.tree_len = tree_len;
    a.B = B; a.H = HV; a.HK = H; a.T = T;
    a.bf16 = in_dtype == CANOPY_BF16;
    a.solver = solver;
    a.O = O; a.U = U; a.ell = ell;
    a.anc_mask = anc_mask; a.depth = depth; a.tree_status = tree_status;
    a.wait_bound = g_wait_bound.load(std::memory_order_relaxed);
    // Trees of at most 16 nodes fit one MFMA tile: AUTO and NEUMANN run the single-wave
    // register kernel (Neumann series in registers). Trees of 17 to 64 nodes run the
    // wave-per-sub-block kernel for AUTO, FWDSUB and NEUMANN. Everything else (LEVEL, and
    // FWDSUB at T <= 16) runs the blocked LDS kernel, which serves any T <= 256.
    if (solver == CANOPY_SOLVE_LEVELSYNC) return from_hip(launch_verify(a, 8, stream));
    if (T <= 16 && (solver == CANOPY_SOLVE_AUTO || solver == CANOPY_SOLVE_NEUMANN))
        return from_hip(launch_verify_small(a, waves, stream));
    if (T > 16 && T <= 64 && solver != CANOPY_SOLVE_LEVEL)
        return from_hip(launch_verify_mid(a, waves == 8 ? 4 : waves, stream));
    // Trees of 65 to 256 nodes with bf16 inputs, AUTO or FWDSUB: the wave-per-sub-block kernel
    // (one workgroup per head and 16 to 64 value columns) while there are few heads, the
    // blocked kernel (one workgroup per head and all columns, no repeated Gram work) beyond,
    // and past one workgroup per CU the blocked solve sized for two workgroups per CU.
    // An explicit width picks the kernel: 1 or 2 column tiles, 4 or 8 blocked waves, or 16
    // for the two-per-CU blocked kernel.
    if (T > 64 && in_dtype == CANOPY_BF16 &&
        (solver == CANOPY_SOLVE_AUTO || solver == CANOPY_SOLVE_FWDSUB)) {
        if (waves == 1 || waves == 2) return from_hip(launch_verify_wide(a, waves, stream));
        if (waves == 16) return from_hip(launch_verify_dual(a, stream));
        if (waves == 0) {
            const long long heads = static_cast<long long>(B) * HV;
            if (heads <= kWideMaxHeads)
                return from_hip(launch_verify_wide(a, heads <= 32 ? 1 : (heads <= 64 ? 2 : 4), stream));
            if (heads >= kDualMinHeads && dual_fits(H, HV, T)) return from_hip(launch_verify_dual(a, stream));
        }
    }
    return from_hip(launch_verify(a, waves ? waves : pick_waves(in_dtype), stream));
}

size_t canopy_workspace_bytes(int B, int HV, int T, canopy_solver solver) {
    if (!sizes_ok(B, HV, T)) return 0;
    return mat_workspace_bytes(B, HV, T, solver);
}

canopy_status canopy_tree_verify_ws(const void *q, const void *k, const void *v,
                                    const float *alpha, const float *beta, const float *S0,
                                    const int32_t *parent, const int32_t *tree_len, int B, int H,
                                    int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                    float *ell, uint32_t *anc_mask, int32_t *depth,
                                    int32_t *tree_status, canopy_solver solver, int waves,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (solver != CANOPY_SOLVE_SERIES && solver != CANOPY_SOLVE_SQUARING && solver != CANOPY_SOLVE_SPLIT)
        return canopy_tree_verify(q, k, v, alpha, beta, S0, parent, tree_len, B, H, HV, T, in_dtype, O, U,
                                  ell, anc_mask, depth, tree_status, solver, waves, stream);
    if (!q || !k || !v || !alpha || !beta || !S0 || !parent || !O || !U || !ell)
        return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T) || !heads_ok(H, HV)) return CANOPY_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S0)) return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    if (!workspace || !aligned16(workspace) || workspace_bytes < mat_workspace_bytes(B, HV, T, solver))
        return CANOPY_ERR_WORKSPACE;
    VerifyArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta; a.S0 = S0; a.parent = parent; a.tree_len = tree_len;
    a.B = B; a.H = HV; a.HK = H; a.T = T;
    a.bf16 = in_dtype == CANOPY_BF16;
    a.solver = solver;
    a.O = O; a.U = U; a.ell = ell;
    a.anc_mask = anc_mask; a.depth = depth; a.tree_status = tree_status;
    a.wait_bound = g_wait_bound.load(std::memory_order_relaxed);
    return from_hip(launch_verify_matrix(a, workspace, stream));
}

canopy_status canopy_tree_verify_static(const void *q, const void *k, const void *v,
                                        const float *alpha, const float *beta, const float *S0,
                                        const int32_t *parent, const int32_t *tree_len, int B,
                                        int H, int HV, int T, canopy_dtype in_dtype, float *O,
                                        float *U, float *ell, uint32_t *anc_mask, int32_t *depth,
                                        int32_t *tree_status, canopy_solver solver, int waves,
                                        hipStream_t stream) {
    if (solver != CANOPY_SOLVE_SERIES && solver != CANOPY_SOLVE_SQUARING && solver != CANOPY_SOLVE_SPLIT)
        return canopy_tree_verify(q, k, v, alpha, beta, S0, parent, tree_len, B, H, HV, T, in_dtype, O, U,
                                  ell, anc_mask, depth, tree_status, solver, waves, stream);
    if (!sizes_ok(B, HV, T)) return CANOPY_ERR_ARG;
    const size_t need = mat_workspace_bytes(B, HV, T, solver);
    if (need > kStaticScratchBytes) return CANOPY_ERR_WORKSPACE;
    void *ws = nullptr;
    if (mat_static_scratch(&ws) != hipSuccess) return CANOPY_ERR_HIP;
    return canopy_tree_verify_ws(q, k, v, alpha, beta, S0, parent, tree_len, B, H, HV, T, in_dtype, O, U,
                                 ell, anc_mask, depth, tree_status, solver, waves, ws, kStaticScratchBytes,
                                 stream);
}

canopy_status canopy_commit(const float *S0, const void *k, canopy_dtype in_dtype,
                            const float *U, const float *alpha, const int32_t *parent,
                            const int32_t *tree_len, const int32_t *path, const int32_t *path_len,
                            int B, int H, int HV, int T, float *S_new, int32_t *path_status,
                            hipStream_t stream) {
    if (!S0 || !k || !U || !alpha || !parent || !path || !path_len || !S_new) return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T) || !heads_ok(H, HV)) return CANOPY_ERR_ARG;
    if (!aligned16(S0) || !aligned16(k) || !aligned16(U) || !aligned16(S_new)) return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    CommitArgs a{S0, k, in_dtype == CANOPY_BF16, U, alpha, parent, tree_len, path, path_len,
                 B, HV, H, T, S_new, path_status};
    return from_hip(launch_commit(a, stream));
}

canopy_status canopy_commit_verify(const float *S0, const void *k_prev, const float *U_prev,
                                   const float *alpha_prev, const int32_t *parent_prev,
                                   const int32_t *tree_len_prev, const int32_t *path,
                                   const int32_t *path_len, int T_prev, const void *q,
                                   const void *k, const void *v, const float *alpha,
                                   const float *beta, const int32_t *parent,
                                   const int32_t *tree_len, int B, int H, int HV, int T,
                                   canopy_dtype in_dtype, float *S_new, int32_t *path_status,
                                   float *O, float *U, float *ell, uint32_t *anc_mask,
                                   int32_t *depth, int32_t *tree_status, canopy_solver solver,
                                   int waves, hipStream_t stream) {
    // The commit's own checks (on the previous tree's sizes), then the verify's, which reads
    // the committed state.
    if (!S0 || !k_prev || !U_prev || !alpha_prev || !parent_prev || !path || !path_len || !S_new)
        return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T_prev) || !heads_ok(H, HV)) return CANOPY_ERR_ARG;
    if (!aligned16(S0) || !aligned16(k_prev) || !aligned16(U_prev) || !aligned16(S_new))
        return CANOPY_ERR_ARG;
    if (!q || !k || !v || !alpha || !beta || !parent || !O || !U || !ell) return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T)) return CANOPY_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    if (solver != CANOPY_SOLVE_AUTO && solver != CANOPY_SOLVE_FWDSUB &&
        solver != CANOPY_SOLVE_NEUMANN && solver != CANOPY_SOLVE_LEVEL && solver != CANOPY_SOLVE_LEVELSYNC)
        return CANOPY_ERR_UNSUPPORTED;
    if (waves != 0 && waves != 1 && waves != 2 && waves != 4 && waves != 8 && waves != 16)
        return CANOPY_ERR_UNSUPPORTED;
    if (solver == CANOPY_SOLVE_LEVELSYNC && (in_dtype != CANOPY_BF16 || (waves != 0 && waves != 8)))
        return CANOPY_ERR_UNSUPPORTED;
    // 16: two column tiles per wave for trees of at most 16 nodes (AUTO, NEUMANN); the
    // two-per-CU blocked kernel for bf16 trees of 65 to 256 nodes (AUTO, FWDSUB).
    if (waves == 16 && !(T <= 16 && (solver == CANOPY_SOLVE_AUTO || solver == CANOPY_SOLVE_NEUMANN)) &&
        (in_dtype != CANOPY_BF16 || T <= 64 || !dual_fits(H, HV, T) ||
         (solver != CANOPY_SOLVE_AUTO && solver != CANOPY_SOLVE_FWDSUB)))
        return CANOPY_ERR_UNSUPPORTED;
    // After a previous tree of at most 64 nodes (one path position per lane): one launch, the
    // committed state kept in registers for the verify, for new trees of at most 16 nodes (AUTO,
    // NEUMANN) and for 17 to 64 nodes where the 17-64 kernel's threads hold at most 2 state
    // pairs (narrow workgroups: up to 32 heads, or 128 at 49-64 nodes). Otherwise the commit
    // kernel, then the verify kernel on the committed state.
    const bool small = T <= 16 && (solver == CANOPY_SOLVE_AUTO || solver == CANOPY_SOLVE_NEUMANN);
    const bool mid = T > 16 && T <= 64 && solver != CANOPY_SOLVE_LEVEL && solver != CANOPY_SOLVE_LEVELSYNC;
    if (T_prev <= 64 && (small || mid)) {
        VerifyArgs a{};
        a.q = q; a.k = k; a.v = v;
        a.alpha = alpha; a.beta = beta; a.S0 = S0; a.parent = parent; a.tree_len = tree_len;
        a.B = B; a.H = HV; a.HK = H; a.T = T;
        a.bf16 = in_dtype == CANOPY_BF16;
        a.solver = solver;
        a.O = O; a.U = U; a.ell = ell;
        a.anc_mask = anc_mask; a.depth = depth; a.tree_status = tree_status;
        a.wait_bound = g_wait_bound.load(std::memory_order_relaxed);
        const PrevCommitArgs c{k_prev, U_prev, alpha_prev, parent_prev, tree_len_prev, path,
                               path_len, T_prev, S_new, path_status};
        if (small) return from_hip(launch_commit_verify_small(a, c, waves, stream));
        int col_tiles = waves == 8 ? 4 : waves;
        // 65 to 128 heads at 49-64 nodes: the one launch at 2 column tiles per workgroup beats
        // the two launches at the 4 the verify alone would take (measured at B = 4, H = 32,
        // T = 64: 18.6 against 20.0 us per step).
        const long long heads = static_cast<long long>(B) * HV;
        if (waves == 0 && T > 48 && heads > 64 && heads <= 128) col_tiles = 2;
        if (commit_verify_mid_fits(a, col_tiles))
            return from_hip(launch_commit_verify_mid(a, c, col_tiles, stream));
    }
    const canopy_status st = canopy_commit(S0, k_prev, in_dtype, U_prev, alpha_prev, parent_prev,
                                           tree_len_prev, path, path_len, B, H, HV, T_prev, S_new,
                                           path_status, stream);
    if (st != CANOPY_OK) return st;
    return canopy_tree_verify(q, k, v, alpha, beta, S_new, parent, tree_len, B, H, HV, T, in_dtype,
                              O, U, ell, anc_mask, depth, tree_status, solver, waves, stream);
}

canopy_status canopy_commit_layers(int L, const float *const *S0, const void *const *k,
                                   canopy_dtype in_dtype, const float *const *U,
                                   const float *const *alpha, const int32_t *parent,
                                   const int32_t *tree_len, const int32_t *path,
                                   const int32_t *path_len, int B, int H, int HV, int T,
                                   float *const *S_new, int32_t *path_status, hipStream_t stream) {
    if (L < 1 || L > kMaxLayers) return CANOPY_ERR_ARG;
    if (!S0 || !k || !U || !alpha || !S_new || !parent || !path || !path_len) return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T) || !heads_ok(H, HV)) return CANOPY_ERR_ARG;
    if (static_cast<long long>(L) * B * HV * 16 > 2147483647LL) return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    CommitLayersArgs la{};
    la.base = CommitArgs{nullptr, nullptr, in_dtype == CANOPY_BF16, nullptr, nullptr, parent, tree_len,
                         path, path_len, B, HV, H, T, nullptr, path_status};
    la.L = L;
    for (int l = 0; l < L; ++l) {
        if (!S0[l] || !k[l] || !U[l] || !alpha[l] || !S_new[l]) return CANOPY_ERR_ARG;
        if (!aligned16(S0[l]) || !aligned16(k[l]) || !aligned16(U[l]) || !aligned16(S_new[l]))
            return CANOPY_ERR_ARG;
        la.S0[l] = S0[l];
        la.k[l] = k[l];
        la.U[l] = U[l];
        la.alpha[l] = alpha[l];
        la.S_new[l] = S_new[l];
    }
    return from_hip(launch_commit_layers(la, stream));
}

canopy_status canopy_serial_verify(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *beta, const float *S0,
                                   const int32_t *parent, const int32_t *tree_len, int B, int H,
                                   int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                   float *snapshots, int32_t *tree_status, hipStream_t stream) {
    if (!q || !k || !v || !alpha || !beta || !S0 || !parent || !O || !U || !snapshots)
        return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T) || !heads_ok(H, HV)) return CANOPY_ERR_ARG;
    if (!aligned16(S0) || !aligned16(v) || !aligned16(O) || !aligned16(U) || !aligned16(snapshots))
        return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    SerialArgs a{q, k, v, alpha, beta, S0, parent, tree_len, B, HV, H, T, in_dtype == CANOPY_BF16,
                 O, U, snapshots, tree_status, g_wait_bound.load(std::memory_order_relaxed)};
    return from_hip(launch_serial(a, stream));
}

canopy_status canopy_hybrid_verify(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *beta, const float *S0,
                                   const int32_t *parent, const int32_t *tree_len, int B, int H,
                                   int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                   float *snapshots, int32_t *tree_status, hipStream_t stream) {
    if (!q || !k || !v || !alpha || !beta || !S0 || !parent || !O || !U || !snapshots)
        return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T) || !heads_ok(H, HV)) return CANOPY_ERR_ARG;
    if (!aligned16(S0) || !aligned16(v) || !aligned16(O) || !aligned16(U) || !aligned16(snapshots))
        return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    SerialArgs a{q, k, v, alpha, beta, S0, parent, tree_len, B, HV, H, T, in_dtype == CANOPY_BF16,
                 O, U, snapshots, tree_status, g_wait_bound.load(std::memory_order_relaxed)};
    return from_hip(launch_hybrid(a, stream));
}

canopy_status canopy_serial_commit(const float *snapshots, const float *S0, const int32_t *parent,
                                   const int32_t *tree_len, const int32_t *path,
                                   const int32_t *path_len, int B, int HV, int T, float *S_new,
                                   int32_t *path_status, hipStream_t stream) {
    if (!snapshots || !S0 || !parent || !path || !path_len || !S_new) return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T)) return CANOPY_ERR_ARG;
    if (!aligned16(snapshots) || !aligned16(S0) || !aligned16(S_new)) return CANOPY_ERR_ARG;
    SerialCommitArgs a{snapshots, S0, parent, tree_len, path, path_len, B, HV, T, S_new, path_status};
    return from_hip(launch_serial_commit(a, stream));
}

// Convolution sizes: channels a positive multiple of 8, kernel size 2..4, and every index of
// the [B,T,C] arrays within 64-bit range with the grid within int range.
static bool conv_sizes_ok(int B, int T, int C, int K) {
    return B >= 1 && T >= 1 && T <= 256 && C >= 8 && C % 8 == 0 && K >= 2 && K <= 4 &&
           static_cast<long long>(B) * ((static_cast<long long>(T) * (C / 8) + 255) / 256) <= 2147483647LL &&
           static_cast<long long>(T) * C <= 2147483647LL;
}

canopy_status canopy_tree_conv(const void *x, canopy_dtype in_dtype, const float *w,
                               const void *conv_state, const int32_t *parent,
                               const int32_t *tree_len, int B, int T, int C, int K, int silu,
                               void *y, int32_t *tree_status, hipStream_t stream) {
    if (!x || !w || !conv_state || !parent || !y) return CANOPY_ERR_ARG;
    if (!conv_sizes_ok(B, T, C, K)) return CANOPY_ERR_ARG;
    if (!aligned16(x) || !aligned16(w) || !aligned16(conv_state) || !aligned16(y)) return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    if (silu != 0 && silu != 1) return CANOPY_ERR_UNSUPPORTED;
    ConvArgs a{x, w, conv_state, parent, tree_len, B, T, C, K, in_dtype == CANOPY_BF16, silu, y,
               tree_status};
    return from_hip(launch_tree_conv(a, stream));
}

canopy_status canopy_conv_commit(const void *x, canopy_dtype in_dtype, const void *conv_state,
                                 const int32_t *parent, const int32_t *tree_len,
                                 const int32_t *path, const int32_t *path_len, int B, int T, int C,
                                 int K, void *state_new, int32_t *path_status, hipStream_t stream) {
    if (!x || !conv_state || !parent || !path || !path_len || !state_new) return CANOPY_ERR_ARG;
    if (!conv_sizes_ok(B, T, C, K)) return CANOPY_ERR_ARG;
    if (!aligned16(x) || !aligned16(conv_state) || !aligned16(state_new)) return CANOPY_ERR_ARG;
    if (in_dtype != CANOPY_FP32 && in_dtype != CANOPY_BF16) return CANOPY_ERR_UNSUPPORTED;
    ConvCommitArgs a{x, conv_state, parent, tree_len, path, path_len, B, T, C, K,
                     in_dtype == CANOPY_BF16, state_new, path_status};
    return from_hip(launch_conv_commit(a, stream));
}

canopy_status canopy_serial_commit_layers(int L, const float *const *snapshots,
                                          const float *const *S0, const int32_t *parent,
                                          const int32_t *tree_len, const int32_t *path,
                                          const int32_t *path_len, int B, int HV, int T,
                                          float *const *S_new, int32_t *path_status,
                                          hipStream_t stream) {
    if (L < 1 || L > kMaxLayers) return CANOPY_ERR_ARG;
    if (!snapshots || !S0 || !S_new || !parent || !path || !path_len) return CANOPY_ERR_ARG;
    if (!sizes_ok(B, HV, T)) return CANOPY_ERR_ARG;
    if (static_cast<long long>(L) * B * HV * 4 > 2147483647LL) return CANOPY_ERR_ARG;
    SerialCommitLayersArgs la{};
    la.base = SerialCommitArgs{nullptr, nullptr, parent, tree_len, path, path_len, B, HV, T, nullptr,
                               path_status};
    la.L = L;
    for (int l = 0; l < L; ++l) {
        if (!snapshots[l] || !S0[l] || !S_new[l]) return CANOPY_ERR_ARG;
        if (!aligned16(snapshots[l]) || !aligned16(S0[l]) || !aligned16(S_new[l])) return CANOPY_ERR_ARG;
        la.snap[l] = snapshots[l];
        la.S0[l] = S0[l];
        la.S_new[l] = S_new[l];
    }
    return from_hip(launch_serial_commit_layers(la, stream));
}

}  // extern "C"
