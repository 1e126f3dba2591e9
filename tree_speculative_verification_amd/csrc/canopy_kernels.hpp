// Host-visible argument blocks and launchers of the libcanopy kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "canopy.h"

namespace canopy {

// Head counts: H is the number of value heads (v, alpha, beta, S0, O, U, ell, states); q and
// k have HK heads, HK dividing H, and value head h reads q/k head h / (H / HK). tree_len, when
// not null, gives each sequence's node count (1..T); arrays keep their T-row extent.
struct VerifyArgs {
    const void *q, *k, *v;
    const float *alpha, *beta, *S0;
    const int32_t *parent, *tree_len;
    int B, H, HK, T;
    int bf16;    // 1: q, k, v are bf16 bit patterns; 0: fp32
    int solver;  // a canopy_solver value
    float *O, *U, *ell;
    uint32_t *anc_mask;
    int32_t *depth, *tree_status;
    int wait_bound;  // sleeps before a wave gives up waiting for another wave's result
};

struct PrepArgs {
    const int32_t *parent, *tree_len;
    const float *alpha;
    int B, H, T;
    uint32_t *anc_mask;
    int32_t *depth;
    float *ell;
    int32_t *tree_status;
};

struct CommitArgs {
    const float *S0;
    const void *k;
    int bf16;
    const float *U, *alpha;
    const int32_t *parent, *tree_len, *path, *path_len;
    int B, H, HK, T;
    float *S_new;
    int32_t *path_status;
};

// The commit that precedes a verify in one call: the previous tree's accepted path applied to
// VerifyArgs::S0, the result written to S_new and used as the verify's initial state. Arrays
// of the previous tree have T rows (its own node count); heads as in VerifyArgs.
struct PrevCommitArgs {
    const void *k;
    const float *U, *alpha;
    const int32_t *parent, *tree_len, *path, *path_len;
    int T;
    float *S_new;
    int32_t *path_status;
};

struct SerialArgs {
    const void *q, *k, *v;
    const float *alpha, *beta, *S0;
    const int32_t *parent, *tree_len;
    int B, H, HK, T;
    int bf16;
    float *O, *U, *snap;
    int32_t *tree_status;
    int wait_bound;  // as in VerifyArgs
};

struct SerialCommitArgs {
    const float *snap, *S0;
    const int32_t *parent, *tree_len, *path, *path_len;
    int B, H, T;
    float *S_new;
    int32_t *path_status;
};

// One launch for the commits of up to kMaxLayers layers that share the tree and the accepted
// path: per-layer pointers by value, the rest from base (whose own per-layer pointers are
// unused).
constexpr int kMaxLayers = 64;
struct CommitLayersArgs {
    CommitArgs base;
    int L;
    const float *S0[kMaxLayers];
    const void *k[kMaxLayers];
    const float *U[kMaxLayers];
    const float *alpha[kMaxLayers];
    float *S_new[kMaxLayers];
};

struct SerialCommitLayersArgs {
    SerialCommitArgs base;
    int L;
    const float *snap[kMaxLayers];
    const float *S0[kMaxLayers];
    float *S_new[kMaxLayers];
};

// Root-path causal convolution: x [B,T,C], w [C,K] fp32, state [B,K-1,C], y [B,T,C]; x, state
// and y in the input dtype.
struct ConvArgs {
    const void *x;
    const float *w;
    const void *state;
    const int32_t *parent, *tree_len;
    int B, T, C, K;
    int bf16, silu;
    void *y;
    int32_t *tree_status;
};

struct ConvCommitArgs {
    const void *x, *state;
    const int32_t *parent, *tree_len, *path, *path_len;
    int B, T, C, K;
    int bf16;
    void *state_new;
    int32_t *path_status;
};

// The node count of sequence b: tree_len[b], or T without a length array. A length outside
// 1..T is reported (bad = true) and the whole T-row extent is then treated as that sequence's
// tree, whose outputs the kernels replace by NaN.
struct SeqLen {
    int n;
    bool bad;
};
__device__ __forceinline__ SeqLen seq_len(const int32_t *tree_len, int b, int T) {
    if (!tree_len) return {T, false};
    const int n = tree_len[b];
    const bool ok = n >= 1 && n <= T;
    return {ok ? n : T, !ok};
}

// Offset of (sequence b, node 0, q/k head of value head h, column 0) in a q or k array of HK
// heads (node stride HK * 128 elements).
__device__ __forceinline__ size_t qk_base(int b, int h, int H, int HK, int T) {
    return (static_cast<size_t>(b) * T * HK + h / (H / HK)) * 128;
}

hipError_t launch_verify(const VerifyArgs &a, int waves, hipStream_t stream);
hipError_t launch_verify_small(const VerifyArgs &a, int waves, hipStream_t stream);
hipError_t launch_commit_verify_small(const VerifyArgs &a, const PrevCommitArgs &c, int waves,
                                      hipStream_t stream);
hipError_t launch_verify_mid(const VerifyArgs &a, int col_tiles, hipStream_t stream);
bool commit_verify_mid_fits(const VerifyArgs &a, int col_tiles);
hipError_t launch_commit_verify_mid(const VerifyArgs &a, const PrevCommitArgs &c, int col_tiles,
                                    hipStream_t stream);
hipError_t launch_verify_wide(const VerifyArgs &a, int col_tiles, hipStream_t stream);
// The blocked solve sized for two workgroups per CU (bf16, 65 <= T <= 256, FWDSUB on every
// diagonal block); dual_fits: a head's rows span less than 2^31 bytes (32-bit offsets).
hipError_t launch_verify_dual(const VerifyArgs &a, hipStream_t stream);
bool dual_fits(int HK, int HV, int T);
// Matrix-form solves (SERIES, SQUARING, SPLIT) with their operators in a workspace of
// mat_workspace_bytes bytes.
size_t mat_workspace_bytes(int B, int H, int T, int solver);
hipError_t launch_verify_matrix(const VerifyArgs &a, void *ws, hipStream_t stream);
// The workspace of canopy_tree_verify_static: a device array of this many bytes per device.
constexpr size_t kStaticScratchBytes = static_cast<size_t>(64) << 20;
hipError_t mat_static_scratch(void **ptr);
hipError_t launch_prep(const PrepArgs &a, hipStream_t stream);
hipError_t launch_commit(const CommitArgs &a, hipStream_t stream);
hipError_t launch_serial(const SerialArgs &a, hipStream_t stream);
hipError_t launch_serial_commit(const SerialCommitArgs &a, hipStream_t stream);
hipError_t launch_hybrid(const SerialArgs &a, hipStream_t stream);
hipError_t launch_commit_layers(const CommitLayersArgs &la, hipStream_t stream);
hipError_t launch_serial_commit_layers(const SerialCommitLayersArgs &la, hipStream_t stream);
hipError_t launch_tree_conv(const ConvArgs &a, hipStream_t stream);
hipError_t launch_conv_commit(const ConvCommitArgs &a, hipStream_t stream);

}  // namespace canopy
