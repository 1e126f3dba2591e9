// Host-visible argument blocks and launchers of the libcanopy kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "canopy.h"

namespace canopy {

struct VerifyArgs {
    const void *q, *k, *v;
    const float *alpha, *beta, *S0;
    const int32_t *parent;
    int B, H, T;
    int bf16;    // 1: q, k, v are bf16 bit patterns; 0: fp32
    int solver;  // a canopy_solver value
    float *O, *U, *ell;
    uint32_t *anc_mask;
    int32_t *depth, *tree_status;
};

struct PrepArgs {
    const int32_t *parent;
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
    const int32_t *parent, *path, *path_len;
    int B, H, T;
    float *S_new;
    int32_t *path_status;
};

struct SerialArgs {
    const void *q, *k, *v;
    const float *alpha, *beta, *S0;
    const int32_t *parent;
    int B, H, T;
    int bf16;
    float *O, *U, *snap;
    int32_t *tree_status;
};

struct SerialCommitArgs {
    const float *snap, *S0;
    const int32_t *parent, *path, *path_len;
    int B, H, T;
    float *S_new;
    int32_t *path_status;
};

hipError_t launch_verify(const VerifyArgs &a, int waves, hipStream_t stream);
hipError_t launch_verify_small(const VerifyArgs &a, int waves, hipStream_t stream);
hipError_t launch_verify_mid(const VerifyArgs &a, int col_tiles, hipStream_t stream);
hipError_t launch_verify_wide(const VerifyArgs &a, int col_tiles, hipStream_t stream);
hipError_t launch_prep(const PrepArgs &a, hipStream_t stream);
hipError_t launch_commit(const CommitArgs &a, hipStream_t stream);
hipError_t launch_serial(const SerialArgs &a, hipStream_t stream);
hipError_t launch_serial_commit(const SerialCommitArgs &a, hipStream_t stream);

}  // namespace canopy
