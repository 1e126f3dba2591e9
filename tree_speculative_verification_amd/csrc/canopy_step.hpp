// One step of the gated delta rule ("The gated delta rule" on the canopy project page) on a
// wave's 128 x 16 slice of one head's state, for the node-by-node kernels (the serial fork
// baseline and the chain hybrid):
//   S <- alpha S,  u = beta (v - S^T k),  S <- S + k u^T,  o = S^T q.
// Lane (rg, cq) (rg = lane / 4, cq = lane % 4) holds rows rg + 16m (m = 0..7) of the slice's
// columns 4cq..4cq+3; o and u come out for those 4 columns in every lane (the sums over the 128
// rows are reduced across the wave).
#pragma once
#include "canopy_device.hpp"

namespace canopy {

struct NodeIn {
    float kv[8], qv[8];  // rows rg + 16m of k and q
    float4 v;            // the slice's 4 columns of v
    float al, be;
};

// k and q of the node at element offset qknode (row 0), v at element offset vcol (the lane's
// first column), alpha and beta at index sidx.
template <bool BF>
__device__ __forceinline__ void load_node(NodeIn &n, const void *q, const void *k, size_t qknode, int rg,
                                          const void *v, size_t vcol, const float *alpha,
                                          const float *beta, size_t sidx) {
    n.al = alpha[sidx];
    n.be = beta[sidx];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const size_t el = qknode + rg + 16 * m;
        n.kv[m] = BF ? bf16_to_f32(static_cast<const uint16_t *>(k)[el]) : static_cast<const float *>(k)[el];
        n.qv[m] = BF ? bf16_to_f32(static_cast<const uint16_t *>(q)[el]) : static_cast<const float *>(q)[el];
    }
    if (BF) {
        const uint16_t *vp = static_cast<const uint16_t *>(v) + vcol;
        n.v = make_float4(bf16_to_f32(vp[0]), bf16_to_f32(vp[1]), bf16_to_f32(vp[2]), bf16_to_f32(vp[3]));
    } else {
        n.v = reinterpret_cast<const float4 *>(static_cast<const float *>(v) + vcol)[0];
    }
}

__device__ __forceinline__ void gdn_step(float4 (&S)[8], const NodeIn &n, float4 &o, float4 &u) {
    float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        S[m].x *= n.al; S[m].y *= n.al; S[m].z *= n.al; S[m].w *= n.al;
        part.x += S[m].x * n.kv[m]; part.y += S[m].y * n.kv[m];
        part.z += S[m].z * n.kv[m]; part.w += S[m].w * n.kv[m];
    }
#pragma unroll
    for (int s = 4; s < 64; s <<= 1) {
        part.x += __shfl_xor(part.x, s, 64); part.y += __shfl_xor(part.y, s, 64);
        part.z += __shfl_xor(part.z, s, 64); part.w += __shfl_xor(part.w, s, 64);
    }
    u = make_float4(n.be * (n.v.x - part.x), n.be * (n.v.y - part.y), n.be * (n.v.z - part.z),
                    n.be * (n.v.w - part.w));
    o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        S[m].x += n.kv[m] * u.x; S[m].y += n.kv[m] * u.y;
        S[m].z += n.kv[m] * u.z; S[m].w += n.kv[m] * u.w;
        o.x += S[m].x * n.qv[m]; o.y += S[m].y * n.qv[m];
        o.z += S[m].z * n.qv[m]; o.w += S[m].w * n.qv[m];
    }
#pragma unroll
    for (int s = 4; s < 64; s <<= 1) {
        o.x += __shfl_xor(o.x, s, 64); o.y += __shfl_xor(o.y, s, 64);
        o.z += __shfl_xor(o.z, s, 64); o.w += __shfl_xor(o.w, s, 64);
    }
}

}  // namespace canopy
