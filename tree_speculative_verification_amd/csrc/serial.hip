// Serial fork baseline ("Design decisions / Serial baseline" on the canopy project page): the
// nodes are visited in order; each starts from its parent's per-node state snapshot (S0 for a
// root), applies one step of the gated delta rule
//   S~ = alpha S_p,  u = beta (v - S~^T k),  S = S~ + k u^T,  o = S^T q,
// and writes its own snapshot, o and u. One wave per (sequence, head, 16 value columns); the
// wave keeps its 128 x 16 state slice in registers (lane: 8 rows x 4 columns) and reloads it
// from a snapshot only when a node's parent is not the node just processed.
#include "canopy_kernels.hpp"
#include "canopy_step.hpp"
#include <limits.h>

namespace canopy {

template <bool BF>
__global__ __launch_bounds__(64) void serial_kernel(SerialArgs a) {
    constexpr int TILES = D / 16;
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = g % TILES;
    const int bh = g / TILES;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x;
    const int cq = lane & 3, rg = lane >> 2;  // columns 4*cq.., rows rg + 16*m
    const int col = tile * 16 + 4 * cq;
    const int32_t *par = a.parent + static_cast<size_t>(b) * T;
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;
    const size_t qkbase = qk_base(b, h, H, a.HK, T), qkrs = static_cast<size_t>(a.HK) * D;
    const size_t SS = static_cast<size_t>(D) * D;
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;  // this sequence's node count: nodes past it are padding

    int bad = sl.bad ? -1 : INT_MAX;
    for (int i = lane; i < Tb; i += 64) {
        const int p = par[i];
        if (p < -1 || p >= i) bad = min(bad, i + 1);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) bad = min(bad, __shfl_xor(bad, o, 64));
    if (a.tree_status && tile == 0 && h == 0 && lane == 0) a.tree_status[b] = bad == INT_MAX ? 0 : bad;
    if (bad != INT_MAX) {
        const float qnan = __builtin_nanf("");
        for (int i = rg; i < Tb; i += 16) {
            reinterpret_cast<float4 *>(a.O + base + i * rs + col)[0] = make_float4(qnan, qnan, qnan, qnan);
            reinterpret_cast<float4 *>(a.U + base + i * rs + col)[0] = make_float4(qnan, qnan, qnan, qnan);
        }
        return;
    }

    float4 S[8];
    int cur = -2;  // node whose state the registers hold
    for (int i = 0; i < Tb; ++i) {
        const int p = par[i];
        if (p != cur) {
            const float *src = (p < 0) ? a.S0 + static_cast<size_t>(bh) * SS
                                       : a.snap + ((static_cast<size_t>(b) * T + p) * H + h) * SS;
            // The snapshot was written by this wave; order those stores before these loads.
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
#pragma unroll
            for (int m = 0; m < 8; ++m) S[m] = reinterpret_cast<const float4 *>(src + (rg + 16 * m) * D + col)[0];
        }
        const size_t node = base + static_cast<size_t>(i) * rs;
        NodeIn in;
        load_node<BF>(in, a.q, a.k, qkbase + static_cast<size_t>(i) * qkrs, rg, a.v, node + col, a.alpha,
                      a.beta, sbase + static_cast<size_t>(i) * H);
        float4 o, u;
        gdn_step(S, in, o, u);
        float *dst = a.snap + ((static_cast<size_t>(b) * T + i) * H + h) * SS;
#pragma unroll
        for (int m = 0; m < 8; ++m) reinterpret_cast<float4 *>(dst + (rg + 16 * m) * D + col)[0] = S[m];
        if (rg == 0) {
            reinterpret_cast<float4 *>(a.O + node + col)[0] = o;
            reinterpret_cast<float4 *>(a.U + node + col)[0] = u;
        }
        cur = i;
    }
}

// Commit for the serial baseline: the accepted node's snapshot becomes the new state. One
// workgroup per (sequence, head, 32 state rows), float4 copies; path checks as canopy_commit.
__device__ __forceinline__ void serial_commit_body(const SerialCommitArgs &a, int g) {
    __shared__ int s_bad;
    const int chunk = g % 4, bh = g / 4;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int m = a.path_len[b];
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int32_t *pb = a.path + static_cast<size_t>(b) * T;
    const int32_t *par = a.parent + static_cast<size_t>(b) * T;
    if (tid == 0) s_bad = (sl.bad || m < 0 || m > sl.n) ? -1 : INT_MAX;
    __syncthreads();
    if (s_bad == INT_MAX)
        for (int t = tid; t < m; t += 256) {
            const int n = pb[t];
            if (!(n >= 0 && n < sl.n && par[n] == (t == 0 ? -1 : pb[t - 1]))) atomicMin(&s_bad, t + 1);
        }
    __syncthreads();
    const int st = (s_bad == INT_MAX) ? 0 : s_bad;
    if (a.path_status && h == 0 && chunk == 0 && tid == 0) a.path_status[b] = st;
    const size_t SS = static_cast<size_t>(D) * D;
    float4 *dst = reinterpret_cast<float4 *>(a.S_new + bh * SS + chunk * 32 * D);
    if (st != 0) {
        const float qnan = __builtin_nanf("");
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[tid + 256 * k] = make_float4(qnan, qnan, qnan, qnan);
        return;
    }
    // Valid path: its last node is in 0..T-1 (or the path is empty).
    const float *state = (m == 0) ? a.S0 + bh * SS
                                  : a.snap + ((static_cast<size_t>(b) * T + pb[m - 1]) * H + h) * SS;
    const float4 *src = reinterpret_cast<const float4 *>(state + chunk * 32 * D);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[tid + 256 * k] = src[tid + 256 * k];
}

__global__ __launch_bounds__(256) void serial_commit_kernel(SerialCommitArgs a) {
    serial_commit_body(a, xcd_remap(blockIdx.x, gridDim.x));
}

// Every layer's serial commit in one launch (layer 0 writes the path status).
__global__ __launch_bounds__(256) void serial_commit_layers_kernel(SerialCommitLayersArgs la) {
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int per_layer = la.base.B * la.base.H * 4;
    const int l = g / per_layer;
    SerialCommitArgs a = la.base;
    a.snap = la.snap[l];
    a.S0 = la.S0[l];
    a.S_new = la.S_new[l];
    if (l != 0) a.path_status = nullptr;
    serial_commit_body(a, g - l * per_layer);
}

hipError_t launch_serial_commit_layers(const SerialCommitLayersArgs &la, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(la.L * la.base.B * la.base.H * 4)), block(256);
    hipLaunchKernelGGL(serial_commit_layers_kernel, grid, block, 0, stream, la);
    return hipGetLastError();
}

hipError_t launch_serial_commit(const SerialCommitArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * 4)), block(256);
    hipLaunchKernelGGL(serial_commit_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_serial(const SerialArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * (D / 16))), block(64);
    if (a.bf16)
        hipLaunchKernelGGL(serial_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(serial_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace canopy
