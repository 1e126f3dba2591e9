// Commit of the accepted path ("What the commit kernel stores" on the canopy project page):
//   S_new = P_a S0 + sum_{t < m} w_t k_{path[t]} u_{path[t]}^T,
//   w_t = exp(sum_{s > t} log alpha_{path[s]}) = Gamma_{a, path[t]},  P_a = exp(sum_s log alpha).
// One workgroup per (sequence, head, 32 state rows); 256 threads, each owning four float4s of
// the 32 x 128 row chunk, so loads and stores of S are fully coalesced. The decay weights are
// suffix sums of log alpha along the path in fp64: the ratio of two nearby nodes is formed
// directly and never as the difference of two large cumulative logs.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

constexpr int CROWS = 32;  // state rows per workgroup
constexpr int CCH = 32;    // path nodes staged per pass

template <bool BF>
__global__ __launch_bounds__(256) void commit_kernel(CommitArgs a) {
    __shared__ double s_la[256];
    __shared__ int s_path[256];
    __shared__ int s_bad;
    __shared__ float s_w[256];
    __shared__ float4 s_u[CCH][D / 4];
    __shared__ float s_kw[CCH][CROWS];

    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = g % (D / CROWS);
    const int bh = g / (D / CROWS);
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int m = a.path_len[b];
    const int32_t *pb = a.path + static_cast<size_t>(b) * T;
    const int32_t *par = a.parent + static_cast<size_t>(b) * T;

    if (tid == 0) s_bad = (m < 0 || m > T) ? -1 : INT_MAX;
    __syncthreads();
    if (s_bad == INT_MAX) {
        for (int t = tid; t < m; t += 256) {
            const int n = pb[t];
            const bool ok = n >= 0 && n < T && par[n] == (t == 0 ? -1 : pb[t - 1]);
            if (!ok) {
                atomicMin(&s_bad, t + 1);
            } else {
                s_path[t] = n;
                s_la[t] = log(static_cast<double>(a.alpha[(static_cast<size_t>(b) * T + n) * H + h]));
            }
        }
    }
    __syncthreads();
    const int st = (s_bad == INT_MAX) ? 0 : s_bad;
    if (a.path_status && h == 0 && chunk == 0 && tid == 0) a.path_status[b] = st;

    const int row0 = chunk * CROWS;
    const int c4 = tid & 31;   // float4 column
    const int rsub = tid >> 5; // rows rsub + 8 * mm
    float *Sn = a.S_new + static_cast<size_t>(bh) * D * D;
    if (st != 0) {
        const float qnan = __builtin_nanf("");
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
            reinterpret_cast<float4 *>(Sn + (row0 + rsub + 8 * mm) * D)[c4] =
                make_float4(qnan, qnan, qnan, qnan);
        return;
    }

    // Inclusive suffix sums of log alpha along the path (Hillis-Steele, m <= 256).
    for (int off = 1; off < 256; off <<= 1) {
        const double add = (tid < m && tid + off < m) ? s_la[tid + off] : 0.0;
        __syncthreads();
        if (tid < m) s_la[tid] += add;
        __syncthreads();
    }
    if (tid < m) s_w[tid] = static_cast<float>(exp(tid + 1 < m ? s_la[tid + 1] : 0.0));
    const float Pa = static_cast<float>(exp(m > 0 ? s_la[0] : 0.0));
    __syncthreads();

    const float *S0 = a.S0 + static_cast<size_t>(bh) * D * D;
    float4 acc[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
        const float4 s = reinterpret_cast<const float4 *>(S0 + (row0 + rsub + 8 * mm) * D)[c4];
        acc[mm] = make_float4(Pa * s.x, Pa * s.y, Pa * s.z, Pa * s.w);
    }
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    for (int t0 = 0; t0 < m; t0 += CCH) {
        const int nt = min(CCH, m - t0);
        for (int x = tid; x < nt * (D / 4); x += 256) {
            const int t = x / (D / 4), cc = x % (D / 4);
            s_u[t][cc] = reinterpret_cast<const float4 *>(a.U + base + s_path[t0 + t] * rs)[cc];
        }
        for (int x = tid; x < nt * CROWS; x += 256) {
            const int t = x / CROWS, rr = x % CROWS;
            const size_t el = base + s_path[t0 + t] * rs + row0 + rr;
            const float kv = BF ? bf16_to_f32(static_cast<const uint16_t *>(a.k)[el])
                                : static_cast<const float *>(a.k)[el];
            s_kw[t][rr] = s_w[t0 + t] * kv;
        }
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            const float4 u = s_u[t][c4];
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const float kw = s_kw[t][rsub + 8 * mm];
                acc[mm].x += kw * u.x;
                acc[mm].y += kw * u.y;
                acc[mm].z += kw * u.z;
                acc[mm].w += kw * u.w;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
        reinterpret_cast<float4 *>(Sn + (row0 + rsub + 8 * mm) * D)[c4] = acc[mm];
}

hipError_t launch_commit(const CommitArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * (D / CROWS))), block(256);
    if (a.bf16)
        hipLaunchKernelGGL(commit_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(commit_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace canopy
