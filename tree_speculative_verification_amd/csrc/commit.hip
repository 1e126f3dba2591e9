// Commit of the accepted path ("What the commit kernel stores" on the canopy project page):
//   S_new = P_a S0 + sum_{t < m} w_t k_{path[t]} u_{path[t]}^T,
//   w_t = exp(sum_{s > t} log alpha_{path[s]}) = Gamma_{a, path[t]},  P_a = exp(sum_s log alpha).
// One workgroup per (sequence, head, 32 state rows); 256 threads, each owning four float4s of
// the 32 x 128 row chunk, so loads and stores of S are fully coalesced. The decay weights are
// suffix sums of log alpha along the path in fp64 (wave shuffles, then the wave totals): the
// ratio of two nearby nodes is a short sum, never the difference of two large cumulative
// logs. S0, the path and the first 32 path nodes' U rows and keys are requested before the
// sums are finished, so the path check, the sums and the loads overlap.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

constexpr int CROWS = 32;  // state rows per workgroup
constexpr int CCH = 32;    // path nodes staged per pass

template <bool BF>
__global__ __launch_bounds__(256) void commit_kernel(CommitArgs a) {
    __shared__ int s_path[256];
    __shared__ double s_wsum[4];
    __shared__ float s_w[256];
    __shared__ float s_pa;
    __shared__ int s_bad;
    __shared__ float4 s_u[CCH][D / 4];
    __shared__ float s_kw[CCH][CROWS];

    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = g % (D / CROWS);
    const int bh = g / (D / CROWS);
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *pb = a.path + static_cast<size_t>(b) * T;
    const int32_t *par = a.parent + static_cast<size_t>(b) * T;
    const int row0 = chunk * CROWS;
    const int c4 = tid & 31;    // float4 column
    const int rsub = tid >> 5;  // rows rsub + 8 * mm
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;

    // ---- requests that need nothing else: the path length, this thread's path entry (and the
    // one before it), and this thread's part of S0
    const int m = a.path_len[b];
    const int nd = tid < T ? pb[tid] : -1;
    const int prev = (tid > 0 && tid < T) ? pb[tid - 1] : -1;
    const float *S0 = a.S0 + static_cast<size_t>(bh) * D * D;
    float4 s0[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) s0[mm] = reinterpret_cast<const float4 *>(S0 + (row0 + rsub + 8 * mm) * D)[c4];

    // ---- path check (positions t < m) and log alpha of the path's nodes
    const bool lenok = m >= 0 && m <= T;
    const bool inpath = lenok && tid < m;
    bool ok = true;
    double la = 0.0;
    if (inpath) {
        ok = nd >= 0 && nd < T;
        if (ok) ok = par[nd] == (tid == 0 ? -1 : prev);
        if (ok) la = log(static_cast<double>(a.alpha[(static_cast<size_t>(b) * T + nd) * H + h]));
    }
    if (tid == 0) s_bad = lenok ? INT_MAX : -1;
    s_path[tid] = (inpath && ok) ? nd : 0;
    // suffix sums of log alpha within the wave: v_t = sum_{s >= t, same wave} la_s
    double v = la;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double t = __shfl_down(v, off, 64);
        if (lane + off < 64) v += t;
    }
    if (lane == 0) s_wsum[wave] = v;
    __syncthreads();
    if (inpath && !ok) atomicMin(&s_bad, tid + 1);
    // ---- request the first 32 path nodes' U rows and k values (they only need s_path)
    const int nt0 = lenok ? min(CCH, m) : 0;
    // CCH x (D/4) float4s of U and CCH x CROWS keys: four of each per thread.
    float4 ureg[4];
    float kreg[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int x = tid + 256 * q, t = x / (D / 4), cc = x % (D / 4);
        ureg[q] = t < nt0 ? reinterpret_cast<const float4 *>(a.U + base + s_path[t] * rs)[cc]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        const int tk = x / CROWS, rr = x % CROWS;
        kreg[q] = 0.f;
        if (tk < nt0) {
            const size_t el = base + s_path[tk] * rs + row0 + rr;
            kreg[q] = BF ? bf16_to_f32(static_cast<const uint16_t *>(a.k)[el]) : static_cast<const float *>(a.k)[el];
        }
    }
    // ---- finish the suffix sums across waves: S_t = sum_{s >= t} log alpha_s;
    // w_t = exp(S_t - log alpha_t) = Gamma_{a, path[t]}, P_a = exp(S_0)
    for (int w2 = wave + 1; w2 < 4; ++w2) v += s_wsum[w2];
    if (inpath) s_w[tid] = static_cast<float>(exp(v - la));
    if (tid == 0) s_pa = static_cast<float>(exp(m > 0 && lenok ? v : 0.0));
    __syncthreads();
    const int st = (s_bad == INT_MAX) ? 0 : s_bad;
    if (a.path_status && h == 0 && chunk == 0 && tid == 0) a.path_status[b] = st;
    float *Sn = a.S_new + static_cast<size_t>(bh) * D * D;
    if (st != 0) {
        const float qnan = __builtin_nanf("");
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
            reinterpret_cast<float4 *>(Sn + (row0 + rsub + 8 * mm) * D)[c4] = make_float4(qnan, qnan, qnan, qnan);
        return;
    }
    const float Pa = s_pa;
    float4 acc[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
        acc[mm] = make_float4(Pa * s0[mm].x, Pa * s0[mm].y, Pa * s0[mm].z, Pa * s0[mm].w);
    for (int t0 = 0; t0 < m; t0 += CCH) {
        const int nt = min(CCH, m - t0);
        if (t0 > 0) {  // later chunks (paths longer than 32 nodes)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int x = tid + 256 * q, t = x / (D / 4), cc = x % (D / 4);
                ureg[q] = t < nt ? reinterpret_cast<const float4 *>(a.U + base + s_path[t0 + t] * rs)[cc]
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
                const int tk = x / CROWS, rr = x % CROWS;
                kreg[q] = 0.f;
                if (tk < nt) {
                    const size_t el = base + s_path[t0 + tk] * rs + row0 + rr;
                    kreg[q] = BF ? bf16_to_f32(static_cast<const uint16_t *>(a.k)[el]) : static_cast<const float *>(a.k)[el];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int x = tid + 256 * q;
            s_u[x / (D / 4)][x % (D / 4)] = ureg[q];
            const int tk = x / CROWS, rr = x % CROWS;
            s_kw[tk][rr] = tk < nt ? s_w[t0 + tk] * kreg[q] : 0.f;
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
