// Root-path causal convolution of a draft tree and its state commit (the canopy project page,
// "M7", stretch item: the short causal convolution before each GDN layer follows each node's
// root path, and commit rolls the convolution state forward with the accepted tokens).
//   y_i[c] = sum_{j<K} w[c][j] * X_i(K-1-j)[c],  then SiLU if asked,
// X_i(0) = x_i, X_i(s) the input s positions up node i's root path, and past the root the
// committed state rows (the last one first). Depthwise, K <= 4, fp32 accumulation.
// One workgroup per (sequence, 128-byte channel segment): it copies that segment of every
// node's row and of the state rows into LDS with LDS-bound loads (each input byte leaves HBM
// once, although a row serves the windows of the node, its children and grandchildren), puts
// the parents in LDS and checks them, then each thread walks K-1 levels up from its nodes and
// reads their windows from LDS. HBM-bound: x read and y written once.
#include "canopy_device.hpp"
#include "canopy_kernels.hpp"
#include <limits.h>

namespace canopy {

constexpr int CONV_NT = 256;
// Bytes of every row a workgroup stages: 128-byte segments (32 KiB of LDS at T = 256) let
// several workgroups share a CU, so one's loads overlap another's stores; measured faster than
// 256- and 512-byte segments at 8192 channels.
constexpr int SEG = 128;

template <bool BF>
struct Chunk8 {
    // 8 consecutive channels of one row, widened to fp32.
    __device__ static __forceinline__ void load(const void *base, size_t elem, float (&v)[8]) {
        if constexpr (BF) {
            const u32x4 r = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + elem);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = __uint_as_float(r[e] << 16);
                v[2 * e + 1] = __uint_as_float(r[e] & 0xFFFF0000u);
            }
        } else {
            const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
            const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
    }
    // Round to the element type (bf16: nearest, ties to even) and store.
    __device__ static __forceinline__ void store(void *base, size_t elem, const float (&v)[8]) {
        if constexpr (BF) {
            u32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * e]));
                const uint16_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * e + 1]));
                r[e] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
            }
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + elem) = r;
        } else {
            float *p = static_cast<float *>(base) + elem;
            *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
    // The same row copied without widening.
    __device__ static __forceinline__ void copy(const void *src, size_t se, void *dst, size_t de) {
        if constexpr (BF) {
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(dst) + de) =
                *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(src) + se);
        } else {
            const float4 *s = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + se);
            float4 *d = reinterpret_cast<float4 *>(static_cast<float *>(dst) + de);
            const float4 a = s[0], b = s[1];
            d[0] = a;
            d[1] = b;
        }
    }
};

template <bool BF, int K, bool SILU>
__global__ __launch_bounds__(CONV_NT) void tree_conv_kernel(ConvArgs a) {
    constexpr int ES = BF ? 2 : 4;
    constexpr int CW = SEG / ES;   // channels per workgroup: a SEG-byte segment of every row
    constexpr int CPR = CW / 8;    // 8-channel chunks per segment
    constexpr int LPR = SEG / 16;  // 16-byte pieces per segment row
    __shared__ __align__(16) uint8_t s_x[256 * SEG];     // the segment of every node's row
    __shared__ __align__(16) uint8_t s_st[(K - 1) * SEG];  // ... and of the state rows
    __shared__ int s_par[256];
    __shared__ int s_bad;
    const int T = a.T, C = a.C;
    const int per_seq = (C + CW - 1) / CW;
    const int b = blockIdx.x / per_seq;
    const int cb = (blockIdx.x % per_seq) * CW;  // first channel of the segment
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // ---- the segment of rows 0..Tb-1 and of the state into LDS: one 1-KB piece (64 / LPR
    // rows) per wave instruction, lane l taking row (64 / LPR) s + l / LPR, piece l % LPR. Rows
    // and channels past the arrays are clamped to valid ones (their LDS copies are never read).
    {
        constexpr int RPP = 64 / LPR;  // rows per 1-KB piece
        const int pieces = (Tb + RPP - 1) / RPP;
        const int piece = lane % LPR, rsub = lane / LPR;
        const int ch = min(cb + piece * (16 / ES), C - 16 / ES);  // 16 bytes = 16 / ES channels
        for (int s = wave; s < pieces; s += CONV_NT / 64) {
            const int row = min(RPP * s + rsub, T - 1);
            dma16(static_cast<const uint8_t *>(a.x) + ((static_cast<size_t>(b) * T + row) * C + ch) * ES,
                  s_x + s * 1024);
        }
        if (wave == 0 && lane < LPR * (K - 1)) {
            const int row = lane / LPR;
            const uint4 v = *reinterpret_cast<const uint4 *>(
                static_cast<const uint8_t *>(a.state) + ((static_cast<size_t>(b) * (K - 1) + row) * C + ch) * ES);
            *reinterpret_cast<uint4 *>(s_st + row * SEG + piece * 16) = v;
        }
    }
    if (tid == 0) s_bad = INT_MAX;
    __syncthreads();
    if (tid < Tb) {
        const int p = a.parent[static_cast<size_t>(b) * T + tid];
        const bool ok = p >= -1 && p < tid;
        s_par[tid] = ok ? p : -1;
        if (!ok) atomicMin(&s_bad, tid + 1);
    }
    wait_vmem();
    __syncthreads();
    const int bad = sl.bad ? -1 : (s_bad == INT_MAX ? 0 : s_bad);
    if (a.tree_status && blockIdx.x % per_seq == 0 && tid == 0) a.tree_status[b] = bad;

    // ---- one (node, 8-channel chunk) per thread and step; CPR divides the workgroup, so a
    // thread's chunk, and its weights, stay the same
    const int chunk = tid % CPR;
    const int c0 = cb + 8 * chunk;
    if (c0 >= C) return;
    float wv[8][K];
    {
        const float *wp = a.w + static_cast<size_t>(c0) * K;  // [C][K]: 8K consecutive floats
        float tmp[8 * K];
#pragma unroll
        for (int q = 0; q < 2 * K; ++q) {
            const float4 f = reinterpret_cast<const float4 *>(wp)[q];
            tmp[4 * q] = f.x; tmp[4 * q + 1] = f.y; tmp[4 * q + 2] = f.z; tmp[4 * q + 3] = f.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int j = 0; j < K; ++j) wv[e][j] = tmp[e * K + j];
    }
    const float qnan = __builtin_nanf("");
    for (int i = tid / CPR; i < Tb; i += CONV_NT / CPR) {
        const size_t yrow = (static_cast<size_t>(b) * T + i) * C + c0;
        float out[8];
        if (bad) {
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = qnan;
        } else {
            // The window's rows, newest first: node i, its parent, ...; past the root the
            // state rows K-2, K-3, ... (the most recent committed input first).
            float xv[K][8];
            int node = i, past = 0;
#pragma unroll
            for (int s = 0; s < K; ++s) {
                if (s > 0 && node >= 0) node = s_par[node];
                if (node < 0) ++past;
                const uint8_t *src = node >= 0 ? s_x + node * SEG + chunk * 8 * ES
                                               : s_st + (K - 1 - past) * SEG + chunk * 8 * ES;
                Chunk8<BF>::load(src, 0, xv[s]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < K; ++j) acc += wv[e][j] * xv[K - 1 - j][e];
                if constexpr (SILU) acc = acc / (1.f + __builtin_amdgcn_exp2f(-acc * 1.4426950408889634f));
                out[e] = acc;
            }
        }
        Chunk8<BF>::store(a.y, yrow, out);
    }
}

// The state after the accepted path: its last K-1 inputs (old state rows, then the path's
// nodes), oldest first. One thread per 8 channels of a sequence handles every row, in
// ascending order, so the new state may overwrite the old one: new row s reads old row s + m.
template <bool BF, int K>
__global__ __launch_bounds__(CONV_NT) void conv_commit_kernel(ConvCommitArgs a) {
    __shared__ int s_bad;
    const int T = a.T, C = a.C, C8 = C / 8;
    const int per_seq = (C8 + CONV_NT - 1) / CONV_NT;
    const int b = blockIdx.x / per_seq;
    const int tid = threadIdx.x;
    const int chunk = (blockIdx.x % per_seq) * CONV_NT + tid;
    const int m = a.path_len[b];
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int32_t *pb = a.path + static_cast<size_t>(b) * T;
    const int32_t *par = a.parent + static_cast<size_t>(b) * T;
    if (tid == 0) s_bad = (sl.bad || m < 0 || m > sl.n) ? -1 : INT_MAX;
    __syncthreads();
    if (s_bad == INT_MAX)
        for (int t = tid; t < m; t += CONV_NT) {
            const int n = pb[t];
            if (!(n >= 0 && n < sl.n && par[n] == (t == 0 ? -1 : pb[t - 1]))) atomicMin(&s_bad, t + 1);
        }
    __syncthreads();
    const int st = s_bad == INT_MAX ? 0 : s_bad;
    if (a.path_status && blockIdx.x % per_seq == 0 && tid == 0) a.path_status[b] = st;
    if (chunk >= C8) return;
    const int c0 = chunk * 8;
    const size_t sbase = static_cast<size_t>(b) * (K - 1) * C + c0;
    if (st != 0) {
        float nan8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) nan8[e] = __builtin_nanf("");
#pragma unroll
        for (int s = 0; s < K - 1; ++s) Chunk8<BF>::store(a.state_new, sbase + static_cast<size_t>(s) * C, nan8);
        return;
    }
#pragma unroll
    for (int s = 0; s < K - 1; ++s) {
        const int pos = m - (K - 1) + s;  // position in the path; negative: the old state
        if (pos >= 0)
            Chunk8<BF>::copy(a.x, (static_cast<size_t>(b) * T + pb[pos]) * C + c0, a.state_new,
                             sbase + static_cast<size_t>(s) * C);
        else
            Chunk8<BF>::copy(a.state, sbase + static_cast<size_t>(K - 1 + pos) * C, a.state_new,
                             sbase + static_cast<size_t>(s) * C);
    }
}

template <bool BF, int K>
static void launch_conv_k(const ConvArgs &a, hipStream_t stream) {
    const int per_seq = (a.C + SEG / (BF ? 2 : 4) - 1) / (SEG / (BF ? 2 : 4));
    const dim3 grid(static_cast<unsigned>(a.B * per_seq)), block(CONV_NT);
    if (a.silu)
        hipLaunchKernelGGL((tree_conv_kernel<BF, K, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((tree_conv_kernel<BF, K, false>), grid, block, 0, stream, a);
}

template <bool BF>
static void launch_conv_bf(const ConvArgs &a, hipStream_t stream) {
    switch (a.K) {
        case 2: launch_conv_k<BF, 2>(a, stream); break;
        case 3: launch_conv_k<BF, 3>(a, stream); break;
        default: launch_conv_k<BF, 4>(a, stream); break;
    }
}

hipError_t launch_tree_conv(const ConvArgs &a, hipStream_t stream) {
    if (a.bf16)
        launch_conv_bf<true>(a, stream);
    else
        launch_conv_bf<false>(a, stream);
    return hipGetLastError();
}

template <bool BF, int K>
static void launch_cc_k(const ConvCommitArgs &a, hipStream_t stream) {
    const int per_seq = (a.C / 8 + CONV_NT - 1) / CONV_NT;
    hipLaunchKernelGGL((conv_commit_kernel<BF, K>), dim3(static_cast<unsigned>(a.B * per_seq)),
                       dim3(CONV_NT), 0, stream, a);
}

template <bool BF>
static void launch_cc_bf(const ConvCommitArgs &a, hipStream_t stream) {
    switch (a.K) {
        case 2: launch_cc_k<BF, 2>(a, stream); break;
        case 3: launch_cc_k<BF, 3>(a, stream); break;
        default: launch_cc_k<BF, 4>(a, stream); break;
    }
}

hipError_t launch_conv_commit(const ConvCommitArgs &a, hipStream_t stream) {
    if (a.bf16)
        launch_cc_bf<true>(a, stream);
    else
        launch_cc_bf<false>(a, stream);
    return hipGetLastError();
}

}  // namespace canopy
