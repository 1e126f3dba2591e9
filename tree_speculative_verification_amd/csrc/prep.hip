// Standalone tree preprocessing: one workgroup per (sequence, head) writes l for its head;
// the head-0 workgroup of a sequence also writes the bitmask, depth and status.
#include "canopy_prep.hpp"
#include "canopy_kernels.hpp"

namespace canopy {

template <int NB>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    constexpr int MAXT = 64 * NB, NT = 256;
    __shared__ PrepSmem<MAXT> ps;
    const int bh = blockIdx.x;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;  // this sequence's node count
    const int pbad = tree_prep_block<MAXT, NT>(ps, a.parent + static_cast<size_t>(b) * T,
                                               a.alpha + sbase, H, T, Tb);
    const int bad = sl.bad ? -1 : pbad;
    const int tid = threadIdx.x;
    if (a.ell)
        for (int i = tid; i < Tb; i += NT)
            a.ell[sbase + static_cast<size_t>(i) * H] =
                bad ? __builtin_nanf("") : static_cast<float>(ps.ell[i] * 0.69314718055994530942);
    if (h != 0) return;
    if (a.tree_status && tid == 0) a.tree_status[b] = bad;
    const int W = (T + 31) >> 5;
    for (int i = tid; i < Tb; i += NT) {
        if (a.depth) a.depth[static_cast<size_t>(b) * T + i] = bad ? 0 : node_depth<MAXT>(ps, i);
        if (a.anc_mask)
            for (int w = 0; w < W; ++w)
                a.anc_mask[(static_cast<size_t>(b) * T + i) * W + w] = bad ? 0u : ps.mask[i][w];
    }
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H)), block(256);
    switch ((a.T + 63) / 64) {
        case 1: hipLaunchKernelGGL(prep_kernel<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(prep_kernel<2>, grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(prep_kernel<3>, grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL(prep_kernel<4>, grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace canopy
