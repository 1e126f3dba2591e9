// Chain-decomposed hybrid ("What the papers report": SpecLA's chain-decomposed hybrid; "M4",
// optional third contender: heavy-light decomposition, each chain serial, chains in parallel).
// The tree is cut into heavy paths: every node's heavy child is the child with the largest
// subtree (the lowest id on ties), and a chain starts at a root or at a light child. A chain's
// level is the number of light edges above it, at most log2(T). Chains of one level run in
// parallel, one per wave, each walking its nodes in order with the state slice in registers
// (the serial recurrence, canopy_step.hpp); it starts from the snapshot of its head's parent,
// which a chain of the level above wrote, or from S0 for a root. Only fork nodes (two or more
// children) write snapshots. One workgroup per (sequence, head, 16 value columns), NW waves;
// the decomposition is computed in LDS from the ancestor bitmask of the shared tree prep.
#include "canopy_kernels.hpp"
#include "canopy_prep.hpp"
#include "canopy_step.hpp"
#include <limits.h>

namespace canopy {

constexpr int HMAXT = 256;

template <bool BF, int NW>
__global__ __launch_bounds__(NW * 64) void hybrid_kernel(SerialArgs a) {
    constexpr int NT = NW * 64, TILES = D / 16;
    __shared__ PrepSmem<HMAXT> ps;
    __shared__ int s_par[HMAXT], s_best[HMAXT], s_heavy[HMAXT], s_nch[HMAXT], s_level[HMAXT];
    __shared__ uint32_t s_headmask[HMAXT / 32];
    __shared__ int s_maxlevel;
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = g % TILES, bh = g / TILES;
    const int H = a.H, T = a.T;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int cq = lane & 3, rg = lane >> 2;  // columns 4cq.., rows rg + 16m
    const int col = tile * 16 + 4 * cq;
    const size_t rs = static_cast<size_t>(H) * D;
    const size_t base = (static_cast<size_t>(b) * T * H + h) * D;
    const size_t sbase = static_cast<size_t>(b) * T * H + h;
    const size_t qkbase = qk_base(b, h, H, a.HK, T), qkrs = static_cast<size_t>(a.HK) * D;
    const size_t SS = static_cast<size_t>(D) * D;
    const SeqLen sl = seq_len(a.tree_len, b, T);
    const int Tb = sl.n;

    // ---- tree: validation and inclusive ancestor masks (the blocked kernel's prep)
    PrepIn<HMAXT, NT> pin;
    pin.load(a.parent + static_cast<size_t>(b) * T, a.alpha + sbase, H, T);
    const int pbad = tree_prep_compute<HMAXT, NT>(ps, pin, Tb);
    const int bad = sl.bad ? -1 : pbad;
    if (a.tree_status && tile == 0 && h == 0 && tid == 0) a.tree_status[b] = bad;
    if (bad) {
        const float qnan = __builtin_nanf("");
        for (int i = wave * 16 + rg; i < Tb; i += NW * 16) {
            reinterpret_cast<float4 *>(a.O + base + i * rs + col)[0] = make_float4(qnan, qnan, qnan, qnan);
            reinterpret_cast<float4 *>(a.U + base + i * rs + col)[0] = make_float4(qnan, qnan, qnan, qnan);
        }
        return;
    }
    // ---- heavy-light decomposition in LDS
#pragma unroll
    for (int t = 0; t < PrepIn<HMAXT, NT>::NPT; ++t) {
        const int i = tid + t * NT;
        if (i < HMAXT) {
            s_par[i] = i < Tb ? pin.p[t] : -1;
            s_best[i] = -1;
            s_nch[i] = 0;
            s_level[i] = -1;
        }
    }
    if (tid < HMAXT / 32) s_headmask[tid] = 0u;
    if (tid == 0) s_maxlevel = 0;
    __syncthreads();
    // subtree size of node i = the nodes whose inclusive mask holds i; the heavy child of each
    // node by an atomic max over (size, -id), and the child counts
    for (int i = tid; i < Tb; i += NT) {
        int size = 0;
        for (int j = i; j < Tb; ++j) size += (ps.mask[j][i >> 5] >> (i & 31)) & 1u;
        const int p = s_par[i];
        if (p >= 0) {
            atomicMax(&s_best[p], (size << 9) | (511 - i));
            atomicAdd(&s_nch[p], 1);
        }
    }
    __syncthreads();
    for (int i = tid; i < Tb; i += NT) {
        const int bst = s_best[i];
        s_heavy[i] = bst >= 0 ? 511 - (bst & 511) : -1;
    }
    __syncthreads();
    for (int i = tid; i < Tb; i += NT) {
        const int p = s_par[i];
        if (p < 0 || s_heavy[p] != i) atomicOr(&s_headmask[i >> 5], 1u << (i & 31));
    }
    __syncthreads();
    // a head's level: the heads on its root path, minus itself
    for (int i = tid; i < Tb; i += NT) {
        if ((s_headmask[i >> 5] >> (i & 31)) & 1u) {
            int c = -1;
#pragma unroll
            for (int w = 0; w < HMAXT / 32; ++w) c += __popc(ps.mask[i][w] & s_headmask[w]);
            s_level[i] = c;
            atomicMax(&s_maxlevel, c);
        }
    }
    __syncthreads();

    // ---- the chains, level by level; wave w takes the heads of a level numbered w, w + NW, ...
    const int maxlevel = s_maxlevel;
    for (int lvl = 0; lvl <= maxlevel; ++lvl) {
        int k = 0;  // heads of this level seen so far, in id order
        for (int c0 = 0; c0 < Tb; c0 += 64) {
            const int i = c0 + lane;
            const unsigned long long hm = __ballot(i < Tb && s_level[i] == lvl);
            unsigned long long mine = hm;
            // keep the heads whose running number k + rank is this wave's modulo NW
            unsigned long long take = 0ull;
            int r = 0;
            while (mine) {
                const int bit = __ffsll(static_cast<unsigned long long>(mine)) - 1;
                mine &= mine - 1ull;
                if ((k + r) % NW == wave) take |= 1ull << bit;
                ++r;
            }
            k += r;
            while (take) {
                const int head = c0 + __ffsll(static_cast<unsigned long long>(take)) - 1;
                take &= take - 1ull;
                // ---- one chain from head: state from the parent's snapshot (or S0)
                const int p = s_par[head];
                const float *src = (p < 0) ? a.S0 + static_cast<size_t>(bh) * SS
                                           : a.snap + ((static_cast<size_t>(b) * T + p) * H + h) * SS;
                float4 S[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) S[m] = reinterpret_cast<const float4 *>(src + (rg + 16 * m) * D + col)[0];
                int node = head;
                NodeIn cur;
                load_node<BF>(cur, a.q, a.k, qkbase + static_cast<size_t>(node) * qkrs, rg, a.v,
                              base + static_cast<size_t>(node) * rs + col, a.alpha, a.beta,
                              sbase + static_cast<size_t>(node) * H);
                while (node >= 0) {
                    const int nxt = s_heavy[node];
                    // the next node's inputs are requested before this step (the node itself
                    // again at the chain's end, unused)
                    const int nl = nxt >= 0 ? nxt : node;
                    NodeIn nin;
                    load_node<BF>(nin, a.q, a.k, qkbase + static_cast<size_t>(nl) * qkrs, rg, a.v,
                                  base + static_cast<size_t>(nl) * rs + col, a.alpha, a.beta,
                                  sbase + static_cast<size_t>(nl) * H);
                    float4 o, u;
                    gdn_step(S, cur, o, u);
                    const size_t nodeo = base + static_cast<size_t>(node) * rs + col;
                    if (rg == 0) {
                        reinterpret_cast<float4 *>(a.O + nodeo)[0] = o;
                        reinterpret_cast<float4 *>(a.U + nodeo)[0] = u;
                    }
                    if (s_nch[node] >= 2) {  // a fork: light chains start from this state
                        float *dst = a.snap + ((static_cast<size_t>(b) * T + node) * H + h) * SS;
#pragma unroll
                        for (int m = 0; m < 8; ++m) reinterpret_cast<float4 *>(dst + (rg + 16 * m) * D + col)[0] = S[m];
                    }
                    cur = nin;
                    node = nxt;
                }
            }
        }
        // the level's fork snapshots are complete before the next level reads them
        __syncthreads();
    }
}

template <int NW>
static hipError_t launch_hybrid_nw(const SerialArgs &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * (D / 16))), block(NW * 64);
    if (a.bf16)
        hipLaunchKernelGGL((hybrid_kernel<true, NW>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((hybrid_kernel<false, NW>), grid, block, 0, stream, a);
    return hipGetLastError();
}

// Waves per workgroup: more waves run more chains of a level at once but leave fewer
// workgroups per CU. Measured on MI355X (µs, 4 / 8 / 16 waves): B = 1, H = 32, T = 16:
// 17.4 / 15.1 / 15.7; T = 256 random: 118 / 96 / 86; B = 16, T = 64: 283 / 403 / 700. With
// 64 or more (sequence, head) pairs, 8 waves also lost on level trees of width 2-8 at
// T = 128-256 (up to 2.5x at B = 4), so only a single sequence's 32 heads get wider groups.
hipError_t launch_hybrid(const SerialArgs &a, hipStream_t stream) {
    if (static_cast<long long>(a.B) * a.H <= 32)
        return a.T > 64 ? launch_hybrid_nw<16>(a, stream) : launch_hybrid_nw<8>(a, stream);
    return launch_hybrid_nw<4>(a, stream);
}

}  // namespace canopy
