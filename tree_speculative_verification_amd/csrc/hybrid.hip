// Chain-decomposed hybrid ("What the papers report": SpecLA's chain-decomposed hybrid; "M4",
// optional third contender: heavy-light decomposition, each chain serial, chains in parallel).
// The tree is cut into heavy paths: every node's heavy child is the child with the largest
// subtree (the lowest id on ties), and a chain starts at a root or at a light child. A chain's
// level is the number of light edges above it, at most log2(T). The chains form one work list
// ordered by (level, head id); each wave takes the next chain, waits until the snapshot of its
// head's parent exists (a chain of a lower level writes it), and walks the chain node by node
// with the state slice in registers (the serial recurrence, canopy_step.hpp), starting from that
// snapshot or from S0 for a root. Only fork nodes (two or more children) write snapshots, and
// each publishes a flag once its snapshot is written. Chains are handed out in level order, so
// the chain a wave waits for is always already held by a wave that does not wait on anything
// later: the list drains. One workgroup per (sequence, head, 16 value columns), NW waves; the
// decomposition is computed in LDS from the ancestor bitmask of the shared tree prep.
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
    __shared__ int s_order[HMAXT], s_ready[HMAXT];
    __shared__ int s_maxlevel, s_nheads, s_next;
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
            s_ready[i] = 0;
        }
    }
    if (tid < HMAXT / 32) s_headmask[tid] = 0u;
    if (tid == 0) {
        s_maxlevel = 0;
        s_next = 0;
    }
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

    // ---- the work list: heads in (level, id) order, built by wave 0
    if (wave == 0) {
        const int maxlevel = s_maxlevel;
        int cnt = 0;
        for (int lvl = 0; lvl <= maxlevel; ++lvl) {
            for (int c0 = 0; c0 < Tb; c0 += 64) {
                const int i = c0 + lane;
                const unsigned long long hm = __ballot(i < Tb && s_level[i] == lvl);
                if ((hm >> lane) & 1ull) s_order[cnt + __popcll(hm & ((1ull << lane) - 1ull))] = i;
                cnt += __popcll(hm);
            }
        }
        if (lane == 0) s_nheads = cnt;
    }
    __syncthreads();

    // ---- the chains, each wave taking the next one from the list
    const int nheads = s_nheads;
    for (;;) {
        int idx = 0;
        if (lane == 0) idx = atomicAdd(&s_next, 1);
        idx = __shfl(idx, 0, 64);
        if (idx >= nheads) break;
        const int head = s_order[idx];
        const int p = s_par[head];
        // the head's inputs are requested before waiting for its starting state
        int node = head;
        NodeIn cur;
        load_node<BF>(cur, a.q, a.k, qkbase + static_cast<size_t>(node) * qkrs, rg, a.v,
                      base + static_cast<size_t>(node) * rs + col, a.alpha, a.beta,
                      sbase + static_cast<size_t>(node) * H);
        // a chain whose starting snapshot never came (or came from such a chain) is lost: its
        // nodes get NaN outputs and its forks pass the loss on
        const bool lost = p >= 0 && wait_flag(&s_ready[p], a.wait_bound) != 1;
        if (lost && lane == 0) report_lost(a.tree_status, b);
        // ---- one chain from head: state from the parent's snapshot (or S0)
        const float *src = (p < 0) ? a.S0 + static_cast<size_t>(bh) * SS
                                   : a.snap + ((static_cast<size_t>(b) * T + p) * H + h) * SS;
        float4 S[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) S[m] = reinterpret_cast<const float4 *>(src + (rg + 16 * m) * D + col)[0];
        while (node >= 0) {
            const int nxt = s_heavy[node];
            // the next node's inputs are requested before this step (the node itself again at
            // the chain's end, unused)
            const int nl = nxt >= 0 ? nxt : node;
            NodeIn nin;
            load_node<BF>(nin, a.q, a.k, qkbase + static_cast<size_t>(nl) * qkrs, rg, a.v,
                          base + static_cast<size_t>(nl) * rs + col, a.alpha, a.beta,
                          sbase + static_cast<size_t>(nl) * H);
            float4 o, u;
            gdn_step(S, cur, o, u);
            const size_t nodeo = base + static_cast<size_t>(node) * rs + col;
            if (rg == 0) {
                // selected per component: a select of whole float4 values goes through scratch
                const float qnan = __builtin_nanf("");
                const float4 ow = make_float4(lost ? qnan : o.x, lost ? qnan : o.y, lost ? qnan : o.z, lost ? qnan : o.w);
                const float4 uw = make_float4(lost ? qnan : u.x, lost ? qnan : u.y, lost ? qnan : u.z, lost ? qnan : u.w);
                reinterpret_cast<float4 *>(a.O + nodeo)[0] = ow;
                reinterpret_cast<float4 *>(a.U + nodeo)[0] = uw;
            }
            if (s_nch[node] >= 2) {  // a fork: light chains start from this state
                float *dst = a.snap + ((static_cast<size_t>(b) * T + node) * H + h) * SS;
#pragma unroll
                for (int m = 0; m < 8; ++m) reinterpret_cast<float4 *>(dst + (rg + 16 * m) * D + col)[0] = S[m];
                // the snapshot is written before the flag that lets other waves read it
                __hip_atomic_store(&s_ready[node], lost ? 2 : 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            cur = nin;
            node = nxt;
        }
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
