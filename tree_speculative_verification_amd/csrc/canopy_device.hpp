// Device-side building blocks shared by the libcanopy kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace canopy {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// Plain 16-byte vector (HIP's uint4 is a struct with a union, which defeats scalar replacement
// of register arrays).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;  // d_k = d_v

// ----------------------------------------------------------------------------- small helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Makes this wave's earlier LDS writes visible to its later LDS reads across lanes: a wave's
// LDS operations complete in order, so it is enough to drain the LDS counter and keep the
// compiler from moving memory accesses across this point. Only LDS (not vector memory) is
// waited for, so loads to registers stay in flight.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier for LDS data only: every wave's earlier LDS writes are visible to every
// wave's later LDS reads. Unlike __syncthreads() it does not wait for this wave's outstanding
// vector memory operations (global stores, loads into registers or into LDS), so a barrier
// placed while such requests are in flight does not wait for them; data loaded into LDS must be
// waited for explicitly (wait_vmem) before the barrier that publishes it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Streaming store (the nt bit: the line is not kept in the caches for reuse), for outputs that
// nothing on the path reads again: the read-out O and the committed state. Measured on MI355X,
// it shortens verify by 4% at B = 16, T = 64 and T = 256 and the commit by 6%; U, which the
// commit reads back, stays an ordinary store (streaming it cost 10% with a cold cache), and so
// does the state of the one-launch step for trees of at most 16 nodes, whose lanes write it in
// 64-byte row segments (streaming was slower there, warm and cold).
__device__ __forceinline__ void store_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    return x;
}

// Tree status of a sequence in which a wave gave up waiting for a result that another wave of
// its workgroup publishes (never expected: see wait_flag).
constexpr int kStatusHandoffLost = -2;
// Default bound, in sleeps, of such a wait.
constexpr int kWaitBound = 1 << 24;

// Wait for a flag that another wave of the workgroup sets with a release store: 1 when its
// result is published, 2 when the publisher itself computed from a lost hand-off. Every wave
// of a workgroup is resident and no publisher waits for a wave that waits for it, so the flag
// is always set; the bound (in sleeps) only guarantees that the wait ends. Returns the flag, or
// 0 when the bound ran out; the value is the same in every lane (the acquire load reads one
// LDS word for the whole wave).
__device__ __forceinline__ int wait_flag(int *flag, int bound) {
    for (int n = 0; n < bound; ++n) {
        const int v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (v != 0) return v;
        __builtin_amdgcn_s_sleep(1);
    }
    return 0;
}

// Record a lost hand-off of sequence b in tree_status (if given). The sequence's own status
// store (0 for a valid tree) comes right after its tree preprocessing; a lost hand-off is only
// known after a full wait bound, so this store lands after it.
__device__ __forceinline__ void report_lost(int32_t *tree_status, int b) {
    if (tree_status)
        __hip_atomic_store(tree_status + b, kStatusHandoffLost, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Blocks of a launch are spread round-robin over the 8 XCDs (each with its own L2). Map the
// hardware block id so that consecutive logical ids run on one XCD: logical ids that share a
// (batch, head) then share that XCD's L2 copy of its keys and queries.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    constexpr int X = 8;
    const int full = (nblk / X) * X;
    if (bid >= full) return bid;
    const int per = nblk / X;
    return (bid % X) * per + bid / X;
}

// ----------------------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32. For a 16x16 output tile and a 32-long
// reduction slice, lane l supplies row (l % 16) of A and column (l % 16) of B, each at the
// 8 reduction indices 8*(l/16) .. 8*(l/16)+7 of the slice. The result holds, in lane l,
// rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16 (and four v_mfma_f32_16x16x4_f32): a 16-long reduction in which
// lane l supplies row (l % 16) of A and column (l % 16) of B at reduction indices
// 4*(l/16) .. 4*(l/16)+3. That is the lane placement of the 16x16 result tile itself (rows
// 4*(l/16) .. +3 of column l % 16), so a result tile whose rows index the next reduction feeds
// that product as its B operand without moving data between lanes.
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
__device__ __forceinline__ f32x4 mfma_bf16_k16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// The same 16-long reduction on fp32 data with exact products: four v_mfma_f32_16x16x4_f32,
// instruction e pairing value e of every lane (row r of A at index 4g+e with row 4g+e of B).
// Operands computed on the VALU feed it directly, with no bf16 splitting.
__device__ __forceinline__ f32x4 mma16f(const float (&a)[4], const float (&b)[4], f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = mfma_f32(a[e], b[e], c);
    return c;
}
__device__ __forceinline__ f32x4 mma16f(const float (&a)[4], f32x4 b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = mfma_f32(a[e], b[e], c);
    return c;
}


// Operand fragments: 8 consecutive reduction-index values of one row (A) or column (B).
// bf16 inputs are exact in one bf16 fragment; fp32 data (S0, G, C, U) used with bf16 inputs is
// split into hi + lo bf16 parts (|x - hi - lo| <= 2^-16 |x|) and multiplied in up to three
// passes (hi*hi + hi*lo + lo*hi). fp32 inputs use fp32 MFMA with exact fp32 products.
//
// Input rows (q, k: 128 values) staged in LDS use 16-byte chunks with the chunk index XORed
// with (row % 16): the 16 rows a fragment read touches then fall in distinct banks.
template <bool BF>
struct Ops;

template <>
struct Ops<true> {
    struct In { bf16x8 x; };            // exact input fragment
    struct Sp { bf16x8 hi, lo; };       // split fp32 fragment
    static constexpr int ROWB = D * 2;  // bytes of one staged input row
    static constexpr int ES = 2;        // bytes per input element

    __device__ static __forceinline__ float in_scalar(const void *base, size_t elem) {
        return bf16_to_f32(static_cast<const uint16_t *>(base)[elem]);
    }
    // Fragment straight from global memory: 8 consecutive elements at `elem` (16-byte aligned).
    template <class F>
    __device__ static __forceinline__ F load_frag(const void *base, size_t elem, bool valid) {
        F r;
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (valid) raw = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + elem);
        r.x = __builtin_bit_cast(bf16x8, raw);
        return r;
    }
    typedef uint16_t Raw;  // an input element as loaded, converted only where it is used
    __device__ static __forceinline__ Raw load_raw(const void *base, size_t elem) {
        return static_cast<const uint16_t *>(base)[elem];
    }
    __device__ static __forceinline__ float raw_f32(Raw r) { return bf16_to_f32(r); }
    // Fragment of staged row `row`, reduction indices 8*g8 .. 8*g8+7.
    __device__ static __forceinline__ In lds_frag(const uint8_t *buf, int row, int g8) {
        In r;
        r.x = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                             buf + row * ROWB + ((g8 ^ (row & 15)) << 4)));
        return r;
    }
    // The inverse of lds_frag: store a fragment into the swizzled row layout.
    __device__ static __forceinline__ void lds_put(uint8_t *buf, int row, int g8, In f) {
        *reinterpret_cast<u32x4 *>(buf + row * ROWB + ((g8 ^ (row & 15)) << 4)) =
            __builtin_bit_cast(u32x4, f.x);
    }
    __device__ static __forceinline__ Sp split(const float (&v)[8]) {
        Sp s;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const __bf16 h = static_cast<__bf16>(v[e]);
            s.hi[e] = h;
            s.lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
        }
        return s;
    }
    __device__ static __forceinline__ f32x4 mma(In a, In b, f32x4 c) { return mfma_bf16(a.x, b.x, c); }
    __device__ static __forceinline__ f32x4 mma(In a, Sp b, f32x4 c) {
        c = mfma_bf16(a.x, b.hi, c);
        return mfma_bf16(a.x, b.lo, c);
    }
    __device__ static __forceinline__ f32x4 mma(Sp a, Sp b, f32x4 c) {
        c = mfma_bf16(a.hi, b.hi, c);
        c = mfma_bf16(a.hi, b.lo, c);
        return mfma_bf16(a.lo, b.hi, c);
    }
    // 16-long reductions on fp32 data (4 values per lane, split like Sp).
    struct Sp4 { i16x4 hi, lo; };
    __device__ static __forceinline__ Sp4 split4(const float (&v)[4]) {
        Sp4 s;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __bf16 h = static_cast<__bf16>(v[e]);
            s.hi[e] = __builtin_bit_cast(short, h);
            s.lo[e] = __builtin_bit_cast(short, static_cast<__bf16>(v[e] - static_cast<float>(h)));
        }
        return s;
    }
    __device__ static __forceinline__ f32x4 mma16(Sp4 a, Sp4 b, f32x4 c) {
        c = mfma_bf16_k16(a.hi, b.hi, c);
        c = mfma_bf16_k16(a.hi, b.lo, c);
        return mfma_bf16_k16(a.lo, b.hi, c);
    }
};

template <>
struct Ops<false> {
    struct In { float x[8]; };
    typedef In Sp;
    static constexpr int ROWB = D * 4;
    static constexpr int ES = 4;

    __device__ static __forceinline__ float in_scalar(const void *base, size_t elem) {
        return static_cast<const float *>(base)[elem];
    }
    template <class F>
    __device__ static __forceinline__ F load_frag(const void *base, size_t elem, bool valid) {
        F r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r.x[e] = 0.f;
        if (valid) {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
            const float4 x = p[0], y = p[1];
            r.x[0] = x.x; r.x[1] = x.y; r.x[2] = x.z; r.x[3] = x.w;
            r.x[4] = y.x; r.x[5] = y.y; r.x[6] = y.z; r.x[7] = y.w;
        }
        return r;
    }
    typedef float Raw;
    __device__ static __forceinline__ Raw load_raw(const void *base, size_t elem) {
        return static_cast<const float *>(base)[elem];
    }
    __device__ static __forceinline__ float raw_f32(Raw r) { return r; }
    __device__ static __forceinline__ In lds_frag(const uint8_t *buf, int row, int g8) {
        In r;
        const uint8_t *p = buf + row * ROWB;
        const float4 a = *reinterpret_cast<const float4 *>(p + (((2 * g8) ^ (row & 15)) << 4));
        const float4 b = *reinterpret_cast<const float4 *>(p + (((2 * g8 + 1) ^ (row & 15)) << 4));
        r.x[0] = a.x; r.x[1] = a.y; r.x[2] = a.z; r.x[3] = a.w;
        r.x[4] = b.x; r.x[5] = b.y; r.x[6] = b.z; r.x[7] = b.w;
        return r;
    }
    __device__ static __forceinline__ void lds_put(uint8_t *buf, int row, int g8, In f) {
        uint8_t *p = buf + row * ROWB;
        *reinterpret_cast<float4 *>(p + (((2 * g8) ^ (row & 15)) << 4)) = make_float4(f.x[0], f.x[1], f.x[2], f.x[3]);
        *reinterpret_cast<float4 *>(p + (((2 * g8 + 1) ^ (row & 15)) << 4)) = make_float4(f.x[4], f.x[5], f.x[6], f.x[7]);
    }
    __device__ static __forceinline__ Sp split(const float (&v)[8]) {
        Sp s;
#pragma unroll
        for (int e = 0; e < 8; ++e) s.x[e] = v[e];
        return s;
    }
    __device__ static __forceinline__ f32x4 mma(In a, In b, f32x4 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = mfma_f32(a.x[e], b.x[e], c);
        return c;
    }
    struct Sp4 { float x[4]; };
    __device__ static __forceinline__ Sp4 split4(const float (&v)[4]) {
        Sp4 s;
#pragma unroll
        for (int e = 0; e < 4; ++e) s.x[e] = v[e];
        return s;
    }
    // Instruction e pairs value e of every lane: row r of A at index 4g+e with row 4g+e of B.
    __device__ static __forceinline__ f32x4 mma16(Sp4 a, Sp4 b, f32x4 c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) c = mfma_f32(a.x[e], b.x[e], c);
        return c;
    }
};

// One 64-row block of q or k (rows row0 .. row0+63 of one head; rows >= T repeat row T-1)
// copied into the swizzled LDS layout through registers: issue() loads each thread's 16-byte
// chunks (consecutive threads, consecutive chunks of a row), commit() stores them. The loads
// stay in flight across other work until commit() needs them.
template <bool BF, int NT>
struct BlockCopy {
    static constexpr int ROWB = Ops<BF>::ROWB;
    static constexpr int ES = ROWB / D;        // bytes per element
    static constexpr int CPR = ROWB / 16;      // chunks per row
    static constexpr int PER = 64 * CPR / NT;  // chunks per thread
    u32x4 r[PER];
    __device__ __forceinline__ void issue(const void *g, size_t base, size_t rs, int row0, int T) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int idx = threadIdx.x + m * NT;
            const int row = idx / CPR, ch = idx % CPR;
            const int gr = min(row0 + row, T - 1);
            r[m] = *reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(g) +
                                                    (base + static_cast<size_t>(gr) * rs) * ES + ch * 16);
        }
    }
    __device__ __forceinline__ void commit(uint8_t *buf) const {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int idx = threadIdx.x + m * NT;
            const int row = idx / CPR, ch = idx % CPR;
            *reinterpret_cast<u32x4 *>(buf + row * ROWB + ((ch ^ (row & 15)) << 4)) = r[m];
        }
    }
};

// One wave's 16 value columns of a 64-row block (rows >= T repeat row T-1), through registers
// into a per-wave LDS buffer [64 rows][16 columns]: each 16-byte chunk holds 8 (bf16) or
// 4 (fp32) columns of one row, so a row is 2 or 4 chunks.
template <bool BF>
struct VCopy {
    static constexpr int ES = Ops<BF>::ES;
    static constexpr int CPR = 16 * ES / 16;  // chunks per row
    static constexpr int PER = 64 * CPR / 64; // chunks per lane
    u32x4 r[PER];
    __device__ __forceinline__ void issue(const void *g, size_t base, size_t rs, int col0, int row0,
                                          int T, int lane) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int idx = lane + 64 * m;
            const int row = idx / CPR, ch = idx % CPR;
            const int gr = min(row0 + row, T - 1);
            r[m] = *reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(g) +
                                                    (base + static_cast<size_t>(gr) * rs + col0) * ES + ch * 16);
        }
    }
    __device__ __forceinline__ void commit(uint8_t *buf, int lane) const {
#pragma unroll
        for (int m = 0; m < PER; ++m) *reinterpret_cast<u32x4 *>(buf + (lane + 64 * m) * 16) = r[m];
    }
    __device__ static __forceinline__ float get(const uint8_t *buf, int row, int col) {
        if constexpr (BF)
            return bf16_to_f32(*reinterpret_cast<const uint16_t *>(buf + (row * 16 + col) * 2));
        else
            return *reinterpret_cast<const float *>(buf + (row * 16 + col) * 4);
    }
};

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane l's
// data lands at lds_base + 16 * l; lds_base must be the same for the whole wave.
__device__ __forceinline__ void dma16(const void *gsrc, void *lds_base) {
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1))) *)gsrc,
        (void __attribute__((address_space(3))) *)lds_base, 16, 0, 0);
}

// The same block copy with LDS-bound loads: no registers are held while the data is in flight.
// Wave w issues the 1-KB pieces w, w + NW, ...; a piece is 1024 / ROWB rows, and lane l fetches
// the global chunk that the swizzle places at piece offset 16 * l.
template <bool BF, int NT>
__device__ __forceinline__ void dma_block(uint8_t *buf, const void *g, size_t base, size_t rs,
                                          int row0, int T) {
    using BC = BlockCopy<BF, NT>;
    constexpr int PIECES = 64 * BC::ROWB / 1024;
    constexpr int RPP = 1024 / BC::ROWB;  // rows per piece
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int s = wave; s < PIECES; s += NT / 64) {
        const int row = RPP * s + lane / BC::CPR;
        const int ch = (lane % BC::CPR) ^ (row & 15);
        const int gr = min(row0 + row, T - 1);
        dma16(static_cast<const uint8_t *>(g) + (base + static_cast<size_t>(gr) * rs) * BC::ES + ch * 16,
              buf + s * 1024);
    }
}

// One wave's 16 value columns of a 64-row block with LDS-bound loads, in the VCopy layout
// [row][16 columns]: a 1-KB piece holds 1024 / (16 * ES) rows.
template <bool BF>
__device__ __forceinline__ void dma_v(uint8_t *buf, const void *g, size_t base, size_t rs, int col0,
                                      int row0, int T, int lane) {
    constexpr int ES = Ops<BF>::ES;
    constexpr int LPR = 16 * ES / 16;          // lanes (16-byte chunks) per row
    constexpr int PIECES = 64 * 16 * ES / 1024;
#pragma unroll
    for (int s = 0; s < PIECES; ++s) {
        const int row = s * (64 / LPR) + lane / LPR;
        const int ch = lane % LPR;
        const int gr = min(row0 + row, T - 1);
        dma16(static_cast<const uint8_t *>(g) + (base + static_cast<size_t>(gr) * rs + col0) * ES + ch * 16,
              buf + s * 1024);
    }
}

// Buffer resource over the memory at p (32-bit byte offsets from it, no range limit): a base
// held in scalar registers, so that per-lane addresses are one 32-bit offset. p must be the
// same in every lane; it is read from the first active lane, which tells the compiler so (a
// resource it takes for divergent would turn every access into a loop over lanes).
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    void *u = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, -1, 0x00020000);
}

// Wait until this wave's LDS-bound loads (and other vector memory operations) have completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same copy without holding the whole block in registers (for small workgroups):
// eight chunks per thread at a time.
template <bool BF, int NT>
__device__ __forceinline__ void copy_block(uint8_t *buf, const void *g, size_t base, size_t rs,
                                           int row0, int T) {
    using BC = BlockCopy<BF, NT>;
    for (int m0 = 0; m0 < BC::PER; m0 += 8) {
        u32x4 r[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int idx = threadIdx.x + (m0 + m) * NT;
            const int row = idx / BC::CPR, ch = idx % BC::CPR;
            const int gr = min(row0 + row, T - 1);
            r[m] = *reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(g) +
                                                    (base + static_cast<size_t>(gr) * rs) * BC::ES + ch * 16);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int idx = threadIdx.x + (m0 + m) * NT;
            const int row = idx / BC::CPR, ch = idx % BC::CPR;
            *reinterpret_cast<u32x4 *>(buf + row * BC::ROWB + ((ch ^ (row & 15)) << 4)) = r[m];
        }
    }
}

}  // namespace canopy
