// Device-side building blocks shared by the libcanopy kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace canopy {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int D = 128;  // d_k = d_v

// ----------------------------------------------------------------------------- small helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Makes this wave's earlier LDS writes visible to its later LDS reads across lanes. A wave's
// LDS operations complete in order; this stops the compiler from moving accesses across it.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    return x;
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

// Operand fragments: 8 consecutive reduction-index values of one row (A) or column (B).
// bf16 inputs are exact in one bf16 fragment; fp32 data (S0, G, C, U) used with bf16 inputs is
// split into hi + lo bf16 parts (|x - hi - lo| <= 2^-16 |x|) and multiplied in up to three
// passes (hi*hi + hi*lo + lo*hi). fp32 inputs use fp32 MFMA with exact fp32 products.
template <bool BF>
struct Ops;

template <>
struct Ops<true> {
    struct In { bf16x8 x; };            // exact input fragment
    struct Sp { bf16x8 hi, lo; };       // split fp32 fragment
    static constexpr int in_bytes = 2;

    __device__ static __forceinline__ In load_in(const void *base, size_t elem, bool valid) {
        In r;
        if (valid) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(
                static_cast<const uint16_t *>(base) + elem);
            r.x = __builtin_bit_cast(bf16x8, raw);
        } else {
            r.x = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        }
        return r;
    }
    __device__ static __forceinline__ float in_scalar(const void *base, size_t elem) {
        return bf16_to_f32(static_cast<const uint16_t *>(base)[elem]);
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
};

template <>
struct Ops<false> {
    struct In { float x[8]; };
    typedef In Sp;
    static constexpr int in_bytes = 4;

    __device__ static __forceinline__ In load_in(const void *base, size_t elem, bool valid) {
        In r;
        if (valid) {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
            const float4 a = p[0], b = p[1];
            r.x[0] = a.x; r.x[1] = a.y; r.x[2] = a.z; r.x[3] = a.w;
            r.x[4] = b.x; r.x[5] = b.y; r.x[6] = b.z; r.x[7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) r.x[e] = 0.f;
        }
        return r;
    }
    __device__ static __forceinline__ float in_scalar(const void *base, size_t elem) {
        return static_cast<const float *>(base)[elem];
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
};

}  // namespace canopy
