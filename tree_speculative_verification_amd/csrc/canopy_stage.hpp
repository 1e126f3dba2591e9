// Staging of 64 x 64 blocks of the masked, decay-weighted Gram matrices (-G and C) in LDS, as
// MFMA A operands, shared by the blocked verify kernels ("The tree closed form" on the canopy
// project page: G and C of one block row against one block column).
#pragma once
#include "canopy_device.hpp"

namespace canopy {

// Staging of one 64 x 64 block pair of -G and C in LDS, as MFMA A operands.
template <bool BF>
struct Stage;

// bf16 hi/lo parts, rows of 8 x 16-byte chunks; chunk index XOR ((row / 2) % 8) so that the
// 16 rows of a fragment read land in distinct banks.
template <>
struct Stage<true> {
    alignas(16) uint8_t gh[64 * 128];
    alignas(16) uint8_t gl[64 * 128];
    alignas(16) uint8_t ch[64 * 128];
    alignas(16) uint8_t cl[64 * 128];
    __device__ static __forceinline__ int off(int r, int c) {
        return r * 128 + ((((c >> 3) ^ ((r >> 1) & 7))) << 4) + ((c & 7) << 1);
    }
    __device__ __forceinline__ void store(int r, int c, float g, float cv) {
        const __bf16 g1 = static_cast<__bf16>(g), c1 = static_cast<__bf16>(cv);
        const __bf16 g2 = static_cast<__bf16>(g - static_cast<float>(g1));
        const __bf16 c2 = static_cast<__bf16>(cv - static_cast<float>(c1));
        const int o = off(r, c);
        *reinterpret_cast<__bf16 *>(gh + o) = g1;
        *reinterpret_cast<__bf16 *>(gl + o) = g2;
        *reinterpret_cast<__bf16 *>(ch + o) = c1;
        *reinterpret_cast<__bf16 *>(cl + o) = c2;
    }
    // G and C at row r, columns c0 .. c0+3 (c0 % 4 == 0): one 8-byte store per array.
    __device__ __forceinline__ void store4(int r, int c0, const float (&g)[4], const float (&cv)[4]) {
        uint16_t gh4[4], gl4[4], ch4[4], cl4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __bf16 g1 = static_cast<__bf16>(g[e]), c1 = static_cast<__bf16>(cv[e]);
            gh4[e] = __builtin_bit_cast(uint16_t, g1);
            gl4[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(g[e] - static_cast<float>(g1)));
            ch4[e] = __builtin_bit_cast(uint16_t, c1);
            cl4[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(cv[e] - static_cast<float>(c1)));
        }
        const int o = off(r, c0);
        auto pack = [](const uint16_t (&x)[4]) {
            return make_uint2(x[0] | (static_cast<uint32_t>(x[1]) << 16), x[2] | (static_cast<uint32_t>(x[3]) << 16));
        };
        *reinterpret_cast<uint2 *>(gh + o) = pack(gh4);
        *reinterpret_cast<uint2 *>(gl + o) = pack(gl4);
        *reinterpret_cast<uint2 *>(ch + o) = pack(ch4);
        *reinterpret_cast<uint2 *>(cl + o) = pack(cl4);
    }
    // G alone at row r, columns c0 .. c0+3.
    __device__ __forceinline__ void store4G(int r, int c0, const float (&g)[4]) {
        uint16_t gh4[4], gl4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __bf16 g1 = static_cast<__bf16>(g[e]);
            gh4[e] = __builtin_bit_cast(uint16_t, g1);
            gl4[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(g[e] - static_cast<float>(g1)));
        }
        const int o = off(r, c0);
        *reinterpret_cast<uint2 *>(gh + o) =
            make_uint2(gh4[0] | (static_cast<uint32_t>(gh4[1]) << 16), gh4[2] | (static_cast<uint32_t>(gh4[3]) << 16));
        *reinterpret_cast<uint2 *>(gl + o) =
            make_uint2(gl4[0] | (static_cast<uint32_t>(gl4[1]) << 16), gl4[2] | (static_cast<uint32_t>(gl4[3]) << 16));
    }
    // Zero the 16 x 16 tile at (r0, c0) of all four arrays: 128 chunks, two per lane.
    __device__ __forceinline__ void zero_tile(int r0, int c0, int lane) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int idx = lane + 64 * a;
            const int row = idx & 15, half = (idx >> 4) & 1, arr = idx >> 5;
            uint8_t *base = arr == 0 ? gh : arr == 1 ? gl : arr == 2 ? ch : cl;
            *reinterpret_cast<uint4 *>(base + off(r0 + row, c0 + 8 * half)) = make_uint4(0, 0, 0, 0);
        }
    }
    // Overwrite G[r0 + i][c0 + lr] (i = 0..15) with x[i]: a column of a 16 x 16 tile.
    __device__ __forceinline__ void put_col16(int r0, int c0, int lr, const float (&x)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const __bf16 h1 = static_cast<__bf16>(x[i]);
            const __bf16 l1 = static_cast<__bf16>(x[i] - static_cast<float>(h1));
            const int o = off(r0 + i, c0 + lr);
            *reinterpret_cast<__bf16 *>(gh + o) = h1;
            *reinterpret_cast<__bf16 *>(gl + o) = l1;
        }
    }
    __device__ __forceinline__ Ops<true>::Sp frag(const uint8_t *h, const uint8_t *l, int r, int k0) const {
        const int o = off(r, k0);
        Ops<true>::Sp s;
        s.hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(h + o));
        s.lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(l + o));
        return s;
    }
    __device__ __forceinline__ Ops<true>::Sp fragG(int r, int k0) const { return frag(gh, gl, r, k0); }
    __device__ __forceinline__ Ops<true>::Sp fragC(int r, int k0) const { return frag(ch, cl, r, k0); }
    __device__ __forceinline__ float getG(int r, int c) const {
        const int o = off(r, c);
        return static_cast<float>(*reinterpret_cast<const __bf16 *>(gh + o)) +
               static_cast<float>(*reinterpret_cast<const __bf16 *>(gl + o));
    }
    // The staged values G[r][c0 .. c0+3] (c0 a multiple of 4): one 8-byte read per part.
    __device__ __forceinline__ void getG4(int r, int c0, float (&out)[4]) const {
        const int o = off(r, c0);
        const uint2 h = *reinterpret_cast<const uint2 *>(gh + o);
        const uint2 l = *reinterpret_cast<const uint2 *>(gl + o);
        const uint32_t hw[2] = {h.x, h.y}, lw[2] = {l.x, l.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t hb = (e & 1) ? (hw[e >> 1] >> 16) : (hw[e >> 1] & 0xFFFFu);
            const uint32_t lb = (e & 1) ? (lw[e >> 1] >> 16) : (lw[e >> 1] & 0xFFFFu);
            out[e] = __uint_as_float(hb << 16) + __uint_as_float(lb << 16);
        }
    }
    // The 16 staged values G[r][c0 .. c0+15] (c0 a multiple of 16).
    __device__ __forceinline__ void rowG16(int r, int c0, float (&out)[16]) const {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int o = off(r, c0 + 8 * hh);
            const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(gh + o));
            const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(gl + o));
#pragma unroll
            for (int e = 0; e < 8; ++e) out[8 * hh + e] = static_cast<float>(a[e]) + static_cast<float>(b[e]);
        }
    }
};

// fp32, rows of 16 x 16-byte chunks, chunk index XOR (row % 16).
template <>
struct Stage<false> {
    alignas(16) uint8_t g[64 * 256];
    alignas(16) uint8_t c[64 * 256];
    __device__ static __forceinline__ int off(int r, int cc) {
        return r * 256 + (((cc >> 2) ^ (r & 15)) << 4) + ((cc & 3) << 2);
    }
    __device__ __forceinline__ void store(int r, int cc, float gv, float cv) {
        const int o = off(r, cc);
        *reinterpret_cast<float *>(g + o) = gv;
        *reinterpret_cast<float *>(c + o) = cv;
    }
    __device__ __forceinline__ void store4(int r, int c0, const float (&gv)[4], const float (&cv)[4]) {
        const int o = off(r, c0);
        *reinterpret_cast<float4 *>(g + o) = make_float4(gv[0], gv[1], gv[2], gv[3]);
        *reinterpret_cast<float4 *>(c + o) = make_float4(cv[0], cv[1], cv[2], cv[3]);
    }
    __device__ __forceinline__ void store4G(int r, int c0, const float (&gv)[4]) {
        *reinterpret_cast<float4 *>(g + off(r, c0)) = make_float4(gv[0], gv[1], gv[2], gv[3]);
    }
    __device__ __forceinline__ void zero_tile(int r0, int c0, int lane) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int idx = lane + 64 * a;
            const int row = idx & 15, q = (idx >> 4) & 3, arr = idx >> 6;
            uint8_t *base = arr == 0 ? g : c;
            *reinterpret_cast<uint4 *>(base + off(r0 + row, c0 + 4 * q)) = make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void put_col16(int r0, int c0, int lr, const float (&x)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) *reinterpret_cast<float *>(g + off(r0 + i, c0 + lr)) = x[i];
    }
    __device__ __forceinline__ Ops<false>::Sp frag(const uint8_t *m, int r, int k0) const {
        Ops<false>::Sp s;
        const float4 x = *reinterpret_cast<const float4 *>(m + off(r, k0));
        const float4 y = *reinterpret_cast<const float4 *>(m + off(r, k0 + 4));
        s.x[0] = x.x; s.x[1] = x.y; s.x[2] = x.z; s.x[3] = x.w;
        s.x[4] = y.x; s.x[5] = y.y; s.x[6] = y.z; s.x[7] = y.w;
        return s;
    }
    __device__ __forceinline__ Ops<false>::Sp fragG(int r, int k0) const { return frag(g, r, k0); }
    __device__ __forceinline__ Ops<false>::Sp fragC(int r, int k0) const { return frag(c, r, k0); }
    __device__ __forceinline__ float getG(int r, int cc) const {
        return *reinterpret_cast<const float *>(g + off(r, cc));
    }
    __device__ __forceinline__ void getG4(int r, int c0, float (&out)[4]) const {
        const float4 x = *reinterpret_cast<const float4 *>(g + off(r, c0));
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    }
    __device__ __forceinline__ void rowG16(int r, int c0, float (&out)[16]) const {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 x = *reinterpret_cast<const float4 *>(g + off(r, c0 + 4 * q));
            out[4 * q] = x.x; out[4 * q + 1] = x.y; out[4 * q + 2] = x.z; out[4 * q + 3] = x.w;
        }
    }
};

}  // namespace canopy
