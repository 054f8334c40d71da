// Device helpers shared by the libtqkv kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16x16x32(const half8& a, const half8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Pins a value in a register.  A hi/lo split h = fp16(v), l = fp16((v - h) * 2^12)
// is only exact if both parts see the same fp32 v; with fp contraction the
// compiler may otherwise fuse the product that forms v into one use (rounding
// the exact product to fp16) and not into the other, and h + l / 2^12 then
// misses v by one fp16 ulp.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

// Bits [BIT, BIT + N) of a little-endian dword array held in registers
// (BIT and N known at compile time after unrolling).
template <int BIT, int N, int NW>
__device__ __forceinline__ uint32_t bits_of(const uint32_t (&w)[NW]) {
    constexpr int i = BIT >> 5, s = BIT & 31;
    constexpr uint32_t mask = (N >= 32) ? 0xffffffffu : ((1u << N) - 1u);
    if constexpr (s + N <= 32) {
        return (w[i] >> s) & mask;
    } else {
        return ((w[i] >> s) | (w[i + 1] << (32 - s))) & mask;
    }
}

// Runtime variant over a byte pointer with dword alignment of the base.
__device__ __forceinline__ uint32_t bits_at(const uint32_t* w, int bit, int n) {
    const int i = bit >> 5, s = bit & 31;
    uint64_t v = w[i];
    if (s + n > 32) v |= (uint64_t)w[i + 1] << 32;
    return (uint32_t)(v >> s) & ((1u << n) - 1u);
}

// Nearest grid angle -pi + 2 pi b / L of the pair (x, y), L = 2^tb, tb = 1 .. 4;
// b = L/2 (angle 0) for an exactly zero pair.  The pair is turned by half a
// bin so that the bin edges become the sector edges 2 pi k / L.  Without
// branches: the octant o of the turned pair (X, Y) follows from three sign
// bits, s_Y, s_X and the sign of |X| - |Y|, in Gray order (o = 4 a + 2 (a ^ b)
// + (a ^ b ^ c)); the half octant from the sign of tan(pi/8) max(|X|, |Y|) -
// min(|X|, |Y|), read the other way round in odd octants (there the octant
// starts on a diagonal).  k16 = 2 o + half is the sector at L = 16, and k16 >>
// (4 - tb) at L = 2^tb.  A decision can differ from the exact one only for a
// pair within about 1e-7 of its radius from a sector edge.  (hc, hs) = (cos,
// sin) of pi / L.
__device__ __forceinline__ int angle_code(float x, float y, int tb, float hc, float hs) {
    const float X = x * hc - y * hs, Y = x * hs + y * hc;
    const float ax = fabsf(X), ay = fabsf(Y);
    const float C = ax - ay;
    const float E = 0.41421356237309505f * fmaxf(ax, ay) - fminf(ax, ay);
    const uint32_t A = __float_as_uint(Y), w1 = A ^ __float_as_uint(X), w2 = w1 ^ __float_as_uint(C),
                   w3 = w2 ^ __float_as_uint(E);
    uint32_t k = A >> 31;
    k = (k << 1) | (w1 >> 31);
    k = (k << 1) | (w2 >> 31);
    k = (k << 1) | (w3 >> 31);
    return (int)((k ^ 8u) >> (4 - tb));  // + L/2: angles from -pi
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float half_at(const uint8_t* p) {
    return (float)(*reinterpret_cast<const _Float16*>(p));
}

}  // namespace tq
