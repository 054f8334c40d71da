// Device helpers shared by the libtqkv kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

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

// Nearest grid angle -pi + 2 pi b / L of the pair (x, y), L = 2^tb, tb = 2 .. 4;
// b = L/2 (angle 0) for an exactly zero pair.  The pair is turned by half a
// bin so that the bin edges become the sector edges 2 pi k / L.  Without
// branches: the octant o of the turned pair (X, Y) follows from three sign
// bits, s_Y, s_X and the sign of |X| - |Y|, in Gray order (o = 4 a + 2 (a ^ b)
// + (a ^ b ^ c)); the half octant from the sign of tan(pi/8) max(|X|, |Y|) -
// min(|X|, |Y|), read the other way round in odd octants (there the octant
// starts on a diagonal).  k16 = 2 o + half is the sector at L = 16, and k16 >>
// (4 - tb) at L = 2^tb, so a format of tb angle bits needs only the first tb
// of the four sign tests (tb 2: the quadrant; tb 3: the octant; tb 4: the
// half octant too).  A decision can differ from the exact one only for a
// pair within about 1e-7 of its radius from a sector edge.  angle_sector_t
// takes the turned pair (X, Y); angle_code_t turns (x, y) itself, with (hc,
// hs) = (cos, sin) of pi / L.
template <int TB>
__device__ __forceinline__ int angle_sector_t(float X, float Y) {
    static_assert(TB >= 2 && TB <= 4, "angle bits 2 .. 4");
    const uint32_t A = __float_as_uint(Y), w1 = A ^ __float_as_uint(X);
    uint32_t k = ((A >> 31) << 1) | (w1 >> 31);
    if constexpr (TB >= 3) {
        const float ax = fabsf(X), ay = fabsf(Y);
        const uint32_t w2 = w1 ^ __float_as_uint(ax - ay);
        k = (k << 1) | (w2 >> 31);
        if constexpr (TB >= 4) {
            const float E = 0.41421356237309505f * fmaxf(ax, ay) - fminf(ax, ay);
            k = (k << 1) | ((w2 ^ __float_as_uint(E)) >> 31);
        }
    }
    return (int)(k ^ (1u << (TB - 1)));  // + L/2: angles from -pi
}
template <int TB>
__device__ __forceinline__ int angle_code_t(float x, float y, float hc, float hs) {
    return angle_sector_t<TB>(x * hc - y * hs, x * hs + y * hc);
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

typedef __attribute__((address_space(3))) void lds_void_t;

__host__ __device__ constexpr uint32_t vmcnt_imm(int n) {
    return (uint32_t)(n & 15) | (7u << 4) | (15u << 8) | ((uint32_t)(n >> 4) << 14);
}

// Waits here for the load that produced v.  A value loaded before the cold
// loop and first read inside it would get its wait at that first read, on
// every turn, and the wait would be vmcnt(0): the compiler does not see the
// ring's copies, so it would drain them once per tile.
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
    asm volatile("" ::"v"(v));
}

// Copy BYTES (a multiple of 256) from global memory to this wave's LDS with
// every lane active: 1 KB per dwordx4 instruction, the rest 256 B per dword
// instruction.  The copies are issued from asm: the compiler's own waits for
// LDS DMA lose track of the target stage at a loop header and would drain
// the whole ring (vmcnt(0)) once per ring turn.  Every read of a stage is
// instead ordered by the explicit vmcnt waits of the ring (loads complete in
// order) and by the memory clobber here (no LDS access moves across a copy).
// M0 holds the wave-uniform LDS base; nothing else in these kernels uses M0.
template <int BYTES>
__device__ __forceinline__ void stage_copy(const uint8_t* g, uint8_t* lds, int lane) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)lds;
#pragma unroll
    for (int off = 0; off + 1024 <= BYTES; off += 1024) {
        const uint8_t* ga = g + off + 16 * lane;
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base + off), "v"(ga) : "memory", "m0");
    }
    constexpr int T0 = BYTES / 1024 * 1024;
#pragma unroll
    for (int off = T0; off < BYTES; off += 256) {
        const uint8_t* ga = g + off + 4 * lane;
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(base + off), "v"(ga) : "memory", "m0");
    }
}
template <int BYTES>
constexpr int stage_instrs() {
    return BYTES / 1024 + (BYTES % 1024) / 256;
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// 8 sign bits -> 8 fp16 +-1 through the nibble table
__device__ __forceinline__ half8 signs8(const uint8_t* stab, uint32_t byte) {
    const uint2 lo = *reinterpret_cast<const uint2*>(stab + 8 * (byte & 15u));
    const uint2 hi = *reinterpret_cast<const uint2*>(stab + 8 * ((byte >> 4) & 15u));
    union {
        uint32_t u[4];
        half8 h;
    } r;
    r.u[0] = lo.x, r.u[1] = lo.y, r.u[2] = hi.x, r.u[3] = hi.y;
    return r.h;
}

__device__ __forceinline__ void split_hl(float v, _Float16& hi, _Float16& lo) {
    pin(v);
    hi = (_Float16)v;
    lo = (_Float16)((v - (float)hi) * LO_SCALE);
}

// Bits [bit, bit + n) of a dword array (bit and n compile-time after unrolling).
template <int NW>
__device__ __forceinline__ uint32_t field(const uint32_t (&al)[NW], int bit, int n) {
    uint32_t v = al[bit >> 5] >> (bit & 31);
    if ((bit & 31) + n > 32) v |= al[(bit >> 5) + 1] << (32 - (bit & 31));
    return v & ((1u << n) - 1u);
}

__device__ __forceinline__ float half_at(const uint8_t* p) {
    return (float)(*reinterpret_cast<const _Float16*>(p));
}

}  // namespace tq
