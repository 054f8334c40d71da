// Read-only HBM streaming probe: the bandwidth a kernel that only reads can
// reach on this GPU, printed beside the decode kernel's achieved rate.
//
// Decode over a compressed cache is a scan: the GPU waits on reads of the
// cache ("TurboQuant: kompresja KV-cache w LLM 6 razy", sudonull.com, section
// "KV-cache jako waskie gardlo inferencji").  A copy kernel's rate mixes reads
// with writes; this probe issues only 16-byte loads (every lane of a wave
// reads consecutive 16-byte pieces, 1 KB per wave instruction) and writes one
// word per block, so its bytes are the buffer's.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

constexpr int PROBE_NT = 512;
constexpr int PROBE_UNROLL = 8;  // loads in flight per thread

// Each block reads a contiguous chunk of the buffer in rounds of
// PROBE_NT * PROBE_UNROLL 16-byte pieces; the XOR of everything read is
// stored per block so that no load can be dropped.
__global__ __launch_bounds__(PROBE_NT) void k_probe_read(const uint4* __restrict__ buf, size_t n16, size_t per_block,
                                                         uint32_t* __restrict__ sink) {
    const size_t b0 = (size_t)blockIdx.x * per_block;
    const size_t b1 = b0 + per_block < n16 ? b0 + per_block : n16;
    uint32_t x = 0;
    constexpr size_t ROUND = (size_t)PROBE_NT * PROBE_UNROLL;
    size_t i = b0 + threadIdx.x;
    for (; i + (PROBE_UNROLL - 1) * PROBE_NT < b1; i += ROUND) {
        uint4 v[PROBE_UNROLL];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = buf[i + (size_t)u * PROBE_NT];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < b1; i += PROBE_NT) {
        const uint4 v = buf[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t s[PROBE_NT / 64];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
        for (int w = 0; w < PROBE_NT / 64; ++w) y ^= s[w];
        sink[blockIdx.x] = y;
    }
}

hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t st) {
    const size_t n16 = bytes / 16;
    const size_t per_block = (n16 + blocks - 1) / blocks;
    k_probe_read<<<blocks, PROBE_NT, 0, st>>>(reinterpret_cast<const uint4*>(buf), n16, per_block, sink);
    return hipGetLastError();
}

}  // namespace tq
