// Maximum inner-product search over the compressed vectors of one cache
// stream.
//
// "Compresion del cache KV de los LLM a 3 bits: TurboQuant" (sudonull.com),
// section "Aplicaciones mas alla de los LLMs": the codec serves vector search
// -- vectors are stored as codes and inner products are estimated from them.
// The score of stored vector j for query q is the estimate the decode path
// uses for a cold key, <q', y_hat_j> + sqrt(pi/2)/m rho_j <S_m q', sigma_j>
// with q' = Pi q; the result is the k best per query (score descending, the
// lower slot first on ties).
//
// Kernels of one search (queries in groups of 8):
//   k_mips_pad   copies the queries into a zero-padded [groups * 8][d] array.
//   k_qprep      (the decode kernel's query prep, 8 queries per block) writes
//                q' and S q' as fp16 hi/lo MFMA operands, in log2 units.
//   k_mips_scan  (next to the decode kernel, whose packed key MFMAs it
//                uses) one wave per (part of the stream's cold tiles, group
//                of 8 queries): the scores of every vector against the 8
//                queries, to 2^-22 (q' split hi / lo), and the part's best k
//                per query.
//   k_mips_merge one block per query: the best k over all parts.
#include "tq_device.h"

namespace tq {

constexpr int MQ = 8;          // queries per group (B columns 0..7; 8..15 repeat them)
constexpr float LN2F = 0.69314718055994530942f;
constexpr float SQRT_HALF_PI_F = 1.25331413731550025121f;

__global__ void k_mips_pad(const _Float16* __restrict__ q, int n_q, int n_qp, int d, _Float16* __restrict__ qp) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_qp * d; i += gridDim.x * blockDim.x)
        qp[i] = i < n_q * d ? q[i] : (_Float16)0.0f;
}

// One block per query: the best k of its group's n_parts sorted lists, by
// repeated block-wide selection (each round takes the best head among the
// lists; score descending, then the lower slot).  Scores leave in natural
// units: <q, x_hat> = log2-unit score * ln 2 * sqrt(d).
__global__ __launch_bounds__(256) void k_mips_merge(const Cand* __restrict__ partial, int n_q, int n_parts, int k,
                                                    float to_natural, int32_t* __restrict__ idx,
                                                    float* __restrict__ score) {
    __shared__ int s_head[1024];  // next entry of each list
    __shared__ float s_bv[256 / 64];
    __shared__ int s_bs[256 / 64], s_bl[256 / 64];
    const int qi = blockIdx.x, grp = qi / MQ, qc = qi % MQ, tid = threadIdx.x;
    for (int p = tid; p < n_parts; p += 256) s_head[p] = 0;
    __syncthreads();
    auto at = [&](int p, int i) { return partial[(((size_t)grp * n_parts + p) * MQ + qc) * k + i]; };
    for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int bs = 0x7fffffff, bl = -1;
        for (int p = tid; p < n_parts; p += 256) {
            const int h = s_head[p];
            if (h >= k) continue;
            const Cand c = at(p, h);
            if (c.slot < 0) continue;
            if (c.v > bv || (c.v == bv && c.slot < bs)) bv = c.v, bs = c.slot, bl = p;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float v2 = __shfl_xor(bv, o, 64);
            const int s2 = __shfl_xor(bs, o, 64), l2 = __shfl_xor(bl, o, 64);
            if (v2 > bv || (v2 == bv && s2 < bs)) bv = v2, bs = s2, bl = l2;
        }
        if ((tid & 63) == 0) s_bv[tid >> 6] = bv, s_bs[tid >> 6] = bs, s_bl[tid >> 6] = bl;
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < 256 / 64; ++w)
                if (s_bv[w] > s_bv[0] || (s_bv[w] == s_bv[0] && s_bs[w] < s_bs[0]))
                    s_bv[0] = s_bv[w], s_bs[0] = s_bs[w], s_bl[0] = s_bl[w];
            const bool ok = s_bl[0] >= 0;
            idx[(size_t)qi * k + r] = ok ? s_bs[0] : -1;
            score[(size_t)qi * k + r] = ok ? s_bv[0] * to_natural : -INFINITY;
            if (ok) s_head[s_bl[0]] += 1;
        }
        __syncthreads();
    }
}

// Workspace layout of a search: padded queries, prepared queries, partials.
struct MipsLayout {
    int n_qp, n_groups, n_parts;
    size_t o_qpad, o_qprep, o_part, total;
};

static MipsLayout mips_layout(const Dims& dm, int n_q, int k, int64_t appended) {
    MipsLayout L{};
    L.n_qp = (n_q + MQ - 1) / MQ * MQ;
    L.n_groups = L.n_qp / MQ;
    // about 3 waves per SIMD over all groups, at least 4 tiles per part, at
    // most 1024 parts
    const int64_t tiles = std::max<int64_t>(1, (appended + TILE - 1) / TILE);
    int64_t parts = std::max<int64_t>(1, 3072 / L.n_groups);
    parts = std::min<int64_t>(parts, std::max<int64_t>(1, tiles / 4));
    L.n_parts = (int)std::min<int64_t>(parts, 1024);
    auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.o_qpad = 0;
    L.o_qprep = a256((size_t)L.n_qp * dm.d * 2);
    L.o_part = L.o_qprep + a256((size_t)L.n_qp * (dm.d + M_MAX) * 4);
    L.total = L.o_part + (size_t)L.n_groups * L.n_parts * MQ * k * sizeof(Cand);
    return L;
}

size_t mips_workspace_bytes(const Dims& dm, int n_q, int k, int64_t appended) {
    return mips_layout(dm, n_q, k, appended).total;
}

hipError_t launch_mips(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, int seq, int kvh, int n_q,
                       const _Float16* q, int k, int32_t* idx, float* score, uint8_t* ws, int64_t appended,
                       hipStream_t st) {
    const MipsLayout L = mips_layout(dm, n_q, k, appended);
    _Float16* qpad = reinterpret_cast<_Float16*>(ws + L.o_qpad);
    Ptrs Pm = P;
    Pm.qprep = reinterpret_cast<float*>(ws + L.o_qprep);
    Cand* part = reinterpret_cast<Cand*>(ws + L.o_part);
    k_mips_pad<<<std::max(1, std::min(1024, (L.n_qp * dm.d + 255) / 256)), 256, 0, st>>>(q, n_q, L.n_qp, dm.d, qpad);
    hipError_t e = launch_qprep8(dm, Pm, qpad, L.n_groups, SQRT_HALF_PI_F / (float)F.m, st);
    if (e != hipSuccess) return e;
    e = launch_mips_scan(dm, Pm, F, layer, seq, kvh, L.n_groups, L.n_parts, k, part, st);
    if (e != hipSuccess) return e;
    const float to_natural = LN2F * sqrtf((float)dm.d);
    k_mips_merge<<<n_q, 256, 0, st>>>(part, n_q, L.n_parts, k, to_natural, idx, score);
    return hipGetLastError();
}

}  // namespace tq
