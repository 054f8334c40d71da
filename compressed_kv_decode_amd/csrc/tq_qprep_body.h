// Query preparation for decode attention on codes: the body of one block
// (sequence, kv head), shared by k_qprep and by the decode-step kernel that
// runs it beside the step's append.
//
// "TurboQuant: optimizacion de memoria para KV caches en inferencia de LLMs"
// (kerneldigest.dev), seven-step flow, step six: logits come from the
// compressed cache, so the query is taken into the codes' rotated domain
// once per step.  A cold logit in log2 units is R * <u, q'> + rho * <sigma,
// S q'> with q' = Pi q * log2(e) / sqrt(d) and the sketch part also scaled by
// the QJL factor sqrt(pi/2) / m ("TurboQuant: kompresja KV-cache w LLM 6
// razy" (sudonull.com), section "Kompensacja bledow przez QJL").
#pragma once

#include "tq_device.h"

namespace tq {

constexpr int QP_NT = 512;  // k_qprep threads; the work is always cut into this many slices
constexpr float LOG2E = 1.44269504088896340736f;

// fp16 hi part and lo part x 2^12 of entry k, in 16-byte blocks of four
// consecutive entries [hi x4 | lo x4] (one 16-byte load per MFMA operand).
__device__ __forceinline__ void put_hl(uint8_t* blk, int k, float v) {
    pin(v);
    const _Float16 hi = (_Float16)v;
    const _Float16 lo = (_Float16)((v - (float)hi) * LO_SCALE);
    _Float16* h = reinterpret_cast<_Float16*>(blk + 16 * (k >> 2));
    h[k & 3] = hi;
    h[4 + (k & 3)] = lo;
}

// Row of the query / output arrays that holds head c of kv head kvh's group
// for call sequence bi.  In a multi-query pass (mq_n > 0) head c is virtual
// head v = mq_v0 + c, token v / mq_g, head v % mq_g of the group, in arrays
// [n_seq][mq_n][hkv * mq_g][d]; heads past the last virtual one read the
// last one (clamp) or are not written (-1).
__device__ __forceinline__ int64_t head_row(const Dims& dm, int bi, int kvh, int c, bool clamp) {
    if (dm.mq_n == 0) return (int64_t)bi * dm.hq + (int64_t)kvh * dm.g + c;
    const int n_virt = dm.mq_n * dm.mq_g;
    int v = dm.mq_v0 + c;
    if (v >= n_virt) {
        if (!clamp) return -1;
        v = n_virt - 1;
    }
    return (int64_t)bi * n_virt * dm.hkv + (int64_t)(v / dm.mq_g) * dm.hkv * dm.mq_g + (int64_t)kvh * dm.mq_g +
           v % dm.mq_g;
}

// LDS floats of qprep_body<D, G, *>: the queries and q' by component (heads
// padded to whole float4s), then the slice sums of q' and of S q'.
template <int D, int G>
struct QprepGeom {
    static constexpr int PQ = QP_NT / D, JP = D / PQ;      // q' input slices, length
    static constexpr int PS = QP_NT / M_MAX, KS = D / PS;  // S q' slices, length
    static constexpr int GP = (G + 3) / 4 * 4;
    static constexpr int FLOATS = GP * (2 * D + PQ * D + PS * M_MAX);
};

// One block of NT threads (NT divides QP_NT) for (sequence bi, kv head kvh):
// the group's G queries share every matrix read.  Slice (p, k) sums q'_k of
// all G heads over the inputs j in [JP p, JP p + JP) from column k of Pi^T
// (row k of Pi); slice (p, j < M_MAX) sums (S q')_j over a stretch of k from
// column j of S^T.  A thread takes QP_NT / NT slices; each slice is the same
// chain of fmas whatever NT is, and the slices are added in LDS in a fixed
// order, so every block size writes the same bits.  The columns' pieces are
// requested at the start, coalesced across the threads (one row of Pi^T or
// S^T per load), and wait in registers: the block waits for memory once.
// No matrix goes through LDS.
template <int D, int G, int NT>
__device__ __forceinline__ void qprep_body(const Dims& dm, const Ptrs& P, int bi, int kvh,
                                           const _Float16* __restrict__ q, float cm, float* lds) {
    using QG = QprepGeom<D, G>;
    constexpr int PQ = QG::PQ, JP = QG::JP, PS = QG::PS, KS = QG::KS, GP = QG::GP;
    constexpr int R = QP_NT / NT;
    static_assert(QP_NT % NT == 0, "whole slices per thread");
    float(*s_q)[GP] = reinterpret_cast<float(*)[GP]>(lds);
    float(*s_r)[GP] = reinterpret_cast<float(*)[GP]>(lds + D * GP);
    float(*s_pq)[D][GP] = reinterpret_cast<float(*)[D][GP]>(lds + 2 * D * GP);
    float(*s_ps)[M_MAX][GP] = reinterpret_cast<float(*)[M_MAX][GP]>(lds + (2 + PQ) * D * GP);
    const int tid = threadIdx.x;
    // slice numbers turned by the block's position, so that blocks running
    // at the same time start on different rows of the shared matrices
    const int turn = bi + kvh;
    const size_t qh0 = (size_t)bi * dm.hq + (size_t)kvh * G;  // first prepared row of the group
    float pcol[R][JP], scol[R][KS];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int vt = tid + r * NT;
        const int k = vt % D, p = (vt / D + turn) % PQ;
        const int js = vt % M_MAX, ps = (vt / M_MAX + turn) % PS;
#pragma unroll
        for (int j = 0; j < JP; ++j) pcol[r][j] = P.pit32[(size_t)(JP * p + j) * D + k];
#pragma unroll
        for (int j = 0; j < KS; ++j) scol[r][j] = P.st32[(size_t)(KS * ps + j) * M_MAX + js];
    }
    for (int e = tid; e < G * D; e += NT) {
        const _Float16 x = q[head_row(dm, bi, kvh, e / D, true) * D + e % D];
        s_q[e % D][e / D] = (float)x;
        if (dm.mq_n > 0) P.qgather[qh0 * D + e] = x;  // the pass's queries, for k_decode's hot phase
    }
    if constexpr (GP > G)
        for (int e = tid; e < (GP - G) * D; e += NT) s_q[e % D][G + e / D] = 0.0f;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int vt = tid + r * NT;
        const int k = vt % D, p = (vt / D + turn) % PQ;
        float acc[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) acc[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < JP; ++j) {
#pragma unroll
            for (int h4 = 0; h4 < GP; h4 += 4) {
                const float4 qv = *reinterpret_cast<const float4*>(&s_q[JP * p + j][h4]);
                acc[h4] = fmaf(pcol[r][j], qv.x, acc[h4]);
                acc[h4 + 1] = fmaf(pcol[r][j], qv.y, acc[h4 + 1]);
                acc[h4 + 2] = fmaf(pcol[r][j], qv.z, acc[h4 + 2]);
                acc[h4 + 3] = fmaf(pcol[r][j], qv.w, acc[h4 + 3]);
            }
        }
#pragma unroll
        for (int h = 0; h < GP; ++h) s_pq[p][k][h] = acc[h];
    }
    __syncthreads();
    const float sc = LOG2E / sqrtf((float)D);
    for (int e = tid; e < D * GP; e += NT) {
        const int kk = e % D, h = e / D;
        float v = s_pq[0][kk][h];
#pragma unroll
        for (int i = 1; i < PQ; ++i) v += s_pq[i][kk][h];
        s_r[kk][h] = v;
        if (h < G) put_hl(reinterpret_cast<uint8_t*>(P.qprep + (qh0 + h) * (D + M_MAX)), kk, v * sc);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int vt = tid + r * NT;
        const int js = vt % M_MAX, ps = (vt / M_MAX + turn) % PS;
        float acc[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) acc[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
#pragma unroll
            for (int h4 = 0; h4 < GP; h4 += 4) {
                const float4 rv = *reinterpret_cast<const float4*>(&s_r[KS * ps + j][h4]);
                acc[h4] = fmaf(scol[r][j], rv.x, acc[h4]);
                acc[h4 + 1] = fmaf(scol[r][j], rv.y, acc[h4 + 1]);
                acc[h4 + 2] = fmaf(scol[r][j], rv.z, acc[h4 + 2]);
                acc[h4 + 3] = fmaf(scol[r][j], rv.w, acc[h4 + 3]);
            }
        }
#pragma unroll
        for (int h = 0; h < GP; ++h) s_ps[ps][js][h] = acc[h];
    }
    __syncthreads();
    for (int e = tid; e < M_MAX * G; e += NT) {
        const int j = e % M_MAX, h = e / M_MAX;
        float v = s_ps[0][j][h];
#pragma unroll
        for (int i = 1; i < PS; ++i) v += s_ps[i][j][h];
        put_hl(reinterpret_cast<uint8_t*>(P.qprep + (qh0 + h) * (D + M_MAX)) + 4 * D, j, v * sc * cm);
    }
}

}  // namespace tq
