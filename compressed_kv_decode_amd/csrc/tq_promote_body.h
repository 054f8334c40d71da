// Attention-weighted promotion with a sticky counter: the body of one block
// (sequence, kv head) of the batch, shared by k_promote and by the kernel that
// runs a deferred promotion of one layer beside a small append of another.
//
// "Monarch v3: Paginacion KV Inspirada en NES" (openclawradar.com), section
// "Como funciona": cold tokens that draw high attention return to the hot
// region, with a persistence mechanism against thrashing; section "Bucle de
// Decodificacion Simplificado": decompressed cold pages move to hot for the
// next step; section "Como probarlo": promotion threshold and sticky
// threshold flags.
//
// One block per (sequence, kv head) of the batch:
//   1. gather the per-query-head candidate lists written by the last
//      attention step (probabilities >= tau) and merge them per slot into
//      P_c = max over heads;
//   2. read each candidate's sticky word (last qualifying step, count): the
//      count continues if the slot also qualified at the previous step, else
//      restarts at 1 (slots that did not qualify keep a stale step and so
//      read as 0);
//   3. slots whose count reaches `sticky` enter the hot ring as the newest
//      entries, P_c descending (ties to the lower slot);
//   4. dequantise each promoted token's K and V codes of the block's kv head,
//      x_hat = Pi^T (y_hat + sqrt(pi/2)/m * rho * S_m^T sigma) (values without
//      the QJL term when it is off), rounded to fp16 into the ring;
//   5. the last block of the sequence to finish writes the bookkeeping:
//      sticky words, tombstones (the promoted cold slots), ring tags, counts.
// Steps 1 - 3 only read state, so every block of a sequence derives the same
// promotion list; the writes of step 5 wait until all of them have read it.
#pragma once

#include "tq_device.h"

namespace tq {

constexpr float SQRT_HALF_PI_P = 1.25331413731550025121f;
constexpr int MAXP = 2048;  // candidate entries per sequence (n_q_heads * floor(1 / tau), checked at creation)
constexpr int PNT = 256;    // threads per block

template <int D, int CB>
__device__ __forceinline__ void promote_body(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                                             const CallSeqs& cs) {
    const int bi = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
    const int seq = cs.ids[bi];
    const size_t sl = sl_index(dm, seq, layer);
    __shared__ int s_slot[MAXP];
    __shared__ float s_p[MAXP];
    __shared__ float s_pc[MAXP];   // merged P_c of a slot's first entry, -1 for the other entries
    __shared__ int s_cnt[MAXP];    // sticky count of a slot's first entry after this step
    __shared__ int s_order[MAXP];  // promoted entries by rank
    __shared__ float s_y[PNT];
    __shared__ int s_n, s_np, s_S, s_head, s_count, s_last;
    SeqLayerMeta* mt = P.meta + sl;
    int* tags = P.tags + sl * dm.cap;
    uint32_t* tomb = P.tomb + sl * (dm.cold_cap / 32);
    uint32_t* stk = P.sticky + sl * dm.cold_cap;
    if (tid == 0) {
        s_n = 0;
        s_np = 0;
    }
    __syncthreads();
    // the metadata is read together with the candidate lists
    int m_S = 0, m_head = 0, m_count = 0;
    if (tid == 0) m_S = mt->attn_step, m_head = mt->head, m_count = mt->count;
    // 1. the valid entries (i < cand_n of the head), in any order
    const int nent = dm.hq * dm.ktop;
    for (int e = tid; e < nent; e += PNT) {
        const int h = e / dm.ktop, i = e - h * dm.ktop;
        const int cnt = P.cand_n[sl * dm.hq + h];
        const Cand c = P.cand[sl * dm.hq * dm.ktop + e];
        if (i < cnt) {
            const int at = atomicAdd(&s_n, 1);
            s_slot[at] = c.slot;
            s_p[at] = c.v;
        }
    }
    if (tid == 0) s_S = m_S, s_head = m_head, s_count = m_count;
    __syncthreads();
    const int n = s_n, S = s_S;
    // No candidate in any head: nothing changes (sticky words of slots that
    // did not qualify go stale by themselves).  Every block of the sequence
    // reads the same lists, so all of them leave here and none counts in.
    if (n == 0) return;
    // 1-2. the first entry of each slot merges its copies and reads the sticky word
    for (int k = tid; k < n; k += PNT) {
        const int c = s_slot[k];
        float pc = s_p[k];
        bool first = true;
        for (int j = 0; j < n; ++j) {
            if (s_slot[j] == c) {
                first = first && j >= k;
                pc = fmaxf(pc, s_p[j]);
            }
        }
        int cnt = 0;
        if (first) {
            const uint32_t w = stk[c];
            const int last = (int)(w >> 8);
            cnt = (last == S - 1) ? min((int)(w & 255u) + 1, 255) : 1;
            if (cnt >= dm.sticky) atomicAdd(&s_np, 1);
        }
        s_pc[k] = first ? pc : -1.0f;
        s_cnt[k] = cnt;
    }
    __syncthreads();
    // 3. rank of each promoted entry: P_c descending, ties to the lower slot
    for (int k = tid; k < n; k += PNT) {
        if (s_pc[k] < 0.0f || s_cnt[k] < dm.sticky) continue;
        const float pk = s_pc[k];
        const int ck = s_slot[k];
        int r = 0;
        for (int j = 0; j < n; ++j) {
            if (s_pc[j] < 0.0f || s_cnt[j] < dm.sticky) continue;
            r += (s_pc[j] > pk || (s_pc[j] == pk && s_slot[j] < ck)) ? 1 : 0;
        }
        s_order[r] = k;
    }
    __syncthreads();
    // This block's reads of the shared state are done (their values are in
    // LDS): count it in now, so that the atomic's round trip overlaps the
    // dequantisation; the last block of the sequence writes the bookkeeping
    // at its end.  No fence: nothing this block wrote is read by the others.
    int prior = 0;
    if (tid == 0) prior = atomicAdd(&mt->done, 1);
    const int count = s_count, head = s_head;
    const int np_all = s_np;
    const int np = min(np_all, dm.cap - count);  // the ring's capacity bounds the promotions
    // 4. dequantisation of this kv head's promoted K and V vectors, PNT / D at a time
    if (np > 0) {
        constexpr int VPB = PNT / D;
        const int k = tid % D, sub = tid / D;
        const int LR = 1 << F.rb;
        const float cm = SQRT_HALF_PI_P / (float)F.m;
        // column k of Pi and of S (rows k of Pi^T and S^T): the same for every vector
        float4 pcol4[D / 4], scol4[M_MAX / 4];
        const float4* pt = reinterpret_cast<const float4*>(P.pit32 + (size_t)k * D);
        const float4* st = reinterpret_cast<const float4*>(P.st32 + (size_t)k * M_MAX);
#pragma unroll
        for (int j = 0; j < D / 4; ++j) pcol4[j] = pt[j];
#pragma unroll
        for (int j = 0; j < M_MAX / 4; ++j) scol4[j] = st[j];
        const float* pcol = reinterpret_cast<const float*>(pcol4);
        const float* scol = reinterpret_cast<const float*>(scol4);
        const size_t rb = ring_base(dm, seq, layer, kvh);
        for (int u0 = 0; u0 < 2 * np; u0 += VPB) {
            const int u = u0 + sub;  // vector u: token rank u / 2, K (even) or V (odd)
            const bool act = u < 2 * np;
            const int r = act ? u >> 1 : 0, kv = u & 1;
            const int c = s_slot[s_order[r]];
            const int tl = c / TILE, ts = c % TILE;
            if (act) {
                const uint8_t* tile = P.cold + cold_tile_offset(dm, F, seq, kvh, kv, tl);
                const uint8_t* meta = tile + TILE * (F.pb + F.sb);
                const float R = half_at(meta + 2 * ts);
                const float rho = half_at(meta + 2 * TILE + 2 * (kv == 0 ? ts : vpos(ts)));
                const int pair = k >> 1;
                uint32_t code;
                if (kv == 0) {
                    // position of the pair inside the K record
                    const int qq = (pair % 16) / 4, b = pair / 16, jj = pair % 4;
                    const int pos_in = qq * (D / 8) + b * 4 + jj;
                    code = bits_at(reinterpret_cast<const uint32_t*>(tile + ts * F.pb), pos_in * CB, CB);
                } else {
                    code = bits_at(reinterpret_cast<const uint32_t*>(tile + (size_t)pair * 4 * CB), vpos(ts) * CB, CB);
                }
                const int a = code & (LR - 1), bb = code >> F.rb;
                const float rh = (float)a * (R / (float)(LR - 1));
                float y = rh * ((k & 1) ? F.sin_t[bb] : F.cos_t[bb]);
                if (kv == 0 || dm.v_qjl) {
                    uint64_t sg;  // sign bit j of the token
                    if (kv == 0) {
                        const uint8_t* sb = tile + TILE * F.pb + ts * F.sb;
                        sg = 0;
                        for (int i = 0; i < F.sb; ++i) sg |= (uint64_t)sb[i] << (8 * i);
                    } else {
                        const uint32_t* planes = reinterpret_cast<const uint32_t*>(tile + TILE * F.pb);
                        sg = 0;
                        for (int j = 0; j < F.m; ++j) sg |= (uint64_t)((planes[j] >> vpos(ts)) & 1u) << j;
                    }
                    float t = 0.0f;
#pragma unroll
                    for (int j = 0; j < M_MAX; ++j)
                        if (j < F.m) t = fmaf(((sg >> j) & 1u) ? 1.0f : -1.0f, scol[j], t);
                    y = fmaf(cm * rho, t, y);
                }
                s_y[tid] = y;
            }
            __syncthreads();
            if (act) {
                float x = 0.0f;
#pragma unroll
                for (int j = 0; j < D; ++j) x = fmaf(pcol[j], s_y[sub * D + j], x);
                const int pos = (head + count + r) % dm.cap;
                if (kv == 0)
                    P.ring_k[rb + (size_t)pos * D + k] = (_Float16)x;
                else
                    P.ring_v[rb + (size_t)(pos / 32) * D * 32 + (size_t)k * 32 + vpos(pos % 32)] = (_Float16)x;
            }
            __syncthreads();
        }
    }
    // 5. the last block of the sequence writes the bookkeeping (every block
    // had read it before counting itself in)
    if (tid == 0) s_last = prior == (int)gridDim.y - 1;
    __syncthreads();
    if (!s_last) return;
    for (int k = tid; k < n; k += PNT) {
        if (s_pc[k] >= 0.0f && s_cnt[k] < dm.sticky) stk[s_slot[k]] = ((uint32_t)S << 8) | (uint32_t)s_cnt[k];
    }
    for (int r = tid; r < np; r += PNT) {
        const int c = s_slot[s_order[r]];
        tags[(head + count + r) % dm.cap] = c;
        atomicOr(tomb + (c >> 5), 1u << (c & 31));
        stk[c] = 0u;
    }
    if (tid == 0) {
        if (np < np_all) atomicOr(P.err, DEVERR_RING_OVERFLOW);
        mt->count = count + np;
        mt->n_promoted += np;
        mt->promoted_step = S;
        mt->done = 0;
    }
}

}  // namespace tq
