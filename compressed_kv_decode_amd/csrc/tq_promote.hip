// Attention-weighted promotion with a sticky counter.
//
// "Monarch v3: Paginacion KV Inspirada en NES" (openclawradar.com), section
// "Como funciona": cold tokens that draw high attention return to the hot
// region, with a persistence mechanism against thrashing; section "Bucle de
// Decodificacion Simplificado": decompressed cold pages move to hot for the
// next step; section "Como probarlo": promotion threshold and sticky
// threshold flags.
//
// k_promote, one block per sequence of the batch:
//   1. thread 0 merges the per-query-head candidate lists written by the
//      last attention step (probabilities >= tau) into P_c = max over heads;
//   2. updates each candidate's sticky word (last qualifying step, count):
//      the count continues if the slot also qualified at the previous step,
//      else restarts at 1; slots that did not qualify keep a stale step and
//      so read as 0;
//   3. slots whose count reaches `sticky` enter the hot ring as the newest
//      entries, P_c descending (ties to the lower slot); their cold slot is
//      tombstoned and the counter cleared;
//   4. all threads dequantise each promoted token's K and V codes of every kv
//      head, x_hat = Pi^T (y_hat + sqrt(pi/2)/m * rho * S_m^T sigma) (values
//      without the QJL term when it is off), round to fp16 into the ring.
#include "tq_device.h"

namespace tq {

constexpr float SQRT_HALF_PI_P = 1.25331413731550025121f;
constexpr int MAXP = 2048;

template <int D, int CB>
__global__ __launch_bounds__(256) void k_promote(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs) {
    constexpr int PAIRS = D / 2;
    const int bi = blockIdx.x, tid = threadIdx.x;
    const int seq = cs.ids[bi];
    const size_t sl = sl_index(dm, seq, layer);
    __shared__ int s_slot[MAXP];
    __shared__ float s_p[MAXP];
    __shared__ int s_pos[MAXP];
    __shared__ int s_np;
    __shared__ float s_y[D];
    SeqLayerMeta* mt = P.meta + sl;
    int* tags = P.tags + sl * dm.cap;
    uint32_t* tomb = P.tomb + sl * (dm.cold_cap / 32);
    uint32_t* stk = P.sticky + sl * dm.cold_cap;
    if (tid == 0) {
        const int S = mt->attn_step;
        int n = 0;
        for (int h = 0; h < dm.hq; ++h) {
            const int cnt = P.cand_n[sl * dm.hq + h];
            const Cand* cc = P.cand + (sl * dm.hq + h) * dm.ktop;
            for (int i = 0; i < cnt; ++i) {
                int f = -1;
                for (int k = 0; k < n; ++k)
                    if (s_slot[k] == cc[i].slot) f = k;
                if (f >= 0) {
                    s_p[f] = fmaxf(s_p[f], cc[i].v);
                } else if (n < MAXP) {
                    s_slot[n] = cc[i].slot;
                    s_p[n] = cc[i].v;
                    ++n;
                }
            }
        }
        // sticky counters; compact the promoted ones to the front
        int np = 0;
        for (int k = 0; k < n; ++k) {
            const int c = s_slot[k];
            const uint32_t w = stk[c];
            const int last = (int)(w >> 8);
            int cnt = (int)(w & 255u);
            cnt = (last == S - 1) ? min(cnt + 1, 255) : 1;
            if (cnt >= dm.sticky) {
                const int ts = s_slot[np];
                const float tp = s_p[np];
                s_slot[np] = c;
                s_p[np] = s_p[k];
                s_slot[k] = ts;
                s_p[k] = tp;
                ++np;
            } else {
                stk[c] = ((uint32_t)S << 8) | (uint32_t)cnt;
            }
        }
        // order: P descending, ties to the lower slot
        for (int a = 1; a < np; ++a) {
            const int cs_ = s_slot[a];
            const float cp = s_p[a];
            int b = a - 1;
            while (b >= 0 && (s_p[b] < cp || (s_p[b] == cp && s_slot[b] > cs_))) {
                s_slot[b + 1] = s_slot[b];
                s_p[b + 1] = s_p[b];
                --b;
            }
            s_slot[b + 1] = cs_;
            s_p[b + 1] = cp;
        }
        const int count = mt->count;
        if (count + np > dm.cap) {
            atomicOr(P.err, DEVERR_RING_OVERFLOW);
            np = dm.cap - count;
        }
        for (int i = 0; i < np; ++i) {
            const int c = s_slot[i];
            const int pos = (mt->head + count + i) % dm.cap;
            s_pos[i] = pos;
            tags[pos] = c;
            tomb[c >> 5] |= 1u << (c & 31);
            stk[c] = 0u;
        }
        mt->count = count + np;
        mt->n_promoted += np;
        mt->promoted_step = S;
        s_np = np;
    }
    __syncthreads();
    const int np = s_np;
    const int LR = 1 << F.rb;
    const float cm = SQRT_HALF_PI_P / (float)F.m;
    for (int i = 0; i < np; ++i) {
        const int c = s_slot[i];
        const int pos = s_pos[i];
        const int tl = c / TILE, ts = c % TILE;
        for (int kvh = 0; kvh < dm.hkv; ++kvh) {
            for (int kv = 0; kv < 2; ++kv) {
                const uint8_t* tile = P.cold + cold_tile_offset(dm, F, seq, kvh, kv, tl);
                const uint8_t* meta = tile + TILE * (F.pb + F.sb);
                const float R = half_at(meta + 2 * ts);
                const float rho = half_at(meta + 2 * TILE + 2 * (kv == 0 ? ts : vpos(ts)));
                if (tid < D) {
                    const int k = tid, pair = k >> 1;
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
                        float t = 0.0f;
                        for (int j = 0; j < F.m; ++j) {
                            const uint32_t bit = kv == 0 ? (tile[TILE * F.pb + ts * F.sb + (j >> 3)] >> (j & 7)) & 1u
                                                         : (reinterpret_cast<const uint32_t*>(tile + TILE * F.pb)[j] >> vpos(ts)) & 1u;
                            t = fmaf(bit ? 1.0f : -1.0f, P.s32[(size_t)j * D + k], t);
                        }
                        y = fmaf(cm * rho, t, y);
                    }
                    s_y[k] = y;
                }
                __syncthreads();
                if (tid < D) {
                    float x = 0.0f;
                    for (int k = 0; k < D; ++k) x = fmaf(P.pi32[(size_t)k * D + tid], s_y[k], x);
                    const size_t rb = ring_base(dm, seq, layer, kvh);
                    if (kv == 0)
                        P.ring_k[rb + (size_t)pos * D + tid] = (_Float16)x;
                    else
                        P.ring_v[rb + (size_t)(pos / 32) * D * 32 + (size_t)tid * 32 + vpos(pos % 32)] = (_Float16)x;
                }
                __syncthreads();
            }
        }
    }
}

hipError_t launch_promote(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                          hipStream_t st) {
    if (cs.n == 0 || dm.ktop == 0) return hipSuccess;
    const int key = dm.d * 10 + F.cb;
    switch (key) {
        case 645: k_promote<64, 5><<<cs.n, 256, 0, st>>>(dm, P, F, layer, cs); break;
        case 647: k_promote<64, 7><<<cs.n, 256, 0, st>>>(dm, P, F, layer, cs); break;
        case 644: k_promote<64, 4><<<cs.n, 256, 0, st>>>(dm, P, F, layer, cs); break;
        case 1285: k_promote<128, 5><<<cs.n, 256, 0, st>>>(dm, P, F, layer, cs); break;
        case 1287: k_promote<128, 7><<<cs.n, 256, 0, st>>>(dm, P, F, layer, cs); break;
        case 1284: k_promote<128, 4><<<cs.n, 256, 0, st>>>(dm, P, F, layer, cs); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
