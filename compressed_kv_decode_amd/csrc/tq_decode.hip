// Decode attention read straight from the compressed cache.
//
// "TurboQuant: optimizacion de memoria para KV caches en inferencia de LLMs"
// (kerneldigest.dev): step six of the quantisation flow computes attention
// logits from the compressed cache; section "Arquitectura del Sistema": the
// QJL correction keeps attention scores accurate.  Cold logit of slot j for
// query q (q' = Pi q):
//   [ R_j/(L_r-1) * sum_i a_ij (q'_2i cos phi_bij + q'_2i+1 sin phi_bij)
//     + sqrt(pi/2)/m * rho_j * <S_m q', sigma_j> ] / sqrt(d)
// "Monarch v3" (openclawradar.com), section "Bucle de Decodificacion
// Simplificado": the hot window is scored at full precision alongside.
//
// Kernels of one tq_decode_attention launch batch:
//   k_qprep   q' = Pi q and S q' per (sequence, query head), fp32.
//   k_decode  split-context attention: one block per (chunk, sequence, kv
//             head).  A hot chunk covers up to 256 ring entries; a cold
//             chunk covers tiles of 256 slots.  Per tile: logits (one token
//             per thread, all query heads of the group), online softmax
//             (wave shuffles, then LDS across waves), value accumulation
//             (cold values in the rotated domain: pair codes times p * R,
//             plus sign sums of p * rho for the QJL term).  Writes per-head
//             partial (max, sum, accumulator) and promotion candidates.
//   k_combine merges the partials of each (sequence, query head), adds the
//             QJL back-projection S_m^T, rotates back with Pi^T, normalises,
//             and turns candidate logits into exact probabilities.
#include <math.h>

#include "tq_device.h"

namespace tq {

constexpr float SQRT_HALF_PI = 1.25331413731550025121f;

__global__ void k_fill(float* p, size_t n, float v) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

template <int D>
__global__ __launch_bounds__(128) void k_qprep(Dims dm, Ptrs P, const _Float16* __restrict__ q) {
    const int bi = blockIdx.x, h = blockIdx.y, k = threadIdx.x;
    __shared__ float s_q[D], s_r[D];
    if (k < D) s_q[k] = (float)q[((size_t)bi * dm.hq + h) * D + k];
    __syncthreads();
    float* out = P.qprep + ((size_t)bi * dm.hq + h) * (D + M_MAX);
    if (k < D) {
        float acc = 0.0f;
        const float* row = P.pi32 + (size_t)k * D;
        for (int j = 0; j < D; ++j) acc = fmaf(row[j], s_q[j], acc);
        s_r[k] = acc;
        out[k] = acc;
    }
    __syncthreads();
    if (k < M_MAX) {
        float acc = 0.0f;
        const float* row = P.s32 + (size_t)k * D;
        for (int j = 0; j < D; ++j) acc = fmaf(row[j], s_r[j], acc);
        out[D + k] = acc;
    }
}

// Block-wide max and sum of G per-thread values (256 threads, 4 waves).
template <int G>
__device__ __forceinline__ void block_max(float (&v)[G], float (*s_red)[4]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float w = wave_max(v[h]);
        if (lane == 0) s_red[h][wave] = w;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) v[h] = fmaxf(fmaxf(s_red[h][0], s_red[h][1]), fmaxf(s_red[h][2], s_red[h][3]));
    __syncthreads();
}

template <int G>
__device__ __forceinline__ void block_sum(float (&v)[G], float (*s_red)[4]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float w = wave_sum(v[h]);
        if (lane == 0) s_red[h][wave] = w;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) v[h] = (s_red[h][0] + s_red[h][1]) + (s_red[h][2] + s_red[h][3]);
    __syncthreads();
}

template <int D, int CB, int G>
__global__ __launch_bounds__(256) void k_decode(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs,
                                                const _Float16* __restrict__ qin, int n_hot_chunks, int chunk_tiles,
                                                float* logits, int lstride) {
    constexpr int PAIRS = D / 2;
    constexpr int PBW = PAIRS * CB / 32;  // dwords per K record
    const int bi = blockIdx.y, kvh = blockIdx.z, c = blockIdx.x;
    const int seq = cs.ids[bi];
    const size_t sl = sl_index(dm, seq, layer);
    const SeqLayerMeta mt = P.meta[sl];
    const int tid = threadIdx.x;
    const bool hot = c < n_hot_chunks;
    const int m = F.m;
    int first, last;
    if (hot) {
        first = c * DTILE;
        last = min(first + DTILE, mt.count);
    } else {
        first = (c - n_hot_chunks) * chunk_tiles * DTILE;
        last = min(first + chunk_tiles * DTILE, mt.cold_len);
    }
    const int stride = part_stride(D);
    const int ktop = dm.ktop;

    __shared__ float s_q[G][D];
    __shared__ float s_sq[G][M_MAX];
    __shared__ float2 s_lut[256];
    __shared__ float s_pw[G][DTILE];
    __shared__ float s_pr[G][DTILE];
    __shared__ float s_red[G][4];
    __shared__ float s_acc[4][G][D];   // value partials per token group (reduced at the end)
    __shared__ Cand s_cand[G][128];
    __shared__ int s_ncand[G];

    // query: original (hot) or rotated + sketched (cold)
    for (int i = tid; i < G * D; i += 256) {
        const int h = i / D, k = i % D;
        const int qh = kvh * G + h;
        s_q[h][k] = hot ? (float)qin[((size_t)bi * dm.hq + qh) * D + k]
                        : P.qprep[((size_t)bi * dm.hq + qh) * (D + M_MAX) + k];
    }
    for (int i = tid; i < G * M_MAX; i += 256) {
        const int h = i / M_MAX, j = i % M_MAX;
        s_sq[h][j] = hot ? 0.0f : P.qprep[((size_t)bi * dm.hq + kvh * G + h) * (D + M_MAX) + D + j];
    }
    {
        const int LR = 1 << F.rb;
        for (int code = tid; code < (1 << CB); code += 256) {
            const int a = code & (LR - 1), b = code >> F.rb;
            const float s = (float)a / (float)(LR - 1);
            s_lut[code] = make_float2(s * F.cos_t[b], s * F.sin_t[b]);
        }
    }
    if (tid < G) s_ncand[tid] = 0;

    float m_run[G], l_run[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.0f;
    }
    // value accumulators: cold -> (pair i, token group), hot -> (component k, token group)
    constexpr int NTG = DTILE / PAIRS;  // token groups over pairs (cold)
    constexpr int NTH = DTILE / D;      // token groups over components (hot)
    float acc[G][2];
    float acc_s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        acc[h][0] = acc[h][1] = 0.0f;
        acc_s[h] = 0.0f;
    }
    const float isd = 1.0f / sqrtf((float)D);
    const float cm = SQRT_HALF_PI / (float)m;
    const size_t rb = ring_base(dm, seq, layer, kvh);
    const uint32_t* tomb = P.tomb + sl * (dm.cold_cap / 32);
    __syncthreads();

    const int ntile = last > first ? (last - first + DTILE - 1) / DTILE : 0;
    for (int tt = 0; tt < ntile; ++tt) {
        const int t0 = first + tt * DTILE;
        const int j = t0 + tid;
        float lg[G];
        float vR = 0.0f, vrho = 0.0f;
        bool live = j < last;
        if (hot) {
            if (live) {
                const int phys = (mt.head + j) % dm.cap;
                const _Float16* kr = P.ring_k + rb + (size_t)phys * D;
                float a[G];
#pragma unroll
                for (int h = 0; h < G; ++h) a[h] = 0.0f;
                for (int k0 = 0; k0 < D; k0 += 8) {
                    const half8 kk = *reinterpret_cast<const half8*>(kr + k0);
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const float kv = (float)kk[r];
#pragma unroll
                        for (int h = 0; h < G; ++h) a[h] = fmaf(s_q[h][k0 + r], kv, a[h]);
                    }
                }
#pragma unroll
                for (int h = 0; h < G; ++h) lg[h] = a[h] * isd;
            } else {
#pragma unroll
                for (int h = 0; h < G; ++h) lg[h] = -INFINITY;
            }
        } else {
            if (live) live = !((tomb[j >> 5] >> (j & 31)) & 1u);
            if (live) {
                const int tl = j / TILE, ts = j % TILE;
                const uint8_t* kt = P.cold + cold_tile_offset(dm, F, seq, kvh, 0, tl);
                const uint8_t* vt = P.cold + cold_tile_offset(dm, F, seq, kvh, 1, tl);
                uint32_t w[PBW + 1];
                const uint32_t* rec = reinterpret_cast<const uint32_t*>(kt + ts * (PAIRS * CB / 8));
#pragma unroll
                for (int i = 0; i < PBW; ++i) w[i] = rec[i];
                w[PBW] = 0u;
                float a[G];
#pragma unroll
                for (int h = 0; h < G; ++h) a[h] = 0.0f;
#pragma unroll
                for (int p = 0; p < PAIRS; ++p) {
                    const int bit = p * CB;
                    const int wi = bit >> 5, sh = bit & 31;
                    uint32_t code = w[wi] >> sh;
                    if (sh + CB > 32) code |= w[wi + 1] << (32 - sh);
                    code &= (1u << CB) - 1u;
                    const float2 u = s_lut[code];
                    const int i = pair_of_pos(p, D);
#pragma unroll
                    for (int h = 0; h < G; ++h) a[h] = fmaf(u.x, s_q[h][2 * i], fmaf(u.y, s_q[h][2 * i + 1], a[h]));
                }
                const float R = half_at(kt + TILE * (F.pb + F.sb) + 2 * ts);
                const float rho = half_at(kt + TILE * (F.pb + F.sb) + 2 * TILE + 2 * ts);
                float sd[G];
#pragma unroll
                for (int h = 0; h < G; ++h) sd[h] = 0.0f;
                const uint32_t* sg = reinterpret_cast<const uint32_t*>(kt + TILE * F.pb + ts * F.sb);
                for (int wd = 0; wd < m / 32; ++wd) {
                    const uint32_t bits = sg[wd];
                    for (int jj = 0; jj < 32; ++jj) {
                        const float s = ((bits >> jj) & 1u) ? 1.0f : -1.0f;
#pragma unroll
                        for (int h = 0; h < G; ++h) sd[h] = fmaf(s, s_sq[h][32 * wd + jj], sd[h]);
                    }
                }
#pragma unroll
                for (int h = 0; h < G; ++h) lg[h] = (a[h] * R + cm * rho * sd[h]) * isd;
                vR = half_at(vt + TILE * (F.pb + F.sb) + 2 * ts);
                vrho = half_at(vt + TILE * (F.pb + F.sb) + 2 * TILE + 2 * ts);
            } else {
#pragma unroll
                for (int h = 0; h < G; ++h) lg[h] = -INFINITY;
            }
        }
        if (logits && j < last) {
            const int pos = hot ? j : dm.cap + j;
#pragma unroll
            for (int h = 0; h < G; ++h) logits[((size_t)bi * dm.hq + kvh * G + h) * lstride + pos] = lg[h];
        }
        // online softmax
        float mt_[G];
#pragma unroll
        for (int h = 0; h < G; ++h) mt_[h] = lg[h];
        block_max<G>(mt_, s_red);
        float alpha[G], p[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mn = fmaxf(m_run[h], mt_[h]);
            alpha[h] = (m_run[h] == mn) ? 1.0f : __expf(m_run[h] - mn);
            p[h] = (lg[h] == -INFINITY) ? 0.0f : __expf(lg[h] - mn);
            m_run[h] = mn;
        }
        float ls[G];
#pragma unroll
        for (int h = 0; h < G; ++h) ls[h] = p[h];
        block_sum<G>(ls, s_red);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            l_run[h] = l_run[h] * alpha[h] + ls[h];
            s_pw[h][tid] = hot ? p[h] : p[h] * vR;
            s_pr[h][tid] = p[h] * vrho;
            acc[h][0] *= alpha[h];
            acc[h][1] *= alpha[h];
            acc_s[h] *= alpha[h];
        }
        // promotion candidates: only a token whose probability within this
        // tile reaches tau can reach it over the whole context
        if (!hot && ktop > 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (p[h] > 0.0f && p[h] >= dm.tau * ls[h]) {
                    const int at = atomicAdd(&s_ncand[h], 1);
                    if (at < 128) s_cand[h][at] = Cand{lg[h], j};
                }
            }
        }
        __syncthreads();
        if (!hot && ktop > 0 && tid < G) {
            // keep the entries still at >= tau of the running chunk softmax
            const int h = tid;
            const int n = min(s_ncand[h], 128);
            int k2 = 0;
            for (int i = 0; i < n; ++i) {
                const Cand cc = s_cand[h][i];
                if (__expf(cc.v - m_run[h]) >= dm.tau * l_run[h]) s_cand[h][k2++] = cc;
            }
            s_ncand[h] = k2;
        }
        // value accumulation for this tile
        if (hot) {
            const int k = tid % D, tg = tid / D;
            for (int t = tg; t < DTILE; t += NTH) {
                const int jj = t0 + t;
                if (jj >= last) break;
                const int phys = (mt.head + jj) % dm.cap;
                const float v = (float)P.ring_v[rb + (size_t)(phys / 32) * D * 32 + (size_t)k * 32 + (phys % 32)];
#pragma unroll
                for (int h = 0; h < G; ++h) acc[h][0] = fmaf(s_pw[h][t], v, acc[h][0]);
            }
        } else {
            const int i = tid % PAIRS, tg = tid / PAIRS;
            for (int t = tg; t < DTILE; t += NTG) {
                const int jj = t0 + t;
                if (jj >= last) break;
                const uint8_t* vt = P.cold + cold_tile_offset(dm, F, seq, kvh, 1, jj / TILE);
                const uint32_t* plane = reinterpret_cast<const uint32_t*>(vt + (size_t)i * 4 * CB);
                const uint32_t code = bits_at(plane, (jj % TILE) * CB, CB);
                const float2 u = s_lut[code];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float wgt = s_pw[h][t];
                    acc[h][0] = fmaf(wgt, u.x, acc[h][0]);
                    acc[h][1] = fmaf(wgt, u.y, acc[h][1]);
                }
            }
            if (tid < m * (DTILE / m)) {
                const int js = tid % m, sg = tid / m, nsg = DTILE / m;
                for (int t = sg; t < DTILE; t += nsg) {
                    const int jj = t0 + t;
                    if (jj >= last) break;
                    const uint8_t* vt = P.cold + cold_tile_offset(dm, F, seq, kvh, 1, jj / TILE);
                    const uint32_t bits = reinterpret_cast<const uint32_t*>(vt + TILE * F.pb)[js];
                    const float s = ((bits >> (jj % TILE)) & 1u) ? 1.0f : -1.0f;
#pragma unroll
                    for (int h = 0; h < G; ++h) acc_s[h] = fmaf(s, s_pr[h][t], acc_s[h]);
                }
            }
        }
        __syncthreads();
    }

    // reduce value accumulators over token groups and write the partials
    float* part0 = P.part + ((size_t)bi * dm.hq + kvh * G) * dm.max_chunks * stride;
    if (hot) {
        const int k = tid % D, tg = tid / D;
#pragma unroll
        for (int h = 0; h < G; ++h) s_acc[tg][h][k] = acc[h][0];
    } else {
        const int i = tid % PAIRS, tg = tid / PAIRS;
        // NTG may exceed 4 (D = 64): fold groups pairwise through LDS
        for (int base = 0; base < NTG; base += 4) {
            if (tg >= base && tg < base + 4) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float* dst = &s_acc[tg - base][h][2 * i];
                    if (base == 0) {
                        dst[0] = acc[h][0];
                        dst[1] = acc[h][1];
                    } else {
                        dst[0] += acc[h][0];
                        dst[1] += acc[h][1];
                    }
                }
            }
            __syncthreads();
        }
    }
    __syncthreads();
    const int ngroups = hot ? NTH : (NTG < 4 ? NTG : 4);
    for (int idx = tid; idx < G * D; idx += 256) {
        const int h = idx / D, k = idx % D;
        float s = 0.0f;
        for (int g2 = 0; g2 < ngroups; ++g2) s += s_acc[g2][h][k];
        float* pp = part0 + ((size_t)h * dm.max_chunks + c) * stride;
        pp[2 + k] = s;
    }
    __syncthreads();
    // sign accumulators (cold): reuse s_acc as [group][G][m]
    if (!hot) {
        float* red = &s_acc[0][0][0];
        const int nsg = DTILE / m;
        if (tid < m * nsg) {
            const int js = tid % m, sg = tid / m;
#pragma unroll
            for (int h = 0; h < G; ++h) red[(sg * G + h) * m + js] = acc_s[h];
        }
        __syncthreads();
        for (int idx = tid; idx < G * m; idx += 256) {
            const int h = idx / m, js = idx % m;
            float s = 0.0f;
            for (int g2 = 0; g2 < nsg; ++g2) s += red[(g2 * G + h) * m + js];
            part0[((size_t)h * dm.max_chunks + c) * stride + 2 + D + js] = s;
        }
    }
    if (tid < G) {
        float* pp = part0 + ((size_t)tid * dm.max_chunks + c) * stride;
        pp[0] = m_run[tid];
        pp[1] = l_run[tid];
        if (!hot && ktop > 0) {
            Cand* cc = P.cand_chunk + (((size_t)bi * dm.hq + kvh * G + tid) * dm.max_chunks + c) * ktop;
            const int n = min(s_ncand[tid], ktop);
            for (int i = 0; i < ktop; ++i) cc[i] = i < n ? s_cand[tid][i] : Cand{-INFINITY, -1};
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_combine(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs, int n_hot_chunks,
                                                 int n_chunks, float* __restrict__ out) {
    extern __shared__ float s_w[];  // [n_chunks]
    __shared__ float s_r[D];
    __shared__ float s_sg[M_MAX];
    __shared__ float s_red[4];
    __shared__ float s_ML[2];
    const int bi = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int seq = cs.ids[bi];
    const int stride = part_stride(D);
    const float* part = P.part + ((size_t)bi * dm.hq + h) * dm.max_chunks * stride;
    float mx = -INFINITY;
    for (int c = tid; c < n_chunks; c += 256) mx = fmaxf(mx, part[(size_t)c * stride]);
    mx = wave_max(mx);
    if ((tid & 63) == 0) s_red[tid >> 6] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();
    float ls = 0.0f;
    for (int c = tid; c < n_chunks; c += 256) {
        const float mc = part[(size_t)c * stride];
        const float w = (mc == -INFINITY) ? 0.0f : __expf(mc - M);
        s_w[c] = w;
        ls += w * part[(size_t)c * stride + 1];
    }
    ls = wave_sum(ls);
    if ((tid & 63) == 0) s_red[tid >> 6] = ls;
    __syncthreads();
    const float L = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    if (tid == 0) {
        s_ML[0] = M;
        s_ML[1] = L;
    }
    const int m = F.m;
    float ah = 0.0f, ar = 0.0f;
    if (tid < D) {
        for (int c = 0; c < n_chunks; ++c) {
            const float v = s_w[c] * part[(size_t)c * stride + 2 + tid];
            if (c < n_hot_chunks)
                ah += v;
            else
                ar += v;
        }
    } else if (tid >= 128 && tid - 128 < m) {
        const int j = tid - 128;
        float as = 0.0f;
        for (int c = n_hot_chunks; c < n_chunks; ++c) as += s_w[c] * part[(size_t)c * stride + 2 + D + j];
        s_sg[j] = as;
    }
    __syncthreads();
    if (tid < D) {
        float r = ar;
        if (dm.v_qjl) {
            const float cm = SQRT_HALF_PI / (float)m;
            float t = 0.0f;
            for (int j = 0; j < m; ++j) t = fmaf(P.s32[(size_t)j * D + tid], s_sg[j], t);
            r = fmaf(cm, t, r);
        }
        s_r[tid] = r;
    }
    __syncthreads();
    if (tid < D) {
        float o = 0.0f;
        for (int k = 0; k < D; ++k) o = fmaf(P.pi32[(size_t)k * D + tid], s_r[k], o);
        o += ah;
        out[((size_t)bi * dm.hq + h) * D + tid] = L > 0.0f ? o / L : 0.0f;
    }
    if (tid == 0) {
        const size_t sl = sl_index(dm, seq, layer);
        if (dm.ktop > 0) {
            Cand* dst = P.cand + (sl * dm.hq + h) * dm.ktop;
            int n = 0;
            for (int c = n_hot_chunks; c < n_chunks; ++c) {
                const Cand* cc = P.cand_chunk + (((size_t)bi * dm.hq + h) * dm.max_chunks + c) * dm.ktop;
                for (int i = 0; i < dm.ktop; ++i) {
                    if (cc[i].slot < 0) break;
                    const float pr = __expf(cc[i].v - M) / L;
                    if (pr >= dm.tau && n < dm.ktop) dst[n++] = Cand{pr, cc[i].slot};
                }
            }
            P.cand_n[sl * dm.hq + h] = n;
        }
        if (h == 0) P.meta[sl].attn_step += 1;
    }
}

template <int D, int CB, int G>
static void decode_launch(dim3 grid, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                          const CallSeqs& cs, const _Float16* q, int nh, int ct, float* logits, int lstride) {
    k_decode<D, CB, G><<<grid, 256, 0, st>>>(dm, P, F, layer, cs, q, nh, ct, logits, lstride);
}

template <int D, int CB>
static hipError_t decode_g(dim3 grid, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                           const CallSeqs& cs, const _Float16* q, int nh, int ct, float* logits, int lstride) {
    switch (dm.g) {
        case 1: decode_launch<D, CB, 1>(grid, st, dm, P, F, layer, cs, q, nh, ct, logits, lstride); break;
        case 2: decode_launch<D, CB, 2>(grid, st, dm, P, F, layer, cs, q, nh, ct, logits, lstride); break;
        case 4: decode_launch<D, CB, 4>(grid, st, dm, P, F, layer, cs, q, nh, ct, logits, lstride); break;
        case 8: decode_launch<D, CB, 8>(grid, st, dm, P, F, layer, cs, q, nh, ct, logits, lstride); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

hipError_t launch_decode(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                         int cold_bound, const _Float16* q, float* out, float* logits, int logits_stride,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (cs.n == 0) return hipSuccess;
    const int n_hot = (dm.cap + DTILE - 1) / DTILE;
    const int cold_tiles = (cold_bound + DTILE - 1) / DTILE;
    // chunk size: enough blocks to fill the chip, at most 16 tiles per chunk
    const int target = 2048;
    const int per_seq = std::max(1, target / std::max(1, cs.n * dm.hkv));
    int ct = cold_tiles > 0 ? (cold_tiles + per_seq - 1) / per_seq : 1;
    ct = std::max(1, std::min(ct, 16));
    const int n_cold = (cold_tiles + ct - 1) / ct;
    const int n_chunks = n_hot + n_cold;
    if (n_chunks > dm.max_chunks) return hipErrorInvalidValue;
    if (logits) {
        const size_t n = (size_t)cs.n * dm.hq * logits_stride;
        k_fill<<<(unsigned)std::min<size_t>((n + 255) / 256, 65536), 256, 0, st>>>(logits, n, -INFINITY);
    }
    const dim3 gq(cs.n, dm.hq);
    if (dm.d == 64)
        k_qprep<64><<<gq, 128, 0, st>>>(dm, P, q);
    else
        k_qprep<128><<<gq, 128, 0, st>>>(dm, P, q);
    if (ev0) hipEventRecord(ev0, st);
    const dim3 grid(n_chunks, cs.n, dm.hkv);
    hipError_t e = hipSuccess;
    const int key = dm.d * 10 + F.cb;
    switch (key) {
        case 645: e = decode_g<64, 5>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, logits, logits_stride); break;
        case 647: e = decode_g<64, 7>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, logits, logits_stride); break;
        case 644: e = decode_g<64, 4>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, logits, logits_stride); break;
        case 1285: e = decode_g<128, 5>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, logits, logits_stride); break;
        case 1287: e = decode_g<128, 7>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, logits, logits_stride); break;
        case 1284: e = decode_g<128, 4>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, logits, logits_stride); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (ev1) hipEventRecord(ev1, st);
    const size_t shm = (size_t)n_chunks * sizeof(float);
    if (dm.d == 64)
        k_combine<64><<<gq, 256, shm, st>>>(dm, P, F, layer, cs, n_hot, n_chunks, out);
    else
        k_combine<128><<<gq, 256, shm, st>>>(dm, P, F, layer, cs, n_hot, n_chunks, out);
    return hipGetLastError();
}

}  // namespace tq
