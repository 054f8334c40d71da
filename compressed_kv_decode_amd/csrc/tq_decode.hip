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
//   k_decode  split-context attention.  Each wave owns one chunk: a range of
//             32-token tiles of either the hot ring or the cold slots of one
//             (sequence, kv head).  Per tile:
//               logits  16x16x32 f16 MFMA.  A = the query rows of the head
//                       group (rows h: fp16 hi part, rows G+h: lo part x 2^12),
//                       B = 16 tokens' dequantised unit pair values (cold:
//                       fp16 hi and lo tables in LDS, two MFMAs) or fp16 keys
//                       (hot).  The QJL term is a second contraction of S q'
//                       (hi/lo rows) against the tokens' signs as +-1.
//               softmax online per head, within the wave.
//               values  16x16x32 f16 MFMA, A = p * R (hi/lo rows), B = the
//                       unit pair values of 8 tokens per lane (V tiles are
//                       pair-major so a lane reads its pair's codes for 8
//                       tokens at once) or the fp16 values of the transposed
//                       hot ring; the QJL term accumulates p * rho against
//                       the sign planes.
//             Cold accumulators stay in the rotated domain.  Writes per-head
//             (max, sum, accumulators) and promotion candidates per chunk.
//   k_combine merges the chunks of each (sequence, query head), adds the QJL
//             back-projection S_m^T, rotates back with Pi^T, normalises, and
//             turns candidate logits into exact probabilities.
#include <math.h>

#include "tq_device.h"

namespace tq {

constexpr float SQRT_HALF_PI = 1.25331413731550025121f;
constexpr float INV_LO = 1.0f / LO_SCALE;

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

// fp16 +-1 for 8 sign bits: bit set -> +1 (0x3C00), clear -> -1 (0xBC00)
__device__ __forceinline__ half8 signs8(uint32_t byte) {
    union {
        uint32_t u[4];
        half8 h;
    } r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t b0 = (byte >> (2 * k)) & 1u, b1 = (byte >> (2 * k + 1)) & 1u;
        r.u[k] = 0xBC00BC00u ^ (b0 << 15) ^ (b1 << 31);
    }
    return r.h;
}

__device__ __forceinline__ void split_hl(float v, _Float16& hi, _Float16& lo) {
    pin(v);
    hi = (_Float16)v;
    lo = (_Float16)((v - (float)hi) * LO_SCALE);
}

// A operand of a query contraction: lane row i = lane % 16 holds, for k =
// 8 (lane / 16) .. +7 of the block, the hi part of head i's vector (i < G),
// the lo part x 2^12 of head i - G (G <= i < 2G), else 0.
template <int G>
__device__ __forceinline__ half8 query_rows(const float* vecs, int stride, int k0, int lane) {
    const int row = lane & 15;
    half8 a;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        _Float16 hi = (_Float16)0.0f, lo = (_Float16)0.0f;
        if (row < 2 * G) {
            const float v = vecs[(row % G) * stride + k0 + 8 * (lane >> 4) + r];
            split_hl(v, hi, lo);
        }
        a[r] = row < G ? hi : (row < 2 * G ? lo : (_Float16)0.0f);
    }
    return a;
}

// Value of query-row contraction for (head h, column col) from accumulators
// whose rows are laid out by query_rows: hi row h and lo row G + h.  The
// caller has written the 2G used rows of each accumulator to LDS.
struct WaveLds {
    float acc[3][16][16];  // logit accumulators, rows x 16 tokens
    float lg[8][32];       // tile logits per head
    float w[8][32];        // p * R per head and token
    float wr[8][32];       // p * rho per head and token
    float alpha[8];        // rescale of the running accumulators per head
    float mrun[8], lrun[8];
    int ncand[8];
};

template <int D, int CB, int M, int G>
__global__ __launch_bounds__(256) void k_decode(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs,
                                                const _Float16* __restrict__ qin, int n_hot_chunks, int hot_tiles,
                                                int cold_tiles, int n_chunks, float* logits, int lstride) {
    constexpr int PAIRS = D / 2;
    constexpr int PB = PAIRS * CB / 8;       // pair-code bytes per K record
    constexpr int SB = M / 8;                // sign bytes per K record
    constexpr int QB = (D / 8) * CB;         // code bits of one record quarter
    constexpr int QW = (QB + 31 + 31) / 32;  // dwords covering a quarter at any shift
    constexpr int NKB = D / 32;              // 32-wide k blocks of a key
    constexpr int NSB = M / 32;              // 32-wide k blocks of the signs
    constexpr int NPG = PAIRS / 16;          // groups of 16 pairs (value n-tiles)
    constexpr int VW = (8 * CB + 31 + 31) / 32;  // dwords covering 8 codes of a plane
    constexpr int NVT = D / 16;              // hot value n-tiles

    __shared__ uint32_t s_khi[1 << CB], s_klo[1 << CB], s_v[1 << CB];
    __shared__ WaveLds s_wave[4];
    extern __shared__ Cand s_cand_all[];  // [4 waves][G][2 * ktop]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q4 = lane >> 4, col = lane & 15;
    const int bi = blockIdx.y, kvh = blockIdx.z;
    const int seq = cs.ids[bi];
    const size_t sl = sl_index(dm, seq, layer);
    const SeqLayerMeta mt = P.meta[sl];
    const int ktop = dm.ktop;
    WaveLds& W = s_wave[wave];
    Cand* s_cand = s_cand_all + (size_t)wave * G * 2 * (ktop > 0 ? ktop : 1);

    // dequantisation tables: unit pair values (a / (L_r - 1)) (cos, sin)(phi_b)
    {
        const int LR = 1 << F.rb;
        for (int code = tid; code < (1 << CB); code += 256) {
            const int a = code & (LR - 1), b = code >> F.rb;
            const float s = (float)a / (float)(LR - 1);
            _Float16 xh, xl, yh, yl;
            split_hl(s * F.cos_t[b], xh, xl);
            split_hl(s * F.sin_t[b], yh, yl);
            union {
                _Float16 h[2];
                uint32_t u;
            } u1, u2, u3;
            u1.h[0] = xh, u1.h[1] = yh;
            u2.h[0] = xl, u2.h[1] = yl;
            u3.h[0] = (_Float16)(s * F.cos_t[b]);
            u3.h[1] = (_Float16)(s * F.sin_t[b]);
            s_khi[code] = u1.u;
            s_klo[code] = u2.u;
            s_v[code] = u3.u;
        }
    }
    if (lane < 8) {
        W.ncand[lane] = 0;
        W.mrun[lane] = -INFINITY;
        W.lrun[lane] = 0.0f;
    }
    __syncthreads();

    const int c = blockIdx.x * 4 + wave;
    if (c >= n_chunks) return;
    const bool hot = c < n_hot_chunks;
    int t_first, t_last;  // tile range of this wave
    if (hot) {
        t_first = c * hot_tiles;
        t_last = min(t_first + hot_tiles, dm.cap / TILE);
    } else {
        t_first = (c - n_hot_chunks) * cold_tiles;
        t_last = min(t_first + cold_tiles, (mt.cold_len + TILE - 1) / TILE);
    }
    const float isd = 1.0f / sqrtf((float)D);
    const float cm = SQRT_HALF_PI / (float)M;
    const size_t rb = ring_base(dm, seq, layer, kvh);
    const uint32_t* tomb = P.tomb + sl * (dm.cold_cap / 32);

    // query operands
    half8 aq[NKB], as[NSB];
    if (hot) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                aq[kb][r] = col < G ? qin[((size_t)bi * dm.hq + kvh * G + col) * D + kb * 32 + 8 * q4 + r]
                                    : (_Float16)0.0f;
        }
    } else {
        const float* qp = P.qprep + ((size_t)bi * dm.hq + kvh * G) * (D + M_MAX);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) aq[kb] = query_rows<G>(qp, D + M_MAX, kb * 32, lane);
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) as[sb] = query_rows<G>(qp + D, D + M_MAX, sb * 32, lane);
    }

    // value accumulators (rows: hi h / lo G + h; columns: components or signs)
    floatx4 vx[NVT];   // hot: component n-tiles; cold: x (even n) and y (odd n) per pair group
    floatx4 vs[M / 16];
#pragma unroll
    for (int n = 0; n < NVT; ++n) vx[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < M / 16; ++n) vs[n] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int T = t_first; T < t_last; ++T) {
        // ---------------- logits of the 32 tokens of tile T ----------------
        for (int st = 0; st < 2; ++st) {
            const int tok = st * 16 + col;  // token within the tile
            floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f}, a3 = {0.f, 0.f, 0.f, 0.f};
            float Rt = 0.0f, rhot = 0.0f;
            bool live;
            if (hot) {
                const int phys = T * TILE + tok;
                live = ((phys - mt.head + dm.cap) % dm.cap) < mt.count;
                const _Float16* kr = P.ring_k + rb + (size_t)phys * D;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const half8 kk = *reinterpret_cast<const half8*>(kr + kb * 32 + 8 * q4);
                    a1 = mfma16x16x32(aq[kb], kk, a1);
                }
            } else {
                const int slot = T * TILE + tok;
                live = slot < mt.cold_len && !((tomb[slot >> 5] >> (slot & 31)) & 1u);
                const uint8_t* kt = P.cold + cold_tile_offset(dm, F, seq, kvh, 0, T);
                // this lane's quarter of the record: codes of pairs 16 b + 4 q4 + j
                const int bit0 = q4 * QB;
                const uint32_t* rw = reinterpret_cast<const uint32_t*>(kt + tok * PB) + (bit0 >> 5);
                uint32_t w[QW];
#pragma unroll
                for (int i = 0; i < QW; ++i) w[i] = rw[i];
                const uint32_t sh = bit0 & 31;
                uint32_t al[QW - 1];
#pragma unroll
                for (int i = 0; i < QW - 1; ++i) al[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    union {
                        uint32_t u[4];
                        half8 h;
                    } bh, bl;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int bo = (4 * kb + j) * CB;
                        uint32_t code = al[bo >> 5] >> (bo & 31);
                        if ((bo & 31) + CB > 32) code |= al[(bo >> 5) + 1] << (32 - (bo & 31));
                        code &= (1u << CB) - 1u;
                        bh.u[j] = s_khi[code];
                        bl.u[j] = s_klo[code];
                    }
                    a1 = mfma16x16x32(aq[kb], bh.h, a1);
                    a2 = mfma16x16x32(aq[kb], bl.h, a2);
                }
                const uint8_t* sgn = kt + TILE * PB + tok * SB;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) a3 = mfma16x16x32(as[sb], signs8(sgn[4 * sb + q4]), a3);
                const uint8_t* meta = kt + TILE * (PB + SB);
                Rt = half_at(meta + 2 * tok);
                rhot = half_at(meta + 2 * TILE + 2 * tok);
            }
            // rows 4 q4 + r of the accumulators, column col -> LDS
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * q4 + r;
                if (row < 2 * G) {
                    W.acc[0][row][col] = a1[r];
                    W.acc[1][row][col] = a2[r];
                    W.acc[2][row][col] = a3[r];
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            // lane (h = lane / 16 + 4 k, column col) assembles logits
#pragma unroll
            for (int k = 0; k < (G + 3) / 4; ++k) {
                const int h = q4 + 4 * k;
                if (h < G) {
                    float lg;
                    if (hot) {
                        lg = W.acc[0][h][col] * isd;
                    } else {
                        const float pol = W.acc[0][h][col] + (W.acc[1][h][col] + W.acc[0][G + h][col]) * INV_LO +
                                          W.acc[1][G + h][col] * (INV_LO * INV_LO);
                        const float sd = W.acc[2][h][col] + W.acc[2][G + h][col] * INV_LO;
                        lg = (pol * Rt + cm * rhot * sd) * isd;
                    }
                    W.lg[h][tok] = live ? lg : -INFINITY;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        // ---------------- online softmax over the tile ----------------
        // lane handles heads q4 + 4 k, tokens col and col + 16
        float vR[2] = {1.0f, 1.0f}, vrho[2] = {0.0f, 0.0f};
        if (!hot) {
            const uint8_t* vm = P.cold + cold_tile_offset(dm, F, seq, kvh, 1, T) + TILE * (PB + SB);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                vR[u] = half_at(vm + 2 * (col + 16 * u));
                vrho[u] = half_at(vm + 2 * TILE + 2 * (col + 16 * u));
            }
        }
#pragma unroll
        for (int k = 0; k < (G + 3) / 4; ++k) {
            const int h = q4 + 4 * k;
            const bool ok = h < G;
            const int hh = ok ? h : 0;
            const float l0 = ok ? W.lg[hh][col] : -INFINITY, l1 = ok ? W.lg[hh][col + 16] : -INFINITY;
            if (logits && ok) {
                float* lrow = logits + ((size_t)bi * dm.hq + kvh * G + h) * lstride;
                for (int u = 0; u < 2; ++u) {
                    const int t = T * TILE + col + 16 * u;
                    const float lv = u ? l1 : l0;
                    if (hot) {
                        const int fifo = (t - mt.head + dm.cap) % dm.cap;
                        if (fifo < mt.count) lrow[fifo] = lv;
                    } else if (t < mt.cold_len) {
                        lrow[dm.cap + t] = lv;
                    }
                }
            }
            float mx = fmaxf(l0, l1);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float mold = W.mrun[hh];
            const float mn = fmaxf(mold, mx);
            const float alpha = (mold == mn) ? 1.0f : __expf(mold - mn);
            const float p0 = (l0 == -INFINITY) ? 0.0f : __expf(l0 - mn);
            const float p1 = (l1 == -INFINITY) ? 0.0f : __expf(l1 - mn);
            float ls = p0 + p1;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) ls += __shfl_xor(ls, o, 64);
            __builtin_amdgcn_wave_barrier();
            if (ok) {
                W.w[h][col] = p0 * vR[0];
                W.w[h][col + 16] = p1 * vR[1];
                W.wr[h][col] = p0 * vrho[0];
                W.wr[h][col + 16] = p1 * vrho[1];
                if (col == 0) {
                    W.alpha[h] = alpha;
                    W.mrun[h] = mn;
                    W.lrun[h] = W.lrun[h] * alpha + ls;
                }
                // promotion candidates: only a token reaching tau within its
                // tile can reach it over the whole context
                if (!hot && ktop > 0) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const float pv = u ? p1 : p0;
                        if (pv > 0.0f && pv >= dm.tau * ls) {
                            const int at = atomicAdd(&W.ncand[h], 1);
                            if (at < 2 * ktop) s_cand[h * 2 * ktop + at] = Cand{u ? l1 : l0, T * TILE + col + 16 * u};
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        if (!hot && ktop > 0 && lane < G) {
            // keep the entries still at >= tau of the running chunk softmax
            const int h = lane;
            const int n = min(W.ncand[h], 2 * ktop);
            int k2 = 0;
            for (int i = 0; i < n; ++i) {
                const Cand cc = s_cand[h * 2 * ktop + i];
                if (__expf(cc.v - W.mrun[h]) >= dm.tau * W.lrun[h] && k2 < ktop) s_cand[h * 2 * ktop + k2++] = cc;
            }
            W.ncand[h] = k2;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        // ---------------- values ----------------
        // rescale the running accumulators (rows 4 q4 + r belong to head row % G)
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * q4 + r;
            ar[r] = row < 2 * G ? W.alpha[row % G] : 1.0f;
        }
#pragma unroll
        for (int n = 0; n < NVT; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) vx[n][r] *= ar[r];
#pragma unroll
        for (int n = 0; n < M / 16; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) vs[n][r] *= ar[r];
        // A operands: row col, tokens 8 q4 .. +7
        half8 av, avs;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            _Float16 hi = (_Float16)0.0f, lo = (_Float16)0.0f, shi = (_Float16)0.0f, slo = (_Float16)0.0f;
            if (col < 2 * G) {
                split_hl(W.w[col % G][8 * q4 + r], hi, lo);
                split_hl(W.wr[col % G][8 * q4 + r], shi, slo);
            }
            av[r] = col < G ? hi : (col < 2 * G ? lo : (_Float16)0.0f);
            avs[r] = col < G ? shi : (col < 2 * G ? slo : (_Float16)0.0f);
        }
        if (hot) {
            const _Float16* vt = P.ring_v + rb + (size_t)T * D * TILE;
#pragma unroll
            for (int n = 0; n < NVT; ++n) {
                const half8 vv = *reinterpret_cast<const half8*>(vt + (size_t)(16 * n + col) * TILE + 8 * q4);
                vx[n] = mfma16x16x32(av, vv, vx[n]);
            }
        } else {
            const uint8_t* vt = P.cold + cold_tile_offset(dm, F, seq, kvh, 1, T);
            const int bit0 = 8 * q4 * CB;
#pragma unroll
            for (int g = 0; g < NPG; ++g) {
                const int pair = 16 * g + col;
                const uint32_t* pw = reinterpret_cast<const uint32_t*>(vt + (size_t)pair * 4 * CB) + (bit0 >> 5);
                uint32_t w[VW];
#pragma unroll
                for (int i = 0; i < VW; ++i) w[i] = (bit0 >> 5) + i < CB ? pw[i] : 0u;
                const uint32_t sh = bit0 & 31;
                uint32_t al[VW - 1];
#pragma unroll
                for (int i = 0; i < VW - 1; ++i) al[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
                union {
                    uint32_t u[4];
                    half8 h;
                } bx, by;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t e2[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int bo = (2 * j + e) * CB;
                        uint32_t code = al[bo >> 5] >> (bo & 31);
                        if ((bo & 31) + CB > 32) code |= al[(bo >> 5) + 1] << (32 - (bo & 31));
                        e2[e] = s_v[code & ((1u << CB) - 1u)];
                    }
                    bx.u[j] = __builtin_amdgcn_perm(e2[1], e2[0], 0x05040100u);  // x halves of tokens 2j, 2j+1
                    by.u[j] = __builtin_amdgcn_perm(e2[1], e2[0], 0x07060302u);  // y halves
                }
                vx[2 * g] = mfma16x16x32(av, bx.h, vx[2 * g]);
                vx[2 * g + 1] = mfma16x16x32(av, by.h, vx[2 * g + 1]);
            }
            const uint32_t* sp = reinterpret_cast<const uint32_t*>(vt + TILE * PB);
#pragma unroll
            for (int n = 0; n < M / 16; ++n) {
                const uint32_t bits = sp[16 * n + col];
                vs[n] = mfma16x16x32(avs, signs8((bits >> (8 * q4)) & 0xffu), vs[n]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---------------- partials ----------------
    const int stride = part_stride(D);
    float* part0 = P.part + ((size_t)bi * dm.hq + kvh * G) * dm.max_chunks * stride;
    // fold hi/lo rows through LDS, 16 columns at a time
    float (*fold)[16] = W.acc[0];
    for (int n = 0; n < NVT + M / 16; ++n) {
        const floatx4 v = n < NVT ? vx[n] : vs[n - NVT];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * q4 + r;
            if (row < 2 * G) fold[row][col] = v[r];
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < (G + 3) / 4; ++k) {
            const int h = q4 + 4 * k;
            if (h < G) {
                const float val = fold[h][col] + fold[G + h][col] * INV_LO;
                float* pp = part0 + ((size_t)h * dm.max_chunks + c) * stride;
                int idx;
                if (n >= NVT) {
                    idx = 2 + D + 16 * (n - NVT) + col;
                } else if (hot) {
                    idx = 2 + 16 * n + col;
                } else {
                    idx = 2 + 2 * (16 * (n >> 1) + col) + (n & 1);  // pair 16 g + col, x (even n) or y
                }
                pp[idx] = val;
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (lane < G) {
        float* pp = part0 + ((size_t)lane * dm.max_chunks + c) * stride;
        pp[0] = W.mrun[lane];
        pp[1] = W.lrun[lane];
        if (!hot && ktop > 0) {
            Cand* cc = P.cand_chunk + (((size_t)bi * dm.hq + kvh * G + lane) * dm.max_chunks + c) * ktop;
            const int n = min(W.ncand[lane], ktop);
            for (int i = 0; i < ktop; ++i) cc[i] = i < n ? s_cand[lane * 2 * ktop + i] : Cand{-INFINITY, -1};
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
    const int m = F.m;
    float ah = 0.0f, ar = 0.0f;
    if (tid < D) {
        for (int c = 0; c < n_chunks; ++c) {
            const float w = s_w[c];
            if (w == 0.0f) continue;
            const float v = w * part[(size_t)c * stride + 2 + tid];
            if (c < n_hot_chunks)
                ah += v;
            else
                ar += v;
        }
    } else if (tid >= 128 && tid - 128 < m) {
        const int j = tid - 128;
        float as = 0.0f;
        for (int c = n_hot_chunks; c < n_chunks; ++c) {
            const float w = s_w[c];
            if (w != 0.0f) as += w * part[(size_t)c * stride + 2 + D + j];
        }
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

template <int D, int CB, int M, int G>
static void decode_launch(dim3 grid, size_t shm, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F,
                          int layer, const CallSeqs& cs, const _Float16* q, int nh, int ht, int ct, int nc,
                          float* logits, int lstride) {
    k_decode<D, CB, M, G><<<grid, 256, shm, st>>>(dm, P, F, layer, cs, q, nh, ht, ct, nc, logits, lstride);
}

template <int D, int CB, int M>
static hipError_t decode_g(dim3 grid, size_t shm, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F,
                           int layer, const CallSeqs& cs, const _Float16* q, int nh, int ht, int ct, int nc,
                           float* logits, int lstride) {
    switch (dm.g) {
        case 1: decode_launch<D, CB, M, 1>(grid, shm, st, dm, P, F, layer, cs, q, nh, ht, ct, nc, logits, lstride); break;
        case 2: decode_launch<D, CB, M, 2>(grid, shm, st, dm, P, F, layer, cs, q, nh, ht, ct, nc, logits, lstride); break;
        case 4: decode_launch<D, CB, M, 4>(grid, shm, st, dm, P, F, layer, cs, q, nh, ht, ct, nc, logits, lstride); break;
        case 8: decode_launch<D, CB, M, 8>(grid, shm, st, dm, P, F, layer, cs, q, nh, ht, ct, nc, logits, lstride); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

template <int D, int CB>
static hipError_t decode_m(dim3 grid, size_t shm, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F,
                           int layer, const CallSeqs& cs, const _Float16* q, int nh, int ht, int ct, int nc,
                           float* logits, int lstride) {
    if (F.m == 32) return decode_g<D, CB, 32>(grid, shm, st, dm, P, F, layer, cs, q, nh, ht, ct, nc, logits, lstride);
    if (F.m == 64) return decode_g<D, CB, 64>(grid, shm, st, dm, P, F, layer, cs, q, nh, ht, ct, nc, logits, lstride);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                         int cold_bound, const _Float16* q, float* out, float* logits, int logits_stride,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (cs.n == 0) return hipSuccess;
    // hot ring: one 32-slot tile per wave; cold: chunks of whole tiles, sized
    // so that the launch has enough waves to cover the chip
    const int hot_tiles = 1;
    const int n_hot = dm.cap / TILE;
    const int cold_tiles_total = (cold_bound + TILE - 1) / TILE;
    const int target_waves = 8192;
    int per = std::max(1, target_waves / std::max(1, cs.n * dm.hkv));
    per = std::min(per, MAX_COLD_CHUNKS);
    int ct = cold_tiles_total > 0 ? (cold_tiles_total + per - 1) / per : 1;
    const int n_cold = cold_tiles_total > 0 ? (cold_tiles_total + ct - 1) / ct : 0;
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
    const dim3 grid((n_chunks + 3) / 4, cs.n, dm.hkv);
    const size_t shm = (size_t)4 * dm.g * 2 * std::max(dm.ktop, 1) * sizeof(Cand);
    hipError_t e = hipSuccess;
    const int key = dm.d * 10 + F.cb;
    switch (key) {
        case 645: e = decode_m<64, 5>(grid, shm, st, dm, P, F, layer, cs, q, n_hot, hot_tiles, ct, n_chunks, logits, logits_stride); break;
        case 647: e = decode_m<64, 7>(grid, shm, st, dm, P, F, layer, cs, q, n_hot, hot_tiles, ct, n_chunks, logits, logits_stride); break;
        case 644: e = decode_m<64, 4>(grid, shm, st, dm, P, F, layer, cs, q, n_hot, hot_tiles, ct, n_chunks, logits, logits_stride); break;
        case 1285: e = decode_m<128, 5>(grid, shm, st, dm, P, F, layer, cs, q, n_hot, hot_tiles, ct, n_chunks, logits, logits_stride); break;
        case 1287: e = decode_m<128, 7>(grid, shm, st, dm, P, F, layer, cs, q, n_hot, hot_tiles, ct, n_chunks, logits, logits_stride); break;
        case 1284: e = decode_m<128, 4>(grid, shm, st, dm, P, F, layer, cs, q, n_hot, hot_tiles, ct, n_chunks, logits, logits_stride); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (ev1) hipEventRecord(ev1, st);
    const size_t shc = (size_t)n_chunks * sizeof(float);
    if (dm.d == 64)
        k_combine<64><<<gq, 256, shc, st>>>(dm, P, F, layer, cs, n_hot, n_chunks, out);
    else
        k_combine<128><<<gq, 256, shc, st>>>(dm, P, F, layer, cs, n_hot, n_chunks, out);
    return hipGetLastError();
}

}  // namespace tq
