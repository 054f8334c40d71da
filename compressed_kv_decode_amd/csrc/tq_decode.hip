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
//             (sequence, kv head).  Cold tiles are staged into LDS with
//             asynchronous global-to-LDS loads, one tile ahead of the tile
//             being computed.  Per tile:
//               logits  16x16x32 f16 MFMA with the tokens as rows (A: the
//                       dequantised unit pair values of 16 tokens, fp16 hi and
//                       lo from a two-code table) and the query heads as
//                       columns (B: q' hi and lo, each head in two columns);
//                       hi*hi and the two cross terms go to separate
//                       accumulators.  The QJL term contracts the tokens'
//                       signs (+-1 from a nibble table) with S q' (hi, lo).
//               softmax online per head, within the wave (lanes of a column
//                       hold 8 tokens; permlane swaps reduce across rows).
//               values  16x16x32 f16 MFMA, A = p * R (rows h: hi, rows G + h:
//                       lo x 2^12), transposed from the logit layout with
//                       permlane swaps; B = the unit pair values of 8 tokens
//                       per lane from the pair-major value planes (two-code
//                       table), or the fp16 values of the transposed hot ring;
//                       the QJL term accumulates p * rho against sign planes.
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

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

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

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0) only

// Copy BYTES (a multiple of 16) from global memory to this wave's LDS, 1 KB
// per instruction with every lane active: lane l of chunk i moves bytes
// [1024 i + 16 l, +16).  In the last chunk the lanes past BYTES re-read the
// final 16 bytes and land in the slack that rounds the LDS buffer up to whole
// KB, so no global byte outside the source is touched.  (A copy whose tail
// ran on part of the wave could be merged by the compiler with the next copy
// under one LDS base, which is wrong: the LDS base of this DMA is taken from
// the first active lane.)
template <int BYTES>
__device__ __forceinline__ void stage_copy(const uint8_t* g, uint8_t* lds, int lane) {
#pragma unroll
    for (int off = 0; off < BYTES; off += 1024) {
        const int o = min(off + 16 * lane, BYTES - 16);
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(g + o), (lds_void_t*)(lds + off), 16, 0, 0);
    }
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

// fp16 bits of the role of this lane's column: hi part (col < G), lo part
// x 2^12 (G <= col < 2G) or 0.
template <int G>
__device__ __forceinline__ uint32_t role_half(float v, int col) {
    _Float16 hi, lo;
    split_hl(v, hi, lo);
    const _Float16 r = col < G ? hi : (col < 2 * G ? lo : (_Float16)0.0f);
    union {
        _Float16 h;
        uint16_t u;
    } c;
    c.h = r;
    return c.u;
}

// Bits [bit, bit + n) of a dword array (bit and n compile-time after unrolling).
template <int NW>
__device__ __forceinline__ uint32_t field(const uint32_t (&al)[NW], int bit, int n) {
    uint32_t v = al[bit >> 5] >> (bit & 31);
    if ((bit & 31) + n > 32) v |= al[(bit >> 5) + 1] << (32 - (bit & 31));
    return v & ((1u << n) - 1u);
}

// Row max / sum across the four 16-lane rows of the wave (same column).
__device__ __forceinline__ float rows_max(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Transpose the value weights of a tile into the A operand of the value MFMA.
// In: lane (row q4, column) holds tokens 4 q4 + r of subtile 0 (lo01 =
// tokens r 0,1 packed, lo23 = r 2,3) and of subtile 1 (hi01, hi23).
// Out: lane (row q4) holds tokens 8 q4 .. 8 q4 + 7 of the tile.
__device__ __forceinline__ half8 tile_transpose(uint32_t s0_01, uint32_t s0_23, uint32_t s1_01, uint32_t s1_23) {
    auto a = __builtin_amdgcn_permlane32_swap(s0_01, s1_01, false, false);
    auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);  // (X01, Y01)
    auto c = __builtin_amdgcn_permlane32_swap(s0_23, s1_23, false, false);
    auto d = __builtin_amdgcn_permlane16_swap(c[0], c[1], false, false);  // (X23, Y23)
    union {
        uint32_t u[4];
        half8 h;
    } r;
    r.u[0] = b[0], r.u[1] = d[0], r.u[2] = b[1], r.u[3] = d[1];
    return r.h;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

template <int D, int CB, int M>
struct Geom {
    static constexpr int PAIRS = D / 2;
    static constexpr int PB = PAIRS * CB / 8;        // pair-code bytes per K record
    static constexpr int SB = M / 8;                 // sign bytes per K record
    static constexpr int TB = TILE * (PB + SB + 4);  // bytes of one K or V tile
    static constexpr int QB = (D / 8) * CB;          // code bits of one record quarter
    static constexpr int QW = (QB + 31 + 31) / 32;   // dwords covering a quarter at any shift
    static constexpr int NKB = D / 32;               // 32-wide k blocks of a key
    static constexpr int NSB = M / 32;               // 32-wide k blocks of the signs
    static constexpr int NPG = PAIRS / 16;           // groups of 16 pairs (value n-tiles)
    static constexpr int VW = (8 * CB + 31 + 31) / 32;  // dwords covering 8 codes of a plane
    static constexpr int NVT = D / 16;               // value n-tiles
    static constexpr bool PAIR2 = CB <= 5;
    static constexpr int KTAB = PAIR2 ? (16 << (2 * CB)) : (8 << CB);
    static constexpr int VTAB = PAIR2 ? (8 << (2 * CB)) : (4 << CB);
    static constexpr int TABS = (KTAB + VTAB + SIGN_TAB_BYTES + 1023) / 1024 * 1024;
    static constexpr int HALF = (TB + 1023) / 1024 * 1024;  // one staged K or V tile, whole KB
};

// Everything one tile of 32 tokens does in one wave: logits, online softmax,
// promotion candidates and value accumulation.  HOT: the tile is ring tile
// T (fp16, read from global memory); else kt / vt are the K / V tile staged
// in LDS and tw is its tombstone word.
template <int D, int CB, int M, int G, bool HOT>
__device__ __forceinline__ void tile_body(const Dims& dm, const Ptrs& P, const SeqLayerMeta& mt, int T,
                                          const uint8_t* kt, const uint8_t* vt, uint32_t tw, size_t rb, int q4,
                                          int col, int lane, const half8* qh, const half8* ql, const half8* sh,
                                          const half8* slo, floatx4* vx, floatx4* vs, float& m_run, float& l_run,
                                          const uint8_t* s_ktab, const uint8_t* s_vtab, const uint8_t* s_stab,
                                          float* lrow, float isd, float cm, float (&lgc)[8], uint32_t& cmask) {
    using Gm = Geom<D, CB, M>;
    // ------------------------------------------------------------ logits
    float lg[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        floatx4 am = {0.f, 0.f, 0.f, 0.f}, alo = {0.f, 0.f, 0.f, 0.f};
        floatx4 as = {0.f, 0.f, 0.f, 0.f}, asl = {0.f, 0.f, 0.f, 0.f};
        const int tokA = st * 16 + col;  // this lane's A-operand token
        if constexpr (HOT) {
            const _Float16* kr = P.ring_k + rb + (size_t)(T * TILE + tokA) * D;
#pragma unroll
            for (int kb = 0; kb < Gm::NKB; ++kb) {
                const half8 kk = *reinterpret_cast<const half8*>(kr + kb * 32 + 8 * q4);
                am = mfma16x16x32(kk, qh[kb], am);
            }
        } else {
            const int bit0 = q4 * Gm::QB;
            const uint8_t* rec = kt + tokA * Gm::PB + 4 * (bit0 >> 5);
            uint32_t w[Gm::QW];
#pragma unroll
            for (int i = 0; i < Gm::QW; ++i) w[i] = lds_u32(rec + 4 * i);
            uint32_t al[Gm::QW - 1];
#pragma unroll
            for (int i = 0; i < Gm::QW - 1; ++i) al[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], bit0 & 31);
#pragma unroll
            for (int kb = 0; kb < Gm::NKB; ++kb) {
                union {
                    uint32_t u[4];
                    half8 h;
                } ah, alw;
                if constexpr (Gm::PAIR2) {
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        const uint32_t idx = field(al, (4 * kb + j) * CB, 2 * CB);
                        const uint4 e = *reinterpret_cast<const uint4*>(s_ktab + 16 * idx);
                        ah.u[j] = e.x, ah.u[j + 1] = e.y, alw.u[j] = e.z, alw.u[j + 1] = e.w;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t idx = field(al, (4 * kb + j) * CB, CB);
                        const uint2 e = *reinterpret_cast<const uint2*>(s_ktab + 8 * idx);
                        ah.u[j] = e.x, alw.u[j] = e.y;
                    }
                }
                am = mfma16x16x32(ah.h, qh[kb], am);
                alo = mfma16x16x32(ah.h, ql[kb], alo);
                alo = mfma16x16x32(alw.h, qh[kb], alo);
            }
            const uint8_t* sg = kt + TILE * Gm::PB + tokA * Gm::SB;
#pragma unroll
            for (int sb = 0; sb < Gm::NSB; ++sb) {
                const half8 sig = signs8(s_stab, sg[4 * sb + q4]);
                as = mfma16x16x32(sig, sh[sb], as);
                asl = mfma16x16x32(sig, slo[sb], asl);
            }
        }
        // output rows are tokens 4 q4 + r of the subtile, columns query heads
        const int t0 = st * 16 + 4 * q4;
        if constexpr (HOT) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int phys = T * TILE + t0 + r;
                const bool live = ((phys - mt.head + dm.cap) % dm.cap) < mt.count;
                lg[st][r] = live ? am[r] * isd : -INFINITY;
            }
        } else {
            const uint8_t* km = kt + TILE * (Gm::PB + Gm::SB);
            const uint2 Rr = *reinterpret_cast<const uint2*>(km + 2 * t0);
            const uint2 Pr = *reinterpret_cast<const uint2*>(km + 2 * TILE + 2 * t0);
            const _Float16* Rh = reinterpret_cast<const _Float16*>(&Rr);
            const _Float16* Ph = reinterpret_cast<const _Float16*>(&Pr);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = T * TILE + t0 + r;
                const bool live = slot < mt.cold_len && !((tw >> (t0 + r)) & 1u);
                const float pol = am[r] + alo[r] * INV_LO;
                const float sd = as[r] + asl[r] * INV_LO;
                lg[st][r] = live ? (pol * (float)Rh[r] + cm * (float)Ph[r] * sd) * isd : -INFINITY;
            }
        }
    }
    if (lrow && col < G) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = T * TILE + st * 16 + 4 * q4 + r;
                if constexpr (HOT) {
                    const int fifo = (t - mt.head + dm.cap) % dm.cap;
                    if (fifo < mt.count) lrow[fifo] = lg[st][r];
                } else {
                    if (t < mt.cold_len) lrow[dm.cap + t] = lg[st][r];
                }
            }
    }
    // ----------------------------------------------------------- softmax
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, lg[st][r]);
    mx = rows_max(mx);
    const float mn = fmaxf(m_run, mx);
    const float alpha = (m_run == mn) ? 1.0f : __expf(m_run - mn);
    float p[2][4];
    float ls = 0.0f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[st][r] = lg[st][r] == -INFINITY ? 0.0f : __expf(lg[st][r] - mn);
            ls += p[st][r];
        }
    ls = rows_sum(ls);
    m_run = mn;
    l_run = l_run * alpha + ls;
    // promotion candidates: only a token reaching tau within its tile can
    // reach it over the whole context.  Marked here, written to LDS by
    // cand_collect once the tile's prefetch has landed (an LDS write issued
    // while the DMA is in flight would make the compiler wait for it).
    if (!HOT) {
        cmask = 0u;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                lgc[4 * st + r] = lg[st][r];
                if (p[st][r] > 0.0f && p[st][r] >= dm.tau * ls) cmask |= 1u << (4 * st + r);
            }
    }
    // ------------------------------------------------------------ values
    if (__any(alpha != 1.0f)) {
        // rows 4 q4 + r of the value accumulators belong to head (row % G)
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, (4 * q4 + r) % G, 16);
#pragma unroll
        for (int n = 0; n < Gm::NVT; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) vx[n][r] *= ar[r];
#pragma unroll
        for (int n = 0; n < M / 16; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) vs[n][r] *= ar[r];
    }
    // weights p * R (and p * rho) in this lane's role, then transposed
    float vR[2][4], vP[2][4];
    if constexpr (HOT) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r) vR[st][r] = 1.0f, vP[st][r] = 0.0f;
    } else {
        const uint8_t* vm = vt + TILE * (Gm::PB + Gm::SB);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int t0 = st * 16 + 4 * q4;
            const uint2 Rr = *reinterpret_cast<const uint2*>(vm + 2 * t0);
            const uint2 Pr = *reinterpret_cast<const uint2*>(vm + 2 * TILE + 2 * t0);
            const _Float16* Rh = reinterpret_cast<const _Float16*>(&Rr);
            const _Float16* Ph = reinterpret_cast<const _Float16*>(&Pr);
#pragma unroll
            for (int r = 0; r < 4; ++r) vR[st][r] = (float)Rh[r], vP[st][r] = (float)Ph[r];
        }
    }
    uint32_t wq[2][2], wrq[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            wq[st][h2] = pack2(role_half<G>(p[st][2 * h2] * vR[st][2 * h2], col),
                               role_half<G>(p[st][2 * h2 + 1] * vR[st][2 * h2 + 1], col));
            if constexpr (!HOT)
                wrq[st][h2] = pack2(role_half<G>(p[st][2 * h2] * vP[st][2 * h2], col),
                                    role_half<G>(p[st][2 * h2 + 1] * vP[st][2 * h2 + 1], col));
        }
    const half8 av = tile_transpose(wq[0][0], wq[0][1], wq[1][0], wq[1][1]);
    if constexpr (HOT) {
        const _Float16* vtile = P.ring_v + rb + (size_t)T * D * TILE;
#pragma unroll
        for (int n = 0; n < Gm::NVT; ++n) {
            const half8 vv = *reinterpret_cast<const half8*>(vtile + (size_t)(16 * n + col) * TILE + 8 * q4);
            vx[n] = mfma16x16x32(av, vv, vx[n]);
        }
    } else {
        const half8 avs = tile_transpose(wrq[0][0], wrq[0][1], wrq[1][0], wrq[1][1]);
        const int bit0 = 8 * q4 * CB;
#pragma unroll
        for (int g = 0; g < Gm::NPG; ++g) {
            const uint8_t* pl = vt + (16 * g + col) * 4 * CB + 4 * (bit0 >> 5);
            uint32_t w[Gm::VW];
#pragma unroll
            for (int i = 0; i < Gm::VW; ++i) w[i] = ((bit0 >> 5) + i < CB) ? lds_u32(pl + 4 * i) : 0u;
            uint32_t al[Gm::VW - 1];
#pragma unroll
            for (int i = 0; i < Gm::VW - 1; ++i) al[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], bit0 & 31);
            union {
                uint32_t u[4];
                half8 h;
            } bx, by;
            if constexpr (Gm::PAIR2) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t idx = field(al, 2 * j * CB, 2 * CB);
                    const uint2 e = *reinterpret_cast<const uint2*>(s_vtab + 8 * idx);
                    bx.u[j] = e.x, by.u[j] = e.y;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t e0 = lds_u32(s_vtab + 4 * field(al, 2 * j * CB, CB));
                    const uint32_t e1 = lds_u32(s_vtab + 4 * field(al, (2 * j + 1) * CB, CB));
                    bx.u[j] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
                    by.u[j] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
                }
            }
            vx[2 * g] = mfma16x16x32(av, bx.h, vx[2 * g]);
            vx[2 * g + 1] = mfma16x16x32(av, by.h, vx[2 * g + 1]);
        }
#pragma unroll
        for (int n = 0; n < M / 16; ++n) {
            const uint32_t bits = lds_u32(vt + TILE * Gm::PB + 4 * (16 * n + col));
            vs[n] = mfma16x16x32(avs, signs8(s_stab, (bits >> (8 * q4)) & 0xffu), vs[n]);
        }
    }
}

// Appends tile T's marked candidates (lanes with col < G hold head col) to the
// wave's list, then drops those below tau of the running softmax and keeps
// at most ktop per head.
template <int G>
__device__ __forceinline__ void cand_collect(const Dims& dm, int T, int q4, int col, int lane, const float (&lgc)[8],
                                             uint32_t cmask, float m_run, float l_run, int* ncand, Cand* s_cand) {
    const int ktop = dm.ktop;
    if (__any(cmask != 0u)) {
        if (col < G) {
            for (uint32_t mk = cmask; mk; mk &= mk - 1) {
                const int i = __builtin_ctz(mk);
                const int at = atomicAdd(&ncand[col], 1);
                if (at < 2 * ktop) s_cand[col * 2 * ktop + at] = Cand{lgc[i], T * TILE + (i >> 2) * 16 + 4 * q4 + (i & 3)};
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < G) {
            const int n = min(ncand[lane], 2 * ktop);
            int k2 = 0;
            for (int i = 0; i < n; ++i) {
                const Cand cc = s_cand[lane * 2 * ktop + i];
                if (__expf(cc.v - m_run) >= dm.tau * l_run && k2 < ktop) s_cand[lane * 2 * ktop + k2++] = cc;
            }
            ncand[lane] = k2;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template <int D, int CB, int M, int G>
__global__ __launch_bounds__(256) void k_decode(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs,
                                                const _Float16* __restrict__ qin, int n_hot_chunks, int cold_tiles,
                                                int n_chunks, float* logits, int lstride) {
    using Gm = Geom<D, CB, M>;
    __shared__ __attribute__((aligned(16))) uint8_t s_tab[Gm::TABS];
    __shared__ __attribute__((aligned(16))) uint8_t s_st0[4][2 * Gm::HALF];
    __shared__ __attribute__((aligned(16))) uint8_t s_st1[4][2 * Gm::HALF];
    __shared__ float s_fold[4][16][17];
    __shared__ int s_ncand[4][8];
    extern __shared__ Cand s_cand_all[];  // [4 waves][G][2 * ktop]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q4 = lane >> 4, col = lane & 15;
    const int bi = blockIdx.y, kvh = blockIdx.z;
    const int seq = cs.ids[bi];
    const size_t sl = sl_index(dm, seq, layer);
    const SeqLayerMeta mt = P.meta[sl];
    const int ktop = dm.ktop;
    Cand* s_cand = s_cand_all + (size_t)wave * G * 2 * (ktop > 0 ? ktop : 1);
    const uint8_t* s_ktab = s_tab;
    const uint8_t* s_vtab = s_tab + Gm::KTAB;
    const uint8_t* s_stab = s_tab + Gm::KTAB + Gm::VTAB;

    // tables (whole KB in global memory too): wave w copies KB w, w + 4, ...
    for (int i = wave; i < Gm::TABS / 1024; i += 4)
        stage_copy<1024>(P.tables + F.tab_off + 1024 * i, s_tab + 1024 * i, lane);
    if (lane < 8) s_ncand[wave][lane] = 0;

    const int c = blockIdx.x * 4 + wave;
    const bool active = c < n_chunks;
    const bool hot = c < n_hot_chunks;
    int t_first = 0, t_last = 0;
    if (active && !hot) {
        t_first = (c - n_hot_chunks) * cold_tiles;
        t_last = min(t_first + cold_tiles, (mt.cold_len + TILE - 1) / TILE);
    }
    const uint8_t* kbase = P.cold + cold_tile_offset(dm, F, seq, kvh, 0, 0);
    const uint8_t* vbase = P.cold + cold_tile_offset(dm, F, seq, kvh, 1, 0);
    if (t_first < t_last) {
        stage_copy<Gm::TB>(kbase + (size_t)t_first * Gm::TB, s_st0[wave], lane);
        stage_copy<Gm::TB>(vbase + (size_t)t_first * Gm::TB, s_st0[wave] + Gm::HALF, lane);
    }
    // tombstone words of the chunk's tiles (at most 64 tiles per chunk)
    const uint32_t tomb_all =
        (t_first + lane < t_last) ? P.tomb[sl * (dm.cold_cap / 32) + t_first + lane] : 0u;
    wait_vmem();
    __syncthreads();
    if (!active) return;

    const float isd = 1.0f / sqrtf((float)D);
    const float cm = SQRT_HALF_PI / (float)M;
    const size_t rb = ring_base(dm, seq, layer, kvh);
    const int head = col % G;  // query head of this lane's column
    float* lrow = logits ? logits + ((size_t)bi * dm.hq + kvh * G + head) * lstride : nullptr;

    // query operands (B): k = 8 q4 + r of each block, column = head col % G
    half8 qh[Gm::NKB], ql[Gm::NKB], sh[Gm::NSB], slo[Gm::NSB];
    {
        const float* qp = P.qprep + ((size_t)bi * dm.hq + kvh * G + head) * (D + M_MAX);
        const _Float16* qo = qin + ((size_t)bi * dm.hq + kvh * G + head) * D;
#pragma unroll
        for (int kb = 0; kb < Gm::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                _Float16 hi = (_Float16)0.0f, lo = (_Float16)0.0f;
                if (hot)
                    hi = qo[kb * 32 + 8 * q4 + r];
                else
                    split_hl(qp[kb * 32 + 8 * q4 + r], hi, lo);
                qh[kb][r] = hi;
                ql[kb][r] = lo;
            }
#pragma unroll
        for (int sb = 0; sb < Gm::NSB; ++sb)
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                _Float16 hi = (_Float16)0.0f, lo = (_Float16)0.0f;
                if (!hot) split_hl(qp[D + sb * 32 + 8 * q4 + r], hi, lo);
                sh[sb][r] = hi;
                slo[sb][r] = lo;
            }
    }

    floatx4 vx[Gm::NVT];
    floatx4 vs[M / 16];
#pragma unroll
    for (int n = 0; n < Gm::NVT; ++n) vx[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < M / 16; ++n) vs[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    int* ncand = &s_ncand[wave][0];
    float lgc[8];
    uint32_t cmask = 0u;

    if (hot) {
        tile_body<D, CB, M, G, true>(dm, P, mt, c, nullptr, nullptr, 0u, rb, q4, col, lane, qh, ql, sh, slo, vx, vs,
                                     m_run, l_run, s_ktab, s_vtab, s_stab, lrow, isd, cm, lgc, cmask);
    } else {
        // two stages, each tile's bytes prefetched while the previous tile is computed
        for (int T = t_first; T < t_last; T += 2) {
            if (T + 1 < t_last) {
                stage_copy<Gm::TB>(kbase + (size_t)(T + 1) * Gm::TB, s_st1[wave], lane);
                stage_copy<Gm::TB>(vbase + (size_t)(T + 1) * Gm::TB, s_st1[wave] + Gm::HALF, lane);
            }
            tile_body<D, CB, M, G, false>(dm, P, mt, T, s_st0[wave], s_st0[wave] + Gm::HALF,
                                          __builtin_amdgcn_readlane(tomb_all, T - t_first), rb, q4, col, lane, qh, ql,
                                          sh, slo, vx, vs, m_run, l_run, s_ktab, s_vtab, s_stab, lrow, isd, cm, lgc,
                                          cmask);
            wait_vmem();
            __builtin_amdgcn_wave_barrier();
            if (ktop > 0) cand_collect<G>(dm, T, q4, col, lane, lgc, cmask, m_run, l_run, ncand, s_cand);
            if (T + 1 >= t_last) break;
            if (T + 2 < t_last) {
                stage_copy<Gm::TB>(kbase + (size_t)(T + 2) * Gm::TB, s_st0[wave], lane);
                stage_copy<Gm::TB>(vbase + (size_t)(T + 2) * Gm::TB, s_st0[wave] + Gm::HALF, lane);
            }
            tile_body<D, CB, M, G, false>(dm, P, mt, T + 1, s_st1[wave], s_st1[wave] + Gm::HALF,
                                          __builtin_amdgcn_readlane(tomb_all, T + 1 - t_first), rb, q4, col, lane, qh,
                                          ql, sh, slo, vx, vs, m_run, l_run, s_ktab, s_vtab, s_stab, lrow, isd, cm, lgc,
                                          cmask);
            wait_vmem();
            __builtin_amdgcn_wave_barrier();
            if (ktop > 0) cand_collect<G>(dm, T + 1, q4, col, lane, lgc, cmask, m_run, l_run, ncand, s_cand);
        }
    }

    // ---------------------------------------------------------- partials
    const int stride = part_stride(D);
    float* part0 = P.part + ((size_t)bi * dm.hq + kvh * G) * dm.max_chunks * stride;
    float (*fold)[17] = s_fold[wave];
    for (int n = 0; n < Gm::NVT + M / 16; ++n) {
        const floatx4 v = n < Gm::NVT ? vx[n] : vs[n - Gm::NVT];
#pragma unroll
        for (int r = 0; r < 4; ++r) fold[4 * q4 + r][col] = v[r];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < (G + 3) / 4; ++k) {
            const int h = q4 + 4 * k;
            if (h < G) {
                const float val = fold[h][col] + fold[G + h][col] * INV_LO;
                float* pp = part0 + ((size_t)h * dm.max_chunks + c) * stride;
                int idx;
                if (n >= Gm::NVT)
                    idx = 2 + D + 16 * (n - Gm::NVT) + col;
                else if (hot)
                    idx = 2 + 16 * n + col;
                else
                    idx = 2 + 2 * (16 * (n >> 1) + col) + (n & 1);  // pair 16 g + col, x (even n) or y
                if (!hot || n < Gm::NVT) pp[idx] = val;
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (lane < G) {
        float* pp = part0 + ((size_t)lane * dm.max_chunks + c) * stride;
        pp[0] = m_run;
        pp[1] = l_run;
        if (!hot && ktop > 0) {
            Cand* cc = P.cand_chunk + (((size_t)bi * dm.hq + kvh * G + lane) * dm.max_chunks + c) * ktop;
            const int n = min(ncand[lane], ktop);
            for (int i = 0; i < ktop; ++i) cc[i] = i < n ? s_cand[lane * 2 * ktop + i] : Cand{-INFINITY, -1};
        }
    }
}

// One block per (sequence, query head): chunk weights, then every thread
// sums one accumulator component over the chunks (8 chunks in flight).
template <int D>
__global__ __launch_bounds__(256) void k_combine(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs, int n_hot_chunks,
                                                 int n_chunks, float* __restrict__ out) {
    extern __shared__ float s_w[];  // [n_chunks]
    __shared__ float s_acc[D + M_MAX];
    __shared__ float s_hot[D];
    __shared__ float s_red[8];
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
    if ((tid & 63) == 0) s_red[4 + (tid >> 6)] = ls;
    __syncthreads();
    const float L = (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]);
    const int m = F.m;
    // components: [0, D) rotated cold sums, [D, D + m) sign sums, then hot sums
    for (int j = tid; j < 2 * D + m; j += 256) {
        const bool hotpart = j >= D + m;
        const int comp = hotpart ? j - D - m : j;
        const int c0 = hotpart ? 0 : n_hot_chunks, c1 = hotpart ? n_hot_chunks : n_chunks;
        float acc = 0.0f;
        int c = c0;
        for (; c + 8 <= c1; c += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(c + u) * stride + 2 + comp];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc = fmaf(s_w[c + u], v[u], acc);
        }
        for (; c < c1; ++c) acc = fmaf(s_w[c], part[(size_t)c * stride + 2 + comp], acc);
        if (hotpart)
            s_hot[comp] = acc;
        else
            s_acc[comp] = acc;
    }
    __syncthreads();
    if (tid < D && dm.v_qjl) {
        const float cm = SQRT_HALF_PI / (float)m;
        float t = 0.0f;
        for (int j = 0; j < m; ++j) t = fmaf(P.s32[(size_t)j * D + tid], s_acc[D + j], t);
        s_acc[tid] = fmaf(cm, t, s_acc[tid]);
    }
    __syncthreads();
    if (tid < D) {
        float o = 0.0f;
        for (int k = 0; k < D; ++k) o = fmaf(P.pi32[(size_t)k * D + tid], s_acc[k], o);
        o += s_hot[tid];
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
static hipError_t decode_launch(dim3 grid, int ktop, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F,
                                int layer, const CallSeqs& cs, const _Float16* q, int nh, int ct, int nc, float* logits,
                                int lstride) {
    const size_t shm = (size_t)4 * G * 2 * std::max(ktop, 1) * sizeof(Cand);
    k_decode<D, CB, M, G><<<grid, 256, shm, st>>>(dm, P, F, layer, cs, q, nh, ct, nc, logits, lstride);
    return hipSuccess;
}

template <int D, int CB, int M>
static hipError_t decode_g(dim3 grid, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                           const CallSeqs& cs, const _Float16* q, int nh, int ct, int nc, float* logits, int lstride) {
    switch (dm.g) {
        case 1: return decode_launch<D, CB, M, 1>(grid, dm.ktop, st, dm, P, F, layer, cs, q, nh, ct, nc, logits, lstride);
        case 2: return decode_launch<D, CB, M, 2>(grid, dm.ktop, st, dm, P, F, layer, cs, q, nh, ct, nc, logits, lstride);
        case 4: return decode_launch<D, CB, M, 4>(grid, dm.ktop, st, dm, P, F, layer, cs, q, nh, ct, nc, logits, lstride);
        case 8: return decode_launch<D, CB, M, 8>(grid, dm.ktop, st, dm, P, F, layer, cs, q, nh, ct, nc, logits, lstride);
        default: return hipErrorInvalidValue;
    }
}

template <int D, int CB>
static hipError_t decode_m(dim3 grid, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                           const CallSeqs& cs, const _Float16* q, int nh, int ct, int nc, float* logits, int lstride) {
    if (F.m == 32) return decode_g<D, CB, 32>(grid, st, dm, P, F, layer, cs, q, nh, ct, nc, logits, lstride);
    if (F.m == 64) return decode_g<D, CB, 64>(grid, st, dm, P, F, layer, cs, q, nh, ct, nc, logits, lstride);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                         int cold_bound, const _Float16* q, float* out, float* logits, int logits_stride,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (cs.n == 0) return hipSuccess;
    // hot ring: one 32-slot tile per wave; cold: chunks of whole tiles, sized
    // so that the launch has enough waves to cover the chip
    const int n_hot = dm.cap / TILE;
    const int cold_tiles_total = (cold_bound + TILE - 1) / TILE;
    const int target_waves = 4096;
    int per = std::max(1, target_waves / std::max(1, cs.n * dm.hkv));
    per = std::min(per, MAX_COLD_CHUNKS);
    const int ct = cold_tiles_total > 0 ? (cold_tiles_total + per - 1) / per : 1;
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
    hipError_t e = hipSuccess;
    const int key = dm.d * 10 + F.cb;
    switch (key) {
        case 645: e = decode_m<64, 5>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, n_chunks, logits, logits_stride); break;
        case 647: e = decode_m<64, 7>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, n_chunks, logits, logits_stride); break;
        case 644: e = decode_m<64, 4>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, n_chunks, logits, logits_stride); break;
        case 1285: e = decode_m<128, 5>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, n_chunks, logits, logits_stride); break;
        case 1287: e = decode_m<128, 7>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, n_chunks, logits, logits_stride); break;
        case 1284: e = decode_m<128, 4>(grid, st, dm, P, F, layer, cs, q, n_hot, ct, n_chunks, logits, logits_stride); break;
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
