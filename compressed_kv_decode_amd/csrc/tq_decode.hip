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
//   k_qprep   q' = Pi q and S q' per (sequence, query head), fp32, pre-scaled
//             so that logits come out in log2 units; one block per (sequence,
//             kv head) covers the group's query heads.
//   k_decode  split-context attention.  Every (sequence, kv head) stream is
//             cut into parts of about equal measured cost, one part per
//             resident wave.  A
//             part first scores its hot ring tiles, then its cold tiles, each
//             phase ending in a partial record (max, sum, accumulators).
//             Cold K|V tile pairs stream through a three-stage LDS ring filled
//             by full-wave global-to-LDS DMA.  Per 32-token tile:
//               logits  16x16x32 f16 MFMA, tokens as rows (A: unit pair
//                       values, fp16 hi and lo from a table), query heads as
//                       columns (B: q' hi and lo).  The QJL term contracts
//                       the tokens' signs (+-1) with S q' (hi, lo).
//               softmax online per head in log2 units, rescaled only when a
//                       logit exceeds the running reference (which is then
//                       set a few units above the new maximum).
//               values  16x16x32 f16 MFMA computing O^T = V^T P^T: A = the
//                       unit values of 16 pairs x 8 tokens per lane (value
//                       tiles store tokens in the order the logit output
//                       holds them, so no transposes), B = the weights p * R
//                       straight from the logit layout, column h the fp16 hi
//                       part and column G + h the lo part x 2^12.  The QJL
//                       term contracts +-rho (sign bits XOR-ed into rho) with
//                       the weights p.
//             Cold accumulators stay in the rotated domain.
//   k_combine merges the partial records of each (sequence, query head),
//             adds the QJL back-projection S_m^T, rotates back with Pi^T,
//             normalises, and turns candidate logits into probabilities.
#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "tq_device.h"
#include "tq_qprep_body.h"

namespace tq {

// Workspace of the decode entry point that allocates nothing
// (tq_decode_attention_static): rotated queries, split-context partial
// records and per-part promotion candidates of one launch batch.  One copy
// per GPU, held until the process ends; calls share it, so calls that
// overlap on one GPU race.  Nothing in it needs clearing: every launch writes
// the queries, record headers and candidate slots it reads, and the combine
// skips the accumulators of records without tokens.
static __device__ __align__(256) uint8_t scratch[STATIC_WS_BYTES];

hipError_t static_workspace(void** ptr) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        // the device address of this GPU's copy (the array's name is only a
        // host-side stand-in)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

constexpr float SQRT_HALF_PI = 1.25331413731550025121f;
constexpr float INV_LO = 1.0f / LO_SCALE;
constexpr float LN2 = 0.69314718055994530942f;
constexpr bool KEY_TWO_CODE = false;
constexpr bool VALUE_TWO_CODE = true;
constexpr bool PRELOAD_VALUES = true;
constexpr bool KEY_TWO_CODE_P = false;  // packed layout: two-code key table (b128; LDS bank conflicts)
constexpr int WAVES_PER_SIMD = 2;
constexpr float HEADROOM = 3.0f;  // log2 units kept above the running max after a rescale
constexpr int MAX_PARTS = 256;    // parts per (sequence, kv head) stream
constexpr int PM_CHUNK = 32;      // a stream of more parts is pre-merged 32 parts at a time
// Cost of a hot ring tile and of a cold tile pair in the split-context plan.
// A hot tile (32 fp16 K and V rows: one round trip to memory, light math)
// costs about as much as a cold tile pair once its rows come from HBM rather
// than the last-level cache (measured: a 128k-token F2.5 stream read from
// HBM, 48.4 us at 3 units against 41.5 us at 5; 8 x 32k-token F3 and F4
// streams within 1 us for hot:cold ratios 3:5 to 5:5, and F4 within 1 us
// for 5:5 to 5:7, so one ratio serves every format).
constexpr int HOT_UNITS = 5;
constexpr int COLD_UNITS = 5;
// The two waves of a SIMD come from the first and the second half of the
// grid (two blocks per CU, dispatched in order), and the younger one ends
// later even under the priority toggle of the tile loop.  Items therefore
// alternate between the halves (even items to the first half's waves), and
// a stream's even items take 1 + AGE_SKEW / 1024 of the average part cost,
// its odd items 1 - AGE_SKEW / 1024 (measured on llama8b F3 on two boxes:
// 31 put the launch 0.1 - 1.3 us ahead of equal costs in each of four
// pairs of runs).
constexpr int AGE_SKEW = 31;


__global__ void k_fill(float* p, size_t n, float v) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// Hot-first gate ("Monarch v3", section "Bucle de Decodificacion
// Simplificado": the cold pages are scored only when the best hot score is
// below a threshold).  Block (sequence bi, kv head, slice) of k_qprep scans
// FIFO entries [slice * n, slice * n + n) of the window, n = ceil(cap /
// HOT_SLICES): four threads per entry, each dotting 16-byte pieces of its
// quarter of the key (a wave reads 16 whole rows, contiguous) with the
// group's G queries; the best logit <q, k>/sqrt(d) per head of the slice goes
// to gate_max.  k_decode takes the maximum over the slices and the minimum
// over the heads.
template <int D, int G>
__device__ void hot_slice(const Dims& dm, const Ptrs& P, int layer, int seq, int bi, int kvh, int slice,
                          const _Float16* __restrict__ q) {
    constexpr int QD = D / 4;  // dims of a key quarter
    __shared__ __attribute__((aligned(16))) float s_q[G][D];
    __shared__ float s_red[G][QP_NT / 64];
    const int tid = threadIdx.x;
    const SeqLayerMeta mt = P.meta[sl_index(dm, seq, layer)];
    const _Float16* rk = P.ring_k + ring_base(dm, seq, layer, kvh);
    const int per = (dm.cap + HOT_SLICES - 1) / HOT_SLICES;
    const int e0 = slice * per, e1 = min(mt.count, e0 + per);
    const int qd = tid & 3;  // this thread's key quarter
    for (int e = tid; e < G * D; e += QP_NT) s_q[e / D][e % D] = (float)q[((size_t)bi * dm.hq + kvh * G) * D + e];
    __syncthreads();
    const float isd = 1.0f / sqrtf((float)D);
    float best[G];
#pragma unroll
    for (int h = 0; h < G; ++h) best[h] = -INFINITY;
    for (int eb = e0; eb < e1; eb += QP_NT / 4) {  // every thread of a wave takes the same trips
        const int e = eb + (tid >> 2);
        float acc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = 0.0f;
        if (e < e1) {
            const uint4* src = reinterpret_cast<const uint4*>(rk + (size_t)((mt.head + e) % dm.cap) * D + qd * QD);
            uint4 w[QD / 8];
#pragma unroll
            for (int c = 0; c < QD / 8; ++c) w[c] = src[c];
#pragma unroll
            for (int c = 0; c < QD / 8; ++c) {
                const _Float16* k8 = reinterpret_cast<const _Float16*>(&w[c]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float kv = (float)k8[j];
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h] = fmaf(s_q[h][qd * QD + 8 * c + j], kv, acc[h]);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float v = acc[h];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);  // the entry's four quarters
            if (e < e1) best[h] = fmaxf(best[h], v * isd);
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float b = wave_max(best[h]);
        if ((tid & 63) == 0) s_red[h][tid >> 6] = b;
    }
    __syncthreads();
    if (tid < G) {
        float b = -INFINITY;
        for (int w = 0; w < QP_NT / 64; ++w) b = fmaxf(b, s_red[tid][w]);
        P.gate_max[(((size_t)bi * dm.hkv + kvh) * HOT_SLICES + slice) * MAX_G + tid] = b;
    }
}

// True when (sequence bi, kv head)'s cold slots are skipped: every query head
// of the group has a hot logit >= the gate (wave-uniform).  Lane h * S + s
// holds slice s of head h.
template <int G>
__device__ __forceinline__ bool gate_closed(const Dims& dm, const Ptrs& P, int bi, int kvh, int lane) {
    constexpr int S = HOT_SLICES;
    const int h = lane / S, s = lane % S;
    float v = (h < G) ? P.gate_max[(((size_t)bi * dm.hkv + kvh) * S + s) * MAX_G + h] : INFINITY;
#pragma unroll
    for (int o = 1; o < S; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));  // best over the slices
#pragma unroll
    for (int o = S; o < 64; o <<= 1) v = fminf(v, __shfl_xor(v, o, 64));  // smallest over the heads
    // every lane holds the same value now: take it as a scalar
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))) >= dm.gate;
}

// q' = Pi q and S q' of one block (sequence, kv head), see qprep_body; blocks
// z >= 1 scan the hot window for the hot-first gate.
template <int D, int G>
__global__ __launch_bounds__(QP_NT) void k_qprep(Dims dm, Ptrs P, int layer, CallSeqs cs,
                                                  const _Float16* __restrict__ q, float cm) {
    __shared__ __attribute__((aligned(16))) float s_lds[QprepGeom<D, G>::FLOATS];
    const int bi = blockIdx.x, kvh = blockIdx.y;
    if (blockIdx.z > 0) {  // a hot-window slice of the hot-first gate
        hot_slice<D, G>(dm, P, layer, cs.ids[bi], bi, kvh, blockIdx.z - 1, q);
        return;
    }
    qprep_body<D, G, QP_NT>(dm, P, bi, kvh, q, cm, s_lds);
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

// fp16 bits of two weights in this lane's column role.  wl is the weight
// times the role's scale (1 on hi lanes, 2^12 on lo lanes, applied through
// the exponent offset).  Both roles round the weight itself to fp16 (h); a
// hi lane keeps h, a lo lane the residual wl - 2^12 h (exact in fp32), so
// hi + lo / 2^12 is the weight to fp16 precision of the residual.
// is = 1 / scale; nb = 0 on hi lanes, -2^12 on lo lanes.
struct RoleK {
    float is, nb;
};
// (The two halves are assembled as a vector, so the second is written by
// v_fma_mixhi_f16 into the upper half, with no shift and or.)
__device__ __forceinline__ uint32_t role_pair(float wl0, float wl1, RoleK rk) {
    const _Float16 h0 = (_Float16)(wl0 * rk.is), h1 = (_Float16)(wl1 * rk.is);
    half2v o;
    o.x = (_Float16)fmaf((float)h0, rk.nb, wl0);
    o.y = (_Float16)fmaf((float)h1, rk.nb, wl1);
    return __builtin_bit_cast(uint32_t, o);
}
// a x b for an fp16 b as one mixed-precision fma (v_fma_mix_f32 with a zero
// addend: a single rounding of the product, as a plain multiply)
__device__ __forceinline__ float mul_h(float a, _Float16 b) { return fmaf(a, (float)b, 0.0f); }

template <int D, int CB, int M>
struct Geom {
    static constexpr int PAIRS = D / 2;
    static constexpr int PB = PAIRS * CB / 8;        // pair-code bytes per K record
    static constexpr int SB = M / 8;                 // sign bytes per K record
    static constexpr int TB = TILE * (PB + SB + 4);  // bytes of one K or V tile
    static constexpr int KVB = 2 * TB;               // one staged K|V tile pair
    static constexpr int NI = stage_instrs<KVB>();   // DMA instructions per tile pair
    static constexpr int QB = (D / 8) * CB;          // code bits of one record quarter
    static constexpr int QW = (QB + 31 + 31) / 32;   // dwords covering a quarter at any shift
    static constexpr int NKB = D / 32;               // 32-wide k blocks of a key
    static constexpr int NSB = M / 32;               // 32-wide k blocks of the signs
    static constexpr int NPG = PAIRS / 16;           // groups of 16 pairs (value n-tile pairs)
    static constexpr int NVS = M / 16;               // value sign n-tiles
    static constexpr int VW = (8 * CB + 31 + 31) / 32;  // dwords covering 8 codes of a pair row
    static constexpr bool PAIR2 = CB <= 5;
    static constexpr int NCODE = 1 << CB;
    // Lookup variants: two-code tables halve the lookups but read large tables
    // at random (LDS bank conflicts); one-code tables are conflict-free.
    static constexpr bool K2 = PAIR2 && KEY_TWO_CODE;
    static constexpr bool V2 = PAIR2 && VALUE_TWO_CODE;
    static constexpr int ONE = onetab_off_of(CB);   // one-code tables: key hi, key lo, value
    static constexpr int V2OFF = v2tab_off_of(CB);  // two-code value table: (x, x, y, y) per code pair
    static constexpr int K2OFF = k2tab_off_of(CB);  // two-code key table
    // the staged prefix of the layer's tables
    static constexpr int TABS = kb_round(K2 ? tables_end_of(CB) : (V2 ? K2OFF : V2OFF));
    static_assert(KVB % 256 == 0, "tile pair must be whole 256-byte DMA chunks");
};

// Per-lane state of one wave's decode work.
template <int D, int M>
struct Acc {
    floatx4 vx[D / 16];  // value accumulators O^T: rows dims (hot) or pair components (cold)
    floatx4 vs[M / 16];  // QJL value accumulators: rows sketch index
    float mref;          // running reference (log2 units), same for every lane of a head
    float madj;          // exponent offset of this lane's role (+inf: weight 0)
    float l_run;         // sum of weights over this lane's rows (hi lanes)
};

template <int D, int M>
__device__ __forceinline__ void acc_reset(Acc<D, M>& a) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) a.vx[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < M / 16; ++n) a.vs[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    a.mref = -INFINITY;
    a.madj = INFINITY;
    a.l_run = 0.0f;
}

// Online softmax of one tile's 8 logits per lane (log2 units): rescale when
// any logit exceeds the reference, then p = 2^(l - madj) (hi lanes: the
// weight; lo lanes: the weight x 2^12; zero lanes: 0).
template <int D, int M>
__device__ __forceinline__ void softmax_tile(Acc<D, M>& a, const float (&lg)[2][4], float (&p)[2][4], int role) {
    const float lmax = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                             fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
    if (__any(lmax > a.mref)) {
        const float mx = rows_max(lmax);
        const float mnew = fmaxf(a.mref, mx + HEADROOM);
        if (mnew != a.mref) {
            const float alpha = a.mref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(a.mref - mnew);
#pragma unroll
            for (int n = 0; n < D / 16; ++n) a.vx[n] *= alpha;
#pragma unroll
            for (int n = 0; n < M / 16; ++n) a.vs[n] *= alpha;
            a.l_run *= alpha;
            a.mref = mnew;
            a.madj = role == 2 ? INFINITY : (role == 1 ? mnew - 12.0f : mnew);
        }
    }
    float ls = 0.0f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[st][r] = __builtin_amdgcn_exp2f(lg[st][r] - a.madj);
            ls += p[st][r];
        }
    a.l_run += ls;
}

// Appends tile T's marked candidates (lanes with col < G hold head col) to
// the wave's list, then drops those below tau of the part's running sum (a
// lower bound of the full sum) and keeps at most ktop per head.
template <int G>
__device__ __forceinline__ void cand_collect(const Dims& dm, int T, int q4, int col, int lane, const float (&lgc)[8],
                                             uint32_t cmask, float mref, float l_run, int* ncand, Cand* s_cand) {
    const int ktop = dm.ktop;
    if (__any(cmask != 0u)) {
        if (col < G) {
            for (uint32_t mk = cmask; mk; mk &= mk - 1) {
                const int i = __builtin_ctz(mk);
                const int at = atomicAdd(&ncand[col], 1);
                if (at < 2 * ktop)
                    s_cand[col * 2 * ktop + at] = Cand{lgc[i], T * TILE + (i >> 2) * 16 + 4 * q4 + (i & 3)};
            }
        }
        const float lw = rows_sum(l_run);  // the part's running sum (hi lanes)
        __builtin_amdgcn_wave_barrier();
        if (lane < G) {
            const int n = min(ncand[lane], 2 * ktop);
            int k2 = 0;
            for (int i = 0; i < n; ++i) {
                const Cand cc = s_cand[lane * 2 * ktop + i];
                if (__builtin_amdgcn_exp2f(cc.v - mref) >= dm.tau * lw && k2 < ktop) s_cand[lane * 2 * ktop + k2++] = cc;
            }
            ncand[lane] = k2;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// One staged cold K|V tile pair (kt: K tile in LDS, V tile at kt + TB).
// live: bit t set when slot 32 T + t is live.  Order of work: key MFMAs, then
// every value operand is read from LDS (it does not depend on the softmax,
// so those reads overlap the logit and softmax arithmetic), then the
// softmax, the weights and the value MFMAs.
template <int D, int CB, int M, int G, bool DBG>
__device__ __forceinline__ void cold_tile(const Dims& dm, const uint8_t* kt, int T, uint32_t live, int q4, int col,
                                          int role, const half8 (&qh)[D / 32], const half8 (&ql)[D / 32],
                                          const half8 (&sh)[M / 32], const half8 (&sl)[M / 32], Acc<D, M>& a,
                                          const uint8_t* s_tab, RoleK rk, float* lrow,
                                          float (&lgc)[8], uint32_t& cmask) {
    using Gm = Geom<D, CB, M>;
    typedef union {
        uint32_t u[4];
        half8 h;
    } op8;
    const uint8_t* s_ktab = s_tab + Gm::K2OFF;
    const uint8_t* s_vtab = s_tab + Gm::V2OFF;
    const uint8_t* s_ksg = s_tab;
    const uint8_t* s_vsm = s_tab + SIGN_TAB_BYTES;
    // ---------------------------------------------------------- key MFMAs
    floatx4 am[2], alo[2], as[2], asl[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        am[st] = alo[st] = as[st] = asl[st] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int tokA = st * 16 + col;  // this lane's A-operand token
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
            op8 ah, alw;
            if constexpr (Gm::K2) {
#pragma unroll
                for (int j = 0; j < 4; j += 2) {
                    const uint32_t idx = field(al, (4 * kb + j) * CB, 2 * CB);
                    const uint4 e = *reinterpret_cast<const uint4*>(s_ktab + 16 * idx);
                    ah.u[j] = e.x, ah.u[j + 1] = e.y, alw.u[j] = e.z, alw.u[j + 1] = e.w;
                }
            } else {
                // hi and lo one-code tables (lo follows hi).  The scheduling
                // barrier keeps the two reads apart, so each lands in its own
                // operand (a merged read2 would need moves).
                const uint8_t* th = s_tab + Gm::ONE;
                const uint8_t* tl = th + 4 * Gm::NCODE;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t idx = field(al, (4 * kb + j) * CB, CB);
                    ah.u[j] = lds_u32(th + 4 * idx);
                    __builtin_amdgcn_sched_barrier(0x7FF);
                    alw.u[j] = lds_u32(tl + 4 * idx);
                }
            }
            am[st] = mfma16x16x32(ah.h, qh[kb], am[st]);
            alo[st] = mfma16x16x32(ah.h, ql[kb], alo[st]);
            alo[st] = mfma16x16x32(alw.h, qh[kb], alo[st]);
        }
        const uint8_t* sg = kt + TILE * Gm::PB + tokA * Gm::SB;
#pragma unroll
        for (int sb = 0; sb < Gm::NSB; ++sb) {
            const half8 sig = signs8(s_ksg, sg[4 * sb + q4]);
            as[st] = mfma16x16x32(sig, sh[sb], as[st]);
            asl[st] = mfma16x16x32(sig, sl[sb], asl[st]);
        }
    }
    // ------------------------------------------------ value operands (LDS)
    const uint8_t* vt = kt + Gm::TB;
    const uint8_t* vm = vt + TILE * (Gm::PB + Gm::SB);
    op8 ax[Gm::NPG], ay[Gm::NPG], asg[Gm::NVS];
    // QJL value operands +-rho of storage positions 8 q4 .. (read early only
    // while registers allow: m = 32)
    constexpr bool PRE_SIGN = M <= 32;
    auto load_sign_ops = [&](op8 (&o)[Gm::NVS]) {
        const uint4 rho8 = *reinterpret_cast<const uint4*>(vm + 2 * TILE + 16 * q4);
#pragma unroll
        for (int n = 0; n < Gm::NVS; ++n) {
            const uint32_t byte = (lds_u32(vt + TILE * Gm::PB + 4 * (16 * n + col)) >> (8 * q4)) & 0xffu;
            const uint2 m0 = *reinterpret_cast<const uint2*>(s_vsm + 8 * (byte & 15u));
            const uint2 m1 = *reinterpret_cast<const uint2*>(s_vsm + 8 * (byte >> 4));
            o[n].u[0] = rho8.x ^ m0.x, o[n].u[1] = rho8.y ^ m0.y;
            o[n].u[2] = rho8.z ^ m1.x, o[n].u[3] = rho8.w ^ m1.y;
        }
    };
    auto load_value_ops = [&]() {
        const int bit0 = 8 * q4 * CB;
#pragma unroll
        for (int g = 0; g < Gm::NPG; ++g) {
            const uint8_t* pl = vt + (16 * g + col) * 4 * CB + 4 * (bit0 >> 5);
            uint32_t w[Gm::VW];
#pragma unroll
            for (int i = 0; i < Gm::VW; ++i) w[i] = lds_u32(pl + 4 * i);
            uint32_t al[Gm::VW - 1];
#pragma unroll
            for (int i = 0; i < Gm::VW - 1; ++i) al[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], bit0 & 31);
            if constexpr (Gm::V2) {
                // two-code (x, x, y, y) entries: one 8-byte read per two tokens
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint2 e = *reinterpret_cast<const uint2*>(s_vtab + 8 * field(al, 2 * j * CB, 2 * CB));
                    ax[g].u[j] = e.x;
                    ay[g].u[j] = e.y;
                }
            } else {
                const uint8_t* t1 = s_tab + Gm::ONE + 8 * Gm::NCODE;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t e0 = lds_u32(t1 + 4 * field(al, 2 * j * CB, CB));
                    const uint32_t e1 = lds_u32(t1 + 4 * field(al, (2 * j + 1) * CB, CB));
                    ax[g].u[j] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
                    ay[g].u[j] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
                }
            }
        }
        if constexpr (PRE_SIGN) load_sign_ops(asg);
    };
    if constexpr (PRELOAD_VALUES) load_value_ops();
    uint2 Rv[2];  // value R of this lane's tokens 16 st + 4 q4 + r
#pragma unroll
    for (int st = 0; st < 2; ++st) Rv[st] = *reinterpret_cast<const uint2*>(vm + 2 * (st * 16 + 4 * q4));
    // ------------------------------------------------------------ logits
    float lg[2][4];
    const uint8_t* km = kt + TILE * (Gm::PB + Gm::SB);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        // rows: tokens 16 st + 4 q4 + r; columns: query heads (col % G)
        const int t0 = st * 16 + 4 * q4;
        const uint2 Rr = *reinterpret_cast<const uint2*>(km + 2 * t0);
        const uint2 Pr = *reinterpret_cast<const uint2*>(km + 2 * TILE + 2 * t0);
        const _Float16* Rh = reinterpret_cast<const _Float16*>(&Rr);
        const _Float16* Ph = reinterpret_cast<const _Float16*>(&Pr);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pol = am[st][r] + alo[st][r] * INV_LO;
            const float sd = as[st][r] + asl[st][r] * INV_LO;
            lg[st][r] = fmaf(sd, (float)Ph[r], mul_h(pol, Rh[r]));
        }
    }
    if (live != 0xFFFFFFFFu) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (!((live >> (st * 16 + 4 * q4 + r)) & 1u)) lg[st][r] = -INFINITY;
    }
    if constexpr (DBG) {
        if (col < G) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = st * 16 + 4 * q4 + r;
                    if ((live >> t) & 1u) lrow[dm.cap + T * TILE + t] = lg[st][r] * LN2;
                }
        }
    }
    // ----------------------------------------------------------- softmax
    float p[2][4];
    softmax_tile(a, lg, p, role);
    // promotion candidates: p >= tau times this lane's running sum is
    // necessary for p >= tau times the full sum
    // promotion candidates: p >= tau times the part's running sum (a lower
    // bound of the full sum; at most 1 / tau tokens pass one test); the
    // lane's own sum, smaller still, screens first
    cmask = 0u;
    if (dm.ktop > 0) {
        const float pm = fmaxf(fmaxf(fmaxf(p[0][0], p[0][1]), fmaxf(p[0][2], p[0][3])),
                               fmaxf(fmaxf(p[1][0], p[1][1]), fmaxf(p[1][2], p[1][3])));
        if (__any(role == 0 && pm > 0.0f && pm >= dm.tau * a.l_run)) {
            const float thr = dm.tau * rows_sum(a.l_run);
            if (role == 0) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        lgc[4 * st + r] = lg[st][r];
                        if (p[st][r] > 0.0f && p[st][r] >= thr) cmask |= 1u << (4 * st + r);
                    }
            }
        }
    }
    // ------------------------------------------------------------ values
    if constexpr (!PRELOAD_VALUES) load_value_ops();
    op8 bw, bp;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const _Float16* Rh = reinterpret_cast<const _Float16*>(&Rv[st]);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const float w0 = mul_h(p[st][2 * h2], Rh[2 * h2]);
            const float w1 = mul_h(p[st][2 * h2 + 1], Rh[2 * h2 + 1]);
            bw.u[2 * st + h2] = role_pair(w0, w1, rk);
            bp.u[2 * st + h2] = role_pair(p[st][2 * h2], p[st][2 * h2 + 1], rk);
        }
    }
#pragma unroll
    for (int g = 0; g < Gm::NPG; ++g) {
        a.vx[2 * g] = mfma16x16x32(ax[g].h, bw.h, a.vx[2 * g]);
        a.vx[2 * g + 1] = mfma16x16x32(ay[g].h, bw.h, a.vx[2 * g + 1]);
    }
    if (dm.v_qjl) {
        if constexpr (!PRE_SIGN) load_sign_ops(asg);
#pragma unroll
        for (int n = 0; n < Gm::NVS; ++n) a.vs[n] = mfma16x16x32(asg[n].h, bp.h, a.vs[n]);
    }
}

// ------------------------------------------------------------------------
// Packed tile layout, for at most 4 query heads per kv head.
//
// Key MFMAs take the fp16 hi and lo parts of a code's unit values in one
// A operand, and the columns of B choose what they contract: lane column
// c, role column r = c % 8:
//   r <  G      main  (head r):      hi . q'hi
//   G <= r < 2G cross (head r - G):  hi . q'lo + lo . q'hi   (all x 2^12)
//   otherwise   zero
// so one MFMA yields both parts of the logit, in columns r and r + G.  The
// sign MFMA does the same with S q' hi / lo.  Each 16-token half of the tile
// has its own accumulator; lanes of columns 0..7 then keep the first
// half's, lanes 8..15 the second half's, so every lane finishes four logits
// (not eight) and the softmax, weights and candidates cost half.
// Value MFMAs: B column c < 8 holds the weights p R (role r: hi, lo x 2^12),
// column 8 + r the QJL weights p, so one B operand serves the value and the
// QJL-value accumulation (value columns 8.., QJL columns ..7 are unused).
// ------------------------------------------------------------------------

constexpr int dpp_quad(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int dpp_ror(int n) { return 0x120 + n; }

template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xF, BANKS, false));
}
// full-row lane permutations (every lane has a source): no old value, so
// the compiler can fold the move into the instruction that uses it
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_m(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// value of lane c + G (main lanes read their cross partner)
template <int G>
__device__ __forceinline__ float from_cross(float v) {
    constexpr int C = G == 4 ? dpp_ror(12) : (G == 2 ? dpp_quad(2, 3, 2, 3) : dpp_quad(1, 1, 3, 3));
    return dpp_m<C>(v);
}
// cross lanes take their main partner's value (lane c - G); others keep v
template <int G>
__device__ __forceinline__ float to_cross(float v) {
    if constexpr (G == 4) return dpp_f<dpp_ror(4), 0xA>(v, v);
    else return dpp_f<G == 2 ? dpp_quad(0, 1, 0, 1) : dpp_quad(0, 0, 2, 3), 0xF>(v, v);
}
// value of lane c ^ 8 (the other token half)
__device__ __forceinline__ float other_half(float v) { return dpp_m<dpp_ror(8)>(v); }

template <int D, int CB, int M>
struct PGeom {
    using Gm = Geom<D, CB, M>;
    static constexpr int NMI = D / 16;      // key MFMAs per 16-token half (two codes per lane each)
    static constexpr bool KT2 = KEY_TWO_CODE_P && CB <= 5;  // two-code key table (b128) or one-code (hi, lo) pairs (b64)
    static constexpr int KOFF = KT2 ? k2tab_off_of(CB) : khl_off_of(CB);
    // the staged prefix of the layer's tables
    static constexpr int TABS = kb_round(KT2 ? tables_end_of(CB) : (Gm::V2 ? k2tab_off_of(CB) : v2tab_off_of(CB)));
};

// B operands of the packed key MFMAs for this lane's column role (0 main,
// 1 cross, 2 zero), from the [hi x4 | lo x4] blocks of the rotated query q'
// and of S q' (log2 units).  Key MFMA mi covers, for lane quarter q4, the pairs of dims d0 .. d0 + 3,
// d0 = 32 (mi / 2) + 8 q4 + 4 (mi % 2) (record positions 2 mi, 2 mi + 1 of
// the quarter); A holds hi(c0), hi(c1), lo(c0), lo(c1) (two-code table) or
// hi(c0), lo(c0), hi(c1), lo(c1) (one-code pairs).
union Op8 {
    uint32_t u[4];
    half8 h;
    uint4 q;
    uint2 d[2];
};

template <int D, int CB, int M>
struct QBlocks {  // the [hi x4 | lo x4] blocks a lane's B operands are made of
    Op8 blk[PGeom<D, CB, M>::NMI], sb2[M / 32][2];
};
template <int D, int CB, int M>
__device__ __forceinline__ void packed_b_load(const uint8_t* qb, int q4, QBlocks<D, CB, M>& r) {
    using PG = PGeom<D, CB, M>;
#pragma unroll
    for (int mi = 0; mi < PG::NMI; ++mi)
        r.blk[mi].q = *reinterpret_cast<const uint4*>(qb + 16 * (8 * (mi >> 1) + 2 * q4 + (mi & 1)));
#pragma unroll
    for (int sb = 0; sb < M / 32; ++sb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            r.sb2[sb][j].q = *reinterpret_cast<const uint4*>(qb + 4 * D + 16 * (8 * sb + 2 * q4 + j));
}
template <int D, int CB, int M>
__device__ __forceinline__ void packed_b(const QBlocks<D, CB, M>& r, int prole, half8 (&bk)[D / 16],
                                         half8 (&bs)[M / 32]) {
    using PG = PGeom<D, CB, M>;
#pragma unroll
    for (int mi = 0; mi < PG::NMI; ++mi) {
        const uint32_t h01 = r.blk[mi].u[0], h23 = r.blk[mi].u[1], l01 = r.blk[mi].u[2], l23 = r.blk[mi].u[3];
        Op8 o;
        if (prole == 0) {
            if constexpr (PG::KT2) o.u[0] = h01, o.u[1] = h23, o.u[2] = 0u, o.u[3] = 0u;
            else o.u[0] = h01, o.u[1] = 0u, o.u[2] = h23, o.u[3] = 0u;
        } else if (prole == 1) {
            if constexpr (PG::KT2) o.u[0] = l01, o.u[1] = l23, o.u[2] = h01, o.u[3] = h23;
            else o.u[0] = l01, o.u[1] = h01, o.u[2] = l23, o.u[3] = h23;
        } else {
            o.u[0] = o.u[1] = o.u[2] = o.u[3] = 0u;
        }
        bk[mi] = o.h;
    }
#pragma unroll
    for (int sb = 0; sb < M / 32; ++sb) {
        Op8 o;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            o.u[2 * j] = prole == 0 ? r.sb2[sb][j].u[0] : (prole == 1 ? r.sb2[sb][j].u[2] : 0u);
            o.u[2 * j + 1] = prole == 0 ? r.sb2[sb][j].u[1] : (prole == 1 ? r.sb2[sb][j].u[3] : 0u);
        }
        bs[sb] = o.h;
    }
}

// Online softmax of a lane's four logits (log2 units); see softmax_tile.
// Both token halves of a head share the reference (max over rows and the
// column c ^ 8).
template <int D, int M>
__device__ __forceinline__ void softmax4(Acc<D, M>& a, const float (&lg)[4], float (&p)[4], int prole) {
    const float lmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (__any(lmax > a.mref)) {
        float mx = rows_max(lmax);
        mx = fmaxf(mx, other_half(mx));
        const float mnew = fmaxf(a.mref, mx + HEADROOM);
        if (mnew != a.mref) {
            const float alpha = a.mref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(a.mref - mnew);
            // (the packed layout's value sums use the first D / 32 accumulators)
#pragma unroll
            for (int n = 0; n < D / 32; ++n) a.vx[n] *= alpha;
#pragma unroll
            for (int n = 0; n < M / 16; ++n) a.vs[n] *= alpha;
            a.l_run *= alpha;
            a.mref = mnew;
            a.madj = prole == 2 ? INFINITY : (prole == 1 ? mnew - 12.0f : mnew);
        }
    }
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(lg[r] - a.madj);
        ls += p[r];
    }
    a.l_run += ls;
}

// Key-side registers of one staged tile pair in the packed layout, filled
// one pipeline step ahead of the tile's finish.
template <int D, int CB, int M>
struct PTile {
    floatx4 kac[2], sac[2];  // key / sign MFMA sums per token half
    uint2 Rr, Pr;            // fp16 key R and rho of this lane's tokens
};
// Value-side registers (read from the stage at the start of the tile's step).
// The value operand of pair group g and token half h holds, for the lane's
// row (pair 16 g + col) and its tokens t0..t3 = 16 h + 4 q4 + 0..3, the k
// slots x(t0) x(t1) y(t0) y(t1) x(t2) x(t3) y(t2) y(t3): two table entries
// as read, no register moves.  The weight operand puts the x slots in
// columns < 8 and the y slots in columns >= 8, so one MFMA yields both
// components of 16 pairs over 16 tokens.
template <int D, int CB, int M>
struct PVals {
    using Gm = Geom<D, CB, M>;
    Op8 av[Gm::NPG][2], asg[Gm::NVS];  // value operands
    uint2 Rv;                          // fp16 value R of this lane's tokens
};

// Key code words and sign bytes of both token halves (one LDS round trip).
template <int D, int CB, int M>
struct PKeyWords {
    using Gm = Geom<D, CB, M>;
    uint32_t al[2][Gm::QW - 1];
    uint32_t sgb[2][Gm::NSB];
};
template <int D, int CB, int M>
__device__ __forceinline__ void pk_words(const uint8_t* kt, int q4, int col, PKeyWords<D, CB, M>& kw) {
    using Gm = Geom<D, CB, M>;
    // every word is requested before the first is used
    const int bit0 = q4 * Gm::QB;
    uint32_t w[2][Gm::QW];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int tokA = st * 16 + col;  // this lane's A-operand token
        const uint8_t* rec = kt + tokA * Gm::PB + 4 * (bit0 >> 5);
#pragma unroll
        for (int i = 0; i < Gm::QW; ++i) w[st][i] = lds_u32(rec + 4 * i);
        const uint8_t* sg = kt + TILE * Gm::PB + tokA * Gm::SB;
#pragma unroll
        for (int sb = 0; sb < Gm::NSB; ++sb) kw.sgb[st][sb] = sg[4 * sb + q4];
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < Gm::QW - 1; ++i) kw.al[st][i] = __builtin_amdgcn_alignbit(w[st][i + 1], w[st][i], bit0 & 31);
}

// Key A operands of one token half: unit-value table reads and sign nibbles.
template <int D, int CB, int M>
struct PKeyOps {
    using Gm = Geom<D, CB, M>;
    Op8 av[PGeom<D, CB, M>::NMI];
    half8 sig[Gm::NSB];
};
template <int D, int CB, int M>
__device__ __forceinline__ void pk_key_reads(const uint8_t* s_tab, const PKeyWords<D, CB, M>& kw, int st,
                                             PKeyOps<D, CB, M>& ko) {
    using Gm = Geom<D, CB, M>;
    using PG = PGeom<D, CB, M>;
    const uint8_t* s_key = s_tab + PG::KOFF;
#pragma unroll
    for (int mi = 0; mi < PG::NMI; ++mi) {
        if constexpr (PG::KT2) {
            ko.av[mi].q = *reinterpret_cast<const uint4*>(s_key + 16 * field(kw.al[st], 2 * mi * CB, 2 * CB));
        } else {
            ko.av[mi].d[0] = *reinterpret_cast<const uint2*>(s_key + 8 * field(kw.al[st], 2 * mi * CB, CB));
            ko.av[mi].d[1] = *reinterpret_cast<const uint2*>(s_key + 8 * field(kw.al[st], (2 * mi + 1) * CB, CB));
        }
    }
#pragma unroll
    for (int sb = 0; sb < Gm::NSB; ++sb) ko.sig[sb] = signs8(s_tab, kw.sgb[st][sb]);
}
template <int D, int CB, int M>
__device__ __forceinline__ void pk_key_mfmas(const PKeyOps<D, CB, M>& ko, const half8 (&bk)[D / 16],
                                             const half8 (&bs)[M / 32], floatx4& kac, floatx4& sac) {
    using Gm = Geom<D, CB, M>;
    kac = sac = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mi = 0; mi < PGeom<D, CB, M>::NMI; ++mi) kac = mfma16x16x32(ko.av[mi].h, bk[mi], kac);
#pragma unroll
    for (int sb = 0; sb < Gm::NSB; ++sb) sac = mfma16x16x32(ko.sig[sb], bs[sb], sac);
}

// Value operands and token metadata of a staged tile pair.
template <int D, int CB, int M>
__device__ __forceinline__ void pk_meta(const uint8_t* kt, int q4, int half, PTile<D, CB, M>& t) {
    using Gm = Geom<D, CB, M>;
    const int t0 = 16 * half + 4 * q4;
    const uint8_t* km = kt + TILE * (Gm::PB + Gm::SB);
    t.Rr = *reinterpret_cast<const uint2*>(km + 2 * t0);
    t.Pr = *reinterpret_cast<const uint2*>(km + 2 * TILE + 2 * t0);
}
// The value side's words of a staged tile pair: code words of the lane's
// pair rows, QJL sign words, rho and R.  They are requested together with
// the key words, so that the table reads of pk_values wait for no LDS read
// issued after them (LDS reads complete in order).
template <int D, int CB, int M>
struct PVWords {
    using Gm = Geom<D, CB, M>;
    uint32_t w[Gm::NPG][Gm::VW], sw[Gm::NVS];
    uint4 rho8;
    uint2 Rv;
};
template <int D, int CB, int M>
__device__ __forceinline__ void pk_vwords(const uint8_t* kt, int q4, int col, int half, PVWords<D, CB, M>& vw) {
    using Gm = Geom<D, CB, M>;
    const uint8_t* vt = kt + Gm::TB;
    const uint8_t* vm = vt + TILE * (Gm::PB + Gm::SB);
    const int bit0 = 8 * q4 * CB;
#pragma unroll
    for (int g = 0; g < Gm::NPG; ++g) {
        const uint8_t* pl = vt + (16 * g + col) * 4 * CB + 4 * (bit0 >> 5);
#pragma unroll
        for (int i = 0; i < Gm::VW; ++i) vw.w[g][i] = lds_u32(pl + 4 * i);
    }
#pragma unroll
    for (int n = 0; n < Gm::NVS; ++n) vw.sw[n] = lds_u32(vt + TILE * Gm::PB + 4 * (16 * n + col));
    // QJL value operands +-rho of storage positions 8 q4 ..
    vw.rho8 = *reinterpret_cast<const uint4*>(vm + 2 * TILE + 16 * q4);
    // value R of this lane's tokens 16 half + 4 q4 + r
    vw.Rv = *reinterpret_cast<const uint2*>(vm + 2 * (16 * half + 4 * q4));
}
template <int D, int CB, int M>
__device__ __forceinline__ void pk_values(const PVWords<D, CB, M>& vw, const uint8_t* s_tab, int q4,
                                          PVals<D, CB, M>& t) {
    using Gm = Geom<D, CB, M>;
    const uint8_t* s_vsm = s_tab + SIGN_TAB_BYTES;
    const int bit0 = 8 * q4 * CB;
#pragma unroll
    for (int g = 0; g < Gm::NPG; ++g) {
        uint32_t al[Gm::VW - 1];
#pragma unroll
        for (int i = 0; i < Gm::VW - 1; ++i) al[i] = __builtin_amdgcn_alignbit(vw.w[g][i + 1], vw.w[g][i], bit0 & 31);
        if constexpr (Gm::V2) {
            // two-code (x, x, y, y) entries: one 8-byte read per two tokens
            const uint8_t* txy = s_tab + Gm::V2OFF;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                t.av[g][j >> 1].d[j & 1] = *reinterpret_cast<const uint2*>(txy + 8 * field(al, 2 * j * CB, 2 * CB));
        } else {
            const uint8_t* t1 = s_tab + Gm::ONE + 8 * Gm::NCODE;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t e0 = lds_u32(t1 + 4 * field(al, 2 * j * CB, CB));
                const uint32_t e1 = lds_u32(t1 + 4 * field(al, (2 * j + 1) * CB, CB));
                t.av[g][j >> 1].u[2 * (j & 1)] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
                t.av[g][j >> 1].u[2 * (j & 1) + 1] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
            }
        }
    }
#pragma unroll
    for (int n = 0; n < Gm::NVS; ++n) {
        const uint32_t byte = (vw.sw[n] >> (8 * q4)) & 0xffu;
        const uint2 m0 = *reinterpret_cast<const uint2*>(s_vsm + 8 * (byte & 15u));
        const uint2 m1 = *reinterpret_cast<const uint2*>(s_vsm + 8 * (byte >> 4));
        t.asg[n].u[0] = vw.rho8.x ^ m0.x, t.asg[n].u[1] = vw.rho8.y ^ m0.y;
        t.asg[n].u[2] = vw.rho8.z ^ m1.x, t.asg[n].u[3] = vw.rho8.w ^ m1.y;
    }
    t.Rv = vw.Rv;
}

// Logits, softmax, promotion candidates, weights and value MFMAs of tile T
// from its registers.  half = lane column / 8: this lane's logits are of
// tokens 16 half + 4 q4 + r.
template <int D, int CB, int M, int G, bool DBG>
__device__ __forceinline__ void pk_finish(const Dims& dm, const PTile<D, CB, M>& t, const PVals<D, CB, M>& v,
                                          int T, uint32_t live, int q4,
                                          int half, int prole, RoleK rk, Acc<D, M>& a, float* lrow, float (&lgc)[4],
                                          uint32_t& cmask) {
    using Gm = Geom<D, CB, M>;
    const int t0 = 16 * half + 4 * q4;
    // ------------------------------------------------------------ logits
    float lg[4];
    {
        const _Float16* Rh = reinterpret_cast<const _Float16*>(&t.Rr);
        const _Float16* Ph = reinterpret_cast<const _Float16*>(&t.Pr);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float kx = half ? t.kac[1][r] : t.kac[0][r];
            const float sx = half ? t.sac[1][r] : t.sac[0][r];
            const float x = fmaf(sx, (float)Ph[r], mul_h(kx, Rh[r]));
            // main lanes: hi part + cross part / 2^12; cross lanes copy it
            lg[r] = to_cross<G>(fmaf(from_cross<G>(x), INV_LO, x));
        }
    }
    if (live != 0xFFFFFFFFu) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (!((live >> (t0 + r)) & 1u)) lg[r] = -INFINITY;
    }
    if constexpr (DBG) {
        if (prole == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if ((live >> (t0 + r)) & 1u) lrow[dm.cap + T * TILE + t0 + r] = lg[r] * LN2;
        }
    }
    // ----------------------------------------------------------- softmax
    float p[4];
    softmax4(a, lg, p, prole);
    // promotion candidates: p >= tau times the part's running sum (a lower
    // bound of the full sum, so no candidate is missed, and at most 1 / tau
    // tokens pass one test); the lane's own sum, smaller still, screens first
    cmask = 0u;
    if (dm.ktop > 0) {
        const float pm = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
        if (__any(prole == 0 && pm > 0.0f && pm >= dm.tau * a.l_run)) {
            float lw = rows_sum(a.l_run);
            const float thr = dm.tau * (lw + other_half(lw));
            if (prole == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lgc[r] = lg[r];
                    if (p[r] > 0.0f && p[r] >= thr) cmask |= 1u << r;
                }
            }
        }
    }
    // ------------------------------------------------------------ values
    // own weights (hi or lo role): value weights p R and QJL weights p
    const _Float16* Rvh = reinterpret_cast<const _Float16*>(&v.Rv);
    uint32_t bw[2], bq[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        bw[h2] = role_pair(mul_h(p[2 * h2], Rvh[2 * h2]), mul_h(p[2 * h2 + 1], Rvh[2 * h2 + 1]), rk);
        bq[h2] = role_pair(p[2 * h2], p[2 * h2 + 1], rk);
    }
    // The weights of the other token half come from lane c ^ 8.  Value
    // operand of token half h: columns < 8 take the weights in the x slots,
    // columns >= 8 in the y slots (zero elsewhere).  QJL operand: storage
    // positions 8 q4 .. 8 q4 + 7, i.e. the lane's tokens of half 0, then of
    // half 1 (every column; columns >= 8 repeat columns < 8).
    uint32_t rw[2], rq[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        rw[h2] = dpp_u<dpp_ror(8)>(bw[h2]);
        rq[h2] = dpp_u<dpp_ror(8)>(bq[h2]);
    }
    Op8 B0, B1, BQ;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        B0.u[2 * h2] = half ? 0u : bw[h2];
        B0.u[2 * h2 + 1] = half ? rw[h2] : 0u;
        B1.u[2 * h2] = half ? 0u : rw[h2];
        B1.u[2 * h2 + 1] = half ? bw[h2] : 0u;
        BQ.u[h2] = half ? rq[h2] : bq[h2];
        BQ.u[2 + h2] = half ? bq[h2] : rq[h2];
    }
#pragma unroll
    for (int g = 0; g < Gm::NPG; ++g) a.vx[g] = mfma16x16x32(v.av[g][0].h, B0.h, a.vx[g]);
#pragma unroll
    for (int g = 0; g < Gm::NPG; ++g) a.vx[g] = mfma16x16x32(v.av[g][1].h, B1.h, a.vx[g]);
    if (dm.v_qjl) {
#pragma unroll
        for (int n = 0; n < Gm::NVS; ++n) a.vs[n] = mfma16x16x32(v.asg[n].h, BQ.h, a.vs[n]);
    }
}

// One hot ring tile T (fp16 K rows, V^T tiles in value storage order).
template <int D, int M, int G, bool DBG>
__device__ __forceinline__ void hot_tile(const Dims& dm, const Ptrs& P, const SeqLayerMeta& mt, size_t rb, int T,
                                         int q4, int col, int role, RoleK rk, const half8 (&qh)[D / 32],
                                         Acc<D, M>& a, float* lrow) {
    const float isd = LOG2E / sqrtf((float)D);
    // hot entries this column's query sees: all of them in a decode step; in
    // multi-query attention (mq_n > 0) the chunk's own newest mq_n entries
    // only up to the query's token j
    int lim = mt.count;
    if (dm.mq_n > 0) {
        const int j = min((dm.mq_v0 + col % G) / dm.mq_g, dm.mq_n - 1);
        lim = mt.count - dm.mq_n + j + 1;
    }
    // every load of the tile first (one round trip to memory per tile)
    half8 kk[2][D / 32], vv[D / 16];
    const _Float16* vtile = P.ring_v + rb + (size_t)T * D * TILE;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const _Float16* kr = P.ring_k + rb + (size_t)(T * TILE + st * 16 + col) * D;
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) kk[st][kb] = *reinterpret_cast<const half8*>(kr + kb * 32 + 8 * q4);
    }
#pragma unroll
    for (int n = 0; n < D / 16; ++n) vv[n] = *reinterpret_cast<const half8*>(vtile + (size_t)(16 * n + col) * TILE + 8 * q4);
    float lg[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        floatx4 am = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) am = mfma16x16x32(kk[st][kb], qh[kb], am);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int phys = T * TILE + st * 16 + 4 * q4 + r;
            const int fifo = (phys - mt.head + dm.cap) % dm.cap;
            lg[st][r] = fifo < lim ? am[r] * isd : -INFINITY;
            if constexpr (DBG)
                if (col < G && fifo < mt.count) lrow[fifo] = lg[st][r] * LN2;
        }
    }
    float p[2][4];
    softmax_tile(a, lg, p, role);
    union {
        uint32_t u[4];
        half8 h;
    } bp;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            bp.u[2 * st + h2] = role_pair(p[st][2 * h2], p[st][2 * h2 + 1], rk);
#pragma unroll
    for (int n = 0; n < D / 16; ++n) a.vx[n] = mfma16x16x32(vv[n], bp.h, a.vx[n]);
}

// Writes one partial record for the G heads of a wave: header (reference,
// sum) and the accumulators folded hi + lo / 2^12.  cold: rows are pair
// components (n-tile 2g + c, row i -> pair 16 g + i, component c).
template <int D, int M, int G>
__device__ __forceinline__ void write_record(float* rec0, int stride, Acc<D, M>& a, bool cold, int q4, int col,
                                             bool qjl) {
    const float l = rows_sum(a.l_run);
    if (q4 == 0 && col < G) {
        float* rec = rec0 + (size_t)col * stride;
        rec[0] = a.mref;
        rec[1] = l;
    }
    if (__all(a.mref == -INFINITY)) return;  // no live token: the header says so
    float* rec = rec0 + (size_t)(col % G) * stride;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = a.vx[n][r] + __shfl_xor(a.vx[n][r], G, 16) * INV_LO;
        if (col < G) {
            if (!cold) {
                *reinterpret_cast<float4*>(rec + 2 + 16 * n + 4 * q4) = float4{o[0], o[1], o[2], o[3]};
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) rec[2 + 2 * (16 * (n >> 1) + 4 * q4 + r) + (n & 1)] = o[r];
            }
        }
    }
    if (cold && qjl) {
#pragma unroll
        for (int n = 0; n < M / 16; ++n) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = a.vs[n][r] + __shfl_xor(a.vs[n][r], G, 16) * INV_LO;
            if (col < G) *reinterpret_cast<float4*>(rec + 2 + D + 16 * n + 4 * q4) = float4{o[0], o[1], o[2], o[3]};
        }
    }
}

// Cold partial record of the packed layout: the sum adds both token halves;
// value accumulator g holds rows (pairs) 16 g + 4 q4 + r, x in columns < 8
// and y in columns >= 8; both fold columns c and c + G (c % 8 < G), QJL
// accumulators columns 8 + c and 8 + c + G.
template <int D, int M, int G>
__device__ __forceinline__ void write_record_p(float* rec0, int stride, Acc<D, M>& a, int q4, int col, bool qjl) {
    float l = rows_sum(a.l_run);
    l += other_half(l);
    if (q4 == 0 && col < G) {
        float* rec = rec0 + (size_t)col * stride;
        rec[0] = a.mref;
        rec[1] = l;
    }
    if (__all(a.mref == -INFINITY)) return;
#pragma unroll
    for (int g = 0; g < D / 32; ++g) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = a.vx[g][r] + __shfl_xor(a.vx[g][r], G, 16) * INV_LO;
        if ((col & 7) < G) {
            float* rec = rec0 + (size_t)(col & 7) * stride;
#pragma unroll
            for (int r = 0; r < 4; ++r) rec[2 + 2 * (16 * g + 4 * q4 + r) + (col >> 3)] = o[r];
        }
    }
    if (qjl) {
#pragma unroll
        for (int n = 0; n < M / 16; ++n) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = a.vs[n][r] + __shfl_xor(a.vs[n][r], G, 16) * INV_LO;
            if (col >= 8 && col < 8 + G)
                *reinterpret_cast<float4*>(rec0 + (size_t)(col - 8) * stride + 2 + D + 16 * n + 4 * q4) =
                    float4{o[0], o[1], o[2], o[3]};
        }
    }
}

// cand_collect for the packed layout: main lanes (prole 0) hold head col % 8
// and tokens 16 half + 4 q4 + i.
template <int G>
__device__ __forceinline__ void cand_collect_p(const Dims& dm, int T, int q4, int col, int lane, const float (&lgc)[4],
                                               uint32_t cmask, float mref, float l_run, int* ncand, Cand* s_cand) {
    const int ktop = dm.ktop;
    if (__any(cmask != 0u)) {
        if (cmask != 0u) {
            const int head = col & 7, t0 = T * TILE + 16 * (col >> 3) + 4 * q4;
            for (uint32_t mk = cmask; mk; mk &= mk - 1) {
                const int i = __builtin_ctz(mk);
                const int at = atomicAdd(&ncand[head], 1);
                if (at < 2 * ktop) s_cand[head * 2 * ktop + at] = Cand{lgc[i], t0 + i};
            }
        }
        float lw = rows_sum(l_run);
        lw += other_half(lw);  // the part's running sum (main lanes)
        __builtin_amdgcn_wave_barrier();
        if (lane < G) {
            const int n = min(ncand[lane], 2 * ktop);
            int k2 = 0;
            for (int i = 0; i < n; ++i) {
                const Cand cc = s_cand[lane * 2 * ktop + i];
                if (__builtin_amdgcn_exp2f(cc.v - mref) >= dm.tau * lw && k2 < ktop) s_cand[lane * 2 * ktop + k2++] = cc;
            }
            ncand[lane] = k2;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Parts: stream (sequence bi, kv head) has cs.n_new[bi] parts (the field is
// reused by the decode batch); part item = part_off[bi] + kvh * parts + k.
template <int D, int CB, int M, int G, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD, WAVES_PER_SIMD))) void k_decode(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs,
                                                const _Float16* __restrict__ qin, int n_items,
                                                float* logits, int lstride) {
    using Gm = Geom<D, CB, M>;
    constexpr bool PACK = G <= 4;  // packed tile layout (two token halves in the two column halves)
    constexpr int TABS = PACK ? PGeom<D, CB, M>::TABS : Gm::TABS;
    __shared__ __attribute__((aligned(16))) uint8_t s_tab[TABS];
    // ring stages per wave (a fourth stage in the packed layout measured no
    // faster for F3 and F2.5 and slower for F4)
    constexpr int NS = 3;
    __shared__ __attribute__((aligned(16))) uint8_t s_st[NS][4][Gm::KVB];
    __shared__ int s_ncand[4][8];
    __shared__ int s_off[MAX_CALL_SEQ + 1];
    extern __shared__ Cand s_cand_all[];  // [4 waves][G][2 * ktop]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar control flow below
    const int q4 = lane >> 4, col = lane & 15;
    const int role = col < G ? 0 : (col < 2 * G ? 1 : 2);
    const int ktop = dm.ktop;
    Cand* s_cand = s_cand_all + (size_t)wave * G * 2 * (ktop > 0 ? ktop : 1);
    int* ncand = &s_ncand[wave][0];
    const RoleK rk = role == 1 ? RoleK{1.0f / LO_SCALE, -(float)LO_SCALE} : RoleK{1.0f, 0.0f};

    // tables (whole KB): wave w copies KB w, w + 4, ...; item offsets per sequence
    for (int i = wave; i < TABS / 1024; i += 4)
        stage_copy<1024>(P.tables + F.tab_off + 1024 * i, s_tab + 1024 * i, lane);
    if (tid <= cs.n) s_off[tid] = tid < cs.n ? cs.in_base[tid] : n_items;  // first item of each sequence
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    const int n_waves = gridDim.x * 4;
    const int nrt = dm.cap / TILE;  // ring tiles
    const int stride = part_stride(D);
    const int n_half = (n_items + 1) >> 1;
    for (int slot = blockIdx.x * 4 + wave; slot < n_items; slot += n_waves) {
        // slots of the grid's first half take the even items, the others the odd ones
        const int item = slot < n_half ? 2 * slot : 2 * (slot - n_half) + 1;
        // locate (sequence, kv head, part)
        int bi = 0;  // the last sequence whose first item is <= item (every sequence has items)
        for (int hi = cs.n - 1; bi < hi;) {
            const int mid = (bi + hi + 1) >> 1;
            if (s_off[mid] <= item)
                bi = mid;
            else
                hi = mid - 1;
        }
        const int parts = cs.n_new[bi];
        const int kvh = (item - s_off[bi]) / parts, k = (item - s_off[bi]) % parts;
        const int seq = cs.ids[bi];
        const size_t sl = sl_index(dm, seq, layer);
        const int head = col % G;
        const int hq_idx = kvh * G + head;
        // The cold phase's query operands are requested first: they travel
        // together with the metadata and have landed by the cold set-up.
        const uint8_t* qb = reinterpret_cast<const uint8_t*>(P.qprep + ((size_t)bi * dm.hq + hq_idx) * (D + M_MAX));
        QBlocks<D, CB, M> qblk;
        if constexpr (PACK) packed_b_load<D, CB, M>(qb, q4, qblk);
        const SeqLayerMeta mt = P.meta[sl];
        // hot-first gate of this (sequence, kv head), from k_qprep's slices
        const bool gating = dm.gate < INFINITY;
        const bool gated = gating && mt.count > 0 && gate_closed<G>(dm, P, bi, kvh, lane);
        // unit split: hot FIFO tiles cost HOT_UNITS each, then cold tiles COLD_UNITS each
        // hot FIFO tiles: ring tiles from the head's tile on, each ring tile once
        // (a full ring whose head is not tile-aligned would otherwise revisit it)
        const int H = mt.count > 0 ? min(nrt, ((mt.head % TILE) + mt.count + TILE - 1) / TILE) : 0;
        const int C = (mt.cold_len + TILE - 1) / TILE;
        const int64_t HS = (int64_t)HOT_UNITS * H;
        const int64_t S = HS + (int64_t)COLD_UNITS * C;
        // cumulative cost of the stream's first kk parts, in 1/1024 of a part
        // (even items 1024 + AGE_SKEW each, odd ones 1024 - AGE_SKEW)
        const int b0 = (s_off[bi] + kvh * parts) & 1;  // parity of the stream's first item
        auto cum = [&](int kk) -> int64_t {
            return (int64_t)kk * 1024 + ((kk & 1) ? (b0 == 0 ? AGE_SKEW : -AGE_SKEW) : 0);
        };
        const int64_t cum_all = cum(parts);
        const int64_t u0 = S * cum(k) / cum_all, u1 = S * cum(k + 1) / cum_all;
        auto clamp = [](int64_t v, int64_t lo, int64_t hi) { return (int)(v < lo ? lo : (v > hi ? hi : v)); };
        // a tile belongs to the part holding its first unit
        int h0 = clamp((u0 + HOT_UNITS - 1) / HOT_UNITS, 0, H);
        int h1 = clamp((u1 + HOT_UNITS - 1) / HOT_UNITS, 0, H);
        int t_first = clamp((u0 - HS + COLD_UNITS - 1) / COLD_UNITS, 0, C);
        int t_last = clamp((u1 - HS + COLD_UNITS - 1) / COLD_UNITS, 0, C);
        if (gating) {
            // under a gate both kinds of tile are split evenly over the parts,
            // so that a gated stream's hot tiles do not all fall to its first
            // part; a gated stream's parts score no cold tile (their cold
            // records stay empty)
            h0 = H * k / parts;
            h1 = H * (k + 1) / parts;
            t_first = C * k / parts;
            t_last = gated ? t_first : C * (k + 1) / parts;
        }
        float* rec_hot = P.part + ((size_t)item * 2 + 0) * G * stride;
        float* rec_cold = P.part + ((size_t)item * 2 + 1) * G * stride;
        float* lrow = DBG ? logits + ((size_t)bi * dm.hq + hq_idx) * lstride : nullptr;
        Acc<D, M> a;
        // The part's first two cold tile pairs are on their way before the
        // hot phase and the cold set-up.  Ring: tile T lives in stage
        // (T - t_first) % NS; every step issues one tile pair (past the end:
        // the last tile again, an L2 hit), so the wait for a tile is always
        // "NS - 1 tile pairs may remain in flight" (loads complete in order).
        const uint8_t* cbase = P.cold + cold_tile_offset(dm, F, seq, kvh, 0, 0);
        auto src = [&](int T) { return cbase + (size_t)min(T, t_last - 1) * Gm::KVB; };
        if (t_first < t_last) {
            stage_copy<Gm::KVB>(src(t_first), s_st[0][wave], lane);
            stage_copy<Gm::KVB>(src(t_first + 1), s_st[1][wave], lane);
        }
        // The tombstone words are requested now too.
        const uint32_t* tomb = P.tomb + sl * (dm.cold_cap / 32);
        // tombstone words of 64 of the part's tiles, one per lane
        int tomb_base = t_first;
        uint32_t tomb_all = (t_first + lane < t_last) ? tomb[t_first + lane] : 0u;
        const int half = col >> 3, r8 = col & 7;
        const int prole = r8 < G ? 0 : (r8 < 2 * G ? 1 : 2);

        // ------------------------------------------------------ hot phase
        acc_reset(a);
        if (h0 < h1) {
            half8 qh[D / 32];
            const _Float16* qo = qin + ((size_t)bi * dm.hq + hq_idx) * D;
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) qh[kb] = *reinterpret_cast<const half8*>(qo + kb * 32 + 8 * q4);
            const size_t rb = ring_base(dm, seq, layer, kvh);
            for (int j = h0; j < h1; ++j)
                hot_tile<D, M, G, DBG>(dm, P, mt, rb, (mt.head / TILE + j) % nrt, q4, col, role, rk, qh, a, lrow);
        }
        write_record<D, M, G>(rec_hot, stride, a, false, q4, col, false);

        // ----------------------------------------------------- cold phase
        acc_reset(a);
        if (lane < 8) ncand[lane] = 0;
        __builtin_amdgcn_wave_barrier();
        if (t_first < t_last) {
            // (called with T = t_first, t_first + 1, ... in order)
            auto live_of = [&](int T) -> uint32_t {
                if (T - tomb_base >= 64) {  // parts of more than 64 tiles: the next 64 words
                    tomb_base += 64;
                    tomb_all = (tomb_base + lane < t_last) ? tomb[tomb_base + lane] : 0u;
                    settle(tomb_all);
                }
                const uint32_t tw = __builtin_amdgcn_readlane(tomb_all, T - tomb_base);
                const int n = mt.cold_len - T * TILE;
                const uint32_t valid = n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u);
                return valid & ~tw;
            };
            auto wait_tile = [&]() {
                if constexpr (DBG)
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // logit stores share the counter
                else
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * Gm::NI));
                __builtin_amdgcn_wave_barrier();
            };
            auto run_ring = [&](auto&& tile) {
                for (int T = t_first; T < t_last; T += 3) {
                    stage_copy<Gm::KVB>(src(T + 2), s_st[2][wave], lane);
                    wait_tile();
                    tile(s_st[0][wave], T);
                    if (T + 1 >= t_last) break;
                    stage_copy<Gm::KVB>(src(T + 3), s_st[0][wave], lane);
                    wait_tile();
                    tile(s_st[1][wave], T + 1);
                    if (T + 2 >= t_last) break;
                    stage_copy<Gm::KVB>(src(T + 4), s_st[1][wave], lane);
                    wait_tile();
                    tile(s_st[2][wave], T + 2);
                }
                // the ring's trailing copies must land before the stages are reused
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            };
            if constexpr (PACK) {
                const RoleK rkp = prole == 1 ? RoleK{1.0f / LO_SCALE, -(float)LO_SCALE} : RoleK{1.0f, 0.0f};
                half8 bk[D / 16], bsx[M / 32];
                packed_b<D, CB, M>(qblk, prole, bk, bsx);
#pragma unroll
                for (int i = 0; i < D / 16; ++i) settle(bk[i]);
#pragma unroll
                for (int i = 0; i < M / 32; ++i) settle(bsx[i]);
                settle(tomb_all);
                float lgc[4];
                uint32_t cmask = 0u;
                PTile<D, CB, M> t;
                PKeyWords<D, CB, M> kw;
                PKeyOps<D, CB, M> ko0, ko1;
                constexpr int SBM = 0x416;  // VALU, SALU, VMEM, transcendental may cross
                // the ring's other tiles: NS tile pairs in flight before the first step
#pragma unroll
                for (int j = 2; j < NS; ++j) stage_copy<Gm::KVB>(src(t_first + j), s_st[j][wave], lane);
                auto step = [&](uint8_t* cur, int T) {
                    // The two waves of a SIMD come from the first and the second
                    // half of the grid (two blocks per CU, dispatched in order);
                    // at equal priority the older wave issues first and finishes
                    // its equal share well ahead of the other.  Raising the
                    // younger wave's priority on two tiles in three and the
                    // older one's on the third shares the issue slots about
                    // evenly (measured).
                    if (blockIdx.x >= gridDim.x / 2 ? (T % 3) != 0 : (T % 3) == 0)
                        __builtin_amdgcn_s_setprio(1);
                    else
                        __builtin_amdgcn_s_setprio(0);
                    // tile T landed: tiles T + 1 .. T + NS - 1 may remain in flight
                    if constexpr (DBG)
                        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    else
                        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * Gm::NI));
                    __builtin_amdgcn_wave_barrier();
                    // the value side's words first: the key words' wait then
                    // covers both (one LDS round trip)
                    PVWords<D, CB, M> vw;
                    pk_vwords(cur, q4, col, half, vw);
                    pk_words(cur, q4, col, kw);
                    pk_key_reads(s_tab, kw, 0, ko0);
                    __builtin_amdgcn_sched_barrier(SBM);
                    pk_key_mfmas(ko0, bk, bsx, t.kac[0], t.sac[0]);
                    pk_key_reads(s_tab, kw, 1, ko1);
                    __builtin_amdgcn_sched_barrier(SBM);
                    pk_key_mfmas(ko1, bk, bsx, t.kac[1], t.sac[1]);
                    pk_meta(cur, q4, half, t);
                    PVals<D, CB, M> v;
                    pk_values(vw, s_tab, q4, v);
                    pk_finish<D, CB, M, G, DBG>(dm, t, v, T, live_of(T), q4, half, prole, rkp, a, lrow, lgc, cmask);
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage's reads are done before it is refilled
                    stage_copy<Gm::KVB>(src(T + NS), cur, lane);
                    __builtin_amdgcn_wave_barrier();
                    if (ktop > 0) cand_collect_p<G>(dm, T, q4, col, lane, lgc, cmask, a.mref, a.l_run, ncand, s_cand);
                };
                for (int T = t_first; T < t_last; T += NS) {
                    bool done = false;
#pragma unroll
                    for (int j = 0; j < NS; ++j) {
                        if (!done) {
                            step(s_st[j][wave], T + j);
                            done = T + j + 1 >= t_last;
                        }
                    }
                    if (done) break;
                }
                // the ring's trailing copies must land before the stages are reused
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            } else {
                half8 qh[D / 32], ql[D / 32], sh[M / 32], slo[M / 32];
                // 8 consecutive values = two [hi x4 | lo x4] blocks
                auto hl8 = [&](const uint8_t* b0, half8& hi, half8& lo) {
                    typedef union {
                        uint32_t u[4];
                        uint4 q;
                        half8 h;
                    } op8;
                    op8 a, b, h, l;
                    a.q = *reinterpret_cast<const uint4*>(b0);
                    b.q = *reinterpret_cast<const uint4*>(b0 + 16);
                    h.u[0] = a.u[0], h.u[1] = a.u[1], h.u[2] = b.u[0], h.u[3] = b.u[1];
                    l.u[0] = a.u[2], l.u[1] = a.u[3], l.u[2] = b.u[2], l.u[3] = b.u[3];
                    hi = h.h;
                    lo = l.h;
                };
#pragma unroll
                for (int kb = 0; kb < D / 32; ++kb) hl8(qb + 16 * (8 * kb + 2 * q4), qh[kb], ql[kb]);
#pragma unroll
                for (int sb = 0; sb < M / 32; ++sb) hl8(qb + 4 * D + 16 * (8 * sb + 2 * q4), sh[sb], slo[sb]);
#pragma unroll
                for (int i = 0; i < D / 32; ++i) settle(qh[i]), settle(ql[i]);
#pragma unroll
                for (int i = 0; i < M / 32; ++i) settle(sh[i]), settle(slo[i]);
                settle(tomb_all);
                float lgc[8];
                uint32_t cmask = 0u;
                run_ring([&](const uint8_t* stg, int T) {
                    cold_tile<D, CB, M, G, DBG>(dm, stg, T, live_of(T), q4, col, role, qh, ql, sh, slo, a, s_tab, rk,
                                                lrow, lgc, cmask);
                    __builtin_amdgcn_wave_barrier();
                    if (ktop > 0) cand_collect<G>(dm, T, q4, col, lane, lgc, cmask, a.mref, a.l_run, ncand, s_cand);
                });
            }
        }
        if constexpr (PACK)
            write_record_p<D, M, G>(rec_cold, stride, a, q4, col, dm.v_qjl != 0);
        else
            write_record<D, M, G>(rec_cold, stride, a, true, q4, col, dm.v_qjl != 0);
        if (ktop > 0 && lane < G) {
            Cand* cc = P.cand_chunk + ((size_t)item * G + lane) * ktop;
            const int n = t_first < t_last ? min(ncand[lane], ktop) : 0;
            for (int i = 0; i < ktop; ++i) cc[i] = i < n ? s_cand[lane * 2 * ktop + i] : Cand{-INFINITY, -1};
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Pre-merge for streams of more than PM_CHUNK parts (launches over few
// streams, e.g. one long sequence): block (sequence, query head, chunk c)
// merges the hot records and the cold records of parts [32 c, 32 c + 32)
// into one record each, written over the chunk's first part: max
// M = max m_r, sum sum_r 2^(m_r - M) s_r, components sum_r 2^(m_r - M) x_r
// (the combine's own merge, so the result is the same up to rounding
// order).  Records of weight 0 are not read; a chunk without tokens leaves a
// header (-inf, 0) and no components.  QJL rows the decode kernel never
// writes are written as 0.
template <int D>
__global__ __launch_bounds__(2 * D + M_MAX) void k_premerge(Dims dm, LayerFmt F, CallSeqs cs, float* __restrict__ part) {
    constexpr int C = PM_CHUNK;
    const int bi = blockIdx.x, h = blockIdx.y, c = blockIdx.z, tid = threadIdx.x;
    const int parts = cs.n_new[bi];
    if (parts <= C || c * C >= parts) return;
    __shared__ float s_w[2][C];
    __shared__ float s_ms[2][2];
    const int G = dm.g, kvh = h / G, hh = h % G;
    const int stride = part_stride(D);
    const int item0 = cs.in_base[bi] + kvh * parts;
    float* rec0 = part + ((size_t)item0 * 2 * G + hh) * stride;
    const size_t rstride = (size_t)G * stride;
    const int u0 = c * C, nu = min(C, parts - u0);
    if (tid < 2 * C) {  // one lane per record: kind tid & 1 (0 hot, 1 cold), part u0 + tid / 2
        const int kind = tid & 1, u = tid >> 1;
        float m = -INFINITY, s = 0.0f;
        if (u < nu) {
            const float* r = rec0 + (size_t)(2 * (u0 + u) + kind) * rstride;
            m = r[0];
            s = r[1];
        }
        float M = m;
#pragma unroll
        for (int o = 2; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
        const float w = m == -INFINITY ? 0.0f : exp2f(m - M);
        float S = w * s;
#pragma unroll
        for (int o = 2; o < 64; o <<= 1) S += __shfl_xor(S, o, 64);
        s_w[kind][u] = w;
        if (tid < 2) s_ms[kind][0] = M, s_ms[kind][1] = S;
    }
    __syncthreads();
    const bool hotpart = tid >= D + M_MAX;
    const int comp = hotpart ? tid - D - M_MAX : tid;
    const int kind = hotpart ? 0 : 1;
    const float* base = rec0 + (size_t)kind * rstride + 2 + comp;
    // a record of weight 0 is read at the chunk's first record instead (one
    // cached line for all of them), so every load is unconditional and all
    // are in flight together
    float cw[C], cx[C];
#pragma unroll
    for (int u = 0; u < C; ++u) {
        cw[u] = s_w[kind][u];  // 0 past the chunk's last part
        cx[u] = base[(size_t)(2 * (u0 + (cw[u] != 0.0f ? u : 0))) * rstride];
    }
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < C; ++u) a[u & 7] = cw[u] != 0.0f ? fmaf(cw[u], cx[u], a[u & 7]) : a[u & 7];
    float sum = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    if (!hotpart && tid >= D && !(dm.v_qjl && tid - D < F.m)) sum = 0.0f;
    __syncthreads();  // every read of the chunk's records is done before its first part is overwritten
    float* dst = rec0 + (size_t)(2 * u0 + kind) * rstride;
    const float M = s_ms[kind][0];
    if (M != -INFINITY) dst[2 + comp] = sum;
    if (comp == 0) dst[0] = M, dst[1] = s_ms[kind][1];
}

// One block per (sequence, query head), one thread per output component
// (hot dims, cold rotated components, QJL sums).  Every global load is issued
// at the start, so the block waits for memory about once: the record headers,
// the thread's component of the first CH records of its kind, the thread's
// slice of a column of [Pi; S Pi] (into registers, coalesced across the
// threads: no matrix in LDS, so two blocks share a CU) and the parts'
// candidate lists (into LDS).  Then:
// record weights 2^(m_c - M) in LDS, the weighted sums over the records
// (records without tokens have weight 0 and finite contents), the rotation
// back, Pi^T (cold + sqrt(pi/2)/m S_m^T qjl) = Pi^T cold + (S_m Pi)^T
// sqrt(pi/2)/m qjl as one dot of D + m terms per output, and the candidates'
// exact probabilities.
// PRE: the [Pi; S Pi] column slice is requested at the start and waits in
// registers (fastest per block; two blocks per CU).  Without PRE it is read
// inside the output dot, after the records: fewer registers, more blocks per
// CU, for launches with more blocks than two per CU.
template <int D, bool PRE>
__global__ __launch_bounds__(2 * D + M_MAX) void k_combine(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs,
                                                           const _Float16* __restrict__ qin, float* __restrict__ out) {
    constexpr int NT = 2 * D + M_MAX;
    constexpr int CH = PM_CHUNK;                        // records of each kind, at most
    constexpr int HR = (2 * CH + NT - 1) / NT;          // record headers per thread
    constexpr int CC = 1024;                            // candidate entries staged in LDS
    static_assert(MAX_PARTS <= PM_CHUNK * CH, "a pre-merged stream has at most CH records of each kind");
    __shared__ float s_w[2 * CH];
    __shared__ float s_acc[NT];  // [0, D) cold rotated, [D, D + M_MAX) QJL sums, [D + M_MAX, +D) hot
    __shared__ float s_red[2 * (NT / 64)];
    __shared__ Cand s_cc[CC];
    __shared__ int s_n;
    __shared__ float s_part[2][D];
    const int bi = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int seq = cs.ids[bi];
    const int G = dm.g, kvh = h / G, hh = h % G;
    const int stride = part_stride(D);
    const int off = cs.in_base[bi];  // first item of the sequence
    const int parts = cs.n_new[bi];
    const int item0 = off + kvh * parts;
    // a stream of more than PM_CHUNK parts was pre-merged (k_premerge): its
    // records are those of parts 0, PM_CHUNK, 2 PM_CHUNK, ...
    const int pstep = parts > PM_CHUNK ? PM_CHUNK : 1;
    const int nv = (parts + pstep - 1) / pstep;  // records of each kind (<= CH)
    const int nrec = 2 * nv;  // record r: merged part r / 2, hot (even) or cold (odd)
    const float* rec0 = P.part + ((size_t)item0 * 2 * G + hh) * stride;
    const size_t rstride = (size_t)G * stride;  // consecutive records
    auto rec_at = [&](int r) { return rec0 + ((size_t)2 * (r >> 1) * pstep + (r & 1)) * rstride; };
    // ------------------------------------------------------------ loads
    // every load below is unconditional (past the end: an address that is
    // read anyway), so that none waits for another
    float hm[HR], hs[HR];
#pragma unroll
    for (int i = 0; i < HR; ++i) {
        const int r = tid + i * NT;
        const float* rh = rec_at(min(r, nrec - 1));
        hm[i] = rh[0];
        hs[i] = rh[1];
    }
    const bool hotpart = tid >= D + M_MAX;
    const int comp = hotpart ? tid - D - M_MAX : tid;
    const int r0 = hotpart ? 0 : 1;
    const float* base = rec_at(r0) + 2 + comp;  // record r0 + 2 u at base + 2 u pstep rstride
    float cv[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) cv[u] = base[(size_t)(2 * min(u, nv - 1) * pstep) * rstride];
    // rows u0 .. u0 + KH of [Pi; S Pi], column i, for the output dot below
    // (threads 2 D .. NT load a valid column they do not use)
    constexpr int KH = (D + M_MAX) / 2;
    const int di = tid % D, du0 = min(tid / D, 1) * KH;
    auto mat = [&](int u) {
        const int row = du0 + u;
        return row < D ? P.pi32[(size_t)row * D + di] : P.sp32[(size_t)(row - D) * D + di];
    };
    float mcol[PRE ? KH : 1];
    if constexpr (PRE) {
#pragma unroll
        for (int u = 0; u < KH; ++u) mcol[u] = mat(u);
    }
    const int ktop = dm.ktop;
    const int ncc = parts * ktop;
    const bool staged = ncc <= CC;
    auto cand_at = [&](int k, int i) { return P.cand_chunk + ((size_t)(item0 + k) * G + hh) * ktop + i; };
    if (staged)
        for (int e = tid; e < ncc; e += NT) s_cc[e] = *cand_at(e / ktop, e % ktop);
    // ------------------------------------------------------------ headers
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < HR; ++i) {
        if (tid + i * NT >= nrec) hm[i] = -INFINITY, hs[i] = 0.0f;
        mx = fmaxf(mx, hm[i]);
    }
    mx = wave_max(mx);
    const int wave = tid >> 6, nwv = NT / 64;
    if ((tid & 63) == 0) s_red[wave] = mx;
    __syncthreads();
    float Mx = s_red[0];
    for (int w = 1; w < nwv; ++w) Mx = fmaxf(Mx, s_red[w]);
    float ls = 0.0f;
#pragma unroll
    for (int i = 0; i < HR; ++i) {
        const int r = tid + i * NT;
        const float w = hm[i] == -INFINITY ? 0.0f : exp2f(hm[i] - Mx);
        if (r < nrec) s_w[r] = w;
        ls = fmaf(w, hs[i], ls);
    }
    ls = wave_sum(ls);
    if ((tid & 63) == 0) s_red[nwv + wave] = ls;
    __syncthreads();
    float L = 0.0f;
    for (int w = 0; w < nwv; ++w) L += s_red[nwv + w];
    // ------------------------------------------------------- components
    {
        // a record without tokens (weight 0) keeps whatever an earlier launch
        // left in its accumulators: it is skipped, not multiplied by 0
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (u < nv) {
                const float w = s_w[r0 + 2 * u];
                a[u & 7] = w != 0.0f ? fmaf(w, cv[u], a[u & 7]) : a[u & 7];
            }
        float sum = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
        if (tid < D) sum *= F.vscale_inv;  // the value tables hold the unit values times vscale
        if (tid >= D && tid < D + M_MAX)  // QJL sum j: weight sqrt(pi/2) / m; rows j >= m (and every row
            // when values take no QJL term) are never written by the decode kernel: selected away, not
            // multiplied by 0, so that whatever the workspace held cannot reach the output
            sum = (dm.v_qjl && tid - D < F.m) ? sum * (SQRT_HALF_PI / (float)F.m) : 0.0f;
        s_acc[tid] = sum;
    }
    __syncthreads();
    // out_i = (sum_k Pi[k][i] cold_k + sum_j (S Pi)[j][i] w_j qjl_j + hot_i) / L,
    // the D + M_MAX terms split in two halves over 2 D threads
    if (tid < 2 * D) {
        float o0 = 0.0f, o1 = 0.0f;
        if constexpr (PRE) {
#pragma unroll
            for (int u = 0; u < KH; u += 2) {
                o0 = fmaf(mcol[u], s_acc[du0 + u], o0);
                o1 = fmaf(mcol[u + 1], s_acc[du0 + u + 1], o1);
            }
        } else {
#pragma unroll 16
            for (int u = 0; u < KH; u += 2) {
                o0 = fmaf(mat(u), s_acc[du0 + u], o0);
                o1 = fmaf(mat(u + 1), s_acc[du0 + u + 1], o1);
            }
        }
        s_part[tid / D][di] = o0 + o1;
    }
    __syncthreads();
    if (tid < D) {
        const float v = (s_part[0][tid] + s_part[1][tid]) + s_acc[D + M_MAX + tid];
        float o = L > 0.0f ? v / L : 0.0f;
        if (dm.tc) {
            // Tensor Cache read ("Tensor Cache", section "Metodologia"):
            // y = y_local + sigmoid(g) (q A)_tid, column tid of the kv head's A
            const float* A = P.tc_a + (sl_index(dm, seq, layer) * dm.hkv + kvh) * (size_t)D * D;
            const _Float16* qh = qin + head_row(dm, bi, kvh, hh, true) * D;
            float r0 = 0.0f, r1 = 0.0f, r2 = 0.0f, r3 = 0.0f;
#pragma unroll 8
            for (int j = 0; j < D; j += 4) {
                r0 = fmaf((float)qh[j], A[(size_t)j * D + tid], r0);
                r1 = fmaf((float)qh[j + 1], A[(size_t)(j + 1) * D + tid], r1);
                r2 = fmaf((float)qh[j + 2], A[(size_t)(j + 2) * D + tid], r2);
                r3 = fmaf((float)qh[j + 3], A[(size_t)(j + 3) * D + tid], r3);
            }
            o += dm.tc_sg * ((r0 + r1) + (r2 + r3));
        }
        const int64_t row = head_row(dm, bi, kvh, hh, false);
        if (row >= 0) out[row * D + tid] = o;
    }
    // promotion candidates: exact probabilities; one thread per part (at most
    // 1 / tau tokens can reach tau, so the list never overflows ktop)
    const size_t sl = sl_index(dm, seq, layer);
    if (ktop > 0) {
        if (tid == 0) s_n = 0;
        __syncthreads();
        Cand* dst = P.cand + (sl * dm.hq + h) * ktop;
        for (int k = tid; k < parts; k += NT) {
            for (int i = 0; i < ktop; ++i) {
                const Cand c = staged ? s_cc[k * ktop + i] : *cand_at(k, i);
                if (c.slot < 0) break;
                const float pr = exp2f(c.v - Mx) / L;
                if (pr >= dm.tau) {
                    const int at = atomicAdd(&s_n, 1);
                    if (at < ktop) dst[at] = Cand{pr, c.slot};
                }
            }
        }
        __syncthreads();
        if (tid == 0) P.cand_n[sl * dm.hq + h] = min(s_n, ktop);
    }
    if (tid == 0 && h == 0 && dm.mq_n == 0) P.meta[sl].attn_step += 1;  // decode steps only
}

// ------------------------------------------------------------------------
// Compressed-vector search scan (the codec's vector-search use:
// "Compresion del cache KV de los LLM a 3 bits: TurboQuant", sudonull.com,
// section "Aplicaciones mas alla de los LLMs").  One wave per (part of a
// stream's cold tiles, group of 8 queries).  Key tiles stream through a
// three-stage LDS ring (value tiles are not read).  Per tile the scores of
// the 8 queries come from the packed key MFMAs above with every column used:
// column c < 8 is query c's main part (hi . q'hi), column 8 + c its cross
// part (hi . q'lo + lo . q'hi), so a lane of column c < 8 finishes the
// scores of 8 vectors for query c.  Scores above the query's running k-th
// best are appended to a per-query LDS list (positions by a prefix over the
// query's four lanes, no atomics); a list that could not take another
// tile's 32 is cut back to its best k by rank (keep_best).
// ------------------------------------------------------------------------
constexpr int MS_Q = 8;       // queries per group
constexpr int MS_CAP = 64;    // candidate list per query (k <= 32 plus one tile's 32)
constexpr int MS_KMAX = 32;   // the largest k

__device__ __forceinline__ bool cand_before(const Cand& a, const Cand& b) {
    return a.v > b.v || (a.v == b.v && a.slot < b.slot);
}

// Keeps the best k of list[0 .. n) (n <= 128) in order, with the whole
// wave: lane i ranks entries i and i + 64 against every entry (broadcast
// LDS reads); slots are distinct, so the ranks are a permutation.
__device__ void keep_best(Cand* list, int n, int k, Cand* tmp, int lane) {
    const Cand none{-INFINITY, 0x7fffffff};
    const Cand e0 = lane < n ? list[lane] : none, e1 = lane + 64 < n ? list[lane + 64] : none;
    int r0 = 0, r1 = 0;
    for (int j = 0; j < n; ++j) {
        const Cand f = list[j];
        r0 += cand_before(f, e0);
        r1 += cand_before(f, e1);
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < n && r0 < k) tmp[r0] = e0;
    if (lane + 64 < n && r1 < k) tmp[r1] = e1;
    __builtin_amdgcn_wave_barrier();
    if (lane < min(n, k)) list[lane] = tmp[lane];
    __builtin_amdgcn_wave_barrier();
}

template <int D, int CB, int M>
__global__ __launch_bounds__(256) void k_mips_scan(Dims dm, Ptrs P, LayerFmt F, int layer, int seq, int kvh,
                                                   int n_groups, int n_parts, int k, Cand* __restrict__ partial) {
    using Gm = Geom<D, CB, M>;
    using PG = PGeom<D, CB, M>;
    static_assert(!PG::KT2, "the scan reads the one-code (hi, lo) key table");
    constexpr int TB = Gm::TB;
    constexpr int TBR = (TB + 255) / 256 * 256;  // whole DMA chunks (the tail reads the V tile that follows)
    constexpr int NI = stage_instrs<TBR>();
    constexpr int TABS = kb_round(PG::KOFF + 8 * Gm::NCODE);
    __shared__ __attribute__((aligned(16))) uint8_t s_tab[TABS];
    __shared__ __attribute__((aligned(16))) uint8_t s_st[4][3][TBR];
    __shared__ Cand s_list[4][MS_Q][MS_CAP];
    __shared__ Cand s_tmp[4][MS_KMAX];
    __shared__ int s_n[4][MS_Q];
    __shared__ float s_thr[4][MS_Q];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q4 = lane >> 4, col = lane & 15, qc = col & 7;
    const int prole = col < MS_Q ? 0 : 1;
    for (int i = wave; i < TABS / 1024; i += 4)
        stage_copy<1024>(P.tables + F.tab_off + 1024 * i, s_tab + 1024 * i, lane);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    const size_t sl = sl_index(dm, seq, layer);
    const SeqLayerMeta mt = P.meta[sl];
    const int C = (mt.cold_len + TILE - 1) / TILE;
    const uint32_t* tomb = P.tomb + sl * (dm.cold_cap / 32);
    const uint8_t* cbase = P.cold + cold_tile_offset(dm, F, seq, kvh, 0, 0);
    for (int item = blockIdx.x * 4 + wave; item < n_groups * n_parts; item += gridDim.x * 4) {
        // the groups of one part are neighbouring items (waves of one block):
        // they read the same key tiles at about the same time
        const int part = item / n_groups, grp = item % n_groups;
        const int t0 = (int)((int64_t)C * part / n_parts), t1 = (int)((int64_t)C * (part + 1) / n_parts);
        const uint8_t* qb = reinterpret_cast<const uint8_t*>(P.qprep + ((size_t)grp * MS_Q + qc) * (D + M_MAX));
        QBlocks<D, CB, M> qblk;
        packed_b_load<D, CB, M>(qb, q4, qblk);
        if (lane < MS_Q) {
            s_n[wave][lane] = 0;
            s_thr[wave][lane] = -INFINITY;
        }
        auto src = [&](int T) { return cbase + (size_t)min(T, t1 - 1) * 2 * TB; };
        if (t0 < t1) {
            stage_copy<TBR>(src(t0), s_st[wave][0], lane);
            stage_copy<TBR>(src(t0 + 1), s_st[wave][1], lane);
        }
        // tombstone words of 64 tiles, one per lane, before the ring (a load
        // first read inside the ring would drain it every turn)
        int tomb_base = t0;
        uint32_t tomb_all = (t0 + lane < t1) ? tomb[t0 + lane] : 0u;
        half8 bk[D / 16], bsx[M / 32];
        packed_b<D, CB, M>(qblk, prole, bk, bsx);
#pragma unroll
        for (int i = 0; i < D / 16; ++i) settle(bk[i]);
#pragma unroll
        for (int i = 0; i < M / 32; ++i) settle(bsx[i]);
        settle(tomb_all);
        __builtin_amdgcn_wave_barrier();
        for (int T = t0; T < t1; ++T) {
            const int stg = (T - t0) % 3;
            if (T - tomb_base >= 64) {  // parts of more than 64 tiles: the next 64 words
                tomb_base += 64;
                tomb_all = (tomb_base + lane < t1) ? tomb[tomb_base + lane] : 0u;
                settle(tomb_all);
            }
            const uint32_t tw = __builtin_amdgcn_readlane(tomb_all, T - tomb_base);
            stage_copy<TBR>(src(T + 2), s_st[wave][(stg + 2) % 3], lane);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NI));  // tile T landed (loads complete in order)
            __builtin_amdgcn_wave_barrier();
            const uint8_t* kt = s_st[wave][stg];
            const float thr = s_thr[wave][qc];
            const int base = s_n[wave][qc];
            PKeyWords<D, CB, M> kw;
            pk_words(kt, q4, col, kw);
            const int nv = mt.cold_len - T * TILE;
            const uint32_t live = (nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u)) & ~tw;
            const uint8_t* km = kt + TILE * (Gm::PB + Gm::SB);
            float sc[2][4];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                PKeyOps<D, CB, M> ko;
                pk_key_reads(s_tab, kw, st, ko);
                floatx4 kac, sac;
                pk_key_mfmas(ko, bk, bsx, kac, sac);
                const int v0 = 16 * st + 4 * q4;  // this lane's vectors v0 .. v0 + 3
                const uint2 Rr = *reinterpret_cast<const uint2*>(km + 2 * v0);
                const uint2 Pr = *reinterpret_cast<const uint2*>(km + 2 * TILE + 2 * v0);
                const _Float16* Rh = reinterpret_cast<const _Float16*>(&Rr);
                const _Float16* Ph = reinterpret_cast<const _Float16*>(&Pr);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = fmaf(sac[r], (float)Ph[r], mul_h(kac[r], Rh[r]));
                    // main lanes: hi part + cross part (lane c + 8) / 2^12
                    const float y = fmaf(other_half(x), 1.0f / LO_SCALE, x);
                    sc[st][r] = ((live >> (v0 + r)) & 1u) ? y : -INFINITY;
                }
            }
            // candidates of main lanes: their position after the query's
            // earlier lanes (the four rows of its column)
            uint32_t m = 0u;
            if (prole == 0) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m |= (sc[st][r] > thr ? 1u : 0u) << (4 * st + r);
            }
            if (__any(m != 0u)) {
                const int c = __builtin_popcount(m);
                const int c0 = __shfl(c, col, 64), c1 = __shfl(c, col + 16, 64), c2 = __shfl(c, col + 32, 64),
                          c3 = __shfl(c, col + 48, 64);
                const int pre = (q4 > 0 ? c0 : 0) + (q4 > 1 ? c1 : 0) + (q4 > 2 ? c2 : 0);
                int at = base + pre;
                Cand* l = &s_list[wave][qc][0];
                // constant indices into sc (a dynamic index would put it in scratch memory)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if ((m >> i) & 1u) l[at++] = Cand{sc[i >> 2][i & 3], T * TILE + 16 * (i >> 2) + 4 * q4 + (i & 3)};
                if (prole == 0 && q4 == 0) s_n[wave][qc] = base + c0 + c1 + c2 + c3;
                __builtin_amdgcn_wave_barrier();
                // a list that could not take another tile's 32 keeps its best k
                const int nl = lane < MS_Q ? s_n[wave][lane] : 0;
                uint64_t need = __ballot(nl > MS_CAP - TILE);
                while (need) {
                    const int qq = __builtin_ctzll(need);
                    need &= need - 1;
                    Cand* lq = &s_list[wave][qq][0];
                    const int n = __builtin_amdgcn_readlane(nl, qq);
                    keep_best(lq, n, k, s_tmp[wave], lane);
                    if (lane == 0) {
                        s_n[wave][qq] = k;
                        s_thr[wave][qq] = lq[k - 1].v;
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the ring's trailing copies
        __builtin_amdgcn_wave_barrier();
        // the part's best k per query, in order (-inf / -1 padded)
        const int nl = lane < MS_Q ? s_n[wave][lane] : 0;
        for (int qq = 0; qq < MS_Q; ++qq) {
            const int n = __builtin_amdgcn_readlane(nl, qq);
            Cand* lq = &s_list[wave][qq][0];
            keep_best(lq, n, k, s_tmp[wave], lane);
            Cand* dst = partial + (((size_t)grp * n_parts + part) * MS_Q + qq) * k;
            if (lane < k) dst[lane] = lane < n ? lq[lane] : Cand{-INFINITY, -1};
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template <int D, int CB, int M>
static void mips_scan_launch(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, int seq, int kvh,
                             int n_groups, int n_parts, int k, Cand* part, hipStream_t st) {
    const int items = n_groups * n_parts;
    k_mips_scan<D, CB, M><<<(items + 3) / 4, 256, 0, st>>>(dm, P, F, layer, seq, kvh, n_groups, n_parts, k, part);
}

hipError_t launch_mips_scan(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, int seq, int kvh,
                            int n_groups, int n_parts, int k, Cand* part, hipStream_t st) {
    switch (dm.d * 1000 + F.cb * 100 + F.m) {
#define TQ_MS(DD, CBB, MM)                                                                        \
    case DD * 1000 + CBB * 100 + MM:                                                              \
        mips_scan_launch<DD, CBB, MM>(dm, P, F, layer, seq, kvh, n_groups, n_parts, k, part, st); \
        break;
        TQ_MS(64, 5, 32) TQ_MS(64, 5, 64) TQ_MS(64, 7, 32) TQ_MS(64, 7, 64) TQ_MS(64, 4, 32) TQ_MS(64, 4, 64)
        TQ_MS(128, 5, 32) TQ_MS(128, 5, 64) TQ_MS(128, 7, 32) TQ_MS(128, 7, 64) TQ_MS(128, 4, 32) TQ_MS(128, 4, 64)
#undef TQ_MS
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Resident waves of a k_decode instantiation (blocks per CU from the
// occupancy calculator times the CU count, times 4 waves), or a launch.
template <int D, int CB, int M, int G>
static hipError_t decode_launch(hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                                const CallSeqs& cs, const _Float16* q, int n_items, float* logits,
                                int lstride, int* resident, hipEvent_t ev0, hipEvent_t ev1) {
    const size_t shm = (size_t)4 * G * 2 * std::max(dm.ktop, 1) * sizeof(Cand);
    auto kern = logits ? k_decode<D, CB, M, G, true> : k_decode<D, CB, M, G, false>;
    if (resident) {
        int nb = 0, dev = 0, n_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, 256, shm);
        if (e != hipSuccess) return e;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        *resident = std::max(1, nb) * std::max(1, n_cu) * 4;
        return hipSuccess;
    }
    const int blocks = std::max(1, (n_items + 3) / 4);
    if (ev0 || ev1) {
        // timed launch: the events are recorded by the dispatch itself, so
        // timing adds no commands between the kernels of a step
        hipExtLaunchKernelGGL(kern, dim3(blocks), dim3(256), (uint32_t)shm, st, ev0, ev1, 0u, dm, P, F, layer, cs, q,
                              n_items, logits, lstride);
    } else {
        kern<<<blocks, 256, shm, st>>>(dm, P, F, layer, cs, q, n_items, logits, lstride);
    }
    return hipGetLastError();
}

template <int D, int CB, int M>
static hipError_t decode_g(hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                           const CallSeqs& cs, const _Float16* q, int n_items, float* logits, int lstride,
                           int* resident, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    switch (dm.g) {
        case 1: return decode_launch<D, CB, M, 1>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 2: return decode_launch<D, CB, M, 2>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 4: return decode_launch<D, CB, M, 4>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 8: return decode_launch<D, CB, M, 8>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

template <int D, int CB>
static hipError_t decode_m(hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                           const CallSeqs& cs, const _Float16* q, int n_items, float* logits, int lstride,
                           int* resident, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    if (F.m == 32) return decode_g<D, CB, 32>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
    if (F.m == 64) return decode_g<D, CB, 64>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
    return hipErrorInvalidValue;
}

static hipError_t decode_any(hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                             const CallSeqs& cs, const _Float16* q, int n_items, float* logits, int lstride,
                             int* resident, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    switch (dm.d * 10 + F.cb) {
        case 645: return decode_m<64, 5>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 647: return decode_m<64, 7>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 644: return decode_m<64, 4>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 1285: return decode_m<128, 5>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 1287: return decode_m<128, 7>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        case 1284: return decode_m<128, 4>(st, dm, P, F, layer, cs, q, n_items, logits, lstride, resident, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

// Parts per (sequence, kv head) stream so that the launch has about one part
// per resident wave, all of about equal cost.  Estimates come from the host's
// count of appended tokens (cold ~ appended - W, hot ~ min(appended, W) plus
// one tile for the ring offset); the kernel splits the true lengths.
static int plan_parts(const Dims& dm, CallSeqs& cs, const int64_t* appended, int resident) {
    double U = 0.0;
    std::vector<double> su(cs.n);
    for (int i = 0; i < cs.n; ++i) {
        const int64_t a = std::min<int64_t>(appended[i], (int64_t)dm.cold_cap + dm.cap);
        const double cold = (double)((std::max<int64_t>(0, a - dm.W) + TILE - 1) / TILE);
        const double hot = a > 0 ? (double)((std::min<int64_t>(a, dm.W) + TILE - 1) / TILE + 1) : 0.0;
        su[i] = COLD_UNITS * cold + HOT_UNITS * hot;
        U += dm.hkv * su[i];
    }
    const int target = std::max(1, std::min(resident, dm.max_chunks));
    double u = std::max(1.0, U / target);
    int n_items = 0;
    for (int pass = 0; pass < 16; ++pass) {
        n_items = 0;
        for (int i = 0; i < cs.n; ++i) {
            int p = (int)std::floor(su[i] / u + 0.5);
            p = std::max(1, std::min(p, MAX_PARTS));
            cs.n_new[i] = p;
            n_items += dm.hkv * p;
        }
        if (n_items <= dm.max_chunks) break;
        u *= (double)n_items / dm.max_chunks * 1.05;
    }
    return n_items;
}

// Query preparation: one block per (sequence, kv head), G = query heads per kv head.
static hipError_t qprep_any(hipStream_t st, const Dims& dm, const Ptrs& P, int layer, const CallSeqs& cs,
                            const _Float16* q, float cm) {
    const dim3 g(cs.n, dm.hkv, dm.gate < INFINITY ? 1 + HOT_SLICES : 1);
    const int key = dm.d * 10 + dm.g;
    switch (key) {
        case 641: k_qprep<64, 1><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        case 642: k_qprep<64, 2><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        case 644: k_qprep<64, 4><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        case 648: k_qprep<64, 8><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        case 1281: k_qprep<128, 1><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        case 1282: k_qprep<128, 2><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        case 1284: k_qprep<128, 4><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        case 1288: k_qprep<128, 8><<<g, QP_NT, 0, st>>>(dm, P, layer, cs, q, cm); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Multi-query attention over the compressed cache: the queries of the newest
// n_new tokens of one sequence (a prefill chunk, or draft tokens being
// verified), each over every live cold slot and the hot entries up to its own
// token.  The G heads x n_new tokens of a kv head are virtual heads v = j G +
// h, run through the decode kernels in passes of up to 8 (the widest group
// the kernels take): the query prep reads the pass's queries as the heads of
// each sequence and the combine writes their outputs back in place
// (head_row), the split-context kernel's hot phase masks the chunk's later
// tokens.  Cold tiles are read once per pass.  A call may hold several
// sequences (each with its own n_new newest tokens as the chunk), which then
// share each pass's launches.
// ------------------------------------------------------------------------
constexpr int MQ_ITEMS = MQ_STREAMS_MAX;  // split-context parts per pass

struct MqLayout {
    size_t o_qg, o_qprep, o_part, o_cand, total;
};
static MqLayout mq_layout(const Dims& dm, int n_seq) {
    auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    MqLayout L{};
    const size_t heads = (size_t)n_seq * dm.hkv * 8;
    L.o_qg = 0;
    L.o_qprep = a256(heads * dm.d * 2);
    L.o_part = L.o_qprep + a256(heads * (dm.d + M_MAX) * 4);
    L.o_cand = L.o_part + a256((size_t)MQ_ITEMS * 2 * 8 * part_stride(dm.d) * 4);
    L.total = L.o_cand + a256((size_t)MQ_ITEMS * 8 * sizeof(Cand));
    return L;
}
size_t multi_query_workspace_bytes(const Dims& dm, int n_seq) { return mq_layout(dm, n_seq).total; }

hipError_t launch_multi_query(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& seqs,
                              int n_new, const int64_t* appended, const _Float16* q, float* out, uint8_t* ws,
                              hipStream_t st) {
    const MqLayout L = mq_layout(dm, seqs.n);
    const int n_virt = n_new * dm.g;
    Ptrs Pm = P;
    Pm.qgather = reinterpret_cast<_Float16*>(ws + L.o_qg);
    Pm.qprep = reinterpret_cast<float*>(ws + L.o_qprep);
    Pm.part = reinterpret_cast<float*>(ws + L.o_part);
    Pm.cand_chunk = reinterpret_cast<Cand*>(ws + L.o_cand);
    // parts of about 8 tiles: a pass over few sequences splits each of their
    // streams less finely than a batch decode step would, so that the parts'
    // start-up and the merge stay small against their tiles
    int64_t want = 0;
    for (int i = 0; i < seqs.n; ++i) want += (int64_t)dm.hkv * std::max<int64_t>(1, (appended[i] + 255) / 256);
    for (int v0 = 0; v0 < n_virt; v0 += 8) {
        const int rem = n_virt - v0;
        const int W = rem >= 8 ? 8 : (rem > 4 ? 8 : (rem > 2 ? 4 : rem));  // widths the kernels take
        Dims dp = dm;
        dp.g = W;
        dp.hq = dm.hkv * W;
        dp.ktop = 0;
        dp.gate = INFINITY;
        dp.max_chunks = (int)std::min<int64_t>(MQ_ITEMS, want);
        dp.mq_n = n_new;
        dp.mq_g = dm.g;
        dp.mq_v0 = v0;
        hipError_t e = launch_decode(dp, Pm, F, layer, seqs, appended, q, out, nullptr, 0, st, nullptr, nullptr);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_qprep8(const Dims& dm, const Ptrs& P, const _Float16* q, int n_groups, float cm, hipStream_t st) {
    Dims d8 = dm;
    d8.hq = n_groups * 8;
    d8.hkv = n_groups;
    d8.g = 8;
    d8.gate = INFINITY;
    CallSeqs cs{};
    cs.n = 1;
    const dim3 g(1, n_groups);
    if (dm.d == 64)
        k_qprep<64, 8><<<g, QP_NT, 0, st>>>(d8, P, 0, cs, q, cm);
    else
        k_qprep<128, 8><<<g, QP_NT, 0, st>>>(d8, P, 0, cs, q, cm);
    return hipGetLastError();
}

float qjl_query_scale(const LayerFmt& F) { return SQRT_HALF_PI / (float)F.m; }

hipError_t launch_decode(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, CallSeqs cs,
                         const int64_t* appended, const _Float16* q, float* out, float* logits, int logits_stride,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, bool q_ready) {
    if (cs.n == 0) return hipSuccess;
    if (q_ready && (dm.gate < INFINITY || dm.mq_n > 0)) return hipErrorInvalidValue;
    int resident = 0;
    hipError_t e = decode_any(st, dm, P, F, layer, cs, q, 0, nullptr, 0, &resident);
    if (e != hipSuccess) return e;
    const int n_items = plan_parts(dm, cs, appended, resident);
    if (n_items > dm.max_chunks) return hipErrorInvalidValue;
    // first item of each sequence (the decode and combine kernels read it)
    for (int i = 0, o = 0; i < cs.n; ++i) {
        cs.in_base[i] = o;
        o += dm.hkv * cs.n_new[i];
    }
    if (logits) {
        const size_t n = (size_t)cs.n * dm.hq * logits_stride;
        k_fill<<<(unsigned)std::min<size_t>((n + 255) / 256, 65536), 256, 0, st>>>(logits, n, -INFINITY);
    }
    const dim3 gq(cs.n, dm.hq);
    const float cm = qjl_query_scale(F);
    if (!q_ready) {  // else the step's append launch prepared the queries
        e = qprep_any(st, dm, P, layer, cs, q, cm);
        if (e != hipSuccess) return e;
    }
    // a multi-query pass's hot phase reads the queries k_qprep gathered
    e = decode_any(st, dm, P, F, layer, cs, dm.mq_n > 0 ? P.qgather : q, n_items, logits, logits_stride, nullptr,
                   ev0, ev1);
    if (e != hipSuccess) return e;
    // more blocks than two per CU: the variant that reads its matrix slice late
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
            n_cu = 256;
    }
    const bool pre = (long)cs.n * dm.hq <= 2L * n_cu;
    int max_parts = 0;
    for (int i = 0; i < cs.n; ++i) max_parts = std::max(max_parts, cs.n_new[i]);
    if (max_parts > PM_CHUNK) {
        const dim3 gm(cs.n, dm.hq, (max_parts + PM_CHUNK - 1) / PM_CHUNK);
        if (dm.d == 64)
            k_premerge<64><<<gm, 2 * 64 + M_MAX, 0, st>>>(dm, F, cs, P.part);
        else
            k_premerge<128><<<gm, 2 * 128 + M_MAX, 0, st>>>(dm, F, cs, P.part);
    }
    if (dm.d == 64) {
        if (pre)
            k_combine<64, true><<<gq, 2 * 64 + M_MAX, 0, st>>>(dm, P, F, layer, cs, q, out);
        else
            k_combine<64, false><<<gq, 2 * 64 + M_MAX, 0, st>>>(dm, P, F, layer, cs, q, out);
    } else {
        if (pre)
            k_combine<128, true><<<gq, 2 * 128 + M_MAX, 0, st>>>(dm, P, F, layer, cs, q, out);
        else
            k_combine<128, false><<<gq, 2 * 128 + M_MAX, 0, st>>>(dm, P, F, layer, cs, q, out);
    }
    return hipGetLastError();
}

}  // namespace tq
